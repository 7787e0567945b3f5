// qstate_kernels.hip — fused quantized recurrent-state decode kernels, gfx950.
//
// One wave (a workgroup of 64 lanes) owns a slice of the rows of one head
// (b, h); small batches split a head into several slices so that enough
// waves exist to fill 256 CUs.  A value row of the state is split across
// adjacent lanes: each lane owns one 16-byte run of codes, i.e. 16 INT8
// elements or 32 INT4 elements, so a row of dk columns spans dk/16 (INT8) or
// dk/32 (INT4) lanes and the wave holds the rest of its 64 lanes as further
// rows.  The loads of the next kPrefetch row iterations are in flight while
// the current one is computed.  Every operation of the step is row-local (LoReS
// blog, "LoReS: State Quantization": value-axis groups, full-precision update,
// readout from the updated state): the two dot products u = d.k and o = S'.q
// finish with DPP butterflies across the row's lanes, the group absmax with
// DPP butterflies across the group's lanes.  No LDS, no atomics, no
// cross-workgroup traffic: each state byte is read once and written once.
//
// Arithmetic follows the semantics written in include/qstate.h operation by
// operation (explicit fmaf, no contraction, IEEE division), so the stored
// codes are bit-identical to any other implementation of those semantics.
// The 16-element chunks and the butterflies realise the summation order
// defined there: sequential fused multiply-adds inside a chunk, then a
// pairwise tree over the chunks (an INT4 lane adds its two adjacent chunks,
// then DPP pairs adjacent lanes, adjacent lane pairs, ...).
//
// Instruction economy (the INT4 + stochastic-rounding path is VALU-bound):
//  * codes are turned into floats with v_cvt_f32_ubyte after flipping the
//    sign bit of each byte/nibble (offset binary c + 2^(n-1)); the decayed
//    value c*sa is then one fma(cu, sa, -2^(n-1)*sa), which is exactly the
//    rounded product c*sa because the addend is exact;
//  * stochastic rounding evaluates floor(S'*inv + R/2^16) as
//    floor(fma(S', inv*2^16, R) / 2^16): the scaling by 2^16 is exact, so the
//    code is byte 2 of floor(fma(...)), gathered with v_perm_b32;
//  * round-to-nearest adds 1.5*2^23 inside the fma, which leaves the rounded
//    code in the low byte of the result.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qstate_launch.h"

namespace qs {
namespace {

constexpr int kThreads = 64;  // one wave per workgroup
constexpr int kPrefetch = 4;  // row iterations whose loads are in flight ahead of compute
constexpr int kGDN = 0, kGLA = 1, kScalar = 2, kKDA = 3;
constexpr int kRTN = 0, kSR = 1, kBDR = 2;  // rounding of the step
// per-key-channel decay (GLA, KDA) and the delta-rule write weight (GDN, KDA)
constexpr bool vector_decay(int m) { return m == kGLA || m == kKDA; }
constexpr bool delta_rule(int m) { return m == kGDN || m == kKDA; }

// ---------------------------------------------------------------------------
// Counter-based random bits (semantics in include/qstate.h).
// ---------------------------------------------------------------------------

// SplitMix64 output function (Steele, Lea & Flood 2014).
__device__ __forceinline__ uint64_t splitmix64_out(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Key of (seed, layer, step, b, h): x = F((x ^ field) + golden) from x = 0.
__device__ __forceinline__ uint32_t head_key(const KParams& p, uint32_t b, uint32_t h) {
  constexpr uint64_t golden = 0x9E3779B97F4A7C15ull;
  uint64_t x = splitmix64_out(p.seed + golden);
  x = splitmix64_out((x ^ (uint64_t)p.layer) + golden);
  x = splitmix64_out((x ^ p.step) + golden);
  x = splitmix64_out((x ^ (uint64_t)b) + golden);
  x = splitmix64_out((x ^ (uint64_t)h) + golden);
  return (uint32_t)(x >> 32) ^ (uint32_t)x;
}

// MurmurHash3 32-bit finalizer (Appleby).
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// Marsaglia's xorshift32, shifts 13, 17, 5.
__device__ __forceinline__ uint32_t xorshift32(uint32_t y) {
  y ^= y << 13;
  y ^= y >> 17;
  y ^= y << 5;
  return y;
}

// The 16 random 16-bit values R of one 16-element block, as floats: one
// hashed seed and a walk of seven xorshift32 steps give the block's eight
// 32-bit words (low half: even element, high half: odd element).
__device__ __forceinline__ void block_r16(uint32_t key, uint32_t block, float* r) {
  uint32_t w = fmix32(key ^ block);
  w = w > 1u ? w : 1u;
#pragma unroll
  for (int pr = 0; pr < 8; ++pr) {
    if (pr) w = xorshift32(w);
    r[2 * pr] = (float)(w & 0xFFFFu);
    r[2 * pr + 1] = (float)(w >> 16);
  }
}

// ---------------------------------------------------------------------------
// DPP butterflies inside a 16-lane row of the wave.  After the two quad
// levels every lane of a quad holds the quad's value, so the half-row mirror
// pairs quad 0 with quad 1 and the row mirror pairs the two halves: each
// level adds adjacent partials of the tree, as xor butterflies would.
// ---------------------------------------------------------------------------

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <int LANES>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LANES >= 2) x = x + dpp<kDppXor1>(x);
  if constexpr (LANES >= 4) x = x + dpp<kDppXor2>(x);
  if constexpr (LANES >= 8) x = x + dpp<kDppHalfMirror>(x);
  if constexpr (LANES >= 16) x = x + dpp<kDppMirror>(x);
  return x;
}

template <int LANES>
__device__ __forceinline__ float lanes_max(float m) {
  if constexpr (LANES >= 2) m = fmaxf(m, dpp<kDppXor1>(m));
  if constexpr (LANES >= 4) m = fmaxf(m, dpp<kDppXor2>(m));
  if constexpr (LANES >= 8) m = fmaxf(m, dpp<kDppHalfMirror>(m));
  return m;
}

// Sequential fused dot product of the 16-element chunk starting at x[off].
template <int N>
__device__ __forceinline__ float chunk_dot(const float (&x)[N], const float (&y)[N], int off) {
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) acc = __builtin_fmaf(x[off + j], y[off + j], acc);
  return acc;
}

// Lane partial of a row dot product: the lane's chunks summed in order.
template <int N>
__device__ __forceinline__ float lane_dot(const float (&x)[N], const float (&y)[N]) {
  float acc = chunk_dot(x, y, 0);
  if constexpr (N == 32) acc = acc + chunk_dot(x, y, 16);
  return acc;
}

// ---------------------------------------------------------------------------
// Scale of a group: s = m / r; inv = r / m rounded toward zero (the largest
// float with inv * m <= r); an all-zero group gets s = inv = 0.
// ---------------------------------------------------------------------------

// s = m / r, correctly rounded, as one product and one fused correction:
// with c = RN(1/r), q = m*c, e = fma(-q, r, m), fma(e, c, q) equals RN(m/r)
// for every normal m when r is 7 or 127 (an exhaustive check over all
// mantissas is part of the tests); tiny m keeps the IEEE division.
template <int R>
__device__ __forceinline__ void group_scale(float m, float& s, float& inv) {
  constexpr float r = (float)R;
  constexpr float c = 1.0f / (float)R;
  const float q = m * c;
  s = __builtin_fmaf(__builtin_fmaf(-q, r, m), c, q);
  if (__builtin_expect(m < 0x1p-100f && m != 0.0f, 0)) s = m / r;
  float v = r / m;
  if (__builtin_fmaf(m, v, -r) > 0.0f) v = __int_as_float(__float_as_int(v) - 1);
  inv = (m == 0.0f) ? 0.0f : v;
}

// ---------------------------------------------------------------------------
// Lane geometry: one 16-byte run of codes per lane.
// ---------------------------------------------------------------------------

template <int DK, int BITS>
struct Geo {
  static constexpr int E = BITS == 4 ? 32 : 16;  // elements per lane
  static constexpr int LPR = DK / E;             // lanes per row
  static constexpr int RPW = 64 / LPR;           // rows per wave iteration
  static constexpr int ROW_BYTES = DK * BITS / 8;
};

// Codes to floats in offset binary: cu = c + 2^(BITS-1).  16 elements from
// four words (INT8) or two words (INT4).
template <int BITS>
__device__ __forceinline__ void unpack16(const uint32_t* w, float* cu) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t x = w[q] ^ 0x80808080u;
      asm("" : "+v"(x));  // convert bytes in place (v_cvt_f32_ubyte0..3)
#pragma unroll
      for (int p = 0; p < 4; ++p) cu[4 * q + p] = (float)((x >> (8 * p)) & 0xFFu);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t x = w[q] ^ 0x88888888u;
      uint32_t lo = x & 0x0F0F0F0Fu;         // even elements, one per byte
      uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // odd elements
      asm("" : "+v"(lo));  // convert bytes in place (v_cvt_f32_ubyte0..3)
      asm("" : "+v"(hi));
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        cu[8 * q + 2 * p] = (float)((lo >> (8 * p)) & 0xFFu);
        cu[8 * q + 2 * p + 1] = (float)((hi >> (8 * p)) & 0xFFu);
      }
    }
  }
}

// Bytes [a.BP, b.BP, c.BP, d.BP] of four words.
template <int BP>
__device__ __forceinline__ uint32_t gather4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  constexpr uint32_t sel = 0x0C0C0000u | ((4u + BP) << 8) | (uint32_t)BP;
  const uint32_t lo = __builtin_amdgcn_perm(b, a, sel);
  const uint32_t hi = __builtin_amdgcn_perm(d, c, sel);
  return lo | (hi << 16);
}

// Pack 16 codes (byte BP of each word of src): four words (INT8) or two (INT4).
template <int BITS, int BP>
__device__ __forceinline__ void pack16(const uint32_t* src, uint32_t* out) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      out[q] = gather4<BP>(src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]);
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t ev = gather4<BP>(src[8 * q], src[8 * q + 2], src[8 * q + 4], src[8 * q + 6]);
      const uint32_t od = gather4<BP>(src[8 * q + 1], src[8 * q + 3], src[8 * q + 5], src[8 * q + 7]);
      out[q] = (ev & 0x0F0F0F0Fu) | ((od << 4) & 0xF0F0F0F0u);
    }
  }
}

// floor(x) as int32 in one instruction.
__device__ __forceinline__ int32_t floor_i32(float x) {
  int32_t r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// Requantize one 16-element chunk with inverse scale inv into 16 packed codes
// (four words for INT8, two for INT4).  block: the chunk's 16-element block
// index in the head (stochastic rounding).  wprev / s_old: the chunk's codes
// and scale before the step, s_new its new scale (bounded directional
// rounding).
template <int BITS, int RND>
__device__ __forceinline__ void quantize16(const float* sp, float inv, uint32_t key, uint32_t block,
                                           const uint32_t* wprev, float s_old, float s_new,
                                           uint32_t* out) {
  uint32_t src[16];
  if constexpr (RND == kSR) {
    float R[16];
    block_r16(key, block, R);
    if (__builtin_expect(inv <= 0x1p100f, 1)) {
      const float i16 = inv * 65536.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) src[j] = (uint32_t)floor_i32(__builtin_fmaf(sp[j], i16, R[j]));
    } else {  // groups of tiny magnitude, where inv * 2^16 could overflow
#pragma unroll
      for (int j = 0; j < 16; ++j)
        src[j] = (uint32_t)floor_i32(__builtin_fmaf(sp[j], inv, R[j] * (1.0f / 65536.0f))) << 16;
    }
    pack16<BITS, 2>(src, out);
  } else {
    // y = 1.5*2^23 + rint(S'*inv): the code sits in the low mantissa bits.
    constexpr float kMagic = 12582912.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) src[j] = __float_as_uint(__builtin_fmaf(sp[j], inv, kMagic));
    if constexpr (RND == kBDR) {
      // prev = c*s_old exactly as stored; the nearest code's stored value
      // (y - magic)*s_new; where prev lies strictly between that value and
      // S', step one code toward S' (y stays in the magic's binade, so +-1
      // is exact), then clamp to [-r, r].
      constexpr int R = (1 << (BITS - 1)) - 1;
      constexpr float bias = (float)(1 << (BITS - 1));
      float prev[16];
      unpack16<BITS>(wprev, prev);
      const float nb = -bias * s_old;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv = __builtin_fmaf(prev[j], s_old, nb);
        float y = __uint_as_float(src[j]);
        const float st = (y - kMagic) * s_new;
        const float x = sp[j];
        if (x > pv && st < pv) y += 1.0f;
        if (x < pv && st > pv) y -= 1.0f;
        y = fminf(fmaxf(y, kMagic - (float)R), kMagic + (float)R);
        src[j] = __float_as_uint(y);
      }
    }
    pack16<BITS, 0>(src, out);
  }
}

// Requantize the lane's E elements of the updated row S' into 16 bytes of
// codes.  LPG = 0: two groups per lane (INT4 with G = 16, one per chunk);
// otherwise one group spanning LPG lanes.  s0/s1: the scales of the lane's
// groups (in: before the step, used by bounded directional rounding; out:
// the new ones).  wprev: the lane's four code words before the step.
template <int BITS, int RND, int E, int LPG>
__device__ __forceinline__ uint4 quantize_lane(const float (&sp)[E], uint32_t key, uint32_t block0,
                                               const uint32_t* wprev, float& s0, float& s1) {
  constexpr int R = (1 << (BITS - 1)) - 1;
  const float so0 = s0, so1 = s1;
  float m0 = 0.0f, m1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m0 = fmaxf(m0, fabsf(sp[j]));
  if constexpr (E == 32) {
#pragma unroll
    for (int j = 16; j < 32; ++j) m1 = fmaxf(m1, fabsf(sp[j]));
  }
  float inv0, inv1;
  if constexpr (LPG == 0) {
    group_scale<R>(m0, s0, inv0);
    group_scale<R>(m1, s1, inv1);
  } else {
    m0 = lanes_max<LPG>(fmaxf(m0, m1));
    group_scale<R>(m0, s0, inv0);
    s1 = s0, inv1 = inv0;
  }
  uint32_t o[4];
  quantize16<BITS, RND>(sp, inv0, key, block0, wprev, so0, s0, o);
  if constexpr (E == 32)
    quantize16<BITS, RND>(sp + 16, inv1, key, block0 + 1, wprev + 2, so1, s1, o + 2);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// Per-head geometry.
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool head_is_int8(const KParams& p, int h) {
  return (p.int8_mask[h >> 5] >> (h & 31)) & 1u;
}

// Byte offset of head (b, h): b * bytes_per_b + sum_{h' < h} bytes(h'), an
// INT8 head being twice an INT4 head.
__device__ __forceinline__ uint64_t head_code_offset(const KParams& p, int b, int h) {
  uint32_t n8 = 0;
  for (int w = 0; w < (h >> 5); ++w) n8 += __popc(p.int8_mask[w]);
  if (h & 31) n8 += __popc(p.int8_mask[h >> 5] & ((1u << (h & 31)) - 1u));
  return (uint64_t)b * p.bytes_per_b + (uint64_t)(h + n8) * p.head_bytes4;
}

template <int N>
__device__ __forceinline__ void loadv(const float* ptr, float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const float4 t = reinterpret_cast<const float4*>(ptr)[q];
    x[4 * q] = t.x, x[4 * q + 1] = t.y, x[4 * q + 2] = t.z, x[4 * q + 3] = t.w;
  }
}

template <int N>
__device__ __forceinline__ void storev(float* ptr, const float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q)
    reinterpret_cast<float4*>(ptr)[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
}

// The wave's head and row slice [r0, r1).
struct Slice {
  int head, b, h, r0, r1;
};

__device__ __forceinline__ Slice wave_slice(const KParams& p) {
  Slice sl;
  sl.head = blockIdx.x / p.slices;
  const int part = blockIdx.x - sl.head * p.slices;
  sl.b = sl.head / p.H;
  sl.h = sl.head - sl.b * p.H;
  sl.r0 = part * p.slice_rows;
  sl.r1 = min(p.dv, sl.r0 + p.slice_rows);
  return sl;
}

// ---------------------------------------------------------------------------
// The decode step on a quantized head of BITS-bit codes.
// ---------------------------------------------------------------------------

struct RowIn {
  uint4 raw;
  float s0, s1, v;
};

template <int MIXER, int RND, int DK, int BITS, int G>
__device__ __forceinline__ void step_quant_head(const KParams& p, const Slice sl) {
  constexpr bool SR = RND == kSR;
  using Gm = Geo<DK, BITS>;
  constexpr int E = Gm::E, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr float bias = (float)(1 << (BITS - 1));
  constexpr bool two_groups = G < E;  // INT4 with G = 16
  constexpr int LPG = two_groups ? 0 : G / E;
  constexpr int ngr = DK / G;
  const int lane = threadIdx.x;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  const int gcol = two_groups ? col0 / 16 : col0 / G;  // first group of the lane in its row

  uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
  float* hscales = p.scales + (size_t)sl.head * p.dv * ngr;
  const float* vh = p.v + (size_t)sl.head * p.dv;
  float* oh = p.o ? p.o + (size_t)sl.head * p.dv : nullptr;
  const int n_it = (sl.r1 - sl.r0 + RPW - 1) / RPW;

  // per-head vectors first, so that waiting for them never drains the ring
  const uint32_t key = SR ? head_key(p, (uint32_t)sl.b, (uint32_t)sl.h) : 0u;
  float kk[E], qq[E], al[E];
  loadv(p.k + (size_t)sl.head * DK + col0, kk);
  loadv(p.q + (size_t)sl.head * DK + col0, qq);
  float alpha_s = 0.0f, beta = 0.0f;
  if constexpr (vector_decay(MIXER)) {
    loadv(p.alpha + (size_t)sl.head * DK + col0, al);
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) al[j] = 0.0f;
    alpha_s = p.alpha[sl.head];
  }
  if constexpr (MIXER != kGLA) beta = p.beta[sl.head];
  asm volatile("" ::: "memory");  // keep these loads ahead of the ring's

  // Every lane always loads an in-range row: rows past the slice (the last
  // iteration's tail and the prefetches beyond the end) re-read the slice's
  // last row and are never stored.  Branch-free loads keep the ring's loads
  // in flight across iterations.
  auto load = [&](int it) {
    RowIn in;
    const int row = min(sl.r0 + it * RPW + rsub, sl.r1 - 1);
    in.raw = *reinterpret_cast<const uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16);
    in.s0 = hscales[(size_t)row * ngr + gcol];
    in.s1 = two_groups ? hscales[(size_t)row * ngr + gcol + 1] : in.s0;
    in.v = vh[row];
    return in;
  };
  RowIn ring[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    ring[k] = load(k);
    asm volatile("" ::: "memory");  // issue the slots in order: slot 0 is needed first
  }

  // Trips of kPrefetch iterations.  A slot's next load is issued once its
  // previous contents (codes, scales, v) are dead, so the load lands in the
  // same registers and stays in flight across trips.
  // Iterations past the end compute on clamped rows and store nothing.
  const int n_trips = (n_it + kPrefetch - 1) / kPrefetch;
  for (int t = 0; t < n_trips; ++t) {
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int it = t * kPrefetch + k;
      const int row = sl.r0 + it * RPW + rsub;
      const bool store_ok = it < n_it && row < sl.r1;
      const uint32_t w[4] = {ring[k].raw.x, ring[k].raw.y, ring[k].raw.z, ring[k].raw.w};
      const float s_0 = ring[k].s0, s_1 = ring[k].s1, vrow = ring[k].v;
      float d[E];
      unpack16<BITS>(w, d);
      if constexpr (E == 32) unpack16<BITS>(w + 2, d + 16);
      // decayed dequantized values (exactly the rounded c*(s*alpha) / (c*s)*alpha_j)
      if constexpr (vector_decay(MIXER)) {
        const float nb0 = -bias * s_0, nb1 = -bias * s_1;
#pragma unroll
        for (int j = 0; j < E; ++j)
          d[j] = __builtin_fmaf(d[j], j < 16 ? s_0 : s_1, j < 16 ? nb0 : nb1) * al[j];
      } else {
        const float sa0 = s_0 * alpha_s, sa1 = s_1 * alpha_s;
        const float nb0 = -bias * sa0, nb1 = -bias * sa1;
#pragma unroll
        for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(d[j], j < 16 ? sa0 : sa1, j < 16 ? nb0 : nb1);
      }
      // write weight
      float wt;
      if constexpr (delta_rule(MIXER)) {
        const float u = row_sum<LPR>(lane_dot(d, kk));
        wt = beta * (vrow - u);
      } else if constexpr (MIXER == kGLA) {
        wt = vrow;
      } else {
        wt = beta * vrow;
      }
      // rank-1 write (in place) and readout from the full-precision S'
#pragma unroll
      for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(wt, kk[j], d[j]);
      ring[k] = load(it + kPrefetch);  // nothing of the slot is live any more
      const float o = row_sum<LPR>(lane_dot(d, qq));
      // requantize
      float s0 = s_0, s1 = s_1;
      const uint32_t block0 = (uint32_t)((row * DK + col0) >> 4);
      const uint4 packed = quantize_lane<BITS, RND, E, LPG>(d, key, block0, w, s0, s1);
      if (store_ok) {
        *reinterpret_cast<uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16) = packed;
        if constexpr (two_groups) {
          hscales[(size_t)row * ngr + gcol] = s0;
          hscales[(size_t)row * ngr + gcol + 1] = s1;
        } else if (lr % LPG == 0) {
          hscales[(size_t)row * ngr + gcol] = s0;
        }
        if (oh && lr == 0) oh[row] = o;
      }
    }
  }
}

// The same step on an unquantized FP32 head: 16 elements per lane.
template <int MIXER, int DK>
__device__ __forceinline__ void step_fp32_head(const KParams& p, const Slice sl) {
  constexpr int E = 16, LPR = DK / E, RPW = 64 / LPR;
  const int lane = threadIdx.x;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  float* hS = reinterpret_cast<float*>(p.state) + (size_t)sl.head * p.dv * DK;
  const float* vh = p.v + (size_t)sl.head * p.dv;
  float* oh = p.o ? p.o + (size_t)sl.head * p.dv : nullptr;
  const int n_it = (sl.r1 - sl.r0 + RPW - 1) / RPW;
  struct FIn {
    float x[E];
    float v;
  };
  float kk[E], qq[E], al[E];
  loadv(p.k + (size_t)sl.head * DK + col0, kk);
  loadv(p.q + (size_t)sl.head * DK + col0, qq);
  float alpha_s = 0.0f, beta = 0.0f;
  if constexpr (vector_decay(MIXER)) {
    loadv(p.alpha + (size_t)sl.head * DK + col0, al);
  } else {
#pragma unroll
    for (int j = 0; j < E; ++j) al[j] = 0.0f;
    alpha_s = p.alpha[sl.head];
  }
  if constexpr (MIXER != kGLA) beta = p.beta[sl.head];
  asm volatile("" ::: "memory");  // keep these loads ahead of the ring's
  // branch-free loads of in-range rows (see step_quant_head)
  auto load = [&](int it) {
    FIn in;
    const int row = min(sl.r0 + it * RPW + rsub, sl.r1 - 1);
    loadv(hS + (size_t)row * DK + col0, in.x);
    in.v = vh[row];
    return in;
  };
  FIn ring[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    ring[k] = load(k);
    asm volatile("" ::: "memory");  // issue the slots in order: slot 0 is needed first
  }
  const int n_trips = (n_it + kPrefetch - 1) / kPrefetch;
  for (int t = 0; t < n_trips; ++t) {
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int it = t * kPrefetch + k;
      const int row = sl.r0 + it * RPW + rsub;
      const bool store_ok = it < n_it && row < sl.r1;
      const float vrow = ring[k].v;
      float d[E];
#pragma unroll
      for (int j = 0; j < E; ++j) d[j] = ring[k].x[j] * (vector_decay(MIXER) ? al[j] : alpha_s);
      float wt;
      if constexpr (delta_rule(MIXER)) {
        const float u = row_sum<LPR>(lane_dot(d, kk));
        wt = beta * (vrow - u);
      } else if constexpr (MIXER == kGLA) {
        wt = vrow;
      } else {
        wt = beta * vrow;
      }
#pragma unroll
      for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(wt, kk[j], d[j]);
      ring[k] = load(it + kPrefetch);  // nothing of the slot is live any more
      const float o = row_sum<LPR>(lane_dot(d, qq));
      if (store_ok) {
        storev(hS + (size_t)row * DK + col0, d);
        if (oh && lr == 0) oh[row] = o;
      }
    }
  }
}

// Import (quantize an FP32 state), export (dequantize) and readout of a
// quantized head, with the step's lane geometry and quantizer.
template <int OP, bool SR, int DK, int BITS, int G>
__device__ __forceinline__ void aux_quant_head(const KParams& p, const Slice sl) {
  using Gm = Geo<DK, BITS>;
  constexpr int E = Gm::E, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr float bias = (float)(1 << (BITS - 1));
  constexpr bool two_groups = G < E;
  constexpr int LPG = two_groups ? 0 : G / E;
  constexpr int ngr = DK / G;
  const int lane = threadIdx.x;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  const int gcol = two_groups ? col0 / 16 : col0 / G;
  uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
  float* hscales = p.scales + (size_t)sl.head * p.dv * ngr;
  const size_t hoff = (size_t)sl.head * p.dv * DK;
  const uint32_t key = (OP == kImport && SR) ? head_key(p, (uint32_t)sl.b, (uint32_t)sl.h) : 0u;
  float qq[E];
  if constexpr (OP == kReadout) loadv(p.q + (size_t)sl.head * DK + col0, qq);
  for (int rbase = sl.r0; rbase < sl.r1; rbase += RPW) {
    const int row = rbase + rsub;
    const bool ok = row < sl.r1;
    if constexpr (OP == kImport) {
      float x[E];
      if (ok)
        loadv(p.src + hoff + (size_t)row * DK + col0, x);
      else
#pragma unroll
        for (int j = 0; j < E; ++j) x[j] = 0.0f;
      float s0 = 0.0f, s1 = 0.0f;
      const uint32_t no_prev[4] = {0u, 0u, 0u, 0u};  // read only by BDR, never on import
      const uint32_t block0 = (uint32_t)((row * DK + col0) >> 4);
      const uint4 packed =
          quantize_lane<BITS, SR ? kSR : kRTN, E, LPG>(x, key, block0, no_prev, s0, s1);
      if (ok) {
        *reinterpret_cast<uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16) = packed;
        if constexpr (two_groups) {
          hscales[(size_t)row * ngr + gcol] = s0;
          hscales[(size_t)row * ngr + gcol + 1] = s1;
        } else if (lr % LPG == 0) {
          hscales[(size_t)row * ngr + gcol] = s0;
        }
      }
    } else {
      uint4 raw = make_uint4(0u, 0u, 0u, 0u);
      float s0 = 0.0f, s1 = 0.0f;
      if (ok) {
        raw = *reinterpret_cast<const uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16);
        s0 = hscales[(size_t)row * ngr + gcol];
        s1 = two_groups ? hscales[(size_t)row * ngr + gcol + 1] : s0;
      }
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      float x[E];
      unpack16<BITS>(w, x);
      if constexpr (E == 32) unpack16<BITS>(w + 2, x + 16);
      const float nb0 = -bias * s0, nb1 = -bias * s1;
#pragma unroll
      for (int j = 0; j < E; ++j) x[j] = __builtin_fmaf(x[j], j < 16 ? s0 : s1, j < 16 ? nb0 : nb1);
      if constexpr (OP == kExport) {
        if (ok) storev(p.dst + hoff + (size_t)row * DK + col0, x);
      } else {
        const float o = row_sum<LPR>(lane_dot(x, qq));
        if (ok && lr == 0) p.o[(size_t)sl.head * p.dv + row] = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key-axis scale groups: G consecutive value rows of one key column share a
// scale (LoReS blog, "Scale grouping", the comparison to the value-axis
// default; C_j of Prop. "per-channel readout error").  A group's absmax spans
// rows held by different lanes and iterations, so a workgroup keeps a block
// of rows' updated values in registers, combines partial column maxima
// through LDS, and requantizes once every column's scale is known.  Each lane
// owns a 16-element run of a row (16 bytes of INT8 or 8 bytes of INT4), so a
// row spans dk/16 lanes and the dot products use the same butterflies and
// summation order as the value-axis kernels.  Scales: [B][H][dv/G][dk].
// ---------------------------------------------------------------------------

template <int DK, int G>
struct KGeo {
  static constexpr int E = 16;                    // elements per lane
  static constexpr int LPR = DK / E;              // lanes per row
  static constexpr int RPW = 64 / LPR;            // rows per wave iteration
  static constexpr int NI = 4;                    // iterations a wave holds
  static constexpr int RB = NI * RPW;             // rows per wave block: 4096 / dk
  static constexpr int NW = G > RB ? G / RB : 1;  // waves per workgroup
  static constexpr int BR = NW * RB;              // rows per workgroup block
  static constexpr int LG = BR / G;               // row groups per block
  static constexpr int PARTS = NW * RPW;          // partial maxima per column and group
};

// Requantize 16 elements with one inverse scale per element (key-axis
// groups).  Same rounding as quantize16; inv16/s_old/s_new per element.
template <int BITS, int RND>
__device__ __forceinline__ void quantize16_cols(const float* sp, const float* inv16, uint32_t key,
                                                uint32_t block, const uint32_t* wprev,
                                                const float* s_old, const float* s_new,
                                                uint32_t* out) {
  uint32_t src[16];
  if constexpr (RND == kSR) {
    float R[16];
    block_r16(key, block, R);
    float imax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) imax = fmaxf(imax, inv16[j]);
    if (__builtin_expect(imax <= 0x1p100f, 1)) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        src[j] = (uint32_t)floor_i32(__builtin_fmaf(sp[j], inv16[j] * 65536.0f, R[j]));
    } else {  // a tiny-magnitude group, where inv * 2^16 could overflow
#pragma unroll
      for (int j = 0; j < 16; ++j)
        src[j] = (uint32_t)floor_i32(__builtin_fmaf(sp[j], inv16[j], R[j] * (1.0f / 65536.0f)))
                 << 16;
    }
    pack16<BITS, 2>(src, out);
  } else {
    constexpr float kMagic = 12582912.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) src[j] = __float_as_uint(__builtin_fmaf(sp[j], inv16[j], kMagic));
    if constexpr (RND == kBDR) {
      constexpr int R = (1 << (BITS - 1)) - 1;
      constexpr float bias = (float)(1 << (BITS - 1));
      float prev[16];
      unpack16<BITS>(wprev, prev);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv = __builtin_fmaf(prev[j], s_old[j], -bias * s_old[j]);
        float y = __uint_as_float(src[j]);
        const float st = (y - kMagic) * s_new[j];
        const float x = sp[j];
        if (x > pv && st < pv) y += 1.0f;
        if (x < pv && st > pv) y -= 1.0f;
        y = fminf(fmaxf(y, kMagic - (float)R), kMagic + (float)R);
        src[j] = __float_as_uint(y);
      }
    }
    pack16<BITS, 0>(src, out);
  }
}

template <int N>
__device__ __forceinline__ void lds_load(const float* ptr, float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const float4 t = reinterpret_cast<const float4*>(ptr)[q];
    x[4 * q] = t.x, x[4 * q + 1] = t.y, x[4 * q + 2] = t.z, x[4 * q + 3] = t.w;
  }
}

// Step (OP = kStep) or import (OP = kImport) of a quantized head with
// key-axis groups.  LDS: partial column maxima, old scales, new scales and
// inverse scales of the block's row groups.
template <int OP, int MIXER, int RND, int DK, int BITS, int G>
__device__ __forceinline__ void key_quant_head(const KParams& p, const Slice sl, float* lds) {
  using K = KGeo<DK, G>;
  constexpr int E = K::E, LPR = K::LPR, RPW = K::RPW, NI = K::NI, RB = K::RB, NW = K::NW;
  constexpr int BR = K::BR, LG = K::LG, PARTS = K::PARTS;
  constexpr int R = (1 << (BITS - 1)) - 1;
  constexpr float bias = (float)(1 << (BITS - 1));
  constexpr int ROW_BYTES = DK * BITS / 8;
  constexpr int LANE_BYTES = E * BITS / 8;  // 16 (INT8) or 8 (INT4)
  constexpr int NWORDS = LANE_BYTES / 4;
  float* pm = lds;                        // [LG][PARTS][DK]
  float* so = pm + LG * PARTS * DK;       // [LG][DK] scales before the step
  float* sn = so + LG * DK;               // [LG][DK] new scales
  float* si = sn + LG * DK;               // [LG][DK] new inverse scales

  const int tid = threadIdx.x;
  const int wv = tid / 64;
  const int lane = tid % 64;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
  float* hscales = p.scales + (size_t)sl.head * (p.dv / G) * DK;
  const uint32_t key =
      (RND == kSR) ? head_key(p, (uint32_t)sl.b, (uint32_t)sl.h) : 0u;

  float kk[E], qq[E], al[E];
  float alpha_s = 0.0f, beta = 0.0f;
  const float* vh = nullptr;
  float* oh = nullptr;
  if constexpr (OP == kStep) {
    loadv(p.k + (size_t)sl.head * DK + col0, kk);
    loadv(p.q + (size_t)sl.head * DK + col0, qq);
    if constexpr (vector_decay(MIXER)) {
      loadv(p.alpha + (size_t)sl.head * DK + col0, al);
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) al[j] = 0.0f;
      alpha_s = p.alpha[sl.head];
    }
    if constexpr (MIXER != kGLA) beta = p.beta[sl.head];
    vh = p.v + (size_t)sl.head * p.dv;
    oh = p.o ? p.o + (size_t)sl.head * p.dv : nullptr;
  }

  for (int base = sl.r0; base < sl.r1; base += BR) {
    // scales of the block's row groups before the step
    if constexpr (OP == kStep) {
      for (int t = tid; t < LG * DK; t += 64 * NW) {
        const int grow = base / G + t / DK;
        so[t] = grow * G < p.dv ? hscales[(size_t)grow * DK + t % DK] : 0.0f;
      }
    }
    // this wave's rows: base + wv*RB + it*RPW + rsub; every row of an
    // iteration lies in one row group, and a group is wholly inside dv or
    // wholly outside (G divides dv, RPW divides G)
    uint32_t wc[NI][4] = {};
    float vr[NI] = {};
    float sp[NI][E];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int row = min(base + wv * RB + it * RPW + rsub, p.dv - 1);
      if constexpr (OP == kStep) {
        const uint8_t* src = hcodes + (size_t)row * ROW_BYTES + lr * LANE_BYTES;
        if constexpr (NWORDS == 4) {
          const uint4 t = *reinterpret_cast<const uint4*>(src);
          wc[it][0] = t.x, wc[it][1] = t.y, wc[it][2] = t.z, wc[it][3] = t.w;
        } else {
          const uint2 t = *reinterpret_cast<const uint2*>(src);
          wc[it][0] = t.x, wc[it][1] = t.y, wc[it][2] = 0u, wc[it][3] = 0u;
        }
        vr[it] = vh[row];
      } else {
        loadv(p.src + ((size_t)sl.head * p.dv + row) * DK + col0, sp[it]);
      }
    }
    if constexpr (OP == kStep) __syncthreads();  // old scales in LDS

    // update (step) and running column maxima per row group
    float cm[E];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int lg = (wv * RB + it * RPW) / G;  // constant per it when NW == 1, else 0
      const bool first = NW > 1 ? it == 0 : (it * RPW) % G == 0;
      const bool last = NW > 1 ? it == NI - 1 : ((it + 1) * RPW) % G == 0;
      if constexpr (OP == kStep) {
        const int row = base + wv * RB + it * RPW + rsub;
        float sc[E];
        lds_load(so + lg * DK + col0, sc);
        float d[E];
        unpack16<BITS>(wc[it], d);
        if constexpr (vector_decay(MIXER)) {
#pragma unroll
          for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(d[j], sc[j], -bias * sc[j]) * al[j];
        } else {
#pragma unroll
          for (int j = 0; j < E; ++j) {
            const float sa = sc[j] * alpha_s;
            d[j] = __builtin_fmaf(d[j], sa, -bias * sa);
          }
        }
        float wt;
        if constexpr (delta_rule(MIXER)) {
          const float u = row_sum<LPR>(lane_dot(d, kk));
          wt = beta * (vr[it] - u);
        } else if constexpr (MIXER == kGLA) {
          wt = vr[it];
        } else {
          wt = beta * vr[it];
        }
#pragma unroll
        for (int j = 0; j < E; ++j) sp[it][j] = __builtin_fmaf(wt, kk[j], d[j]);
        const float o = row_sum<LPR>(lane_dot(sp[it], qq));
        if (oh && lr == 0 && row < p.dv) oh[row] = o;
      }
#pragma unroll
      for (int j = 0; j < E; ++j)
        cm[j] = first ? fabsf(sp[it][j]) : fmaxf(cm[j], fabsf(sp[it][j]));
      if (last) {
        float* dst = pm + ((size_t)lg * PARTS + wv * RPW + rsub) * DK + col0;
#pragma unroll
        for (int q4 = 0; q4 < E / 4; ++q4)
          reinterpret_cast<float4*>(dst)[q4] =
              make_float4(cm[4 * q4], cm[4 * q4 + 1], cm[4 * q4 + 2], cm[4 * q4 + 3]);
      }
    }
    __syncthreads();  // every partial maximum in LDS

    // one thread per (row group, column): absmax, scale, inverse scale
    for (int t = tid; t < LG * DK; t += 64 * NW) {
      const int lg = t / DK, j = t % DK;
      float m = 0.0f;
#pragma unroll 8
      for (int q = 0; q < PARTS; ++q) m = fmaxf(m, pm[((size_t)lg * PARTS + q) * DK + j]);
      float s, inv;
      group_scale<R>(m, s, inv);
      sn[t] = s;
      si[t] = inv;
      const int grow = base / G + lg;
      if (grow * G < p.dv) hscales[(size_t)grow * DK + j] = s;
    }
    __syncthreads();  // new scales in LDS

    // requantize and store
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int lg = (wv * RB + it * RPW) / G;
      const int row = base + wv * RB + it * RPW + rsub;
      float inv16[E], s_old[E], s_new[E];
      lds_load(si + lg * DK + col0, inv16);
      if constexpr (RND == kBDR) {
        lds_load(so + lg * DK + col0, s_old);
        lds_load(sn + lg * DK + col0, s_new);
      }
      uint32_t out[4];
      const uint32_t block = (uint32_t)((row * DK + col0) >> 4);
      quantize16_cols<BITS, (OP == kImport && RND == kBDR) ? kRTN : RND>(
          sp[it], inv16, key, block, wc[it], s_old, s_new, out);
      if (row < p.dv) {
        uint8_t* dst = hcodes + (size_t)row * ROW_BYTES + lr * LANE_BYTES;
        if constexpr (NWORDS == 4)
          *reinterpret_cast<uint4*>(dst) = make_uint4(out[0], out[1], out[2], out[3]);
        else
          *reinterpret_cast<uint2*>(dst) = make_uint2(out[0], out[1]);
      }
    }
    __syncthreads();  // LDS free for the next block
  }
}

// Export (dequantize) or readout of a quantized head with key-axis groups.
template <int OP, int DK, int BITS, int G>
__device__ __forceinline__ void key_aux_head(const KParams& p, const Slice sl) {
  using K = KGeo<DK, G>;
  constexpr int E = K::E, LPR = K::LPR, RPW = K::RPW, NW = K::NW;
  constexpr float bias = (float)(1 << (BITS - 1));
  constexpr int ROW_BYTES = DK * BITS / 8;
  constexpr int LANE_BYTES = E * BITS / 8;
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int lr = lane % LPR;
  const int col0 = lr * E;
  const uint8_t* hcodes =
      reinterpret_cast<const uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
  const float* hscales = p.scales + (size_t)sl.head * (p.dv / G) * DK;
  float qq[E];
  if constexpr (OP == kReadout) loadv(p.q + (size_t)sl.head * DK + col0, qq);
  // the workgroup's NW waves take consecutive row iterations
  for (int rbase = sl.r0 + (tid / 64) * RPW; rbase < sl.r1; rbase += NW * RPW) {
    const int row = rbase + lane / LPR;
    const bool ok = row < sl.r1;
    const int rr = min(row, p.dv - 1);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    const uint8_t* src = hcodes + (size_t)rr * ROW_BYTES + lr * LANE_BYTES;
    if constexpr (LANE_BYTES == 16) {
      const uint4 t = *reinterpret_cast<const uint4*>(src);
      w[0] = t.x, w[1] = t.y, w[2] = t.z, w[3] = t.w;
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(src);
      w[0] = t.x, w[1] = t.y;
    }
    float sc[E], d[E];
    loadv(hscales + (size_t)(rr / G) * DK + col0, sc);
    unpack16<BITS>(w, d);
#pragma unroll
    for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(d[j], sc[j], -bias * sc[j]);
    if constexpr (OP == kExport) {
      if (ok) storev(p.dst + ((size_t)sl.head * p.dv + row) * DK + col0, d);
    } else {
      const float o = row_sum<LPR>(lane_dot(d, qq));
      if (ok && lr == 0) p.o[(size_t)sl.head * p.dv + row] = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------

template <int MIXER, int RND, int DK, int G>
__global__ __launch_bounds__(kThreads) void step_kernel(const KParams p) {
  const Slice sl = wave_slice(p);
  if (head_is_int8(p, sl.h))
    step_quant_head<MIXER, RND, DK, 8, G>(p, sl);
  else
    step_quant_head<MIXER, RND, DK, 4, G>(p, sl);
}

template <int MIXER, int DK>
__global__ __launch_bounds__(kThreads) void step_fp32_kernel(const KParams p) {
  step_fp32_head<MIXER, DK>(p, wave_slice(p));
}

template <int OP, bool SR, int DK, int G>
__global__ __launch_bounds__(kThreads) void aux_kernel(const KParams p) {
  const Slice sl = wave_slice(p);
  if (head_is_int8(p, sl.h))
    aux_quant_head<OP, SR, DK, 8, G>(p, sl);
  else
    aux_quant_head<OP, SR, DK, 4, G>(p, sl);
}

template <int OP, int MIXER, int RND, int DK, int G>
__global__ __launch_bounds__((64 * KGeo<DK, G>::NW)) void key_kernel(const KParams p) {
  using K = KGeo<DK, G>;
  __shared__ float lds[K::LG * (K::PARTS + 3) * DK];
  const Slice sl = wave_slice(p);
  if (head_is_int8(p, sl.h))
    key_quant_head<OP, MIXER, RND, DK, 8, G>(p, sl, lds);
  else
    key_quant_head<OP, MIXER, RND, DK, 4, G>(p, sl, lds);
}

template <int OP, int DK, int G>
__global__ __launch_bounds__((64 * KGeo<DK, G>::NW)) void key_aux_kernel(const KParams p) {
  const Slice sl = wave_slice(p);
  if (head_is_int8(p, sl.h))
    key_aux_head<OP, DK, 8, G>(p, sl);
  else
    key_aux_head<OP, DK, 4, G>(p, sl);
}

// FP32-state readout: o = S q.
template <int DK>
__global__ __launch_bounds__(kThreads) void readout_fp32_kernel(const KParams p) {
  constexpr int E = 16, LPR = DK / E, RPW = 64 / LPR;
  const Slice sl = wave_slice(p);
  const int lane = threadIdx.x;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  float qq[E];
  loadv(p.q + (size_t)sl.head * DK + col0, qq);
  const float* hS = reinterpret_cast<const float*>(p.state) + (size_t)sl.head * p.dv * DK;
  for (int rbase = sl.r0; rbase < sl.r1; rbase += RPW) {
    const int row = rbase + rsub;
    float x[E];
    if (row < sl.r1)
      loadv(hS + (size_t)row * DK + col0, x);
    else
#pragma unroll
      for (int j = 0; j < E; ++j) x[j] = 0.0f;
    const float o = row_sum<LPR>(lane_dot(x, qq));
    if (row < sl.r1 && lr == 0) p.o[(size_t)sl.head * p.dv + row] = o;
  }
}

// ---------------------------------------------------------------------------
// Dispatch.
// ---------------------------------------------------------------------------

inline dim3 grid_of(const KParams& p) { return dim3((unsigned)(p.B * p.H * p.slices)); }

template <int DK, int G>
hipError_t launch_quant(Op op, int mixer, int rnd, const KParams& p, hipStream_t s) {
  const dim3 grid = grid_of(p), block(kThreads);
  if (op == kStep) {
#define QS_STEP(M)                                                    \
  if (mixer == M) {                                                   \
    switch (rnd) {                                                    \
      case kRTN: step_kernel<M, kRTN, DK, G><<<grid, block, 0, s>>>(p); break; \
      case kSR: step_kernel<M, kSR, DK, G><<<grid, block, 0, s>>>(p); break;   \
      case kBDR: step_kernel<M, kBDR, DK, G><<<grid, block, 0, s>>>(p); break; \
      default: return hipErrorInvalidValue;                           \
    }                                                                 \
    return hipGetLastError();                                         \
  }
    QS_STEP(kGDN) QS_STEP(kGLA) QS_STEP(kScalar) QS_STEP(kKDA)
#undef QS_STEP
    return hipErrorInvalidValue;
  }
  switch (op) {
    case kImport:  // nothing stored before an import: BDR rounds to nearest
      if (rnd == kSR)
        aux_kernel<kImport, true, DK, G><<<grid, block, 0, s>>>(p);
      else
        aux_kernel<kImport, false, DK, G><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kExport:
      aux_kernel<kExport, false, DK, G><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kReadout:
      aux_kernel<kReadout, false, DK, G><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    default:
      return hipErrorInvalidValue;
  }
}

// Key-axis groups: workgroups of KGeo::NW waves over blocks of KGeo::BR rows.
template <int DK, int G>
hipError_t launch_key(Op op, int mixer, int rnd, const KParams& p, hipStream_t s) {
  using K = KGeo<DK, G>;
  if (p.slice_rows % K::BR != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.B * p.H * p.slices)), block(64 * K::NW);
  switch (op) {
    case kStep:
#define QS_KSTEP(M)                                                                  \
  if (mixer == M) {                                                                  \
    switch (rnd) {                                                                   \
      case kRTN: key_kernel<kStep, M, kRTN, DK, G><<<grid, block, 0, s>>>(p); break; \
      case kSR: key_kernel<kStep, M, kSR, DK, G><<<grid, block, 0, s>>>(p); break;   \
      case kBDR: key_kernel<kStep, M, kBDR, DK, G><<<grid, block, 0, s>>>(p); break; \
      default: return hipErrorInvalidValue;                                          \
    }                                                                                \
    return hipGetLastError();                                                        \
  }
      QS_KSTEP(kGDN) QS_KSTEP(kGLA) QS_KSTEP(kScalar) QS_KSTEP(kKDA)
#undef QS_KSTEP
      return hipErrorInvalidValue;
    case kImport:  // nothing stored before an import: BDR rounds to nearest
      if (rnd == kSR)
        key_kernel<kImport, kGDN, kSR, DK, G><<<grid, block, 0, s>>>(p);
      else
        key_kernel<kImport, kGDN, kRTN, DK, G><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kExport:
      key_aux_kernel<kExport, DK, G><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kReadout:
      key_aux_kernel<kReadout, DK, G><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    default:
      return hipErrorInvalidValue;
  }
}

template <int DK>
hipError_t launch_dk(Op op, int mixer, int rnd, int fp32, const KParams& p, hipStream_t s) {
  const dim3 grid = grid_of(p), block(kThreads);
  if (fp32) {
    if (op == kStep) {
      switch (mixer) {
        case kGDN: step_fp32_kernel<kGDN, DK><<<grid, block, 0, s>>>(p); break;
        case kGLA: step_fp32_kernel<kGLA, DK><<<grid, block, 0, s>>>(p); break;
        case kScalar: step_fp32_kernel<kScalar, DK><<<grid, block, 0, s>>>(p); break;
        case kKDA: step_fp32_kernel<kKDA, DK><<<grid, block, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
    if (op == kReadout) {
      readout_fp32_kernel<DK><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;  // import/export of an FP32 state are plain copies
  }
  if (p.axis == 1) {
    switch (p.G) {
      case 16: return launch_key<DK, 16>(op, mixer, rnd, p, s);
      case 32: return launch_key<DK, 32>(op, mixer, rnd, p, s);
      case 64: return launch_key<DK, 64>(op, mixer, rnd, p, s);
      case 128: return launch_key<DK, 128>(op, mixer, rnd, p, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.slice_rows % 32 != 0) return hipErrorInvalidValue;
  switch (p.G) {
    case 16: return launch_quant<DK, 16>(op, mixer, rnd, p, s);
    case 32: return launch_quant<DK, 32>(op, mixer, rnd, p, s);
    case 64: return launch_quant<DK, 64>(op, mixer, rnd, p, s);
    case 128: return launch_quant<DK, 128>(op, mixer, rnd, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch(Op op, int mixer, int rounding, int fp32, int dk, const KParams& p,
                  hipStream_t stream) {
  if (p.slices < 1 || p.slice_rows < 1 || (int64_t)p.slices * p.slice_rows < p.dv)
    return hipErrorInvalidValue;
  const int rnd = fp32 ? kRTN : rounding;
  const int f = fp32 ? 1 : 0;
  switch (dk) {
    case 64: return launch_dk<64>(op, mixer, rnd, f, p, stream);
    case 128: return launch_dk<128>(op, mixer, rnd, f, p, stream);
    case 256: return launch_dk<256>(op, mixer, rnd, f, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qs
