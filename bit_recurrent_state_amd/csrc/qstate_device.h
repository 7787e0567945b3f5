// qstate_device.h — device helpers shared by the gfx950 decode kernels:
// counter-based random bits, DPP row reductions, the fixed-order dot
// products, group scales, code unpacking/packing and requantization of
// 16-element chunks, per-head geometry.  Included by each kernel source;
// everything here has internal linkage.
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
//  * stochastic rounding needs no float conversion of the random bits: one
//    fma with 1.5*2^23 leaves N = rint(S'*inv*2^f) in the low bits of the
//    result, one integer add of R16 (an SDWA half-word operand) forms
//    N*2^(16-f) + R16, and the code is byte 2 of the sum (sr_word);
//  * round-to-nearest adds 1.5*2^23 inside the fma, which leaves the rounded
//    code in the low byte of the result.

#pragma once

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

// One step of the two 16-bit linear congruential streams of a word, x' =
// (a x + c) mod 2^16 with a = 0xC36D in the low half and 0xC23D in the high
// half, c = 13849 in both: one packed 16-bit multiply-add.
__device__ __forceinline__ uint32_t lcg16x2(uint32_t w) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 a = {0xC36Du, 0xC23Du};
  const u16x2 c = {13849u, 13849u};
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, w) * a + c);
}

// The eight random words of one 16-element block: one hashed seed word and
// seven steps of its linear congruential streams; word p carries R16 of
// element 2p (low half) and of element 2p + 1 (high half).
__device__ __forceinline__ void block_words(uint32_t key, uint32_t block, uint32_t* w) {
  uint32_t x = fmix32(key ^ block);
#pragma unroll
  for (int pr = 0; pr < 8; ++pr) {
    if (pr) x = lcg16x2(x);
    // materialise the word, so that its low half reaches the adds as an SDWA
    // operand rather than through a separate masked copy
    asm("" : "+v"(x));
    w[pr] = x;
  }
}

// R16 of element j of a block from its words.
__device__ __forceinline__ uint32_t r16_of(const uint32_t* w, int j) {
  return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xFFFFu);
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
  if constexpr (LANES >= 16) m = fmaxf(m, dpp<kDppMirror>(m));
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
// for every m (subnormal results included) when r is 7 or 127, and for every
// m >= 2^-100 when r is 448 (exhaustive checks over the mantissas are part of
// the tests); r = 448 keeps the IEEE division below 2^-100.
template <int R>
__device__ __forceinline__ void group_scale(float m, float& s, float& inv) {
  constexpr float r = (float)R;
  constexpr float c = 1.0f / (float)R;
  const float q = m * c;
  s = __builtin_fmaf(__builtin_fmaf(-q, r, m), c, q);
  if constexpr (R != 7 && R != 127)
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

// The rounded products c*s of a lane's E codes (E = 16: four INT8 words;
// E = 32: four INT4 words) with the scales s0 (first 16) and s1 (last 16).
// INT4 takes a shortcut: an offset nibble cu = c + 8 in [0, 15], alone in a
// byte, read as an OCP E4M3 code is exactly cu * 2^-9 (subnormals below 8,
// the lowest normal binade from 8), so one packed FP8 conversion widens two
// elements; fma(cu * 2^-9, s * 2^9, -8 s) has the exact product cu * s, as
// fma(cu, s, -8 s) has (power-of-two scalings are exact for |s| < 2^118).
template <int BITS, int E>
__device__ __forceinline__ void dequant_lane(const uint32_t* w, float s0, float s1, float* d) {
  constexpr float bias = (float)(1 << (BITS - 1));
  const float nb0 = -bias * s0, nb1 = -bias * s1;
  if constexpr (BITS == 8) {
    unpack16<8>(w, d);
#pragma unroll
    for (int j = 0; j < 16; ++j) d[j] = __builtin_fmaf(d[j], s0, nb0);
  } else {
    const float u0 = s0 * 512.0f, u1 = s1 * 512.0f;
#pragma unroll
    for (int q = 0; q < E / 8; ++q) {
      // offset nibbles c + 8 = c ^ 8, each alone in a byte (one bitop3 each)
      const uint32_t lo = (w[q] & 0x0F0F0F0Fu) ^ 0x08080808u;         // elements 8q + 0, 2, 4, 6
      const uint32_t hi = ((w[q] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;  // elements 8q + 1, 3, 5, 7
      const auto e01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
      const auto e23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
      const auto o01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
      const auto o23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
      const float u = 8 * q < 16 ? u0 : u1, nb = 8 * q < 16 ? nb0 : nb1;
      d[8 * q + 0] = __builtin_fmaf(e01[0], u, nb);
      d[8 * q + 1] = __builtin_fmaf(o01[0], u, nb);
      d[8 * q + 2] = __builtin_fmaf(e01[1], u, nb);
      d[8 * q + 3] = __builtin_fmaf(o01[1], u, nb);
      d[8 * q + 4] = __builtin_fmaf(e23[0], u, nb);
      d[8 * q + 5] = __builtin_fmaf(o23[0], u, nb);
      d[8 * q + 6] = __builtin_fmaf(e23[1], u, nb);
      d[8 * q + 7] = __builtin_fmaf(o23[1], u, nb);
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

// Stochastic rounding (semantics in include/qstate.h) of one element whose
// y = fma(S', inv * 2^f, 1.5 * 2^23) has the bits 0x4B400000 + N, N =
// rint(S' * inv * 2^f) (the fma rounds the exact product once, to an integer,
// since |N| <= r 2^f < 2^22).  The result's byte 2 is the code
// floor((N 2^(16-f) + R16) / 2^16): 4-bit codes (f = 16) take bits(y) + R16,
// whose byte 2 carries an extra 0x40 that the nibble drops; 8-bit codes
// (f = 15) take 2 bits(y) + R16 + 2^23, where 2 * 0x4B400000 + 2^23 leaves
// bits 16..23 clear.
template <bool IS8>
__device__ __forceinline__ uint32_t sr_word(float y, uint32_t r16) {
  const uint32_t yb = __float_as_uint(y);
  if constexpr (IS8)
    return yb + (yb + r16) + 0x00800000u;
  else
    return yb + r16;
}

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

// Bounded directional rounding of one element.  y = kMagic + n holds the
// nearest code n of the updated value x, pv the value stored before the step,
// s_new the new scale, r the code range.  Where pv lies strictly between
// n*s_new and x, step one code toward x; then clamp to [-r, r].  (y stays in
// the magic's binade, so +-1 is exact.)
__device__ __forceinline__ float bdr_adjust(float y, float x, float pv, float s_new, float r) {
  const float st = (y - kMagic) * s_new;
  if (x > pv && st < pv) y += 1.0f;
  if (x < pv && st > pv) y -= 1.0f;
  return fminf(fmaxf(y, kMagic - r), kMagic + r);
}

// The same decision without compares, on the bit pattern of y, for the INT4
// lanes of the steps that do not take bdr_step_fast below (measured faster
// there than the compares, which the INT8, key-axis and mixed-width paths
// keep).  With a = pv - x and
// b = n*s_new - pv (signs exact), pv lies strictly between n*s_new and x
// exactly when a and b are nonzero with one sign, the sign opposite to the
// step; med3(a, b, 0) is then the one of them nearer zero, and zero
// otherwise.  Neither a nor b can be -0: pv = c*s_old - 2^(n-1)*s_old is zero
// only by exact cancellation, which rounds to +0, and n*s_new is -0 only for
// n < 0 with s_new = 0, while a zero scale has every n = 0.  So the bit
// pattern of med3's result, read as an integer and clamped to [-1, 1], is
// minus the step, and the codes, bit patterns of floats of one binade, order
// as integers for the final clamp.
__device__ __forceinline__ uint32_t bdr_adjust_bits(uint32_t ybits, float x, float pv, float s_new,
                                                    float r) {
  const float st = (__uint_as_float(ybits) - kMagic) * s_new;
  const float m = __builtin_amdgcn_fmed3f(pv - x, st - pv, 0.0f);
  const int t = min(max(__float_as_int(m), -1), 1);
  const int lo = __float_as_int(kMagic - r), hi = __float_as_int(kMagic + r);
  return (uint32_t)min(max((int)ybits - t, lo), hi);
}

// The same step in fewer instructions (INT4 lanes of the persistent step and
// of the delta-rule window steps): the [-1, 1] clamp is one v_med3_i32 (the
// compiler otherwise folds the negation into a shift, a compare and a
// select), and the final clamp to [-r, r] is left out (CLAMP = false) where
// no group of the wave has an absmax m below 2^-100.  It can only act for
// such m: for m >= 2^-100, RN(r * RN(m / r)) is m or a float neighbour of m
// (every mantissa checked for r = 7 and 127), so no stored value lies
// strictly between the value of code +-r and an |x| <= m, and no step
// leaves [-r, r].
template <bool CLAMP>
__device__ __forceinline__ uint32_t bdr_step_fast(uint32_t ybits, float x, float pv, float s_new,
                                                  float r) {
  const float st = (__uint_as_float(ybits) - kMagic) * s_new;
  const float m = __builtin_amdgcn_fmed3f(pv - x, st - pv, 0.0f);
  int t;
  asm("v_med3_i32 %0, %1, -1, 1" : "=v"(t) : "v"(__float_as_int(m)));
  const int y = (int)ybits - t;
  if constexpr (!CLAMP) return (uint32_t)y;
  const int lo = __float_as_int(kMagic - r), hi = __float_as_int(kMagic + r);
  return (uint32_t)min(max(y, lo), hi);
}

// Requantize one 16-element chunk with inverse scale inv into 16 packed codes
// (four words for INT8, two for INT4).  block: the chunk's 16-element block
// index in the head (stochastic rounding).  wprev / s_old: the chunk's codes
// and scale before the step, s_new its new scale (bounded directional
// rounding).  FAST (INT4 BDR of the persistent and delta-rule window steps):
// bdr_step_fast, with the clamp to [-r, r] only when tiny, i.e. when some
// group of the wave has an absmax below 2^-100 or NaN (wave-uniform).
template <int BITS, int RND, bool FAST = false>
__device__ __forceinline__ void quantize16(const float* sp, float inv, uint32_t key, uint32_t block,
                                           const uint32_t* wprev, float s_old, float s_new,
                                           uint32_t* out, bool tiny = true) {
  uint32_t src[16];
  if constexpr (RND == kSR) {
    constexpr float scale_f = BITS == 8 ? 32768.0f : 65536.0f;  // 2^f
    uint32_t w[8];
    block_words(key, block, w);
    float y[16];
    if (__builtin_expect(inv <= 0x1p100f, 1)) {
      const float inv_f = inv * scale_f;
#pragma unroll
      for (int j = 0; j < 16; ++j) y[j] = __builtin_fmaf(sp[j], inv_f, kMagic);
    } else {  // groups of tiny magnitude, where inv * 2^f could overflow: same exact product
#pragma unroll
      for (int j = 0; j < 16; ++j) y[j] = __builtin_fmaf(sp[j] * scale_f, inv, kMagic);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) src[j] = sr_word<BITS == 8>(y[j], r16_of(w, j));
    pack16<BITS, 2>(src, out);
  } else {
    // y = 1.5*2^23 + rint(S'*inv): the code sits in the low mantissa bits.
#pragma unroll
    for (int j = 0; j < 16; ++j) src[j] = __float_as_uint(__builtin_fmaf(sp[j], inv, kMagic));
    if constexpr (RND == kBDR) {
      // prev = c*s_old exactly as stored
      constexpr float R = (float)((1 << (BITS - 1)) - 1);
      if constexpr (BITS == 4 && FAST) {
        // widened as in dequant_lane, four elements at a time, each four
        // adjusted as soon as they are widened (fewer live registers)
        const float u = s_old * 512.0f, nb = -8.0f * s_old;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          uint32_t wq = wprev[q];
          asm("" : "+v"(wq));
          const uint32_t lo = (wq & 0x0F0F0F0Fu) ^ 0x08080808u;
          const uint32_t hi = ((wq >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const auto e = h ? __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true)
                             : __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
            const auto o = h ? __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true)
                             : __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
            const float pv4[4] = {__builtin_fmaf(e[0], u, nb), __builtin_fmaf(o[0], u, nb),
                                  __builtin_fmaf(e[1], u, nb), __builtin_fmaf(o[1], u, nb)};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = 8 * q + 4 * h + i;
              src[j] = tiny ? bdr_step_fast<true>(src[j], sp[j], pv4[i], s_new, R)
                            : bdr_step_fast<false>(src[j], sp[j], pv4[i], s_new, R);
            }
          }
        }
      } else if constexpr (BITS == 4) {
        // widened as the step's dequantization widens INT4 codes; the words
        // pass through an empty asm so that the widening is redone here
        // rather than kept live from the dequantization (E more registers
        // through the whole update)
        uint32_t wp[2] = {wprev[0], wprev[1]};
        asm("" : "+v"(wp[0]));
        asm("" : "+v"(wp[1]));
        float pv[16];
        dequant_lane<4, 16>(wp, s_old, s_old, pv);
#pragma unroll
        for (int j = 0; j < 16; ++j) src[j] = bdr_adjust_bits(src[j], sp[j], pv[j], s_new, R);
      } else {
        float prev[16];
        unpack16<BITS>(wprev, prev);
        const float nb = -128.0f * s_old;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pv = __builtin_fmaf(prev[j], s_old, nb);
          src[j] = __float_as_uint(bdr_adjust(__uint_as_float(src[j]), sp[j], pv, s_new, R));
        }
      }
    }
    pack16<BITS, 0>(src, out);
  }
}

// Stochastic rounding of 16 elements with one inverse scale per element
// (key-axis groups, per-block widths): word j gets code j in byte 2.  The
// width is 8-bit when is8.
__device__ __forceinline__ void sr16_cols(const float* sp, const float* inv16, uint32_t key,
                                          uint32_t block, bool is8, uint32_t* src) {
  uint32_t w[8];
  block_words(key, block, w);
  const float scale_f = is8 ? 32768.0f : 65536.0f;
  float imax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) imax = fmaxf(imax, inv16[j]);
  float y[16];
  if (__builtin_expect(imax <= 0x1p100f, 1)) {
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = __builtin_fmaf(sp[j], inv16[j] * scale_f, kMagic);
  } else {  // a tiny-magnitude group, where inv * 2^f could overflow: same exact product
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = __builtin_fmaf(sp[j] * scale_f, inv16[j], kMagic);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t r = r16_of(w, j);
    src[j] = is8 ? sr_word<true>(y[j], r) : sr_word<false>(y[j], r);
  }
}

// The same for 16 elements of a lane whose width is chosen at run time, with
// one instruction sequence for both widths: (bits(y) << sh) + (R16 | add)
// (one shift-add and one byte permute), sh = 1 and add = 2^23 for an 8-bit
// lane, 0 and 0 for a 4-bit one: that is 2 bits(y) + R16 + 2^23 and
// bits(y) + R16, the two forms of sr_word, so byte 2 is the code either way
// and lanes of the two widths no longer run both forms and a select.
__device__ __forceinline__ void sr16_rt(const float* sp, const float* inv16, uint32_t key,
                                        uint32_t block, bool is8, uint32_t* src) {
  uint32_t w[8];
  block_words(key, block, w);
  const float scale_f = is8 ? 32768.0f : 65536.0f;
  const uint32_t sh = is8 ? 1u : 0u;
  const uint32_t add = is8 ? 0x00800000u : 0u;
  float imax = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) imax = fmaxf(imax, inv16[j]);
  float y[16];
  if (__builtin_expect(imax <= 0x1p100f, 1)) {
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = __builtin_fmaf(sp[j], inv16[j] * scale_f, kMagic);
  } else {  // a tiny-magnitude group, where inv * 2^f could overflow: same exact product
#pragma unroll
    for (int j = 0; j < 16; ++j) y[j] = __builtin_fmaf(sp[j] * scale_f, inv16[j], kMagic);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    // R16 (the low or high half of the word) with add's byte 2 above it
    const uint32_t r = __builtin_amdgcn_perm(add, w[j >> 1], (j & 1) ? 0x0C060302u : 0x0C060100u);
    src[j] = (__float_as_uint(y[j]) << sh) + r;
  }
}

// Requantize the lane's E elements of the updated row S' into 16 bytes of
// codes.  LPG = 0: two groups per lane (INT4 with G = 16, one per chunk);
// otherwise one group spanning LPG lanes.  s0/s1: the scales of the lane's
// groups (in: before the step, used by bounded directional rounding; out:
// the new ones).  wprev: the lane's four code words before the step.
template <int BITS, int RND, int E, int LPG, bool FAST = false>
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
  bool tiny = true;
  if constexpr (FAST && RND == kBDR && BITS == 4) {
    const float mmin = LPG == 0 ? fminf(m0, m1) : m0;
    tiny = __builtin_amdgcn_ballot_w64(!(mmin >= 0x1p-100f)) != 0;
  }
  uint32_t o[4];
  quantize16<BITS, RND, FAST>(sp, inv0, key, block0, wprev, so0, s0, o, tiny);
  if constexpr (E == 32)
    quantize16<BITS, RND, FAST>(sp + 16, inv1, key, block0 + 1, wprev + 2, so1, s1, o + 2, tiny);
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// Widths chosen per lane at run time (heads with per-channel bits): one
// lane's 16 codes are INT8 (four words) or INT4 (two words).  The rounding
// arithmetic is shared; only widening and packing depend on the width.
// ---------------------------------------------------------------------------

// Offset-binary floats cu = c + 2^(n-1) of 16 codes; INT4 nibbles are first
// widened to bytes in element order, so one set of byte conversions serves
// both widths.
__device__ __forceinline__ void unpack16_rt(const uint32_t* w, bool is8, float* cu) {
  uint32_t b[4];
  if (is8) {
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = w[q] ^ 0x80808080u;
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t x = w[q] ^ 0x88888888u;
      const uint32_t lo = x & 0x0F0F0F0Fu;         // even elements of the word
      const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // odd elements
      b[2 * q] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
      b[2 * q + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int p = 0; p < 4; ++p) cu[4 * q + p] = (float)((b[q] >> (8 * p)) & 0xFFu);
}

// group_scale with r = 127 (INT8) or 7 (INT4) chosen at run time; the same
// operations and constants as group_scale<R>.
__device__ __forceinline__ void group_scale_rt(float m, bool is8, float& s, float& inv) {
  const float r = is8 ? 127.0f : 7.0f;
  const float c = is8 ? 1.0f / 127.0f : 1.0f / 7.0f;
  const float q = m * c;
  s = __builtin_fmaf(__builtin_fmaf(-q, r, m), c, q);
  float v = r / m;
  if (__builtin_fmaf(m, v, -r) > 0.0f) v = __int_as_float(__float_as_int(v) - 1);
  inv = (m == 0.0f) ? 0.0f : v;
}

// Requantize 16 elements; the same rounding as quantize16 with the lane's
// width chosen at run time.  inv16/s_old16/s_new16: one inverse scale and
// old/new scale per element (key-axis groups) or the lane's group values
// repeated (value-axis groups).
template <int RND>
__device__ __forceinline__ void quantize16_rt(const float* sp, const float* inv16, uint32_t key,
                                              uint32_t block, const uint32_t* wprev,
                                              const float* s_old16, const float* s_new16,
                                              bool is8, uint32_t* out) {
  uint32_t src[16];
  if constexpr (RND == kSR) {
    sr16_rt(sp, inv16, key, block, is8, src);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) src[j] = __float_as_uint(__builtin_fmaf(sp[j], inv16[j], kMagic));
    if constexpr (RND == kBDR) {
      const float r = is8 ? 127.0f : 7.0f;
      const float bias = is8 ? 128.0f : 8.0f;
      float prev[16];
      unpack16_rt(wprev, is8, prev);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv = __builtin_fmaf(prev[j], s_old16[j], -bias * s_old16[j]);
        src[j] = __float_as_uint(bdr_adjust(__uint_as_float(src[j]), sp[j], pv, s_new16[j], r));
      }
    }
  }
  constexpr int BP = RND == kSR ? 2 : 0;
  if (is8) {
    pack16<8, BP>(src, out);
  } else {
    pack16<4, BP>(src, out);
    out[2] = out[3] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Per-head geometry.
// ---------------------------------------------------------------------------

// Byte offset of head (b, h): b * bytes_per_b + 8 dv * head_units[h], where
// head_units counts the 8-byte units of the rows of the heads before h.
__device__ __forceinline__ uint64_t head_code_offset(const KParams& p, int b, int h) {
  return (uint64_t)b * p.bytes_per_b + (uint64_t)8 * p.dv * p.head_units[h];
}

template <int N>
__device__ __forceinline__ void loadv(const float* ptr, float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const float4 t = reinterpret_cast<const float4*>(ptr)[q];
    x[4 * q] = t.x, x[4 * q + 1] = t.y, x[4 * q + 2] = t.z, x[4 * q + 3] = t.w;
  }
}

// N floats of a run in LDS whose 16-float blocks are each followed by 4
// floats of padding (run start: column c at c + c / 4).  Lanes that read
// 16- or 32-float runs 64 or 128 bytes apart hit the same LDS banks; with
// 80-byte blocks they spread over the banks (a probe of the unpadded
// pattern read LDS 1.8x slower).
template <int N>
__device__ __forceinline__ void loadv_padded(const float* ptr, float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q) {
    const float4 t = reinterpret_cast<const float4*>(ptr + 4 * q + (q / 4) * 4)[0];
    x[4 * q] = t.x, x[4 * q + 1] = t.y, x[4 * q + 2] = t.z, x[4 * q + 3] = t.w;
  }
}

template <int N>
__device__ __forceinline__ void storev(float* ptr, const float (&x)[N]) {
#pragma unroll
  for (int q = 0; q < N / 4; ++q)
    reinterpret_cast<float4*>(ptr)[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
}

// ---------------------------------------------------------------------------
// Streaming accesses to the quantized state.  A step reads every code once
// and writes it once, from the same lane, and nothing touches it again before
// the next step of the layer; the code loads and stores of the quantized step
// kernels (and the scale loads of the persistent one) therefore carry the
// non-temporal hint (`nt`).  Measured on the chip: 3-15 % less step time,
// but only with loads and stores together (either alone changes nothing);
// the hint on the scale loads of the sliced kernel cost 3 %, and on the FP32
// state step (four 16-byte loads per lane and row) it made the step 1.7x
// slower, so those stay cached.  The hint changes cache policy only, not
// what a later kernel reads.
// ---------------------------------------------------------------------------

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
  const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ float ld_stream(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
  const u32x4_t x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_stream(uint2* p, uint2 v) {
  const u32x2_t x = {v.x, v.y};
  __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void st_stream(float* p, float v) { __builtin_nontemporal_store(v, p); }

// The wave's head and row slice [r0, r1).
struct Slice {
  int head, b, h, r0, r1;
};

// The launch's workgroups are handed to the chip's 8 XCDs round-robin
// (workgroup i to XCD i % 8).  In plain (b, h) order with H a multiple of 8,
// head h of every batch row would land on XCD h % 8, and heads of different
// widths (different costs) would load the XCDs unevenly.  Batch row b
// therefore takes its heads rotated by b: workgroup position h0 in the row
// runs head (h0 + b) mod H, so every XCD sees every head index, while the
// workgroups in flight still cover one contiguous stretch of the state (the
// HBM access pattern of the plain order).
__device__ __forceinline__ Slice wave_slice(const KParams& p) {
  Slice sl;
  const int pos = blockIdx.x / p.slices;
  const int part = blockIdx.x - pos * p.slices;
  sl.b = pos / p.H;
  const int h0 = pos - sl.b * p.H;
  sl.h = (int)(((unsigned)h0 + (unsigned)sl.b) % (unsigned)p.H);
  sl.head = sl.b * p.H + sl.h;
  sl.r0 = part * p.slice_rows;
  sl.r1 = min(p.dv, sl.r0 + p.slice_rows);
  return sl;
}

}  // namespace
}  // namespace qs
