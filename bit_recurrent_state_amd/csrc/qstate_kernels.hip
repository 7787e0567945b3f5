// qstate_kernels.hip — fused quantized recurrent-state decode kernels, gfx950.
//
// One workgroup (4 x wave64) owns one head (b, h).  A value row of the state
// is split into 16-element chunks, one per lane, so a row of dk columns spans
// LPR = dk/16 adjacent lanes and a wave holds 64/LPR rows at a time.  Every
// operation of the step is row-local (LoReS blog, "LoReS: State
// Quantization": value-axis groups, full-precision update, readout from the
// updated state): the two dot products u = d.k and o = S'.q finish with an
// xor butterfly over the row's lanes, and the group absmax with a butterfly
// over the G/16 lanes of the group.  No LDS, no atomics, no cross-workgroup
// traffic: each state byte is read once and written once per step.
//
// Arithmetic follows the semantics written in include/qstate.h operation by
// operation (explicit fmaf, no contraction, IEEE division), so the stored
// codes are bit-identical to any other implementation of those semantics.
// The per-lane 16-element chunk and the butterfly realise the summation
// order defined there: sequential fused multiply-adds inside a chunk, then a
// pairwise tree over chunks (xor 1, 2, 4, ... pairs adjacent partials).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qstate_launch.h"

namespace qs {
namespace {

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kChunk = 16;     // row elements per lane
constexpr int kBatch = 4;      // row iterations whose loads are in flight together

constexpr int kGDN = 0, kGLA = 1, kScalar = 2;

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

// The 16 stochastic-rounding uniforms of one lane's chunk: the chunk is
// exactly one 16-element block of the head, so one hashed seed and a walk of
// seven xorshift32 steps give its eight 32-bit words.
__device__ __forceinline__ void chunk_uniforms(uint32_t key, uint32_t block, float (&u)[kChunk]) {
  uint32_t w = fmix32(key ^ block);
  w = w > 1u ? w : 1u;
#pragma unroll
  for (int pr = 0; pr < kChunk / 2; ++pr) {
    if (pr) w = xorshift32(w);
    u[2 * pr] = (float)(w & 0xFFFFu) * (1.0f / 65536.0f);
    u[2 * pr + 1] = (float)(w >> 16) * (1.0f / 65536.0f);
  }
}

// ---------------------------------------------------------------------------
// Cross-lane reductions inside a row / a group (wave64 xor butterflies).
// ---------------------------------------------------------------------------

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) x = x + __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float group_max(float m, int lanes_per_group) {
  for (int off = 1; off < lanes_per_group; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  return m;
}

// Sequential fused dot product of one 16-element chunk, from +0.
__device__ __forceinline__ float chunk_dot(const float (&x)[kChunk], const float (&y)[kChunk]) {
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kChunk; ++j) acc = __builtin_fmaf(x[j], y[j], acc);
  return acc;
}

// ---------------------------------------------------------------------------
// Scale of a group: s = m / r; inv = r / m rounded toward zero (the largest
// float with inv * m <= r); an all-zero group gets s = inv = 0.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void group_scale(float m, float r, float& s, float& inv) {
  s = m / r;
  float v = r / m;
  if (__builtin_fmaf(m, v, -r) > 0.0f) v = __int_as_float(__float_as_int(v) - 1);
  inv = (m == 0.0f) ? 0.0f : v;
}

// ---------------------------------------------------------------------------
// Code chunks: INT8 = 16 bytes (4 dwords), INT4 = 8 bytes (2 dwords, even
// element in the low nibble).  Codes are two's complement.
// ---------------------------------------------------------------------------

template <int BITS>
struct Codes {
  uint32_t w[BITS / 2];
};

template <int BITS>
__device__ __forceinline__ Codes<BITS> load_codes(const uint8_t* ptr) {
  Codes<BITS> c;
  if constexpr (BITS == 8) {
    const uint4 t = *reinterpret_cast<const uint4*>(ptr);
    c.w[0] = t.x, c.w[1] = t.y, c.w[2] = t.z, c.w[3] = t.w;
  } else {
    const uint2 t = *reinterpret_cast<const uint2*>(ptr);
    c.w[0] = t.x, c.w[1] = t.y;
  }
  return c;
}

template <int BITS>
__device__ __forceinline__ void store_codes(uint8_t* ptr, const Codes<BITS>& c) {
  if constexpr (BITS == 8) {
    *reinterpret_cast<uint4*>(ptr) = make_uint4(c.w[0], c.w[1], c.w[2], c.w[3]);
  } else {
    *reinterpret_cast<uint2*>(ptr) = make_uint2(c.w[0], c.w[1]);
  }
}

template <int BITS>
__device__ __forceinline__ void unpack(const Codes<BITS>& c, float (&x)[kChunk]) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int p = 0; p < 4; ++p) x[4 * q + p] = (float)(int32_t)(int8_t)(c.w[q] >> (8 * p));
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int p = 0; p < 8; ++p)
        x[8 * q + p] = (float)(((int32_t)(c.w[q] << (28 - 4 * p))) >> 28);
  }
}

template <int BITS>
__device__ __forceinline__ Codes<BITS> pack(const int32_t (&n)[kChunk]) {
  Codes<BITS> c;
  if constexpr (BITS == 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      c.w[q] = (uint32_t)(n[4 * q] & 0xFF) | ((uint32_t)(n[4 * q + 1] & 0xFF) << 8) |
               ((uint32_t)(n[4 * q + 2] & 0xFF) << 16) | ((uint32_t)(n[4 * q + 3] & 0xFF) << 24);
  } else {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t w = 0;
#pragma unroll
      for (int p = 0; p < 8; ++p) w |= (uint32_t)(n[8 * q + p] & 0xF) << (4 * p);
      c.w[q] = w;
    }
  }
  return c;
}

// Requantize one lane's chunk of the updated row S' (value-axis group of the
// chunk; the group spans lanes_per_group lanes).  Returns the scale s'.
template <int BITS, bool SR>
__device__ __forceinline__ float quantize_chunk(const float (&sp)[kChunk], int lanes_per_group,
                                                uint32_t key, uint32_t block,
                                                int32_t (&n)[kChunk]) {
  constexpr float r = (float)((1 << (BITS - 1)) - 1);
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < kChunk; ++j) m = fmaxf(m, fabsf(sp[j]));
  m = group_max(m, lanes_per_group);
  float s, inv;
  group_scale(m, r, s, inv);
  if constexpr (SR) {
    float u[kChunk];
    chunk_uniforms(key, block, u);
#pragma unroll
    for (int j = 0; j < kChunk; ++j) n[j] = (int32_t)floorf(__builtin_fmaf(sp[j], inv, u[j]));
  } else {
    // round-half-even of the exact product: adding 1.5*2^23 inside the fma
    // leaves rint(sp*inv) in the low mantissa bits (|sp*inv| <= r).
#pragma unroll
    for (int j = 0; j < kChunk; ++j)
      n[j] = __float_as_int(__builtin_fmaf(sp[j], inv, 12582912.0f)) - 0x4B400000;
  }
  return s;
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

__device__ __forceinline__ void load16(const float* ptr, float (&x)[kChunk]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 t = reinterpret_cast<const float4*>(ptr)[q];
    x[4 * q] = t.x, x[4 * q + 1] = t.y, x[4 * q + 2] = t.z, x[4 * q + 3] = t.w;
  }
}

__device__ __forceinline__ void store16(float* ptr, const float (&x)[kChunk]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    reinterpret_cast<float4*>(ptr)[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
}

// Per-lane view of one head.
struct Lane {
  int b, h, head;  // head = b*H + h
  int lr;          // chunk index inside the row (lane % LPR)
  int rsub;        // row offset inside one workgroup iteration
  int col0;        // first column of the chunk
};

// ---------------------------------------------------------------------------
// The decode step on a quantized head of BITS-bit codes.
// ---------------------------------------------------------------------------

template <int MIXER, bool SR, int LPR, int BITS>
__device__ __forceinline__ void step_quant_head(const KParams& p, const Lane& L, uint8_t* hcodes,
                                                float* hscales, const float (&kk)[kChunk],
                                                const float (&qq)[kChunk], const float (&al)[kChunk],
                                                float alpha_s, float beta, uint32_t key) {
  constexpr int DK = LPR * kChunk;
  constexpr int RPI = (kThreads / 64) * (64 / LPR);
  constexpr int ROW_BYTES = DK * BITS / 8;
  constexpr int CHUNK_BYTES = kChunk * BITS / 8;
  const int lpg = p.G / kChunk;
  const int ng = DK / p.G;
  const int n_it = (p.dv + RPI - 1) / RPI;
  const float* vh = p.v + (size_t)L.head * p.dv;
  float* oh = p.o ? p.o + (size_t)L.head * p.dv : nullptr;

  for (int it0 = 0; it0 < n_it; it0 += kBatch) {
    Codes<BITS> raw[kBatch];
    float sc[kBatch], vi[kBatch];
#pragma unroll
    for (int n = 0; n < kBatch; ++n) {
      const int row = (it0 + n) * RPI + L.rsub;
      if (row < p.dv) {
        raw[n] = load_codes<BITS>(hcodes + (size_t)row * ROW_BYTES + L.lr * CHUNK_BYTES);
        sc[n] = hscales[(size_t)row * ng + L.col0 / p.G];
        vi[n] = vh[row];
      } else {
#pragma unroll
        for (int q = 0; q < BITS / 2; ++q) raw[n].w[q] = 0u;
        sc[n] = 0.0f;
        vi[n] = 0.0f;
      }
    }
#pragma unroll
    for (int n = 0; n < kBatch; ++n) {
      const int row = (it0 + n) * RPI + L.rsub;
      float c[kChunk], d[kChunk];
      unpack<BITS>(raw[n], c);
      // decayed dequantized chunk
      if constexpr (MIXER == kGLA) {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) d[j] = (c[j] * sc[n]) * al[j];
      } else {
        const float sa = sc[n] * alpha_s;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) d[j] = c[j] * sa;
      }
      // write weight
      float w;
      if constexpr (MIXER == kGDN) {
        const float u = row_sum<LPR>(chunk_dot(d, kk));
        w = beta * (vi[n] - u);
      } else if constexpr (MIXER == kGLA) {
        w = vi[n];
      } else {
        w = beta * vi[n];
      }
      // rank-1 write and readout from the full-precision S'
      float sp[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) sp[j] = __builtin_fmaf(w, kk[j], d[j]);
      const float o = row_sum<LPR>(chunk_dot(sp, qq));
      // requantize
      int32_t code[kChunk];
      const uint32_t block = (uint32_t)row * LPR + (uint32_t)L.lr;
      const float s_new = quantize_chunk<BITS, SR>(sp, lpg, key, block, code);
      if (row < p.dv) {
        store_codes<BITS>(hcodes + (size_t)row * ROW_BYTES + L.lr * CHUNK_BYTES, pack<BITS>(code));
        if (L.lr % lpg == 0) hscales[(size_t)row * ng + L.col0 / p.G] = s_new;
        if (oh && L.lr == 0) oh[row] = o;
      }
    }
  }
}

// The same step on an unquantized FP32 head.
template <int MIXER, int LPR>
__device__ __forceinline__ void step_fp32_head(const KParams& p, const Lane& L, float* hS,
                                               const float (&kk)[kChunk], const float (&qq)[kChunk],
                                               const float (&al)[kChunk], float alpha_s, float beta) {
  constexpr int DK = LPR * kChunk;
  constexpr int RPI = (kThreads / 64) * (64 / LPR);
  const int n_it = (p.dv + RPI - 1) / RPI;
  const float* vh = p.v + (size_t)L.head * p.dv;
  float* oh = p.o ? p.o + (size_t)L.head * p.dv : nullptr;
  for (int it0 = 0; it0 < n_it; it0 += kBatch) {
    float x[kBatch][kChunk], vi[kBatch];
#pragma unroll
    for (int n = 0; n < kBatch; ++n) {
      const int row = (it0 + n) * RPI + L.rsub;
      if (row < p.dv) {
        load16(hS + (size_t)row * DK + L.col0, x[n]);
        vi[n] = vh[row];
      } else {
#pragma unroll
        for (int j = 0; j < kChunk; ++j) x[n][j] = 0.0f;
        vi[n] = 0.0f;
      }
    }
#pragma unroll
    for (int n = 0; n < kBatch; ++n) {
      const int row = (it0 + n) * RPI + L.rsub;
      float d[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) d[j] = x[n][j] * (MIXER == kGLA ? al[j] : alpha_s);
      float w;
      if constexpr (MIXER == kGDN) {
        const float u = row_sum<LPR>(chunk_dot(d, kk));
        w = beta * (vi[n] - u);
      } else if constexpr (MIXER == kGLA) {
        w = vi[n];
      } else {
        w = beta * vi[n];
      }
      float sp[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) sp[j] = __builtin_fmaf(w, kk[j], d[j]);
      const float o = row_sum<LPR>(chunk_dot(sp, qq));
      if (row < p.dv) {
        store16(hS + (size_t)row * DK + L.col0, sp);
        if (oh && L.lr == 0) oh[row] = o;
      }
    }
  }
}

// Import (quantize an FP32 state), export (dequantize) and readout of a
// quantized head.
template <int OP, bool SR, int LPR, int BITS>
__device__ __forceinline__ void aux_quant_head(const KParams& p, const Lane& L, uint8_t* hcodes,
                                               float* hscales, const float (&qq)[kChunk],
                                               uint32_t key) {
  constexpr int DK = LPR * kChunk;
  constexpr int RPI = (kThreads / 64) * (64 / LPR);
  constexpr int ROW_BYTES = DK * BITS / 8;
  constexpr int CHUNK_BYTES = kChunk * BITS / 8;
  const int lpg = p.G / kChunk;
  const int ng = DK / p.G;
  const size_t hoff = (size_t)L.head * p.dv * DK;
  for (int it = 0; it * RPI < p.dv; ++it) {
    const int row = it * RPI + L.rsub;
    const bool ok = row < p.dv;
    if constexpr (OP == kImport) {
      float x[kChunk];
      if (ok)
        load16(p.src + hoff + (size_t)row * DK + L.col0, x);
      else
#pragma unroll
        for (int j = 0; j < kChunk; ++j) x[j] = 0.0f;
      int32_t code[kChunk];
      const uint32_t block = (uint32_t)row * LPR + (uint32_t)L.lr;
      const float s_new = quantize_chunk<BITS, SR>(x, lpg, key, block, code);
      if (ok) {
        store_codes<BITS>(hcodes + (size_t)row * ROW_BYTES + L.lr * CHUNK_BYTES, pack<BITS>(code));
        if (L.lr % lpg == 0) hscales[(size_t)row * ng + L.col0 / p.G] = s_new;
      }
    } else {
      Codes<BITS> raw;
      float s = 0.0f;
      if (ok) {
        raw = load_codes<BITS>(hcodes + (size_t)row * ROW_BYTES + L.lr * CHUNK_BYTES);
        s = hscales[(size_t)row * ng + L.col0 / p.G];
      } else {
#pragma unroll
        for (int q = 0; q < BITS / 2; ++q) raw.w[q] = 0u;
      }
      float c[kChunk], x[kChunk];
      unpack<BITS>(raw, c);
#pragma unroll
      for (int j = 0; j < kChunk; ++j) x[j] = c[j] * s;
      if constexpr (OP == kExport) {
        if (ok) store16(p.dst + hoff + (size_t)row * DK + L.col0, x);
      } else {
        const float o = row_sum<LPR>(chunk_dot(x, qq));
        if (ok && L.lr == 0) p.o[(size_t)L.head * p.dv + row] = o;
      }
    }
  }
}

template <int LPR>
__device__ __forceinline__ Lane make_lane(const KParams& p) {
  Lane L;
  L.head = blockIdx.x;
  L.b = L.head / p.H;
  L.h = L.head - L.b * p.H;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  L.lr = lane % LPR;
  L.rsub = wave * (64 / LPR) + lane / LPR;
  L.col0 = L.lr * kChunk;
  return L;
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------

template <int MIXER, bool SR, bool FP32, int LPR>
__global__ __launch_bounds__(kThreads) void step_kernel(const KParams p) {
  constexpr int DK = LPR * kChunk;
  const Lane L = make_lane<LPR>(p);
  float kk[kChunk], qq[kChunk], al[kChunk];
  load16(p.k + (size_t)L.head * DK + L.col0, kk);
  load16(p.q + (size_t)L.head * DK + L.col0, qq);
  float alpha_s = 0.0f, beta = 0.0f;
  if constexpr (MIXER == kGLA) {
    load16(p.alpha + (size_t)L.head * DK + L.col0, al);
  } else {
#pragma unroll
    for (int j = 0; j < kChunk; ++j) al[j] = 0.0f;
    alpha_s = p.alpha[L.head];
    beta = p.beta[L.head];
  }
  if constexpr (FP32) {
    float* hS = reinterpret_cast<float*>(p.state) + (size_t)L.head * p.dv * DK;
    step_fp32_head<MIXER, LPR>(p, L, hS, kk, qq, al, alpha_s, beta);
  } else {
    uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, L.b, L.h);
    float* hscales = p.scales + (size_t)L.head * p.dv * (DK / p.G);
    const uint32_t key = SR ? head_key(p, (uint32_t)L.b, (uint32_t)L.h) : 0u;
    if (head_is_int8(p, L.h))
      step_quant_head<MIXER, SR, LPR, 8>(p, L, hcodes, hscales, kk, qq, al, alpha_s, beta, key);
    else
      step_quant_head<MIXER, SR, LPR, 4>(p, L, hcodes, hscales, kk, qq, al, alpha_s, beta, key);
  }
}

template <int OP, bool SR, int LPR>
__global__ __launch_bounds__(kThreads) void aux_kernel(const KParams p) {
  constexpr int DK = LPR * kChunk;
  const Lane L = make_lane<LPR>(p);
  float qq[kChunk];
  if constexpr (OP == kReadout)
    load16(p.q + (size_t)L.head * DK + L.col0, qq);
  else
#pragma unroll
    for (int j = 0; j < kChunk; ++j) qq[j] = 0.0f;
  uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, L.b, L.h);
  float* hscales = p.scales + (size_t)L.head * p.dv * (DK / p.G);
  const uint32_t key = (OP == kImport && SR) ? head_key(p, (uint32_t)L.b, (uint32_t)L.h) : 0u;
  if (head_is_int8(p, L.h))
    aux_quant_head<OP, SR, LPR, 8>(p, L, hcodes, hscales, qq, key);
  else
    aux_quant_head<OP, SR, LPR, 4>(p, L, hcodes, hscales, qq, key);
}

// FP32-state readout: o = S q.
template <int LPR>
__global__ __launch_bounds__(kThreads) void readout_fp32_kernel(const KParams p) {
  constexpr int DK = LPR * kChunk;
  constexpr int RPI = (kThreads / 64) * (64 / LPR);
  const Lane L = make_lane<LPR>(p);
  float qq[kChunk];
  load16(p.q + (size_t)L.head * DK + L.col0, qq);
  const float* hS = reinterpret_cast<const float*>(p.state) + (size_t)L.head * p.dv * DK;
  for (int it = 0; it * RPI < p.dv; ++it) {
    const int row = it * RPI + L.rsub;
    float x[kChunk];
    if (row < p.dv)
      load16(hS + (size_t)row * DK + L.col0, x);
    else
#pragma unroll
      for (int j = 0; j < kChunk; ++j) x[j] = 0.0f;
    const float o = row_sum<LPR>(chunk_dot(x, qq));
    if (row < p.dv && L.lr == 0) p.o[(size_t)L.head * p.dv + row] = o;
  }
}

// ---------------------------------------------------------------------------
// Dispatch.
// ---------------------------------------------------------------------------

template <int LPR>
hipError_t launch_lpr(Op op, int mixer, int sr, int fp32, const KParams& p, hipStream_t s) {
  const dim3 grid((unsigned)(p.B * p.H)), block(kThreads);
  if (op == kStep) {
#define QS_STEP(M, S, F) \
  if (mixer == M && sr == S && fp32 == F) { step_kernel<M, S, F, LPR><<<grid, block, 0, s>>>(p); return hipGetLastError(); }
    QS_STEP(kGDN, false, false) QS_STEP(kGDN, true, false) QS_STEP(kGLA, false, false)
    QS_STEP(kGLA, true, false) QS_STEP(kScalar, false, false) QS_STEP(kScalar, true, false)
    QS_STEP(kGDN, false, true) QS_STEP(kGLA, false, true) QS_STEP(kScalar, false, true)
#undef QS_STEP
    return hipErrorInvalidValue;
  }
  if (fp32) {
    if (op == kReadout) {
      readout_fp32_kernel<LPR><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;  // import/export of an FP32 state are plain copies
  }
  switch (op) {
    case kImport:
      if (sr) aux_kernel<kImport, true, LPR><<<grid, block, 0, s>>>(p);
      else aux_kernel<kImport, false, LPR><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kExport:
      aux_kernel<kExport, false, LPR><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kReadout:
      aux_kernel<kReadout, false, LPR><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch(Op op, int mixer, int rounding, int fp32, int dk, const KParams& p,
                  hipStream_t stream) {
  const int sr = (rounding == 1 && !fp32) ? 1 : 0;
  const int f = fp32 ? 1 : 0;
  switch (dk) {
    case 64: return launch_lpr<4>(op, mixer, sr, f, p, stream);
    case 128: return launch_lpr<8>(op, mixer, sr, f, p, stream);
    case 256: return launch_lpr<16>(op, mixer, sr, f, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qs
