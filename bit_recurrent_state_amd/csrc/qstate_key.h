// qstate_key.h — key-axis decode kernels (scale groups of G value rows
// inside one key column), templated on dk.  Each qstate_key_dk*.hip
// instantiates one dk.

#pragma once

#include "qstate_device.h"

namespace qs {
namespace {

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
    sr16_cols(sp, inv16, key, block, BITS == 8, src);
    pack16<BITS, 2>(src, out);
  } else {
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
        src[j] = __float_as_uint(bdr_adjust(__uint_as_float(src[j]), sp[j], pv, s_new[j], (float)R));
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

// Code placement of a lane's 16-column block in a row.  BITS = 8 or 4: a
// head of one width (compile-time); BITS = 0: widths per block from the
// head's INT8-block mask, a row holding 16 bytes per INT8 block and 8 per
// INT4 block in column order.
template <int DK, int BITS>
struct LaneCodes {
  bool is8;        // this lane's block stores INT8 codes
  int row_bytes;   // bytes of one row of the head
  int lane_off;    // byte offset of the lane's block inside a row
  __device__ __forceinline__ LaneCodes(uint32_t mask, int lr) {
    constexpr int LPR = DK / 16;
    if constexpr (BITS != 0) {
      is8 = BITS == 8;
      row_bytes = DK * BITS / 8;
      lane_off = lr * 2 * BITS;
    } else {
      is8 = (mask >> lr) & 1u;
      row_bytes = 8 * (LPR + __popc(mask));
      lane_off = 8 * (lr + __popc(mask & ((1u << lr) - 1u)));
    }
  }
};

// Step (OP = kStep) or import (OP = kImport) of a quantized head with
// key-axis groups.  LDS: partial column maxima, old scales, new scales and
// inverse scales of the block's row groups, and the head's vectors.  BITS =
// 0: mixed widths.
template <int OP, int MIXER, int RND, int DK, int BITS, int G, bool PF>
__device__ __forceinline__ void key_quant_head(const KParams& p, const Slice sl, float* lds) {
  using K = KGeo<DK, G>;
  constexpr int E = K::E, LPR = K::LPR, RPW = K::RPW, NI = K::NI, RB = K::RB, NW = K::NW;
  constexpr int BR = K::BR, LG = K::LG, PARTS = K::PARTS;
  const uint32_t mask = p.int8_blocks[sl.h];
  // Every LDS vector is padded to PDK floats, 4 after every 16 (column j at
  // j + j / 16 * 4): the lanes of a row read 16-float runs, which would
  // otherwise start 64 bytes apart and share LDS banks.
  constexpr int PDK = DK + DK / 4;
  float* pm = lds;                        // [LG][PARTS][PDK]
  float* so = pm + LG * PARTS * PDK;      // [LG][PDK] scales before the step
  float* sn = so + LG * PDK;              // [LG][PDK] new scales
  float* si = sn + LG * PDK;              // [LG][PDK] new inverse scales
  float* skq = si + LG * PDK;             // [3][PDK] the head's k, q, alpha (PF)

  const int tid = threadIdx.x;
  const int wv = tid / 64;
  const int lane = tid % 64;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  const int pcol0 = col0 + col0 / 4;  // the lane's run in the padded LDS vectors
  const LaneCodes<DK, BITS> lc(mask, lr);
  const float bias = lc.is8 ? 128.0f : 8.0f;
  uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
  float* hscales = p.scales + (size_t)sl.head * (p.dv / G) * DK;
  const uint32_t key =
      (RND == kSR) ? head_key(p, (uint32_t)sl.b, (uint32_t)sl.h) : 0u;

  // PF (a step; see key_prefetch): the head's k, q and alpha go to LDS and
  // are read there in every row iteration instead of being held in 2-3 x E
  // registers per lane, and the freed registers hold the next block's codes,
  // loaded while this block computes.  Otherwise the vectors stay in
  // registers and each block is loaded when it starts.  The block loop's
  // first barrier publishes the vectors.
  static_assert(!PF || OP == kStep, "prefetch is a step layout");
  float kk[E], qq[E], al[E];
  float alpha_s = 0.0f, beta = 0.0f;
  const float* vh = nullptr;
  float* oh = nullptr;
  if constexpr (OP == kStep) {
    if constexpr (PF) {
      constexpr int NV = vector_decay(MIXER) ? 3 : 2;
      const float* src3[3] = {p.k + (size_t)sl.head * DK, p.q + (size_t)sl.head * DK,
                              vector_decay(MIXER) ? p.alpha + (size_t)sl.head * DK : nullptr};
#pragma unroll
      for (int vi = 0; vi < NV; ++vi)
        for (int f = tid; f < DK / 4; f += 64 * NW)
          reinterpret_cast<float4*>(skq + vi * PDK)[f + f / 4] =
              reinterpret_cast<const float4*>(src3[vi])[f];
    } else {
      loadv(p.k + (size_t)sl.head * DK + col0, kk);
      loadv(p.q + (size_t)sl.head * DK + col0, qq);
      if constexpr (vector_decay(MIXER)) loadv(p.alpha + (size_t)sl.head * DK + col0, al);
    }
    if constexpr (!vector_decay(MIXER)) {
#pragma unroll
      for (int j = 0; j < E; ++j) al[j] = 0.0f;
      alpha_s = p.alpha[sl.head];
    }
    if constexpr (MIXER != kGLA) beta = p.beta[sl.head];
    vh = p.v + (size_t)sl.head * p.dv;
    oh = p.o ? p.o + (size_t)sl.head * p.dv : nullptr;
  }

  // This wave's rows of a block: base + wv*RB + it*RPW + rsub; every row of
  // an iteration lies in one row group, and a group is wholly inside dv or
  // wholly outside (G divides dv, RPW divides G).
  // (standin: every load from the slice's first row instead, a stand-in that
  // costs one cache line per lane group)
  auto load_block = [&](int base_, bool standin, uint32_t (&w_)[NI][4], float (&v_)[NI]) {
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int row = standin ? sl.r0 : min(base_ + wv * RB + it * RPW + rsub, p.dv - 1);
      const uint8_t* src = hcodes + (size_t)row * lc.row_bytes + lc.lane_off;
      if (lc.is8) {
        const uint4 t = ld_stream(reinterpret_cast<const uint4*>(src));
        w_[it][0] = t.x, w_[it][1] = t.y, w_[it][2] = t.z, w_[it][3] = t.w;
      } else {
        const uint2 t = ld_stream(reinterpret_cast<const uint2*>(src));
        w_[it][0] = t.x, w_[it][1] = t.y, w_[it][2] = 0u, w_[it][3] = 0u;
      }
      v_[it] = vh[row];
    }
  };
  // PFS: the old scales of a block's row groups are loaded with its codes,
  // one block ahead, NSO per thread (in-bounds stand-ins past the slice,
  // stored as zeros), so the block does not wait on them before its first
  // barrier.  KDA, at its register bound, issues them later instead, before
  // the block's requantization (PFL, groups of 64 rows: with 32 or 128
  // it spills), where fewer registers are live.
  constexpr bool PFS = PF && MIXER != kKDA;
  constexpr bool PFL = PF && !PFS && G == 64;
  constexpr int NSO = (LG * DK + 64 * NW - 1) / (64 * NW);
  auto load_scales = [&](int base_, float (&sv)[NSO]) {
#pragma unroll
    for (int i = 0; i < NSO; ++i) {
      const int t = tid + i * 64 * NW;
      const int grow = base_ / G + t / DK, j = t % DK;
      const bool ok = t < LG * DK && base_ < sl.r1 && grow * G < p.dv;
      const float x = hscales[ok ? (size_t)grow * DK + j : (size_t)j];
      sv[i] = ok ? x : 0.0f;
    }
  };
  float son[NSO];
  uint32_t wc[NI][4] = {};
  float vr[NI] = {};
  if constexpr (PF) load_block(sl.r0, false, wc, vr);
  if constexpr (PFS || PFL) load_scales(sl.r0, son);
  for (int base = sl.r0; base < sl.r1; base += BR) {
    // without PF this block's codes and v, issued before its old scales so
    // that the two loads' latencies overlap
    if constexpr (OP == kStep && !PF) load_block(base, false, wc, vr);
    // scales of the block's row groups before the step
    if constexpr (OP == kStep && (PFS || PFL)) {
#pragma unroll
      for (int i = 0; i < NSO; ++i) {
        const int t = tid + i * 64 * NW, j = t % DK;
        if (t < LG * DK) so[(t / DK) * PDK + j + j / 16 * 4] = son[i];
      }
    } else if constexpr (OP == kStep) {
      for (int t = tid; t < LG * DK; t += 64 * NW) {
        const int grow = base / G + t / DK;
        const int j = t % DK;
        so[(t / DK) * PDK + j + j / 16 * 4] = grow * G < p.dv ? hscales[(size_t)grow * DK + j] : 0.0f;
      }
    }
    // PF: the next block's codes and v (issued unconditionally, so that the
    // waits on this block's loads stay exact: after the last block a
    // stand-in that is never used)
    uint32_t wn[NI][4] = {};
    float vn[NI] = {};
    if constexpr (PF) {
      load_block(base + BR, base + BR >= sl.r1, wn, vn);
      if constexpr (PFS) load_scales(base + BR, son);
    }
    float sp[NI][E];
    if constexpr (OP == kImport) {
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int row = min(base + wv * RB + it * RPW + rsub, p.dv - 1);
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
        if constexpr (PF) {
          asm volatile("" ::: "memory");  // the head's vectors from LDS here, not held
          lds_load(skq + pcol0, kk);
          lds_load(skq + PDK + pcol0, qq);
          if constexpr (vector_decay(MIXER)) lds_load(skq + 2 * PDK + pcol0, al);
        }
        float sc[E];
        lds_load(so + lg * PDK + pcol0, sc);
        float d[E];
        if constexpr (BITS != 0)
          unpack16<BITS>(wc[it], d);
        else
          unpack16_rt(wc[it], lc.is8, d);
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
        float* dst = pm + ((size_t)lg * PARTS + wv * RPW + rsub) * PDK + pcol0;
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
      const int pj = j + j / 16 * 4;
      float m = 0.0f;
#pragma unroll 8
      for (int q = 0; q < PARTS; ++q) m = fmaxf(m, pm[((size_t)lg * PARTS + q) * PDK + pj]);
      float s, inv;
      if constexpr (BITS != 0)
        group_scale<(1 << (BITS - 1)) - 1>(m, s, inv);
      else
        group_scale_rt(m, (mask >> (j / 16)) & 1u, s, inv);
      sn[lg * PDK + pj] = s;
      si[lg * PDK + pj] = inv;
      const int grow = base / G + lg;
      if (grow * G < p.dv) st_stream(hscales + (size_t)grow * DK + j, s);
    }
    __syncthreads();  // new scales in LDS

    if constexpr (PFL) load_scales(base + BR, son);
    // requantize and store
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int lg = (wv * RB + it * RPW) / G;
      const int row = base + wv * RB + it * RPW + rsub;
      float inv16[E], s_old[E], s_new[E];
      lds_load(si + lg * PDK + pcol0, inv16);
      if constexpr (RND == kBDR) {
        lds_load(so + lg * PDK + pcol0, s_old);
        lds_load(sn + lg * PDK + pcol0, s_new);
      }
      uint32_t out[4];
      const uint32_t block = (uint32_t)((row * DK + col0) >> 4);
      constexpr int QR = (OP == kImport && RND == kBDR) ? kRTN : RND;
      if constexpr (BITS != 0)
        quantize16_cols<BITS, QR>(sp[it], inv16, key, block, wc[it], s_old, s_new, out);
      else
        quantize16_rt<QR>(sp[it], inv16, key, block, wc[it], s_old, s_new, lc.is8, out);
      if (row < p.dv) {
        uint8_t* dst = hcodes + (size_t)row * lc.row_bytes + lc.lane_off;
        if (lc.is8)
          st_stream(reinterpret_cast<uint4*>(dst), make_uint4(out[0], out[1], out[2], out[3]));
        else
          st_stream(reinterpret_cast<uint2*>(dst), make_uint2(out[0], out[1]));
      }
    }
    __syncthreads();  // LDS free for the next block
    if constexpr (PF) {
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        vr[it] = vn[it];
#pragma unroll
        for (int q = 0; q < 4; ++q) wc[it][q] = wn[it][q];
      }
    }
  }
}

// Export (dequantize) or readout of a quantized head with key-axis groups.
template <int OP, int DK, int BITS, int G>
__device__ __forceinline__ void key_aux_head(const KParams& p, const Slice sl) {
  using K = KGeo<DK, G>;
  constexpr int E = K::E, LPR = K::LPR, RPW = K::RPW, NW = K::NW;
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int lr = lane % LPR;
  const int col0 = lr * E;
  const LaneCodes<DK, BITS> lc(p.int8_blocks[sl.h], lr);
  const float bias = lc.is8 ? 128.0f : 8.0f;
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
    const uint8_t* src = hcodes + (size_t)rr * lc.row_bytes + lc.lane_off;
    if (lc.is8) {
      const uint4 t = *reinterpret_cast<const uint4*>(src);
      w[0] = t.x, w[1] = t.y, w[2] = t.z, w[3] = t.w;
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(src);
      w[0] = t.x, w[1] = t.y;
    }
    float sc[E], d[E];
    loadv(hscales + (size_t)(rr / G) * DK + col0, sc);
    if constexpr (BITS != 0)
      unpack16<BITS>(w, d);
    else
      unpack16_rt(w, lc.is8, d);
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
// Kernels and dispatch.
// ---------------------------------------------------------------------------

// Heads of one width each.  Three waves per SIMD (at most 168 VGPRs, a few
// spilled by the BDR and SR variants): the workgroup barriers of the column
// reductions need the other waves to fill the SIMD, and measured, three
// waves with spills beat two without by 8-12 %.
// Whether a key-axis step stages the head's vectors in LDS and prefetches
// the next block (measured per variant, same-box A/B): yes for every step
// but two: BDR (slower: it keeps the previous codes through the
// requantization and sits at its register bound) and one-width GLA with
// round to nearest (3 % slower; its INT8 rows already keep enough loads in
// flight).  Gains: mixed widths -16 %, GLA SR -13 %, Gated DeltaNet SR -9 %,
// KDA -7 %.
template <int OP, int MIXER, int RND, bool MIXED>
constexpr bool key_prefetch() {
  return OP == kStep && RND != kBDR && (MIXED || !(MIXER == kGLA && RND == kRTN));
}

template <int OP, int MIXER, int RND, int DK, int G>
__global__ __launch_bounds__((64 * KGeo<DK, G>::NW)) __attribute__((amdgpu_waves_per_eu(3)))
void key_kernel(const KParams p) {
  using K = KGeo<DK, G>;
  constexpr bool PF = key_prefetch<OP, MIXER, RND, false>();
  __shared__ float lds[(K::LG * (K::PARTS + 3) + (PF ? 3 : 0)) * (DK + DK / 4)];
  const Slice sl = wave_slice(p);
  if (p.int8_blocks[sl.h] != 0u)
    key_quant_head<OP, MIXER, RND, DK, 8, G, PF>(p, sl, lds);
  else
    key_quant_head<OP, MIXER, RND, DK, 4, G, PF>(p, sl, lds);
}

// A launch with heads of mixed widths: every head takes the per-block path
// (held to three waves per SIMD, this path would spill heavily).
template <int OP, int MIXER, int RND, int DK, int G>
__global__ __launch_bounds__((64 * KGeo<DK, G>::NW)) void key_mixed_kernel(const KParams p) {
  using K = KGeo<DK, G>;
  constexpr bool PF = key_prefetch<OP, MIXER, RND, true>();
  __shared__ float lds[(K::LG * (K::PARTS + 3) + (PF ? 3 : 0)) * (DK + DK / 4)];
  key_quant_head<OP, MIXER, RND, DK, 0, G, PF>(p, wave_slice(p), lds);
}

template <int OP, int DK, int G>
__global__ __launch_bounds__((64 * KGeo<DK, G>::NW)) void key_aux_kernel(const KParams p) {
  const Slice sl = wave_slice(p);
  const uint32_t m = p.int8_blocks[sl.h];
  if (m == (1u << (DK / 16)) - 1u)
    key_aux_head<OP, DK, 8, G>(p, sl);
  else if (m == 0u)
    key_aux_head<OP, DK, 4, G>(p, sl);
  else
    key_aux_head<OP, DK, 0, G>(p, sl);
}

// FP32-state readout: o = S q.
template <int DK, int G>
hipError_t launch_key(Op op, int mixer, int rnd, const KParams& p, hipStream_t s) {
  using K = KGeo<DK, G>;
  if (p.slice_rows % K::BR != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.B * p.H * p.slices)), block(64 * K::NW);
  switch (op) {
    case kStep:
#define QS_KSTEP(M)                                                                  \
  if (mixer == M) {                                                                  \
    if (p.mixed) {                                                                   \
      switch (rnd) {                                                                 \
        case kRTN: key_mixed_kernel<kStep, M, kRTN, DK, G><<<grid, block, 0, s>>>(p); break; \
        case kSR: key_mixed_kernel<kStep, M, kSR, DK, G><<<grid, block, 0, s>>>(p); break;   \
        case kBDR: key_mixed_kernel<kStep, M, kBDR, DK, G><<<grid, block, 0, s>>>(p); break; \
        default: return hipErrorInvalidValue;                                        \
      }                                                                              \
    } else {                                                                         \
      switch (rnd) {                                                                 \
        case kRTN: key_kernel<kStep, M, kRTN, DK, G><<<grid, block, 0, s>>>(p); break; \
        case kSR: key_kernel<kStep, M, kSR, DK, G><<<grid, block, 0, s>>>(p); break;   \
        case kBDR: key_kernel<kStep, M, kBDR, DK, G><<<grid, block, 0, s>>>(p); break; \
        default: return hipErrorInvalidValue;                                        \
      }                                                                              \
    }                                                                                \
    return hipGetLastError();                                                        \
  }
      QS_KSTEP(kGDN) QS_KSTEP(kGLA) QS_KSTEP(kScalar) QS_KSTEP(kKDA)
#undef QS_KSTEP
      return hipErrorInvalidValue;
    case kImport:  // nothing stored before an import: BDR rounds to nearest
      if (p.mixed) {
        if (rnd == kSR)
          key_mixed_kernel<kImport, kGDN, kSR, DK, G><<<grid, block, 0, s>>>(p);
        else
          key_mixed_kernel<kImport, kGDN, kRTN, DK, G><<<grid, block, 0, s>>>(p);
      } else {
        if (rnd == kSR)
          key_kernel<kImport, kGDN, kSR, DK, G><<<grid, block, 0, s>>>(p);
        else
          key_kernel<kImport, kGDN, kRTN, DK, G><<<grid, block, 0, s>>>(p);
      }
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
hipError_t launch_key_dk(Op op, int mixer, int rnd, const KParams& p, hipStream_t s) {
  switch (p.G) {
    case 16: return launch_key<DK, 16>(op, mixer, rnd, p, s);
    case 32: return launch_key<DK, 32>(op, mixer, rnd, p, s);
    case 64: return launch_key<DK, 64>(op, mixer, rnd, p, s);
    case 128: return launch_key<DK, 128>(op, mixer, rnd, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace qs
