// qstate_value.h — value-axis decode kernels (scale groups of G key columns
// inside one value row) and the FP32-state kernels, templated on dk.  Each
// qstate_value_dk*.hip instantiates one dk.
//
// Lane geometry (all value-axis kernels): a value row of the state is split
// across adjacent lanes, each lane owning one 16-byte run of codes, i.e. 16
// INT8 elements or 32 INT4 elements, so a row of dk columns spans dk/16
// (INT8) or dk/32 (INT4) lanes and the wave holds the rest of its 64 lanes as
// further rows.  The loads of the next kPrefetch row iterations are in
// flight while the current one is computed.  Every operation of the step is
// row-local (LoReS blog, "LoReS: State Quantization": value-axis groups,
// full-precision update, readout from the updated state): the two dot
// products u = d.k and o = S'.q finish with DPP butterflies across the row's
// lanes, the group absmax with DPP butterflies across the group's lanes.
// Each state byte is read once and written once.
//
// Here: import / export / readout, the step of heads with mixed widths, the
// step of heads of one width where the persistent kernel of
// qstate_persist.h does not apply, and the FP32-state kernels: one wave (a
// workgroup of 64 lanes) owns a slice of the rows of one head (b, h), and
// small batches split a head into several slices so that enough waves exist
// to fill 256 CUs.

#pragma once

#include "qstate_device.h"

namespace qs {
namespace {

// Lane data of one row of a quantized head of one width: its 16 code bytes,
// its group scales and v_i (one slot of a load ring).
struct RowIn {
  uint4 raw;
  float s0, s1, v;
};

// The step of one head slice of BITS-bit codes (heads of one width; the
// kernels whose registers allow fewer than four waves per SIMD, where the
// persistent step of qstate_persist.h cannot share out its units evenly).
template <int MIXER, int RND, int DK, int BITS, int G>
__device__ __forceinline__ void step_quant_head(const KParams& p, const Slice sl) {
  constexpr bool SR = RND == kSR;
  using Gm = Geo<DK, BITS>;
  constexpr int E = Gm::E, LPR = Gm::LPR, RPW = Gm::RPW;
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
    in.raw = ld_stream(reinterpret_cast<const uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16));
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
      // decayed dequantized values (exactly the rounded c*(s*alpha) / (c*s)*alpha_j)
      if constexpr (vector_decay(MIXER)) {
        dequant_lane<BITS, E>(w, s_0, s_1, d);
#pragma unroll
        for (int j = 0; j < E; ++j) d[j] *= al[j];
      } else {
        dequant_lane<BITS, E>(w, s_0 * alpha_s, s_1 * alpha_s, d);
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
        st_stream(reinterpret_cast<uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16), packed);
        if constexpr (two_groups) {
          st_stream(hscales + (size_t)row * ngr + gcol, s0);
          st_stream(hscales + (size_t)row * ngr + gcol + 1, s1);
        } else if (lr % LPG == 0) {
          st_stream(hscales + (size_t)row * ngr + gcol, s0);
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
  // branch-free loads of in-range rows, as the quantized steps do
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
// Heads whose 16-column blocks have different widths (per-channel bits,
// LoReS 2/4).  Every lane owns the 16 columns of one block, 16 bytes of INT8
// or 8 bytes of INT4 codes, so a row spans dk/16 lanes whatever the widths;
// the block starts 8 * (q + INT8 blocks before q) bytes into its row.  A
// value-axis group covers G/16 lanes of one width (checked at create).  The
// loads follow the same prefetch ring as the uniform heads: every lane loads
// two 8-byte halves, an INT4 lane reading its one half twice, so the loads
// stay unconditional.
// ---------------------------------------------------------------------------

struct MixedLane {
  bool is8;
  int row_bytes, lane_off;
  __device__ __forceinline__ MixedLane(uint32_t mask, int lr, int lpr) {
    is8 = (mask >> lr) & 1u;
    row_bytes = 8 * (lpr + __popc(mask));
    lane_off = 8 * (lr + __popc(mask & ((1u << lr) - 1u)));
  }
};

struct RowMixed {
  uint2 a, b;  // codes: bytes 0..7 and 8..15 of an INT8 block; an INT4 block in a
  float s, v;
};

__device__ __forceinline__ void store_block(uint8_t* dst, bool is8, const uint32_t (&w)[4]) {
  if (is8)
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  else
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
}

__device__ __forceinline__ void store_block_stream(uint8_t* dst, bool is8, const uint32_t (&w)[4]) {
  if (is8)
    st_stream(reinterpret_cast<uint4*>(dst), make_uint4(w[0], w[1], w[2], w[3]));
  else
    st_stream(reinterpret_cast<uint2*>(dst), make_uint2(w[0], w[1]));
}

// Group absmax over the G/16 lanes of the lane's group, scale, and the
// lane's 16 codes.
template <int RND, int LPG>
__device__ __forceinline__ void quantize_block(const float (&sp)[16], bool is8, uint32_t key,
                                               uint32_t block, const uint32_t (&wprev)[4],
                                               float s_old, float& s_new, uint32_t (&out)[4]) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(sp[j]));
  m = lanes_max<LPG>(m);
  float inv;
  group_scale_rt(m, is8, s_new, inv);
  float inv16[16], so16[16], sn16[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) inv16[j] = inv, so16[j] = s_old, sn16[j] = s_new;
  quantize16_rt<RND>(sp, inv16, key, block, wprev, so16, sn16, is8, out);
}

template <int MIXER, int RND, int DK, int G>
__device__ __forceinline__ void step_mixed_head(const KParams& p, const Slice sl) {
  constexpr int E = 16, LPR = DK / 16, RPW = 64 / LPR, LPG = G / 16;
  constexpr int ngr = DK / G;
  const int lane = threadIdx.x;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  const int gcol = col0 / G;
  const MixedLane ml(p.int8_blocks[sl.h], lr, LPR);
  const float bias = ml.is8 ? 128.0f : 8.0f;
  const int half2 = ml.is8 ? 8 : 0;  // offset of the second 8-byte load
  uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
  float* hscales = p.scales + (size_t)sl.head * p.dv * ngr;
  const float* vh = p.v + (size_t)sl.head * p.dv;
  float* oh = p.o ? p.o + (size_t)sl.head * p.dv : nullptr;
  const int n_it = (sl.r1 - sl.r0 + RPW - 1) / RPW;

  const uint32_t key = RND == kSR ? head_key(p, (uint32_t)sl.b, (uint32_t)sl.h) : 0u;
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

  auto load = [&](int it) {  // in-range rows only (clamped); stored only if real
    RowMixed in;
    const int row = min(sl.r0 + it * RPW + rsub, sl.r1 - 1);
    const uint8_t* src = hcodes + (size_t)row * ml.row_bytes + ml.lane_off;
    in.a = ld_stream(reinterpret_cast<const uint2*>(src));
    in.b = ld_stream(reinterpret_cast<const uint2*>(src + half2));
    in.s = hscales[(size_t)row * ngr + gcol];
    in.v = vh[row];
    return in;
  };
  RowMixed ring[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    ring[k] = load(k);
    asm volatile("" ::: "memory");
  }
  const int n_trips = (n_it + kPrefetch - 1) / kPrefetch;
  for (int t = 0; t < n_trips; ++t) {
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int it = t * kPrefetch + k;
      const int row = sl.r0 + it * RPW + rsub;
      const bool store_ok = it < n_it && row < sl.r1;
      const uint32_t w[4] = {ring[k].a.x, ring[k].a.y, ring[k].b.x, ring[k].b.y};
      const float s_old = ring[k].s, vrow = ring[k].v;
      float d[E];
      unpack16_rt(w, ml.is8, d);
      if constexpr (vector_decay(MIXER)) {
        const float nb = -bias * s_old;
#pragma unroll
        for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(d[j], s_old, nb) * al[j];
      } else {
        const float sa = s_old * alpha_s, nb = -bias * sa;
#pragma unroll
        for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(d[j], sa, nb);
      }
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
      float s_new;
      uint32_t out[4];
      quantize_block<RND, LPG>(d, ml.is8, key, (uint32_t)((row * DK + col0) >> 4), w, s_old,
                               s_new, out);
      if (store_ok) {
        store_block_stream(hcodes + (size_t)row * ml.row_bytes + ml.lane_off, ml.is8, out);
        if (lr % LPG == 0) st_stream(hscales + (size_t)row * ngr + gcol, s_new);
        if (oh && lr == 0) oh[row] = o;
      }
    }
  }
}

// Import, export and readout of a mixed-width head.
template <int OP, bool SR, int DK, int G>
__device__ __forceinline__ void aux_mixed_head(const KParams& p, const Slice sl) {
  constexpr int E = 16, LPR = DK / 16, RPW = 64 / LPR, LPG = G / 16;
  constexpr int ngr = DK / G;
  const int lane = threadIdx.x;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  const int gcol = col0 / G;
  const MixedLane ml(p.int8_blocks[sl.h], lr, LPR);
  const float bias = ml.is8 ? 128.0f : 8.0f;
  const int half2 = ml.is8 ? 8 : 0;
  uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
  float* hscales = p.scales + (size_t)sl.head * p.dv * ngr;
  const size_t hoff = (size_t)sl.head * p.dv * DK;
  const uint32_t key = (OP == kImport && SR) ? head_key(p, (uint32_t)sl.b, (uint32_t)sl.h) : 0u;
  float qq[E];
  if constexpr (OP == kReadout) loadv(p.q + (size_t)sl.head * DK + col0, qq);
  for (int rbase = sl.r0; rbase < sl.r1; rbase += RPW) {
    const int row = rbase + rsub;
    const bool ok = row < sl.r1;
    const int rr = min(row, sl.r1 - 1);
    uint8_t* codes = hcodes + (size_t)rr * ml.row_bytes + ml.lane_off;
    if constexpr (OP == kImport) {
      float x[E];
      loadv(p.src + hoff + (size_t)rr * DK + col0, x);
      const uint32_t no_prev[4] = {0u, 0u, 0u, 0u};  // read only by BDR, never on import
      float s_new;
      uint32_t out[4];
      quantize_block<SR ? kSR : kRTN, LPG>(x, ml.is8, key, (uint32_t)((row * DK + col0) >> 4),
                                           no_prev, 0.0f, s_new, out);
      if (ok) {
        store_block(codes, ml.is8, out);
        if (lr % LPG == 0) hscales[(size_t)row * ngr + gcol] = s_new;
      }
    } else {
      const uint2 a = *reinterpret_cast<const uint2*>(codes);
      const uint2 b = *reinterpret_cast<const uint2*>(codes + half2);
      const uint32_t w[4] = {a.x, a.y, b.x, b.y};
      const float s = hscales[(size_t)rr * ngr + gcol];
      float d[E];
      unpack16_rt(w, ml.is8, d);
#pragma unroll
      for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(d[j], s, -bias * s);
      if constexpr (OP == kExport) {
        if (ok) storev(p.dst + hoff + (size_t)row * DK + col0, d);
      } else {
        const float o = row_sum<LPR>(lane_dot(d, qq));
        if (ok && lr == 0) p.o[(size_t)sl.head * p.dv + row] = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels and dispatch.
// ---------------------------------------------------------------------------

// The step of a launch with heads of mixed widths: every head takes the
// per-block path.
template <int MIXER, int RND, int DK, int G>
__global__ __launch_bounds__(kThreads) void step_mixed_kernel(const KParams p) {
  step_mixed_head<MIXER, RND, DK, G>(p, wave_slice(p));
}

// The step of heads of one width each, one wave per head slice (when the
// persistent step does not apply); the width is chosen per workgroup.  Held
// to three waves per SIMD (168 VGPRs): the GLA and KDA variants would take
// up to 196 and run two, and three measured 3-5 % faster.
template <int MIXER, int RND, int DK, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void step_sliced_kernel(const KParams p) {
  const Slice sl = wave_slice(p);
  if (p.int8_blocks[sl.h] != 0u)
    step_quant_head<MIXER, RND, DK, 8, G>(p, sl);
  else
    step_quant_head<MIXER, RND, DK, 4, G>(p, sl);
}

template <int MIXER, int DK>
__global__ __launch_bounds__(kThreads) void step_fp32_kernel(const KParams p) {
  step_fp32_head<MIXER, DK>(p, wave_slice(p));
}

template <int OP, bool SR, int DK, int G, bool MIXED>
__global__ __launch_bounds__(kThreads) void aux_kernel(const KParams p) {
  const Slice sl = wave_slice(p);
  if constexpr (MIXED) {
    aux_mixed_head<OP, SR, DK, G>(p, sl);
  } else {
    if (p.int8_blocks[sl.h] != 0u)
      aux_quant_head<OP, SR, DK, 8, G>(p, sl);
    else
      aux_quant_head<OP, SR, DK, 4, G>(p, sl);
  }
}

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

inline dim3 grid_of(const KParams& p) { return dim3((unsigned)(p.B * p.H * p.slices)); }

// The persistent step of heads of one width each (qstate_persist.h):
// launches it and returns true, or returns false where it does not apply.
template <int MIXER, int RND, int DK, int G>
bool launch_persist(const KParams& p, hipStream_t s, hipError_t* err);

template <int DK, int G, bool MIXED>
hipError_t launch_quant(Op op, int mixer, int rnd, const KParams& p, hipStream_t s) {
  const dim3 grid = grid_of(p), block(kThreads);
  if (op == kStep) {
#define QS_STEP(M)                                                                  \
  if (mixer == M) {                                                                 \
    if constexpr (MIXED) {                                                          \
      switch (rnd) {                                                                \
        case kRTN: step_mixed_kernel<M, kRTN, DK, G><<<grid, block, 0, s>>>(p); break; \
        case kSR: step_mixed_kernel<M, kSR, DK, G><<<grid, block, 0, s>>>(p); break;   \
        case kBDR: step_mixed_kernel<M, kBDR, DK, G><<<grid, block, 0, s>>>(p); break; \
        default: return hipErrorInvalidValue;                                       \
      }                                                                             \
      return hipGetLastError();                                                     \
    } else {                                                                        \
      hipError_t e = hipSuccess;                                                    \
      switch (rnd) {                                                                \
        case kRTN:                                                                  \
          if (launch_persist<M, kRTN, DK, G>(p, s, &e)) return e;                   \
          step_sliced_kernel<M, kRTN, DK, G><<<grid, block, 0, s>>>(p);             \
          break;                                                                    \
        case kSR:                                                                   \
          if (launch_persist<M, kSR, DK, G>(p, s, &e)) return e;                    \
          step_sliced_kernel<M, kSR, DK, G><<<grid, block, 0, s>>>(p);              \
          break;                                                                    \
        case kBDR:                                                                  \
          if (launch_persist<M, kBDR, DK, G>(p, s, &e)) return e;                   \
          step_sliced_kernel<M, kBDR, DK, G><<<grid, block, 0, s>>>(p);             \
          break;                                                                    \
        default: return hipErrorInvalidValue;                                       \
      }                                                                             \
      return hipGetLastError();                                                     \
    }                                                                               \
  }
    QS_STEP(kGDN) QS_STEP(kGLA) QS_STEP(kScalar) QS_STEP(kKDA)
#undef QS_STEP
    return hipErrorInvalidValue;
  }
  switch (op) {
    case kImport:  // nothing stored before an import: BDR rounds to nearest
      if (rnd == kSR)
        aux_kernel<kImport, true, DK, G, MIXED><<<grid, block, 0, s>>>(p);
      else
        aux_kernel<kImport, false, DK, G, MIXED><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kExport:
      aux_kernel<kExport, false, DK, G, MIXED><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kReadout:
      aux_kernel<kReadout, false, DK, G, MIXED><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    default:
      return hipErrorInvalidValue;
  }
}

// Key-axis groups: workgroups of KGeo::NW waves over blocks of KGeo::BR rows.
template <int DK>
hipError_t launch_value_dk(Op op, int mixer, int rnd, int fp32, const KParams& p, hipStream_t s) {
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
  if (p.slice_rows % 32 != 0) return hipErrorInvalidValue;
  switch (p.G) {
    case 16:
      return p.mixed ? launch_quant<DK, 16, true>(op, mixer, rnd, p, s)
                     : launch_quant<DK, 16, false>(op, mixer, rnd, p, s);
    case 32:
      return p.mixed ? launch_quant<DK, 32, true>(op, mixer, rnd, p, s)
                     : launch_quant<DK, 32, false>(op, mixer, rnd, p, s);
    case 64:
      return p.mixed ? launch_quant<DK, 64, true>(op, mixer, rnd, p, s)
                     : launch_quant<DK, 64, false>(op, mixer, rnd, p, s);
    case 128:
      return p.mixed ? launch_quant<DK, 128, true>(op, mixer, rnd, p, s)
                     : launch_quant<DK, 128, false>(op, mixer, rnd, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace qs
