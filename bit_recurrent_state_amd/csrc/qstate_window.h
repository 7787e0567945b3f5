// qstate_window.h — the decode step with a pure-write window ("Low-Bit GDN
// Recurrent-State Quantization: Global Gradient-aware Allocation and
// Pure-Write Sliding Windows", abstract): the last W pure writes of a head
// are kept beside its low-bit state H as FP8 (OCP E4M3) vector pairs (a, b),
// the full state being H + sum a b^T.  Each step propagates every pair's key
// through the transition (b <- A^T b), merges the oldest pair into H (it
// leaves the window), pushes the new pure write into its slot, reads out the
// full state and requantizes H.
//
// Window area of a head: a codes [dv][W] (row i holds its W values), then two
// copies of the key side, each b codes [W][dk] followed by scales [W][2]
// (s_a, s_b).  A step reads copy (counter & 1) and writes copy
// (counter + 1) & 1, so that waves sharing a head never see a half-written
// key side; the a codes are partitioned by row and updated in place.
//
// Low-rank bypass ("Preserving Updates in Low-Bit Recurrent State
// Quantization", abstract) runs in the same kernels: between merges its step
// is the window step above (the leaving slot is empty then); at a counter
// that is a multiple of W every pair's propagated key goes to LDS, each
// element sums the W pairs' terms, keeps the sum where it reaches the
// threshold times the element's stored scale, and the buffer empties but
// for the new pair.
//
// Work split: the per-head window work (W*dk key elements) is spread over all
// 64 lanes, 16 consecutive key columns of one pair per lane, with the same
// 16-element chunks and DPP trees as the rows; every wave of a head does it
// (only the first slice stores it).  The rows then run the value-axis step
// with two extra terms: the merge fma a_o,i b_o,j per element and the
// window's share of the readout per row.  FP8 conversions use the gfx950
// E4M3 instructions, whose rounding (nearest even) and decoding match the
// format exactly.

#pragma once

#include "qstate_value.h"

namespace qs {
namespace {

struct WinHead {
  uint8_t* a;        // [dv][W]
  uint8_t* b_rd;     // [W][dk], copy read this step
  uint8_t* b_wr;     // [W][dk], copy written this step
  const float* s_rd; // [W][2]
  float* s_wr;
};

__device__ __forceinline__ WinHead win_head(const KParams& p, int head, int dk, int W) {
  uint8_t* base = p.window + (uint64_t)head * p.window_head_bytes;
  const size_t copy = (size_t)W * dk + 8 * (size_t)W;
  uint8_t* b0 = base + (size_t)p.dv * W;
  const int rd = (int)(p.step & 1u);
  WinHead w;
  w.a = base;
  w.b_rd = b0 + rd * copy;
  w.b_wr = b0 + (rd ^ 1) * copy;
  w.s_rd = reinterpret_cast<const float*>(w.b_rd + (size_t)W * dk);
  w.s_wr = reinterpret_cast<float*>(w.b_wr + (size_t)W * dk);
  return w;
}

// E4M3 of 16 floats (four codes per word, element 0 in byte 0).
__device__ __forceinline__ void fp8_pack16(const float* x, uint32_t* w) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q], x[4 * q + 1], 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q + 2], x[4 * q + 3], v, true);
    w[q] = (uint32_t)v;
  }
}

__device__ __forceinline__ void fp8_unpack16(const uint32_t* w, float* x) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[4 * q] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 0);
    x[4 * q + 1] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 1);
    x[4 * q + 2] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 2);
    x[4 * q + 3] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 3);
  }
}

// E4M3 value of byte `sel` of w (a switch that folds when sel is a constant).
__device__ __forceinline__ float fp8_byte(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Max of x over the whole wave (every lane gets it).
__device__ __forceinline__ float wave_max(float x) {
  x = lanes_max<16>(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// The W code bytes of a row (W / 4 words).
template <int W>
struct ARow {
  uint32_t w[W / 4];
};

template <int W>
__device__ __forceinline__ ARow<W> load_arow(const uint8_t* src) {
  ARow<W> r;
  if constexpr (W == 4) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(src);
  } else if constexpr (W == 8) {
    const uint2 t = *reinterpret_cast<const uint2*>(src);
    r.w[0] = t.x, r.w[1] = t.y;
  } else {
    const uint4 t = *reinterpret_cast<const uint4*>(src);
    r.w[0] = t.x, r.w[1] = t.y, r.w[2] = t.z, r.w[3] = t.w;
  }
  return r;
}

// The W code bytes of a row, rotated so that byte j belongs to the pair of
// age j (slot `oldest` first).  W in {4, 8, 16}; `oldest` is wave-uniform.
template <int W>
__device__ __forceinline__ void age_order(const ARow<W>& raw, int oldest, uint32_t (&r)[4]) {
  if constexpr (W == 4) {
    r[0] = __builtin_amdgcn_alignbit(raw.w[0], raw.w[0], 8 * oldest);
  } else if constexpr (W == 8) {
    uint32_t lo = raw.w[0], hi = raw.w[1];
    if (oldest >= 4) {
      const uint32_t t = lo;
      lo = hi, hi = t;
    }
    const int sh = 8 * (oldest & 3);
    r[0] = __builtin_amdgcn_alignbit(hi, lo, sh);
    r[1] = __builtin_amdgcn_alignbit(lo, hi, sh);
  } else {
    uint32_t x[4] = {raw.w[0], raw.w[1], raw.w[2], raw.w[3]};
    const int dw = oldest >> 2;  // whole words first
    uint32_t y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = (i + dw) & 3;
      y[i] = s == 0 ? x[0] : s == 1 ? x[1] : s == 2 ? x[2] : x[3];
    }
    const int sh = 8 * (oldest & 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __builtin_amdgcn_alignbit(y[(i + 1) & 3], y[i], sh);
  }
}

// Per-head window quantities of this step, into LDS: the oldest pair's
// propagated key b_o [dk], c_t = b'_t . q [W] and s_a [W] in slot order; and
// the new pair's c = k . q and a-side scale.  The writer (the head's first
// slice) stores the propagated keys of the pairs that stay and the new
// pair's key and scales into the written copy.
//
// A low-rank bypass merge step (MERGE) instead puts every pair's
// propagated key into LDS [W][dk] (lds_bo then points at W * dk floats) and
// empties every slot but the new pair's.
template <int MIXER, int DK, int W, bool MERGE>
__device__ __forceinline__ void window_prologue(const KParams& p, const Slice sl, const WinHead& wh,
                                                int slot, bool writer, float beta, float alpha_s,
                                                float* lds_bo, float* lds_c, float* lds_sa,
                                                float* lds_kq, float& c_new, float& s_anew,
                                                float& inv_anew) {
  constexpr bool merge = MERGE;
  constexpr int LPP = DK / 16;         // lanes per pair
  constexpr int PPP = 64 / LPP;        // pairs per pass
  constexpr int PASSES = (W + PPP - 1) / PPP;
  const int lane = threadIdx.x;
  const int lp = lane % LPP, psub = lane / LPP;
  const int c0 = lp * 16;
  float k16[16], q16[16], a16[16];
  loadv(p.k + (size_t)sl.head * DK + c0, k16);
  loadv(p.q + (size_t)sl.head * DK + c0, q16);
  if constexpr (vector_decay(MIXER)) loadv(p.alpha + (size_t)sl.head * DK + c0, a16);
  // the rows' copy of the head's vectors (padded, 4 floats after every 16),
  // from the first pass's lanes, which together hold all dk columns
  if (psub == 0) {
    constexpr int PDK = DK + DK / 4;
    storev(lds_kq + c0 + c0 / 4, k16);
    storev(lds_kq + PDK + c0 + c0 / 4, q16);
    if constexpr (vector_decay(MIXER)) storev(lds_kq + 2 * PDK + c0 + c0 / 4, a16);
  }
  if (lane < W) lds_sa[lane] = wh.s_rd[2 * lane];
  c_new = row_sum<LPP>(chunk_dot(k16, q16, 0));
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int t = pass * PPP + psub;
    const bool act = t < W;
    const int tt = act ? t : 0;
    const uint4 raw = *reinterpret_cast<const uint4*>(wh.b_rd + (size_t)tt * DK + c0);
    const float sb = wh.s_rd[2 * tt + 1];
    const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
    float b[16];
    fp8_unpack16(rw, b);
#pragma unroll
    for (int j = 0; j < 16; ++j) b[j] = (b[j] * sb) * (vector_decay(MIXER) ? a16[j] : alpha_s);
    float bp[16];
    if constexpr (delta_rule(MIXER)) {
      const float wb = -(beta * row_sum<LPP>(chunk_dot(b, k16, 0)));
#pragma unroll
      for (int j = 0; j < 16; ++j) bp[j] = __builtin_fmaf(wb, k16[j], b[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) bp[j] = b[j];
    }
    const float c = row_sum<LPP>(chunk_dot(bp, q16, 0));
    if (act && lp == 0) lds_c[t] = c;
    const bool leaves = act && t == slot;
    if constexpr (merge) {
      if (act) storev(lds_bo + (size_t)t * (DK + DK / 4) + c0 + c0 / 4, bp);
    } else if (leaves) {
      storev(lds_bo + c0 + c0 / 4, bp);
    }
    const bool emptied = merge && act && t != slot;
    // stored key: b' for the pairs that stay, k for the new pair
    float x[16];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      x[j] = leaves ? k16[j] : bp[j];
      m = fmaxf(m, fabsf(x[j]));
    }
    m = lanes_max<LPP>(m);
    float s, inv;
    group_scale<448>(m, s, inv);
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = x[j] * inv;
    uint32_t w[4];
    fp8_pack16(x, w);
    if (writer && act) {
      *reinterpret_cast<uint4*>(wh.b_wr + (size_t)t * DK + c0) =
          emptied ? make_uint4(0u, 0u, 0u, 0u) : make_uint4(w[0], w[1], w[2], w[3]);
      if (lp == 0) {
        wh.s_wr[2 * t + 1] = emptied ? 0.0f : s;
        if (!leaves) wh.s_wr[2 * t] = emptied ? 0.0f : wh.s_rd[2 * t];
      }
    }
  }
  // a side of the new pair: one scale over its dv values
  float m = 0.0f;
  for (int i = lane; i < p.dv; i += 64) {
    const float vi = p.v[(size_t)sl.head * p.dv + i];
    m = fmaxf(m, fabsf(MIXER == kGLA ? vi : beta * vi));
  }
  m = wave_max(m);
  group_scale<448>(m, s_anew, inv_anew);
  if (writer && lane == 0) wh.s_wr[2 * slot] = s_anew;
}

template <int MIXER, int RND, int DK, int BITS, int G, int W, bool MERGE>
__device__ __forceinline__ void step_pw_head(const KParams& p, const Slice sl, float* lds) {
  using Gm = Geo<DK, BITS>;
  constexpr int E = Gm::E, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr bool SR = RND == kSR;
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
  const float* vh = p.v + (size_t)sl.head * p.dv;
  float* oh = p.o ? p.o + (size_t)sl.head * p.dv : nullptr;
  const int n_it = (sl.r1 - sl.r0 + RPW - 1) / RPW;

  const uint32_t key = SR ? head_key(p, (uint32_t)sl.b, (uint32_t)sl.h) : 0u;
  float alpha_s = 0.0f, beta = 0.0f;
  if constexpr (!vector_decay(MIXER)) alpha_s = p.alpha[sl.head];
  if constexpr (MIXER != kGLA) beta = p.beta[sl.head];

  // window of the head
  const WinHead wh = win_head(p, sl.head, DK, W);
  const int slot = (int)(p.step % (uint64_t)W);
  // the state rows' loads go first, so that they are in flight while the
  // per-head window work runs
  struct RowW {
    uint4 raw;
    ARow<W> a;
    float s0, s1, v;
  };
  auto load = [&](int it) {
    RowW in;
    const int row = min(sl.r0 + it * RPW + rsub, sl.r1 - 1);
    in.raw = ld_stream(reinterpret_cast<const uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16));
    in.a = load_arow<W>(wh.a + (size_t)row * W);
    in.s0 = hscales[(size_t)row * ngr + gcol];
    in.s1 = two_groups ? hscales[(size_t)row * ngr + gcol + 1] : in.s0;
    in.v = vh[row];
    return in;
  };
  RowW ring[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    ring[k] = load(k);
    asm volatile("" ::: "memory");
  }
  // LDS vectors padded to PDK floats (4 after every 16: loadv_padded)
  constexpr int PDK = DK + DK / 4;
  float* lds_bo = lds;  // the leaving pair's key [dk], or every key [W][dk] (bypass merge)
  float* lds_c = lds + W * PDK;
  float* lds_sa = lds_c + W;
  float* lds_kq = lds_sa + W;  // the head's k, q and (GLA, KDA) alpha, [3][dk]
  constexpr bool merge = MERGE;
  float c_new, s_anew, inv_anew;
  // The rows read the head's vectors from LDS in every iteration instead of
  // holding them in registers (2 or 3 x E floats per lane), which keeps the
  // kernel within the registers of four waves per SIMD; the prologue, which
  // loads them for the keys' transition, leaves them there.
  window_prologue<MIXER, DK, W, MERGE>(p, sl, wh, slot, sl.r0 == 0, beta, alpha_s, lds_bo, lds_c,
                                lds_sa, lds_kq, c_new, s_anew, inv_anew);
  __syncthreads();
  float ca[W], sa[W];  // by age: 0 = oldest (leaving), W-1 = newest before this step
#pragma unroll
  for (int g = 0; g < W; ++g) {
    const int t = (slot + g) % W;
    ca[g] = uniform(lds_c[t]);
    sa[g] = uniform(lds_sa[t]);
  }
  c_new = uniform(c_new);
  inv_anew = uniform(inv_anew);
  const float* lk = lds_kq + col0 + col0 / 4;

  const int n_trips = (n_it + kPrefetch - 1) / kPrefetch;
  for (int t = 0; t < n_trips; ++t) {
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
      const int it = t * kPrefetch + k;
      const int row = sl.r0 + it * RPW + rsub;
      const bool store_ok = it < n_it && row < sl.r1;
      const uint32_t w[4] = {ring[k].raw.x, ring[k].raw.y, ring[k].raw.z, ring[k].raw.w};
      const float s_0 = ring[k].s0, s_1 = ring[k].s1, vrow = ring[k].v;
      uint32_t ab[4] = {0u, 0u, 0u, 0u};
      age_order<W>(ring[k].a, slot, ab);
      asm volatile("" ::: "memory");  // read the head's vectors from LDS here, not once
      float kk[E], al[E];
      loadv_padded(lk, kk);
      if constexpr (vector_decay(MIXER)) loadv_padded(lk + 2 * PDK, al);
      float d[E];
      if constexpr (vector_decay(MIXER)) {
        dequant_lane<BITS, E>(w, s_0, s_1, d);
#pragma unroll
        for (int j = 0; j < E; ++j) d[j] *= al[j];
      } else {
        dequant_lane<BITS, E>(w, s_0 * alpha_s, s_1 * alpha_s, d);
      }
      const float a_new = MIXER == kGLA ? vrow : beta * vrow;
      float o;
      if constexpr (merge) {
        // bypass merge: H A, then the buffer's elements m = sum_g a_g b'_g (oldest
        // first; slot 0 is the oldest here) that reach theta * the stored scale
        if constexpr (delta_rule(MIXER)) {
          const float wt = -(beta * row_sum<LPR>(lane_dot(d, kk)));
#pragma unroll
          for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(wt, kk[j], d[j]);
        }
        float m[E];
#pragma unroll
        for (int j = 0; j < E; ++j) m[j] = 0.0f;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int g = 0; g < W; ++g) {
          const float a_g = fp8_byte(ab[g >> 2], g & 3) * sa[g];
          float bg[E];
          loadv_padded(lds_bo + (size_t)g * PDK + col0 + col0 / 4, bg);
#pragma unroll
          for (int j = 0; j < E; ++j) m[j] = __builtin_fmaf(a_g, bg[j], m[j]);
        }
        const float thr0 = p.lrb_theta * s_0, thr1 = p.lrb_theta * s_1;
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const float thr = (two_groups && j >= 16) ? thr1 : thr0;
          d[j] = fabsf(m[j]) >= thr ? d[j] + m[j] : d[j];
        }
        ring[k] = load(it + kPrefetch);
        float qq[E];
        loadv_padded(lk + PDK, qq);
        o = __builtin_fmaf(a_new, c_new, row_sum<LPR>(lane_dot(d, qq)));
      } else {
        // H A (transition), then the leaving pair: S' = fma(a_o, b_o, H A); its
        // key is read from LDS each iteration rather than held in E registers
        const float a_o = __builtin_amdgcn_cvt_f32_fp8((int)ab[0], 0) * sa[0];
        float bo[E];
        asm volatile("" ::: "memory");
        loadv_padded(lds_bo + col0 + col0 / 4, bo);
        if constexpr (delta_rule(MIXER)) {
          const float wt = -(beta * row_sum<LPR>(lane_dot(d, kk)));
#pragma unroll
          for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(a_o, bo[j], __builtin_fmaf(wt, kk[j], d[j]));
        } else {
#pragma unroll
          for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(a_o, bo[j], d[j]);
        }
        ring[k] = load(it + kPrefetch);
        // readout of the full state: H'q, the pairs that stay (oldest first), the new pair
        float qq[E];
        loadv_padded(lk + PDK, qq);
        o = row_sum<LPR>(lane_dot(d, qq));
#pragma unroll
        for (int g = 1; g < W; ++g) {
          const float a_g = fp8_byte(ab[g >> 2], g & 3) * sa[g];
          o = __builtin_fmaf(a_g, ca[g], o);
        }
        o = __builtin_fmaf(a_new, c_new, o);
      }
      float s0 = s_0, s1 = s_1;
      const uint32_t block0 = (uint32_t)((row * DK + col0) >> 4);
      // the INT4 BDR fast path where the kernel already runs at three waves
      // per SIMD (delta-rule mixers), whose register bound leaves room for it
      constexpr bool FAST = delta_rule(MIXER);
      const uint4 packed = quantize_lane<BITS, RND, E, LPG, FAST>(d, key, block0, w, s0, s1);
      if (store_ok) {
        st_stream(reinterpret_cast<uint4*>(hcodes + (size_t)row * Gm::ROW_BYTES + lr * 16), packed);
        if constexpr (two_groups) {
          st_stream(hscales + (size_t)row * ngr + gcol, s0);
          st_stream(hscales + (size_t)row * ngr + gcol + 1, s1);
        } else if (lr % LPG == 0) {
          st_stream(hscales + (size_t)row * ngr + gcol, s0);
        }
        if (lr == 0) {
          if (oh) oh[row] = o;
          const int code = __builtin_amdgcn_cvt_pk_fp8_f32(a_new * inv_anew, 0.0f, 0, false);
          if constexpr (merge) {  // the new pair in slot 0, the emptied slots zero
            const uint32_t c0w = (uint32_t)code & 0xFFu;
            uint8_t* arow = wh.a + (size_t)row * W;
            if constexpr (W == 4) {
              *reinterpret_cast<uint32_t*>(arow) = c0w;
            } else if constexpr (W == 8) {
              *reinterpret_cast<uint2*>(arow) = make_uint2(c0w, 0u);
            } else {
              *reinterpret_cast<uint4*>(arow) = make_uint4(c0w, 0u, 0u, 0u);
            }
          } else {
            wh.a[(size_t)row * W + slot] = (uint8_t)(code & 0xFF);
          }
        }
      }
    }
  }
}

// Import (quantize H, empty the window), export of the full state and readout
// of the full state, for a head with a window.
template <int OP, bool SR, int DK, int BITS, int G, int W>
__device__ __forceinline__ void aux_pw_head(const KParams& p, const Slice sl, float* lds) {
  using Gm = Geo<DK, BITS>;
  constexpr int E = Gm::E, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr float bias = (float)(1 << (BITS - 1));
  constexpr int ngr = DK / G;
  constexpr bool two_groups = G < E;
  constexpr int LPP = DK / 16, PPP = 64 / LPP, PASSES = (W + PPP - 1) / PPP;
  const int lane = threadIdx.x;
  if constexpr (OP == kImport) {
    aux_quant_head<kImport, SR, DK, BITS, G>(p, sl);
    if (sl.r0 == 0) {  // the first slice empties the head's window (both copies)
      uint8_t* base = p.window + (uint64_t)sl.head * p.window_head_bytes;
      for (uint64_t off = (uint64_t)lane * 16; off < p.window_head_bytes; off += 64 * 16)
        *reinterpret_cast<uint4*>(base + off) = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  } else {
    const WinHead wh = win_head(p, sl.head, DK, W);
    const int oldest = (int)(p.step % (uint64_t)W);  // at the next step's counter
    // decoded keys: every pair into LDS [W][dk]; c_t = b_t . q (readout)
    const int lp = lane % LPP, psub = lane / LPP, c0 = lp * 16;
    float q16[16];
    if constexpr (OP == kReadout) loadv(p.q + (size_t)sl.head * DK + c0, q16);
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int t = pass * PPP + psub;
      if (t < W) {
        const uint4 raw = *reinterpret_cast<const uint4*>(wh.b_rd + (size_t)t * DK + c0);
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
        float b[16];
        fp8_unpack16(rw, b);
        const float sb = wh.s_rd[2 * t + 1];
#pragma unroll
        for (int j = 0; j < 16; ++j) b[j] = b[j] * sb;
        if constexpr (OP == kExport) {
          storev(lds + (size_t)t * DK + c0, b);
        } else {
          const float c = row_sum<LPP>(chunk_dot(b, q16, 0));
          if (lp == 0) lds[t] = c;
        }
      }
    }
    __syncthreads();
    float sa[W], ca[W];
#pragma unroll
    for (int g = 0; g < W; ++g) {
      const int t = (oldest + g) % W;
      sa[g] = uniform(wh.s_rd[2 * t]);
      ca[g] = OP == kReadout ? uniform(lds[t]) : 0.0f;
    }
    const int lr = lane % LPR, rsub = lane / LPR, col0 = lr * E;
    const int gcol = two_groups ? col0 / 16 : col0 / G;
    const uint8_t* hcodes =
        reinterpret_cast<const uint8_t*>(p.state) + head_code_offset(p, sl.b, sl.h);
    const float* hscales = p.scales + (size_t)sl.head * p.dv * ngr;
    float qq[E];
    if constexpr (OP == kReadout) loadv(p.q + (size_t)sl.head * DK + col0, qq);
    for (int rbase = sl.r0; rbase < sl.r1; rbase += RPW) {
      const int row = rbase + rsub;
      const bool ok = row < sl.r1;
      const int rr = min(row, sl.r1 - 1);
      const uint4 raw = *reinterpret_cast<const uint4*>(hcodes + (size_t)rr * Gm::ROW_BYTES + lr * 16);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      const float s0 = hscales[(size_t)rr * ngr + gcol];
      const float s1 = two_groups ? hscales[(size_t)rr * ngr + gcol + 1] : s0;
      float d[E];
      unpack16<BITS>(w, d);
      if constexpr (E == 32) unpack16<BITS>(w + 2, d + 16);
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const float s = j < 16 ? s0 : s1;
        d[j] = __builtin_fmaf(d[j], s, -bias * s);
      }
      uint32_t ab[4] = {0u, 0u, 0u, 0u};
      age_order<W>(load_arow<W>(wh.a + (size_t)rr * W), oldest, ab);
      if constexpr (OP == kExport) {
#pragma unroll
        for (int g = 0; g < W; ++g) {
          const float a_g = fp8_byte(ab[g >> 2], g & 3) * sa[g];
          const float* bt = lds + (size_t)((oldest + g) % W) * DK + col0;
#pragma unroll
          for (int j = 0; j < E; ++j) d[j] = __builtin_fmaf(a_g, bt[j], d[j]);
        }
        if (ok) storev(p.dst + ((size_t)sl.head * p.dv + row) * DK + col0, d);
      } else {
        float o = row_sum<LPR>(lane_dot(d, qq));
#pragma unroll
        for (int g = 0; g < W; ++g) {
          const float a_g = fp8_byte(ab[g >> 2], g & 3) * sa[g];
          o = __builtin_fmaf(a_g, ca[g], o);
        }
        if (ok && lr == 0) p.o[(size_t)sl.head * p.dv + row] = o;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Kernels and dispatch.  Heads of one width only (per-channel widths and
// key-axis groups are not combined with the window).
// ---------------------------------------------------------------------------

template <int DK, int W>
constexpr int window_lds_floats() {
  // keys, c, s_a, then the head's k, q, alpha; the vectors of the step
  // kernel padded to DK + DK / 4 floats
  return W * (DK + DK / 4) + 2 * W + 3 * (DK + DK / 4);
}

// MERGE: the low-rank bypass merge step (a kernel of its own, so that the
// other steps keep the window kernel's registers).
template <int MIXER, int RND, int DK, int G, int W, bool MERGE>
__global__ __launch_bounds__(kThreads) void step_pw_kernel(const KParams p) {
  __shared__ float lds[window_lds_floats<DK, W>()];
  const Slice sl = wave_slice(p);
  if (p.int8_blocks[sl.h] != 0u)
    step_pw_head<MIXER, RND, DK, 8, G, W, MERGE>(p, sl, lds);
  else
    step_pw_head<MIXER, RND, DK, 4, G, W, MERGE>(p, sl, lds);
}

template <int OP, bool SR, int DK, int G, int W>
__global__ __launch_bounds__(kThreads) void aux_pw_kernel(const KParams p) {
  __shared__ float lds[window_lds_floats<DK, W>()];
  const Slice sl = wave_slice(p);
  if (p.int8_blocks[sl.h] != 0u)
    aux_pw_head<OP, SR, DK, 8, G, W>(p, sl, lds);
  else
    aux_pw_head<OP, SR, DK, 4, G, W>(p, sl, lds);
}

template <int DK, int G, int W>
hipError_t launch_pw(Op op, int mixer, int rnd, const KParams& p, hipStream_t s) {
  if (p.slice_rows % 32 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(p.B * p.H * p.slices)), block(kThreads);
  if (op == kStep) {
#define QS_PW_R(M, R)                                                          \
  if (p.lrb_merge)                                                             \
    step_pw_kernel<M, R, DK, G, W, true><<<grid, block, 0, s>>>(p);            \
  else                                                                         \
    step_pw_kernel<M, R, DK, G, W, false><<<grid, block, 0, s>>>(p);
#define QS_PW(M)                                                               \
  if (mixer == M) {                                                            \
    switch (rnd) {                                                             \
      case kRTN: QS_PW_R(M, kRTN) break;                                       \
      case kSR: QS_PW_R(M, kSR) break;                                         \
      case kBDR: QS_PW_R(M, kBDR) break;                                       \
      default: return hipErrorInvalidValue;                                    \
    }                                                                          \
    return hipGetLastError();                                                  \
  }
    QS_PW(kGDN) QS_PW(kGLA) QS_PW(kScalar) QS_PW(kKDA)
#undef QS_PW
#undef QS_PW_R
    return hipErrorInvalidValue;
  }
  switch (op) {
    case kImport:
      if (rnd == kSR)
        aux_pw_kernel<kImport, true, DK, G, W><<<grid, block, 0, s>>>(p);
      else
        aux_pw_kernel<kImport, false, DK, G, W><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kExport:
      aux_pw_kernel<kExport, false, DK, G, W><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    case kReadout:
      aux_pw_kernel<kReadout, false, DK, G, W><<<grid, block, 0, s>>>(p);
      return hipGetLastError();
    default:
      return hipErrorInvalidValue;
  }
}

template <int DK, int W>
hipError_t launch_pw_g(Op op, int mixer, int rnd, const KParams& p, hipStream_t s) {
  switch (p.G) {
    case 16: return launch_pw<DK, 16, W>(op, mixer, rnd, p, s);
    case 32: return launch_pw<DK, 32, W>(op, mixer, rnd, p, s);
    case 64: return launch_pw<DK, 64, W>(op, mixer, rnd, p, s);
    case 128: return launch_pw<DK, 128, W>(op, mixer, rnd, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace qs
