// qstate_persist.h — the value-axis decode step on quantized heads of one
// width each, as a persistent kernel.
//
// With one workgroup per head, the chip's dispatcher starts a new head
// wherever a wave ends, and the last heads of a step run alone on a few
// SIMDs while the rest of the chip idles (about a tenth of the step at 8192
// heads).  Here a fixed grid of W waves (what the chip holds at once) shares
// the work out in units of UNIT_ROWS rows of one head: wave w takes units
// w, w + W, w + 2W, ..., so every wave has the same number of units (one
// less for some), and every SIMD the same work.  Among the waves of one SIMD
// the issue arbiter favours the oldest; each wave therefore lowers its issue
// priority as its units run out, so that the waves of a SIMD advance
// together instead of the youngest being left to finish alone.  A wave's load ring runs on from one unit into the next, and the
// per-head data (k, q, alpha for GLA and KDA, and the scalar gates) is
// staged through LDS one unit ahead, so a new unit costs no wait on memory;
// keeping k and q in LDS rather than in registers also leaves room for four
// waves per SIMD.  No atomics, no shared counters.
//
// Units: runs of UNIT_ROWS = kPrefetch * (INT4 rows per wave iteration) rows
// of one head, i.e. one trip of the INT4 ring and two of the INT8 ring.  All
// INT8 heads come first (every batch row), then the INT4 heads, each class in
// (b, h) order; a wave's units increase, so they change width at most once.

#pragma once

#include <algorithm>

#include "qstate_value.h"

namespace qs {
namespace {

template <int DK>
struct PGeo {
  static constexpr int RPW4 = 64 / (DK / 32);           // INT4 rows per iteration
  static constexpr int UNIT_ROWS = kPrefetch * RPW4;    // rows per unit
  static_assert(UNIT_ROWS == persist_unit_rows(DK), "unit rows as the host assumes");
};

// Unsigned division by a launch constant d (x < 2^31): q = (mulhi(x, m) + x)
// >> s with s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1.
__device__ __forceinline__ uint32_t fast_div(uint32_t x, FastDiv f) {
  return (__umulhi(x, f.m) + x) >> f.s;
}

struct PUnit {
  int b, h, r0;  // b < 0: no unit
  bool is8;
};

// Unit u of the launch (wave-uniform).
template <int DK>
__device__ __forceinline__ PUnit decode_unit(const KParams& p, uint32_t u) {
  PUnit r;
  r.b = -1, r.h = 0, r.r0 = 0, r.is8 = false;
  if (u >= p.n_units) return r;
  const uint32_t n8 = (uint32_t)p.n8_heads;
  const uint32_t u8 = (uint32_t)p.B * n8 * (uint32_t)p.units_per_head;
  r.is8 = u < u8;
  const uint32_t v = r.is8 ? u : u - u8;
  const uint32_t n = r.is8 ? n8 : (uint32_t)p.H - n8;
  // Heads in groups of 8, each group's units ordered part-major: the units
  // of one head lie 8 apart, so they go to waves on the same XCD (the chip
  // hands workgroups to its 8 XCDs round-robin), whose L2 then serves the
  // head's vectors to all of them.
  const uint32_t uph = (uint32_t)p.units_per_head;
  const uint32_t grp = fast_div(v, p.div_group);  // by 8 * units_per_head
  const uint32_t rem = v - grp * 8u * uph;
  const uint32_t hg = min(8u, (uint32_t)p.B * n - grp * 8u);  // heads in this group
  const uint32_t part = hg == 8u ? rem >> 3 : rem / hg;
  const uint32_t hi = grp * 8u + (rem - part * hg);  // head index inside the class
  const uint32_t bb = fast_div(hi, r.is8 ? p.div_n8 : p.div_n4);
  r.b = (int)bb;
  r.h = p.head_order[(r.is8 ? 0u : n8) + hi - bb * n];
  r.r0 = (int)part * PGeo<DK>::UNIT_ROWS;
  return r;
}

__device__ __forceinline__ uint32_t lane0(uint32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// The per-head data of one unit: k, q (and alpha) as N4 = NV*DK/4 float4s,
// one or more per lane, then one float4 (alpha, beta, 0, 0) of scalar gates.
// A unit's data travels global -> registers (at the switch into the unit
// before it) -> LDS (half a trip later), and is read from LDS while the unit
// is computed, so no wave waits on these loads.
template <int MIXER, int DK>
struct Stage {
  static constexpr int NV = vector_decay(MIXER) ? 3 : 2;
  static constexpr int N4 = NV * DK / 4;
  static constexpr int S4 = (N4 + 63) / 64;
  static constexpr int LDS4 = N4 + 1;  // float4s of one LDS buffer
  float x[S4][4];  // scalars, not float4s: keeps the stage in registers
  float g0, g1;
  __device__ __forceinline__ void load(const KParams& p, int head) {
    // per-lane choice among the three vectors, without indexing the kernel
    // arguments
    const uint64_t base_k = reinterpret_cast<uint64_t>(p.k + (size_t)head * DK);
    const uint64_t base_q = reinterpret_cast<uint64_t>(p.q + (size_t)head * DK);
    const uint64_t base_a =
        vector_decay(MIXER) ? reinterpret_cast<uint64_t>(p.alpha + (size_t)head * DK) : 0;
#pragma unroll
    for (int s = 0; s < S4; ++s) {
      const int f = (int)threadIdx.x + 64 * s;
      if (N4 % 64 == 0 || f < N4) {
        const int vec = f / (DK / 4), off = f - vec * (DK / 4);
        const uint64_t b = vec == 0 ? base_k : (vec == 1 ? base_q : base_a);
        const float4 t = reinterpret_cast<const float4*>(b)[off];
        x[s][0] = t.x, x[s][1] = t.y, x[s][2] = t.z, x[s][3] = t.w;
      }
    }
    g0 = vector_decay(MIXER) ? 0.0f : p.alpha[head];
    g1 = MIXER == kGLA ? 0.0f : p.beta[head];
  }
  __device__ __forceinline__ void store(float4* lds) const {
#pragma unroll
    for (int s = 0; s < S4; ++s) {
      const int f = (int)threadIdx.x + 64 * s;
      if (N4 % 64 == 0 || f < N4) lds[f] = make_float4(x[s][0], x[s][1], x[s][2], x[s][3]);
    }
    if (threadIdx.x == 0) lds[N4] = make_float4(g0, g1, 0.0f, 0.0f);
  }
};

// Everything a wave keeps across units.
template <int MIXER, int DK>
struct PState {
  uint32_t u;           // index of cur
  PUnit cur, nxt;       // units u and u + W
  int slot;             // LDS buffer of cur (nxt's is slot ^ 1)
  Stage<MIXER, DK> st;  // nxt's data, loaded at the switch into cur
};

// cur <- nxt; nxt <- the wave's unit after it; load the new nxt's data.
template <int MIXER, int DK>
__device__ __forceinline__ void advance(const KParams& p, PState<MIXER, DK>& ps) {
  ps.u += gridDim.x;
  ps.cur = ps.nxt;
  ps.slot ^= 1;
  if (ps.cur.b < 0) return;
  ps.nxt = decode_unit<DK>(p, ps.u + gridDim.x);
  if (ps.nxt.b >= 0) ps.st.load(p, ps.nxt.b * p.H + ps.nxt.h);
}

// Issue priority from the units the wave has left (cur included): a wave
// that has got ahead of the others of its SIMD yields the issue slots to
// them, so the waves of a SIMD (equal work each) advance together.
__device__ __forceinline__ void set_priority(const KParams& p, uint32_t u) {
  const uint32_t left = (p.n_units - 1u - u) / gridDim.x + 1u;
  if (left >= 4u)
    __builtin_amdgcn_s_setprio(3);
  else if (left == 3u)
    __builtin_amdgcn_s_setprio(2);
  else if (left == 2u)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Run the units of width BITS from ps.cur on, while they last.
template <int MIXER, int RND, int DK, int BITS, int G>
__device__ __forceinline__ void persist_class(const KParams& p, PState<MIXER, DK>& ps,
                                              float4 (*lds)[Stage<MIXER, DK>::LDS4]) {
  constexpr bool SR = RND == kSR;
  using Gm = Geo<DK, BITS>;
  constexpr int E = Gm::E, LPR = Gm::LPR, RPW = Gm::RPW;
  constexpr int TRIPS = PGeo<DK>::UNIT_ROWS / (kPrefetch * RPW);  // per unit: 1 (INT4) or 2
  constexpr bool two_groups = G < E;
  constexpr int LPG = two_groups ? 0 : G / E;
  constexpr int ngr = DK / G;
  constexpr bool IS8 = BITS == 8;
  const int lane = threadIdx.x;
  const int lr = lane % LPR;
  const int rsub = lane / LPR;
  const int col0 = lr * E;
  const int gcol = two_groups ? col0 / 16 : col0 / G;

  if (ps.cur.b < 0 || ps.cur.is8 != IS8) return;

  // Lane data of one row of a unit.  Rows past the head's end re-read its
  // last row and are never stored.  it < 0: a stand-in load of row ur0 by
  // every lane of a row group, for the ring slots refilled when no unit of
  // this width follows (never computed; one cache line per lane group, where
  // loading the rows past the unit read 11 MB more per headline launch; the
  // loads stay unconditional so the waits on the ring stay exact).
  auto load = [&](int ub, int uh, int ur0, int it) {
    RowIn in;
    const int row = it < 0 ? ur0 : min(ur0 + it * RPW + rsub, p.dv - 1);
    const size_t head = (size_t)ub * p.H + uh;
    const uint8_t* hc = reinterpret_cast<const uint8_t*>(p.state) + head_code_offset(p, ub, uh);
    const float* hs = p.scales + head * p.dv * ngr;
    // 32-bit offsets from wave-uniform bases (a row is < 4096 rows of
    // <= 256 bytes into its head): scalar base + vector offset addressing
    in.raw = ld_stream(reinterpret_cast<const uint4*>(hc + (uint32_t)(row * Gm::ROW_BYTES + lr * 16)));
    in.s0 = ld_stream(hs + (uint32_t)(row * ngr + gcol));
    in.s1 = two_groups ? ld_stream(hs + (uint32_t)(row * ngr + gcol + 1)) : in.s0;
    in.v = (p.v + head * p.dv)[(uint32_t)row];
    return in;
  };
  RowIn ring[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    ring[k] = load(ps.cur.b, ps.cur.h, ps.cur.r0, k);
    asm volatile("" ::: "memory");  // issue the slots in order: slot 0 is needed first
  }

  for (;;) {
    const int head = ps.cur.b * p.H + ps.cur.h;
    uint8_t* hcodes = reinterpret_cast<uint8_t*>(p.state) + head_code_offset(p, ps.cur.b, ps.cur.h);
    float* hscales = p.scales + (size_t)head * p.dv * ngr;
    float* oh = p.o ? p.o + (size_t)head * p.dv : nullptr;
    set_priority(p, ps.u);
    const uint32_t key = SR ? head_key(p, (uint32_t)ps.cur.b, (uint32_t)ps.cur.h) : 0u;
    const float4 gates = lds[ps.slot][Stage<MIXER, DK>::N4];
    const float alpha_s = gates.x, beta = gates.y;
    const float* lk = reinterpret_cast<const float*>(lds[ps.slot]) + col0;
    float4* lds_next = lds[ps.slot ^ 1];
    const bool next_same = ps.nxt.b >= 0 && ps.nxt.is8 == IS8;
#pragma unroll
    for (int trip = 0; trip < TRIPS; ++trip) {
      // The slots refilled in this trip feed the next one: cur's next trip,
      // or in cur's last trip nxt's first (without a next unit of this width,
      // stand-in loads that are never computed).
      const bool to_next = trip + 1 == TRIPS && next_same;
      const int rb = to_next ? ps.nxt.b : ps.cur.b;  // values, not a reference: keeps ps in registers
      const int rh = to_next ? ps.nxt.h : ps.cur.h;
      const int rr0 = to_next ? ps.nxt.r0 : ps.cur.r0;
      const int rbase = to_next ? 0 : (trip + 1) * kPrefetch;
#pragma unroll
      for (int k = 0; k < kPrefetch; ++k) {
        const int it = trip * kPrefetch + k;
        const int row = ps.cur.r0 + it * RPW + rsub;
        const bool store_ok = row < p.dv;
        const uint32_t w[4] = {ring[k].raw.x, ring[k].raw.y, ring[k].raw.z, ring[k].raw.w};
        const float s_0 = ring[k].s0, s_1 = ring[k].s1, vrow = ring[k].v;
        asm volatile("" ::: "memory");  // read the head's vectors from LDS here, not once
        float kk[E], al[E];
        loadv(lk, kk);
        if constexpr (vector_decay(MIXER)) loadv(lk + 2 * DK, al);
        float d[E];
        // decayed dequantized values (exactly the rounded c*(s*alpha) / (c*s)*alpha_j)
        if constexpr (vector_decay(MIXER)) {
          dequant_lane<BITS, E>(w, s_0, s_1, d);
#pragma unroll
          for (int j = 0; j < E; ++j) d[j] *= al[j];
        } else {
          dequant_lane<BITS, E>(w, s_0 * alpha_s, s_1 * alpha_s, d);
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
        // nothing of the slot is live any more
        ring[k] = load(rb, rh, rr0, trip + 1 == TRIPS && !next_same ? -1 : rbase + k);
        float qq[E];
        loadv(lk + DK, qq);
        const float o = row_sum<LPR>(lane_dot(d, qq));
        float s0 = s_0, s1 = s_1;
        const uint32_t block0 = (uint32_t)((row * DK + col0) >> 4);
        const uint4 packed = quantize_lane<BITS, RND, E, LPG, true>(d, key, block0, w, s0, s1);
        if (store_ok) {
          st_stream(reinterpret_cast<uint4*>(hcodes + (uint32_t)(row * Gm::ROW_BYTES + lr * 16)), packed);
          if constexpr (two_groups) {
            st_stream(hscales + (uint32_t)(row * ngr + gcol), s0);
            st_stream(hscales + (uint32_t)(row * ngr + gcol + 1), s1);
          } else if (lr % LPG == 0) {
            st_stream(hscales + (uint32_t)(row * ngr + gcol), s0);
          }
          if (oh && lr == 0) oh[row] = o;
        }
        // nxt's vectors into its LDS buffer, half a trip after they were loaded
        if (trip == 0 && k == kPrefetch / 2 && ps.nxt.b >= 0) {
          asm volatile("" ::: "memory");
          ps.st.store(lds_next);
        }
      }
    }
    advance<MIXER, DK>(p, ps);
    if (!next_same) return;  // the ring holds nothing of the new cur
  }
}

template <int MIXER, int RND, int DK, int G>
__global__ __launch_bounds__(kThreads) void step_persist_kernel(const KParams p) {
  using St = Stage<MIXER, DK>;
  __shared__ float4 lds[2][St::LDS4];
  PState<MIXER, DK> ps;
  // the first unit's data straight into LDS buffer 0, the second's into the
  // stage (LDS buffer 1 during the first unit)
  ps.u = blockIdx.x;
  ps.slot = 0;
  ps.cur = decode_unit<DK>(p, ps.u);
  ps.nxt = decode_unit<DK>(p, ps.u + gridDim.x);
  if (ps.cur.b >= 0) {
    ps.st.load(p, ps.cur.b * p.H + ps.cur.h);
    ps.st.store(lds[0]);
  }
  if (ps.nxt.b >= 0) ps.st.load(p, ps.nxt.b * p.H + ps.nxt.h);
  __syncthreads();
  persist_class<MIXER, RND, DK, 8, G>(p, ps, lds);
  persist_class<MIXER, RND, DK, 4, G>(p, ps, lds);
}

// Compute units of the current device (cached per device).
inline int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (dev < 64) cache[dev] = cus;
  return cus;
}

// Launch the persistent step: one wave per resident slot of the chip (or
// one per unit when there are fewer units).  It applies where the kernel
// fits four waves per SIMD: with three, the grid of 3 waves per SIMD does
// not divide the units of the usual shapes evenly (e.g. 8192 units over 3072
// waves), and the waves left with an extra unit end alone; those kernels
// (and states without a persistent layout) run the sliced step instead.
template <int MIXER, int RND, int DK, int G>
bool launch_persist(const KParams& p, hipStream_t s, hipError_t* err) {
  if (!p.persist) return false;
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(step_persist_kernel<MIXER, RND, DK, G>), kThreads,
            0) != hipSuccess)
      n = 0;
    return n;
  }();
  if (occ < 16) return false;  // fewer than 4 waves per SIMD
  const int64_t waves = std::min<int64_t>((int64_t)device_cus() * occ, p.n_units);
  if (waves < 1) return false;
  step_persist_kernel<MIXER, RND, DK, G><<<(unsigned)waves, kThreads, 0, s>>>(p);
  *err = hipGetLastError();
  return true;
}

}  // namespace
}  // namespace qs
