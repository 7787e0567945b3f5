/*
 * qstate.h — C ABI of the quantized recurrent-state decode library (gfx950).
 *
 * One decode step of a linear-attention / state-space layer whose fixed-size
 * recurrent state S[b][h][dv][dk] is stored in INT8 or packed INT4 between
 * steps.  Each step dequantizes the stored state, applies the full-precision
 * update, reads out o = S'q and writes the state back through the quantizer.
 *
 * Sources (web pages on the method):
 *  - "Quantizing Recurrent Language Models Is Easier Than You Think" (LoReS
 *    blog), Fig. 1 "Recurrent state: overwrite": the recurrence takes q, k, v
 *    and the previous state and overwrites the whole state through a
 *    quantizer after each update.
 *  - same page, "LoReS: State Quantization": updates stay in full precision,
 *    only the state kept between decode steps is quantized; value-axis (row)
 *    scale groups (1/4), decay-based per-head bits (2/4), stochastic rounding
 *    (3/4); symmetric absmax scale s = max|S_G| / r, r = 2^(b-1) - 1
 *    (Prop. "per-channel readout error" and 4/4 animation details).
 *  - same page, Prop. "decaying error": delta correction with unit-norm keys
 *    and 0 < beta < 2, decay |alpha|_inf < 1; Prop. "repeated quantization",
 *    animation: the scalar-decay form S_t = alpha S_{t-1} + a v_t k_t^T.
 *  - "Preserving Updates in Low-Bit Recurrent State Quantization" abstract:
 *    Gated DeltaNet, GLA, Mamba2 and RetNet as the recurrences in question,
 *    with savings measured against FP32 states.
 *
 * Semantics (exact, shared with the CPU reference; every FP32 operation below
 * is one IEEE-754 binary32 operation with round-to-nearest-even unless noted):
 *
 *  Per head (b,h) with bit width n (4 or 8), r = 2^(n-1) - 1, and per value
 *  row i (0 <= i < dv), key column j (0 <= j < dk), the element's scale
 *  group is (i, g = j / G) for value-axis groups and (g = i / G, j) for
 *  key-axis groups; s_ig below stands for that group's scale:
 *   1. decayed dequantized row
 *        GDN, SCALAR: d_j = c_ij * (s_ig * alpha)
 *        GLA, KDA:    d_j = (c_ij * s_ig) * alpha_j
 *        (FP32 state: d_j = S_ij * alpha   or   S_ij * alpha_j)
 *   2. write weight
 *        GDN, KDA: u = dot(d, k);  w = beta * (v_i - u)
 *        GLA:      w = v_i
 *        SCALAR:   w = beta * v_i        (beta carries Mamba2's dt)
 *   3. S'_ij = fma(w, k_j, d_j)
 *      so GDN computes S' = alpha S (I - beta k k^T) + beta v k^T,
 *      GLA S' = S diag(alpha) + v k^T, SCALAR S' = alpha S + dt v k^T,
 *      KDA S' = S diag(alpha) (I - beta k k^T) + beta v k^T (LoReS blog,
 *      Table 1 "KDA"; vector gates of Prop. "decaying error").
 *   4. o_i = dot(S'_i, q)       (from the full-precision S', before requant)
 *   5. m = max over the group of |S'|;  m == 0: s' = 0, inv = 0, codes 0;
 *      else s' = m / r (correctly rounded), inv = the largest float with
 *      inv * m <= r (r / m rounded toward zero), so |S' * inv| <= r.
 *   6. RTN: code = round-half-even(S'_ij * inv)   (exact product)
 *      SR:  x = S'_ij * inv (exact product) rounded to the nearest multiple
 *           of 2^-f, ties to even, f = 16 for 4-bit and 15 for 8-bit codes;
 *           code = floor(x + R16_ij * 2^-16).  Over R16 the mean code is
 *           exactly x, within 2^-(f+1) of S'_ij * inv.
 *      No clamp is ever active: both stay within [-r, r].
 *      BDR ("Preserving Updates" abstract: reversed elements are rounded
 *      toward their update, with no extra storage): n = the RTN code,
 *      p = c_ij * s_ig (the element's stored value before the step, one
 *      FP32 product), t = n * s'_ig (FP32).  If S'_ij > p and t < p, n += 1;
 *      if S'_ij < p and t > p, n -= 1; then clamp n to [-r, r].  An import
 *      (no stored value before it) rounds to nearest.
 *   dot(x, y): 16-element chunks, each accumulated p = fma(x_j, y_j, p) from
 *   p = 0 in ascending j, then a pairwise tree over the chunk partials
 *   (((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)) for dk = 128).
 *
 *  Stochastic-rounding bits R16_ij (counter-based, a pure function of
 *  (seed, layer, step, b, h, element)):
 *   key  = F(F(F(F(F(0 ^ seed + g) ^ layer + g) ^ step + g) ^ b + g) ^ h + g),
 *          i.e. x = F((x XOR v) + g) for v = seed, layer, step, b, h from
 *          x = 0, where F is the SplitMix64 output function and
 *          g = 0x9E3779B97F4A7C15;  K = (uint32)(key >> 32) ^ (uint32)key.
 *   e = i*dk + j (element index within the head), block q = e / 16,
 *   pair p = (e % 16) / 2.
 *   z_q = fmix32(K ^ q)                  (MurmurHash3 32-bit finalizer)
 *   W   = L^p (z_q), where L steps the two 16-bit halves of a word as
 *         linear congruential generators: low (0xC36D x + 13849) mod 2^16,
 *         high (0xC23D x + 13849) mod 2^16 (each of full period 2^16).
 *   R16 = W & 0xFFFF for even e, W >> 16 for odd e.
 *  Each quantization event (a step, or an FP32 import) uses the handle's
 *  current step counter and then increments it.
 *
 * Layout (all device buffers are caller-owned, 16-byte aligned, contiguous):
 *   q, k            float [B][H][dk]
 *   v, o            float [B][H][dv]
 *   alpha           float [B][H]      (GDN, SCALAR)  or  [B][H][dk] (GLA, KDA)
 *   beta            float [B][H]      (GDN, KDA: beta, SCALAR: dt; GLA: unused)
 *   codes           heads in (b, h) order; head (b,h) starts at byte
 *                   b*P + sum_{h'<h} dv*R_{h'}, P = sum_h dv*R_h, where R_h
 *                   is a row's bytes: 16 per INT8 and 8 per INT4 block of
 *                   16 key columns (dk*n_h/8 for a head of one width n_h).
 *                   Rows follow each other inside a head; a row holds its
 *                   blocks in column order.  INT8: int8 two's complement.
 *                   INT4: two's-complement nibbles, within a block byte t/2
 *                   holds even column t in bits 0..3, odd t in bits 4..7.
 *   scales          float [B][H][dv][dk/G] (value axis) or [B][H][dv/G][dk]
 *                   (key axis)
 *   FP32 state      float [B][H][dv][dk]  (fp32_state = 1)
 *
 * Pure-write window (cfg.window = W > 0; "Low-Bit GDN Recurrent-State
 * Quantization ... Pure-Write Sliding Windows", abstract): the full state of
 * a head is H + sum_t a_t b_t^T, H the low-bit state above and (a_t, b_t) the
 * last W pure writes stored as OCP E4M3 vectors with one absmax scale each
 * (s = max|x| / 448, inv = the largest float with inv * max|x| <= 448, code =
 * E4M3 nearest-even of x * inv, value = decode(code) * s).  At counter t the
 * pair in slot t mod W is the oldest; a step at counter t:
 *   1. keys: b'_s = A^T b_s for every slot s: d_j = b_sj * alpha (or
 *      alpha_j); with the delta rule b'_sj = fma(-(beta * dot(d, k)), k_j,
 *      d_j), else b'_sj = d_j;  c_s = dot(b'_s, q);
 *   2. H'_ij = fma(a_o,i, b'_o,j, fma(-(beta * u_i), k_j, d_ij)) with the
 *      leaving pair o = t mod W (without the delta rule: fma(a_o,i, b'_o,j,
 *      d_ij)); d, u as in steps 1-2 above;
 *   3. new pair in slot o: a = w v (w = beta, or 1 for GLA), b = k;
 *   4. o_i = dot(H'_i, q), then fma(a_s,i, c_s, .) over the other slots
 *      oldest first, then fma(a_new,i, dot(k, q), .);
 *   5. H' requantized as above; the kept pairs' b' and the new pair
 *      re-encoded.
 * Low-rank bypass (window_merge = 1; "Preserving Updates in Low-Bit
 * Recurrent State Quantization", abstract: small updates accumulate in a
 * compact low-rank buffer whose sufficiently large elements are merged into
 * the state periodically).  The buffer is the same W pairs (rank <= W),
 * filled and propagated as above; the difference is the merge.  A step at a
 * counter t with t mod W != 0 is the window step above (its slot is always
 * empty then).  The step at t mod W == 0 merges the whole buffer instead:
 *   m_ij = sum over the W pairs oldest first of fma(a_s,i, b'_s,j, m_ij)
 *   from 0; T_ij = fma(-(beta * u_i), k_j, d_ij) with the delta rule, else
 *   d_ij; H'_ij = T_ij + m_ij if |m_ij| >= lrb_threshold * s_ig (s_ig the
 *   element's group scale before the step), else T_ij (the element drops);
 *   o_i = fma(a_new,i, dot(k, q), dot(H'_i, q)); the new pair takes slot 0
 *   and every other slot is emptied (zero codes and scales).
 *
 * Window area per head (after the codes, 16-byte aligned, heads in (b, h)
 * order, each align16(dv*W + 2*(W*dk + 8*W)) bytes): a codes [dv][W], then two
 * copies of (b codes [W][dk], scales [W][2] = (s_a, s_b)); counter t reads
 * copy t & 1 and writes copy (t + 1) & 1.  An import empties the window
 * (zero codes and scales, which contribute exactly nothing); export and
 * readout return the full state.
 *
 * Range: state magnitudes stay below 2^120 (far beyond any FP32 recurrence
 * that does not overflow within a few steps).
 *
 * Ownership: the library never allocates or frees device memory; a handle
 * owns only host memory.  The state is updated in place.  o must not alias
 * any input.  Calls are asynchronous on the given HIP stream (NULL = the
 * default stream); device faults surface at the caller's next
 * synchronisation.  A handle must not be used from two threads at once.
 *
 * Errors: every call returns QSTATE_OK (0) or a negative QSTATE_E_* code.
 * Argument checks are synchronous and happen before any launch; a failed
 * check leaves the handle and the buffers untouched.
 */
#ifndef QSTATE_H
#define QSTATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QSTATE_OK = 0,
  QSTATE_E_INVALID = -1,     /* null/misaligned pointer, bad size or enum  */
  QSTATE_E_UNSUPPORTED = -2, /* valid but not built: shape, group, heads   */
  QSTATE_E_LAUNCH = -3,      /* the HIP runtime refused a launch           */
  QSTATE_E_NOMEM = -4        /* host allocation of the handle failed       */
};

typedef enum {
  QSTATE_GDN = 0,    /* S' = a S (I - b k k^T) + b v k^T   (Gated DeltaNet) */
  QSTATE_GLA = 1,    /* S' = S diag(alpha[dk]) + v k^T     (beta unused)    */
  QSTATE_SCALAR = 2, /* S' = a S + b v k^T   (Mamba2 with b = dt; RetNet)   */
  QSTATE_KDA = 3     /* S' = S diag(alpha[dk]) (I - b k k^T) + b v k^T      */
} qstate_mixer;

/* Shape of a scale group (LoReS blog, "Scale grouping"). */
typedef enum {
  QSTATE_VALUE_AXIS = 0, /* G key columns of one value row: scales [dv][dk/G]
                            (the default: one output channel per group)     */
  QSTATE_KEY_AXIS = 1    /* G value rows of one key column: scales [dv/G][dk] */
} qstate_group_axis;

typedef enum {
  QSTATE_RTN = 0, /* round to nearest, ties to even                        */
  QSTATE_SR = 1,  /* stochastic rounding (counter-based bits)              */
  QSTATE_BDR = 2  /* bounded directional rounding (nearest for an import)  */
} qstate_rounding;

typedef struct {
  int32_t batch;            /* B >= 1                                         */
  int32_t heads;            /* H, 1..256                                      */
  int32_t dk;               /* key dim (columns): 64, 128 or 256              */
  int32_t dv;               /* value dim (rows): 1..4096                      */
  int32_t group;            /* G: 16, 32, 64 or 128; divides dk (value axis)
                               or dv (key axis)                               */
  int32_t mixer;            /* qstate_mixer                                   */
  int32_t rounding;         /* qstate_rounding                                */
  int32_t fp32_state;       /* 1: unquantized FP32 state (baseline); the
                               group, rounding and head_bits are ignored      */
  const uint8_t* head_bits; /* host [heads], each 4 or 8; copied at create;
                               NULL = all 8                                   */
  uint64_t seed;            /* stochastic-rounding key                        */
  uint32_t layer;           /* stochastic-rounding key                        */
  int32_t group_axis;       /* qstate_group_axis; 0 = value axis (default)    */
  const uint8_t* channel_bits; /* host [heads][dk/16] or NULL: the width (4 or 8)
                               of each block of 16 key columns, overriding
                               head_bits (LoReS 2/4: more bits for the
                               slowest-decaying channels; order channels so
                               that slow ones share blocks).  Value-axis
                               groups may not mix widths.  Copied at create. */
  int32_t window;           /* W = 0 (none), 4, 8 or 16: keep the last W pure
                               writes of each head as FP8 pairs beside its
                               low-bit state (value-axis groups, heads of one
                               width); their area follows the codes in the
                               codes buffer (see the pure-write window below) */
  int32_t window_merge;     /* with W > 0: 0 = pure-write window (the oldest
                               pair merges at every step); 1 = low-rank bypass
                               (every W steps the whole buffer merges, see
                               below)                                         */
  float lrb_threshold;      /* low-rank bypass: a buffer element merges when
                               its magnitude is at least this times its group
                               scale; finite, >= 0 (0 merges every element)  */
} qstate_config;

typedef struct qstate qstate; /* opaque; host-side metadata only */

/* Sizes in bytes of the caller-owned state buffers for cfg.  For an FP32
 * state, *codes_bytes is the FP32 state size and *scales_bytes is 0. */
int qstate_state_bytes(const qstate_config* cfg, size_t* codes_bytes,
                       size_t* scales_bytes);

/* Validate cfg, record the two state buffers (device pointers; scales_dev
 * ignored for an FP32 state) and return a handle with step counter 0.
 * Host only: no device work, no device allocation. */
int qstate_create(const qstate_config* cfg, void* codes_dev, void* scales_dev,
                  qstate** out);

/* Import: quantize the FP32 state S_dev [B][H][dv][dk] into the handle's
 * codes and scales (steps 5-6 above, counter = current step), then step++.
 * For an FP32 handle this is a device copy and the counter is unchanged. */
int qstate_load_fp32(qstate* h, const float* S_dev, void* stream);

/* The decode step (steps 1-6 above) for every head, in place; o may be NULL.
 * alpha: [B][H] (GDN, SCALAR) or [B][H][dk] (GLA, KDA); beta: [B][H] (GDN,
 * SCALAR, KDA), ignored for GLA.  Increments the step counter. */
int qstate_step(qstate* h, const float* q, const float* k, const float* v,
                const float* alpha, const float* beta, float* o, void* stream);

/* Readout without update: o_i = dot(c_ij * s_ig, q) (FP32 state: dot(S, q)).
 * The counter is unchanged. */
int qstate_readout(qstate* h, const float* q, float* o, void* stream);

/* Export the dequantized state S_ij = c_ij * s_ig into S_dev (FP32 state:
 * a copy).  The counter is unchanged. */
int qstate_store_fp32(qstate* h, float* S_dev, void* stream);

/* Step counter (the stochastic-rounding counter used by the next event). */
int qstate_get_step(const qstate* h, uint64_t* step);
int qstate_set_step(qstate* h, uint64_t step);

/* Free the handle (host memory only).  NULL is accepted. */
int qstate_destroy(qstate* h);

/* Static message for a status code. */
const char* qstate_strerror(int status);

/* Decay-based bit allocation (LoReS 2/4: more bits for the slowest-decaying
 * heads or channels).  retention[h] is larger for slower decay (e.g. alpha_h,
 * exp(-softplus(A_h)), or the mean retention of a group of key channels when
 * allocating channel_bits); `heads` is the number of entries.
 *   mode 0: out[h] = hi if retention[h] > thr_or_frac else lo
 *   mode 1: the round(thr_or_frac * heads) heads with the largest retention
 *           get hi (ties: the lower head index first), the rest lo. */
int qstate_bits_by_decay(const float* retention, int heads, int mode,
                         float thr_or_frac, uint8_t lo_bits, uint8_t hi_bits,
                         uint8_t* out_bits);

#ifdef __cplusplus
}
#endif

#endif /* QSTATE_H */
