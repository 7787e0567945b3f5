/*
 * oracle.h — plain single-threaded CPU reference of the quantized
 * recurrent-state decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant
 * generator with the HIP library; the two implement the same written
 * semantics independently.
 *
 * Every function follows the pages on the method ("Quantizing Recurrent
 * Language Models Is Easier Than You Think", LoReS blog, section "LoReS:
 * State Quantization" and Fig. 1) plus the readings stated where the pages
 * are silent; the citation sits on each definition in oracle.cpp.
 *
 * Parity pins: see tests/test_oracle_*.py.  Each function below is pinned by
 * a closed form, a brute-force search, a published test vector, an exact
 * mathematical property or a statistical property of the method.  The
 * particular 16-element-chunk summation order of dot() is a reading (any
 * fixed order is equally correct); its result is pinned only to the exact
 * dot product within the FP32 error bound.
 */
#ifndef QSTATE_ORACLE_H
#define QSTATE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t B, H, dk, dv, G;
  int32_t mixer;    /* 0 Gated DeltaNet, 1 GLA, 2 scalar decay (Mamba2), 3 KDA */
  int32_t rounding; /* 0 round-to-nearest-even, 1 stochastic,
                       2 bounded directional (nearest for an import)     */
  uint64_t seed;
  uint32_t layer;
  int32_t axis;     /* 0 value-axis groups (G key columns of one row, scales
                       [dv][dk/G]); 1 key-axis groups (G value rows of one
                       column, scales [dv/G][dk])                       */
  int32_t window;   /* pair buffer length W (0: none)                   */
  int32_t window_merge; /* 0 pure-write window: the oldest pair merges at
                           every step; 1 low-rank bypass: every W steps all
                           pairs merge, elements below the threshold drop */
  float lrb_threshold;  /* low-rank bypass: an element merges when its
                           magnitude is at least this times its group scale */
} oracle_cfg;

/* ---- counter-based random bits ---- */
uint64_t oracle_splitmix64_output(uint64_t z);
uint32_t oracle_fmix32(uint32_t h);
uint32_t oracle_lcg16x2(uint32_t w);
uint32_t oracle_head_key(uint64_t seed, uint32_t layer, uint64_t step,
                         uint32_t b, uint32_t h);
uint32_t oracle_sr_bits(uint32_t key, uint64_t element);

/* ---- scalar pieces ---- */
float oracle_dot(const float* x, const float* y, int n);
void oracle_group_scale(float m, int r, float* s, float* inv);
int oracle_round_rtn(float x, float inv);
int oracle_round_sr(float x, float inv, uint32_t r16, int bits);
int oracle_round_bdr(float x, float inv, float s_new, float prev, int r);
/* distance (code units) from x*inv to the nearest point where the code
 * changes; stochastic != 0: stochastic rounding with the given r16 */
double oracle_threshold_distance(float x, float inv, int stochastic, uint32_t r16, int bits);

/* ---- layout ----
 * Bit widths come per block of 16 key columns: block_bits of one head holds
 * dk/16 entries (4 or 8); the batch functions take [H][dk/16].  A row stores
 * its blocks in column order (16 bytes per INT8 block, 8 per INT4 block). */
size_t oracle_codes_bytes(const oracle_cfg* c, const uint8_t* block_bits);
size_t oracle_head_offset(const oracle_cfg* c, const uint8_t* block_bits,
                          int b, int h);
int oracle_get_code(const uint8_t* head_codes, int bits, int64_t e);
void oracle_set_code(uint8_t* head_codes, int bits, int64_t e, int code);

/* ---- one head (b, h): buffers point at that head's data ---- */
/* alpha: 1 value (GDN, scalar) or dk values (GLA, KDA); beta: beta (GDN,
 * KDA) / dt (scalar), unused for GLA.
 * o, pre, tdist may be NULL.  pre receives S' [dv][dk] before requantizing;
 * tdist receives, per element, the distance in code units from the exact
 * pre-rounding value S'*inv to the nearest point where its code changes
 * (oracle_threshold_distance). */
void oracle_head_step(const oracle_cfg* c, int b, int h, const uint8_t* block_bits,
                      uint8_t* codes, float* scales, const float* q,
                      const float* k, const float* v, const float* alpha,
                      float beta, float* o, uint64_t step, float* pre,
                      double* tdist);
void oracle_head_step_fp32(const oracle_cfg* c, float* S, const float* q,
                           const float* k, const float* v, const float* alpha,
                           float beta, float* o);
void oracle_head_quantize(const oracle_cfg* c, int b, int h, const uint8_t* block_bits,
                          const float* S, uint8_t* codes, float* scales,
                          uint64_t step, double* tdist);
void oracle_head_dequantize(const oracle_cfg* c, const uint8_t* block_bits,
                            const uint8_t* codes, const float* scales,
                            float* S);
void oracle_head_readout(const oracle_cfg* c, const uint8_t* block_bits, const uint8_t* codes,
                         const float* scales, const float* q, float* o);

/* ---- every head of a [B][H] batch, arrays in the library's layout ---- */
void oracle_step(const oracle_cfg* c, const uint8_t* block_bits,
                 uint8_t* codes, float* scales, const float* q,
                 const float* k, const float* v, const float* alpha,
                 const float* beta, float* o, uint64_t step);
void oracle_step_fp32(const oracle_cfg* c, float* S, const float* q,
                      const float* k, const float* v, const float* alpha,
                      const float* beta, float* o);
void oracle_quantize(const oracle_cfg* c, const uint8_t* block_bits,
                     const float* S, uint8_t* codes, float* scales,
                     uint64_t step);
void oracle_dequantize(const oracle_cfg* c, const uint8_t* block_bits,
                       const uint8_t* codes, const float* scales, float* S);
void oracle_readout(const oracle_cfg* c, const uint8_t* block_bits,
                    const uint8_t* codes, const float* scales, const float* q,
                    float* o);

/* the same on the listed heads only (indices b*H + h; other heads untouched) */
void oracle_step_heads(const oracle_cfg* c, const uint8_t* block_bits, int n,
                       const int32_t* heads, uint8_t* codes, float* scales, const float* q,
                       const float* k, const float* v, const float* alpha, const float* beta,
                       float* o, uint64_t step);
void oracle_step_fp32_heads(const oracle_cfg* c, int n, const int32_t* heads, float* S,
                            const float* q, const float* k, const float* v,
                            const float* alpha, const float* beta, float* o);
void oracle_quantize_heads(const oracle_cfg* c, const uint8_t* block_bits, int n,
                           const int32_t* heads, const float* S, uint8_t* codes,
                           float* scales, uint64_t step);

/* ---- pure-write window: W FP8 (E4M3) pairs per head, see oracle.cpp ---- */
float oracle_fp8_decode(uint8_t code);
uint8_t oracle_fp8_encode(float x);
size_t oracle_window_bytes(const oracle_cfg* c);
void oracle_head_step_pw(const oracle_cfg* c, int b, int h, const uint8_t* block_bits,
                         uint8_t* codes, float* scales, uint8_t* window,
                         const float* q, const float* k, const float* v,
                         const float* alpha, float beta, float* o, uint64_t step,
                         float* pre, double* tdist);
void oracle_head_window_state(const oracle_cfg* c, const uint8_t* block_bits,
                              const uint8_t* codes, const float* scales,
                              const uint8_t* window, uint64_t step, float* S);
void oracle_head_window_readout(const oracle_cfg* c, const uint8_t* block_bits,
                                const uint8_t* codes, const float* scales,
                                const uint8_t* window, uint64_t step, const float* q,
                                float* o);

/* ---- decay-based bit allocation (LoReS 2/4) ---- */
int oracle_bits_by_decay(const float* retention, int heads, int mode,
                         float thr_or_frac, uint8_t lo, uint8_t hi,
                         uint8_t* out);

#ifdef __cplusplus
}
#endif

#endif
