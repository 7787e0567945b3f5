// oracle.cpp — plain, slow, single-threaded CPU reference of the quantized
// recurrent-state decode step.  TEST INFRASTRUCTURE ONLY (see oracle.h): the
// product library never includes, links or calls it.
//
// Build: g++ -std=c++17 -O2 -ffp-contract=off -fPIC -shared (no fast-math).
// Float arithmetic is IEEE binary32 with round-to-nearest-even; std::fma is
// the correctly rounded fused multiply-add; products that must be exact are
// formed in double, where the product of two floats is exact.

#include "oracle.h"

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstring>
#include <numeric>
#include <vector>

namespace {

const int kMixerGDN = 0, kMixerGLA = 1, kMixerKDA = 3;

// Per-key-channel decay (GLA, KDA) versus one decay per head (GDN, scalar).
bool vector_decay(int mixer) { return mixer == kMixerGLA || mixer == kMixerKDA; }
// Delta correction w = beta * (v - d.k) (GDN, KDA).
bool delta_rule(int mixer) { return mixer == kMixerGDN || mixer == kMixerKDA; }
const int kRoundSR = 1, kRoundBDR = 2;
const int kAxisKey = 1;  // scale groups along the value axis of one key column

int qmax(int bits) { return (1 << (bits - 1)) - 1; }  // r = 2^(b-1) - 1

}  // namespace

extern "C" {

// ---------------------------------------------------------------------------
// Counter-based random bits for stochastic rounding.
// The pages ask only for conditionally unbiased rounding (LoReS 3/4,
// "Rounding"); the bits are a pure function of (seed, layer, step, b, h,
// element) so that any implementation draws the same ones.
// ---------------------------------------------------------------------------

// SplitMix64 output function (Steele, Lea & Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014; constants of Stafford's
// "Mix13" variant as used by SplitMix64).
uint64_t oracle_splitmix64_output(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// 32-bit finalizer of MurmurHash3 (Appleby, public domain).
uint32_t oracle_fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// One step of the two 16-bit linear congruential streams that share a 32-bit
// word (Lehmer's mixed generator x' = (a x + c) mod 2^16, one per half; Knuth,
// TAOCP vol. 2, 3.2.1).  Low half a = 0xC36D, high half a = 0xC23D: both are
// 5 mod 8, so with c odd each half has full period 2^16 (Hull-Dobell theorem),
// and both were picked by the spectral test (TAOCP 3.3.4), with normalized
// figures of merit of at least 0.75 in 2 to 5 dimensions.  c = 13849, about
// (1/2 - sqrt(3)/6) 2^16, Knuth's increment for the smallest serial
// correlation bound (TAOCP 3.3.3).
uint32_t oracle_lcg16x2(uint32_t w) {
  const uint32_t lo = w & 0xFFFFu;
  const uint32_t hi = w >> 16;
  const uint32_t lo_next = (0xC36Du * lo + 13849u) & 0xFFFFu;
  const uint32_t hi_next = (0xC23Du * hi + 13849u) & 0xFFFFu;
  return lo_next | (hi_next << 16);
}

// Per-(seed, layer, step, b, h) key: each field is absorbed through the
// SplitMix64 output function, x = F((x ^ v) + golden), starting from x = 0.
uint32_t oracle_head_key(uint64_t seed, uint32_t layer, uint64_t step,
                         uint32_t b, uint32_t h) {
  const uint64_t golden = 0x9E3779B97F4A7C15ull;
  const uint64_t fields[5] = {seed, layer, step, b, h};
  uint64_t x = 0;
  for (uint64_t v : fields) x = oracle_splitmix64_output((x ^ v) + golden);
  return (uint32_t)(x >> 32) ^ (uint32_t)x;
}

// The 16 random bits of element e of a head: blocks of 16 elements share one
// hashed seed word, and the 8 element pairs of a block walk its two
// linear congruential streams.
uint32_t oracle_sr_bits(uint32_t key, uint64_t element) {
  const uint32_t block = (uint32_t)(element / 16);
  const int pair = (int)((element % 16) / 2);
  uint32_t w = oracle_fmix32(key ^ block);
  for (int p = 0; p < pair; ++p) w = oracle_lcg16x2(w);
  return (element % 2 == 0) ? (w & 0xFFFFu) : (w >> 16);
}

// ---------------------------------------------------------------------------
// Scalar pieces.
// ---------------------------------------------------------------------------

// Dot product in FP32: the pages fix no order, so one is written down.
// Consecutive 16-element chunks are each accumulated with fused multiply-adds
// from 0 in ascending index; the chunk partials are then summed pairwise,
// adjacent pairs first, an odd last partial carried to the next level.
float oracle_dot(const float* x, const float* y, int n) {
  std::vector<float> part;
  for (int c0 = 0; c0 < n; c0 += 16) {
    float p = 0.0f;
    for (int j = c0; j < std::min(n, c0 + 16); ++j) p = std::fma(x[j], y[j], p);
    part.push_back(p);
  }
  if (part.empty()) return 0.0f;
  while (part.size() > 1) {
    std::vector<float> next;
    for (size_t i = 0; i + 1 < part.size(); i += 2) next.push_back(part[i] + part[i + 1]);
    if (part.size() % 2 == 1) next.push_back(part.back());
    part.swap(next);
  }
  return part[0];
}

// Symmetric absmax scale of a group (LoReS 4/4: s = |S_G|_inf / r, with
// r = 2^(b-1) - 1 from Prop. "per-channel readout error").  The scaled value
// is formed with inv, the largest float whose product with m does not exceed
// r, so that no scaled value leaves [-r, r].  An all-zero group gets s = 0.
void oracle_group_scale(float m, int r, float* s, float* inv) {
  if (m == 0.0f) {
    *s = 0.0f;
    *inv = 0.0f;
    return;
  }
  *s = m / (float)r;
  float v = (float)((double)r / (double)m);
  while ((double)v * (double)m > (double)r) v = std::nextafter(v, 0.0f);
  *inv = v;
}

// Round-to-nearest (LoReS 3/4 "RTN"): nearest integer to the exact product,
// ties to even.  The double product of two floats is exact.
int oracle_round_rtn(float x, float inv) {
  return (int)std::rint((double)x * (double)inv);
}

// Stochastic rounding (LoReS 3/4, conditionally unbiased).  The exact
// product x*inv is first rounded to the nearest multiple of 2^-f, ties to
// even, with f = 16 fraction bits for 4-bit codes and 15 for 8-bit codes;
// the code is floor(that + r16 / 2^16).  Over the 2^16 equally likely r16 the
// mean code is exactly the f-bit value, within 2^-(f+1) of x*inv.  The double
// product of two floats is exact, and so are the power-of-two scalings.
int oracle_round_sr(float x, float inv, uint32_t r16, int bits) {
  const int f = bits == 8 ? 15 : 16;
  const double n = std::nearbyint(std::ldexp((double)x * (double)inv, f));
  const double t = std::ldexp(n, 16 - f) + (double)(r16 & 0xFFFFu);
  return (int)std::floor(t / 65536.0);
}

// Bounded directional rounding ("Preserving Updates", abstract: reversed
// elements are rounded toward their update, with no extra storage).  The
// element's stored value was prev = c*s before the step and its full-precision
// update takes it to x; round-to-nearest gives the code n whose stored value is
// n*s_new.  When prev lies strictly between n*s_new and x, the stored value
// moved against the update: take one grid step toward the update (the other
// neighbour of x*inv, so the rounding error stays below one step), then clamp
// to [-r, r].  A lost update (n*s_new == prev) or no update (x == prev) is
// left as rounded.
int oracle_round_bdr(float x, float inv, float s_new, float prev, int r) {
  int n = oracle_round_rtn(x, inv);
  const float stored = (float)n * s_new;
  const bool up = x > prev, down = x < prev;
  if (up && stored < prev) n += 1;
  if (down && stored > prev) n -= 1;
  return std::max(-r, std::min(r, n));
}

// Distance, in code units, from the pre-rounding value t = x*inv (exact) to
// the nearest value of t at which the element's code changes, its random
// bits held fixed.  Parity between two implementations of the quantizer
// exempts a differing code only when this distance is tiny.
//  * Round to nearest (and bounded directional rounding, which starts from
//    it): the code steps from n to n + 1 at t = n + 1/2, for n in [-r, r-1].
//  * Stochastic rounding with f fraction bits: the code is
//    floor((N 2^(16-f) + r16) / 2^16) with N = RN(t 2^f), and N steps at the
//    half-integers of t 2^f.  The code reaches n where N first satisfies
//    N 2^(16-f) + r16 >= n 2^16.  For f = 16 that step sits at
//    t = n - (r16 + 1/2) 2^-16; for f = 15 the first such N is
//    ceil((n 2^16 - r16) / 2), and the step sits half a unit of 2^-15 below
//    it: t = n - (r16 + 1) 2^-16 for even r16 and n - r16 2^-16 for odd r16,
//    that is t = n - (r16 | 1) 2^-16.  So u = t + c 2^-16 (c = r16 + 1/2 or
//    r16 | 1) crosses an integer n in [-r+1, r] exactly where the code
//    steps from n - 1 to n (the clamp to [-r, r] removes the steps to r + 1
//    and from -r - 1).
// The double sums carry t's 48 significant bits; any rounding in them is
// below 2^-50 code units.
double oracle_threshold_distance(float x, float inv, int stochastic, uint32_t r16, int bits) {
  const int r = qmax(bits);
  const double t = (double)x * (double)inv;
  if (!stochastic) {
    const double h = std::max(-r + 0.5, std::min(r - 0.5, std::floor(t) + 0.5));
    return std::fabs(t - h);
  }
  const double c = bits == 8 ? (double)((r16 & 0xFFFFu) | 1u) : (double)(r16 & 0xFFFFu) + 0.5;
  const double u = t + c / 65536.0;
  const double n = std::max((double)(-r + 1), std::min((double)r, std::nearbyint(u)));
  return std::fabs(u - n);
}

// ---------------------------------------------------------------------------
// Layout.  Bit widths are given per block of 16 key columns of a head
// (LoReS 2/4: more bits for the slowest-decaying heads or channels; a head
// with one width has all its blocks alike).  A value row stores its blocks in
// column order, 16 bytes for an INT8 block and 8 for an INT4 block; rows are
// contiguous, heads follow each other in (b, h) order.  INT8 codes are int8;
// INT4 codes are two's-complement nibbles, even column in the low nibble.
// ---------------------------------------------------------------------------

namespace {

struct Layout {
  int nb = 0;            // blocks of 16 key columns
  int bits[16] = {};     // width of each block
  size_t off[16] = {};   // byte offset of each block inside a row
  size_t row_bytes = 0;
};

Layout head_layout(const oracle_cfg* c, const uint8_t* block_bits) {
  Layout L;
  L.nb = c->dk / 16;
  for (int q = 0; q < L.nb; ++q) {
    L.bits[q] = block_bits[q];
    L.off[q] = L.row_bytes;
    L.row_bytes += (size_t)16 * block_bits[q] / 8;
  }
  return L;
}

int get_code_at(const Layout& L, const uint8_t* codes, int i, int j) {
  const int q = j / 16, t = j % 16;
  const uint8_t* row = codes + (size_t)i * L.row_bytes + L.off[q];
  if (L.bits[q] == 8) return (int)(int8_t)row[t];
  const uint8_t byte = row[t / 2];
  const int nib = (t % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  return nib >= 8 ? nib - 16 : nib;
}

void set_code_at(const Layout& L, uint8_t* codes, int i, int j, int code) {
  const int q = j / 16, t = j % 16;
  uint8_t* row = codes + (size_t)i * L.row_bytes + L.off[q];
  if (L.bits[q] == 8) {
    row[t] = (uint8_t)(int8_t)code;
    return;
  }
  const uint8_t nib = (uint8_t)(code & 0xF);
  uint8_t& byte = row[t / 2];
  byte = (t % 2 == 0) ? (uint8_t)((byte & 0xF0) | nib) : (uint8_t)((byte & 0x0F) | (nib << 4));
}

}  // namespace

static size_t head_bytes(const oracle_cfg* c, const uint8_t* block_bits) {
  return (size_t)c->dv * head_layout(c, block_bits).row_bytes;
}

size_t oracle_codes_bytes(const oracle_cfg* c, const uint8_t* block_bits) {
  const int nb = c->dk / 16;
  size_t per_b = 0;
  for (int h = 0; h < c->H; ++h) per_b += head_bytes(c, block_bits + (size_t)h * nb);
  return per_b * (size_t)c->B;
}

size_t oracle_head_offset(const oracle_cfg* c, const uint8_t* block_bits, int b, int h) {
  const int nb = c->dk / 16;
  size_t per_b = 0, before = 0;
  for (int hh = 0; hh < c->H; ++hh) {
    const size_t n = head_bytes(c, block_bits + (size_t)hh * nb);
    if (hh < h) before += n;
    per_b += n;
  }
  return (size_t)b * per_b + before;
}

int oracle_get_code(const uint8_t* codes, int bits, int64_t e) {
  if (bits == 8) return (int)(int8_t)codes[e];
  const uint8_t byte = codes[e / 2];
  const int nib = (e % 2 == 0) ? (byte & 0xF) : (byte >> 4);
  return nib >= 8 ? nib - 16 : nib;
}

void oracle_set_code(uint8_t* codes, int bits, int64_t e, int code) {
  if (bits == 8) {
    codes[e] = (uint8_t)(int8_t)code;
    return;
  }
  const uint8_t nib = (uint8_t)(code & 0xF);
  uint8_t& byte = codes[e / 2];
  if (e % 2 == 0)
    byte = (uint8_t)((byte & 0xF0) | nib);
  else
    byte = (uint8_t)((byte & 0x0F) | (nib << 4));
}

// ---------------------------------------------------------------------------
// Requantization of a head (LoReS "Scale grouping" (1/4): a group of G state
// elements shares one absmax scale, taken from the state being stored (4/4,
// "noisy" scale)).  Value-axis groups, the LoReS default, are G consecutive
// key columns of one value row: scales [dv][dk/G].  Key-axis groups, the
// comparison in the same section (C_j of Prop. "per-channel readout error"
// when G = dv), are G consecutive value rows of one key column: scales
// [dv/G][dk].
// ---------------------------------------------------------------------------

// Scales per head: dv * dk / G for either axis (G divides the grouped axis).
static size_t head_scales(const oracle_cfg* c) {
  if (c->axis == kAxisKey) return (size_t)(c->dv / c->G) * c->dk;
  return (size_t)c->dv * (c->dk / c->G);
}

static size_t scale_index(const oracle_cfg* c, int i, int j) {
  if (c->axis == kAxisKey) return (size_t)(i / c->G) * c->dk + j;
  return (size_t)i * (c->dk / c->G) + j / c->G;
}

// Quantize one group: elements e[0..n) (indices i*dk + j into the head) of
// S, with scale slot si.  prev: the head's stored values before the step
// (BDR); NULL for an import, where BDR has nothing to compare with and
// rounds to nearest.
// All elements of a group share one width (a value-axis group lies inside
// blocks of one width; a key-axis group is one column).
static void quantize_group(const oracle_cfg* c, const Layout& L, uint32_t key,
                           const std::vector<int64_t>& e, size_t si,
                           const float* S, const float* prev, uint8_t* codes,
                           float* scales, double* tdist) {
  const int bits = L.bits[(int)(e[0] % c->dk) / 16];
  const int r = qmax(bits);
  float m = 0.0f;
  for (int64_t x : e) m = std::max(m, std::fabs(S[x]));
  float s, inv;
  oracle_group_scale(m, r, &s, &inv);
  scales[si] = s;
  for (int64_t x : e) {
    int n;
    uint32_t r16 = 0;
    if (c->rounding == kRoundSR) {
      r16 = oracle_sr_bits(key, (uint64_t)x);
      n = oracle_round_sr(S[x], inv, r16, bits);
    } else if (c->rounding == kRoundBDR && prev) {
      n = oracle_round_bdr(S[x], inv, s, prev[x], r);
    } else {
      n = oracle_round_rtn(S[x], inv);
    }
    if (tdist) tdist[x] = oracle_threshold_distance(S[x], inv, c->rounding == kRoundSR, r16, bits);
    n = std::max(-r, std::min(r, n));
    set_code_at(L, codes, (int)(x / c->dk), (int)(x % c->dk), n);
  }
}

static void quantize_head(const oracle_cfg* c, const Layout& L, uint32_t key,
                          const float* S, const float* prev, uint8_t* codes,
                          float* scales, double* tdist) {
  const int dk = c->dk, dv = c->dv, G = c->G;
  std::vector<int64_t> e(G);
  if (c->axis == kAxisKey) {
    for (int g = 0; g < dv / G; ++g)
      for (int j = 0; j < dk; ++j) {
        for (int t = 0; t < G; ++t) e[t] = (int64_t)(g * G + t) * dk + j;
        quantize_group(c, L, key, e, scale_index(c, g * G, j), S, prev, codes, scales, tdist);
      }
  } else {
    for (int i = 0; i < dv; ++i)
      for (int g = 0; g < dk / G; ++g) {
        for (int t = 0; t < G; ++t) e[t] = (int64_t)i * dk + g * G + t;
        quantize_group(c, L, key, e, scale_index(c, i, g * G), S, prev, codes, scales, tdist);
      }
  }
}

// ---------------------------------------------------------------------------
// One decode step of one head.  Fig. 1 "Recurrent state: overwrite": the
// recurrence reads the stored state and overwrites all of it through the
// quantizer; "LoReS: State Quantization": the update itself is full
// precision.  Update forms: Gated DeltaNet S' = a S (I - b k k^T) + b v k^T
// (Prop. "decaying error": unit keys, 0 < b < 2); GLA S' = S diag(alpha) +
// v k^T; scalar decay S' = a S + dt v k^T (Prop. "repeated quantization",
// animation details); KDA (Table 1's "KDA": per-channel decay with delta
// correction, the same proposition's vector gates) S' = S diag(alpha)
// (I - b k k^T) + b v k^T.  Readout o = S' q from the unquantized S'.
// ---------------------------------------------------------------------------

void oracle_head_step(const oracle_cfg* c, int b, int h, const uint8_t* block_bits,
                      uint8_t* codes, float* scales, const float* q,
                      const float* k, const float* v, const float* alpha,
                      float beta, float* o, uint64_t step, float* pre,
                      double* tdist) {
  const int dk = c->dk, dv = c->dv;
  const Layout L = head_layout(c, block_bits);
  const uint32_t key = oracle_head_key(c->seed, c->layer, step, (uint32_t)b, (uint32_t)h);
  std::vector<float> d(dk), Sp((size_t)dv * dk), stored((size_t)dv * dk);
  for (int i = 0; i < dv; ++i) {
    float* sp = Sp.data() + (size_t)i * dk;
    // dequantize and decay
    for (int j = 0; j < dk; ++j) {
      const int64_t x = (int64_t)i * dk + j;
      const float code = (float)get_code_at(L, codes, i, j);
      const float s = scales[scale_index(c, i, j)];
      stored[x] = code * s;
      if (vector_decay(c->mixer))
        d[j] = (code * s) * alpha[j];
      else
        d[j] = code * (s * alpha[0]);
    }
    // write weight
    float w;
    if (delta_rule(c->mixer)) {
      const float u = oracle_dot(d.data(), k, dk);
      w = beta * (v[i] - u);
    } else if (c->mixer == kMixerGLA) {
      w = v[i];
    } else {
      w = beta * v[i];
    }
    // rank-1 write
    for (int j = 0; j < dk; ++j) sp[j] = std::fma(w, k[j], d[j]);
    if (o) o[i] = oracle_dot(sp, q, dk);
  }
  if (pre) std::memcpy(pre, Sp.data(), sizeof(float) * Sp.size());
  quantize_head(c, L, key, Sp.data(), stored.data(), codes, scales, tdist);
}

// The same step on an unquantized FP32 state (the "FP32 states" the pages
// compare against).
void oracle_head_step_fp32(const oracle_cfg* c, float* S, const float* q,
                           const float* k, const float* v, const float* alpha,
                           float beta, float* o) {
  const int dk = c->dk, dv = c->dv;
  std::vector<float> d(dk);
  for (int i = 0; i < dv; ++i) {
    float* row = S + (size_t)i * dk;
    for (int j = 0; j < dk; ++j)
      d[j] = row[j] * (vector_decay(c->mixer) ? alpha[j] : alpha[0]);
    float w;
    if (delta_rule(c->mixer)) {
      const float u = oracle_dot(d.data(), k, dk);
      w = beta * (v[i] - u);
    } else if (c->mixer == kMixerGLA) {
      w = v[i];
    } else {
      w = beta * v[i];
    }
    for (int j = 0; j < dk; ++j) row[j] = std::fma(w, k[j], d[j]);
    if (o) o[i] = oracle_dot(row, q, dk);
  }
}

void oracle_head_quantize(const oracle_cfg* c, int b, int h, const uint8_t* block_bits,
                          const float* S, uint8_t* codes, float* scales,
                          uint64_t step, double* tdist) {
  const uint32_t key = oracle_head_key(c->seed, c->layer, step, (uint32_t)b, (uint32_t)h);
  quantize_head(c, head_layout(c, block_bits), key, S, nullptr, codes, scales, tdist);
}

void oracle_head_dequantize(const oracle_cfg* c, const uint8_t* block_bits,
                            const uint8_t* codes, const float* scales, float* S) {
  const int dk = c->dk;
  const Layout L = head_layout(c, block_bits);
  for (int i = 0; i < c->dv; ++i)
    for (int j = 0; j < dk; ++j)
      S[(size_t)i * dk + j] = (float)get_code_at(L, codes, i, j) * scales[scale_index(c, i, j)];
}

void oracle_head_readout(const oracle_cfg* c, const uint8_t* block_bits, const uint8_t* codes,
                         const float* scales, const float* q, float* o) {
  std::vector<float> S((size_t)c->dv * c->dk);
  oracle_head_dequantize(c, block_bits, codes, scales, S.data());
  for (int i = 0; i < c->dv; ++i) o[i] = oracle_dot(S.data() + (size_t)i * c->dk, q, c->dk);
}

// ---------------------------------------------------------------------------
// Pure-write window ("Low-Bit GDN Recurrent-State Quantization: ... Pure-Write
// Sliding Windows", abstract): the last W pure writes are kept apart from the
// low-bit state as FP8 vector pairs (a, b), so that the full state is
// H + sum a b^T; every step propagates each pair through the state
// transition (b <- A^T b), and a pair is added into H only when it leaves
// the window.  Readings (the abstract fixes no format or order): FP8 is OCP
// E4M3 with one absmax scale per vector (s = max|x| / 448); the pair pushed
// at counter t lives in slot t mod W, so slot t mod W holds the oldest pair
// at counter t; an empty slot has zero scales and contributes exactly 0.
//
// Window area of one head: a codes [dv][W], b codes [W][dk], then the scales
// [W][2] (s_a, s_b), padded to a multiple of 16 bytes.
//
// Low-rank bypass ("Preserving Updates in Low-Bit Recurrent State
// Quantization", abstract: small updates accumulate in a compact low-rank
// buffer whose sufficiently large elements are merged into the state
// periodically) uses the same buffer of W pairs with another merge rule.
// Readings (the abstract gives no rank, period, threshold or format): the
// buffer is the W most recent writes (rank <= W) in the pair format above,
// propagated through the transition like the window; the period is W: the
// step at a counter that is a multiple of W merges the whole buffer, every
// element m_ij = sum over the pairs (oldest first) of a_i b'_j whose
// magnitude reaches threshold * s_ig (s_ig the element's stored group scale
// before the step) is added to the transitioned state, the others are
// dropped, and the buffer is emptied; between merges the slot of the
// counter is always empty, so those steps are the window step with an empty
// leaving pair.
// ---------------------------------------------------------------------------

// OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 holds
// the subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; no infinities; 448 is
// the largest finite value.
float oracle_fp8_decode(uint8_t code) {
  const int e = (code >> 3) & 0xF, m = code & 7;
  const float sign = (code & 0x80) ? -1.0f : 1.0f;
  if (e == 15 && m == 7) return std::nanf("");
  if (e == 0) return sign * std::ldexp((float)m, -9);
  return sign * std::ldexp(1.0f + (float)m / 8.0f, e - 7);
}

// Nearest E4M3 value to a finite x with |x| <= 448, ties to the even
// mantissa; the sign is kept (also for results of zero).
uint8_t oracle_fp8_encode(float x) {
  const uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  const double a = std::fabs((double)x);
  int best = 0;
  double best_err = a;  // code 0 (+0)
  for (int c = 1; c < 0x7F; ++c) {
    const double err = std::fabs((double)oracle_fp8_decode((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

size_t oracle_window_bytes(const oracle_cfg* c) {
  const size_t W = (size_t)c->window;
  const size_t raw = (size_t)c->dv * W + W * (size_t)c->dk + 8 * W;
  return (raw + 15) / 16 * 16;
}

namespace {

struct Window {
  const oracle_cfg* c;
  uint8_t* base;
  uint8_t* acode(int i, int t) const { return base + (size_t)i * c->window + t; }
  uint8_t* bcode(int t, int j) const {
    return base + (size_t)c->dv * c->window + (size_t)t * c->dk + j;
  }
  float* scale(int t, int which) const {
    return reinterpret_cast<float*>(base + (size_t)c->dv * c->window +
                                    (size_t)c->window * c->dk) + 2 * t + which;
  }
};

// Encode x[0..n) with one absmax scale: codes and the scale.
void fp8_vector(const float* x, int n, uint8_t* codes, size_t stride, float* scale) {
  float m = 0.0f;
  for (int j = 0; j < n; ++j) m = std::max(m, std::fabs(x[j]));
  float s, inv;
  oracle_group_scale(m, 448, &s, &inv);
  *scale = s;
  for (int j = 0; j < n; ++j) codes[(size_t)j * stride] = oracle_fp8_encode(x[j] * inv);
}

// Slot order by age at counter t: oldest first.
int age_slot(const oracle_cfg* c, uint64_t t, int age) {
  return (int)((t + (uint64_t)age) % (uint64_t)c->window);
}

}  // namespace

void oracle_head_step_pw(const oracle_cfg* c, int b, int h, const uint8_t* block_bits,
                         uint8_t* codes, float* scales, uint8_t* window,
                         const float* q, const float* k, const float* v,
                         const float* alpha, float beta, float* o, uint64_t step,
                         float* pre, double* tdist) {
  const int dk = c->dk, dv = c->dv, W = c->window;
  const Layout L = head_layout(c, block_bits);
  const uint32_t key = oracle_head_key(c->seed, c->layer, step, (uint32_t)b, (uint32_t)h);
  const Window win{c, window};
  const int slot = (int)(step % (uint64_t)W);
  const bool delta = delta_rule(c->mixer);
  auto decay = [&](int j) { return vector_decay(c->mixer) ? alpha[j] : alpha[0]; };

  // propagated keys b' = A^T b of every pair, and c_t = b'.q
  std::vector<float> Bp((size_t)W * dk), A((size_t)W * dv), cq(W), db(dk);
  for (int t = 0; t < W; ++t) {
    const float sa = *win.scale(t, 0), sb = *win.scale(t, 1);
    for (int i = 0; i < dv; ++i) A[(size_t)t * dv + i] = oracle_fp8_decode(*win.acode(i, t)) * sa;
    for (int j = 0; j < dk; ++j) db[j] = (oracle_fp8_decode(*win.bcode(t, j)) * sb) * decay(j);
    float* bp = Bp.data() + (size_t)t * dk;
    if (delta) {
      const float wb = -(beta * oracle_dot(db.data(), k, dk));
      for (int j = 0; j < dk; ++j) bp[j] = std::fma(wb, k[j], db[j]);
    } else {
      for (int j = 0; j < dk; ++j) bp[j] = db[j];
    }
    cq[t] = oracle_dot(bp, q, dk);
  }
  // the new pure write (a, b) = (weight * v, k)
  std::vector<float> anew(dv);
  for (int i = 0; i < dv; ++i) anew[i] = (c->mixer == kMixerGLA) ? v[i] : beta * v[i];
  const float cnew = oracle_dot(k, q, dk);

  // H' = H A + a_o b_o^T (the pair in `slot` leaves), o = H'q + window terms;
  // a bypass merge step instead adds the buffer's large elements
  const bool merge_all = c->window_merge == 1 && slot == 0;
  std::vector<float> d(dk), Sp((size_t)dv * dk), stored((size_t)dv * dk);
  const float* bo = Bp.data() + (size_t)slot * dk;
  for (int i = 0; i < dv; ++i) {
    float* sp = Sp.data() + (size_t)i * dk;
    for (int j = 0; j < dk; ++j) {
      const float code = (float)get_code_at(L, codes, i, j);
      const float s = scales[scale_index(c, i, j)];
      stored[(size_t)i * dk + j] = code * s;
      d[j] = vector_decay(c->mixer) ? (code * s) * alpha[j] : code * (s * alpha[0]);
    }
    if (merge_all) {
      const float wh = delta ? -(beta * oracle_dot(d.data(), k, dk)) : 0.0f;
      for (int j = 0; j < dk; ++j) {
        const float t = delta ? std::fma(wh, k[j], d[j]) : d[j];
        float m = 0.0f;
        for (int age = 0; age < W; ++age) {
          const int u = age_slot(c, step, age);
          m = std::fma(A[(size_t)u * dv + i], Bp[(size_t)u * dk + j], m);
        }
        const float thr = c->lrb_threshold * scales[scale_index(c, i, j)];
        sp[j] = std::fabs(m) >= thr ? t + m : t;
      }
      if (o) o[i] = std::fma(anew[i], cnew, oracle_dot(sp, q, dk));
      continue;
    }
    const float ao = A[(size_t)slot * dv + i];
    if (delta) {
      const float wh = -(beta * oracle_dot(d.data(), k, dk));
      for (int j = 0; j < dk; ++j) sp[j] = std::fma(ao, bo[j], std::fma(wh, k[j], d[j]));
    } else {
      for (int j = 0; j < dk; ++j) sp[j] = std::fma(ao, bo[j], d[j]);
    }
    if (o) {
      float acc = oracle_dot(sp, q, dk);
      for (int age = 1; age < W; ++age) {
        const int t = age_slot(c, step, age);
        acc = std::fma(A[(size_t)t * dv + i], cq[t], acc);
      }
      o[i] = std::fma(anew[i], cnew, acc);
    }
  }
  if (pre) std::memcpy(pre, Sp.data(), sizeof(float) * Sp.size());
  quantize_head(c, L, key, Sp.data(), stored.data(), codes, scales, tdist);

  // store the window: propagated keys of the remaining pairs (after a bypass
  // merge none remain), the new pair
  for (int t = 0; t < W; ++t) {
    if (t == slot) continue;
    if (merge_all) {
      for (int i = 0; i < dv; ++i) *win.acode(i, t) = 0;
      for (int j = 0; j < dk; ++j) *win.bcode(t, j) = 0;
      *win.scale(t, 0) = 0.0f;
      *win.scale(t, 1) = 0.0f;
      continue;
    }
    fp8_vector(Bp.data() + (size_t)t * dk, dk, win.bcode(t, 0), 1, win.scale(t, 1));
  }
  fp8_vector(anew.data(), dv, win.acode(0, slot), (size_t)W, win.scale(slot, 0));
  fp8_vector(k, dk, win.bcode(slot, 0), 1, win.scale(slot, 1));
}

// The full state H + sum a b^T (pairs oldest first) as the next step at
// counter `step` would see it.
void oracle_head_window_state(const oracle_cfg* c, const uint8_t* block_bits,
                              const uint8_t* codes, const float* scales,
                              const uint8_t* window, uint64_t step, float* S) {
  const int dk = c->dk, dv = c->dv, W = c->window;
  oracle_head_dequantize(c, block_bits, codes, scales, S);
  const Window win{c, const_cast<uint8_t*>(window)};
  for (int age = 0; age < W; ++age) {
    const int t = age_slot(c, step, age);
    const float sa = *win.scale(t, 0), sb = *win.scale(t, 1);
    for (int i = 0; i < dv; ++i) {
      const float a = oracle_fp8_decode(*win.acode(i, t)) * sa;
      for (int j = 0; j < dk; ++j)
        S[(size_t)i * dk + j] =
            std::fma(a, oracle_fp8_decode(*win.bcode(t, j)) * sb, S[(size_t)i * dk + j]);
    }
  }
}

// Readout of the stored full state: o = H q + sum a (b.q), pairs oldest first.
void oracle_head_window_readout(const oracle_cfg* c, const uint8_t* block_bits,
                                const uint8_t* codes, const float* scales,
                                const uint8_t* window, uint64_t step, const float* q,
                                float* o) {
  const int dk = c->dk, dv = c->dv, W = c->window;
  std::vector<float> H((size_t)dv * dk), bb(dk);
  oracle_head_dequantize(c, block_bits, codes, scales, H.data());
  const Window win{c, const_cast<uint8_t*>(window)};
  std::vector<float> cq(W);
  for (int t = 0; t < W; ++t) {
    const float sb = *win.scale(t, 1);
    for (int j = 0; j < dk; ++j) bb[j] = oracle_fp8_decode(*win.bcode(t, j)) * sb;
    cq[t] = oracle_dot(bb.data(), q, dk);
  }
  for (int i = 0; i < dv; ++i) {
    float acc = oracle_dot(H.data() + (size_t)i * dk, q, dk);
    for (int age = 0; age < W; ++age) {
      const int t = age_slot(c, step, age);
      acc = std::fma(oracle_fp8_decode(*win.acode(i, t)) * *win.scale(t, 0), cq[t], acc);
    }
    o[i] = acc;
  }
}

// ---------------------------------------------------------------------------
// Whole batch, in the library's array layout.
// ---------------------------------------------------------------------------

void oracle_step(const oracle_cfg* c, const uint8_t* block_bits, uint8_t* codes,
                 float* scales, const float* q, const float* k, const float* v,
                 const float* alpha, const float* beta, float* o, uint64_t step) {
  const int dk = c->dk, dv = c->dv;
  const int na = vector_decay(c->mixer) ? dk : 1;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t bh = (size_t)b * c->H + h;
      const uint8_t* bb = block_bits + (size_t)h * (dk / 16);
      oracle_head_step(c, b, h, bb, codes + oracle_head_offset(c, block_bits, b, h),
                       scales + bh * head_scales(c), q + bh * dk, k + bh * dk, v + bh * dv,
                       alpha + bh * na, (c->mixer == kMixerGLA) ? 0.0f : beta[bh],
                       o ? o + bh * dv : nullptr, step, nullptr, nullptr);
    }
}

void oracle_step_fp32(const oracle_cfg* c, float* S, const float* q, const float* k,
                      const float* v, const float* alpha, const float* beta, float* o) {
  const int dk = c->dk, dv = c->dv;
  const int na = vector_decay(c->mixer) ? dk : 1;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t bh = (size_t)b * c->H + h;
      oracle_head_step_fp32(c, S + bh * dv * dk, q + bh * dk, k + bh * dk, v + bh * dv,
                            alpha + bh * na, (c->mixer == kMixerGLA) ? 0.0f : beta[bh],
                            o ? o + bh * dv : nullptr);
    }
}

void oracle_quantize(const oracle_cfg* c, const uint8_t* block_bits, const float* S,
                     uint8_t* codes, float* scales, uint64_t step) {
  const int dk = c->dk, dv = c->dv;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t bh = (size_t)b * c->H + h;
      oracle_head_quantize(c, b, h, block_bits + (size_t)h * (dk / 16), S + bh * dv * dk,
                           codes + oracle_head_offset(c, block_bits, b, h),
                           scales + bh * head_scales(c), step, nullptr);
    }
}

void oracle_dequantize(const oracle_cfg* c, const uint8_t* block_bits,
                       const uint8_t* codes, const float* scales, float* S) {
  const int dk = c->dk, dv = c->dv;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t bh = (size_t)b * c->H + h;
      oracle_head_dequantize(c, block_bits + (size_t)h * (dk / 16),
                             codes + oracle_head_offset(c, block_bits, b, h),
                             scales + bh * head_scales(c), S + bh * dv * dk);
    }
}

void oracle_readout(const oracle_cfg* c, const uint8_t* block_bits, const uint8_t* codes,
                    const float* scales, const float* q, float* o) {
  const int dk = c->dk, dv = c->dv;
  for (int b = 0; b < c->B; ++b)
    for (int h = 0; h < c->H; ++h) {
      const size_t bh = (size_t)b * c->H + h;
      oracle_head_readout(c, block_bits + (size_t)h * (dk / 16),
                          codes + oracle_head_offset(c, block_bits, b, h),
                          scales + bh * head_scales(c), q + bh * dk, o + bh * dv);
    }
}

// The same three operations on a list of heads (indices b*H + h) of a batch
// in the library's layout; the other heads' data is neither read nor
// written, so disjoint lists may run on separate threads.

static size_t batch_head_offset(const oracle_cfg* c, const uint8_t* block_bits, int32_t bh) {
  return oracle_head_offset(c, block_bits, bh / c->H, bh % c->H);
}

void oracle_step_heads(const oracle_cfg* c, const uint8_t* block_bits, int n,
                       const int32_t* heads, uint8_t* codes, float* scales, const float* q,
                       const float* k, const float* v, const float* alpha, const float* beta,
                       float* o, uint64_t step) {
  const int dk = c->dk, dv = c->dv;
  const int na = vector_decay(c->mixer) ? dk : 1;
  for (int t = 0; t < n; ++t) {
    const size_t bh = (size_t)heads[t];
    const int h = (int)(bh % c->H);
    oracle_head_step(c, (int)(bh / c->H), h, block_bits + (size_t)h * (dk / 16),
                     codes + batch_head_offset(c, block_bits, heads[t]),
                     scales + bh * head_scales(c), q + bh * dk, k + bh * dk, v + bh * dv,
                     alpha + bh * na, (c->mixer == kMixerGLA) ? 0.0f : beta[bh],
                     o ? o + bh * dv : nullptr, step, nullptr, nullptr);
  }
}

void oracle_step_fp32_heads(const oracle_cfg* c, int n, const int32_t* heads, float* S,
                            const float* q, const float* k, const float* v,
                            const float* alpha, const float* beta, float* o) {
  const int dk = c->dk, dv = c->dv;
  const int na = vector_decay(c->mixer) ? dk : 1;
  for (int t = 0; t < n; ++t) {
    const size_t bh = (size_t)heads[t];
    oracle_head_step_fp32(c, S + bh * dv * dk, q + bh * dk, k + bh * dk, v + bh * dv,
                          alpha + bh * na, (c->mixer == kMixerGLA) ? 0.0f : beta[bh],
                          o ? o + bh * dv : nullptr);
  }
}

void oracle_quantize_heads(const oracle_cfg* c, const uint8_t* block_bits, int n,
                           const int32_t* heads, const float* S, uint8_t* codes,
                           float* scales, uint64_t step) {
  const int dk = c->dk, dv = c->dv;
  for (int t = 0; t < n; ++t) {
    const size_t bh = (size_t)heads[t];
    const int h = (int)(bh % c->H);
    oracle_head_quantize(c, (int)(bh / c->H), h, block_bits + (size_t)h * (dk / 16),
                         S + bh * dv * dk, codes + batch_head_offset(c, block_bits, heads[t]),
                         scales + bh * head_scales(c), step, nullptr);
  }
}

// ---------------------------------------------------------------------------
// Decay-based mixed precision (LoReS 2/4: more bits for the slowest-decaying
// heads).  retention is larger for slower decay.
//   mode 0: hi bits where retention > threshold;
//   mode 1: hi bits for the round(frac * heads) heads of largest retention,
//           ties resolved toward the lower head index.
// ---------------------------------------------------------------------------

int oracle_bits_by_decay(const float* retention, int heads, int mode,
                         float thr_or_frac, uint8_t lo, uint8_t hi, uint8_t* out) {
  if (heads <= 0) return -1;
  if (mode == 0) {
    for (int h = 0; h < heads; ++h) out[h] = retention[h] > thr_or_frac ? hi : lo;
    return 0;
  }
  if (mode != 1 || !(thr_or_frac >= 0.0f && thr_or_frac <= 1.0f)) return -1;
  const int n_hi = (int)std::floor((double)thr_or_frac * heads + 0.5);
  std::vector<int> order(heads);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return retention[a] > retention[b]; });
  for (int h = 0; h < heads; ++h) out[h] = lo;
  for (int n = 0; n < n_hi; ++n) out[order[n]] = hi;
  return 0;
}

}  // extern "C"
