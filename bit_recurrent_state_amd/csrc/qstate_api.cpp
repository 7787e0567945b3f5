// qstate_api.cpp — the C ABI declared in include/qstate.h: argument checks,
// the host-side handle, per-head layout and kernel dispatch.  Host code only;
// every byte of the step is computed by the kernels in qstate_value_dk*.hip
// and qstate_key_dk*.hip.

#include "qstate.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "qstate_launch.h"

struct qstate {
  qstate_config cfg;          // head_bits / channel_bits pointers cleared
  uint16_t int8_blocks[256];  // per head: bit q set = 16-column block q is INT8
  uint32_t head_units[256];   // per head: byte offset in a batch row / (8 dv)
  void* state;            // codes or FP32 state (device)
  float* scales;          // device, quantized only
  uint64_t step;
  uint64_t bytes_per_b;   // code bytes of one batch row
};

namespace {

constexpr int kMaxHeads = 256;
constexpr int kMaxDv = 4096;
constexpr int64_t kTargetWaves = 4096;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Width of block q (16 key columns) of head h: channel_bits, else head_bits,
// else INT8.
int block_width(const qstate_config* c, int h, int q) {
  if (c->channel_bits) return c->channel_bits[(size_t)h * (c->dk / 16) + q];
  return c->head_bits ? c->head_bits[h] : 8;
}

uint16_t int8_blocks(const qstate_config* c, int h) {
  uint16_t m = 0;
  for (int q = 0; q < c->dk / 16; ++q)
    if (block_width(c, h, q) == 8) m = (uint16_t)(m | (1u << q));
  return m;
}

int check_config(const qstate_config* c) {
  if (!c) return QSTATE_E_INVALID;
  if (c->batch < 1 || c->heads < 1 || c->dk < 1 || c->dv < 1) return QSTATE_E_INVALID;
  if (c->mixer < QSTATE_GDN || c->mixer > QSTATE_KDA) return QSTATE_E_INVALID;
  if (c->fp32_state != 0 && c->fp32_state != 1) return QSTATE_E_INVALID;
  if (!c->fp32_state) {
    if (c->rounding < QSTATE_RTN || c->rounding > QSTATE_BDR) return QSTATE_E_INVALID;
    if (c->group_axis != QSTATE_VALUE_AXIS && c->group_axis != QSTATE_KEY_AXIS)
      return QSTATE_E_INVALID;
    // value-axis groups split a row's dk columns, key-axis groups a column's dv rows
    const int grouped = c->group_axis == QSTATE_KEY_AXIS ? c->dv : c->dk;
    if (c->group < 1 || grouped % c->group != 0) return QSTATE_E_INVALID;
    if (c->head_bits)
      for (int h = 0; h < c->heads && h < kMaxHeads; ++h)
        if (c->head_bits[h] != 4 && c->head_bits[h] != 8) return QSTATE_E_INVALID;
    if (c->channel_bits && c->dk % 16 == 0 && c->dk <= 256) {
      const int nb = c->dk / 16;
      for (int h = 0; h < c->heads && h < kMaxHeads; ++h)
        for (int q = 0; q < nb; ++q) {
          const int w = c->channel_bits[(size_t)h * nb + q];
          if (w != 4 && w != 8) return QSTATE_E_INVALID;
          // a value-axis scale group never mixes widths
          if (c->group_axis == QSTATE_VALUE_AXIS && c->group > 16 && c->group % 16 == 0 &&
              q % (c->group / 16) != 0 && w != c->channel_bits[(size_t)h * nb + q - 1])
            return QSTATE_E_INVALID;
        }
    }
  }
  if (!c->fp32_state && c->window != 0) {
    if (c->window < 0) return QSTATE_E_INVALID;
    // the window kernels take value-axis groups and heads of one width
    if (c->window != 4 && c->window != 8 && c->window != 16) return QSTATE_E_UNSUPPORTED;
    if (c->group_axis != QSTATE_VALUE_AXIS || c->channel_bits) return QSTATE_E_UNSUPPORTED;
  }
  if (c->window_merge != 0) {
    if (c->window_merge != 1 || c->fp32_state || c->window == 0) return QSTATE_E_INVALID;
    if (!(c->lrb_threshold >= 0.0f && c->lrb_threshold <= FLT_MAX)) return QSTATE_E_INVALID;
  }
  if (c->dk != 64 && c->dk != 128 && c->dk != 256) return QSTATE_E_UNSUPPORTED;
  if (c->heads > kMaxHeads || c->dv > kMaxDv) return QSTATE_E_UNSUPPORTED;
  if (!c->fp32_state && c->group != 16 && c->group != 32 && c->group != 64 && c->group != 128)
    return QSTATE_E_UNSUPPORTED;
  // every index the kernels form must stay inside 63-bit sizes and a 32-bit grid
  const double elems = (double)c->batch * c->heads * c->dv * c->dk;
  if (elems * 4.0 > 9.0e18 || (double)c->batch * c->heads * ((c->dv + 31) / 32) > 2147483647.0)
    return QSTATE_E_UNSUPPORTED;
  return QSTATE_OK;
}

uint64_t align16(uint64_t n) { return (n + 15) / 16 * 16; }


// Bytes of one head's pure-write window area: a codes [dv][W], then two
// copies of (b codes [W][dk], scales [W][2]).
uint64_t window_head_bytes(const qstate_config* c) {
  const uint64_t W = c->fp32_state ? 0 : (uint64_t)c->window;
  return W ? align16((uint64_t)c->dv * W + 2 * (W * c->dk + 8 * W)) : 0;
}

void layout(const qstate_config* c, size_t* codes_bytes, size_t* scales_bytes, uint64_t* per_b) {
  const size_t bh = (size_t)c->batch * c->heads;
  if (c->fp32_state) {
    *codes_bytes = bh * c->dv * c->dk * sizeof(float);
    *scales_bytes = 0;
    if (per_b) *per_b = 0;
    return;
  }
  uint64_t pb = 0;
  for (int h = 0; h < c->heads; ++h)
    for (int q = 0; q < c->dk / 16; ++q) pb += (uint64_t)c->dv * 2 * block_width(c, h, q);
  *codes_bytes = (size_t)pb * c->batch;
  if (c->window)  // the window areas follow the codes
    *codes_bytes = (size_t)(align16(*codes_bytes) + bh * window_head_bytes(c));
  const size_t per_head = c->group_axis == QSTATE_KEY_AXIS
                              ? (size_t)(c->dv / c->group) * c->dk
                              : (size_t)c->dv * (c->dk / c->group);
  *scales_bytes = bh * per_head * sizeof(float);
  if (per_b) *per_b = pb;
}

qs::KParams base_params(const qstate* s) {
  qs::KParams p;
  std::memset(&p, 0, sizeof(p));
  p.state = s->state;
  p.scales = s->scales;
  p.B = s->cfg.batch;
  p.H = s->cfg.heads;
  p.dv = s->cfg.dv;
  p.G = s->cfg.fp32_state ? 16 : s->cfg.group;
  p.axis = s->cfg.fp32_state ? 0 : s->cfg.group_axis;
  // Split heads into row slices until the launch has at least kTargetWaves
  // waves (16 per CU on 256 CUs).  Value axis: one wave per slice, slices of
  // whole 32-row units.  Key axis: workgroups of max(1, G / rb) waves, each
  // owning whole blocks of max(G, rb) rows, rb = 4096 / dk rows per wave.
  const int64_t heads = (int64_t)s->cfg.batch * s->cfg.heads;
  int unit_rows = 32, waves_per_slice = 1;
  if (p.axis == QSTATE_KEY_AXIS) {
    const int rb = 4096 / s->cfg.dk;
    unit_rows = std::max(p.G, rb);
    waves_per_slice = std::max(1, p.G / rb);
  }
  const int units = (s->cfg.dv + unit_rows - 1) / unit_rows;
  const int64_t want = (kTargetWaves + heads * waves_per_slice - 1) / (heads * waves_per_slice);
  int slices = (int)std::min<int64_t>(want, units);
  slices = std::max(slices, 1);
  const int units_per_slice = (units + slices - 1) / slices;
  p.slice_rows = unit_rows * units_per_slice;
  p.slices = (units + units_per_slice - 1) / units_per_slice;
  p.bytes_per_b = s->bytes_per_b;
  std::memcpy(p.int8_blocks, s->int8_blocks, sizeof(p.int8_blocks));
  const uint16_t full = (uint16_t)((1u << (s->cfg.dk / 16)) - 1u);
  for (int h = 0; h < s->cfg.heads; ++h)
    if (s->int8_blocks[h] != 0 && s->int8_blocks[h] != full) p.mixed = 1;
  std::memcpy(p.head_units, s->head_units, sizeof(p.head_units));
  p.seed = s->cfg.seed;
  p.layer = s->cfg.layer;
  p.step = s->step;
  if (!s->cfg.fp32_state && s->cfg.window > 0) {
    p.window_len = s->cfg.window;
    p.lrb_merge = s->cfg.window_merge == 1 && s->step % (uint64_t)s->cfg.window == 0;
    p.lrb_theta = s->cfg.lrb_threshold;
    p.window_head_bytes = window_head_bytes(&s->cfg);
    p.window = static_cast<uint8_t*>(s->state) + align16(s->bytes_per_b * s->cfg.batch);
  }
  return p;
}

// q = (mulhi(x, m) + x) >> s computes x / d for x < 2^31.
qs::FastDiv fast_div(uint32_t d) {
  qs::FastDiv f;
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  f.s = l;
  f.m = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
  return f;
}

// The persistent step's work units (value-axis heads of one width each, no
// window): units of persist_unit_rows(dk) rows, INT8 heads first.
void persist_params(const qstate* s, qs::KParams& p) {
  const qstate_config& c = s->cfg;
  if (c.fp32_state || c.group_axis != QSTATE_VALUE_AXIS || c.window != 0 || p.mixed) return;
  const int uph = (c.dv + qs::persist_unit_rows(c.dk) - 1) / qs::persist_unit_rows(c.dk);
  int n8 = 0;
  for (int h = 0; h < c.heads; ++h)
    if (s->int8_blocks[h] != 0) p.head_order[n8++] = (uint32_t)h;
  int i = n8;
  for (int h = 0; h < c.heads; ++h)
    if (s->int8_blocks[h] == 0) p.head_order[i++] = (uint32_t)h;
  p.persist = 1;
  p.units_per_head = uph;
  p.n_units = (uint32_t)((int64_t)c.batch * c.heads * uph);
  p.n8_heads = n8;
  p.div_group = fast_div((uint32_t)(8 * uph));
  p.div_n8 = fast_div((uint32_t)std::max(n8, 1));
  p.div_n4 = fast_div((uint32_t)std::max(c.heads - n8, 1));
}

int run(const qstate* s, qs::Op op, const qs::KParams& p, void* stream) {
  const qstate_config& c = s->cfg;
  const hipError_t e = qs::launch(op, c.mixer, c.rounding, c.fp32_state, c.dk, p,
                                  reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? QSTATE_OK : QSTATE_E_LAUNCH;
}

}  // namespace

extern "C" {

int qstate_state_bytes(const qstate_config* cfg, size_t* codes_bytes, size_t* scales_bytes) {
  const int rc = check_config(cfg);
  if (rc != QSTATE_OK) return rc;
  if (!codes_bytes || !scales_bytes) return QSTATE_E_INVALID;
  layout(cfg, codes_bytes, scales_bytes, nullptr);
  return QSTATE_OK;
}

int qstate_create(const qstate_config* cfg, void* codes_dev, void* scales_dev, qstate** out) {
  if (!out) return QSTATE_E_INVALID;
  *out = nullptr;
  const int rc = check_config(cfg);
  if (rc != QSTATE_OK) return rc;
  if (!codes_dev || !aligned(codes_dev, 16)) return QSTATE_E_INVALID;
  if (!cfg->fp32_state && (!scales_dev || !aligned(scales_dev, 16))) return QSTATE_E_INVALID;
  qstate* s = new (std::nothrow) qstate;
  if (!s) return QSTATE_E_NOMEM;
  std::memset(s, 0, sizeof(*s));
  s->cfg = *cfg;
  if (!cfg->fp32_state) {
    // head (b, h) starts at b * bytes_per_b + 8 dv * head_units[h]: a row
    // of head h takes 8 bytes per INT4 block and 16 per INT8 block
    uint32_t units = 0;
    for (int h = 0; h < cfg->heads; ++h) {
      s->int8_blocks[h] = int8_blocks(cfg, h);
      s->head_units[h] = units;
      units += (uint32_t)(cfg->dk / 16 + __builtin_popcount(s->int8_blocks[h]));
    }
  }
  s->cfg.head_bits = nullptr;
  s->cfg.channel_bits = nullptr;
  size_t cb = 0, sb = 0;
  qstate_config tmp = *cfg;
  layout(&tmp, &cb, &sb, &s->bytes_per_b);
  s->state = codes_dev;
  s->scales = cfg->fp32_state ? nullptr : static_cast<float*>(scales_dev);
  s->step = 0;
  *out = s;
  return QSTATE_OK;
}

int qstate_load_fp32(qstate* s, const float* S_dev, void* stream) {
  if (!s || !S_dev || !aligned(S_dev, 16)) return QSTATE_E_INVALID;
  const qstate_config& c = s->cfg;
  if (c.fp32_state) {
    const size_t bytes = (size_t)c.batch * c.heads * c.dv * c.dk * sizeof(float);
    const hipError_t e = hipMemcpyAsync(s->state, S_dev, bytes, hipMemcpyDeviceToDevice,
                                        reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? QSTATE_OK : QSTATE_E_LAUNCH;
  }
  qs::KParams p = base_params(s);
  p.src = S_dev;
  const int rc = run(s, qs::kImport, p, stream);
  if (rc == QSTATE_OK) ++s->step;
  return rc;
}

int qstate_step(qstate* s, const float* q, const float* k, const float* v, const float* alpha,
                const float* beta, float* o, void* stream) {
  if (!s || !q || !k || !v || !alpha) return QSTATE_E_INVALID;
  const qstate_config& c = s->cfg;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 4)) return QSTATE_E_INVALID;
  const bool vector_gate = c.mixer == QSTATE_GLA || c.mixer == QSTATE_KDA;
  if (!aligned(alpha, vector_gate ? 16 : 4)) return QSTATE_E_INVALID;
  if (c.mixer != QSTATE_GLA && (!beta || !aligned(beta, 4))) return QSTATE_E_INVALID;
  if (o && !aligned(o, 4)) return QSTATE_E_INVALID;
  qs::KParams p = base_params(s);
  p.q = q;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.beta = c.mixer == QSTATE_GLA ? nullptr : beta;
  p.o = o;
  persist_params(s, p);
  const int rc = run(s, qs::kStep, p, stream);
  if (rc == QSTATE_OK) ++s->step;
  return rc;
}

int qstate_readout(qstate* s, const float* q, float* o, void* stream) {
  if (!s || !q || !o || !aligned(q, 16) || !aligned(o, 4)) return QSTATE_E_INVALID;
  qs::KParams p = base_params(s);
  p.q = q;
  p.o = o;
  return run(s, qs::kReadout, p, stream);
}

int qstate_store_fp32(qstate* s, float* S_dev, void* stream) {
  if (!s || !S_dev || !aligned(S_dev, 16)) return QSTATE_E_INVALID;
  const qstate_config& c = s->cfg;
  if (c.fp32_state) {
    const size_t bytes = (size_t)c.batch * c.heads * c.dv * c.dk * sizeof(float);
    const hipError_t e = hipMemcpyAsync(S_dev, s->state, bytes, hipMemcpyDeviceToDevice,
                                        reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? QSTATE_OK : QSTATE_E_LAUNCH;
  }
  qs::KParams p = base_params(s);
  p.dst = S_dev;
  return run(s, qs::kExport, p, stream);
}

int qstate_get_step(const qstate* s, uint64_t* step) {
  if (!s || !step) return QSTATE_E_INVALID;
  *step = s->step;
  return QSTATE_OK;
}

int qstate_set_step(qstate* s, uint64_t step) {
  if (!s) return QSTATE_E_INVALID;
  s->step = step;
  return QSTATE_OK;
}

int qstate_destroy(qstate* s) {
  delete s;
  return QSTATE_OK;
}

const char* qstate_strerror(int status) {
  switch (status) {
    case QSTATE_OK: return "ok";
    case QSTATE_E_INVALID: return "invalid argument (null or misaligned pointer, bad size or enum)";
    case QSTATE_E_UNSUPPORTED: return "unsupported configuration (dk, group, heads or dv)";
    case QSTATE_E_LAUNCH: return "kernel launch failed";
    case QSTATE_E_NOMEM: return "host allocation failed";
    default: return "unknown status";
  }
}

int qstate_bits_by_decay(const float* retention, int heads, int mode, float thr_or_frac,
                         uint8_t lo_bits, uint8_t hi_bits, uint8_t* out_bits) {
  if (!retention || !out_bits || heads < 1) return QSTATE_E_INVALID;
  if ((lo_bits != 4 && lo_bits != 8) || (hi_bits != 4 && hi_bits != 8)) return QSTATE_E_INVALID;
  if (mode == 0) {
    for (int h = 0; h < heads; ++h) out_bits[h] = retention[h] > thr_or_frac ? hi_bits : lo_bits;
    return QSTATE_OK;
  }
  if (mode != 1 || !(thr_or_frac >= 0.0f && thr_or_frac <= 1.0f)) return QSTATE_E_INVALID;
  const int take = (int)std::floor((double)thr_or_frac * (double)heads + 0.5);
  // heads ranked by retention, largest first; equal retention keeps index order
  std::vector<int> rank(heads);
  std::iota(rank.begin(), rank.end(), 0);
  std::stable_sort(rank.begin(), rank.end(),
                   [retention](int a, int b) { return retention[a] > retention[b]; });
  std::fill(out_bits, out_bits + heads, lo_bits);
  for (int i = 0; i < take; ++i) out_bits[rank[i]] = hi_bits;
  return QSTATE_OK;
}

}  // extern "C"
