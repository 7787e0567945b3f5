// abi_host_harness.cpp — host-side checks of the C ABI (qstate_api.cpp) built
// with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, without a
// GPU: the kernel dispatcher and the HIP copy are replaced by stand-ins that
// check the launch parameters the host code derives from each configuration
// and return success.  Exits non-zero on the first failed check (the
// sanitizers abort on their own findings).

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "qstate.h"
#include "qstate_launch.h"

static int g_fail = 0;
static long g_launches = 0, g_persist = 0, g_valid = 0;
static qstate_config g_cfg;     // the configuration of the handle being exercised
static size_t g_codes_bytes = 0;

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);    \
      g_fail = 1;                                                                \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

static int width(const qstate_config& c, const uint8_t* hb, const uint8_t* cb, int h, int q) {
  if (cb) return cb[h * (c.dk / 16) + q];
  return hb ? hb[h] : 8;
}

static std::vector<uint8_t> g_hb, g_cb;

// Stand-in for the kernel dispatcher: the parameters must describe the
// configuration exactly.
namespace qs {
hipError_t launch(Op op, int mixer, int rounding, int fp32, int dk, const KParams& p,
                  hipStream_t) {
  ++g_launches;
  const qstate_config& c = g_cfg;
  CHECK(mixer == c.mixer && fp32 == c.fp32_state && dk == c.dk);
  if (!fp32) CHECK(rounding == c.rounding);
  CHECK(p.B == c.batch && p.H == c.heads && p.dv == c.dv);
  CHECK(p.slices >= 1 && p.slice_rows >= 1);
  CHECK((int64_t)p.slices * p.slice_rows >= c.dv);
  CHECK((int64_t)(p.slices - 1) * p.slice_rows < c.dv);  // no empty slice
  if (!fp32) {
    // per-head offsets: 8 dv bytes per unit; INT8 blocks take two units
    uint32_t units = 0;
    const uint16_t full = (uint16_t)((1u << (c.dk / 16)) - 1u);
    bool mixed = false;
    for (int h = 0; h < c.heads; ++h) {
      CHECK(p.head_units[h] == units);
      uint16_t m = 0;
      for (int q = 0; q < c.dk / 16; ++q)
        if (width(c, g_hb.empty() ? nullptr : g_hb.data(), g_cb.empty() ? nullptr : g_cb.data(),
                  h, q) == 8)
          m = (uint16_t)(m | (1u << q));
      CHECK(p.int8_blocks[h] == m);
      if (m != 0 && m != full) mixed = true;
      units += (uint32_t)(c.dk / 16 + __builtin_popcount(m));
    }
    CHECK(p.bytes_per_b == (uint64_t)8 * c.dv * units);
    CHECK(p.mixed == (mixed ? 1 : 0));
    CHECK(p.bytes_per_b * (uint64_t)c.batch <= g_codes_bytes);
    if (c.window > 0) {
      CHECK(p.window_len == c.window && p.window != nullptr);
      const uint64_t wb = (uint64_t)p.window_head_bytes;
      CHECK(wb % 16 == 0);
      const uint8_t* end = p.window + wb * (uint64_t)c.batch * c.heads;
      CHECK(end == static_cast<const uint8_t*>(p.state) + g_codes_bytes);
      CHECK(p.lrb_merge == (c.window_merge == 1 && p.step % (uint64_t)c.window == 0 ? 1 : 0));
    }
  }
  if (op == kStep && p.persist) {
    ++g_persist;
    CHECK(!fp32 && c.group_axis == QSTATE_VALUE_AXIS && c.window == 0 && !p.mixed);
    const int ur = persist_unit_rows(c.dk);
    CHECK(p.units_per_head == (c.dv + ur - 1) / ur);
    CHECK(p.n_units == (uint32_t)((int64_t)c.batch * c.heads * p.units_per_head));
    // head order: the INT8 heads, then the INT4 heads, each ascending
    std::vector<int> seen(c.heads, 0);
    int n8 = 0;
    for (int i = 0; i < c.heads; ++i) {
      const uint32_t h = p.head_order[i];
      CHECK(h < (uint32_t)c.heads && !seen[h]);
      seen[h] = 1;
      const bool is8 = p.int8_blocks[h] != 0;
      if (i < p.n8_heads) CHECK(is8); else CHECK(!is8);
      if (i > 0 && i != p.n8_heads) CHECK(p.head_order[i - 1] < h);
      n8 += is8;
    }
    CHECK(n8 == p.n8_heads);
    // the fast divisions, exhaustively over every value the kernel divides
    auto div_ok = [](FastDiv f, uint32_t d, uint32_t upto) {
      for (uint32_t x = 0; x < upto; ++x) {
        const uint32_t q = (uint32_t)((((uint64_t)x * f.m) >> 32) + x) >> f.s;
        if (q != x / d) return false;
      }
      return true;
    };
    CHECK(div_ok(p.div_group, 8u * p.units_per_head, p.n_units));
    CHECK(div_ok(p.div_n8, (uint32_t)std::max(p.n8_heads, 1), (uint32_t)c.batch * c.heads));
    CHECK(div_ok(p.div_n4, (uint32_t)std::max(c.heads - p.n8_heads, 1),
                 (uint32_t)c.batch * c.heads));
  }
  if (op == kStep) CHECK(p.q && p.k && p.v && p.alpha);
  if (op == kImport) CHECK(p.src != nullptr);
  if (op == kExport) CHECK(p.dst != nullptr);
  if (op == kReadout) CHECK(p.q && p.o);
  return hipSuccess;
}
}  // namespace qs

// Stand-in for the device-to-device copy of the FP32 state.
extern "C" hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) {
  return hipSuccess;
}

static void* fake(uintptr_t a) { return reinterpret_cast<void*>(a); }

static void exercise(qstate_config c, std::mt19937& rng) {
  g_cfg = c;
  size_t cb = 0, sb = 0;
  const int rc = qstate_state_bytes(&c, &cb, &sb);
  if (rc != QSTATE_OK) {
    qstate* h = nullptr;
    CHECK(qstate_create(&c, fake(1 << 20), fake(1 << 21), &h) == rc && h == nullptr);
    return;
  }
  g_codes_bytes = cb;
  ++g_valid;
  qstate* s = nullptr;
  CHECK(qstate_create(&c, fake(0), fake(1 << 21), &s) == QSTATE_E_INVALID && !s);
  CHECK(qstate_create(&c, fake((1 << 20) + 8), fake(1 << 21), &s) == QSTATE_E_INVALID && !s);
  CHECK(qstate_create(&c, fake(1 << 20), fake(1 << 21), &s) == QSTATE_OK && s);
  // the handle copied the widths: clobbering the caller's arrays after create
  // changes nothing (the checks above compare against the saved copies)
  std::vector<uint8_t> keep_hb = g_hb, keep_cb = g_cb;
  if (c.head_bits) std::memset(const_cast<uint8_t*>(c.head_bits), 0, g_hb.size());
  if (c.channel_bits) std::memset(const_cast<uint8_t*>(c.channel_bits), 0, g_cb.size());
  g_hb.swap(keep_hb);
  g_cb.swap(keep_cb);
  const float* f = static_cast<const float*>(fake(1 << 24));
  float* o = static_cast<float*>(fake(1 << 25));
  uint64_t st = 0;
  CHECK(qstate_load_fp32(s, f, nullptr) == QSTATE_OK);
  CHECK(qstate_get_step(s, &st) == QSTATE_OK && st == (c.fp32_state ? 0u : 1u));
  const int steps = 1 + (int)(rng() % 5);
  const float* beta = c.mixer == QSTATE_GLA ? nullptr : f;
  for (int t = 0; t < steps; ++t) CHECK(qstate_step(s, f, f, f, f, beta, o, nullptr) == QSTATE_OK);
  CHECK(qstate_step(s, f, f, f, f, beta, nullptr, nullptr) == QSTATE_OK);
  CHECK(qstate_step(s, nullptr, f, f, f, beta, o, nullptr) == QSTATE_E_INVALID);
  CHECK(qstate_step(s, static_cast<const float*>(fake((1 << 24) + 4)), f, f, f, beta, o,
                    nullptr) == QSTATE_E_INVALID);
  if (c.mixer != QSTATE_GLA) CHECK(qstate_step(s, f, f, f, f, nullptr, o, nullptr) == QSTATE_E_INVALID);
  CHECK(qstate_readout(s, f, o, nullptr) == QSTATE_OK);
  CHECK(qstate_store_fp32(s, o, nullptr) == QSTATE_OK);
  CHECK(qstate_set_step(s, 1000) == QSTATE_OK);
  CHECK(qstate_step(s, f, f, f, f, beta, o, nullptr) == QSTATE_OK);
  CHECK(qstate_get_step(s, &st) == QSTATE_OK && st == 1001u);
  CHECK(qstate_destroy(s) == QSTATE_OK);
}

int main() {
  std::mt19937 rng(12345);
  long configs = 0;
  const int dks[] = {64, 128, 256, 96, 512};
  const int dvs[] = {1, 16, 37, 64, 128, 129, 4096, 5000};
  const int groups[] = {16, 32, 64, 128, 48, 8};
  for (int trial = 0; trial < 6000; ++trial) {
    qstate_config c;
    std::memset(&c, 0, sizeof(c));
    c.batch = 1 + (int)(rng() % 4) * (trial % 7 == 0 ? 64 : 1);
    c.heads = (trial % 11 == 0) ? 256 : 1 + (int)(rng() % 40);
    if (trial % 97 == 0) c.heads = 300;
    c.dk = dks[rng() % 5];
    c.dv = dvs[rng() % 8];
    c.group = groups[rng() % 6];
    c.mixer = (int)(rng() % 4);
    c.rounding = (int)(rng() % 3);
    c.fp32_state = (rng() % 8 == 0) ? 1 : 0;
    c.seed = rng();
    c.layer = rng() % 24;
    c.group_axis = (rng() % 4 == 0) ? QSTATE_KEY_AXIS : QSTATE_VALUE_AXIS;
    g_hb.clear();
    g_cb.clear();
    const int nb = c.dk / 16;
    const int kind = (int)(rng() % 4);
    if (kind == 1 || kind == 2) {
      g_hb.resize(c.heads);
      for (auto& b : g_hb) b = (kind == 1) ? 4 : ((rng() & 1) ? 8 : 4);
      c.head_bits = g_hb.data();
    } else if (kind == 3 && c.dk % 16 == 0 && c.dk <= 256) {
      g_cb.resize((size_t)c.heads * nb);
      const int gb = (c.group_axis == QSTATE_VALUE_AXIS && c.group % 16 == 0) ? c.group / 16 : 1;
      for (int h = 0; h < c.heads; ++h)
        for (int q = 0; q < nb; q += gb) {
          const uint8_t w = (rng() & 1) ? 8 : 4;
          for (int r = 0; r < gb && q + r < nb; ++r) g_cb[(size_t)h * nb + q + r] = w;
        }
      c.channel_bits = g_cb.data();
    }
    if (!c.fp32_state && c.group_axis == QSTATE_VALUE_AXIS && rng() % 4 == 0) {
      const int ws[] = {4, 8, 16};
      c.window = ws[rng() % 3];
      c.window_merge = (int)(rng() % 2);
      c.lrb_threshold = 0.5f;
    }
    exercise(c, rng);
    ++configs;
  }
  // decay-based bits
  for (int trial = 0; trial < 2000; ++trial) {
    const int heads = 1 + (int)(rng() % 300);
    std::vector<float> r(heads);
    for (auto& x : r) x = (float)(rng() % 17) / 16.0f;  // many ties
    std::vector<uint8_t> out(heads, 0);
    const float frac = (float)(rng() % 11) / 10.0f;
    CHECK(qstate_bits_by_decay(r.data(), heads, 1, frac, 4, 8, out.data()) == QSTATE_OK);
    int n8 = 0;
    for (int h = 0; h < heads; ++h) n8 += out[h] == 8;
    CHECK(n8 == (int)std::floor((double)frac * heads + 0.5));
    for (int a = 0; a < heads; ++a)  // every INT8 head decays no faster than every INT4 head
      for (int b = 0; b < heads; ++b)
        if (out[a] == 8 && out[b] == 4) CHECK(r[a] > r[b] || (r[a] == r[b] && a < b));
    CHECK(qstate_bits_by_decay(r.data(), heads, 0, 0.5f, 4, 8, out.data()) == QSTATE_OK);
    for (int h = 0; h < heads; ++h) CHECK(out[h] == (r[h] > 0.5f ? 8 : 4));
  }
  std::vector<float> r(4, 1.0f);
  std::vector<uint8_t> out(4);
  CHECK(qstate_bits_by_decay(nullptr, 4, 0, 0.5f, 4, 8, out.data()) == QSTATE_E_INVALID);
  CHECK(qstate_bits_by_decay(r.data(), 0, 0, 0.5f, 4, 8, out.data()) == QSTATE_E_INVALID);
  CHECK(qstate_bits_by_decay(r.data(), 4, 2, 0.5f, 4, 8, out.data()) == QSTATE_E_INVALID);
  CHECK(qstate_bits_by_decay(r.data(), 4, 1, 1.5f, 4, 8, out.data()) == QSTATE_E_INVALID);
  CHECK(qstate_bits_by_decay(r.data(), 4, 0, 0.5f, 5, 8, out.data()) == QSTATE_E_INVALID);
  for (int st = -6; st <= 1; ++st) CHECK(qstate_strerror(st) != nullptr);
  CHECK(qstate_destroy(nullptr) == QSTATE_OK);
  std::printf("ok: %ld configurations (%ld valid), %ld launches checked (%ld persistent)\n",
              configs, g_valid, g_launches, g_persist);
  CHECK(g_valid > 1000 && g_persist > 500);
  return g_fail;
}
