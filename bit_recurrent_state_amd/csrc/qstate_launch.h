// qstate_launch.h — internal interface between the C ABI (qstate_api.cpp)
// and the gfx950 kernels (qstate_value_dk*.hip, qstate_key_dk*.hip).  Not
// installed, not part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace qs {

// Division by a launch constant d: q = (mulhi(x, m) + x) >> s for x < 2^31,
// with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1.
struct FastDiv {
  uint32_t m, s;
};

// Everything a kernel needs for one launch, passed by value.
struct KParams {
  void* state;           // codes (quantized) or float S (FP32 state)
  float* scales;         // [B][H][dv][dk/G] (value axis) or [B][H][dv/G][dk] (key axis)
  const float* q;        // [B][H][dk]
  const float* k;        // [B][H][dk]
  const float* v;        // [B][H][dv]
  const float* alpha;    // [B][H] or [B][H][dk] (GLA, KDA)
  const float* beta;     // [B][H] (GDN, scalar, KDA) or null
  float* o;              // [B][H][dv] or null
  const float* src;      // import: FP32 state to quantize
  float* dst;            // export: dequantized FP32 state
  int32_t B, H, dv, G;
  int32_t axis;          // scale groups: 0 value axis, 1 key axis
  int32_t slices;        // workgroups per head (row slices); the grid is B*H*slices
  int32_t slice_rows;    // rows per slice: a multiple of 32 (value axis) or of
                         // the key-axis block rows max(G, 4096/dk)
  uint64_t bytes_per_b;        // code bytes of one batch row (all heads)
  uint16_t int8_blocks[256];   // per head: bit q set = 16-column block q is INT8
  int32_t mixed;               // some head mixes INT8 and INT4 blocks
  uint32_t head_units[256];    // per head: byte offset in a batch row / (8 dv)
  uint64_t seed;
  uint32_t layer;
  uint64_t step;         // stochastic-rounding counter of this event
  uint8_t* window;       // pure-write window areas of all heads, or null
  int32_t window_len;    // W: 0 (none), 4, 8 or 16
  uint64_t window_head_bytes;  // bytes of one head's window area
  int32_t lrb_merge;     // low-rank bypass: this step merges the whole buffer
  float lrb_theta;       // low-rank bypass: merge threshold, in group scales
  // Persistent value-axis step (persist != 0): work units of a fixed row
  // count, INT8 heads first, then INT4 heads, each class in (b, h) order.
  int32_t persist;
  uint32_t n_units;            // B * H * units_per_head
  int32_t units_per_head;
  int32_t n8_heads;            // head indices h with INT8 width
  FastDiv div_group, div_n8, div_n4;  // by 8 * units_per_head, n8_heads, H - n8_heads
  uint32_t head_order[256];    // the INT8 head indices, then the INT4 ones, ascending
};

enum Op { kStep = 0, kImport = 1, kExport = 2, kReadout = 3 };

// Rows of one work unit of the persistent step: one trip of the INT4 load
// ring (4 iterations of 64 / (dk / 32) rows).
constexpr int persist_unit_rows(int dk) { return 4 * 64 / (dk / 32); }

// Launch one kernel over all B*H heads on `stream`.  Returns hipSuccess or
// the launch error.  mixer/rounding as in qstate.h; fp32 selects the
// unquantized-state kernels.  (qstate_dispatch.cpp)
hipError_t launch(Op op, int mixer, int rounding, int fp32, int dk,
                  const KParams& p, hipStream_t stream);

// Per-dk (and per window length) entry points of the kernel sources
// (qstate_value_dk*.hip, qstate_key_dk*.hip, qstate_window_dk*_w*.hip), one
// translation unit each.
hipError_t launch_value_dk64(Op op, int mixer, int rounding, int fp32, const KParams& p,
                             hipStream_t stream);
hipError_t launch_value_dk128(Op op, int mixer, int rounding, int fp32, const KParams& p,
                              hipStream_t stream);
hipError_t launch_value_dk256(Op op, int mixer, int rounding, int fp32, const KParams& p,
                              hipStream_t stream);
hipError_t launch_window_dk64_w4(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk64_w8(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk64_w16(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk128_w4(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk128_w8(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk128_w16(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk256_w4(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk256_w8(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_window_dk256_w16(Op op, int mixer, int rounding, const KParams& p,
                                hipStream_t stream);
hipError_t launch_key_dk64(Op op, int mixer, int rounding, const KParams& p, hipStream_t stream);
hipError_t launch_key_dk128(Op op, int mixer, int rounding, const KParams& p, hipStream_t stream);
hipError_t launch_key_dk256(Op op, int mixer, int rounding, const KParams& p, hipStream_t stream);

}  // namespace qs
