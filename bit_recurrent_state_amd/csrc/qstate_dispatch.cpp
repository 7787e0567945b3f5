// qstate_dispatch.cpp — picks the kernel source for a launch: the window
// kernels when the state keeps a pure-write window, the key-axis kernels for
// key-axis scale groups, otherwise the value-axis / FP32-state kernels, each
// instantiated per dk in its own translation unit.

#include "qstate_launch.h"

namespace qs {

hipError_t launch(Op op, int mixer, int rounding, int fp32, int dk, const KParams& p,
                  hipStream_t stream) {
  if (p.slices < 1 || p.slice_rows < 1 || (int64_t)p.slices * p.slice_rows < p.dv)
    return hipErrorInvalidValue;
  const int rnd = fp32 ? 0 : rounding;  // the FP32 state has no rounding
  if (!fp32 && p.window_len > 0) {
#define QS_WIN(DK)                                                                   \
  case DK:                                                                           \
    switch (p.window_len) {                                                          \
      case 4: return launch_window_dk##DK##_w4(op, mixer, rnd, p, stream);           \
      case 8: return launch_window_dk##DK##_w8(op, mixer, rnd, p, stream);           \
      case 16: return launch_window_dk##DK##_w16(op, mixer, rnd, p, stream);         \
      default: return hipErrorInvalidValue;                                          \
    }
    switch (dk) {
      QS_WIN(64)
      QS_WIN(128)
      QS_WIN(256)
      default: return hipErrorInvalidValue;
    }
#undef QS_WIN
  }
  if (!fp32 && p.axis == 1) {
    switch (dk) {
      case 64: return launch_key_dk64(op, mixer, rnd, p, stream);
      case 128: return launch_key_dk128(op, mixer, rnd, p, stream);
      case 256: return launch_key_dk256(op, mixer, rnd, p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  const int f = fp32 ? 1 : 0;
  switch (dk) {
    case 64: return launch_value_dk64(op, mixer, rnd, f, p, stream);
    case 128: return launch_value_dk128(op, mixer, rnd, f, p, stream);
    case 256: return launch_value_dk256(op, mixer, rnd, f, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qs
