// qstate_value_dk256.hip — value-axis and FP32-state kernels for dk = 256.

#include "qstate_persist.h"

namespace qs {

hipError_t launch_value_dk256(Op op, int mixer, int rounding, int fp32, const KParams& p,
                         hipStream_t stream) {
  return launch_value_dk<256>(op, mixer, rounding, fp32, p, stream);
}

}  // namespace qs
