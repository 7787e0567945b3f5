// qstate_key_dk128.hip — key-axis kernels for dk = 128.

#include "qstate_key.h"

namespace qs {

hipError_t launch_key_dk128(Op op, int mixer, int rounding, const KParams& p,
                       hipStream_t stream) {
  return launch_key_dk<128>(op, mixer, rounding, p, stream);
}

}  // namespace qs
