// qstate_key_dk256.hip — key-axis kernels for dk = 256.

#include "qstate_key.h"

namespace qs {

hipError_t launch_key_dk256(Op op, int mixer, int rounding, const KParams& p,
                       hipStream_t stream) {
  return launch_key_dk<256>(op, mixer, rounding, p, stream);
}

}  // namespace qs
