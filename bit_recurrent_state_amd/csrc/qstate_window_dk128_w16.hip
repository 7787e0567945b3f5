// qstate_window_dk128_w16.hip — decode step with a pure-write window of W = 16
// pairs for dk = 128.

#include "qstate_window.h"

namespace qs {

hipError_t launch_window_dk128_w16(Op op, int mixer, int rounding, const KParams& p,
                              hipStream_t stream) {
  return launch_pw_g<128, 16>(op, mixer, rounding, p, stream);
}

}  // namespace qs
