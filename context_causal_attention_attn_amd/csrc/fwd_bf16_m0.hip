// Forward kernel instantiations of mode 0 (keys in natural order).
#include "fwd_bf16_kernel.h"

namespace cpattn {
int launch_fwd_bf16_m0(const FwdParams &p, int head_dim, void *stream) {
  return launch_fwd_mode_d<0>(p, head_dim, stream);
}
}  // namespace cpattn
