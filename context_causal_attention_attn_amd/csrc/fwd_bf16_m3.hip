// Forward kernel instantiations of mode 3 (a user attention mask).
#include "fwd_bf16_kernel.h"

namespace cpattn {
int launch_fwd_bf16_m3(const FwdParams &p, int head_dim, void *stream) {
  return launch_fwd_mode_d<3>(p, head_dim, stream);
}
}  // namespace cpattn
