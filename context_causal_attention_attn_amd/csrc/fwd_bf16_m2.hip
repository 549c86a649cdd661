// Forward kernel instantiations of mode 2 (packed sequences).
#include "fwd_bf16_kernel.h"

namespace cpattn {
int launch_fwd_bf16_m2(const FwdParams &p, int head_dim, void *stream) {
  return launch_fwd_mode_d<2>(p, head_dim, stream);
}
}  // namespace cpattn
