// Forward kernel instantiations of mode 1 (a KV chunk table).
#include "fwd_bf16_kernel.h"

namespace cpattn {
int launch_fwd_bf16_m1(const FwdParams &p, int head_dim, void *stream) {
  return launch_fwd_mode_d<1>(p, head_dim, stream);
}
}  // namespace cpattn
