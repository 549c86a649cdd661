// dQ kernel instantiations of mode 3 (a user attention mask).
#include "bwd_bf16_kernels.h"

namespace cpattn {
int launch_bwd_dq_m3(const BwdParams &p, int head_dim, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128) return launch_dq_mode<128, 3>(p, s);
  if (head_dim == 64) return launch_dq_mode<64, 3>(p, s);
  return (int)hipErrorInvalidValue;
}
}  // namespace cpattn
