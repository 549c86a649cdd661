// dQ kernel instantiations of mode 0 (keys in natural order).
#include "bwd_bf16_kernels.h"

namespace cpattn {
int launch_bwd_dq_m0(const BwdParams &p, int head_dim, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128) return launch_dq_mode<128, 0>(p, s);
  if (head_dim == 64) return launch_dq_mode<64, 0>(p, s);
  return (int)hipErrorInvalidValue;
}
}  // namespace cpattn
