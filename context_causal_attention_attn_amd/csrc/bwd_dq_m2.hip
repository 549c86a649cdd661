// dQ kernel instantiations of mode 2 (packed sequences).
#include "bwd_bf16_kernels.h"

namespace cpattn {
int launch_bwd_dq_m2(const BwdParams &p, int head_dim, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128) return launch_dq_mode<128, 2>(p, s);
  if (head_dim == 64) return launch_dq_mode<64, 2>(p, s);
  return (int)hipErrorInvalidValue;
}
}  // namespace cpattn
