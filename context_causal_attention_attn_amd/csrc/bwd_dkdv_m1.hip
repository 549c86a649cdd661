// dK/dV kernel instantiations of mode 1 (packed sequences).
#include "bwd_bf16_kernels.h"

namespace cpattn {
int launch_bwd_dkdv_m1(const BwdParams &p, int head_dim, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128) launch_dkdv_mode<128, 1>(p, s);
  else if (head_dim == 64) launch_dkdv_mode<64, 1>(p, s);
  else return (int)hipErrorInvalidValue;
  return 0;
}
}  // namespace cpattn
