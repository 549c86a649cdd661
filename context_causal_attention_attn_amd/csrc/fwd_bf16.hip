// Forward dispatch: the instantiation of the share's mode (keys in natural
// order, a KV chunk table, packed sequences, a user mask). The kernel lives in
// fwd_bf16_kernel.h; each mode is compiled in a file of its own.
#include <hip/hip_runtime.h>

#include "plan.h"

namespace cpattn {

int launch_fwd_bf16(const FwdParams &p, int head_dim, void *stream) {
  if (p.mask) return launch_fwd_bf16_m3(p, head_dim, stream);
  if (p.docs.n > 0) return launch_fwd_bf16_m2(p, head_dim, stream);
  if (p.kv.n > 1) return launch_fwd_bf16_m1(p, head_dim, stream);
  return launch_fwd_bf16_m0(p, head_dim, stream);
}

}  // namespace cpattn
