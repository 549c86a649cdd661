// Backward dispatch: the Delta pre-pass (and a user mask's bit tables), then
// the dK/dV and dQ instantiations
// of the share's mode (keys in natural order, a KV chunk table, packed
// sequences, a user mask). The kernels live in bwd_bf16_kernels.h; each mode
// is compiled in a file of its own.
#include "bwd_bf16_kernels.h"

namespace cpattn {
namespace {

template <int D>
int launch_d(const BwdParams &p, void *stream, void *const *events) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) {
    return events ? (int)hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : 0;
  };
  if (int e = mark(0)) return e;
  const int64_t rows = (int64_t)p.batch * p.hq * p.sq;
  if (rows > 0) {
    const int64_t blocks = (rows * 16 + 255) / 256;
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(blocks), dim3(256), 0, s, p);
  }
  // The row bits first: for an additive mask that pass also decides whether
  // the tables are used at all.
  if (p.mask_rowbits) {
    if (int e = launch_mask_rowbits(p.mask, p.m_sb, p.m_sh, p.m_ss, p.mb_batches, p.mb_heads, p.sq, p.skv,
                                    p.mask_add != 0, const_cast<uint64_t *>(p.mask_rowbits),
                                    const_cast<uint32_t *>(p.mask_flag), stream))
      return e;
  }
  if (p.mask_bits && p.skv > 0 && p.sq > 0) {
    const int64_t blocks = (int64_t)((p.skv + kMaskBitsBlockKeys - 1) / kMaskBitsBlockKeys) * p.n_q_chunks *
                           p.mb_tpc * p.mb_batches * p.mb_heads;
    hipLaunchKernelGGL(bwd_mask_bits_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, p);
  }
  if (int e = mark(1)) return e;
  int e = p.mask ? launch_bwd_dkdv_m2(p, D, stream)
                 : p.docs.n > 0 ? launch_bwd_dkdv_m1(p, D, stream) : launch_bwd_dkdv_m0(p, D, stream);
  if (e) return e;
  if (int e2 = mark(2)) return e2;
  e = p.mask ? launch_bwd_dq_m3(p, D, stream)
             : p.docs.n > 0 ? launch_bwd_dq_m2(p, D, stream)
                            : p.kv.n > 1 ? launch_bwd_dq_m1(p, D, stream) : launch_bwd_dq_m0(p, D, stream);
  if (e) return e;
  if (int e3 = mark(3)) return e3;
  return (int)hipGetLastError();
}

}  // namespace

int launch_bwd_bf16(const BwdParams &p, int head_dim, void *stream, void *const *events) {
  if (head_dim == 128) return launch_d<128>(p, stream, events);
  if (head_dim == 64) return launch_d<64>(p, stream, events);
  return (int)hipErrorInvalidValue;
}

}  // namespace cpattn
