// A boolean user mask as row bits, for the forward and dQ kernels (bf16).
//
// The query-in-lane kernels hold, per lane, one query row and the keys
// 16*kb + 4*g + i (kb = 0..3, i = 0..3) of a 64-key tile, g the lane's
// group. Word [(bm * heads + hm) * ktiles + kt][row] of the table holds the
// row's 64 keys of tile kt with bit 16*g + 4*kb + i for key 64*kt + 16*kb +
// 4*g + i (1: may be attended; 0 also for keys past the end), so that a lane
// takes its 16 bits with one shift and a wave reads consecutive rows'
// words. bm and hm index the mask's batch and head (0 where it broadcasts).
#include <hip/hip_runtime.h>

#include "plan.h"

namespace cpattn {
namespace {

// One thread per (mask batch/head, key tile, row), rows fastest.
__global__ void __launch_bounds__(256) mask_rowbits_kernel(const uint8_t *mask, int64_t m_sb, int64_t m_sh,
                                                           int64_t m_ss, int32_t heads, int32_t sq, int32_t skv,
                                                           int32_t ktiles, int64_t total, uint64_t *bits) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int row = (int)(idx % sq);
  const int kt = (int)((idx / sq) % ktiles);
  const int bh = (int)(idx / ((int64_t)sq * ktiles));
  const int bm = bh / heads, hm = bh % heads;
  const uint8_t *src = mask + bm * m_sb + hm * m_sh + (int64_t)row * m_ss + (int64_t)kt * 64;
  const int n = min(64, skv - kt * 64);
  uint64_t w = 0;
  if (n == 64) {
    // 16 words of 4 keys (rows start on 4-byte boundaries): word e4 holds
    // keys 4*e4 .. +3, i.e. kb = e4 / 4, g = e4 % 4.
#pragma unroll
    for (int e4 = 0; e4 < 16; ++e4) {
      const uint32_t v = reinterpret_cast<const uint32_t *>(src)[e4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((v >> (8 * i)) & 0xffu) w |= (uint64_t)1 << (16 * (e4 % 4) + 4 * (e4 / 4) + i);
    }
  } else {
    for (int e = 0; e < n; ++e)
      if (src[e]) w |= (uint64_t)1 << (16 * ((e >> 2) & 3) + 4 * (e >> 4) + (e & 3));
  }
  bits[idx] = w;
}

}  // namespace

int launch_mask_rowbits(const uint8_t *mask, int64_t m_sb, int64_t m_sh, int64_t m_ss, int32_t batches,
                        int32_t heads, int32_t sq, int32_t skv, uint64_t *bits, void *stream) {
  const int32_t ktiles = (skv + 63) / 64;
  const int64_t total = (int64_t)batches * heads * ktiles * sq;
  if (total == 0) return 0;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(mask_rowbits_kernel, dim3((uint32_t)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     mask, m_sb, m_sh, m_ss, heads, sq, skv, ktiles, total, bits);
  return (int)hipGetLastError();
}

}  // namespace cpattn
