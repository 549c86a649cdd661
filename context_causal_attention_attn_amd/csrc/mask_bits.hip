// A user mask as row bits, for the forward and dQ kernels (bf16).
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

// One thread per (mask batch/head, key tile, row), rows fastest. ADD: the
// mask holds float32 values; a key is kept unless its value is at most
// kMaskHide, and a value that is neither 0 nor hiding marks *flag. Once the
// flag is seen marked the table is not used and wavefronts stop early.
template <bool ADD>
__global__ void __launch_bounds__(256) mask_rowbits_kernel(const uint8_t *mask, int64_t m_sb, int64_t m_sh,
                                                           int64_t m_ss, int32_t heads, int32_t sq, int32_t skv,
                                                           int32_t ktiles, int64_t total, uint64_t *bits,
                                                           uint32_t *flag) {
  if constexpr (ADD) {
    if (__atomic_load_n(flag, __ATOMIC_RELAXED) != 0) return;
  }
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  bool impure = false;
  if (idx < total) {
    const int row = (int)(idx % sq);
    const int kt = (int)((idx / sq) % ktiles);
    const int bh = (int)(idx / ((int64_t)sq * ktiles));
    const int bm = bh / heads, hm = bh % heads;
    const uint8_t *src = mask + bm * m_sb + hm * m_sh + (int64_t)row * m_ss + (int64_t)kt * 64 * (ADD ? 4 : 1);
    const int n = min(64, skv - kt * 64);
    uint64_t w = 0;
    if constexpr (ADD) {
      const float *f = reinterpret_cast<const float *>(src);
      auto take = [&](float v, int e) {
        if (!(v <= kMaskHide)) w |= (uint64_t)1 << (16 * ((e >> 2) & 3) + 4 * (e >> 4) + (e & 3));
        impure = impure || !(v <= kMaskHide || v == 0.0f);
      };
      if (n == 64) {
        // 16 reads of 4 keys (rows start on 16-byte boundaries).
#pragma unroll
        for (int e4 = 0; e4 < 16; ++e4) {
          const float4 v = reinterpret_cast<const float4 *>(f)[e4];
          take(v.x, 4 * e4);
          take(v.y, 4 * e4 + 1);
          take(v.z, 4 * e4 + 2);
          take(v.w, 4 * e4 + 3);
        }
      } else {
        for (int e = 0; e < n; ++e) take(f[e], e);
      }
    } else if (n == 64) {
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
  if constexpr (ADD) {
    // One atomic per wavefront that saw such a value, skipped once the flag
    // is seen set.
    if (__ballot(impure) != 0 && (threadIdx.x & 63) == 0 && __atomic_load_n(flag, __ATOMIC_RELAXED) == 0)
      atomicOr(flag, 1u);
  }
}

__global__ void mask_flag_clear_kernel(uint32_t *flag) { *flag = 0; }

}  // namespace

int launch_mask_rowbits(const uint8_t *mask, int64_t m_sb, int64_t m_sh, int64_t m_ss, int32_t batches,
                        int32_t heads, int32_t sq, int32_t skv, bool additive, uint64_t *bits, uint32_t *flag,
                        void *stream) {
  const int32_t ktiles = (skv + 63) / 64;
  const int64_t total = (int64_t)batches * heads * ktiles * sq;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (additive) hipLaunchKernelGGL(mask_flag_clear_kernel, dim3(1), dim3(1), 0, s, flag);
  if (total > 0) {
    const int64_t blocks = (total + 255) / 256;
    if (additive)
      hipLaunchKernelGGL(mask_rowbits_kernel<true>, dim3((uint32_t)blocks), dim3(256), 0, s, mask, m_sb, m_sh, m_ss,
                         heads, sq, skv, ktiles, total, bits, flag);
    else
      hipLaunchKernelGGL(mask_rowbits_kernel<false>, dim3((uint32_t)blocks), dim3(256), 0, s, mask, m_sb, m_sh,
                         m_ss, heads, sq, skv, ktiles, total, bits, flag);
  }
  return (int)hipGetLastError();
}

}  // namespace cpattn
