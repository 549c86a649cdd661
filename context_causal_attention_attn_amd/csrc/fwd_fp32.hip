// Forward of one CP rank's attention share for float32 inputs (the tiny
// full-precision share): fp32 products and sums throughout.
//
// Same computation as the bf16 path ("新流程 CP 多通信模式迁移设计方案" §6.1
// local-Q / global-KV attention, §8 global-position causal mask, §9.2 GQA),
// built for accuracy rather than speed: one thread owns one query row and
// keeps q and its output row in registers; 32-key K/V tiles are staged through
// LDS and read as broadcasts; the online softmax runs per key in fp32.
#include <hip/hip_runtime.h>
#include <math.h>

#include "plan.h"

namespace cpattn {
namespace {

// Storage offset (elements) of key row j beyond j * row stride.
__device__ __forceinline__ int64_t kv_row_adj(const KvChunks &kv, int64_t j) {
  return (kv.store_lg < 31 ? j >> kv.store_lg : j / kv.len) * kv.cadj;
}

constexpr int kRows = 64;     // query rows per workgroup (one per thread)
constexpr int kKeys = 32;     // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(kRows) fwd_fp32_kernel(const FwdParams p) {
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];
  const int tiles_per_chunk = (p.chunk_len + kRows - 1) / kRows;
  const int chunk = blockIdx.x / tiles_per_chunk;
  const int row0 = (blockIdx.x % tiles_per_chunk) * kRows;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  const int hkv = head / p.group;
  const int t = threadIdx.x;

  // chunk_pos/chunk_idx are in scheduling order; find this chunk's position.
  int64_t chunk_pos = 0;
  for (int i = 0; i < p.n_q_chunks; ++i)
    if (p.chunk_idx[i] == chunk) chunk_pos = p.chunk_pos[i];

  const int nrows = min(kRows, p.chunk_len - row0);
  const bool valid = t < nrows;
  const int local_row = chunk * p.chunk_len + row0 + (valid ? t : 0);
  const int64_t qpos = chunk_pos + row0 + (valid ? t : 0);
  const int64_t qhi = chunk_pos + row0 + nrows - 1;

  float q[D], o[D];
  const float *qp = static_cast<const float *>(p.q) + b * p.q_sb + head * p.q_sh + chunk * p.q_cadj +
                    (int64_t)local_row * p.q_ss;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = valid ? qp[d] : 0.0f;
    o[d] = 0.0f;
  }
  const float scale = p.scale;
  float m = -INFINITY, l = 0.0f;
  // Packed sequences: keys before the start of this row's sequence (the last
  // bound <= its position; the scan is uniform over the block) are hidden.
  int64_t ds = INT64_MIN;
  for (int i = 0; i < p.docs.n; ++i) ds = p.docs.pos[i] <= qpos ? p.docs.pos[i] : ds;
  // User mask row of this query (NULL: no mask).
  const uint8_t *mrow = p.mask ? p.mask + b * p.m_sb + head * p.m_sh + (int64_t)local_row * p.m_ss : nullptr;

  const float *kb = static_cast<const float *>(p.k) + b * p.kv_sb + hkv * p.kv_sh;
  const float *vb = static_cast<const float *>(p.v) + b * p.kv_sb + hkv * p.kv_sh;
  // KV chunk by KV chunk (the natural order is one chunk): the keys of chunk
  // kc at positions kpos.. that the block's last row can see.
  for (int kc = 0; kc < p.kv.n; ++kc) {
    const int64_t kpos = p.kv.pos[kc];
    const int krow0 = kc * p.kv.len;
    int nvis = p.kv.len;
    if (p.causal) {
      const int64_t n = qhi - kpos + 1;
      nvis = (int)(n < 0 ? 0 : (n > p.kv.len ? p.kv.len : n));
    }
    for (int j0 = 0; j0 < nvis; j0 += kKeys) {
      __syncthreads();
      for (int e = t; e < kKeys * D; e += kRows) {
        const int r = e / D, d = e % D;
        const int key = krow0 + j0 + r;
        ks[r][d] = j0 + r < p.kv.len ? kb[(int64_t)key * p.kv_ss + kv_row_adj(p.kv, key) + d] : 0.0f;
        vs[r][d] = j0 + r < p.kv.len ? vb[(int64_t)key * p.kv_ss + kv_row_adj(p.kv, key) + d] : 0.0f;
      }
      __syncthreads();
      const int nk = min(kKeys, nvis - j0);
      for (int r = 0; r < nk; ++r) {
        if (p.causal && (kpos + j0 + r > qpos || kpos + j0 + r < ds)) continue;
        float madd = 0.0f;   // additive user mask (natural units)
        if (mrow) {
          if (p.mask_add) {
            madd = reinterpret_cast<const float *>(mrow)[krow0 + j0 + r];
            if (madd <= kMaskHide) continue;   // hidden (-inf included)
          } else if (mrow[krow0 + j0 + r] == 0) {
            continue;
          }
        }
        float s = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(q[d], ks[r][d], s);
        s = s * scale + madd;
        const float m_new = fmaxf(m, s);
        const float alpha = expf(m - m_new);   // 0 on the first visible key
        const float w = expf(s - m_new);
        l = l * alpha + w;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(w, vs[r][d], o[d] * alpha);
        m = m_new;
      }
    }
  }
  if (!valid) return;
  float *op = static_cast<float *>(p.out) + b * p.o_sb + head * p.o_sh + chunk * p.o_cadj +
              (int64_t)local_row * p.o_ss;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int d = 0; d < D; ++d) op[d] = o[d] * inv;
  p.lse[((int64_t)b * p.hq + head) * p.sq + local_row] = l > 0.0f ? m + logf(l) : -INFINITY;
}

}  // namespace

int launch_fwd_fp32(const FwdParams &p, int head_dim, void *stream) {
  const int tiles = (p.chunk_len + kRows - 1) / kRows;
  const int batch = p.n_head_packs * p.heads_per_item / p.hq;
  if (tiles == 0) return 0;
  dim3 grid(tiles * p.n_q_chunks, p.hq, batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64) {
    hipLaunchKernelGGL(fwd_fp32_kernel<64>, grid, dim3(kRows), 0, s, p);
  } else if (head_dim == 128) {
    hipLaunchKernelGGL(fwd_fp32_kernel<128>, grid, dim3(kRows), 0, s, p);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace cpattn
