// Backward of one CP rank's attention share for float32 inputs: fp32
// products and sums throughout, built for accuracy on small shares.
//
// Same gradients as the bf16 path ("新流程 CP 多通信模式迁移设计方案" §6.1
// backward, §9.2 GQA): with P = exp(scale*q.k - LSE) on visible pairs,
// Delta = rowsum(dO o O), dS = P o (dO.v - Delta):
//   dQ_i = scale * sum_j dS_ij k_j      (one thread per query row)
//   dV_j = sum_i P_ij dO_i,  dK_j = scale * sum_i dS_ij q_i
//                                       (one thread per key row, summing over
//                                        every query row of every head of the
//                                        key's GQA group)
#include <hip/hip_runtime.h>
#include <math.h>

#include "plan.h"

namespace cpattn {
namespace {

// Storage offset (elements) of key row j beyond j * row stride.
__device__ __forceinline__ int64_t kv_row_adj(const KvChunks &kv, int64_t j) {
  return (kv.store_lg < 31 ? j >> kv.store_lg : j / kv.len) * kv.cadj;
}

__device__ __forceinline__ int64_t row_pos(const BwdParams &p, int r) {
  return p.chunk_pos[r / p.chunk_len] + r % p.chunk_len;
}

// Global position of key row j (its KV chunk's position plus the offset in it).
__device__ __forceinline__ int64_t key_pos(const BwdParams &p, int j) {
  return p.kv.pos[j / p.kv.len] + j % p.kv.len;
}

// Start of the packed sequence holding position pos (the last bound <= pos;
// INT64_MIN without bounds). The loop runs over every bound, so it is uniform
// across threads whatever pos is.
__device__ __forceinline__ int64_t seq_start(const BwdParams &p, int64_t pos) {
  int64_t ds = INT64_MIN;
  for (int i = 0; i < p.docs.n; ++i) ds = p.docs.pos[i] <= pos ? p.docs.pos[i] : ds;
  return ds;
}

template <int D>
__global__ void __launch_bounds__(64) bwd_fp32_delta_dq_kernel(const BwdParams p) {
  const int r = blockIdx.x * 64 + threadIdx.x;   // local query row
  const int h = blockIdx.y, b = blockIdx.z;
  if (r >= p.sq) return;
  const int hk = h / p.group;
  const int64_t qoff = b * p.q_sb + h * p.q_sh + (int64_t)r * p.q_ss + (r / p.chunk_len) * p.q_cadj;
  const int64_t ooff = b * p.o_sb + h * p.o_sh + (int64_t)r * p.o_ss + (r / p.chunk_len) * p.o_cadj;
  const float *q = static_cast<const float *>(p.q) + qoff;
  const float *o = static_cast<const float *>(p.out) + ooff;
  const float *g = static_cast<const float *>(p.dout) + ooff;
  float delta = 0.0f;
  for (int d = 0; d < D; ++d) delta = fmaf(o[d], g[d], delta);
  const int64_t row = ((int64_t)b * p.hq + h) * p.sq + r;
  p.delta[row] = delta;
  const float lse = p.lse[row];
  float dq[D];
  for (int d = 0; d < D; ++d) dq[d] = 0.0f;
  const int64_t qp = row_pos(p, r);
  const int64_t qds = seq_start(p, qp);
  const float *kb = static_cast<const float *>(p.k) + b * p.kv_sb + hk * p.kv_sh;
  const float *vb = static_cast<const float *>(p.v) + b * p.kv_sb + hk * p.kv_sh;
  if (lse != -INFINITY) {
    for (int j = 0; j < p.skv; ++j) {
      if (p.causal && key_pos(p, j) > qp) {
        if (p.kv.n == 1) break;   // natural order: every later key is later still
        continue;
      }
      if (key_pos(p, j) < qds) continue;   // before this row's sequence
      float madd = 0.0f;   // additive user mask (natural units)
      if (p.mask) {
        const uint8_t *mr = p.mask + b * p.m_sb + h * p.m_sh + (int64_t)r * p.m_ss;
        if (p.mask_add) {
          madd = reinterpret_cast<const float *>(mr)[j];
          if (madd <= kMaskHide) continue;   // hidden (-inf included)
        } else if (mr[j] == 0) {
          continue;
        }
      }
      const float *kj = kb + (int64_t)j * p.kv_ss + kv_row_adj(p.kv, j);
      const float *vj = vb + (int64_t)j * p.kv_ss + kv_row_adj(p.kv, j);
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(q[d], kj[d], s);
        dp = fmaf(g[d], vj[d], dp);
      }
      const float pij = expf(s * p.scale + madd - lse);
      const float ds = pij * (dp - delta);
      for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, kj[d], dq[d]);
    }
  }
  float *dst = static_cast<float *>(p.dq) + ooff;
  for (int d = 0; d < D; ++d) dst[d] = dq[d] * p.scale;
}

template <int D>
__global__ void __launch_bounds__(64) bwd_fp32_dkv_kernel(const BwdParams p) {
  const int j = blockIdx.x * 64 + threadIdx.x;   // key row
  const int hk = blockIdx.y, b = blockIdx.z;
  if (j >= p.skv) return;
  const int64_t koff = b * p.kv_sb + hk * p.kv_sh + (int64_t)j * p.kv_ss + kv_row_adj(p.kv, j);
  const float *kj = static_cast<const float *>(p.k) + koff;
  const float *vj = static_cast<const float *>(p.v) + koff;
  float dk[D], dv[D];
  for (int d = 0; d < D; ++d) {
    dk[d] = 0.0f;
    dv[d] = 0.0f;
  }
  const int64_t kp = key_pos(p, j);
  for (int hh = 0; hh < p.group; ++hh) {
    const int h = hk * p.group + hh;
    for (int r = 0; r < p.sq; ++r) {
      if (p.causal && kp > row_pos(p, r)) continue;
      if (kp < seq_start(p, row_pos(p, r))) continue;   // not in the row's sequence
      float madd = 0.0f;   // additive user mask (natural units)
      if (p.mask) {
        const uint8_t *mr = p.mask + b * p.m_sb + h * p.m_sh + (int64_t)r * p.m_ss;
        if (p.mask_add) {
          madd = reinterpret_cast<const float *>(mr)[j];
          if (madd <= kMaskHide) continue;   // hidden (-inf included)
        } else if (mr[j] == 0) {
          continue;
        }
      }
      const int64_t row = ((int64_t)b * p.hq + h) * p.sq + r;
      const float lse = p.lse[row];
      if (lse == -INFINITY) continue;
      const float *q = static_cast<const float *>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)r * p.q_ss +
                       (r / p.chunk_len) * p.q_cadj;
      const float *g = static_cast<const float *>(p.dout) + b * p.o_sb + h * p.o_sh + (int64_t)r * p.o_ss +
                       (r / p.chunk_len) * p.o_cadj;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s = fmaf(q[d], kj[d], s);
        dp = fmaf(g[d], vj[d], dp);
      }
      const float pij = expf(s * p.scale + madd - lse);
      const float ds = pij * (dp - p.delta[row]);
      for (int d = 0; d < D; ++d) {
        dv[d] = fmaf(pij, g[d], dv[d]);
        dk[d] = fmaf(ds, q[d], dk[d]);
      }
    }
  }
  float *dkp = p.dk + (((int64_t)b * p.hkv + hk) * p.skv + j) * D;
  float *dvp = p.dv + (((int64_t)b * p.hkv + hk) * p.skv + j) * D;
  for (int d = 0; d < D; ++d) {
    dkp[d] = dk[d] * p.scale;
    dvp[d] = dv[d];
  }
}

template <int D>
int launch_d(const BwdParams &p, void *stream, void *const *events) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) {
    return events ? (int)hipEventRecord(static_cast<hipEvent_t>(events[i]), s) : 0;
  };
  if (int e = mark(0)) return e;
  if (p.sq > 0) {
    dim3 g1((p.sq + 63) / 64, p.hq, p.batch);
    hipLaunchKernelGGL(bwd_fp32_delta_dq_kernel<D>, g1, dim3(64), 0, s, p);
  }
  if (int e = mark(1)) return e;
  if (p.skv > 0) {
    dim3 g2((p.skv + 63) / 64, p.hkv, p.batch);
    hipLaunchKernelGGL(bwd_fp32_dkv_kernel<D>, g2, dim3(64), 0, s, p);
  }
  if (int e = mark(2)) return e;
  if (int e = mark(3)) return e;
  return (int)hipGetLastError();
}

}  // namespace

int launch_bwd_fp32(const BwdParams &p, int head_dim, void *stream, void *const *events) {
  if (head_dim == 128) return launch_d<128>(p, stream, events);
  if (head_dim == 64) return launch_d<64>(p, stream, events);
  return (int)hipErrorInvalidValue;
}

}  // namespace cpattn
