// Forward of one CP rank's attention share, bf16 inputs, fp32 accumulation,
// on gfx950 matrix cores.
//
// What is computed: for every local query row (global position from its
// chunk) the softmax over the visible gathered keys of scale * q.k, applied to
// v, plus the natural-log LSE ("新流程 CP 多通信模式迁移设计方案" §6.1 local-Q /
// global-KV attention, §8 global-position causal mask, §9.2 GQA).
//
// How (one workgroup = 4 wavefronts = one work item):
//  * a work item is a tile of query rows of one chunk for a pack of query
//    heads that read the same KV head (GQA); K/V tiles of 64 keys are staged
//    through LDS once per workgroup and read by every head of the pack;
//  * each wavefront owns 32 query rows of one head and computes the transposed
//    score tile S^T = K Q^T (keys x queries) with v_mfma_f32_32x32x16_bf16, so
//    that a lane holds one query column: the row max and sum of the online
//    softmax are lane-local plus one permlane32 swap between the two halves of
//    the wavefront;
//  * the probabilities P^T, converted to bf16 in registers, are the B operand
//    of O^T += V^T P^T without any shuffle: the contraction index (keys) is
//    permuted identically in both operands, and V^T is read from the
//    row-major V tile with the gfx950 LDS transpose read ds_read_b64_tr_b16;
//  * KV tiles wholly after a wavefront's last query are skipped; only tiles
//    crossing the causal diagonal (or the ragged end of K/V) are masked
//    element-wise; the running max is only moved (and O rescaled) when a new
//    score exceeds it by more than 2^8, which keeps exp2 arguments <= 8;
//  * K/V tiles are double-buffered: the global loads of tile t+1 are in flight
//    while tile t is computed.
#include <hip/hip_runtime.h>
#include <math.h>

#include "gfx950_common.h"
#include "plan.h"

namespace cpattn {
namespace {

constexpr int BN = kFwdBlockKV;
constexpr int NT = kFwdWaves * 64;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D, int RB>
__global__ void __launch_bounds__(NT, 2) fwd_bf16_kernel(const FwdParams p) {
  constexpr int HPW = kFwdWaves / RB;  // heads per work item
  constexpr int BM = kWaveRows * RB;   // query rows per work item
  constexpr int NC = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int LOADS = BN * NC / NT;
  using T = Tile<D>;

  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BN * D];  // [stage][K,V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work item ---------------------------------------------------------
  const int bid = blockIdx.x;
  const int pack = bid % p.n_head_packs;
  const int rank = bid / p.n_head_packs;
  const int ci = rank / p.tiles_per_chunk;
  const int tile = p.tiles_per_chunk - 1 - (rank % p.tiles_per_chunk);
  const int chunk = p.chunk_idx[ci];
  const int64_t chunk_pos = p.chunk_pos[ci];
  const int packs_per_batch = p.hq / HPW;
  const int b = pack / packs_per_batch;
  const int head0 = (pack % packs_per_batch) * HPW;
  const int hkv = head0 / p.group;
  const int item_row0 = tile * BM;                          // row within the chunk
  const int item_rows = min(BM, p.chunk_len - item_row0);
  const int64_t item_qhi = chunk_pos + item_row0 + item_rows - 1;

  const int head = head0 + wave / RB;
  const int wrow0 = (wave % RB) * kWaveRows;
  const int wrows = max(0, min(kWaveRows, item_rows - wrow0));
  const int64_t wave_qlo = chunk_pos + item_row0 + wrow0;
  const int64_t wave_qhi = wave_qlo + max(wrows, 1) - 1;
  const bool qvalid = col < wrows;
  const int64_t qpos = wave_qlo + min(col, max(wrows - 1, 0));
  const int local_row = chunk * p.chunk_len + item_row0 + wrow0 + col;

  int nvis = p.skv;
  if (p.causal) {
    const int64_t n = item_qhi - p.kv_pos0 + 1;
    nvis = (int)(n < 0 ? 0 : (n > p.skv ? p.skv : n));
  }
  const int ntiles = (nvis + BN - 1) / BN;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole item
  bf16x8 qf[KSTEPS];
  {
    const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + head * p.q_sh +
                       (int64_t)local_row * p.q_ss + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (qvalid) {
        qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[s][e] = (__bf16)0.0f;
      }
    }
  }

  // ---- K/V staging --------------------------------------------------------
  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + hkv * p.kv_sh;
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + hkv * p.kv_sh;
  u32x4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = tid + NT * i;
      const int row = idx / NC, c = idx % NC;
      const int key = kt * BN + row;
      if (key < p.skv) {
        const int64_t o = (int64_t)key * p.kv_ss + c * 8;
        kreg[i] = *reinterpret_cast<const u32x4 *>(kbase + o);
        vreg[i] = *reinterpret_cast<const u32x4 *>(vbase + o);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto swrite = [&](int stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = tid + NT * i;
      const int row = idx / NC, c = idx % NC;
      *reinterpret_cast<u32x4 *>(&smem[stage][0][T::chunk_off(row, c)]) = kreg[i];
      *reinterpret_cast<u32x4 *>(&smem[stage][1][T::chunk_off(row, c)]) = vreg[i];
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
  float m_run = -INFINITY;  // running max of scale*log2(e)*s (may lag the true max)
  float l_part = 0.0f;      // this lane's partial row sum (its half of the keys)
  const float c = p.scale_log2;

  if (ntiles > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int kt = 0; kt < ntiles; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < ntiles) gload(kt + 1);
    const int64_t tile_plo = p.kv_pos0 + (int64_t)kt * BN;
    const bool active = wrows > 0 && (!p.causal || tile_plo <= wave_qhi);
    if (active) {
      const __bf16 *ks = smem[st][0];
      const __bf16 *vs = smem[st][1];
      // S^T tile [64 keys x 32 queries] as two 32x32 accumulators.
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(ks + T::chunk_off(kb * 32 + col, 2 * s + half));
          sacc[kb] = mfma32(kf, qf[s], sacc[kb]);
        }
      }
      const bool need_mask = (kt * BN + BN > p.skv) || (p.causal && tile_plo + BN - 1 > wave_qlo);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt * BN + kb * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
            const bool hide = key >= p.skv || (p.causal && p.kv_pos0 + key > qpos);
            if (hide) sacc[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = pair_max(mx) * c;
      const bool upd = mx > m_run + kRescaleSlack;
      if (__any(upd)) {
        const float m_new = upd ? mx : m_run;
        const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_run = m_new;
      }
      const float mneg = (m_run == -INFINITY) ? 0.0f : -m_run;
      // P^T = exp2(c*s - m) as bf16 B operands, one per 16-key step.
      bf16x8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, mneg));
          l_part += pv;
          pf[kb * 2 + (i >> 3)][i & 7] = (__bf16)pv;
        }
      // O^T += V^T P^T.
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2)
          oacc[db] = mfma32(tr_operand<D>(vs, 16 * k2, 32 * db, lane), pf[k2], oacc[db]);
    }
    if (kt + 1 < ntiles) swrite(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  if (wrows == 0) return;
  const float l = pair_sum(l_part);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  if (qvalid) {
    __bf16 *op = static_cast<__bf16 *>(p.out) + b * p.o_sb + head * p.o_sh + (int64_t)local_row * p.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * g + 4 * half) = o4;
      }
    if (half == 0) {
      const float lse = l > 0.0f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
      p.lse[((int64_t)b * p.hq + head) * p.sq + local_row] = lse;
    }
  }
}

template <int D>
int launch_d(const FwdParams &p, void *stream) {
  const int64_t grid = fwd_grid_size(p);
  if (grid == 0) return 0;
  const int rb = kFwdWaves / p.heads_per_item;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (rb) {
    case 1: hipLaunchKernelGGL((fwd_bf16_kernel<D, 1>), dim3(grid), dim3(NT), 0, s, p); break;
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<D, 2>), dim3(grid), dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((fwd_bf16_kernel<D, 4>), dim3(grid), dim3(NT), 0, s, p); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_fwd_bf16(const FwdParams &p, int head_dim, void *stream) {
  if (head_dim == 128) return launch_d<128>(p, stream);
  if (head_dim == 64) return launch_d<64>(p, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace cpattn
