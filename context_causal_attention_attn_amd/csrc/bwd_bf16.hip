// Backward of one CP rank's attention share, bf16 inputs, fp32 accumulation,
// on gfx950 matrix cores.
//
// Gradients of sum(dout * out) for the share ("新流程 CP 多通信模式迁移设计方案"
// §6.1 backward: dQ stays local and needs no communication; dK/dV are this
// share's partial sums over the gathered K/V, which a reduce-scatter(sum)
// would combine across ranks; §9.2: under GQA a KV head collects the sum over
// its group of query heads). With P = exp(scale*q.k - LSE) on visible pairs:
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - Delta),  Delta = rowsum(dO o O),
//     dQ = scale * dS K,  dK = scale * dS^T Q.
//
// Three launches:
//  1. bwd_pre: Delta for every local row, and the fp32 dQ accumulator zeroed;
//  2. bwd_main: one workgroup (4 wavefronts) per 128-key tile of one KV head.
//     Each wavefront owns 32 keys and keeps their K and V rows (MFMA B
//     operands) and their dK^T/dV^T accumulators in registers, while the
//     workgroup streams 32-row query tiles -- of every head of the GQA group
//     and every chunk of the share -- that can see one of its keys. Per tile:
//     S = Q K^T and dP = dO V^T (lane = key column), P and dS in registers,
//     dV^T += dO^T P and dK^T += Q^T dS with dO^T/Q^T read by LDS transpose
//     reads; dS^T goes once through LDS so that dQ^T = K^T dS^T (K^T resident
//     per wavefront) sums over the 128 keys, and is added to the fp32 dQ
//     accumulator with atomics. Query tiles wholly before the key tile are
//     never visited; tiles crossing the diagonal are masked element-wise.
//  3. bwd_dq_convert: dQ = scale * accumulator, rounded to bf16.
#include <hip/hip_runtime.h>
#include <math.h>

#include "gfx950_common.h"
#include "plan.h"

namespace cpattn {
namespace {

constexpr int BK = kBwdBlockKV;   // keys per workgroup
constexpr int BQ = kBwdBlockQ;    // query rows per step
constexpr int NT = 256;

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO o O) and dQ accumulator = 0. 16 lanes per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const BwdParams p) {
  constexpr int LPR = 16;                  // lanes per row
  constexpr int EPL = D / LPR;             // elements per lane (8 or 4)
  const int64_t rows = (int64_t)p.batch * p.hq * p.sq;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < rows) {
    const int64_t bh = row / p.sq;
    const int r = (int)(row % p.sq);
    const int b = (int)(bh / p.hq), h = (int)(bh % p.hq);
    const int64_t off = b * p.o_sb + h * p.o_sh + (int64_t)r * p.o_ss + part * EPL;
    const __bf16 *o = static_cast<const __bf16 *>(p.out) + off;
    const __bf16 *g = static_cast<const __bf16 *>(p.dout) + off;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    float *dqa = p.dq_acc + row * D + part * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4) *reinterpret_cast<f32x4 *>(dqa + e) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && part == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * accumulator -> bf16
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) bwd_dq_convert_kernel(const BwdParams p) {
  constexpr int VPR = D / 4;  // float4 vectors per row
  const int64_t n = (int64_t)p.batch * p.hq * p.sq * VPR;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t row = i / VPR;
  const int c = (int)(i % VPR);
  const int64_t bh = row / p.sq;
  const int r = (int)(row % p.sq);
  const int b = (int)(bh / p.hq), h = (int)(bh % p.hq);
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p.dq_acc + row * D + 4 * c);
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = (__bf16)(a[e] * p.scale);
  *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(p.dq) + b * p.o_sb + h * p.o_sh +
                              (int64_t)r * p.o_ss + 4 * c) = o;
}

// ---------------------------------------------------------------------------
// 2. main backward
// ---------------------------------------------------------------------------
struct StepGeom {
  int chunk, tile, head_in_group;
};

template <int D>
__global__ void __launch_bounds__(NT, 1) bwd_main_kernel(const BwdParams p) {
  constexpr int NC = D / 8;
  constexpr int KSTEPS = D / 16;          // MFMA k-steps over head_dim
  constexpr int DB = D / 32;              // 32-wide blocks of head_dim
  constexpr int WPD = 4 / DB;             // wavefronts sharing one dQ d-block (1 or 2)
  constexpr int QK_KEYS = BK / WPD;       // keys each wavefront sums for dQ
  constexpr int QK_STEPS = QK_KEYS / 16;
  constexpr int Q_LOADS = BQ * NC / NT;   // 16-byte chunks per thread per Q (or dO) tile
  constexpr int K_LOADS = BK * NC / NT;
  static_assert(Q_LOADS >= 1 && K_LOADS >= 1, "tile sizes");
  using TQ = Tile<D>;
  using TS = Tile<BQ>;

  // LDS: [0, BK*D) holds the K tile during set-up, then the two stages of the
  // Q and dO tiles; dS^T [BK keys][BQ queries] follows; then LSE and Delta.
  __shared__ __attribute__((aligned(16))) __bf16 lds[BK * D + BK * BQ];
  __shared__ float lse_s[2][BQ];
  __shared__ float dl_s[2][BQ];
  __bf16 *const k_s = lds;
  __bf16 *const ds_s = lds + BK * D;
  auto q_s = [&](int st) { return lds + st * (2 * BQ * D); };
  auto do_s = [&](int st) { return lds + st * (2 * BQ * D) + BQ * D; };
  static_assert(4 * BQ * D <= BK * D, "Q/dO stages must fit in the K set-up region");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int groups = p.batch * p.hkv;
  const int g = blockIdx.x % groups;
  const int kt = blockIdx.x / groups;
  const int b = g / p.hkv;
  const int hk = g % p.hkv;
  const int key0 = kt * BK;
  const int wkey0 = key0 + 32 * wave;     // first key of this wavefront's S/dP columns
  const int my_key = wkey0 + col;
  const bool key_ok = my_key < p.skv;
  const int64_t kv_lo = p.kv_pos0 + key0;

  const __bf16 *kg = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + hk * p.kv_sh;
  const __bf16 *vg = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + hk * p.kv_sh;

  // ---- set-up: K/V rows of this lane's key (B operands of S and dP) ------
  bf16x8 kf[KSTEPS], vf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    if (key_ok) {
      kf[s] = *reinterpret_cast<const bf16x8 *>(kg + (int64_t)my_key * p.kv_ss + 16 * s + 8 * half);
      vf[s] = *reinterpret_cast<const bf16x8 *>(vg + (int64_t)my_key * p.kv_ss + 16 * s + 8 * half);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kf[s][e] = (__bf16)0.0f;
        vf[s][e] = (__bf16)0.0f;
      }
    }
  }
  // K tile into LDS, then K^T operands of dQ^T = K^T dS^T for this wavefront.
#pragma unroll
  for (int i = 0; i < K_LOADS; ++i) {
    const int idx = tid + NT * i;
    const int row = idx / NC, c = idx % NC;
    const int key = key0 + row;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (key < p.skv) val = *reinterpret_cast<const u32x4 *>(kg + (int64_t)key * p.kv_ss + 8 * c);
    *reinterpret_cast<u32x4 *>(k_s + TQ::chunk_off(row, c)) = val;
  }
  __syncthreads();
  const int dq_dblk = wave % DB;          // d-block of dQ this wavefront produces
  const int dq_key0 = (wave / DB) * QK_KEYS;  // its keys within the tile
  bf16x8 ktf[QK_STEPS];
#pragma unroll
  for (int s = 0; s < QK_STEPS; ++s) ktf[s] = tr_operand<D>(k_s, dq_key0 + 16 * s, 32 * dq_dblk, lane);
  __syncthreads();  // the K region is reused for the Q/dO stages below

  // ---- the query tiles this key tile meets --------------------------------
  const int nq_tiles = (p.chunk_len + BQ - 1) / BQ;
  int first_tile[kMaxQChunks];
  int total = 0;
  for (int c = 0; c < p.n_q_chunks; ++c) {
    int t0 = 0;
    if (p.causal) {
      const int64_t rel = kv_lo - p.chunk_pos[c];   // rows before it cannot see the tile
      t0 = rel <= 0 ? 0 : (int)min<int64_t>(nq_tiles, rel / BQ);
    }
    first_tile[c] = t0;
    total += (nq_tiles - t0) * p.group;
  }
  auto decode = [&](int it) {
    StepGeom sg{0, 0, 0};
    for (int c = 0; c < p.n_q_chunks; ++c) {
      const int n = (nq_tiles - first_tile[c]) * p.group;
      if (it < n) {
        sg.chunk = c;
        sg.tile = first_tile[c] + it / p.group;
        sg.head_in_group = it % p.group;
        return sg;
      }
      it -= n;
    }
    return sg;
  };

  // ---- staging of Q, dO, LSE, Delta -----------------------------------------
  u32x4 qreg[Q_LOADS], oreg[Q_LOADS];
  float aux = 0.0f;   // LSE (threads 0..31) or Delta (threads 32..63)
  auto gload = [&](int it) {
    const StepGeom sg = decode(it);
    const int head = hk * p.group + sg.head_in_group;
    const int row0 = sg.tile * BQ;
    const __bf16 *qg = static_cast<const __bf16 *>(p.q) + b * p.q_sb + head * p.q_sh;
    const __bf16 *og = static_cast<const __bf16 *>(p.dout) + b * p.o_sb + head * p.o_sh;
#pragma unroll
    for (int i = 0; i < Q_LOADS; ++i) {
      const int idx = tid + NT * i;
      const int r = idx / NC, c = idx % NC;
      const bool ok = row0 + r < p.chunk_len;
      const int64_t lr = (int64_t)sg.chunk * p.chunk_len + row0 + r;
      qreg[i] = ok ? *reinterpret_cast<const u32x4 *>(qg + lr * p.q_ss + 8 * c) : u32x4{0u, 0u, 0u, 0u};
      oreg[i] = ok ? *reinterpret_cast<const u32x4 *>(og + lr * p.o_ss + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < 2 * BQ) {
      const int r = tid % BQ;
      const bool ok = row0 + r < p.chunk_len;
      const int64_t idx = ((int64_t)b * p.hq + head) * p.sq + (int64_t)sg.chunk * p.chunk_len + row0 + r;
      if (tid < BQ) {
        // exp2 argument offset: LSE * log2(e); +inf for rows with no visible
        // key or past the chunk end, which makes every P of the row 0.
        const float l = ok ? p.lse[idx] : -INFINITY;
        aux = (l == -INFINITY) ? INFINITY : l * kLog2e;
      } else {
        aux = ok ? p.delta[idx] : 0.0f;
      }
    }
  };
  auto swrite = [&](int st) {
#pragma unroll
    for (int i = 0; i < Q_LOADS; ++i) {
      const int idx = tid + NT * i;
      const int r = idx / NC, c = idx % NC;
      *reinterpret_cast<u32x4 *>(q_s(st) + TQ::chunk_off(r, c)) = qreg[i];
      *reinterpret_cast<u32x4 *>(do_s(st) + TQ::chunk_off(r, c)) = oreg[i];
    }
    if (tid < BQ) lse_s[st][tid] = aux;
    else if (tid < 2 * BQ) dl_s[st][tid - BQ] = aux;
  };

  f32x16 dv[DB], dk[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dv[db][i] = 0.0f;
      dk[db][i] = 0.0f;
    }
  const float c2 = p.scale_log2;

  if (total > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int st = it & 1;
    const StepGeom sg = decode(it);
    if (it + 1 < total) gload(it + 1);
    const __bf16 *qs = q_s(st);
    const __bf16 *os = do_s(st);
    const int64_t qpos0 = p.chunk_pos[sg.chunk] + sg.tile * BQ;  // global position of the tile's row 0

    // S = Q K^T and dP = dO V^T for 32 queries x this wavefront's 32 keys.
    f32x16 sacc, pacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sacc[i] = 0.0f;
      pacc[i] = 0.0f;
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const bf16x8 qa = *reinterpret_cast<const bf16x8 *>(qs + TQ::chunk_off(col, 2 * s + half));
      const bf16x8 oa = *reinterpret_cast<const bf16x8 *>(os + TQ::chunk_off(col, 2 * s + half));
      sacc = mfma32(qa, kf[s], sacc);
      pacc = mfma32(oa, vf[s], pacc);
    }
    // P and dS; register i holds query row 8*(i/4) + 4*half + i%4 of the tile.
    const bool need_mask = !key_ok || (p.causal && p.kv_pos0 + wkey0 + 31 > qpos0) ||
                           (sg.tile * BQ + BQ > p.chunk_len);
    bf16x8 pf[2], dsf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qr = 8 * (i >> 2) + 4 * half + (i & 3);
      float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i], c2, -lse_s[st][qr]));
      if (need_mask) {
        const bool hide = !key_ok || (p.causal && p.kv_pos0 + my_key > qpos0 + qr);
        if (hide) pv = 0.0f;
      }
      const float dsv = pv * (pacc[i] - dl_s[st][qr]);
      pf[i >> 3][i & 7] = (__bf16)pv;
      dsf[i >> 3][i & 7] = (__bf16)dsv;
    }
    // dV^T += dO^T P and dK^T += Q^T dS (d rows x this wavefront's keys).
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        dv[db] = mfma32(tr_operand<D>(os, 16 * k2, 32 * db, lane), pf[k2], dv[db]);
        dk[db] = mfma32(tr_operand<D>(qs, 16 * k2, 32 * db, lane), dsf[k2], dk[db]);
      }
    // dS^T -> LDS: row = key in tile, 4 consecutive queries per 8-byte store.
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = dsf[gq >> 1][4 * (gq & 1) + e];
      *reinterpret_cast<bf16x4 *>(ds_s + TS::elem_off(32 * wave + col, 8 * gq + 4 * half)) = w;
    }
    __syncthreads();
    // dQ^T (32 d x 32 queries) = K^T dS^T over this wavefront's keys.
    f32x16 qacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) qacc[i] = 0.0f;
#pragma unroll
    for (int s = 0; s < QK_STEPS; ++s)
      qacc = mfma32(ktf[s], tr_operand<BQ>(ds_s, dq_key0 + 16 * s, 0, lane), qacc);
    // Accumulate: lane = query column, registers = d rows.
    if (sg.tile * BQ + col < p.chunk_len) {
      const int head = hk * p.group + sg.head_in_group;
      const int64_t lr = (int64_t)sg.chunk * p.chunk_len + sg.tile * BQ + col;
      float *dst = p.dq_acc + (((int64_t)b * p.hq + head) * p.sq + lr) * D + 32 * dq_dblk + 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) atomicAdd(dst + 8 * (i >> 2) + (i & 3), qacc[i]);
    }
    if (it + 1 < total) swrite(st ^ 1);
    __syncthreads();
  }

  // ---- dK, dV of this wavefront's keys (zeros where no query sees them) ----
  if (!key_ok) return;
  float *dvp = p.dv + (((int64_t)b * p.hkv + hk) * p.skv + my_key) * D;
  float *dkp = p.dk + (((int64_t)b * p.hkv + hk) * p.skv + my_key) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * db + 8 * gq + 4 * half;
      f32x4 a, c;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[e] = dv[db][4 * gq + e];
        c[e] = dk[db][4 * gq + e] * p.scale;
      }
      *reinterpret_cast<f32x4 *>(dvp + d) = a;
      *reinterpret_cast<f32x4 *>(dkp + d) = c;
    }
}

template <int D>
int launch_d(const BwdParams &p, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)p.batch * p.hq * p.sq;
  if (rows > 0) {
    const int64_t blocks = (rows * 16 + 255) / 256;
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3(blocks), dim3(256), 0, s, p);
  }
  const int64_t kv_tiles = (p.skv + BK - 1) / BK;
  if (kv_tiles > 0) {
    hipLaunchKernelGGL(bwd_main_kernel<D>, dim3(kv_tiles * p.batch * p.hkv), dim3(NT), 0, s, p);
  }
  if (rows > 0) {
    const int64_t blocks = (rows * (D / 4) + 255) / 256;
    hipLaunchKernelGGL(bwd_dq_convert_kernel<D>, dim3(blocks), dim3(256), 0, s, p);
  }
  return (int)hipGetLastError();
}

}  // namespace

int launch_bwd_bf16(const BwdParams &p, int head_dim, void *stream) {
  if (head_dim == 128) return launch_d<128>(p, stream);
  if (head_dim == 64) return launch_d<64>(p, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace cpattn
