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
// Three launches, no atomics:
//  1. bwd_pre: Delta for every local row.
//  2. bwd_dkdv (key-stationary): one workgroup of 8 wavefronts per 128-key
//     tile of one KV head; it streams the 32-row query tiles -- of every
//     head of the GQA group and every chunk -- that can see one of its keys.
//     Wavefronts w and w+4 own the same 32 keys: the first keeps K rows and
//     dV^T (S = Q K^T, P, dV^T += dO^T P), the second, one tile behind, V
//     rows and dK^T (dP = dO V^T, dS = P o (dP - Delta) with P from LDS,
//     dK^T += Q^T dS). Query tiles wholly before the keys are never visited.
//  3. bwd_dq (query-stationary, scheduled like the forward): the transposed
//     tiles S^T = K Q^T and dP^T = V dO^T put the query in the lane, so P^T and
//     dS^T come from the saved LSE and Delta with per-lane scalars and feed
//     dQ^T += K^T dS^T straight from registers (K^T by transpose reads).
// Recomputing S and dP in the second kernel costs two extra contractions per
// visible tile but removes every cross-workgroup reduction of dQ.
#include <hip/hip_runtime.h>
#include <math.h>

#include "gfx950_common.h"
#include "plan.h"

namespace cpattn {
namespace {

constexpr int BK = kBwdBlockKV;   // keys per key-stationary workgroup
constexpr int BQ = kBwdBlockQ;    // query rows per step of that workgroup
constexpr int BN = kDqBlockKV;    // keys per tile of the query-stationary kernel
constexpr int NT = kDqWaves * 64;

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO o O), 16 lanes per row.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const BwdParams p) {
  constexpr int LPR = 16;
  constexpr int EPL = D / LPR;
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
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && part == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// 2. dK, dV (key-stationary)
// ---------------------------------------------------------------------------
// One workgroup of 8 wavefronts per 128-key tile of one KV head; wavefronts
// w and w+4 (which share a SIMD) own the same 32 keys, in two roles:
//  * P wavefronts (0..3) keep their keys' K rows and dV^T accumulators in
//    registers; for query tile t they compute S = Q K^T, P = exp(S - LSE)
//    (masked), add dV^T += dO^T P and hand P (bf16, in MFMA-operand layout)
//    to LDS;
//  * dS wavefronts (4..7) keep V rows and dK^T accumulators; one step behind,
//    they compute dP = dO V^T, dS = P o (dP - Delta) with P from LDS, and add
//    dK^T += Q^T dS.
// Each role thus has the same matrix work per step (two products of 8
// MFMAs) and half of the element-wise work, so the two wavefronts of a SIMD
// keep its matrix core busy in turn. dO^T and Q^T come from transpose reads
// of the staged tiles. Query tiles go through a 3-stage LDS ring (being
// loaded / used by P wavefronts / used by dS wavefronts), P through a 2-stage
// exchange; one barrier per step.
constexpr int kDkdvWaves = 8;
constexpr int kDkdvThreads = kDkdvWaves * 64;

template <int D>
__global__ void __launch_bounds__(kDkdvThreads, 1) bwd_dkdv_kernel(const BwdParams p) {
  constexpr int NT2 = kDkdvThreads;
  constexpr int NC = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int Q_CHUNKS = BQ * NC;           // 16-byte chunks per Q (and dO) tile
  constexpr int Q_LOADS = (Q_CHUNKS + NT2 - 1) / NT2;
  constexpr int QSTAGES = 3;
  using TQ = Tile<D>;

  __shared__ __attribute__((aligned(16))) __bf16 q_s[QSTAGES][BQ * D];
  __shared__ __attribute__((aligned(16))) __bf16 do_s[QSTAGES][BQ * D];
  __shared__ __attribute__((aligned(16))) float lse_s[QSTAGES][BQ];
  __shared__ __attribute__((aligned(16))) float dl_s[QSTAGES][BQ];
  // P exchange: [stage][key wavefront][k-step][lane] x 8 bf16
  __shared__ __attribute__((aligned(16))) bf16x8 xs[2][4][2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool prole = wave < 4;             // P role (else dS role)
  const int kw = wave & 3;                 // which 32 keys of the tile
  const int half = lane >> 5;
  const int col = lane & 31;

  const int groups = p.batch * p.hkv;
  const int g = blockIdx.x % groups;
  const int kt = blockIdx.x / groups;      // ascending: earliest keys (most work) first
  const int b = g / p.hkv;
  const int hk = g % p.hkv;
  const int key0 = kt * BK;
  const int wkey0 = key0 + 32 * kw;
  const int my_key = wkey0 + col;
  const bool key_ok = my_key < p.skv;
  const int64_t kv_lo = p.kv_pos0 + key0;

  // Query tiles this key tile meets: per chunk, tiles first_tile(c) ..
  // nq_tiles-1, each for every head of the GQA group. A cursor walks them in
  // that order (chunk, tile, head), one step per tile of one head.
  const int nq_tiles = (p.chunk_len + BQ - 1) / BQ;
  auto first_tile = [&](int c) {
    if (!p.causal) return 0;
    const int64_t rel = kv_lo - p.chunk_pos[c];
    return rel <= 0 ? 0 : (int)min<int64_t>(nq_tiles, rel / BQ);
  };
  int total = 0;
  for (int c = 0; c < p.n_q_chunks; ++c) total += (nq_tiles - first_tile(c)) * p.group;
  struct Cursor {
    int c, t, h;       // chunk, query tile in the chunk, head in the group
    int64_t cpos;      // global position of the chunk's first row
  };
  // Moves to the next chunk with a tile to visit (or past the last chunk).
  auto next_chunk = [&](Cursor &u) {
    int t0 = nq_tiles;
    while (t0 >= nq_tiles && ++u.c < p.n_q_chunks) t0 = first_tile(u.c);
    if (u.c < p.n_q_chunks) {
      u.t = t0;
      u.cpos = p.chunk_pos[u.c];
    }
  };
  auto advance = [&](Cursor &u) {
    if (++u.h == p.group) {
      u.h = 0;
      if (++u.t >= nq_tiles) next_chunk(u);
    }
  };
  Cursor c0{0, first_tile(0), 0, p.chunk_pos[0]};
  if (c0.t >= nq_tiles) next_chunk(c0);

  // Staging of query tiles (Q, dO and the rows' LSE and Delta): loaded into
  // registers two steps ahead and written to the LDS ring one step ahead of
  // use, through two register sets.
  int woff[Q_LOADS], grow[Q_LOADS], gcol[Q_LOADS];
#pragma unroll
  for (int i = 0; i < Q_LOADS; ++i) {
    const int idx = min(tid + NT2 * i, Q_CHUNKS - 1);
    grow[i] = idx / NC;
    gcol[i] = 8 * (idx % NC);
    woff[i] = TQ::chunk_off(grow[i], idx % NC);
  }
  struct Staged {
    u32x4 q[Q_LOADS], o[Q_LOADS];
    float aux;   // raw LSE (threads 0..31) or Delta (threads 32..63) of one row
    int ok;      // that row lies inside the chunk
  };
  // Wave-uniform copies of the two row-statistics pointers: selecting between
  // them per lane must not turn into a per-lane load of the pointer itself.
  const float *const lse_ptr = p.lse;
  const float *const delta_ptr = p.delta;
  const int rr = tid % BQ;
  // Loads only: anything computed from the loaded values waits until swrite,
  // so the loads stay in flight. Every thread loads (the statistics too), so
  // that all paths carry the same number of loads.
  // All addressing is a wave-uniform base (scalar registers) plus a 32-bit
  // lane offset; row strides are bounded on the host so that the offsets
  // within a tile fit in 31 bits.
  auto gload = [&](const Cursor &u, Staged &r) {
    const int head = hk * p.group + u.h;
    const int row0 = u.t * BQ;
    const int rows_left = p.chunk_len - 1 - row0;   // rows past the chunk end read its last row
    const int64_t lrow0 = (int64_t)u.c * p.chunk_len + row0;
    const char *qb = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.q) + b * p.q_sb +
                                                    head * p.q_sh + lrow0 * p.q_ss);
    const char *ob = reinterpret_cast<const char *>(static_cast<const __bf16 *>(p.dout) + b * p.o_sb +
                                                    head * p.o_sh + lrow0 * p.o_ss);
#pragma unroll
    for (int i = 0; i < Q_LOADS; ++i) {
      const int rw = min(grow[i], rows_left);
      r.q[i] = *reinterpret_cast<const u32x4 *>(qb + 2 * (rw * (int)p.q_ss + gcol[i]));
      r.o[i] = *reinterpret_cast<const u32x4 *>(ob + 2 * (rw * (int)p.o_ss + gcol[i]));
    }
    r.ok = rr <= rows_left;
    const int64_t sbase = ((int64_t)b * p.hq + head) * p.sq + lrow0;
    r.aux = (tid < BQ ? lse_ptr : delta_ptr)[sbase + min(rr, rows_left)];
  };
  auto swrite = [&](int st, const Staged &r) {
#pragma unroll
    for (int i = 0; i < Q_LOADS; ++i) {
      if (Q_CHUNKS % NT2 == 0 || tid + NT2 * i < Q_CHUNKS) {
        *reinterpret_cast<u32x4 *>(q_s[st] + woff[i]) = r.q[i];
        *reinterpret_cast<u32x4 *>(do_s[st] + woff[i]) = r.o[i];
      }
    }
    // LSE is stored as LSE*log2(e), +inf for rows with no visible key or past
    // the chunk end (P = 0); Delta is 0 past the chunk end.
    if (tid < BQ) lse_s[st][tid] = (!r.ok || r.aux == -INFINITY) ? INFINITY : r.aux * kLog2e;
    else if (tid < 2 * BQ) dl_s[st][tid - BQ] = r.ok ? r.aux : 0.0f;
  };
  // Load cursor: the step whose tile the next gload fetches. Past the last
  // step it stays on the last one (the loads are then repeated, unused).
  Cursor cl = c0;
  auto next_load = [&](int step_to_load) {
    if (step_to_load < total) advance(cl);
  };
  Staged sa, sb;   // register sets: step s is loaded into (s % 2 ? sb : sa)
  const float c2 = p.scale_log2;
  const bool wave_keys_ok = wkey0 + 31 < p.skv;

  // Prologue: step 0 staged, step 1 in registers.
  if (total > 0) {
    gload(cl, sa);
    swrite(0, sa);
    next_load(1);
    gload(cl, sb);
  }
  __syncthreads();

  // Step it: P wavefronts handle query tile it (it < total), dS wavefronts
  // tile it-1 (it >= 1); tile it+2 is loaded and tile it+1 written to the
  // ring meanwhile. The two roles run separate loops (so their register sets
  // do not add up) with the same barriers. Each loop is unrolled by two so
  // that the register sets alternate at compile time.
  // (Only called when total > 0, so the load cursor is always valid.)
  auto staging_begin = [&](int it, Staged &ld) {
    next_load(it + 2);
    gload(cl, ld);
  };
  auto staging_end = [&](int it, const Staged &wr) {
    if (it + 1 < total) swrite((it + 1) % QSTAGES, wr);
    __syncthreads();
  };
  TrOffsets<D> tro;   // Q^T and dO^T transpose reads (same tile layout)
  tro.init(lane);
  int qoff[KSTEPS];   // A-operand reads of Q (P role) or dO (dS role) rows
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) qoff[s] = TQ::chunk_off(col, 2 * s + half);
  // This lane's key row of K (P role) or V (dS role): the B operand.
  bf16x8 kvf[KSTEPS];
  {
    const __bf16 *src = static_cast<const __bf16 *>(prole ? p.k : p.v) + b * p.kv_sb + hk * p.kv_sh;
    const int64_t ro = (int64_t)min(my_key, p.skv - 1) * p.kv_ss + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) kvf[s] = *reinterpret_cast<const bf16x8 *>(src + ro + 16 * s);
    wait_vmem_all();
  }
  f32x16 acc[DB];     // dV^T (P role) or dK^T (dS role) of the 32 keys
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;

  if (prole) {
    Cursor cs = c0;   // the step being processed
    auto step_p = [&](int it, Staged &ld, const Staged &wr) {
      staging_begin(it, ld);
      if (it < total) {
        const int st = it % QSTAGES;
        const __bf16 *qs = q_s[st];
        const __bf16 *os = do_s[st];
        const int64_t qpos0 = cs.cpos + cs.t * BQ;
        // S = Q K^T: register i holds query row 8*(i/4) + 4*half + i%4.
        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
        bf16x8 qa[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) qa[s] = *reinterpret_cast<const bf16x8 *>(qs + qoff[s]);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) sacc = mfma32(qa[s], kvf[s], sacc);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, KSTEPS / 2, 0);
#pragma unroll
        for (int j = 0; j < KSTEPS / 2; ++j) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, KSTEPS / 2, 0);
        // dO^T operands of dV^T += dO^T P, read while S completes.
        bf16x8 ao[2][DB];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < DB; ++db) ao[k2][db] = tro.read(os, 16 * k2, db);
        // The lane's key is visible to rows >= its first visible row.
        const bool need_mask = !wave_keys_ok || (p.causal && p.kv_pos0 + wkey0 + 31 > qpos0);
        int t = -BQ;
        if (need_mask) {
          int rel = -1;
          if (p.causal) {
            const int64_t r = p.kv_pos0 + my_key - qpos0;
            rel = (int)(r < -1 ? -1 : (r > BQ ? BQ : r));
          }
          t = key_ok ? rel - 4 * half : BQ;
        }
        float pv[16];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lse_s[st][8 * gq + 4 * half]);
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[4 * gq + e] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * gq + e], c2, -l4[e]));
        }
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = (8 * (i >> 2) + (i & 3) < t) ? 0.0f : pv[i];
        }
        bf16x8 pf[2];
        to_bf16_operands(pv, pf);
        const int xst = it & 1;
        xs[xst][kw][0][lane] = pf[0];
        xs[xst][kw][1][lane] = pf[1];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] = mfma32(ao[k2][db], pf[k2], acc[db]);
        advance(cs);
      }
      staging_end(it, wr);
    };
    if (total > 0) {
      for (int it = 0; it <= total; it += 2) {
        step_p(it, sa, sb);
        if (it + 1 <= total) step_p(it + 1, sb, sa);
      }
    }
  } else {
    auto step_ds = [&](int it, Staged &ld, const Staged &wr) {
      staging_begin(it, ld);
      if (it >= 1) {
        const int st = (it + QSTAGES - 1) % QSTAGES;
        const int xst = (it - 1) & 1;
        const __bf16 *qs = q_s[st];
        const __bf16 *os = do_s[st];
        // dP = dO V^T (same layout as S).
        f32x16 pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) pacc[i] = 0.0f;
        bf16x8 oa[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) oa[s] = *reinterpret_cast<const bf16x8 *>(os + qoff[s]);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) pacc = mfma32(oa[s], kvf[s], pacc);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, KSTEPS / 2, 0);
#pragma unroll
        for (int j = 0; j < KSTEPS / 2; ++j) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, KSTEPS / 2, 0);
        // Q^T operands of dK^T += Q^T dS and P, read while dP completes.
        bf16x8 aq[2][DB], pk[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          pk[k2] = xs[xst][kw][k2][lane];
#pragma unroll
          for (int db = 0; db < DB; ++db) aq[k2][db] = tro.read(qs, 16 * k2, db);
        }
        float dsv[16];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&dl_s[st][8 * gq + 4 * half]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * gq + e;
            dsv[i] = (float)pk[i >> 3][i & 7] * (pacc[i] - d4[e]);
          }
        }
        bf16x8 dsf[2];
        to_bf16_operands(dsv, dsf);
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] = mfma32(aq[k2][db], dsf[k2], acc[db]);
      }
      staging_end(it, wr);
    };
    if (total > 0) {
      for (int it = 0; it <= total; it += 2) {
        step_ds(it, sa, sb);
        if (it + 1 <= total) step_ds(it + 1, sb, sa);
      }
    }
  }

  if (!key_ok) return;
  float *dst = (prole ? p.dv : p.dk) + (((int64_t)b * p.hkv + hk) * p.skv + my_key) * D;
  const float mul = prole ? 1.0f : p.scale;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * db + 8 * gq + 4 * half;
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = acc[db][4 * gq + e] * mul;
      *reinterpret_cast<f32x4 *>(dst + d) = a;
    }
}

// ---------------------------------------------------------------------------
// 3. dQ (query-stationary; work items and K/V staging as in the forward)
// ---------------------------------------------------------------------------
template <int D, int RB>
__global__ void __launch_bounds__(NT, 2) bwd_dq_kernel(const BwdParams p) {
  constexpr int HPW = kDqWaves / RB;
  constexpr int BM = kDqWaveRows * RB;
  constexpr int NC = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int LOADS = BN * NC / NT;
  using T = Tile<D>;

  __shared__ __attribute__((aligned(16))) __bf16 smem[2][2][BN * D];  // [stage][K,V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int col = lane & 31;

  const int bid = blockIdx.x;
  const int pack = bid % p.n_head_packs;
  const int rank = bid / p.n_head_packs;
  const int ci = rank / p.tiles_per_chunk;
  const int tile = p.tiles_per_chunk - 1 - (rank % p.tiles_per_chunk);
  const int chunk = p.lpt_chunk_idx[ci];
  const int64_t chunk_pos = p.lpt_chunk_pos[ci];
  const int packs_per_batch = p.hq / HPW;
  const int b = pack / packs_per_batch;
  const int head0 = (pack % packs_per_batch) * HPW;
  const int hkv = head0 / p.group;
  const int item_row0 = tile * BM;
  const int item_rows = min(BM, p.chunk_len - item_row0);
  const int64_t item_qhi = chunk_pos + item_row0 + item_rows - 1;

  const int head = head0 + wave / RB;
  const int wrow0 = (wave % RB) * kDqWaveRows;
  const int wrows = max(0, min(kDqWaveRows, item_rows - wrow0));
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

  // Q and dO rows of this lane's query: B operands of S^T and dP^T. Lanes past
  // the item's last row read its first row and get LSE = +inf (P = 0).
  bf16x8 qf[KSTEPS], gf[KSTEPS];
  float lse2 = INFINITY, delta = 0.0f;
  {
    const int load_row = qvalid ? local_row : chunk * p.chunk_len + item_row0;
    const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + head * p.q_sh +
                       (int64_t)load_row * p.q_ss + 8 * half;
    const __bf16 *gp = static_cast<const __bf16 *>(p.dout) + b * p.o_sb + head * p.o_sh +
                       (int64_t)load_row * p.o_ss + 8 * half;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
      gf[s] = *reinterpret_cast<const bf16x8 *>(gp + 16 * s);
    }
    if (qvalid) {
      const int64_t row = ((int64_t)b * p.hq + head) * p.sq + local_row;
      const float l = p.lse[row];
      lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;
      delta = p.delta[row];
    }
    wait_vmem_all();
  }

  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + hkv * p.kv_sh;
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + hkv * p.kv_sh;
  // Per-lane addressing, computed once.
  int koff[KSTEPS];                     // A-operand reads of K and V rows
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = T::chunk_off(col, 2 * s + half);
  TrOffsets<D> tro;                     // K^T transpose reads
  tro.init(lane);
  // Staging: thread tid moves chunk (tid % NC) of rows tid / NC + i * RSTEP.
  // Row steps of RSTEP (a multiple of 16) keep the swizzle, so every load's
  // LDS and global offsets are the first one's plus a constant.
  constexpr int RSTEP = NT / NC;
  static_assert(RSTEP % 16 == 0, "row step must preserve the swizzle");
  const int srow = tid / NC, scol = 8 * (tid % NC);
  const int woff0 = T::chunk_off(srow, tid % NC);
  const uint32_t goff0 = (uint32_t)(((int64_t)srow * p.kv_ss + scol) * 2);
  const int64_t tile_stride = (int64_t)BN * p.kv_ss;
  const int64_t rstep_bytes = (int64_t)RSTEP * p.kv_ss * 2;
  u32x4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int kt) {
    if (kt * BN + BN <= p.skv) {
      // Full tile: scalar tile base plus a 32-bit per-lane byte offset.
      const char *kt_base = reinterpret_cast<const char *>(kbase + (int64_t)kt * tile_stride);
      const char *vt_base = reinterpret_cast<const char *>(vbase + (int64_t)kt * tile_stride);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        kreg[i] = *reinterpret_cast<const u32x4 *>(kt_base + i * rstep_bytes + goff0);
        vreg[i] = *reinterpret_cast<const u32x4 *>(vt_base + i * rstep_bytes + goff0);
      }
    } else {
      // Ragged last tile: rows past the end read the last row (always masked).
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int64_t o = (int64_t)min(kt * BN + srow + i * RSTEP, p.skv - 1) * p.kv_ss + scol;
        kreg[i] = *reinterpret_cast<const u32x4 *>(kbase + o);
        vreg[i] = *reinterpret_cast<const u32x4 *>(vbase + o);
      }
    }
  };
  auto swrite = [&](int stage) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      *reinterpret_cast<u32x4 *>(&smem[stage][0][woff0 + i * RSTEP * D]) = kreg[i];
      *reinterpret_cast<u32x4 *>(&smem[stage][1][woff0 + i * RSTEP * D]) = vreg[i];
    }
  };

  f32x16 qacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) qacc[db][i] = 0.0f;
  const float c2 = p.scale_log2;

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
      const bool need_mask = (kt * BN + BN > p.skv) || (p.causal && tile_plo + BN - 1 > wave_qlo);
      int t = BN;   // key kb*32 + 8*(i/4) + 4*half + i%4 visible iff (that - 4*half) <= t
      if (need_mask) {
        int lim = p.skv - 1 - kt * BN;
        if (p.causal) {
          const int64_t rel = qpos - tile_plo;
          lim = min(lim, (int)(rel < -1 ? -1 : (rel > BN ? BN : rel)));
        }
        t = lim - 4 * half;
      }
      // One 32-key block at a time keeps only one S^T/dP^T pair live.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sacc[i] = 0.0f;
          pacc[i] = 0.0f;
        }
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const int off = koff[s] + kb * 32 * D;
          sacc = mfma32(*reinterpret_cast<const bf16x8 *>(ks + off), qf[s], sacc);
          pacc = mfma32(*reinterpret_cast<const bf16x8 *>(vs + off), gf[s], pacc);
        }
        bf16x8 dsf[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i], c2, -lse2));
          if (need_mask) pv = (kb * 32 + 8 * (i >> 2) + (i & 3) > t) ? 0.0f : pv;
          dsf[i >> 3][i & 7] = (__bf16)(pv * (pacc[i] - delta));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2)
            qacc[db] = mfma32(tro.read(ks, 32 * kb + 16 * k2, db), dsf[k2], qacc[db]);
      }
    }
    if (kt + 1 < ntiles) swrite(st ^ 1);
    __syncthreads();
  }

  if (!qvalid) return;
  __bf16 *dst = static_cast<__bf16 *>(p.dq) + b * p.o_sb + head * p.o_sh + (int64_t)local_row * p.o_ss;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(qacc[db][4 * gq + e] * p.scale);
      *reinterpret_cast<bf16x4 *>(dst + 32 * db + 8 * gq + 4 * half) = o4;
    }
}

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
  if (int e = mark(1)) return e;
  const int64_t kv_tiles = (p.skv + BK - 1) / BK;
  if (kv_tiles > 0) {
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3(kv_tiles * p.batch * p.hkv), dim3(kDkdvThreads), 0, s, p);
  }
  if (int e = mark(2)) return e;
  const int64_t items = (int64_t)p.n_head_packs * p.n_q_chunks * p.tiles_per_chunk;
  if (rows > 0 && items > 0) {
    const int rb = kDqWaves / p.heads_per_item;
    switch (rb) {
      case 2: hipLaunchKernelGGL((bwd_dq_kernel<D, 2>), dim3(items), dim3(NT), 0, s, p); break;
      case 4: hipLaunchKernelGGL((bwd_dq_kernel<D, 4>), dim3(items), dim3(NT), 0, s, p); break;
      case 8: hipLaunchKernelGGL((bwd_dq_kernel<D, 8>), dim3(items), dim3(NT), 0, s, p); break;
      default: return (int)hipErrorInvalidValue;
    }
  }
  if (int e = mark(3)) return e;
  return (int)hipGetLastError();
}

}  // namespace

int launch_bwd_bf16(const BwdParams &p, int head_dim, void *stream, void *const *events) {
  if (head_dim == 128) return launch_d<128>(p, stream, events);
  if (head_dim == 64) return launch_d<64>(p, stream, events);
  return (int)hipErrorInvalidValue;
}

}  // namespace cpattn
