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
//    heads that read the same KV head (GQA); K/V tiles of 32 keys pass through
//    a 3-stage LDS ring once per workgroup and are read by every head;
//  * each wavefront owns 32 query rows of one head and computes the transposed
//    score tile S^T = K Q^T (keys x queries) with v_mfma_f32_32x32x16_bf16, so
//    that a lane holds one query column: the row max and sum of the online
//    softmax are lane-local plus one permlane32 swap between the two halves of
//    the wavefront;
//  * the probabilities P^T, converted to bf16 in registers, are the B operand
//    of O^T += V^T P^T without any shuffle: the contraction index (keys) is
//    permuted identically in both operands, and V^T is read from the
//    row-major V tile with the gfx950 LDS transpose read ds_read_b64_tr_b16;
//  * software pipeline: while the vector ALU exponentiates tile j, the matrix
//    cores already compute S^T of tile j+1 (the two are interleaved
//    instruction by instruction), and the global loads of tile j+2 are in
//    flight;
//  * KV tiles wholly after the work item's last query are never visited; only
//    tiles crossing the causal diagonal (or the ragged end of K/V) are masked;
//    the running max is only moved (and O rescaled) when a new score exceeds
//    it by more than 2^8, which keeps every exp2 argument <= 8.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "gfx950_common.h"
#include "plan.h"

namespace cpattn {
namespace {

constexpr int BN = kFwdBlockKV;          // keys per tile (32)
constexpr int NT = kFwdWaves * 64;
constexpr int STAGES = 3;
constexpr float kRescaleSlack = 8.0f;    // log2 units

// sched_group_barrier masks
constexpr int kSchedMfma = 0x008;
constexpr int kSchedValu = 0x002;
constexpr int kSchedDsRead = 0x100;

template <int D, int RB>
__global__ void __launch_bounds__(NT, 2) fwd_bf16_kernel(const FwdParams p) {
  constexpr int HPW = kFwdWaves / RB;  // heads per work item
  constexpr int BM = kWaveRows * RB;   // query rows per work item
  constexpr int NC = D / 8;
  constexpr int KSTEPS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BN * D;
  constexpr int CHUNKS = BN * NC;      // 16-byte chunks per K (or V) tile
  constexpr int LOADS = (CHUNKS + NT - 1) / NT;
  static_assert(BN == 32 && (CHUNKS % NT == 0 || LOADS == 1), "tile shape");
  using T = Tile<D>;

  __shared__ __attribute__((aligned(16))) __bf16 smem[STAGES][2][TILE];  // [stage][K,V]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
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
  const int64_t wave_qlo = chunk_pos + item_row0 + min(wrow0, item_rows - 1);
  const bool qvalid = col < wrows;
  // Lanes past the last row of the item act as its last row (never stored).
  const int qrow = min(wrow0 + col, item_rows - 1);
  const int64_t qpos = chunk_pos + item_row0 + qrow;
  const int local_row = chunk * p.chunk_len + item_row0 + qrow;

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
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8 *>(qp + 16 * s);
    wait_vmem_all();
  }

  // ---- per-lane addressing, computed once ----------------------------------
  int koff[KSTEPS];                        // K-fragment reads: row col, chunk 2s+half
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = T::chunk_off(col, 2 * s + half);
  int troff[2][DB];                        // V^T transpose reads (k-step 1 adds 16 rows)
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      troff[u][db] = T::elem_off(8 * u + 4 * half + ((lane & 15) >> 2),
                                 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + hkv * p.kv_sh;
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + hkv * p.kv_sh;
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
  // Two register sets: tile t is loaded into set t % 2 two steps before it is
  // written to the LDS ring, which gives each load two steps of latency cover.
  u32x4 kreg[2][LOADS], vreg[2][LOADS];
  // With fewer chunks than threads (D = 64) only the first CHUNKS threads stage.
  const bool stager = (CHUNKS % NT == 0) || tid < CHUNKS;
  auto gload = [&](int kt, auto set_tag) {
    constexpr int SET = decltype(set_tag)::value;
    if (!stager) return;
    if (kt * BN + BN <= p.skv) {
      // Full tile: scalar tile base plus a 32-bit per-lane byte offset.
      const char *kt_base = reinterpret_cast<const char *>(kbase + (int64_t)kt * tile_stride);
      const char *vt_base = reinterpret_cast<const char *>(vbase + (int64_t)kt * tile_stride);
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        kreg[SET][i] = *reinterpret_cast<const u32x4 *>(kt_base + i * rstep_bytes + goff0);
        vreg[SET][i] = *reinterpret_cast<const u32x4 *>(vt_base + i * rstep_bytes + goff0);
      }
    } else {
      // Ragged last tile: rows past the end read the last row (always masked).
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int64_t o = (int64_t)min(kt * BN + srow + i * RSTEP, p.skv - 1) * p.kv_ss + scol;
        kreg[SET][i] = *reinterpret_cast<const u32x4 *>(kbase + o);
        vreg[SET][i] = *reinterpret_cast<const u32x4 *>(vbase + o);
      }
    }
  };
  auto swrite = [&](int stage, auto set_tag) {
    constexpr int SET = decltype(set_tag)::value;
    if (!stager) return;
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      *reinterpret_cast<u32x4 *>(&smem[stage][0][woff0 + i * RSTEP * D]) = kreg[SET][i];
      *reinterpret_cast<u32x4 *>(&smem[stage][1][woff0 + i * RSTEP * D]) = vreg[SET][i];
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.0f;
  float m_run = -INFINITY;  // running max of scale*log2(e)*s (may lag the true max)
  float l_part = 0.0f;      // this lane's partial row sum (its half of the keys)
  const float c = p.scale_log2;

  // ---- prologue: tiles 0 and 1 staged, S^T of tile 0 ----------------------
  f32x16 sacc;
#pragma unroll
  for (int i = 0; i < 16; ++i) sacc[i] = 0.0f;
  if (ntiles > 0) {
    gload(0, I0{});
    swrite(0, I0{});
    if (ntiles > 1) {
      gload(1, I1{});
      swrite(1, I1{});
    }
    gload(min(2, ntiles - 1), I0{});
  }
  __syncthreads();
  if (ntiles > 0) {
    const __bf16 *ks = smem[0][0];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      sacc = mfma32(*reinterpret_cast<const bf16x8 *>(ks + koff[s]), qf[s], sacc);
  }

  // One step of the pipeline on tile kt held in stage ST (kt % 3 == ST);
  // PAR = kt % 2 selects the register set of tile kt + 2 (written to the ring
  // at the end of this step); tile kt + 3 is loaded into the other set.
  auto step = [&](auto st_tag, auto par_tag, int kt) {
    constexpr int ST = decltype(st_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    constexpr int NEXT = (ST + 1) % STAGES;
    constexpr int FREE = (ST + 2) % STAGES;
    // Unconditional (past the end it re-reads the last tile): every path then
    // has the same number of loads in flight, so the wait before the ring
    // write below covers only the older set.
    gload(min(kt + 3, ntiles - 1), std::integral_constant<int, 1 - PAR>{});
    const int64_t tile_plo = p.kv_pos0 + (int64_t)kt * BN;

    // Mask (diagonal or ragged tiles only): key 8*(i/4) + 4*half + i%4 of the
    // tile is visible iff it is <= lim.
    const bool need_mask = (kt * BN + BN > p.skv) || (p.causal && tile_plo + BN - 1 > wave_qlo);
    if (need_mask) {
      int lim = p.skv - 1 - kt * BN;
      if (p.causal) {
        const int64_t rel = qpos - tile_plo;
        lim = min(lim, (int)(rel < -1 ? -1 : (rel > BN ? BN : rel)));
      }
      const int t = lim - 4 * half;
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = (8 * (i >> 2) + (i & 3) > t) ? -INFINITY : sacc[i];
    }
    // Online softmax bookkeeping for tile kt.
    float mx = sacc[0];
#pragma unroll
    for (int i = 1; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sacc[i]), sacc[i + 1]);   // v_max3 chain
    mx = fmaxf(mx, sacc[15]);
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

    // S^T of tile kt+1 on the matrix cores, interleaved with exp2 of tile kt.
    // (After the last tile this reads a stale stage; the result is unused.)
    f32x16 snext;
#pragma unroll
    for (int i = 0; i < 16; ++i) snext[i] = 0.0f;
    const __bf16 *ksn = smem[NEXT][0];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      snext = mfma32(*reinterpret_cast<const bf16x8 *>(ksn + koff[s]), qf[s], snext);
    // The row sum uses the unrounded fp32 probabilities (summing the bf16
    // values instead costs up to ~2^-9 relative error in short rows).
    bf16x8 pf[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, mneg));
      l_part += pv;
      pf[i >> 3][i & 7] = (__bf16)pv;
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 6, 0);
    }

    // O^T += V^T P^T for tile kt.
    const __bf16 *vs = smem[ST][1];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vs + troff[0][db] + 16 * D * k2));
        const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vs + troff[1][db] + 16 * D * k2));
        const i16x8 av = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = mfma32(__builtin_bit_cast(bf16x8, av), pf[k2], oacc[db]);
      }
    if (kt + 2 < ntiles) swrite(FREE, par_tag);
    __syncthreads();
    sacc = snext;
  };

  for (int kt = 0; kt < ntiles; kt += 2 * STAGES) {
    step(I0{}, I0{}, kt);
    if (kt + 1 < ntiles) step(I1{}, I1{}, kt + 1);
    if (kt + 2 < ntiles) step(I2{}, I0{}, kt + 2);
    if (kt + 3 < ntiles) step(I0{}, I1{}, kt + 3);
    if (kt + 4 < ntiles) step(I1{}, I0{}, kt + 4);
    if (kt + 5 < ntiles) step(I2{}, I1{}, kt + 5);
  }

  // ---- epilogue -------------------------------------------------------------
  if (!qvalid) return;
  const float l = pair_sum(l_part);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
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

template <int D>
int launch_d(const FwdParams &p, void *stream) {
  const int64_t grid = fwd_grid_size(p);
  if (grid == 0) return 0;
  const int rb = kFwdWaves / p.heads_per_item;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (rb) {
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<D, 2>), dim3(grid), dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((fwd_bf16_kernel<D, 4>), dim3(grid), dim3(NT), 0, s, p); break;
    case 8: hipLaunchKernelGGL((fwd_bf16_kernel<D, 8>), dim3(grid), dim3(NT), 0, s, p); break;
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
