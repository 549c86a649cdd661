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
//  1. bwd_pre: -Delta (and LSE in log2 units) for every local row.
//  2. bwd_dkdv (key-stationary): one workgroup of 8 wavefronts per 128-key
//     tile of one KV head; it streams the 64-row query tiles -- of every
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
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>

#include "gfx950_common.h"
#include "plan.h"

namespace cpattn {
namespace {

constexpr int BK = kBwdBlockKV;   // keys per key-stationary workgroup
constexpr int BQ = kBwdBlockQ;    // query rows per step of that workgroup
constexpr int BN = kDqBlockKV;    // keys per tile of the query-stationary kernel
constexpr int NT = kDqWaves * 64;

// ---------------------------------------------------------------------------
// 1. Delta = rowsum(dO o O), 16 lanes per row, stored negated (the matrix
//    kernels start their dP accumulators from -Delta, so the products come
//    out as dP - Delta); also LSE in log2 units.
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
    const int64_t off = b * p.o_sb + h * p.o_sh + (int64_t)r * p.o_ss + (r / p.chunk_len) * p.o_cadj + part * EPL;
    const __bf16 *o = static_cast<const __bf16 *>(p.out) + off;
    const __bf16 *g = static_cast<const __bf16 *>(p.dout) + off;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (row < rows && part == 0) {
    p.delta[row] = -acc;
    const float l = p.lse[row];
    p.lse2[row] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// 1b. A user mask as bits (see BwdParams::mask_bits): one thread per 4
//     consecutive keys and 64-row query tile, consecutive threads on
//     consecutive keys (the mask's values of one row, and the table's words,
//     are contiguous in keys). A thread reads each row's 4 bytes (an
//     additive mask: 4 floats) as one 32-bit (16-byte) word; a group that
//     runs past the last key reads them one by one.
// ---------------------------------------------------------------------------
constexpr int kMaskBitsKeys = kMaskBitsBlockKeys / 256;   // keys per thread of the column-bit pass

__device__ __forceinline__ int col_bit(int r) { return 16 * ((r >> 2) & 3) + 4 * (r >> 4) + (r & 3); }

__global__ void __launch_bounds__(256) bwd_mask_bits_kernel(const BwdParams p) {
  constexpr int KPB = kMaskBitsBlockKeys;
  static_assert(kMaskBitsKeys == 4, "one 32-bit word of bytes per row");
  const int nkb = (p.skv + KPB - 1) / KPB;
  const int ntiles = p.n_q_chunks * p.mb_tpc;
  const int64_t blk = blockIdx.x;
  const int key = (int)(blk % nkb) * KPB + kMaskBitsKeys * (int)threadIdx.x;
  const int n = (int)((blk / nkb) % ntiles);
  const int bh = (int)(blk / ((int64_t)nkb * ntiles));
  if (key >= p.skv) return;
  const int c = n / p.mb_tpc, t = n % p.mb_tpc;
  const int rows = min(kBwdBlockQ, p.chunk_len - t * kBwdBlockQ);
  const int bm = bh / p.mb_heads, hm = bh % p.mb_heads;
  const int nk = min(kMaskBitsKeys, p.skv - key);
  uint32_t lo[kMaskBitsKeys] = {}, hi[kMaskBitsKeys] = {};
  if (p.mask_add) {
    // Additive: a key is kept unless its value is at most kMaskHide; a row's
    // 4 values are one 16-byte read (rows start on 16-byte boundaries). The
    // row-bit pass runs first: once it has marked the mask as holding other
    // values than 0 and hiding ones, the table is not used.
    if (__atomic_load_n(p.mask_flag, __ATOMIC_RELAXED) != 0) return;
    const float *colf = reinterpret_cast<const float *>(
        p.mask + bm * p.m_sb + hm * p.m_sh + ((int64_t)c * p.chunk_len + (int64_t)t * kBwdBlockQ) * p.m_ss) + key;
    for (int r = 0; r < rows; ++r) {
      const float *rowp = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(colf) + (int64_t)r * p.m_ss);
      float v[kMaskBitsKeys];
      if (nk == kMaskBitsKeys) {
        const float4 q = *reinterpret_cast<const float4 *>(rowp);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
      } else {
#pragma unroll
        for (int i = 0; i < kMaskBitsKeys; ++i) v[i] = i < nk ? rowp[i] : kMaskHide;
      }
      const int b = col_bit(r);
#pragma unroll
      for (int i = 0; i < kMaskBitsKeys; ++i) {
        const uint32_t x = !(v[i] <= kMaskHide) ? 1u : 0u;
        if (b < 32) lo[i] |= x << b;
        else hi[i] |= x << (b - 32);
      }
    }
    uint64_t *dst = p.mask_bits + ((int64_t)bh * ntiles + n) * p.skv + key;
#pragma unroll
    for (int i = 0; i < kMaskBitsKeys; ++i)
      if (i < nk) dst[i] = ((uint64_t)hi[i] << 32) | lo[i];
    return;
  }
  const uint8_t *col = p.mask + bm * p.m_sb + hm * p.m_sh +
                       ((int64_t)c * p.chunk_len + (int64_t)t * kBwdBlockQ) * p.m_ss + key;
  // Bit of row r in the word of key i: from the top bit of byte i of v
  // (set iff the byte is nonzero).
  auto add_row = [&](uint32_t v, int r) {
    const uint32_t nz = (((v & 0x7f7f7f7fu) + 0x7f7f7f7fu) | v) & 0x80808080u;
    const int b = col_bit(r);
#pragma unroll
    for (int i = 0; i < kMaskBitsKeys; ++i) {
      const uint32_t x = (nz >> (8 * i + 7)) & 1u;
      if (b < 32) lo[i] |= x << b;
      else hi[i] |= x << (b - 32);
    }
  };
  if (nk == kMaskBitsKeys && rows == kBwdBlockQ) {
#pragma unroll
    for (int r0 = 0; r0 < kBwdBlockQ; r0 += 16) {
      uint32_t v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = *reinterpret_cast<const uint32_t *>(col + (int64_t)(r0 + r) * p.m_ss);
#pragma unroll
      for (int r = 0; r < 16; ++r) add_row(v[r], r0 + r);
    }
  } else {
    for (int r = 0; r < rows; ++r) {
      uint32_t v = 0;
      for (int i = 0; i < nk; ++i) v |= (uint32_t)col[(int64_t)r * p.m_ss + i] << (8 * i);
      const uint32_t nz = (((v & 0x7f7f7f7fu) + 0x7f7f7f7fu) | v) & 0x80808080u;
      const int b = col_bit(r);
      for (int i = 0; i < kMaskBitsKeys; ++i) {
        const uint64_t x = (nz >> (8 * i + 7)) & 1u;
        if (b < 32) lo[i] |= (uint32_t)(x << b);
        else hi[i] |= (uint32_t)(x << (b - 32));
      }
    }
  }
  uint64_t *dst = p.mask_bits + ((int64_t)bh * ntiles + n) * p.skv + key;
#pragma unroll
  for (int i = 0; i < kMaskBitsKeys; ++i)
    if (i < nk) dst[i] = ((uint64_t)hi[i] << 32) | lo[i];
}

// ---------------------------------------------------------------------------
// 2. dK, dV (key-stationary)
// ---------------------------------------------------------------------------
// One workgroup of 8 wavefronts per 128-key tile of one KV head; wavefronts
// w and w+4 (which share a SIMD) own the same 32 keys (two 16-key blocks, the
// columns of v_mfma_f32_16x16x32_bf16 products), in two roles:
//  * P wavefronts (0..3) keep their keys' K rows and dV^T accumulators in
//    registers; for the 64-row query tile of step t they compute
//    P(t) = exp2(S(t) * scale*log2(e) - LSE*log2(e)) (masked), hand it to
//    LDS and add dV^T += dO(t)^T P(t); S(t+1) = Q(t+1) K^T is computed in the
//    same step, under the exponentials;
//  * dS wavefronts (4..7) keep V rows and dK^T accumulators; in step t they
//    add dK^T += Q(t-2)^T dS(t-2), compute dP(t) = dO(t) V^T and, under it,
//    dS(t-1) = P(t-1) o (dP(t-1) - Delta) with P(t-1) from LDS.
// Each role issues 64 matrix instructions per step: the P role's vector work
// runs under its first 32, the dS role's under its last 32, so the two
// wavefronts of a SIMD take turns with the vector ALU. Every Q, dO, Q^T or
// dO^T fragment read from LDS feeds both key blocks. Every step is written
// as slots of one matrix instruction, one operand read a few operands ahead
// and a share of the vector work, with scheduling fences between slots. Query
// tiles (Q, dO and the rows' LSE*log2(e) and Delta) are loaded straight from
// global memory into LDS rings; query tiles wholly before the keys are never
// visited; one barrier per step. Only the P wavefronts issue the loads.
constexpr int kDkdvWaves = 8;
constexpr int kDkdvThreads = kDkdvWaves * 64;

// Zero dK/dV rows outside the key tiles [kt0, kt1) the key-stationary kernel
// computes (keys no local query can see), as workgroup `w` of `nw` doing this:
// 16-byte stores of both, grid-stride over every (batch, KV head)'s rows.
template <int D>
__device__ __forceinline__ void zero_unseen_keys(const BwdParams &p, int w, int nw, int tid, int nthreads) {
  constexpr int VPR = D / 4;                        // float4 per row
  const int64_t front = (int64_t)p.kt0 * BK;        // rows [0, front) and [back, skv)
  const int64_t back = min((int64_t)p.kt1 * BK, (int64_t)p.skv);
  const int64_t per_head = (front + (p.skv - back)) * VPR;
  const int64_t n = per_head * p.batch * p.hkv;
  const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t i = (int64_t)w * nthreads + tid; i < n; i += (int64_t)nw * nthreads) {
    const int64_t g = i / per_head, e = i % per_head;
    const int64_t r = e / VPR;
    const int64_t row = r < front ? r : back + (r - front);
    const int64_t off = (g * p.skv + row) * D + (e % VPR) * 4;
    *reinterpret_cast<f32x4 *>(p.dk + off) = z;
    *reinterpret_cast<f32x4 *>(p.dv + off) = z;
  }
}

// KMODE 0: plain; 1: packed-sequence boundaries (keys are visible only to
// rows of their own sequence); 2: a user attention mask.
template <int D, int KMODE>
__global__ void __launch_bounds__(kDkdvThreads, 2) bwd_dkdv_kernel(const BwdParams p) {
  constexpr bool DOCS = KMODE == 1;
  constexpr bool UMASK = KMODE == 2;
  constexpr int NW = kDkdvWaves;
  constexpr int NC = D / 8;
  constexpr int KSTEPS = D / 32;              // k-steps of S, dP (over D)
  constexpr int DB = D / 16;                  // 16-row blocks of dV^T, dK^T
  constexpr int KN = 2;                       // 16-key blocks per wavefront
  constexpr int QT = BQ;                      // query rows per step (64)
  constexpr int RB = QT / 16;                 // 16-row blocks per step
  constexpr int QSTEPS = QT / 32;             // k-steps over rows (dV, dK)
  constexpr int QTILE = QT * D;               // elements of a Q or dO tile
  constexpr int QSTG = 5;                     // Q ring (with LSE2, Delta): tiles t-2 .. t+2
  constexpr int OSTG = 2;                     // dO ring: tiles t, t+1
  constexpr int NXOP = KN * QSTEPS;           // P operands per lane per step
  constexpr int XPER = NXOP * 8;              // P values per lane per step
  // LDS layout (bytes)
  constexpr int Q_OFF = 0;
  constexpr int O_OFF = Q_OFF + QSTG * QTILE * 2;
  constexpr int X_OFF = O_OFF + OSTG * QTILE * 2;                    // [2][4 waves][NXOP][64 lanes] bf16x8
  constexpr int L_OFF = X_OFF + 2 * 4 * 64 * XPER * 2;               // [QSTG][QT] LSE*log2(e)
  constexpr int DL_OFF = L_OFF + QSTG * QT * 4;                      // [QSTG][QT] Delta
  constexpr int MB_OFF = DL_OFF + QSTG * QT * 4;                     // [QSTG][BK] mask bit words
  constexpr int LDS_BYTES = MB_OFF + (UMASK ? QSTG * BK * 8 : 0);
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(QT == 64 && XPER == 32, "step shape");
  using T = Tile16<D>;
  // A user mask's bit table stands for it when it is boolean, or additive
  // with only 0 and hiding values (the row-bit pass says which; a share
  // without keys has no table, and no flag, and reads no mask).
  bool use_bits = false;
  if constexpr (UMASK) use_bits = !p.mask_add || (p.mask_flag != nullptr && *p.mask_flag == 0);

  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool prole = wave < 4;             // P role (else dS role)
  const int kw = wave & 3;                 // which 32 keys of the tile
  const int grp = lane >> 4;               // operand k-slice / accumulator row quarter
  const int col = lane & 15;               // operand row / accumulator column (key)

  const int groups = p.batch * p.hkv;
  // Workgroups past the key tiles' zero dK/dV of the keys no local row sees
  // (they run last, in the tail of the grid).
  const int n_compute = (p.kt1 - p.kt0) * p.kv_parts * groups;
  if ((int)blockIdx.x >= n_compute) {
    zero_unseen_keys<D>(p, (int)blockIdx.x - n_compute, (int)gridDim.x - n_compute, threadIdx.x, kDkdvThreads);
    return;
  }
  const int g = blockIdx.x % groups;
  const int unit = blockIdx.x / groups;          // key tile, then part: earliest keys (most work) first
  const int part = unit % p.kv_parts;
  const int kt = p.kt0 + unit / p.kv_parts;
  const int b = g / p.hkv;
  const int hk = g % p.hkv;
  const int key0 = kt * BK;
  const int wkey0 = key0 + 32 * kw;
  // This lane's key in each 16-key block of the wavefront's 32.
  int my_key[KN];
  bool key_ok[KN];
#pragma unroll
  for (int kn = 0; kn < KN; ++kn) {
    my_key[kn] = wkey0 + 16 * kn + col;
    key_ok[kn] = my_key[kn] < p.skv;
  }
  const bool wave_keys_ok = wkey0 + 31 < p.skv;
  // Global position of storage row 0 as seen from this tile's KV chunk (a
  // tile never straddles two chunks): key j sits at kv_base + j.
  const int kc = key0 / p.kv.len;
  const int64_t kv_base = p.kv.pos[kc] - (int64_t)kc * p.kv.len;
  const int64_t kv_lo = kv_base + key0;
  // Packed sequences: a key is seen only by rows before the end of its
  // sequence (the first bound > its position; none: +inf), per lane key
  // (de_key), for the wave's first key (the earliest end among the wave's
  // keys: de_wave) and the tile's last key (the latest: de_tile). The scan over
  // the bounds is wave-uniform.
  int64_t de_key[KN], de_wave = INT64_MAX, de_tile = INT64_MAX;
  if constexpr (DOCS) {
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) de_key[kn] = INT64_MAX;
    const int64_t wave_k0 = kv_base + wkey0, tile_k1 = kv_base + key0 + BK - 1;
    for (int i = p.docs.n - 1; i >= 0; --i) {
      const int64_t bd = p.docs.pos[i];
#pragma unroll
      for (int kn = 0; kn < KN; ++kn) de_key[kn] = bd > kv_base + my_key[kn] ? bd : de_key[kn];
      if (bd > wave_k0) de_wave = bd;
      if (bd > tile_k1) de_tile = bd;
    }
  }

  // Query tiles this key tile meets: per chunk, tiles first_tile(c) ..
  // end_tile(c)-1, each for every head of the GQA group. A cursor walks them
  // in that order (chunk, tile, head), one step per tile of one head.
  const int nq_tiles = (p.chunk_len + QT - 1) / QT;
  auto first_tile = [&](int c) {
    if (!p.causal) return 0;
    const int64_t rel = kv_lo - p.chunk_pos[c];
    return rel <= 0 ? 0 : (int)min<int64_t>(nq_tiles, rel / QT);
  };
  auto end_tile = [&](int c) {
    if constexpr (DOCS) {
      if (de_tile == INT64_MAX) return nq_tiles;
      const int64_t rel = de_tile - p.chunk_pos[c];   // rows before it may see the tile
      const int e = rel <= 0 ? 0 : (int)min<int64_t>(nq_tiles, (rel + QT - 1) / QT);
      return max(e, first_tile(c));
    } else {
      return nq_tiles;
    }
  };
  int all_steps = 0;
  for (int c = 0; c < p.n_q_chunks; ++c) all_steps += (end_tile(c) - first_tile(c)) * p.group;
  // This workgroup's part of the tile's steps (all of them unless the tile is
  // split over kv_parts workgroups).
  const int s_begin = (int)((int64_t)all_steps * part / p.kv_parts);
  const int total = (int)((int64_t)all_steps * (part + 1) / p.kv_parts) - s_begin;
  // A cursor also carries the element offsets of its step's first row from
  // the group's first head: `off` in the tensor it loads (Q or dO), `soff` in
  // the per-row statistics. Steps move them by additions; only a new chunk
  // recomputes them.
  struct Cursor {
    int c, t, h;       // chunk, query tile in the chunk, head in the group
    int64_t cpos;      // global position of the chunk's first row
    int64_t off, soff;
  };
  struct Walk {
    int64_t sh, ss, cadj;   // head, row and chunk strides (elements)
  };
  const Walk wq{p.q_sh, p.q_ss, p.q_cadj}, wo{p.o_sh, p.o_ss, p.o_cadj}, wst{p.sq, 1, 0};
  auto offset = [&](const Walk &w, int c, int t, int h) {
    return (int64_t)h * w.sh + ((int64_t)c * p.chunk_len + (int64_t)t * QT) * w.ss + (int64_t)c * w.cadj;
  };
  auto next_chunk = [&](Cursor &u) {
    int t0 = 0, t1 = 0;
    while (t0 >= t1 && ++u.c < p.n_q_chunks) {
      t0 = first_tile(u.c);
      t1 = end_tile(u.c);
    }
    if (u.c < p.n_q_chunks) {
      u.t = t0;
      u.cpos = p.chunk_pos[u.c];
    }
  };
  // One step on: the next head of the group, then the next query tile, then
  // the next chunk with tiles to visit. `w` walks `off`; `stats`: also soff.
  auto advance = [&](Cursor &u, const Walk &w, bool stats) {
    if (++u.h == p.group) {
      u.h = 0;
      if (++u.t >= end_tile(u.c)) {
        next_chunk(u);
        u.off = offset(w, u.c, u.t, 0);
        if (stats) u.soff = offset(wst, u.c, u.t, 0);
      } else {
        u.off += (int64_t)QT * w.ss - (int64_t)(p.group - 1) * w.sh;
        if (stats) u.soff += QT - (int64_t)(p.group - 1) * p.sq;
      }
    } else {
      u.off += w.sh;
      if (stats) u.soff += p.sq;
    }
  };
  // The cursor at step s_begin: skip whole chunks, then tiles of G steps.
  Cursor c0{0, first_tile(0), 0, p.chunk_pos[0], 0, 0};
  {
    int rem = s_begin, c = 0;
    for (; c < p.n_q_chunks; ++c) {
      const int n = (end_tile(c) - first_tile(c)) * p.group;
      if (rem < n) break;
      rem -= n;
    }
    if (c < p.n_q_chunks) c0 = Cursor{c, first_tile(c) + rem / p.group, rem % p.group, p.chunk_pos[c], 0, 0};
    else if (c0.t >= end_tile(0)) next_chunk(c0);   // no step left (total == 0)
  }

  // ---- staging: global -> LDS directly (see the forward kernel) -------------
  // Only the P wavefronts stage (the dS wavefronts carry the longer chain of
  // each step). One instruction of a wavefront moves RPI rows of a Q or dO
  // tile; lane l lands at LDS offset 16*l of them and fetches the chunk that
  // the row's swizzle puts there. P wavefront kw's instruction i covers rows
  // (i*SW + kw)*RPI ...; the row modulo 16 does not depend on i.
  constexpr int SW = 4;                       // staging wavefronts
  constexpr int RPI = 64 / NC;
  constexpr int INSTS = QT / (SW * RPI);
  static_assert(INSTS >= 1 && (SW * RPI) % 16 == 0, "staging shape");
  const int srow = kw * RPI + lane / NC;
  const int scol = 8 * ((lane % NC) ^ T::swz(srow));
  auto dma16 = [](uint32_t m0, uint32_t voff, const void *sbase) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
  };
  auto dma4 = [](uint32_t m0, uint32_t voff, const void *sbase) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
  };
  // Per-lane byte offsets of the first instruction's rows in full tiles (Q
  // rows q_ss apart, dO rows o_ss); instruction i adds a wave-uniform step.
  const uint32_t goq = (uint32_t)(((int64_t)srow * p.q_ss + scol) * 2);
  const uint32_t goo = (uint32_t)(((int64_t)srow * p.o_ss + scol) * 2);
  const __bf16 *qhead = static_cast<const __bf16 *>(p.q) + b * p.q_sb + (int64_t)hk * p.group * p.q_sh;
  const __bf16 *ohead = static_cast<const __bf16 *>(p.dout) + b * p.o_sb + (int64_t)hk * p.group * p.o_sh;
  // LDS destination of this wavefront's first row of a tile at byte offset
  // 0, kept in one scalar register (otherwise the compiler keeps one
  // destination per instruction and stage, beyond the scalar registers).
  uint32_t m0w = lds0 + 2 * kw * RPI * D;
  asm volatile("" : "+s"(m0w));
  // Rows of step u's tile of Q (is_q) or dO into LDS at byte offset dst;
  // rows past the chunk end read its last row.
  auto dma_tile = [&](const Cursor &u, bool is_q, uint32_t dst) {
    const int rows_left = p.chunk_len - 1 - u.t * QT;
    const int64_t ss = is_q ? p.q_ss : p.o_ss;
    const __bf16 *tbase = (is_q ? qhead : ohead) + u.off;
    uint32_t m0 = m0w + dst;
    asm volatile("" : "+s"(m0));
    if (rows_left >= QT - 1) {
#pragma unroll
      for (int i = 0; i < INSTS; ++i)
        dma16(m0 + 2 * i * SW * RPI * D, (is_q ? goq : goo) + (uint32_t)(i * SW * RPI * ss * 2), tbase);
    } else {
#pragma unroll
      for (int i = 0; i < INSTS; ++i) {
        const int r = min(srow + i * SW * RPI, rows_left);
        dma16(m0 + 2 * i * SW * RPI * D, (uint32_t)((r * ss + scol) * 2), tbase);
      }
    }
  };
  // LSE*log2(e) (wave 0) and Delta (wave 1) of step u's rows.
  const float *stat0 = (wave == 0 ? p.lse2 : p.delta) + ((int64_t)b * p.hq + (int64_t)hk * p.group) * p.sq;
  auto dma_stats = [&](const Cursor &u, int stage) {
    if (wave >= 2) return;
    const int rows_left = p.chunk_len - 1 - u.t * QT;
    const uint32_t dst = lds0 + (wave == 0 ? L_OFF : DL_OFF) + stage * QT * 4;
    dma4(dst, (uint32_t)(min(lane, rows_left) * 4), stat0 + u.soff);
  };
  Cursor cq = c0;   // step whose Q tile the next Q load fetches
  cq.off = offset(wq, c0.c, c0.t, c0.h);
  cq.soff = offset(wst, c0.c, c0.t, c0.h);
  Cursor co = c0;   // step whose dO tile the next dO load fetches
  co.off = offset(wo, c0.c, c0.t, c0.h);
  // A boolean user mask's bit-table words of step u's query tile for this
  // P wavefront's 32 keys (two lanes per word; keys past the end read the
  // last key's word), beside the statistics.
  auto dma_bits = [&](const Cursor &u, int stage) {
    if constexpr (UMASK) {
      if (!use_bits) return;
      const int bhm = (p.mb_batches > 1 ? b : 0) * p.mb_heads + (p.mb_heads > 1 ? hk * p.group + u.h : 0);
      const int64_t tile = (int64_t)bhm * p.n_q_chunks * p.mb_tpc + u.c * p.mb_tpc + u.t;
      const int k0 = min(wkey0, p.skv - 1);
      const uint32_t voff = (uint32_t)((min(wkey0 + (lane >> 1), p.skv - 1) - k0) * 8 + 4 * (lane & 1));
      dma4(lds0 + MB_OFF + stage * BK * 8 + kw * 32 * 8, voff, p.mask_bits + tile * p.skv + k0);
    }
  };
  auto load_q = [&](int s) {   // Q tile (and statistics) of step s = cq's
    const int st = s % QSTG;
    dma_tile(cq, true, Q_OFF + st * QTILE * 2);
    dma_stats(cq, st);
    dma_bits(cq, st);
    advance(cq, wq, true);
  };
  auto load_o = [&](int s) {   // dO tile of step s = co's
    dma_tile(co, false, O_OFF + (s % OSTG) * QTILE * 2);
    advance(co, wo, false);
  };

  // ---- per-lane LDS addressing ----------------------------------------------
  // Row reads (A operands of S = Q K^T and dP = dO V^T): row col of a 16-row
  // block, chunk 4s+grp; transpose reads (A operands of dV^T = dO^T P and
  // dK^T = Q^T dS): rows 4grp .. 4grp+3 and 16 + 4grp .. of a 32-row k-step,
  // column 16db + col, as in the forward's V^T. Row blocks, k-steps and the
  // second transpose read only add constants (the swizzle repeats every 16
  // rows).
  const uint32_t rbase = lds0 + (prole ? Q_OFF : O_OFF);
  const uint32_t tbase = lds0 + (prole ? O_OFF : Q_OFF);
  uint32_t raddr[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) raddr[s] = rbase + 2 * T::chunk_off(col, 4 * s + grp);
  uint32_t taddr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) taddr[db] = tbase + 2 * T::elem_off(4 * grp + (col >> 2), 16 * db + 4 * (lane & 3));
  auto lds_b128 = [](uint32_t addr) -> bf16x8 {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>((uintptr_t)addr);
  };
  auto lds_f4 = [](uint32_t addr) -> f32x4 {
    return *reinterpret_cast<const __attribute__((address_space(3))) f32x4 *>((uintptr_t)addr);
  };
  auto lds_tr2 = [](uint32_t addr) -> bf16x8 {
    const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)addr);
    const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)(addr + 2 * 16 * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // P exchange: operand x (key block x / QSTEPS, row k-step x % QSTEPS) of
  // lane l of key group kw at stage s, 16 bytes per lane. Lane l takes slot
  // l ^ 4*(l/32): each 16-lane pass of a 16-byte access (lanes sharing bits
  // 2 and 4) then covers all 64 banks.
  // The exchange and the statistics lie beyond the reach of an instruction
  // offset (16 bits) from LDS 0: their bases are made opaque registers that
  // hold the region start, so the per-read displacements fold into offsets.
  uint32_t xaddr = lds0 + X_OFF + (kw * NXOP * 64 + (lane ^ ((lane >> 5) << 2))) * 16;
  asm volatile("" : "+v"(xaddr));
  constexpr uint32_t XSTAGE = 4 * 64 * XPER * 2;
  constexpr uint32_t XOP = 64 * 16;   // bytes between a lane's operands
  // This lane's rows 4grp .. 4grp+3 of the statistics of stage 0 (LSE*log2(e)
  // at lstat, -Delta at dstat).
  uint32_t lstat = lds0 + L_OFF + 16 * grp, dstat = lds0 + DL_OFF + 16 * grp;
  asm volatile("" : "+v"(lstat), "+v"(dstat));
  // This P wavefront's mask bit words of stage 0 (boolean user mask).
  const uint32_t mbase = lds0 + MB_OFF + kw * 32 * 8;

  // This lane's key rows of K (P role) or V (dS role): the B operands.
  bf16x8 kvf[KN][KSTEPS];
  {
    const int64_t adj = (p.kv.store_lg < 31 ? (int64_t)key0 >> p.kv.store_lg : (int64_t)kc) * p.kv.cadj;
    const __bf16 *src = static_cast<const __bf16 *>(prole ? p.k : p.v) + b * p.kv_sb + hk * p.kv_sh + adj;
#pragma unroll
    for (int kn = 0; kn < KN; ++kn) {
      const int64_t ro = (int64_t)min(my_key[kn], p.skv - 1) * p.kv_ss + 8 * grp;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) kvf[kn][s] = *reinterpret_cast<const bf16x8 *>(src + ro + 32 * s);
    }
    wait_vmem_all();
  }
  f32x4 acc[DB][KN];     // dV^T (P role) or dK^T (dS role) of the 32 keys
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kn = 0; kn < KN; ++kn)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[db][kn][i] = 0.0f;
  const float c2 = p.scale_log2;
  constexpr int AHEAD = 2;
  constexpr int NBUF = AHEAD + 1;
  constexpr int NOA = RB * KSTEPS;      // S or dP operands per step (each used by KN products)
  constexpr int NOB = QSTEPS * DB;      // dV or dK operands per step
  constexpr int NSA = KN * NOA;         // S or dP products per step
  constexpr int NSB = KN * NOB;         // dV or dK products per step
  constexpr int NPAIR = RB * KN * 2;    // pairs of P (or dS) values per lane per step
  constexpr int SPP = NSA / NPAIR;      // slots per pair
  static_assert(NSA == SPP * NPAIR, "whole slots per pair");

  // Prologue: Q of steps 0 and 1 (when there is a step 1), dO of step 0.
  // Every load is of a step that exists: the cursors never run past the last.
  if (prole && total > 0) {
    load_q(0);
    if (total > 1) load_q(1);
    load_o(0);
  }
  wait_vmem_all();
  __syncthreads();
  // Loads issued at the start of step it: Q of step it+2, dO of step it+1.
  auto staging = [&](int it) {
    if (it + 2 < total) load_q(it + 2);
    if (it + 1 < total) load_o(it + 1);
  };
  auto finish = [&]() {
    wait_vmem_all();   // this wave's rows of the tiles loaded in this step are in LDS
    __syncthreads();
  };

  if (prole) {
    // Scores ([row block][key block]) alternate between two register sets by
    // step parity.
    f32x4 sbuf[2][RB][KN];
    Cursor cs = c0;   // the step being processed
    if (total > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int kn = 0; kn < KN; ++kn)
#pragma unroll
          for (int i = 0; i < 4; ++i) sbuf[0][rb][kn][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const bf16x8 a = lds_b128(raddr[s] + 2 * 16 * rb * D);
#pragma unroll
          for (int kn = 0; kn < KN; ++kn) sbuf[0][rb][kn] = mfma16(a, kvf[kn][s], sbuf[0][rb][kn]);
        }
      }
    }
    auto step_p = [&](auto par_tag, int it) {
      constexpr int PAR = decltype(par_tag)::value;
      staging(it);
      if (it < total) {
        f32x4 (&sacc)[RB][KN] = sbuf[PAR];
        f32x4 (&snext)[RB][KN] = sbuf[1 - PAR];
        uint32_t qnext = 2 * ((it + 1) % QSTG) * QTILE;         // Q stage of step it+1
        asm volatile("" : "+s"(qnext));   // one scalar: each address below takes one add
        constexpr uint32_t ocur = 2 * PAR * QTILE;              // dO stage of step it
        const int st = it % QSTG;
        // LSE*log2(e) of this lane's rows: row block rb holds rows
        // 16rb + 4grp .. +3, read one block ahead.
        const uint32_t lbase = lstat + 4 * st * QT;
        f32x4 lg[2];
        lg[0] = lds_f4(lbase);
        // Mask: row r of the tile sees this lane's key of block kn iff
        // lo[kn] <= r <= hi.
        const int64_t qpos0 = cs.cpos + cs.t * QT;
        const int rows_left = p.chunk_len - 1 - cs.t * QT;
        bool need_mask = !wave_keys_ok || rows_left < QT - 1 ||
                         (p.causal && kv_base + wkey0 + 31 > qpos0);
        if constexpr (DOCS) need_mask = need_mask || qpos0 + QT - 1 >= de_wave;
        // (A user mask is applied to every step, the range mask only where needed.)
        if (need_mask || UMASK) {
#pragma unroll
          for (int kn = 0; kn < KN; ++kn) {
            if (!UMASK || need_mask) {
              int hi = rows_left;
              if constexpr (DOCS) {
                // ... and rows before the end of the key's sequence.
                const int64_t e = de_key[kn] - qpos0 - 1;
                hi = (int)min<int64_t>(hi, e < -1 ? -1 : e);
              }
              const int hi_g = hi - 4 * grp;
              int lo = 0;
              if (p.causal) {
                const int64_t r = kv_base + my_key[kn] - qpos0;
                lo = (int)(r < 0 ? 0 : (r > QT ? QT : r));
              }
              if (!key_ok[kn]) lo = QT;
              const int lo_g = lo - 4 * grp;
#pragma unroll
              for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int r = 16 * rb + i;
                  sacc[rb][kn][i] = (r < lo_g || r > hi_g) ? -INFINITY : sacc[rb][kn][i];
                }
            }
            if constexpr (UMASK) {
              if (!use_bits) {
                // ... plus an additive user mask with biases (else the
                // column bits below): rows 16rb + 4grp + i of the
                // query tile (of head cs.h of the group), this lane's key, in
                // the raw score's units (at or below kMaskHide: hidden; a
                // hidden score stays -inf). The sixteen reads are issued
                // before any is used. A key past the end reads the last key
                // and, in a partial tile, a row past the chunk end its last
                // row: both are hidden above. The reads go through a buffer
                // descriptor of the tile's mask rows: a full tile's row offsets
                // (16rb + i) * m_ss are wave-uniform scalar offsets and each
                // lane adds one 32-bit offset (the host bounds 64 mask rows
                // below 2^31 bytes).
                const uint8_t *mb = p.mask + b * p.m_sb + (int64_t)(hk * p.group + cs.h) * p.m_sh +
                                    ((int64_t)cs.c * p.chunk_len + cs.t * QT) * p.m_ss;
                const __amdgpu_buffer_rsrc_t mrs =
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(mb), 0, 0x7fffffff, kBufferFlags);
                const uint32_t koff = 4u * (uint32_t)min(my_key[kn], p.skv - 1);
                const int mss = (int)p.m_ss;
                auto ld = [&](uint32_t off, int soff) {
                  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(mrs, off, soff, 0));
                };
                float a[RB][4];
                if (rows_left >= QT - 1) {
                  const uint32_t lane_off = (uint32_t)(4 * grp * mss) + koff;
#pragma unroll
                  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) a[rb][i] = ld(lane_off, (16 * rb + i) * mss);
                } else {
#pragma unroll
                  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                      const int r = min(16 * rb + 4 * grp + i, rows_left);
                      a[rb][i] = ld((uint32_t)(r * mss) + koff, 0);
                    }
                }
                const float inv = 1.0f / p.scale;
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    const float sv = sacc[rb][kn][i];
                    sacc[rb][kn][i] = (a[rb][i] <= kMaskHide || sv == -INFINITY) ? -INFINITY : fmaf(a[rb][i], inv, sv);
                  }
              } else {
                // ... and allowed by a boolean user mask: one word of its bit
                // table per key and query tile, bit 16grp + 4rb + i for row
                // 16rb + 4grp + i (a key past the end has the last key's:
                // hidden above), staged in LDS with the step's statistics;
                // this lane reads its 16 bits.
                const uint32_t w16 = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t *>(
                    (uintptr_t)(mbase + st * BK * 8 + (16 * kn + col) * 8 + 2 * grp));
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                  for (int i = 0; i < 4; ++i)
                    sacc[rb][kn][i] = keep_if_bit(sacc[rb][kn][i], w16, 4 * rb + i);
              }
            }
          }
        }
        bf16x8 pcur[KN][QSTEPS];
        bf16x8 opnd[NBUF];
        // Bases of this step's Q reads, made opaque so that the row-block
        // offsets stay instruction immediates.
        uint32_t rbq[KSTEPS];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          rbq[s] = raddr[s] + qnext;
          asm volatile("" : "+v"(rbq[s]));
        }
        // Half A: S(it+1) (operand o: k-step o / RB of row block o % RB, so
        // that products accumulating into one block are 2*RB slots apart)
        // under P(it).
        auto read_a = [&](auto o_tag) -> bf16x8 {
          constexpr int o = decltype(o_tag)::value, rb = o % RB, s = o / RB;
          return lds_b128(rbq[s] + 2 * 16 * rb * D);
        };
        static_for<AHEAD>([&](auto o) { opnd[decltype(o)::value] = read_a(o); });
        float xp[NPAIR][2];   // a pair's probabilities between its two slots
        static_for<NSA>([&](auto t_tag) {
          constexpr int t = decltype(t_tag)::value, o = t / KN, kn = t % KN, rb = o % RB, s = o / RB;
          if constexpr (kn == 0 && o + AHEAD < NOA) opnd[(o + AHEAD) % NBUF] = read_a(IC<o + AHEAD>{});
          if constexpr (s == 0) {
            f32x4 z;
#pragma unroll
            for (int i = 0; i < 4; ++i) z[i] = 0.0f;
            snext[rb][kn] = mfma16(opnd[o % NBUF], kvf[kn][s], z);
          } else {
            snext[rb][kn] = mfma16(opnd[o % NBUF], kvf[kn][s], snext[rb][kn]);
          }
          // The slot's vector work is issued after its matrix instruction.
          __builtin_amdgcn_sched_barrier(0);
          // Pair u (row block u / 4, key block (u / 2) % 2, elements 2(u%2),
          // 2(u%2)+1): exponentials in slot SPP*u, bf16 conversion two slots
          // later (at D = 128 the next slot with an operand read; the last
          // pair's in the last slot); it lands in elements 4(rb%2) + i of the
          // key block's P operand of k-step rb/2 (the row order of the dO^T
          // reads).
          static_for<NPAIR>([&](auto u_tag) {
            constexpr int u = decltype(u_tag)::value;
            constexpr int rq = u / 4, kq = (u / 2) % 2, i = 2 * (u % 2);
            if constexpr (SPP * u == t) {
              if constexpr (u % 4 == 0 && rq + 1 < RB) lg[(rq + 1) % 2] = lds_f4(lbase + 4 * 16 * (rq + 1));
              xp[u][0] = fmaf(sacc[rq][kq][i], c2, -lg[rq % 2][i]);
              xp[u][1] = fmaf(sacc[rq][kq][i + 1], c2, -lg[rq % 2][i + 1]);
              xp[u][0] = __builtin_amdgcn_exp2f(xp[u][0]);
              xp[u][1] = __builtin_amdgcn_exp2f(xp[u][1]);
            }
            if constexpr ((SPP * u + 2 < NSA ? SPP * u + 2 : NSA - 1) == t) {
              const bf16x2 t2 = __builtin_convertvector((f32x2){xp[u][0], xp[u][1]}, bf16x2);
              pcur[kq][rq >> 1][4 * (rq & 1) + i] = t2[0];
              pcur[kq][rq >> 1][4 * (rq & 1) + i + 1] = t2[1];
            }
          });
          __builtin_amdgcn_sched_barrier(0);
        });
        // P(it) to the dS wavefront of these keys.
#pragma unroll
        for (int kn = 0; kn < KN; ++kn)
#pragma unroll
          for (int ps = 0; ps < QSTEPS; ++ps)
            *reinterpret_cast<__attribute__((address_space(3))) bf16x8 *>(
                (uintptr_t)(xaddr + PAR * XSTAGE + XOP * (kn * QSTEPS + ps))) = pcur[kn][ps];
        // Half B: dV^T += dO(it)^T P(it) (operand o: k-step o / DB, block o % DB).
        auto read_b = [&](auto o_tag) -> bf16x8 {
          constexpr int o = decltype(o_tag)::value, ps = o / DB, db = o % DB;
          return lds_tr2(taddr[db] + ocur + 2 * 32 * D * ps);
        };
        static_for<AHEAD>([&](auto o) { opnd[decltype(o)::value] = read_b(o); });
        static_for<NSB>([&](auto t_tag) {
          constexpr int t = decltype(t_tag)::value, o = t / KN, kn = t % KN, ps = o / DB, db = o % DB;
          if constexpr (kn == 0 && o + AHEAD < NOB) opnd[(o + AHEAD) % NBUF] = read_b(IC<o + AHEAD>{});
          acc[db][kn] = mfma16(opnd[o % NBUF], pcur[kn][ps], acc[db][kn]);
          __builtin_amdgcn_sched_barrier(0);
        });
        advance(cs, wq, false);
      }
      finish();
    };
    for (int it = 0; it <= total + 1; it += 2) {
      step_p(IC<0>{}, it);
      if (it + 1 <= total + 1) step_p(IC<1>{}, it + 1);
    }
  } else {
    // dP alternates between two register sets by step parity; dS(it-1),
    // made in the second half of step it, feeds the first half of step it+1,
    // where it meets Q(it-1), still held by the 5-stage Q ring.
    f32x4 pbuf[2][RB][KN];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int kn = 0; kn < KN; ++kn)
#pragma unroll
          for (int i = 0; i < 4; ++i) pbuf[q][rb][kn][i] = 0.0f;
    bf16x8 dsf[KN][QSTEPS];
#pragma unroll
    for (int kn = 0; kn < KN; ++kn)
#pragma unroll
      for (int ps = 0; ps < QSTEPS; ++ps)
#pragma unroll
        for (int e = 0; e < 8; ++e) dsf[kn][ps][e] = (__bf16)0.0f;
    auto step_ds = [&](auto par_tag, int it) {
      constexpr int PAR = decltype(par_tag)::value;
      bf16x8 opnd[NBUF];
      // Half A: dK^T += Q(it-2)^T dS(it-2).
      if (it >= 2) {
        uint32_t qold = 2 * ((it - 2) % QSTG) * QTILE;
        asm volatile("" : "+s"(qold));    // one scalar: each address below takes one add
        // Bases of this step's Q^T reads (opaque: see the P role).
        uint32_t tb[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          tb[db] = taddr[db] + qold;
          asm volatile("" : "+v"(tb[db]));
        }
        auto read_a = [&](auto o_tag) -> bf16x8 {
          constexpr int o = decltype(o_tag)::value, ps = o / DB, db = o % DB;
          return lds_tr2(tb[db] + 2 * 32 * D * ps);
        };
        static_for<AHEAD>([&](auto o) { opnd[decltype(o)::value] = read_a(o); });
        static_for<NSB>([&](auto t_tag) {
          constexpr int t = decltype(t_tag)::value, o = t / KN, kn = t % KN, ps = o / DB, db = o % DB;
          if constexpr (kn == 0 && o + AHEAD < NOB) opnd[(o + AHEAD) % NBUF] = read_a(IC<o + AHEAD>{});
          acc[db][kn] = mfma16(opnd[o % NBUF], dsf[kn][ps], acc[db][kn]);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // Half B: dP(it) - Delta = dO(it) V^T - Delta under
      // dS(it-1) = P(it-1) o (dP(it-1) - Delta).
      if (it <= total) {
        f32x4 (&pnext)[RB][KN] = pbuf[PAR];
        f32x4 (&pprev)[RB][KN] = pbuf[1 - PAR];
        constexpr uint32_t ocur = 2 * PAR * QTILE;              // dO stage of step it
        const int st = it % QSTG;                               // statistics of step it
        bf16x8 pk[KN][QSTEPS];
#pragma unroll
        for (int kn = 0; kn < KN; ++kn)
#pragma unroll
          for (int ps = 0; ps < QSTEPS; ++ps)
            pk[kn][ps] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>(
                (uintptr_t)(xaddr + (1 - PAR) * XSTAGE + XOP * (kn * QSTEPS + ps)));
        // -Delta of this step's rows (row block rb: rows 16rb + 4grp .. +3) is
        // the starting value of dP(it), which so comes out as dP - Delta.
        f32x4 nd[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) nd[rb] = lds_f4(dstat + 4 * st * QT + 4 * 16 * rb);
        auto read_b = [&](auto o_tag) -> bf16x8 {
          constexpr int o = decltype(o_tag)::value, rb = o % RB, s = o / RB;
          return lds_b128(raddr[s] + ocur + 2 * 16 * rb * D);
        };
        static_for<AHEAD>([&](auto o) { opnd[decltype(o)::value] = read_b(o); });
        float xd[NPAIR][2];   // a pair's dS values between its two slots
        static_for<NSA>([&](auto t_tag) {
          constexpr int t = decltype(t_tag)::value, o = t / KN, kn = t % KN, rb = o % RB, s = o / RB;
          if constexpr (kn == 0 && o + AHEAD < NOA) opnd[(o + AHEAD) % NBUF] = read_b(IC<o + AHEAD>{});
          if constexpr (s == 0) {
            pnext[rb][kn] = mfma16(opnd[o % NBUF], kvf[kn][s], nd[rb]);
          } else {
            pnext[rb][kn] = mfma16(opnd[o % NBUF], kvf[kn][s], pnext[rb][kn]);
          }
          __builtin_amdgcn_sched_barrier(0);
          // Pair u as in the P role: products in slot SPP*u, conversion two
          // slots later.
          static_for<NPAIR>([&](auto u_tag) {
            constexpr int u = decltype(u_tag)::value;
            constexpr int rq = u / 4, kq = (u / 2) % 2, i = 2 * (u % 2), ps = rq >> 1, e = 4 * (rq & 1) + i;
            if constexpr (SPP * u == t) {
              const float p0 = (float)pk[kq][ps][e], p1 = (float)pk[kq][ps][e + 1];
              xd[u][0] = p0 * pprev[rq][kq][i];
              xd[u][1] = p1 * pprev[rq][kq][i + 1];
            }
            if constexpr ((SPP * u + 2 < NSA ? SPP * u + 2 : NSA - 1) == t) {
              const bf16x2 t2 = __builtin_convertvector((f32x2){xd[u][0], xd[u][1]}, bf16x2);
              dsf[kq][ps][e] = t2[0];
              dsf[kq][ps][e + 1] = t2[1];
            }
          });
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      finish();
    };
    for (int it = 0; it <= total + 1; it += 2) {
      step_ds(IC<0>{}, it);
      if (it + 1 <= total + 1) step_ds(IC<1>{}, it + 1);
    }
  }

  // Part 0 writes dK/dV; the other parts of a split tile write partials for
  // the reduction kernel ([part-1][tile][group][dk, dv][key in tile][D]).
  float *dst = part == 0
                   ? (prole ? p.dv : p.dk) + ((int64_t)b * p.hkv + hk) * p.skv * D
                   : p.kv_partial +
                         ((((int64_t)(part - 1) * (p.kt1 - p.kt0) + (kt - p.kt0)) * groups + g) * 2 + (prole ? 1 : 0)) *
                             BK * D - (int64_t)key0 * D;
  const float mul = prole ? 1.0f : p.scale;
#pragma unroll
  for (int kn = 0; kn < KN; ++kn) {
    if (!key_ok[kn]) continue;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = acc[db][kn][e] * mul;
      *reinterpret_cast<f32x4 *>(dst + (int64_t)my_key[kn] * D + 16 * db + 4 * grp) = a;
    }
  }
}

// Adds the partial dK/dV of the split key tiles' parts 1.. into dK/dV: one
// float4 of dK and of dV per thread; grid (key tiles x groups, BK*D/4/256).
template <int D>
__global__ void __launch_bounds__(256) bwd_dkdv_reduce_kernel(const BwdParams p) {
  const int groups = p.batch * p.hkv;
  const int tiles = p.kt1 - p.kt0;
  const int tg = blockIdx.x;                                  // tile * groups + group
  const int e = (blockIdx.y * 256 + threadIdx.x) * 4;         // element of the tile's BK x D block
  const int64_t key = (int64_t)(p.kt0 + tg / groups) * BK + e / D;
  if (e >= BK * D || key >= p.skv) return;
  const int g = tg % groups;
  const int64_t out = ((int64_t)g * p.skv + key) * D + e % D;   // g = b * hkv + hk
  f32x4 sk = *reinterpret_cast<const f32x4 *>(p.dk + out);
  f32x4 sv = *reinterpret_cast<const f32x4 *>(p.dv + out);
  for (int j = 1; j < p.kv_parts; ++j) {
    const float *slot = p.kv_partial + (((int64_t)(j - 1) * tiles + tg / groups) * groups + g) * 2 * BK * D;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(slot + e);
    const f32x4 c = *reinterpret_cast<const f32x4 *>(slot + BK * D + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sk[i] += a[i];
      sv[i] += c[i];
    }
  }
  *reinterpret_cast<f32x4 *>(p.dk + out) = sk;
  *reinterpret_cast<f32x4 *>(p.dv + out) = sv;
}

// ---------------------------------------------------------------------------
// 3. dQ (query-stationary; work items as in the forward)
// ---------------------------------------------------------------------------
// One workgroup = 8 wavefronts = one work item (a tile of query rows of one
// chunk for a pack of query heads of one GQA group); each wavefront owns 32
// query rows of one head, as two 16-row blocks. K/V tiles of 64 keys are
// loaded straight from global memory into 4-stage LDS rings and read by every
// head. With the query in the lane (v_mfma_f32_16x16x32_bf16), S^T = K Q^T
// and dP^T = V dO^T give P^T = exp2(S^T * scale*log2(e) - LSE*log2(e)) and
// dS^T = P^T o (dP^T - Delta) from per-lane scalars, and dS^T feeds
// dQ^T += K^T dS^T straight from registers (K^T by transpose reads; every K,
// V or K^T fragment read from LDS feeds both row blocks). Software pipeline
// over 32-key blocks: in block b the matrix core computes dQ^T of block b-1
// and S^T, dP^T of block b+1 while the vector ALU forms dS^T of block b; one
// barrier per 64-key tile.
// MODE 0: keys in natural order; 1: several KV chunks; 2: natural order with
// packed-sequence boundaries; 3: natural order with a user attention mask.
template <int D, int RB, int MODE>
__global__ void __launch_bounds__(NT, 2) bwd_dq_kernel(const BwdParams p) {
  constexpr bool MKV = MODE == 1;
  constexpr bool DOCS = MODE == 2;
  constexpr bool UMASK = MODE == 3;
  constexpr int HPW = kDqWaves / RB;
  constexpr int BM = kDqWaveRows * RB;
  constexpr int NC = D / 8;
  constexpr int QB = kDqWaveRows / 16;         // 16-row query blocks per wavefront
  constexpr int KSTEPS = D / 32;               // k-steps of S^T, dP^T (over D)
  constexpr int DB = D / 16;                   // 16-row blocks of dQ^T
  constexpr int TILE = BN * D;                 // elements of a K or V tile (64 keys)
  constexpr int STG = 4;                       // ring stages (K and V)
  constexpr int K_OFF = 0;
  constexpr int V_OFF = STG * TILE * 2;
  // After the K/V rings, a user mask's region: [STG][waves][32 rows] row-bit
  // words, or (an additive mask with biases, shared by the item's heads)
  // [2][64 rows][64 keys] float values of a tile, each row's 16-byte chunks
  // swizzled (chunk c of row r at slot c ^ (r % 16)).
  constexpr int MB_OFF = 2 * STG * TILE * 2;
  constexpr int MB_WAVE = kDqWaveRows * 8;
  constexpr bool ADDS_LDS = UMASK && RB == 2;   // (items of more rows: their tiles do not fit)
  constexpr int MA_TILE = kDqWaveRows * RB * BN * 4;
  constexpr int MB_BYTES =
      !ADDS_LDS || STG * kDqWaves * MB_WAVE > 2 * MA_TILE ? STG * kDqWaves * MB_WAVE : 2 * MA_TILE;
  constexpr int LDS_BYTES = MB_OFF + (UMASK ? MB_BYTES : 0);
  static_assert(BN == 64 && QB == 2 && LDS_BYTES <= 160 * 1024, "tile shape");
  using T = Tile16<D>;
  // A user mask's bit table stands for it when it is boolean, or additive
  // with only 0 and hiding values (the row-bit pass says which; a share
  // without keys has no table, and no flag, and reads no mask).
  bool use_bits = false;
  if constexpr (UMASK) use_bits = !p.mask_add || (p.mask_flag != nullptr && *p.mask_flag == 0);

  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = lane >> 4;   // operand k-slice / accumulator row quarter
  const int col = lane & 15;   // operand row / accumulator column

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
  // This lane's query in each 16-row block.
  bool qvalid[QB];
  int64_t qpos[QB];
  int local_row[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = 16 * qb + col;
    qvalid[qb] = r < wrows;
    qpos[qb] = wave_qlo + min(r, max(wrows - 1, 0));
    local_row[qb] = chunk * p.chunk_len + item_row0 + wrow0 + r;
  }

  // KV tiles to visit: per KV chunk the prefix its rows can see. One chunk
  // (MKV false): pipeline tile J is storage tile J. Several: the chunks'
  // prefixes one after another, handed out by a scalar cursor as (storage
  // tile, global position of storage row 0 seen from the tile's chunk), as in
  // the forward kernel.
  auto vis_tiles = [&](int c) {
    int nv = p.kv.len;
    if (p.causal) {
      const int64_t n = item_qhi - p.kv.pos[c] + 1;
      nv = (int)(n < 0 ? 0 : (n > p.kv.len ? p.kv.len : n));
    }
    return (nv + BN - 1) / BN;
  };
  int ntiles = 0;
  if constexpr (MKV) {
    for (int c = 0; c < p.kv.n; ++c) ntiles += vis_tiles(c);
  } else {
    ntiles = vis_tiles(0);
  }
  const int64_t kv_pos0 = p.kv.pos[0];
  // User mask: this lane's mask row per row block (lanes past the wave's last
  // row read the item's first row, like Q).
  // A boolean mask comes as row bits instead (FwdParams::mask_rowbits'
  // layout): each tile's words of the wavefront's rows are staged in LDS with
  // the tile's K and V; the lane's 16 bits of a 64-key tile lie at bit
  // 16*grp + 4*kb + i for key 16*kb + 4*grp + i, kb = 2 * (32-key block) +
  // half.
  const uint8_t *mrow[QB];
  if constexpr (UMASK) {
    static_assert(BN == 64, "row-bit words cover 64-key tiles");
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int mr = qvalid[qb] ? local_row[qb] : chunk * p.chunk_len + item_row0;
      mrow[qb] = p.mask + b * p.m_sb + head * p.m_sh + (int64_t)mr * p.m_ss;
    }
  }
  // Packed sequences, as in the forward kernel: this lane's rows see keys
  // from their sequence's start (lo_key, a key row index); the item skips the
  // tiles before its first row's sequence start (t0); a block that starts
  // before the wave's last row's sequence start (wave_ds) is masked.
  int t0 = 0;
  int lo_key[QB];
  int64_t wave_ds = INT64_MIN;
  if constexpr (DOCS) {
    int64_t ds[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ds[qb] = INT64_MIN;
    int64_t item_ds = INT64_MIN;
    const int64_t item_qlo = chunk_pos + item_row0;
    const int64_t wave_qhi = wave_qlo + max(wrows - 1, 0);
    for (int i = 0; i < p.docs.n; ++i) {
      const int64_t bd = p.docs.pos[i];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) ds[qb] = bd <= qpos[qb] ? bd : ds[qb];
      if (bd <= item_qlo) item_ds = bd;
      if (bd <= wave_qhi) wave_ds = bd;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lo_key[qb] = ds[qb] > kv_pos0 ? (int)min<int64_t>(ds[qb] - kv_pos0, p.skv) : 0;
    if (item_ds > kv_pos0) t0 = (int)min<int64_t>(ntiles, (item_ds - kv_pos0) / BN);
    ntiles -= t0;
  }
  struct TileRef {
    int kt;          // storage tile
    int64_t base;    // global position of storage row 0 (this tile's chunk)
    int64_t adj;     // extra elements of its chunk's storage (chunk strides)
  };
  int cur_c = 0, cur_left = vis_tiles(0), cur_kt = 0;
  auto next_tile = [&]() -> TileRef {
    // At most ntiles calls: a chunk with tiles left always follows (the bound
    // only guards the loop; the ragged-tile staging clamps rows into K/V).
    while (cur_left == 0 && cur_c + 1 < p.kv.n) {
      ++cur_c;
      cur_left = vis_tiles(cur_c);
      cur_kt = cur_c * (p.kv.len / BN);
    }
    const TileRef r{cur_kt, p.kv.pos[cur_c] - (int64_t)cur_c * p.kv.len, (int64_t)cur_c * p.kv.cadj};
    ++cur_kt;
    --cur_left;
    return r;
  };

  // Q and dO rows of this lane's queries: B operands of S^T and dP^T. Lanes
  // past the item's last row read its first row and get LSE = +inf (P = 0).
  bf16x8 qf[QB][KSTEPS], gf[QB][KSTEPS];
  float lse2[QB], ndelta[QB];   // LSE*log2(e) and -Delta of this lane's queries
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int load_row = qvalid[qb] ? local_row[qb] : chunk * p.chunk_len + item_row0;
    const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + head * p.q_sh + chunk * p.q_cadj +
                       (int64_t)load_row * p.q_ss + 8 * grp;
    const __bf16 *gp = static_cast<const __bf16 *>(p.dout) + b * p.o_sb + head * p.o_sh + chunk * p.o_cadj +
                       (int64_t)load_row * p.o_ss + 8 * grp;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[qb][s] = *reinterpret_cast<const bf16x8 *>(qp + 32 * s);
      gf[qb][s] = *reinterpret_cast<const bf16x8 *>(gp + 32 * s);
    }
    lse2[qb] = INFINITY;
    ndelta[qb] = 0.0f;
    if (qvalid[qb]) {
      const int64_t row = ((int64_t)b * p.hq + head) * p.sq + local_row[qb];
      lse2[qb] = p.lse2[row];
      ndelta[qb] = p.delta[row];
    }
  }
  wait_vmem_all();

  // ---- staging: global -> LDS directly (see the forward kernel) -------------
  constexpr int RPI = 64 / NC;
  constexpr int INSTS = BN / (kDqWaves * RPI);
  static_assert(INSTS >= 1 && (kDqWaves * RPI) % 16 == 0, "staging shape");
  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + hkv * p.kv_sh;
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + hkv * p.kv_sh;
  const int srow = wave * RPI + lane / NC;
  const int scol = 8 * ((lane % NC) ^ T::swz(srow));
  const int64_t tile_stride = (int64_t)BN * p.kv_ss;
  const int64_t istep_bytes = (int64_t)kDqWaves * RPI * p.kv_ss * 2;
  const uint32_t goff0 = (uint32_t)(((int64_t)srow * p.kv_ss + scol) * 2);
  const uint32_t dst0 = lds0 + 2 * wave * RPI * D;
  auto dma1 = [](uint32_t m0, uint32_t voff, const void *sbase) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
  };
  auto dma4 = [](uint32_t m0, uint32_t voff, const void *sbase) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
  };
  // Boolean user mask: the row-bit words of the item's rows (tile 0), two
  // lanes per word of the wavefront's rows (rows past its last read the
  // item's first row).
  const uint64_t *rb_item = nullptr;
  uint32_t rb_voff = 0;
  if constexpr (UMASK) {
    const int64_t bhm = (int64_t)(p.mb_batches > 1 ? b : 0) * p.mb_heads + (p.mb_heads > 1 ? head : 0);
    rb_item = p.mask_rowbits + bhm * p.mb_ktiles * p.sq + chunk * p.chunk_len + item_row0;
    const int w = lane >> 1;
    rb_voff = (uint32_t)((w < wrows ? wrow0 + w : 0) * 8 + 4 * (lane & 1));
  }
  // An additive mask with biases that all the item's heads share: its values
  // of tile kt for the item's rows into LDS stage st (two 1 KiB loads per
  // wavefront, four rows each, with the swizzle above; rows past the item's
  // last read its last row). A ragged tile is not staged (its reads stay
  // per lane, with the end test).
  const bool stage_adds = ADDS_LDS && !use_bits && p.mb_heads == 1 && p.mask_add;
  auto dma_adds = [&](int kt, int st) {
    if constexpr (ADDS_LDS) {
      if (!stage_adds || kt * BN + BN > p.skv) return;
      const uint8_t *rows0 = p.mask + b * p.m_sb + (int64_t)(chunk * p.chunk_len + item_row0) * p.m_ss +
                             (int64_t)kt * BN * 4;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = 4 * (2 * wave + i) + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);
        const uint32_t vo = (uint32_t)min(r, item_rows - 1) * (uint32_t)p.m_ss + 16u * (uint32_t)c;
        dma1(lds0 + MB_OFF + st * MA_TILE + (2 * wave + i) * 1024, vo, rows0);
      }
    }
  };
  // K and V of storage tile kt (adj: its KV chunk's extra elements) into
  // ring stage st (and the tile's mask words).
  auto dma = [&](int kt, int64_t adj, int st) {
    if constexpr (UMASK) {
      if (use_bits) dma4(lds0 + MB_OFF + (st * kDqWaves + wave) * MB_WAVE, rb_voff, rb_item + (int64_t)kt * p.sq);
    }
    const uint32_t kd = dst0 + K_OFF + 2 * st * TILE;
    const uint32_t vd = dst0 + V_OFF + 2 * st * TILE;
    const char *kt_base = reinterpret_cast<const char *>(kbase + (int64_t)kt * tile_stride + adj);
    const char *vt_base = reinterpret_cast<const char *>(vbase + (int64_t)kt * tile_stride + adj);
    if (kt * BN + BN <= p.skv) {
#pragma unroll
      for (int i = 0; i < INSTS; ++i) {
        dma1(kd + 2 * i * kDqWaves * RPI * D, goff0, kt_base + i * istep_bytes);
        dma1(vd + 2 * i * kDqWaves * RPI * D, goff0, vt_base + i * istep_bytes);
      }
    } else {
      // Ragged last tile: rows past the end read the last row (always masked).
      // Offsets count from the tile's own 64-bit base, so they stay below BN
      // row strides (< 2^31 bytes) however far the tile lies from the head's.
      const int last = p.skv - 1 - kt * BN;
#pragma unroll
      for (int i = 0; i < INSTS; ++i) {
        const uint32_t r = (uint32_t)min(srow + i * kDqWaves * RPI, last);
        const uint32_t o = (r * (uint32_t)p.kv_ss + (uint32_t)scol) * 2u;
        dma1(kd + 2 * i * kDqWaves * RPI * D, o, kt_base);
        dma1(vd + 2 * i * kDqWaves * RPI * D, o, vt_base);
      }
    }
  };

  // ---- per-lane LDS addressing ----------------------------------------------
  // Row reads of K and V (A operands of S^T and dP^T: key row col of a 16-key
  // block, chunk 4s+grp) and transpose reads of K (A operand of
  // dQ^T = K^T dS^T: keys 4grp .. 4grp+3 and 16 + 4grp .. of a 32-key block,
  // column 16db + col); stage, key block and k-step are immediates.
  // (Separate K and V bases: the V ring starts 64 KiB in, beyond the reach
  // of an immediate.)
  // This lane's byte of its row's mask word (boolean mask) at stage 0, row
  // block 0 and 32-key block 0, beyond the reach of an immediate as well.
  uint32_t mbits = lds0 + MB_OFF + wave * MB_WAVE + col * 8 + 2 * grp;
  // This lane's row of a staged additive tile (stage 0, row block 0).
  uint32_t madds = lds0 + MB_OFF + (wrow0 + col) * BN * 4;
  uint32_t kaddr[KSTEPS], vaddr[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    kaddr[s] = lds0 + K_OFF + 2 * T::chunk_off(col, 4 * s + grp);
    vaddr[s] = lds0 + V_OFF + 2 * T::chunk_off(col, 4 * s + grp);
  }
  uint32_t taddr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) taddr[db] = lds0 + 2 * T::elem_off(4 * grp + (col >> 2), 16 * db + 4 * (lane & 3));
  auto lds_b128 = [](uint32_t addr) -> bf16x8 {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>((uintptr_t)addr);
  };
  auto lds_tr = [&](int db, uint32_t off) -> bf16x8 {
    const i16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)(taddr[db] + off));
    const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)(taddr[db] + off + 2 * 16 * D));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x4 qacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) qacc[qb][db][i] = 0.0f;
  const float c2 = p.scale_log2;

  // Operand reads at compile-time offsets: K or V rows of 16-key block h of
  // 32-key block kb (k-step s), K^T of 32-key block kb (O^T block db).
  auto kv_row = [&](bool v, int st, int kb, int h, int s) {
    return lds_b128((v ? vaddr[s] : kaddr[s]) + 2 * (st * TILE + (32 * kb + 16 * h) * D));
  };
  auto k_tr = [&](int st, int kb, int db) { return lds_tr(db, K_OFF + 2 * (st * TILE + 32 * kb * D)); };

  // ---- prologue ---------------------------------------------------------------
  // K stage 3 stands for "tile -1" in block 0 (its dS is zero): clear it.
  {
    u32x4 *k3 = reinterpret_cast<u32x4 *>(smem + K_OFF + 2 * 3 * TILE);
    for (int i = tid; i < TILE / 8; i += NT) k3[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // S^T, dP^T of a block ([16-key half][row block]) alternate between two
  // register sets by block parity.
  f32x4 sbuf[2][2][QB], pbuf[2][2][QB];
  bf16x8 dsbuf[2][QB];   // dS^T of the last two blocks (bf16 B operands)
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int e = 0; e < 8; ++e) dsbuf[q][qb][e] = (__bf16)0.0f;
  // Tiles J, J+1, J+2 of the pipeline.
  TileRef t_cur{t0, kv_pos0, 0}, t_nx1{t0 + 1, kv_pos0, 0}, t_nx2{t0 + 2, kv_pos0, 0};
  if constexpr (MKV) {
    if (ntiles > 0) t_cur = next_tile();
    if (ntiles > 1) t_nx1 = next_tile();
    if (ntiles > 2) t_nx2 = next_tile();
  }
  // Storage offset of a natural-order tile (merged chunks; 0 for one chunk).
  auto nat_adj = [&](int kt) { return ((int64_t)kt * BN >> p.kv.store_lg) * p.kv.cadj; };
  if (ntiles > 0) dma(t_cur.kt, MKV ? t_cur.adj : nat_adj(t_cur.kt), 0);
  if constexpr (UMASK) {
    if (ntiles > 0) dma_adds(t0, 0);
  }
  if (ntiles > 1) dma(t_nx1.kt, MKV ? t_nx1.adj : nat_adj(t_nx1.kt), 1);
  wait_vmem_all();
  __syncthreads();
  if (ntiles > 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sbuf[0][h][qb][i] = 0.0f;
          pbuf[0][h][qb][i] = ndelta[qb];   // dP^T - Delta, as in the blocks
        }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 ka = kv_row(false, 0, 0, h, s), va = kv_row(true, 0, 0, h, s);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sbuf[0][h][qb] = mfma16(ka, qf[qb][s], sbuf[0][h][qb]);
          pbuf[0][h][qb] = mfma16(va, gf[qb][s], pbuf[0][h][qb]);
        }
      }
  }

  constexpr int AHEAD = 2;
  constexpr int NBUF = AHEAD + 1;
  constexpr int NDQ = DB;                // K^T operands of a block (db)
  constexpr int NOP = NDQ + 4 * KSTEPS;  // + K and V rows of both 16-key halves
  constexpr int NSLOT = QB * NOP;
  constexpr int NPAIR = 2 * QB * 2;      // pairs of dS^T values per lane per block

  // One block bb = 2*J + KB (tile J, 32-key block KB; J4 = J % 4): dQ^T(bb-1)
  // and S^T, dP^T(bb+1) on the matrix core, dS^T(bb) on the VALU. sb is the
  // block's index in storage, base the position of storage row 0 seen from it.
  auto block = [&](auto j4_tag, auto kb_tag, int sb, int64_t base) {
    constexpr int J4 = decltype(j4_tag)::value, KB = decltype(kb_tag)::value;
    constexpr int SET = KB;                       // block parity
    constexpr int ST_PREV = KB == 0 ? (J4 + 3) % STG : J4;   // stage of block bb-1
    constexpr int KB_PREV = 1 - KB;
    constexpr int ST_NEXT = KB == 0 ? J4 : (J4 + 1) % STG;   // stage of block bb+1
    constexpr int KB_NEXT = 1 - KB;
    f32x4 (&scur)[2][QB] = sbuf[SET];
    f32x4 (&pcur)[2][QB] = pbuf[SET];
    f32x4 (&snext)[2][QB] = sbuf[1 - SET];
    f32x4 (&pnext)[2][QB] = pbuf[1 - SET];
    const bf16x8 (&dsprev)[QB] = dsbuf[1 - SET];
    bf16x8 (&dscur)[QB] = dsbuf[SET];
    // Mask of block bb (diagonal or ragged blocks only): key 16*h + 4*grp + i
    // of the block is visible iff it is <= lim; masked scores become -inf
    // (P = 0).
    const int64_t blk_plo = base + (int64_t)sb * 32;
    bool need_mask = (sb * 32 + 32 > p.skv) || (p.causal && blk_plo + 31 > wave_qlo);
    if constexpr (DOCS) need_mask = need_mask || blk_plo < wave_ds;
    // (A user mask is applied to every block, the range mask only where needed.)
    if (need_mask || UMASK) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (!UMASK || need_mask) {
          int lim = p.skv - 1 - sb * 32;
          if (p.causal) {
            const int64_t rel = qpos[qb] - blk_plo;
            lim = min(lim, (int)(rel < -1 ? -1 : (rel > 32 ? 32 : rel)));
          }
          const int t = lim - 4 * grp;
          if constexpr (DOCS) {
            // ... and >= the row's sequence start.
            const int tl = min(max(lo_key[qb] - sb * 32, 0), 32) - 4 * grp;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                scur[h][qb][i] = (16 * h + i > t || 16 * h + i < tl) ? -INFINITY : scur[h][qb][i];
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i) scur[h][qb][i] = (16 * h + i > t) ? -INFINITY : scur[h][qb][i];
          }
        }
        if constexpr (UMASK) {
          // ... and the user mask (the row bits unless additive with biases).
          // Additive: the 4 floats of this lane's keys
          // 16*h + 4*grp .. +3 of the block, every read issued before any is
          // used; in a ragged block keys past the end read nothing (no bias on
          // a score the range mask hid).
          if (!use_bits) {
            const bool full = sb * 32 + 32 <= p.skv;
            // Additive: value / softmax_scale; at or below kMaskHide: hidden.
            const float inv = 1.0f / p.scale;
            const float *mf = reinterpret_cast<const float *>(mrow[qb]);
            f32x4 a[2];
            if (ADDS_LDS && stage_adds && (sb >> 1) * BN + BN <= p.skv) {
              // The tile's values staged in LDS: row wrow0 + 16qb + col,
              // chunk 8KB + 4h + grp at its swizzled slot.
#pragma unroll
              for (int h = 0; h < 2; ++h)
                a[h] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4 *>(
                    (uintptr_t)(madds + (J4 & 1) * MA_TILE + 16 * qb * BN * 4 + (((grp ^ col) ^ (8 * KB + 4 * h)) << 4)));
            } else {
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const int k0 = sb * 32 + 16 * h + 4 * grp;
                if (full) {
                  a[h] = *reinterpret_cast<const f32x4 *>(mf + k0);
                } else {
#pragma unroll
                  for (int i = 0; i < 4; ++i) a[h][i] = k0 + i < p.skv ? mf[k0 + i] : 0.0f;
                }
              }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                scur[h][qb][i] = a[h][i] <= kMaskHide ? -INFINITY : fmaf(a[h][i], inv, scur[h][qb][i]);
          } else {
            // Boolean: the block's 8 bits of the row's word of the tile.
            const uint32_t w8 = *reinterpret_cast<const __attribute__((address_space(3))) uint8_t *>(
                (uintptr_t)(mbits + J4 * kDqWaves * MB_WAVE + 16 * qb * 8 + KB));
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                scur[h][qb][i] = keep_if_bit(scur[h][qb][i], w8, 4 * h + i);
          }
        }
      }
    }
    // Operand o (used by both row blocks in consecutive slots): o < NDQ is
    // K^T of block bb-1 (db = o); then, for u = o - NDQ, k-step s = u / 4 of
    // the K (u even) or V (u odd) rows of 16-key half h = (u / 2) % 2 of
    // block bb+1, so that products accumulating into one S^T or dP^T block
    // are eight slots apart.
    auto read = [&](auto o_tag) -> bf16x8 {
      constexpr int o = decltype(o_tag)::value;
      if constexpr (o < NDQ) {
        return k_tr(ST_PREV, KB_PREV, o);
      } else {
        constexpr int u = o - NDQ;
        return kv_row(u & 1, ST_NEXT, KB_NEXT, (u >> 1) & 1, u >> 2);
      }
    };
    bf16x8 opnd[NBUF];
    static_for<AHEAD>([&](auto o) { opnd[decltype(o)::value] = read(o); });
    static_for<NSLOT>([&](auto t_tag) {
      constexpr int t = decltype(t_tag)::value;
      constexpr int o = t / QB, qb = t % QB;
      if constexpr (qb == 0 && o + AHEAD < NOP) opnd[(o + AHEAD) % NBUF] = read(IC<o + AHEAD>{});
      if constexpr (o < NDQ) {
        qacc[qb][o] = mfma16(opnd[o % NBUF], dsprev[qb], qacc[qb][o]);
      } else {
        constexpr int u = o - NDQ, s = u >> 2, h = (u >> 1) & 1;
        f32x4 &dst = (u & 1) ? pnext[h][qb] : snext[h][qb];
        const bf16x8 &bop = (u & 1) ? gf[qb][s] : qf[qb][s];
        if constexpr (s == 0) {
          // dP^T starts from -Delta (so it comes out as dP^T - Delta), S^T from 0.
          const float z0 = (u & 1) ? ndelta[qb] : 0.0f;
          f32x4 z;
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] = z0;
          dst = mfma16(opnd[o % NBUF], bop, z);
        } else {
          dst = mfma16(opnd[o % NBUF], bop, dst);
        }
      }
      // The slot's vector work is issued after its matrix instruction.
      __builtin_amdgcn_sched_barrier(0);
      // dS^T pair e (row block e / 4, half (e / 2) % 2, elements 2(e%2),
      // 2(e%2)+1) in slot e * NSLOT / NPAIR; it lands in elements 4h + i of
      // the row block's B operand (the key order of the K^T reads).
      static_for<NPAIR>([&](auto e_tag) {
        constexpr int e = decltype(e_tag)::value;
        if constexpr (e * NSLOT / NPAIR == t) {
          constexpr int rq = e / 4, h = (e / 2) % 2, i = 2 * (e % 2);
          const float p0 = __builtin_amdgcn_exp2f(fmaf(scur[h][rq][i], c2, -lse2[rq]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(scur[h][rq][i + 1], c2, -lse2[rq]));
          const float x0 = p0 * pcur[h][rq][i];
          const float x1 = p1 * pcur[h][rq][i + 1];
          const bf16x2 t2 = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
          dscur[rq][4 * h + i] = t2[0];
          dscur[rq][4 * h + i + 1] = t2[1];
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // Pin dS^T(bb) to the slots above (otherwise the compiler sinks it past
    // the next block's mask branch, away from the products it overlaps).
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" ::"v"(dscur[qb]));
  };

  // Tile step J (J4 = J % 4): tile J+2 on its way into the rings (into the
  // stage of tile J-2, last read in step J-1), then the tile's two blocks.
  auto tile_step = [&](auto j4_tag, int J) {
    constexpr int J4 = decltype(j4_tag)::value;
    if (J + 2 < ntiles) dma(MKV ? t_nx2.kt : t0 + J + 2, MKV ? t_nx2.adj : nat_adj(t0 + J + 2), (J4 + 2) % STG);
    if constexpr (UMASK) {
      if (J + 1 < ntiles) dma_adds(t0 + J + 1, (J4 + 1) & 1);
    }
    // Opaque bases: the V ring's start (64 KiB) and the stage offsets then
    // stay instruction offsets instead of per-read address arithmetic.
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(taddr[db]));
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("" : "+v"(kaddr[s]), "+v"(vaddr[s]));
    if constexpr (UMASK) asm volatile("" : "+v"(mbits), "+v"(madds));
    TileRef t{t0 + J, kv_pos0, 0};
    if constexpr (MKV) {
      t = t_cur;
      t_cur = t_nx1;
      t_nx1 = t_nx2;
      if (J + 3 < ntiles) t_nx2 = next_tile();
    }
    block(j4_tag, IC<0>{}, 2 * t.kt, t.base);
    block(j4_tag, IC<1>{}, 2 * t.kt + 1, t.base);
    wait_vmem_all();
    __syncthreads();
  };
  for (int J = 0; J < ntiles; J += STG) {
    tile_step(IC<0>{}, J);
    if (J + 1 < ntiles) tile_step(IC<1>{}, J + 1);
    if (J + 2 < ntiles) tile_step(IC<2>{}, J + 2);
    if (J + 3 < ntiles) tile_step(IC<3>{}, J + 3);
  }
  // dQ^T of the last block (tile ntiles-1, 32-key block 1; dS^T in set 1).
  if (ntiles > 0) {
    const int st = (ntiles - 1) % STG;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 a = k_tr(st, 1, db);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) qacc[qb][db] = mfma16(a, dsbuf[1][qb], qacc[qb][db]);
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    if (!qvalid[qb]) continue;
    __bf16 *dst = static_cast<__bf16 *>(p.dq) + b * p.o_sb + head * p.o_sh + chunk * p.o_cadj +
                  (int64_t)local_row[qb] * p.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(qacc[qb][db][e] * p.scale);
      *reinterpret_cast<bf16x4 *>(dst + 16 * db + 4 * grp) = o4;
    }
  }
}

// Launches of one mode's instantiations.
template <int D, int KMODE>
void launch_dkdv_mode(const BwdParams &p, hipStream_t s) {
  // Key tiles (and their parts) first, then workgroups that zero the dK/dV
  // rows of the keys no local row sees: about 64 KiB of stores each, at most
  // one per compute unit.
  const int64_t tiles = p.kt1 - p.kt0;
  const int64_t back = (int64_t)p.kt1 * BK < p.skv ? (int64_t)p.kt1 * BK : (int64_t)p.skv;
  const int64_t zbytes = ((int64_t)p.kt0 * BK + (p.skv - back)) * D * 4 * 2 * p.batch * p.hkv;
  const int64_t zw = zbytes > 0 ? std::min<int64_t>((zbytes + 65535) / 65536, 256) : 0;
  const int64_t grid = tiles * p.kv_parts * p.batch * p.hkv + zw;
  if (grid > 0) hipLaunchKernelGGL((bwd_dkdv_kernel<D, KMODE>), dim3(grid), dim3(kDkdvThreads), 0, s, p);
  if (tiles > 0 && p.kv_parts > 1)
    hipLaunchKernelGGL(bwd_dkdv_reduce_kernel<D>, dim3(tiles * p.batch * p.hkv, (BK * D / 4 + 255) / 256),
                       dim3(256), 0, s, p);
}

template <int D, int MODE>
int launch_dq_mode(const BwdParams &p, hipStream_t s) {
  const int64_t items = (int64_t)p.n_head_packs * p.n_q_chunks * p.tiles_per_chunk;
  const int64_t rows = (int64_t)p.batch * p.hq * p.sq;
  if (rows == 0 || items == 0) return 0;
  switch (kDqWaves / p.heads_per_item) {
    case 2: hipLaunchKernelGGL((bwd_dq_kernel<D, 2, MODE>), dim3(items), dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((bwd_dq_kernel<D, 4, MODE>), dim3(items), dim3(NT), 0, s, p); break;
    case 8: hipLaunchKernelGGL((bwd_dq_kernel<D, 8, MODE>), dim3(items), dim3(NT), 0, s, p); break;
    default: return (int)hipErrorInvalidValue;
  }
  return 0;
}

}  // namespace
}  // namespace cpattn
