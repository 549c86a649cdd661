// Forward of one CP rank's attention share, bf16 inputs, fp32 accumulation,
// on gfx950 matrix cores: the kernel template, instantiated per mode by the
// fwd_bf16_m*.hip files (one compile each) and dispatched by fwd_bf16.hip.
//
// What is computed: for every local query row (global position from its
// chunk) the softmax over the visible gathered keys of scale * q.k, applied to
// v, plus the natural-log LSE ("新流程 CP 多通信模式迁移设计方案" §6.1 local-Q /
// global-KV attention, §8 global-position causal mask, §9.2 GQA).
//
// How (one workgroup = 8 wavefronts = one work item, two wavefronts per SIMD):
//  * a work item is a tile of query rows of one chunk for a pack of query
//    heads that read the same KV head (GQA); K/V tiles of 64 keys pass
//    through 4-stage LDS rings once per workgroup, loaded straight from
//    global memory into LDS (global_load_lds_dwordx4), and are read by every
//    head; the workgroup synchronises once per two tiles (K is loaded three
//    tiles ahead, V one, so that no stage is refilled or read across a step
//    without a barrier between);
//  * each wavefront owns 32 query rows of one head (two 16-row blocks) and
//    computes transposed score tiles S^T = K Q^T (keys x queries) with
//    v_mfma_f32_16x16x32_bf16, so that a lane holds one query column: the
//    row statistics of the online softmax are lane-local plus a reduction
//    over the four lanes of a column. Each K fragment read from LDS feeds both
//    row blocks. (Under the chip's power limit this shape sustains about 12 %
//    more bf16 throughput than the 32x32x16 one.);
//  * the probabilities P^T, converted to bf16 in registers, are the B operand
//    of O^T += V^T P^T without any shuffle: the contraction index (keys) is
//    permuted identically in both operands, and V^T is read from the
//    row-major V tile with the gfx950 LDS transpose read ds_read_b64_tr_b16
//    (the tiles' row swizzle keeps both the row reads of K and the
//    transpose reads of V free of bank conflicts);
//  * three-way software pipeline: in step j the matrix core computes
//    O^T += V^T P^T of tile j-1 and S^T of tile j+1 while the vector ALU turns
//    the scores of tile j into probabilities. The three are independent; the
//    step is written as slots of one matrix instruction plus a share of the
//    vector work, so a wavefront keeps its matrix core fed while it
//    exponentiates;
//  * KV tiles wholly after the work item's last query are never visited; only
//    tiles crossing the causal diagonal (or the ragged end of K/V) are masked;
//  * the running max is a reference point, not recomputed per tile: the
//    probabilities of a tile are formed against the current reference, and
//    only when a lane's partial tile sum exceeds 2^16 (or the row has no reference
//    yet) is its max taken, O rescaled and the tile redone.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "gfx950_common.h"
#include "plan.h"

namespace cpattn {
namespace {

constexpr int BN = kFwdBlockKV;          // keys per tile (64)
constexpr int NW = kFwdWaves;            // wavefronts per workgroup (8)
constexpr int NT = NW * 64;
constexpr int QB = kFwdWaveRows / 16;    // 16-row query blocks per wavefront
constexpr int KSTAGES = 4;               // K ring: tile t in stage t % 4
constexpr int VSTAGES = 4;               // V ring: tile t in stage t % 4
constexpr int K_AHEAD = 3;               // step j loads K of tile j+3 ...
constexpr int V_AHEAD = 1;               // ... and V of tile j+1
constexpr int UNROLL = 4;                // steps per loop trip (both ring indices fixed)
constexpr float kSumLimit = 65536.0f;    // largest tile sum kept without a new max


// MODE 0: keys in natural order (one KV chunk); 1: several KV chunks; 2:
// natural order with packed-sequence boundaries; 3: natural order with a user
// attention mask.
template <int D, int RB, int MODE>
__global__ void __launch_bounds__(NT, 2) fwd_bf16_kernel(const FwdParams p) {
  constexpr bool MKV = MODE == 1;
  constexpr bool DOCS = MODE == 2;
  constexpr bool UMASK = MODE == 3;
  constexpr int HPW = NW / RB;         // heads per work item
  constexpr int BM = kFwdWaveRows * RB;  // query rows per work item
  constexpr int NC = D / 8;            // 16-byte chunks per row
  constexpr int KSTEPS = D / 32;       // k-steps of S^T (contraction over D)
  constexpr int DB = D / 16;           // 16-row blocks of O^T
  constexpr int KB = BN / 16;          // 16-key blocks of S^T
  constexpr int PSTEPS = BN / 32;      // k-steps of O^T (contraction over keys)
  constexpr int TILE = BN * D;
  static_assert(BN == 64 && QB == 2, "tile shape");
  using T = Tile16<D>;   // K tiles (row reads) and V tiles (transpose reads)
  // A user mask's bit table stands for it when it is boolean, or additive
  // with only 0 and hiding values (the row-bit pass says which; a share
  // without keys has no table, and no flag, and reads no mask).
  bool use_bits = false;
  if constexpr (UMASK) use_bits = !p.mask_add || (p.mask_flag != nullptr && *p.mask_flag == 0);

  // K ring followed by the V ring, in one LDS array: 128 KiB at D = 128.
  // Barriers close the odd steps only. Step j reads K of tile j+1 and V of
  // tile j-1; K of tile t is loaded in step t-3 into the stage that K of
  // tile t-4 left in step t-5, and V of tile t in step t-1 into the stage
  // that V of tile t-4 left in step t-3: of any two consecutive steps one
  // ends in a barrier, so every load is published before its tile is read
  // and starts after the previous occupant's last reader passed a barrier.
  // A boolean user mask's row-bit words follow the rings: per K stage, the
  // words of each wavefront's 32 rows for that stage's tile.
  // Or, for an additive mask with biases that all the item's heads share
  // (items of 64 rows), [2][64 rows][64 keys] float values of a tile, each
  // row's 16-byte chunks swizzled (chunk c of row r at slot c ^ (r % 16)).
  constexpr int MB_OFF = (KSTAGES + VSTAGES) * TILE * 2;
  constexpr int MB_WAVE = kFwdWaveRows * 8;
  constexpr bool ADDS_LDS = UMASK && RB == 2;
  constexpr int MA_TILE = BM * BN * 4;
  constexpr int MB_BYTES =
      !ADDS_LDS || KSTAGES * NW * MB_WAVE > 2 * MA_TILE ? KSTAGES * NW * MB_WAVE : 2 * MA_TILE;
  constexpr int LDS_BYTES = MB_OFF + (UMASK ? MB_BYTES : 0);
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  static_assert((KSTAGES + VSTAGES) * TILE * 2 <= 128 * 1024 && LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(KSTAGES >= K_AHEAD + 1 && VSTAGES >= V_AHEAD + 3 && K_AHEAD >= 3 && V_AHEAD >= 1 &&
                    UNROLL % KSTAGES == 0 && UNROLL % VSTAGES == 0 && UNROLL % 2 == 0,
                "ring depths for one barrier per two steps");
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void *)smem;   // LDS byte address of smem

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
  const int grp = lane >> 4;   // operand k-slice / accumulator row quarter
  const int col = lane & 15;   // operand row / accumulator column

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
  const int wrow0 = (wave % RB) * kFwdWaveRows;
  const int64_t wave_qlo = chunk_pos + item_row0 + min(wrow0, item_rows - 1);
  // This lane's query row in each 16-row block; rows past the item's last act
  // as its last row (never stored).
  int local_row[QB];
  int64_t qpos[QB];
  bool qvalid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = wrow0 + 16 * qb + col;
    const int qrow = min(r, item_rows - 1);
    qvalid[qb] = r < item_rows;
    qpos[qb] = chunk_pos + item_row0 + qrow;
    local_row[qb] = chunk * p.chunk_len + item_row0 + qrow;
  }

  // ---- KV tiles to visit ---------------------------------------------------
  // Per KV chunk, the prefix of its tiles that the item's last row can see.
  // With one chunk (MODE 0 and 2: the natural order) that prefix is the whole
  // visit list and pipeline tile j is storage tile j. With several (MKV), the
  // pipeline runs over the chunks' prefixes one after another and a scalar
  // cursor hands out the next tile as its storage tile and the global
  // position of storage row 0 as seen from its chunk. The softmax state
  // carries over between chunks, so the chunk order does not change the
  // result.
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
  // User mask: this lane's mask row per row block (rows past the item's last
  // read its last row, like Q). A boolean mask is read from its row-bit table
  // instead, staged in LDS with the K tiles.
  const uint8_t *mrow[QB];
  if constexpr (UMASK) {
    static_assert(BN == 64, "row-bit words cover 64-key tiles");
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      mrow[qb] = p.mask + b * p.m_sb + head * p.m_sh + (int64_t)local_row[qb] * p.m_ss;
  }
  // Packed sequences: each of this lane's rows sees keys from its sequence's
  // start (the last bound <= its position) on, as a key row index (lo_key);
  // the item skips the tiles before its first row's sequence start (t0), and a
  // tile that starts before the wave's last row's sequence start (wave_ds) is
  // masked. The scan over the bounds is wave-uniform.
  int t0 = 0;
  int lo_key[QB];
  int64_t wave_ds = INT64_MIN;
  if constexpr (DOCS) {
    int64_t ds[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) ds[qb] = INT64_MIN;
    int64_t item_ds = INT64_MIN;
    const int64_t item_qlo = chunk_pos + item_row0;
    const int64_t wave_qhi = chunk_pos + item_row0 + min(wrow0 + kFwdWaveRows, item_rows) - 1;
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
  // Natural order: the first tile that needs a mask (crossing the causal
  // diagonal of the wave's first row, or the ragged end of K/V); every later
  // tile needs one too.
  int mask_from = INT32_MAX;
  if constexpr (!MKV) {
    const int64_t rag = (int64_t)p.skv - BN;                 // kt*BN > rag: ragged
    int64_t mf = rag < 0 ? 0 : rag / BN + 1;
    if (p.causal) {
      const int64_t lim = wave_qlo - kv_pos0 - BN + 1;       // kt*BN > lim: crosses the diagonal
      mf = min(mf, lim < 0 ? (int64_t)0 : lim / BN + 1);
    }
    mask_from = (int)min(mf, (int64_t)INT32_MAX);
  }
  struct TileRef {
    int kt;          // storage tile
    int64_t base;    // global position of storage row 0 (this tile's chunk)
    int64_t adj;     // extra elements of its chunk's storage (chunk strides)
  };
  int cur_c = 0, cur_left = vis_tiles(0), cur_kt = 0;
  auto next_tile = [&]() -> TileRef {
    // Called at most ntiles times, so a chunk with tiles left always follows;
    // the bound keeps a stray call on the last chunk (its ragged-tile path
    // clamps every row into the tensor).
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

  // ---- Q fragments (B operands of S^T = K Q^T), resident for the whole item
  bf16x8 qf[QB][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const __bf16 *qp = static_cast<const __bf16 *>(p.q) + b * p.q_sb + head * p.q_sh + chunk * p.q_cadj +
                       (int64_t)local_row[qb] * p.q_ss + 8 * grp;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[qb][s] = *reinterpret_cast<const bf16x8 *>(qp + 32 * s);
  }
  wait_vmem_all();

  // ---- per-lane LDS addressing, computed once ------------------------------
  // Byte addresses of this lane's operand reads in stage 0; the stage, key
  // block and k-step only add constants, which become instruction immediates.
  uint32_t kaddr[KSTEPS];                  // K-fragment reads: row col, chunk 4s+grp
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) kaddr[s] = lds0 + 2 * T::chunk_off(col, 4 * s + grp);
  // V^T transpose reads: lane group grp takes keys 4grp .. 4grp+3 and
  // 16 + 4grp .. of a 32-key k-step, column 16db + col; its 16 lanes address
  // 4 rows x 16 columns. The swizzle repeats every 16 rows, so the second
  // read (16 rows on) and k-step ps (32 rows on) only add constants.
  uint32_t vaddr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    vaddr[db] = lds0 + 2 * (KSTAGES * TILE + T::elem_off(4 * grp + (col >> 2), 16 * db + 4 * (lane & 3)));
  auto lds_b128 = [](uint32_t addr) -> bf16x8 {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8 *>((uintptr_t)addr);
  };
  auto lds_tr = [](uint32_t addr) -> i16x4 {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(uintptr_t)addr);
  };

  // ---- staging of K/V tiles: global -> LDS directly --------------------------
  // global_load_lds_dwordx4 writes lane l's 16 bytes to LDS address
  // M0 + 16*l, so one instruction of a wavefront fills RPI consecutive tile
  // rows; each lane fetches the global chunk that the row's swizzle puts at its
  // position (a permutation within the row: still one contiguous row read).
  // Wavefront w's instruction i covers rows (i*NW + w)*RPI ...; the row
  // modulo 16 (which fixes the swizzle) does not depend on i. The loads are
  // issued from inline assembly so that the compiler does not make every LDS
  // read wait for them; before each barrier (after odd steps) a wavefront
  // waits for all of its loads (vmcnt(0)), and the barrier publishes them.
  constexpr int RPI = 64 / NC;                       // rows per instruction
  constexpr int INSTS = BN / (NW * RPI);             // instructions per wave per tile
  static_assert(INSTS >= 1 && (NW * RPI) % 16 == 0, "staging shape");
  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + b * p.kv_sb + hkv * p.kv_sh;
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + b * p.kv_sb + hkv * p.kv_sh;
  const int srow = wave * RPI + lane / NC;           // tile row of instruction 0
  const int scol = 8 * ((lane % NC) ^ T::swz(srow));   // logical column of this lane's chunk
  const int64_t tile_stride = (int64_t)BN * p.kv_ss;
  const int64_t istep_bytes = (int64_t)NW * RPI * p.kv_ss * 2;
  const uint32_t goff0 = (uint32_t)(((int64_t)srow * p.kv_ss + scol) * 2);
  const uint32_t dst0 = lds0 + 2 * wave * RPI * D;   // this wave's rows in K stage 0
  // M0 is saved and restored around the load: the compiler owns it.
  auto dma1 = [](uint32_t m0, uint32_t voff, const void *sbase) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
  };
  // Rows of storage tile kt of K (is_v = false) or V into LDS at dst (this
  // wave's first row of the stage); adj: its KV chunk's extra elements.
  auto dma = [&](int kt, int64_t adj, bool is_v, uint32_t dst) {
    const __bf16 *base = is_v ? vbase : kbase;
    const char *t_base = reinterpret_cast<const char *>(base + (int64_t)kt * tile_stride + adj);
    if (kt * BN + BN <= p.skv) {
#pragma unroll
      for (int i = 0; i < INSTS; ++i) dma1(dst + 2 * i * NW * RPI * D, goff0, t_base + i * istep_bytes);
    } else {
      // Ragged last tile: rows past the end read the last row (always masked).
      // Offsets count from the tile's own 64-bit base, so they stay below BN
      // row strides (< 2^31 bytes) however far the tile lies from the head's.
      const int last = p.skv - 1 - kt * BN;
#pragma unroll
      for (int i = 0; i < INSTS; ++i) {
        const uint32_t r = (uint32_t)min(srow + i * NW * RPI, last);
        dma1(dst + 2 * i * NW * RPI * D, (r * (uint32_t)p.kv_ss + (uint32_t)scol) * 2u, t_base);
      }
    }
  };
  // Boolean user mask: the row-bit words of the item's rows (tile 0), two
  // lanes per word of the wavefront's rows (rows past the item's last read
  // its last row); K stage st also receives tile kt's words.
  auto dma4 = [](uint32_t m0, uint32_t voff, const void *sbase) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, %3\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(sbase) : "memory");
  };
  const uint64_t *rb_item = nullptr;
  uint32_t rb_voff = 0;
  if constexpr (UMASK) {
    const int64_t bhm = (int64_t)(p.mb_batches > 1 ? b : 0) * p.mb_heads + (p.mb_heads > 1 ? head : 0);
    rb_item = p.mask_rowbits + bhm * p.mb_ktiles * p.sq + chunk * p.chunk_len + item_row0;
    rb_voff = (uint32_t)(min(wrow0 + (lane >> 1), item_rows - 1) * 8 + 4 * (lane & 1));
  }
  auto dma_k = [&](int kt, int64_t adj, int stage) {
    if constexpr (UMASK) {
      if (use_bits) dma4(lds0 + MB_OFF + (stage * NW + wave) * MB_WAVE, rb_voff, rb_item + (int64_t)kt * p.sq);
    }
    dma(kt, adj, false, dst0 + 2 * stage * TILE);
  };
  auto dma_v = [&](int kt, int64_t adj, int stage) { dma(kt, adj, true, dst0 + 2 * (KSTAGES + stage) * TILE); };
  // An additive mask with biases that all the item's heads share: its values
  // of tile kt for the item's rows into LDS stage st (two 1 KiB loads per
  // wavefront, four rows each, with the swizzle above; rows past the item's
  // last read its last row). A ragged tile is not staged (its reads stay per
  // lane, with the end test). In this mode every step ends with a barrier:
  // a step loads the next tile's values, which the next step reads.
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

  f32x4 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[qb][db][i] = 0.0f;
  // Running max of scale*log2(e)*s (may lag the true max) and this lane's
  // partial row sum (its quarter of the keys), per row block.
  float m_run[QB], l_part[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_part[qb] = 0.0f;
  }
  const float c = p.scale_log2;

  // Matrix-instruction slots of a step. Operand o (one LDS read, used by the
  // QB row blocks in consecutive slots): o in [0, NPV) is V^T of k-step
  // ps = o / DB, O^T block db = o % DB (two transpose reads); o in [NPV, NOP)
  // is K of k-step s = u / KB, key block kb = u % KB (u = o - NPV), so that
  // the products accumulating into one S^T block are KB*QB slots apart.
  constexpr int NPV = PSTEPS * DB;
  constexpr int NOP = NPV + KB * KSTEPS;
  constexpr int NSLOT = QB * NOP;
  constexpr int AHEAD = 2;                 // operand reads run this many operands ahead
  constexpr int NBUF = AHEAD + 1;
  // Operand o of a step whose K stage is KS and V stage VS.
  auto read_opnd = [&](auto ks_tag, auto vs_tag, auto o_tag) -> bf16x8 {
    constexpr int KS = decltype(ks_tag)::value, VS = decltype(vs_tag)::value;
    constexpr int o = decltype(o_tag)::value;
    if constexpr (o < NPV) {
      constexpr int ps = o / DB, db = o % DB;
      constexpr uint32_t off = 2 * (VS * TILE + 32 * D * ps);
      const i16x4 a0 = lds_tr(vaddr[db] + off);
      const i16x4 a1 = lds_tr(vaddr[db] + off + 2 * 16 * D);
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      constexpr int u = o - NPV, s = u / KB, kb = u % KB;
      return lds_b128(kaddr[s] + 2 * (KS * TILE + kb * 16 * D));
    }
  };
  // S^T of one tile from K stage 0 (prologue only).
  auto qk0 = [&](f32x4 (&sa)[QB][KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[qb][kb][i] = 0.0f;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8 a = lds_b128(kaddr[s] + 2 * kb * 16 * D);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sa[qb][kb] = mfma16(a, qf[qb][s], sa[qb][kb]);
      }
    }
  };
  // O^T += V^T P^T of one tile from V stage `stage` (epilogue only).
  auto pv = [&](int stage, const bf16x8 (&pf)[QB][PSTEPS]) {
#pragma unroll
    for (int ps = 0; ps < PSTEPS; ++ps)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t off = 2 * (stage * TILE + 32 * D * ps);
        const i16x4 a0 = lds_tr(vaddr[db] + off);
        const i16x4 a1 = lds_tr(vaddr[db] + off + 2 * 16 * D);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma16(a, pf[qb][ps], oacc[qb][db]);
      }
  };

  // ---- prologue ---------------------------------------------------------------
  // V stage 2 stands for "tile -1" in step 0 (its P is zero), so it must
  // not hold NaN bit patterns: clear it.
  {
    constexpr int VEC = TILE / 8;
    u32x4 *vlast = reinterpret_cast<u32x4 *>(smem + 2 * (KSTAGES + VSTAGES - 1) * TILE);
    for (int i = tid; i < VEC; i += NT) vlast[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // Scores and probabilities alternate between two register sets by step
  // parity: step j reads S^T(j) from set j%2 and writes S^T(j+1) into the
  // other; it reads P(j-1) from set (j+1)%2 and writes P(j) into set j%2.
  // (Sets are always chosen by a compile-time index: a runtime index would
  // put them in scratch memory.)
  f32x4 sbuf[2][QB][KB];
  bf16x8 pbuf[2][QB][PSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int ps = 0; ps < PSTEPS; ++ps)
#pragma unroll
      for (int e = 0; e < 8; ++e) pbuf[1][qb][ps][e] = (__bf16)0.0f;
  // Tiles j .. j+3 of the pipeline (step j masks tile j, loads V of j+1 and
  // K of j+3).
  TileRef t_cur{t0, kv_pos0, 0}, t_nx1{t0 + 1, kv_pos0, 0}, t_nx2{t0 + 2, kv_pos0, 0},
      t_nx3{t0 + 3, kv_pos0, 0};
  if constexpr (MKV) {
    if (ntiles > 0) t_cur = next_tile();
    if (ntiles > 1) t_nx1 = next_tile();
    if (ntiles > 2) t_nx2 = next_tile();
    if (ntiles > 3) t_nx3 = next_tile();
  }
  // Storage offset of a natural-order tile (merged chunks; 0 for one chunk).
  auto nat_adj = [&](int kt) { return ((int64_t)kt * BN >> p.kv.store_lg) * p.kv.cadj; };
  if (ntiles > 0) {
    dma_k(t_cur.kt, MKV ? t_cur.adj : nat_adj(t_cur.kt), 0);
    dma_v(t_cur.kt, MKV ? t_cur.adj : nat_adj(t_cur.kt), 0);
    if constexpr (ADDS_LDS) dma_adds(t_cur.kt, 0);
  }
  if (ntiles > 1) dma_k(t_nx1.kt, MKV ? t_nx1.adj : nat_adj(t_nx1.kt), 1);
  if (ntiles > 2) dma_k(t_nx2.kt, MKV ? t_nx2.adj : nat_adj(t_nx2.kt), 2);
  wait_vmem_all();
  __syncthreads();
  if (ntiles > 0) qk0(sbuf[0]);
  // The S^T product above reads K stage 0 as an odd "step -1" would: K of
  // tile 4 refills that stage in step 1.
  __syncthreads();
  // Boolean user mask: this lane's 16 bits of its row's word (keys
  // 16*kb + 4*grp + i at bit 16*grp + 4*kb + i) in K stage 0, row block 0;
  // beyond the reach of an immediate from LDS 0.
  uint32_t mbits = lds0 + MB_OFF + wave * MB_WAVE + col * 8 + 2 * grp;
  // This lane's row of a staged additive tile (stage 0, row block 0).
  uint32_t madds = lds0 + MB_OFF + (wrow0 + col) * BN * 4;

  // One step on tile j (J4 = j % 4): PV(j-1) and S^T(j+1) on the matrix
  // core, softmax of S^T(j) on the VALU, and K of tile j+3 and V of tile j+1
  // on their way into the rings. Slots are separated by scheduling fences so
  // that the interleave is the one written here.
  auto step = [&](auto j4_tag, int j) {
    constexpr int J4 = decltype(j4_tag)::value;
    constexpr int SET = J4 & 1;
    f32x4 (&sacc)[QB][KB] = sbuf[SET];
    f32x4 (&snext)[QB][KB] = sbuf[1 - SET];
    const bf16x8 (&pprev)[QB][PSTEPS] = pbuf[1 - SET];
    bf16x8 (&pcur)[QB][PSTEPS] = pbuf[SET];
    using KS = IC<(J4 + 1) % KSTAGES>;             // K of tile j+1
    using VS = IC<(J4 + VSTAGES - 1) % VSTAGES>;   // V of tile j-1
    // The next tile's staged mask values go out before the tiles' loads, so
    // that the wait after an even step counts only those (2 * INSTS) as
    // still in flight.
    if constexpr (ADDS_LDS) {
      if (j + 1 < ntiles) dma_adds(t0 + j + 1, (J4 + 1) & 1);
    }
    // K of tile j+3 replaces K of tile j-1 (read in step j-2); V of tile j+1
    // replaces V of tile j-3 (read in step j-2). In natural order the last
    // steps load the item's last tile again instead of branching around the
    // loads (those stages are never read; the epilogue waits for them).
    if constexpr (!MKV) {
      const int ktk = min(t0 + j + K_AHEAD, t0 + ntiles - 1);
      const int ktv = min(t0 + j + V_AHEAD, t0 + ntiles - 1);
      dma_k(ktk, nat_adj(ktk), (J4 + K_AHEAD) % KSTAGES);
      dma_v(ktv, nat_adj(ktv), (J4 + V_AHEAD) % VSTAGES);
    } else {
      if (j + K_AHEAD < ntiles) dma_k(t_nx3.kt, t_nx3.adj, (J4 + K_AHEAD) % KSTAGES);
      if (j + V_AHEAD < ntiles) dma_v(t_nx1.kt, t_nx1.adj, (J4 + V_AHEAD) % VSTAGES);
    }
    // Keep the operand bases opaque per step: otherwise the compiler hoists a
    // base-plus-stage address per stage out of the loop (several times the
    // registers) instead of folding the stage into the read's immediate.
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) asm volatile("" : "+v"(kaddr[s]));
#pragma unroll
    for (int db = 0; db < DB; ++db) asm volatile("" : "+v"(vaddr[db]));
    if constexpr (UMASK) asm volatile("" : "+v"(mbits), "+v"(madds));
    int kt = t0 + j;
    int64_t tile_plo = kv_pos0 + (int64_t)kt * BN;
    if constexpr (MKV) {
      kt = t_cur.kt;
      tile_plo = t_cur.base + (int64_t)kt * BN;
      t_cur = t_nx1;
      t_nx1 = t_nx2;
      t_nx2 = t_nx3;
      if (j + 4 < ntiles) t_nx3 = next_tile();
    }

    // Mask (diagonal or ragged tiles only): key 16*kb + 4*grp + i of the tile
    // is visible to a row iff it is <= that row's limit.
    bool need_mask = MKV ? (kt * BN + BN > p.skv) || (p.causal && tile_plo + BN - 1 > wave_qlo) : kt >= mask_from;
    if constexpr (DOCS) need_mask = need_mask || tile_plo < wave_ds;
    // (A user mask is applied to every tile, the range mask only where needed.)
    if (need_mask || UMASK) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (!UMASK || need_mask) {
          int lim = p.skv - 1 - kt * BN;
          if (p.causal) {
            const int64_t rel = qpos[qb] - tile_plo;
            lim = min(lim, (int)(rel < -1 ? -1 : (rel > BN ? BN : rel)));
          }
          const int t = lim - 4 * grp;
          if constexpr (DOCS) {
            // ... and >= the row's sequence start.
            const int tl = min(max(lo_key[qb] - kt * BN, 0), BN) - 4 * grp;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sacc[qb][kb][i] = (16 * kb + i > t || 16 * kb + i < tl) ? -INFINITY : sacc[qb][kb][i];
          } else {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sacc[qb][kb][i] = (16 * kb + i > t) ? -INFINITY : sacc[qb][kb][i];
          }
        }
        if constexpr (UMASK) {
          // ... and the user mask. Additive with biases: the 4 floats of
          // this lane's keys 16*kb + 4*grp .. +3 per block, every read issued
          // before any is used; in the ragged last tile keys past the end
          // read nothing (no bias on a score the range mask hid). Boolean, or
          // additive of 0 and hiding values only: the row bits.
          if (!use_bits) {
            const bool full = kt * BN + BN <= p.skv;
            // Additive: in the raw score's units (value / softmax_scale); a
            // value at or below kMaskHide hides the key.
            const float inv = 1.0f / p.scale;
            const float *mf = reinterpret_cast<const float *>(mrow[qb]);
            f32x4 a[KB];
            if (ADDS_LDS && stage_adds && full) {
              // The tile's values staged in LDS: row wrow0 + 16qb + col,
              // chunk 4kb + grp at its swizzled slot.
#pragma unroll
              for (int kb = 0; kb < KB; ++kb)
                a[kb] = *reinterpret_cast<const __attribute__((address_space(3))) f32x4 *>(
                    (uintptr_t)(madds + (J4 & 1) * MA_TILE + 16 * qb * BN * 4 + (((grp ^ col) ^ (4 * kb)) << 4)));
            } else {
#pragma unroll
              for (int kb = 0; kb < KB; ++kb) {
                const int k0 = kt * BN + 16 * kb + 4 * grp;
                if (full) {
                  a[kb] = *reinterpret_cast<const f32x4 *>(mf + k0);
                } else {
#pragma unroll
                  for (int i = 0; i < 4; ++i) a[kb][i] = k0 + i < p.skv ? mf[k0 + i] : 0.0f;
                }
              }
            }
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sacc[qb][kb][i] = a[kb][i] <= kMaskHide ? -INFINITY : fmaf(a[kb][i], inv, sacc[qb][kb][i]);
          } else {
            // Boolean: this row's 16 bits of the tile.
            const uint32_t w16 = *reinterpret_cast<const __attribute__((address_space(3))) uint16_t *>(
                (uintptr_t)(mbits + J4 * NW * MB_WAVE + 16 * qb * 8));
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                sacc[qb][kb][i] = keep_if_bit(sacc[qb][kb][i], w16, 4 * kb + i);
          }
        }
      }
    }

    // Probabilities of tile j against the current running max (no max is
    // taken on this path: see the check after the slots).
    bf16x8 opnd[NBUF];
    float mneg[QB], tsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      mneg[qb] = (m_run[qb] == -INFINITY) ? 0.0f : -m_run[qb];
      tsum[qb] = 0.0f;
    }
    // Probabilities of elements i, i+1 of key block kb of row block rq, in
    // two halves that the slots below issue apart: the exponentials, then
    // the row sum and the bf16 P^T operand. Pair (i, i+1) goes to elements
    // 4*(kb%2) + i, +1 of the operand of k-step kb/2: the key order of the
    // V^T reads.
    auto prob_exp = [&](int rq, int kb, int i, float mn, float (&x)[2]) {
      x[0] = fmaf(sacc[rq][kb][i], c, mn);
      x[1] = fmaf(sacc[rq][kb][i + 1], c, mn);
      x[0] = __builtin_amdgcn_exp2f(x[0]);
      x[1] = __builtin_amdgcn_exp2f(x[1]);
    };
    auto prob_keep = [&](int rq, int kb, int i, const float (&x)[2], float &sum) {
      // The row sum uses the unrounded fp32 probabilities (summing the bf16
      // values instead costs up to 2^-8 relative error in short rows).
      sum += x[0];
      sum += x[1];
      const bf16x2 t2 = __builtin_convertvector((f32x2){x[0], x[1]}, bf16x2);
      pcur[rq][kb >> 1][4 * (kb & 1) + i] = t2[0];
      pcur[rq][kb >> 1][4 * (kb & 1) + i + 1] = t2[1];
    };
    float xp[QB * KB * 2][2];   // a pair's probabilities between its two slots
    static_for<AHEAD>([&](auto o) { opnd[decltype(o)::value] = read_opnd(KS{}, VS{}, o); });
    static_for<NSLOT>([&](auto t_tag) {
      constexpr int t = decltype(t_tag)::value;
      constexpr int o = t / QB, qb = t % QB;
      if constexpr (qb == 0 && o + AHEAD < NOP)
        opnd[(o + AHEAD) % NBUF] = read_opnd(KS{}, VS{}, IC<o + AHEAD>{});
      // matrix instruction of slot t
      if constexpr (o < NPV) {
        constexpr int ps = o / DB, db = o % DB;
        oacc[qb][db] = mfma16(opnd[o % NBUF], pprev[qb][ps], oacc[qb][db]);
      } else {
        constexpr int u = o - NPV, s = u / KB, kb = u % KB;
        if constexpr (s == 0) {
          f32x4 z;
#pragma unroll
          for (int i = 0; i < 4; ++i) z[i] = 0.0f;
          snext[qb][kb] = mfma16(opnd[o % NBUF], qf[qb][s], z);
        } else {
          snext[qb][kb] = mfma16(opnd[o % NBUF], qf[qb][s], snext[qb][kb]);
        }
      }
      // The slot's vector work is issued after its matrix instruction.
      __builtin_amdgcn_sched_barrier(0);
      // Vector work: pair u of the NPAIR pairs (row block u / (KB*2), key
      // block (u / 2) % KB, elements 2(u%2), 2(u%2)+1) owns SPP slots from
      // slot SPP*u: the exponentials in the first, the sum and the bf16
      // conversion SPP/2 slots later. Every vector instruction thus shares a
      // slot that opens an operand (the slots with an LDS read), and no slot
      // holds more than four. (Measured against one slot per pair: 3-4 %
      // faster on the 32K shares, the same bits.)
      constexpr int NPAIR = QB * KB * 2;
      constexpr int SPP = NSLOT / NPAIR;
      static_assert(NSLOT == SPP * NPAIR && SPP % 2 == 0, "an even number of slots per pair");
      static_for<NPAIR>([&](auto u_tag) {
        constexpr int u = decltype(u_tag)::value;
        constexpr int rq = u / (KB * 2), kb = (u / 2) % KB, i = 2 * (u % 2);
        if constexpr (SPP * u == t) prob_exp(rq, kb, i, mneg[rq], xp[u]);
        if constexpr (SPP * u + SPP / 2 == t) prob_keep(rq, kb, i, xp[u], tsum[rq]);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // Pin P(j) and the tile sums to the slots above: without a use here the
    // compiler sinks the exponentials past the branch below, away from the
    // products they are meant to overlap.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int ps = 0; ps < PSTEPS; ++ps) asm volatile("" ::"v"(pcur[qb][ps]));
      asm volatile("" ::"v"(tsum[qb]));
    }

    // The running max is only a reference point: the probabilities above are
    // exact as long as none overflows. While every lane's partial tile sum
    // stays at most 2^16 (so every probability does), they are kept.
    // Otherwise -- the first tile of a row (no reference yet), a score more
    // than 16 (log2) above the reference, or a non-finite sum -- the row max
    // is taken, O and the row sum are rescaled to it (after this step's
    // PV(j-1) products, which used the old reference) and the tile's
    // probabilities are recomputed.
    bool redo = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) redo = redo || !(tsum[qb] <= kSumLimit) || m_run[qb] == -INFINITY;
    if (__any(redo)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float m = sacc[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, sacc[qb][kb][i]);
        const float mr = quad_max(m) * c;
        const float m_new = fmaxf(m_run[qb], mr);
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[qb][db][i] *= alpha;
        l_part[qb] *= alpha;
        m_run[qb] = m_new;
        const float mn = (m_new == -INFINITY) ? 0.0f : -m_new;
        tsum[qb] = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            float x[2];
            prob_exp(qb, kb, i, mn, x);
            prob_keep(qb, kb, i, x, tsum[qb]);
          }
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_part[qb] += tsum[qb];
    if constexpr (J4 & 1) {
      wait_vmem_all();   // this wave's rows of every tile loaded so far are in LDS
      __syncthreads();
    } else if constexpr (ADDS_LDS) {
      if (stage_adds) {
        // The next tile's mask values (older than this step's 2 * INSTS
        // tile loads, which may stay in flight) are in LDS.
        __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * INSTS));
        __syncthreads();
      }
    }
  };

  for (int j = 0; j < ntiles; j += UNROLL) {
    step(IC<0>{}, j);
    if (j + 1 < ntiles) step(IC<1>{}, j + 1);
    if (j + 2 < ntiles) step(IC<2>{}, j + 2);
    if (j + 3 < ntiles) step(IC<3>{}, j + 3);
  }
  // The last tile's PV product. Its V tile was loaded in the step before the
  // last one (or before step 0), and whichever of those two steps is odd
  // published it.
  if (ntiles > 0) {
    const int last = ntiles - 1;
    if (last & 1) pv(last % VSTAGES, pbuf[1]);
    else pv(last % VSTAGES, pbuf[0]);
  }

  wait_vmem_all();   // the repeated loads of the last steps land before the workgroup ends

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = quad_sum(l_part[qb]);
    if (!qvalid[qb]) continue;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    __bf16 *op = static_cast<__bf16 *>(p.out) + b * p.o_sb + head * p.o_sh + chunk * p.o_cadj +
                 (int64_t)local_row[qb] * p.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      bf16x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(oacc[qb][db][e] * inv);
      *reinterpret_cast<bf16x4 *>(op + 16 * db + 4 * grp) = o4;
    }
    if (grp == 0) {
      const float lse = l > 0.0f ? (m_run[qb] + __log2f(l)) * kLn2 : -INFINITY;
      p.lse[((int64_t)b * p.hq + head) * p.sq + local_row[qb]] = lse;
    }
  }
}

// Launch of one mode's instantiation (rb = 32-row blocks per head of a work
// item: 2, 4 or 8 by the GQA group size).
template <int D, int MODE>
int launch_fwd_mode(const FwdParams &p, void *stream) {
  const int64_t grid = fwd_grid_size(p);
  if (grid == 0) return 0;
  const int rb = NW / p.heads_per_item;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (rb) {
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<D, 2, MODE>), dim3(grid), dim3(NT), 0, s, p); break;
    case 4: hipLaunchKernelGGL((fwd_bf16_kernel<D, 4, MODE>), dim3(grid), dim3(NT), 0, s, p); break;
    case 8: hipLaunchKernelGGL((fwd_bf16_kernel<D, 8, MODE>), dim3(grid), dim3(NT), 0, s, p); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

template <int MODE>
int launch_fwd_mode_d(const FwdParams &p, int head_dim, void *stream) {
  if (head_dim == 128) return launch_fwd_mode<128, MODE>(p, stream);
  if (head_dim == 64) return launch_fwd_mode<64, MODE>(p, stream);
  return (int)hipErrorInvalidValue;
}

}  // namespace
}  // namespace cpattn
