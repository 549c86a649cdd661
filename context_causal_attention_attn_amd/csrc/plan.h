// Internal host/device contract of the share kernels: the validated share
// geometry, the forward tile schedule and the kernel parameter blocks.
//
// The schedule follows the causal structure of a CP share
// ("新流程 CP 多通信模式迁移设计方案" §8: every query row carries its own global
// position; "HyperModels 新 Trainer Context Parallel 接入设计方案" §4.4: each
// Head-Tail segment keeps its own global interval). A work item is one tile of
// query rows of one chunk, for a pack of query heads that share one KV head;
// it visits only the KV tiles its rows can see.
#pragma once

#include <stdint.h>

#include "cp_attn.h"

namespace cpattn {

constexpr int kMaxQChunks = CP_ATTN_MAX_Q_CHUNKS;
// Additive user-mask values at or below this hide their key, like -inf.
constexpr float kMaskHide = CP_ATTN_MASK_HIDE;
constexpr int kMaxKvChunks = CP_ATTN_MAX_KV_CHUNKS;

// Packed-sequence boundaries a share can meet (global positions, ascending).
// Query row q's sequence starts at the last bound <= q (none: -inf); key k's
// sequence ends before the first bound > k (none: +inf). The host keeps every
// bound that can decide either for this share.
constexpr int kMaxDocBounds = CP_ATTN_MAX_DOC_BOUNDS;
struct DocBounds {
  int32_t n;
  int64_t pos[kMaxDocBounds];
};

// KV chunk table as the kernels see it: chunk c holds key rows
// [c*len, (c+1)*len) at global positions pos[c] .. pos[c]+len-1. One chunk
// (len = skv) is the natural order. With several, len is a multiple of every
// kernel's key tile, so a key tile lies in one chunk and its positions are
// consecutive: row j of chunk c sits at (pos[c] - c*len) + j.
struct KvChunks {
  int32_t n;
  int32_t len;
  int64_t pos[kMaxKvChunks];
  // Storage: key row j sits at j * row stride + s(j) * cadj elements from its
  // head's base, s(j) its storage chunk: j >> store_lg when store_lg < 31
  // (the host merged a table of consecutive, equally strided chunks of
  // 2^store_lg rows into one chunk), else j / len (cadj = chunk stride - chunk
  // length * row stride; 0 when the rows follow on).
  int64_t cadj;
  int32_t store_lg;
};

// ---------------------------------------------------------------------------
// Forward, bf16 MFMA kernel
// ---------------------------------------------------------------------------
// Keys per KV tile staged in LDS, query rows per wavefront and wavefronts per
// workgroup of the forward kernel.
constexpr int kFwdBlockKV = 64;
constexpr int kFwdWaveRows = 32;
constexpr int kFwdWaves = 8;

struct FwdParams {
  const void *q;
  const void *k;
  const void *v;
  void *out;
  float *lse;
  int64_t q_sb, q_sh, q_ss;     // element strides of q (batch, head, row)
  int64_t kv_sb, kv_sh, kv_ss;  // of k and v
  int64_t o_sb, o_sh, o_ss;     // of out
  int64_t q_cadj, o_cadj;       // extra elements per query chunk index (chunk strides; 0: rows follow on)
  KvChunks kv;                  // positions of the key rows
  DocBounds docs;               // packed-sequence boundaries (n = 0: none)
  const uint8_t *mask;          // user attention mask (NULL: none), [b][h][row][key]
  int64_t m_sb, m_sh, m_ss;     // its byte strides (batch, head, row)
  int32_t mask_add;             // 0: bytes (nonzero = may attend); 1: float32 added to the scaled score
  int32_t hq, hkv, group;       // group = hq / hkv
  int32_t heads_per_item;       // query heads of one KV group packed in a work item
  int32_t n_head_packs;         // batch * hq / heads_per_item
  int32_t sq, skv;
  int32_t chunk_len;            // rows per query chunk
  int32_t n_q_chunks;
  int32_t tiles_per_chunk;      // ceil(chunk_len / block rows)
  int32_t causal;
  float scale;                  // softmax_scale
  float scale_log2;             // softmax_scale * log2(e)
  // Query chunks in scheduling order (latest global position first, so the
  // longest causal rows start first); chunk_idx maps back to local order.
  int64_t chunk_pos[kMaxQChunks];
  int32_t chunk_idx[kMaxQChunks];
  // A user mask as row bits (bf16; NULL otherwise): word
  // [(bm * mb_heads + hm) * mb_ktiles + kt][row], bit 16*g + 4*kb + i for key
  // 64*kt + 16*kb + 4*g + i (see launch_mask_rowbits), 1 where the key may
  // be attended. An additive mask's table is used only while *mask_flag is 0:
  // every value then is 0 or hides its key, and the bits say everything.
  const uint64_t *mask_rowbits;
  const uint32_t *mask_flag;
  int32_t mb_batches, mb_heads, mb_ktiles;
};

// Geometry derived from a validated descriptor.
struct Share {
  int32_t n_q_chunks;
  int64_t chunk_len;
  int64_t chunk_pos[kMaxQChunks];   // local chunk order
  int32_t order[kMaxQChunks];       // chunk indices, latest position first
};

int32_t make_share(const cp_attn_desc *d, Share *s);
int32_t collect_doc_bounds(const cp_attn_desc *d, DocBounds *out);

// Heads packed per work item of the query-stationary kernels (forward, dQ)
// for a GQA group of size g: a divisor of g, at most 4.
inline int item_heads(int g) { return (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1; }
// Query rows per forward work item (per head).
inline int fwd_block_rows(int g) { return kFwdWaveRows * (kFwdWaves / item_heads(g)); }

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
// The backward runs two main kernels. The key-stationary one owns a tile of
// kBwdBlockKV keys of one KV head, keeps that tile's dK/dV in registers and
// visits every query tile (of every head of the GQA group, of every chunk)
// that can see one of its keys. The query-stationary one owns a query tile
// (scheduled exactly like the forward) and accumulates its dQ over the keys
// it can see.
constexpr int kBwdBlockKV = 128;
constexpr int kBwdBlockQ = 64;
// Keys per 256-thread workgroup of the backward's column-bit pass.
constexpr int kMaskBitsBlockKeys = 1024;
constexpr int kDqBlockKV = 64;    // keys per tile of the query-stationary dQ kernel
constexpr int kDqWaveRows = 32;   // query rows per wavefront of the dQ kernel
constexpr int kDqWaves = 8;       // wavefronts per dQ workgroup
static_assert(CP_ATTN_KV_CHUNK_ALIGN % kBwdBlockKV == 0 && CP_ATTN_KV_CHUNK_ALIGN % kDqBlockKV == 0 &&
                  CP_ATTN_KV_CHUNK_ALIGN % kFwdBlockKV == 0,
              "a key tile must not straddle two KV chunks");
// Query rows per dQ work item (per head).
inline int dq_block_rows(int g) { return kDqWaveRows * (kDqWaves / item_heads(g)); }

struct BwdParams {
  const void *q;
  const void *k;
  const void *v;
  const void *out;
  const void *dout;
  const float *lse;
  float *delta;                 // workspace [B, Hq, Sq]: rowsum(dO o O) (fp32 kernels), its negative (bf16 kernels)
  float *lse2;                  // workspace [B, Hq, Sq]: LSE * log2(e), +inf for rows with no visible key
  void *dq;
  float *dk;                    // [B, Hkv, Skv, D]
  float *dv;
  int64_t q_sb, q_sh, q_ss;
  int64_t kv_sb, kv_sh, kv_ss;
  int64_t o_sb, o_sh, o_ss;     // out, dout and dq
  int64_t q_cadj, o_cadj;       // extra elements per query chunk index (chunk strides; 0: rows follow on)
  KvChunks kv;                  // positions of the key rows
  DocBounds docs;               // packed-sequence boundaries (n = 0: none)
  const uint8_t *mask;          // user attention mask (NULL: none), [b][h][row][key]
  int64_t m_sb, m_sh, m_ss;     // its byte strides (batch, head, row)
  int32_t mask_add;             // 0: bytes (nonzero = may attend); 1: float32 added to the scaled score
  int32_t batch, hq, hkv, group;
  int32_t sq, skv;
  int32_t chunk_len, n_q_chunks;
  int32_t causal;
  float scale;
  float scale_log2;
  int64_t chunk_pos[kMaxQChunks];   // local chunk order
  // Schedule of the query-stationary dQ kernel (longest first, like the forward's).
  int32_t heads_per_item, n_head_packs, tiles_per_chunk;
  int64_t lpt_chunk_pos[kMaxQChunks];
  int32_t lpt_chunk_idx[kMaxQChunks];
  // Key tiles (of kBwdBlockKV keys) the key-stationary kernel runs on:
  // [kt0, kt1). Keys outside them are seen by no local query (before the
  // first local row's sequence, after the last local row) and get zero
  // dK/dV from a plain fill instead.
  int32_t kt0, kt1;
  // Each key tile's query steps are split over kv_parts workgroups (1, 2, 4
  // or 8); part 0 writes dK/dV, parts 1.. write fp32 partials to kv_partial
  // ([kv_parts-1][tile][batch*hkv][dk, dv][kBwdBlockKV][D]), which a
  // reduction kernel adds into dK/dV.
  int32_t kv_parts;
  float *kv_partial;
  // A user mask as bits, for the key-stationary bf16 kernel (NULL: none, or
  // the fp32 kernels; an additive mask's only while *mask_flag is 0): word
  // [(bm * mb_heads + hm) * n_q_chunks * mb_tpc + c * mb_tpc + t][key] holds
  // the 64 rows of query tile t of chunk c, bit 16*g + 4*rb + i for row
  // 16*rb + 4*g + i of the tile (1: the key may be attended; 0 also past the
  // chunk end); bm, hm index the mask's batch and head (0 where it broadcasts).
  uint64_t *mask_bits;
  int32_t mb_batches, mb_heads, mb_tpc;
  // The same mask as row bits for the query-stationary kernel (FwdParams::
  // mask_rowbits' layout; NULL: none), and FwdParams::mask_flag.
  const uint64_t *mask_rowbits;
  const uint32_t *mask_flag;
  int32_t mb_ktiles;
};

void fill_fwd_params(const cp_attn_desc *d, const Share &s, FwdParams *p);
// allow_split = false keeps every key tile in one workgroup (kv_parts = 1).
void fill_bwd_params(const cp_attn_desc *d, const Share &s, BwdParams *p, bool allow_split = true);
// Bytes of the backward's per-row statistics (-Delta and LSE*log2e, each on a
// 256-byte boundary), the part of the workspace every backward needs.
// Workspace bytes of the backward: the per-row statistics, the partial dK/dV
// of split key tiles (allow_split) and a user mask's bit tables and flag.
size_t bwd_workspace_bytes(const cp_attn_desc *d, bool allow_split);
// cp_attn_bwd_timed with the choice of splitting key tiles (the no-alloc
// entry point passes allow_split = false: its scratch holds no partials).
int32_t bwd_run(const cp_attn_desc *d, const void *q, const void *k, const void *v, const void *out,
                const float *lse, const void *dout, void *dq, float *dk, float *dv, void *workspace,
                size_t workspace_bytes, void *stream, void *const *events, int32_t n_events, bool allow_split);
int64_t fwd_grid_size(const FwdParams &p);

// Launchers (defined with their kernels); return a hipError_t as int.
int launch_fwd_bf16(const FwdParams &p, int head_dim, void *stream);
// Writes a mask [batches][heads][sq][skv] (byte strides m_sb, m_sh, m_ss;
// batches/heads 1 where it broadcasts; bytes, or float32 values when
// additive) as row bits (FwdParams::mask_rowbits): batches * heads *
// ceil(skv/64) * sq 64-bit words. For an additive mask it also sets *flag
// to 0 when every value is 0 or at most kMaskHide, else to nonzero.
int launch_mask_rowbits(const uint8_t *mask, int64_t m_sb, int64_t m_sh, int64_t m_ss, int32_t batches,
                        int32_t heads, int32_t sq, int32_t skv, bool additive, uint64_t *bits, uint32_t *flag,
                        void *stream);
// Per-mode instantiations (0: natural order, 1: KV chunk table, 2: packed
// sequences, 3: user mask), each compiled in a file of its own.
int launch_fwd_bf16_m0(const FwdParams &p, int head_dim, void *stream);
int launch_fwd_bf16_m1(const FwdParams &p, int head_dim, void *stream);
int launch_fwd_bf16_m2(const FwdParams &p, int head_dim, void *stream);
int launch_fwd_bf16_m3(const FwdParams &p, int head_dim, void *stream);
int launch_bwd_dq_m0(const BwdParams &p, int head_dim, void *stream);
int launch_bwd_dq_m1(const BwdParams &p, int head_dim, void *stream);
int launch_bwd_dq_m2(const BwdParams &p, int head_dim, void *stream);
int launch_bwd_dq_m3(const BwdParams &p, int head_dim, void *stream);
// dK/dV: 0 plain (natural order or a KV chunk table), 1 packed sequences, 2 user mask.
int launch_bwd_dkdv_m0(const BwdParams &p, int head_dim, void *stream);
int launch_bwd_dkdv_m1(const BwdParams &p, int head_dim, void *stream);
int launch_bwd_dkdv_m2(const BwdParams &p, int head_dim, void *stream);
int launch_fwd_fp32(const FwdParams &p, int head_dim, void *stream);
// `events` is NULL or four hipEvent_t recorded at the phase boundaries.
int launch_bwd_bf16(const BwdParams &p, int head_dim, void *stream, void *const *events);
int launch_bwd_fp32(const BwdParams &p, int head_dim, void *stream, void *const *events);

}  // namespace cpattn
