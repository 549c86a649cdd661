// C ABI of the CP attention share: descriptor validation, share geometry,
// workspace sizing, the forward tile schedule, and dispatch to the kernels.
//
// Fail-fast policy ("新流程 CP 多通信模式迁移设计方案" §13.2 and
// "HyperModels 新 Trainer Context Parallel 接入设计方案" §4.4): every check runs
// on the host before any device work is enqueued, and a failed check returns
// a negative status with no buffer touched. Nothing falls back to a slower or
// different computation.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "cp_attn.h"
#include "plan.h"

namespace cpattn {

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int32_t elem_bytes(int32_t dtype) { return dtype == CP_ATTN_BF16 ? 2 : 4; }

int32_t make_share(const cp_attn_desc *d, Share *s) {
  s->n_q_chunks = d->n_q_chunks;
  s->chunk_len = d->sq_local / d->n_q_chunks;
  for (int c = 0; c < d->n_q_chunks; ++c) {
    s->chunk_pos[c] = d->q_chunk_pos[c];
    s->order[c] = c;
  }
  // Latest global position first: under the causal mask those rows see the
  // most keys, so their work items are dispatched first (longest first).
  std::stable_sort(s->order, s->order + d->n_q_chunks,
                   [&](int a, int b) { return s->chunk_pos[a] > s->chunk_pos[b]; });
  return CP_ATTN_OK;
}

// The sequence boundaries that can decide anything for this share: per query
// chunk [lo, hi], the last start <= lo (its first rows' sequence), every start
// in (lo, hi], and the first start > hi (where the sequence of the chunk's last
// rows, and of every key visible to the chunk, ends). A query's sequence start
// is the last kept bound <= it; a key visible to some local query ends its
// sequence at the first kept bound > it (keys of sequences no local row
// touches are cut off by the query side). Ascending, duplicates dropped.
int32_t collect_doc_bounds(const cp_attn_desc *d, DocBounds *out) {
  out->n = 0;
  if (d->n_docs <= 0) return CP_ATTN_OK;
  const int64_t *b = d->doc_starts, *e = d->doc_starts + d->n_docs;
  const int64_t L = d->sq_local / d->n_q_chunks;
  std::vector<int64_t> keep;
  for (int c = 0; c < d->n_q_chunks; ++c) {
    if (L == 0) break;
    const int64_t lo = d->q_chunk_pos[c], hi = lo + L - 1;
    const int64_t *first_after_lo = std::upper_bound(b, e, lo);
    if (first_after_lo != b) keep.push_back(*(first_after_lo - 1));
    const int64_t *first_after_hi = std::upper_bound(b, e, hi);
    keep.insert(keep.end(), first_after_lo, first_after_hi);
    if (first_after_hi != e) keep.push_back(*first_after_hi);
  }
  std::sort(keep.begin(), keep.end());
  keep.erase(std::unique(keep.begin(), keep.end()), keep.end());
  if ((int64_t)keep.size() > kMaxDocBounds) return CP_ATTN_ERR_UNSUPPORTED;
  out->n = (int32_t)keep.size();
  for (size_t i = 0; i < keep.size(); ++i) out->pos[i] = keep[i];
  return CP_ATTN_OK;
}

static int32_t validate(const cp_attn_desc *d) {
  if (!d) return CP_ATTN_ERR_NULL_PTR;
  if (d->abi_version != CP_ATTN_ABI_VERSION) return CP_ATTN_ERR_ABI;
  if (d->dtype != CP_ATTN_BF16 && d->dtype != CP_ATTN_FP32) return CP_ATTN_ERR_UNSUPPORTED;
  if (d->batch < 1 || d->hq < 1 || d->hkv < 1 || d->hq % d->hkv != 0) return CP_ATTN_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return CP_ATTN_ERR_UNSUPPORTED;
  if (d->sq_local < 0 || d->skv < 0) return CP_ATTN_ERR_BAD_SHAPE;
  if (d->sq_local > INT32_MAX || d->skv > INT32_MAX) return CP_ATTN_ERR_UNSUPPORTED;
  if (d->layout != CP_ATTN_LAYOUT_CONTIGUOUS && d->layout != CP_ATTN_LAYOUT_HEAD_TAIL &&
      d->layout != CP_ATTN_LAYOUT_CHUNKED)
    return CP_ATTN_ERR_BAD_LAYOUT;
  if (d->n_q_chunks < 1 || d->n_q_chunks > CP_ATTN_MAX_Q_CHUNKS) return CP_ATTN_ERR_BAD_LAYOUT;
  if (d->layout == CP_ATTN_LAYOUT_CONTIGUOUS && d->n_q_chunks != 1) return CP_ATTN_ERR_BAD_LAYOUT;
  if (d->layout == CP_ATTN_LAYOUT_HEAD_TAIL && d->n_q_chunks != 2) return CP_ATTN_ERR_BAD_LAYOUT;
  if (!d->q_chunk_pos || !d->kv_chunk_pos) return CP_ATTN_ERR_NULL_PTR;
  if (d->n_kv_chunks < 1 || d->n_kv_chunks > CP_ATTN_MAX_KV_CHUNKS) return CP_ATTN_ERR_BAD_LAYOUT;
  if (d->sq_local % d->n_q_chunks != 0 || d->skv % d->n_kv_chunks != 0) return CP_ATTN_ERR_BAD_SHAPE;
  // Several KV chunks: no key tile of any kernel may straddle two of them.
  if (d->n_kv_chunks > 1 && (d->skv / d->n_kv_chunks) % CP_ATTN_KV_CHUNK_ALIGN != 0)
    return CP_ATTN_ERR_UNSUPPORTED;
  if (d->causal != 0 && d->causal != 1) return CP_ATTN_ERR_BAD_SHAPE;
  if (!isfinite(d->softmax_scale) || !(d->softmax_scale > 0.0f)) return CP_ATTN_ERR_BAD_SHAPE;
  // Positions: non-negative, far from overflow, and the query chunks disjoint.
  const int64_t L = d->sq_local / d->n_q_chunks;
  const int64_t lim = (int64_t)1 << 60;
  for (int c = 0; c < d->n_q_chunks; ++c) {
    const int64_t p = d->q_chunk_pos[c];
    if (p < 0 || p > lim) return CP_ATTN_ERR_BAD_POSITIONS;
    for (int e = 0; e < c; ++e) {
      const int64_t o = d->q_chunk_pos[e];
      if (L > 0 && p < o + L && o < p + L) return CP_ATTN_ERR_BAD_POSITIONS;
    }
  }
  const int64_t Lkv = d->skv / d->n_kv_chunks;
  for (int c = 0; c < d->n_kv_chunks; ++c) {
    const int64_t p = d->kv_chunk_pos[c];
    if (p < 0 || p > lim) return CP_ATTN_ERR_BAD_POSITIONS;
    for (int e = 0; e < c; ++e) {
      const int64_t o = d->kv_chunk_pos[e];
      if (Lkv > 0 && p < o + Lkv && o < p + Lkv) return CP_ATTN_ERR_BAD_POSITIONS;
    }
  }
  // Packed sequences: causal only, natural key order, ascending starts.
  if (d->n_docs < 0) return CP_ATTN_ERR_BAD_SHAPE;
  if (d->n_docs > 0) {
    if (!d->doc_starts) return CP_ATTN_ERR_NULL_PTR;
    if (!d->causal || d->n_kv_chunks != 1) return CP_ATTN_ERR_UNSUPPORTED;
    for (int i = 0; i < d->n_docs; ++i) {
      const int64_t p = d->doc_starts[i];
      if (p < 0 || p > lim || (i > 0 && p <= d->doc_starts[i - 1])) return CP_ATTN_ERR_BAD_POSITIONS;
    }
    DocBounds db;
    if (collect_doc_bounds(d, &db) != CP_ATTN_OK) return CP_ATTN_ERR_UNSUPPORTED;
  }
  // User mask: natural key order, no packed sequences, 4-byte words.
  if (d->attn_mask) {
    if (d->n_kv_chunks != 1 || d->n_docs > 0) return CP_ATTN_ERR_UNSUPPORTED;
    if (d->mask_additive != 0 && d->mask_additive != 1) return CP_ATTN_ERR_BAD_SHAPE;
    const int64_t al = d->mask_additive ? 16 : 4;
    if (reinterpret_cast<uintptr_t>(d->attn_mask) % al) return CP_ATTN_ERR_ALIGNMENT;
    for (int i = 0; i < 3; ++i) {
      if (d->mask_strides[i] < 0) return CP_ATTN_ERR_BAD_SHAPE;
      if (d->mask_strides[i] % al != 0) return CP_ATTN_ERR_ALIGNMENT;
    }
    // The key-stationary kernel addresses 64 mask rows with 32-bit offsets.
    if (d->mask_strides[2] >= ((int64_t)1 << 25)) return CP_ATTN_ERR_BAD_SHAPE;
  }
  // Strides: non-negative, and every row start 16-byte aligned given an
  // aligned base pointer (the kernels move 16-byte vectors along the dim).
  const int64_t vec = 16 / elem_bytes(d->dtype);
  const int64_t *all[3] = {d->q_strides, d->kv_strides, d->o_strides};
  for (auto st : all)
    for (int i = 0; i < 3; ++i) {
      if (st[i] < 0) return CP_ATTN_ERR_BAD_SHAPE;
      if (st[i] % vec != 0) return CP_ATTN_ERR_ALIGNMENT;
    }
  // Row strides below 2^24 elements: the kernels address rows within a tile
  // with 32-bit byte offsets from a per-tile base.
  for (auto st : all)
    if (st[2] >= (int64_t(1) << 24)) return CP_ATTN_ERR_UNSUPPORTED;
  // Chunk strides: non-negative element counts that keep rows 16-byte aligned.
  for (int i = 0; i < 3; ++i) {
    if (d->chunk_strides[i] < 0) return CP_ATTN_ERR_BAD_SHAPE;
    if (d->chunk_strides[i] % vec != 0) return CP_ATTN_ERR_ALIGNMENT;
  }
  return CP_ATTN_OK;
}

// Extra elements per chunk index when a chunk stride is given: chunk c's row
// t sits at c * stride + t * row stride instead of (c * len + t) * row stride.
static int64_t chunk_adj(int64_t chunk_stride, int64_t len, int64_t row_stride) {
  return chunk_stride == 0 ? 0 : chunk_stride - len * row_stride;
}

static void fill_kv_chunks(const cp_attn_desc *d, KvChunks *kv) {
  kv->n = d->n_kv_chunks;
  kv->len = (int32_t)(d->skv / d->n_kv_chunks);
  for (int c = 0; c < d->n_kv_chunks; ++c) kv->pos[c] = d->kv_chunk_pos[c];
  kv->cadj = chunk_adj(d->chunk_strides[1], kv->len, d->kv_strides[2]);
  kv->store_lg = 31;
  // Chunks that follow each other in position order with power-of-two
  // lengths (e.g. the blocks a Ulysses all-to-all delivers) are one chunk in
  // natural order for the kernels; only their storage offset stays per chunk.
  bool natural = kv->n > 1 && (kv->len & (kv->len - 1)) == 0;
  for (int c = 1; natural && c < kv->n; ++c) natural = kv->pos[c] == kv->pos[0] + (int64_t)c * kv->len;
  if (natural) {
    int lg = 0;
    while ((1 << lg) < kv->len) ++lg;
    kv->store_lg = lg;
    kv->n = 1;
    kv->len = (int32_t)d->skv;
  }
}

// A user mask's row bits (FwdParams::mask_rowbits; bf16), 256-byte aligned:
// one 64-bit word per mask batch/head, 64-key tile and local row.
static size_t mask_rowbits_table_bytes(const cp_attn_desc *d) {
  if (!d->attn_mask || d->dtype != CP_ATTN_BF16) return 0;
  const size_t words = (size_t)(d->mask_strides[0] ? d->batch : 1) * (d->mask_strides[1] ? d->hq : 1) *
                       (size_t)((d->skv + 63) / 64) * (size_t)d->sq_local;
  return (words * 8 + 255) & ~(size_t)255;
}

// The row bits and, for an additive mask, FwdParams::mask_flag in 256 more
// bytes after them.
static size_t mask_rowbits_bytes(const cp_attn_desc *d) {
  const size_t t = mask_rowbits_table_bytes(d);
  return t > 0 && d->mask_additive ? t + 256 : t;
}
static const uint32_t *mask_flag_at(const uint64_t *rowbits, const cp_attn_desc *d) {
  if (!d->mask_additive) return nullptr;
  return reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(rowbits) + mask_rowbits_table_bytes(d));
}

// A launch's grid counts its work-items in 32 bits.
static bool fits_grid(int64_t blocks, int64_t threads) { return blocks * threads <= (int64_t)UINT32_MAX; }

// The row-bit pass runs one thread per word, 256 per workgroup.
static bool mask_rowbits_grid_ok(const cp_attn_desc *d) {
  return fits_grid((int64_t)(mask_rowbits_bytes(d) / 8 + 255) / 256, 256);
}

void fill_fwd_params(const cp_attn_desc *d, const Share &s, FwdParams *p) {
  memset(p, 0, sizeof(*p));
  collect_doc_bounds(d, &p->docs);
  p->mask = static_cast<const uint8_t *>(d->attn_mask);
  p->mask_add = d->mask_additive;
  p->m_sb = d->mask_strides[0]; p->m_sh = d->mask_strides[1]; p->m_ss = d->mask_strides[2];
  p->mb_batches = d->mask_strides[0] ? d->batch : 1;
  p->mb_heads = d->mask_strides[1] ? d->hq : 1;
  p->mb_ktiles = (int32_t)((d->skv + 63) / 64);
  p->q_sb = d->q_strides[0]; p->q_sh = d->q_strides[1]; p->q_ss = d->q_strides[2];
  p->kv_sb = d->kv_strides[0]; p->kv_sh = d->kv_strides[1]; p->kv_ss = d->kv_strides[2];
  p->o_sb = d->o_strides[0]; p->o_sh = d->o_strides[1]; p->o_ss = d->o_strides[2];
  fill_kv_chunks(d, &p->kv);
  p->q_cadj = chunk_adj(d->chunk_strides[0], d->sq_local / d->n_q_chunks, d->q_strides[2]);
  p->o_cadj = chunk_adj(d->chunk_strides[2], d->sq_local / d->n_q_chunks, d->o_strides[2]);
  p->hq = d->hq;
  p->hkv = d->hkv;
  p->group = d->hq / d->hkv;
  p->heads_per_item = item_heads(p->group);
  p->n_head_packs = d->batch * (d->hq / p->heads_per_item);
  p->sq = (int32_t)d->sq_local;
  p->skv = (int32_t)d->skv;
  p->chunk_len = (int32_t)s.chunk_len;
  p->n_q_chunks = s.n_q_chunks;
  const int rows = fwd_block_rows(p->group);
  p->tiles_per_chunk = (int32_t)((s.chunk_len + rows - 1) / rows);
  p->causal = d->causal;
  p->scale = d->softmax_scale;
  p->scale_log2 = d->softmax_scale * 1.4426950408889634f;
  for (int i = 0; i < s.n_q_chunks; ++i) {
    p->chunk_idx[i] = s.order[i];
    p->chunk_pos[i] = s.chunk_pos[s.order[i]];
  }
}

// Workgroups that run at once on the chip for the key-stationary dK/dV kernel
// (one per compute unit: its LDS use leaves room for one): MI355X's 256 CUs.
constexpr int kDkdvSlots = 256;

// How many workgroups share each key tile of the dK/dV kernel. A key tile's
// work is the query steps (64-row query tiles of every head of its GQA group)
// that can see it; under the causal mask early key tiles have many times the
// steps of late ones. With few KV heads (a Ulysses share has one) there are
// few workgroups, and the longest tiles decide the kernel's time. The launch
// order is tile by tile, longest first; this simulates that list schedule on
// the chip's workgroup slots for 1, 2, 4 and 8 parts per tile (each part
// also pays a fixed start-up and, beyond the first, an fp32 partial written
// and reduced) and keeps the fastest.
static int32_t dkdv_parts(const cp_attn_desc *d, const Share &s, int kt0, int kt1) {
  if (d->dtype != CP_ATTN_BF16 || kt1 <= kt0 || s.chunk_len == 0) return 1;
  const int64_t groups = (int64_t)d->batch * d->hkv;
  // Grids of many workgroups balance by themselves (and would make the
  // simulation long).
  if ((int64_t)(kt1 - kt0) * groups > 16 * kDkdvSlots) return 1;
  const int G = d->hq / d->hkv;
  const int64_t nq = (s.chunk_len + kBwdBlockQ - 1) / kBwdBlockQ;
  const int64_t Lkv = d->skv / d->n_kv_chunks;
  std::vector<double> steps;
  steps.reserve(kt1 - kt0);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int64_t key0 = (int64_t)kt * kBwdBlockKV;
    const int64_t kc = key0 / Lkv;
    const int64_t kv_lo = d->kv_chunk_pos[kc] + (key0 - kc * Lkv);
    // Steps from the tile's causal first query tile to the end of each chunk.
    // With packed sequences that overcounts the tiles whose sequence ends
    // before the chunk does (the kernel stops there); counting exactly made
    // the planner keep a packed share's tiles whole, which measured slower
    // than the split this count picks.
    int64_t n = 0;
    for (int c = 0; c < s.n_q_chunks; ++c) {
      int64_t first = 0;
      if (d->causal) {
        const int64_t rel = kv_lo - s.chunk_pos[c];
        first = rel <= 0 ? 0 : std::min<int64_t>(nq, rel / kBwdBlockQ);
      }
      n += nq - first;
    }
    steps.push_back((double)(n * G));
  }
  const double kStartup = 2.0;   // steps' worth of a workgroup's fixed work
  // Writing and reducing one partial (2 x 64 KiB of fp32, written and read
  // back) costs about this many steps of one workgroup when spread over the chip.
  const double kPartial = 0.03;
  int best = 1;
  double best_t = 0.0;
  for (int parts = 1; parts <= 8; parts *= 2) {
    std::priority_queue<double, std::vector<double>, std::greater<double>> slots;
    for (int i = 0; i < kDkdvSlots; ++i) slots.push(0.0);
    double span = 0.0;
    for (double st : steps)
      for (int j = 0; j < parts; ++j) {
        const double w = kStartup + st / parts;
        for (int64_t g = 0; g < groups; ++g) {
          const double t = slots.top() + w;
          slots.pop();
          slots.push(t);
          span = std::max(span, t);
        }
      }
    const double t = span + kPartial * (parts - 1) * groups * (double)steps.size();
    if (parts == 1 || t < best_t * 0.97) {
      best = parts;
      best_t = t;
    }
  }
  return best;
}

void fill_bwd_params(const cp_attn_desc *d, const Share &s, BwdParams *p, bool allow_split) {
  memset(p, 0, sizeof(*p));
  collect_doc_bounds(d, &p->docs);
  p->mask = static_cast<const uint8_t *>(d->attn_mask);
  p->mask_add = d->mask_additive;
  p->m_sb = d->mask_strides[0]; p->m_sh = d->mask_strides[1]; p->m_ss = d->mask_strides[2];
  p->q_sb = d->q_strides[0]; p->q_sh = d->q_strides[1]; p->q_ss = d->q_strides[2];
  p->kv_sb = d->kv_strides[0]; p->kv_sh = d->kv_strides[1]; p->kv_ss = d->kv_strides[2];
  p->o_sb = d->o_strides[0]; p->o_sh = d->o_strides[1]; p->o_ss = d->o_strides[2];
  fill_kv_chunks(d, &p->kv);
  p->q_cadj = chunk_adj(d->chunk_strides[0], d->sq_local / d->n_q_chunks, d->q_strides[2]);
  p->o_cadj = chunk_adj(d->chunk_strides[2], d->sq_local / d->n_q_chunks, d->o_strides[2]);
  p->batch = d->batch;
  p->hq = d->hq;
  p->hkv = d->hkv;
  p->group = d->hq / d->hkv;
  p->sq = (int32_t)d->sq_local;
  p->skv = (int32_t)d->skv;
  p->chunk_len = (int32_t)s.chunk_len;
  p->n_q_chunks = s.n_q_chunks;
  p->causal = d->causal;
  p->scale = d->softmax_scale;
  p->scale_log2 = d->softmax_scale * 1.4426950408889634f;
  for (int i = 0; i < s.n_q_chunks; ++i) p->chunk_pos[i] = s.chunk_pos[i];
  p->heads_per_item = item_heads(p->group);
  p->n_head_packs = d->batch * (d->hq / p->heads_per_item);
  const int rows = dq_block_rows(p->group);
  p->tiles_per_chunk = (int32_t)((s.chunk_len + rows - 1) / rows);
  for (int i = 0; i < s.n_q_chunks; ++i) {
    p->lpt_chunk_pos[i] = s.chunk_pos[s.order[i]];
    p->lpt_chunk_idx[i] = s.order[i];
  }
  // Key tiles some local query can see. With keys in natural order, a key is
  // visible only if it is not after the last local row (causal) and not
  // before the sequence start of the earliest local row (packed sequences);
  // a user mask can only hide more. Several KV chunks out of position order:
  // every tile.
  const int64_t n_tiles = (d->skv + kBwdBlockKV - 1) / kBwdBlockKV;
  p->kt0 = 0;
  p->kt1 = (int32_t)n_tiles;
  if (p->kv.n == 1 && s.chunk_len > 0 && d->skv > 0) {
    const int64_t kv0 = p->kv.pos[0];
    int64_t qlo = INT64_MAX, qhi = INT64_MIN;
    for (int c = 0; c < s.n_q_chunks; ++c) {
      qlo = std::min(qlo, s.chunk_pos[c]);
      qhi = std::max(qhi, s.chunk_pos[c] + s.chunk_len - 1);
    }
    int64_t lo = 0, hi = d->skv - 1;                 // key rows
    if (d->causal) hi = std::min(hi, qhi - kv0);
    if (d->n_docs > 0) {
      int64_t start = INT64_MIN;                     // sequence start of the earliest local row
      for (int i = 0; i < p->docs.n; ++i)
        if (p->docs.pos[i] <= qlo) start = p->docs.pos[i];
      if (start != INT64_MIN) lo = std::max<int64_t>(0, start - kv0);
    }
    if (hi < lo) {
      p->kt0 = p->kt1 = 0;
    } else {
      p->kt0 = (int32_t)(lo / kBwdBlockKV);
      p->kt1 = (int32_t)(hi / kBwdBlockKV + 1);
    }
  }
  p->kv_parts = allow_split ? dkdv_parts(d, s, p->kt0, p->kt1) : 1;
  p->kv_partial = nullptr;
  p->mask_bits = nullptr;
  p->mb_batches = d->mask_strides[0] ? d->batch : 1;
  p->mb_heads = d->mask_strides[1] ? d->hq : 1;
  p->mb_tpc = (int32_t)((p->chunk_len + kBwdBlockQ - 1) / kBwdBlockQ);
  p->mask_rowbits = nullptr;
  p->mb_ktiles = (int32_t)((d->skv + 63) / 64);
}

// The bit table of a user mask for the bf16 key-stationary kernel (see
// BwdParams::mask_bits), 256-byte aligned.
static size_t bwd_mask_bits_bytes(const cp_attn_desc *d, const BwdParams &p) {
  if (!d->attn_mask || d->dtype != CP_ATTN_BF16) return 0;
  const size_t words = (size_t)p.mb_batches * p.mb_heads * (size_t)p.n_q_chunks * p.mb_tpc * (size_t)d->skv;
  return (words * 8 + 255) & ~(size_t)255;
}

// fp32 partial dK/dV of the split key tiles (see BwdParams::kv_parts).
static size_t bwd_partial_bytes(const BwdParams &p, int head_dim) {
  if (p.kv_parts <= 1) return 0;
  return (size_t)(p.kv_parts - 1) * (size_t)(p.kt1 - p.kt0) * (size_t)p.batch * p.hkv * 2 *
         (size_t)kBwdBlockKV * head_dim * sizeof(float);
}

int64_t fwd_grid_size(const FwdParams &p) {
  return (int64_t)p.n_head_packs * p.n_q_chunks * p.tiles_per_chunk;
}

}  // namespace cpattn

using namespace cpattn;

extern "C" {

int32_t cp_attn_abi_version(void) { return CP_ATTN_ABI_VERSION; }

const char *cp_attn_error_string(int32_t status) {
  switch (status) {
    case CP_ATTN_OK: return "ok";
    case CP_ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case CP_ATTN_ERR_BAD_SHAPE: return "inconsistent sizes or strides (hq % hkv, chunk lengths, negative strides, non-finite or non-positive scale, causal flag)";
    case CP_ATTN_ERR_BAD_LAYOUT: return "layout does not match the chunk table (contiguous: 1 Q chunk, head_tail: 2, chunked: 1..16; 1..64 KV chunks)";
    case CP_ATTN_ERR_BAD_POSITIONS: return "chunk positions negative, too large, or overlapping";
    case CP_ATTN_ERR_UNSUPPORTED: return "unsupported head_dim, dtype, size, row stride (>= 2^24 elements), or KV chunk length not a multiple of 128 with several KV chunks";
    case CP_ATTN_ERR_WORKSPACE: return "workspace missing or smaller than cp_attn_workspace_bytes()";
    case CP_ATTN_ERR_HIP: return "HIP launch or runtime error";
    case CP_ATTN_ERR_ABI: return "descriptor abi_version does not match the library";
    case CP_ATTN_ERR_ALIGNMENT: return "device pointer or stride not 16-byte aligned";
    case CP_ATTN_ERR_DIVISIBILITY: return "sequence length not divisible by cp_size (contiguous) or 2*cp_size (head_tail)";
    case CP_ATTN_ERR_SCRATCH_LIMIT: return "the share's rows (CP_ATTN_NOALLOC_MAX_ROWS) or workspace exceed the fixed scratch of cp_attn_bwd_noalloc; use cp_attn_bwd with a workspace";
    default: return "unknown status";
  }
}

int32_t cp_attn_share_positions(int32_t layout, int64_t s_global, int32_t cp_size,
                                int32_t cp_rank, int64_t *q_chunk_pos,
                                int32_t *n_q_chunks, int64_t *chunk_len) {
  if (!q_chunk_pos || !n_q_chunks || !chunk_len) return CP_ATTN_ERR_NULL_PTR;
  if (cp_size < 1 || cp_rank < 0 || cp_rank >= cp_size || s_global < 0) return CP_ATTN_ERR_BAD_SHAPE;
  if (layout == CP_ATTN_LAYOUT_CONTIGUOUS) {
    if (s_global % cp_size != 0) return CP_ATTN_ERR_DIVISIBILITY;
    const int64_t n = s_global / cp_size;
    q_chunk_pos[0] = (int64_t)cp_rank * n;
    *n_q_chunks = 1;
    *chunk_len = n;
    return CP_ATTN_OK;
  }
  if (layout == CP_ATTN_LAYOUT_HEAD_TAIL) {
    if (s_global % (2 * (int64_t)cp_size) != 0) return CP_ATTN_ERR_DIVISIBILITY;
    const int64_t n = s_global / (2 * (int64_t)cp_size);
    q_chunk_pos[0] = (int64_t)cp_rank * n;
    q_chunk_pos[1] = (int64_t)(2 * cp_size - 1 - cp_rank) * n;
    *n_q_chunks = 2;
    *chunk_len = n;
    return CP_ATTN_OK;
  }
  return CP_ATTN_ERR_BAD_LAYOUT;
}

int32_t cp_attn_validate(const cp_attn_desc *desc) { return validate(desc); }

int32_t cp_attn_share_pairs(const cp_attn_desc *d, int64_t *pairs) {
  int32_t st = validate(d);
  if (st) return st;
  if (!pairs) return CP_ATTN_ERR_NULL_PTR;
  const int64_t L = d->sq_local / d->n_q_chunks;
  const int64_t skv = d->skv / d->n_kv_chunks;   // keys per KV chunk
  int64_t total = 0;
  if (d->n_docs > 0) {
    // Row at position p sees keys max(kv0, start of its sequence) .. min(p, kv0+skv-1).
    const int64_t kv0 = d->kv_chunk_pos[0];
    const int64_t *b = d->doc_starts, *e = d->doc_starts + d->n_docs;
    for (int c = 0; c < d->n_q_chunks; ++c)
      for (int64_t t = 0; t < L; ++t) {
        const int64_t p = d->q_chunk_pos[c] + t;
        const int64_t *up = std::upper_bound(b, e, p);
        const int64_t lo = std::max(kv0, up == b ? kv0 : *(up - 1));
        const int64_t hi = std::min(p, kv0 + skv - 1);
        if (hi >= lo) total += hi - lo + 1;
      }
    *pairs = total;
    return CP_ATTN_OK;
  }
  for (int kc = 0; kc < d->n_kv_chunks; ++kc) {
    const int64_t kv0 = d->kv_chunk_pos[kc];
    for (int c = 0; c < d->n_q_chunks; ++c) {
      if (!d->causal) { total += L * skv; continue; }
      // Row at position p sees keys kv0..min(p, kv0+skv-1): clamp(p-kv0+1, 0, skv).
      const int64_t p0 = d->q_chunk_pos[c], p1 = p0 + L - 1;
      // Rows with p < kv0 see nothing; rows with p >= kv0+skv-1 see all skv.
      const int64_t a = std::max(p0, kv0), b = std::min(p1, kv0 + skv - 1);
      if (a <= b) {
        const int64_t n = b - a + 1, f = a - kv0 + 1;  // counts f, f+1, ..., f+n-1
        total += n * f + n * (n - 1) / 2;
      }
      const int64_t full_from = std::max(p0, kv0 + skv);
      if (full_from <= p1) total += (p1 - full_from + 1) * skv;
    }
  }
  *pairs = total;
  return CP_ATTN_OK;
}

static size_t bwd_stat_bytes(const cp_attn_desc *d) {
  const size_t rows = (size_t)d->batch * d->hq * (size_t)d->sq_local;
  return (rows * 4 + 255) & ~(size_t)255;
}


int32_t cp_attn_workspace_bytes(const cp_attn_desc *d, int32_t backward, size_t *bytes) {
  int32_t st = validate(d);
  if (st) return st;
  if (!bytes) return CP_ATTN_ERR_NULL_PTR;
  if (!backward) { *bytes = mask_rowbits_bytes(d); return CP_ATTN_OK; }
  // Backward: Delta = rowsum(dO o O) and LSE * log2(e), each [B, Hq, Sq]
  // fp32, each starting on a 256-byte boundary; then the fp32 partial dK/dV
  // of key tiles split over several workgroups (none for most shares); then
  // a user mask's bit tables (bf16): per key and query tile for dK/dV, per
  // row and key tile for dQ, and an additive mask's flag. Forward: the row
  // table (and flag) only.
  *bytes = cpattn::bwd_workspace_bytes(d, true);
  return CP_ATTN_OK;
}

int32_t cp_attn_plan_stats_fwd(const cp_attn_desc *d, cp_attn_plan_stats *out) {
  int32_t st = validate(d);
  if (st) return st;
  if (!out) return CP_ATTN_ERR_NULL_PTR;
  Share s;
  make_share(d, &s);
  FwdParams p;
  fill_fwd_params(d, s, &p);
  const int rows = fwd_block_rows(p.group);
  const int bn = kFwdBlockKV;
  // The kernel's visit order: per KV chunk, the prefix of its tiles that
  // the item's last row can see.
  int64_t visits = 0, masked = 0;
  for (int c = 0; c < p.n_q_chunks; ++c)
    for (int t = 0; t < p.tiles_per_chunk; ++t) {
      const int64_t r0 = (int64_t)t * rows;
      const int64_t nrow = std::min<int64_t>(rows, p.chunk_len - r0);
      const int64_t qlo = p.chunk_pos[c] + r0, qhi = qlo + nrow - 1;
      // Packed sequences: tiles before the sequence start of the item's first
      // row are skipped; a tile starting before the last row's sequence start
      // is masked.
      int64_t ds_first = INT64_MIN, ds_last = INT64_MIN;
      for (int i = 0; i < p.docs.n; ++i) {
        if (p.docs.pos[i] <= qlo) ds_first = p.docs.pos[i];
        if (p.docs.pos[i] <= qhi) ds_last = p.docs.pos[i];
      }
      for (int kc = 0; kc < p.kv.n; ++kc) {
        const int64_t kpos = p.kv.pos[kc], krow0 = (int64_t)kc * p.kv.len;
        int64_t nvis = p.kv.len;
        if (p.causal) nvis = std::min<int64_t>(p.kv.len, std::max<int64_t>(0, qhi - kpos + 1));
        const int64_t nt = (nvis + bn - 1) / bn;
        const int64_t t0 = ds_first > kpos ? std::min<int64_t>(nt, (ds_first - kpos) / bn) : 0;
        visits += nt - t0;
        for (int64_t kt = t0; kt < nt; ++kt) {
          const int64_t klast = kt * bn + bn - 1;
          if (krow0 + klast >= p.skv || (p.causal && kpos + klast > qlo) || kpos + kt * bn < ds_last) ++masked;
        }
      }
    }
  out->work_items = fwd_grid_size(p);
  out->kv_tile_visits = visits * p.n_head_packs;
  out->masked_tile_visits = masked * p.n_head_packs;
  out->block_q_rows = rows;
  out->block_kv_rows = bn;
  out->heads_per_item = p.heads_per_item;
  return CP_ATTN_OK;
}

int32_t cp_attn_fwd(const cp_attn_desc *d, const void *q, const void *k, const void *v,
                    void *out, float *lse, void *workspace, size_t workspace_bytes,
                    void *stream) {
  int32_t st = validate(d);
  if (st) return st;
  if (d->sq_local == 0) return CP_ATTN_OK;
  if (!q || !out || !lse) return CP_ATTN_ERR_NULL_PTR;
  if (d->skv > 0 && (!k || !v)) return CP_ATTN_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(out) || (d->skv > 0 && (!aligned16(k) || !aligned16(v))))
    return CP_ATTN_ERR_ALIGNMENT;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return CP_ATTN_ERR_ALIGNMENT;
  const size_t need = mask_rowbits_bytes(d);
  if (!mask_rowbits_grid_ok(d)) return CP_ATTN_ERR_UNSUPPORTED;
  if (need > 0 && (!workspace || workspace_bytes < need)) return CP_ATTN_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return CP_ATTN_ERR_ALIGNMENT;
  Share s;
  make_share(d, &s);
  FwdParams p;
  fill_fwd_params(d, s, &p);
  p.q = q; p.k = k; p.v = v; p.out = out; p.lse = lse;
  if (need > 0) {
    uint64_t *rb = static_cast<uint64_t *>(workspace);
    p.mask_rowbits = rb;
    p.mask_flag = mask_flag_at(rb, d);
    if (launch_mask_rowbits(p.mask, p.m_sb, p.m_sh, p.m_ss, p.mb_batches, p.mb_heads, p.sq, p.skv, p.mask_add != 0,
                            rb, const_cast<uint32_t *>(p.mask_flag), stream))
      return CP_ATTN_ERR_HIP;
  }
  const int e = (d->dtype == CP_ATTN_BF16) ? launch_fwd_bf16(p, d->head_dim, stream)
                                           : launch_fwd_fp32(p, d->head_dim, stream);
  return e == 0 ? CP_ATTN_OK : CP_ATTN_ERR_HIP;
}

int32_t cp_attn_bwd_timed(const cp_attn_desc *d, const void *q, const void *k, const void *v,
                          const void *out, const float *lse, const void *dout, void *dq, float *dk,
                          float *dv, void *workspace, size_t workspace_bytes, void *stream,
                          void *const *events, int32_t n_events) {
  return bwd_run(d, q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream, events,
                 n_events, true);
}

int32_t cp_attn_bwd(const cp_attn_desc *d, const void *q, const void *k, const void *v,
                    const void *out, const float *lse, const void *dout, void *dq, float *dk,
                    float *dv, void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_run(d, q, k, v, out, lse, dout, dq, dk, dv, workspace, workspace_bytes, stream, nullptr, 0,
                 true);
}

}  // extern "C"

namespace cpattn {

size_t bwd_workspace_bytes(const cp_attn_desc *d, bool allow_split) {
  Share s;
  make_share(d, &s);
  BwdParams p;
  fill_bwd_params(d, s, &p, allow_split);
  return 2 * bwd_stat_bytes(d) + bwd_partial_bytes(p, d->head_dim) + bwd_mask_bits_bytes(d, p) +
         mask_rowbits_bytes(d);
}

int32_t bwd_run(const cp_attn_desc *d, const void *q, const void *k, const void *v, const void *out,
                const float *lse, const void *dout, void *dq, float *dk, float *dv, void *workspace,
                size_t workspace_bytes, void *stream, void *const *events, int32_t n_events,
                bool allow_split) {
  int32_t st = validate(d);
  if (st) return st;
  if (!(n_events == 0 && events == nullptr) && n_events != 4) return CP_ATTN_ERR_BAD_SHAPE;
  if (n_events == 4) {
    if (!events) return CP_ATTN_ERR_NULL_PTR;
    for (int i = 0; i < 4; ++i)
      if (!events[i]) return CP_ATTN_ERR_NULL_PTR;
  }
  Share s;
  make_share(d, &s);
  BwdParams p;
  fill_bwd_params(d, s, &p, allow_split);
  const size_t partial = bwd_partial_bytes(p, d->head_dim);
  const size_t bits = bwd_mask_bits_bytes(d, p);
  const size_t rowbits = mask_rowbits_bytes(d);
  const size_t need = 2 * bwd_stat_bytes(d) + partial + bits + rowbits;
  // The bit tables' passes run one workgroup per kMaskBitsBlockKeys keys,
  // query tile and mask head, and per 256 row words.
  if (bits > 0 && !fits_grid((int64_t)((d->skv + kMaskBitsBlockKeys - 1) / kMaskBitsBlockKeys) * p.n_q_chunks *
                                 p.mb_tpc * p.mb_batches * p.mb_heads, 256))
    return CP_ATTN_ERR_UNSUPPORTED;
  if (!mask_rowbits_grid_ok(d)) return CP_ATTN_ERR_UNSUPPORTED;
  if (d->sq_local > 0 && (!q || !out || !lse || !dout || !dq)) return CP_ATTN_ERR_NULL_PTR;
  if (d->skv > 0 && (!k || !v || !dk || !dv)) return CP_ATTN_ERR_NULL_PTR;
  if (need > 0 && (!workspace || workspace_bytes < need)) return CP_ATTN_ERR_WORKSPACE;
  const void *ptrs16[] = {q, out, dout, dq, k, v, dk, dv, workspace};
  for (const void *ptr : ptrs16)
    if (ptr && !aligned16(ptr)) return CP_ATTN_ERR_ALIGNMENT;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return CP_ATTN_ERR_ALIGNMENT;
  p.q = q; p.k = k; p.v = v; p.out = out; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.delta = static_cast<float *>(workspace);
  p.lse2 = reinterpret_cast<float *>(static_cast<char *>(workspace) + bwd_stat_bytes(d));
  if (p.kv_parts > 1)
    p.kv_partial = reinterpret_cast<float *>(static_cast<char *>(workspace) + 2 * bwd_stat_bytes(d));
  if (bits > 0)
    p.mask_bits = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + 2 * bwd_stat_bytes(d) + partial);
  if (rowbits > 0) {   // written by the backward's first passes
    p.mask_rowbits = reinterpret_cast<uint64_t *>(static_cast<char *>(workspace) + 2 * bwd_stat_bytes(d) + partial + bits);
    p.mask_flag = mask_flag_at(p.mask_rowbits, d);
  }
  void *const *ev = n_events == 4 ? events : nullptr;
  const int e = (d->dtype == CP_ATTN_BF16) ? launch_bwd_bf16(p, d->head_dim, stream, ev)
                                           : launch_bwd_fp32(p, d->head_dim, stream, ev);
  return e == 0 ? CP_ATTN_OK : CP_ATTN_ERR_HIP;
}

}  // namespace cpattn
