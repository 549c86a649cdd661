/*
 * cp_attn.h -- C ABI of one context-parallel (CP) rank's causal attention share
 * on AMD Instinct MI355X (gfx950).
 *
 * A "share" is the attention a single CP rank computes: its local query rows
 * against the gathered (global) keys and values, masked causally by GLOBAL
 * token position. Sources, by page title and section:
 *
 *  [CP-migration] "新流程 CP 多通信模式迁移设计方案" (hyper-parallel issue 7):
 *      §6.1 AllGather / Pure Colossal (local Q, all-gathered K/V, output stays
 *      local; backward: dQ local, dK/dV reduce-scattered with sum),
 *      §6.2 Pure Ulysses and §6.3 Hybrid (head-sliced shares),
 *      §8 Causal mask (the per-strategy global Q offsets; a flash backend
 *      should take the offsets natively instead of a materialised mask),
 *      §9.2 GQA/MQA, §9.3 Layout (BNSD by default).
 *  [Trainer-CP] "HyperModels 新 Trainer Context Parallel 接入设计方案":
 *      §0 (Head-Tail load balance), §4.2 (padding / divisibility policy),
 *      §4.3 (the three synchronous strategies), §4.4 (Head-Tail: two Q
 *      segments, each with its own global interval; fail fast, no fallback).
 *  [FLA-CP] "flash-linear-attention 上下文并行CP 从 CP2TP、Ring CP 到 True CP
 *      的设计取舍与源码实现" §3.2 (contiguous vs zigzag layout, [front; back]
 *      local order) and §3.3 (divisibility errors).
 *
 * Every call validates its descriptor on the host first and returns a negative
 * status without touching any buffer when something is wrong; there is no
 * silent fallback to a slower path. All functions are thread-safe and
 * reentrant; the library keeps no state between calls and never allocates,
 * frees or retains device memory: the caller owns every buffer, including the
 * workspace.
 *
 * Device work is enqueued on the caller's stream (a hipStream_t passed as
 * `void *`; NULL means the default stream) and the call returns without
 * synchronising. The caller keeps every buffer alive until the stream has
 * passed the work. Kernel faults surface at the caller's next synchronisation.
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bumped whenever cp_attn_desc's layout or a declaration's meaning changes
 * (3: the user-mask fields attn_mask, mask_strides, mask_additive and the
 * additive-mask hide threshold; 4: chunk_strides and the chunked layout). */
#define CP_ATTN_ABI_VERSION 4
#define CP_ATTN_MAX_Q_CHUNKS 16
/* Most KV chunks a descriptor may list (a Head-Tail all-gather at cp = 32
 * delivers 64 chunks). */
#define CP_ATTN_MAX_KV_CHUNKS 64
/* With more than one KV chunk, each chunk's length must be a multiple of this
 * many rows (the largest key tile of the kernels, so no tile straddles two
 * chunks). */
#define CP_ATTN_KV_CHUNK_ALIGN 128
/* Most packed-sequence boundaries a share may meet (see cp_attn_desc.doc_starts). */
#define CP_ATTN_MAX_DOC_BOUNDS 256
/* An additive user-mask value at or below this hides its key exactly like
 * -inf. Padding masks use -1e4, -1e9 or the float32 minimum for "hidden"; a
 * row whose every key carries such a bias has no representable float32 LSE
 * near the bias (one ulp of 1e9 is 64) and its backward would be meaningless,
 * so all of them are treated as hidden keys. */
#define CP_ATTN_MASK_HIDE (-1.0e4f)

/* Local row order of the query shard. */
typedef enum {
  /* One chunk of consecutive global positions: the all-gather (Colossal)
   * share at offset cp_rank*S/cp, the Ulysses share (offset 0, whole
   * sequence) and the Hybrid share (offset co_rank*S/C). [CP-migration] §8. */
  CP_ATTN_LAYOUT_CONTIGUOUS = 0,
  /* Head-Tail (zigzag): exactly two equal chunks, front = chunk r, back =
   * chunk 2*cp-1-r of 2*cp chunks. [Trainer-CP] §4.4, [FLA-CP] §3.2. */
  CP_ATTN_LAYOUT_HEAD_TAIL = 1,
  /* Any number (1..CP_ATTN_MAX_Q_CHUNKS) of equal chunks at the listed,
   * pairwise disjoint positions. With chunk_strides it describes a Ulysses
   * head shard still laid out as the sequence->head all-to-all delivered it:
   * chunk p (rows p*L .. p*L+L-1 of the sequence) is block p of the received
   * buffer [u, batch, heads, L, head_dim] ([CP-migration] §6.2, §6.3). */
  CP_ATTN_LAYOUT_CHUNKED = 2
} cp_attn_layout;

/* Element type of q, k, v, out, dout and dq. lse, the backward workspace and
 * dk/dv are always float32. */
typedef enum { CP_ATTN_BF16 = 0, CP_ATTN_FP32 = 1 } cp_attn_dtype;

/* Status codes. 0 is success; every error is negative. */
typedef enum {
  CP_ATTN_OK = 0,
  CP_ATTN_ERR_NULL_PTR = -1,      /* a required pointer is NULL */
  CP_ATTN_ERR_BAD_SHAPE = -2,     /* sizes/strides inconsistent (hq % hkv, chunk lengths, ...) */
  CP_ATTN_ERR_BAD_LAYOUT = -3,    /* layout vs chunk count, or unknown layout */
  CP_ATTN_ERR_BAD_POSITIONS = -4, /* negative or overlapping chunk positions, unsorted doc_starts */
  CP_ATTN_ERR_UNSUPPORTED = -5,   /* head_dim / dtype / KV chunk length / row stride >= 2^24 not implemented */
  CP_ATTN_ERR_WORKSPACE = -6,     /* workspace NULL or smaller than cp_attn_workspace_bytes() */
  CP_ATTN_ERR_HIP = -7,           /* a HIP launch or query failed */
  CP_ATTN_ERR_ABI = -8,           /* desc->abi_version != CP_ATTN_ABI_VERSION */
  CP_ATTN_ERR_ALIGNMENT = -9,     /* a device pointer or stride breaks the 16-byte vector alignment */
  CP_ATTN_ERR_DIVISIBILITY = -10, /* cp_attn_share_positions: S not divisible by cp (or 2*cp) */
  CP_ATTN_ERR_SCRATCH_LIMIT = -11 /* cp_attn_bwd_noalloc: the share's workspace exceeds its fixed scratch */
} cp_attn_status;

/*
 * Descriptor of one share. Tensors are indexed [batch][head][row][dim] with
 * the dim index contiguous (stride 1) and the other three strides given in
 * ELEMENTS, so BNSD tensors, head slices and row slices of a larger tensor can
 * be passed without copies ([CP-migration] §9.3).
 *
 *   q           [batch, hq,  sq_local, head_dim]  q_strides
 *   k, v        [batch, hkv, skv,      head_dim]  kv_strides (shared by k and v)
 *   out, dout,
 *   dq          [batch, hq,  sq_local, head_dim]  o_strides (shared by the three)
 *   lse         [batch, hq,  sq_local]            contiguous float32
 *   dk, dv      [batch, hkv, skv, head_dim]       contiguous float32
 *
 * With chunk_strides[0] = C != 0, row i of q (chunk c = i / L, t = i % L) is
 * at batch/head offset + c * C + t * q_strides[2] instead of i * q_strides[2];
 * likewise out, dout and dq with chunk_strides[2], and key row j of k and v
 * (KV chunk c = j / Lkv) with chunk_strides[1]. lse, dk and dv keep the
 * plain row order. This lets the kernels read a Ulysses all-to-all's
 * received blocks [u, batch, heads, L, head_dim] in place (batch stride
 * heads*L*head_dim, head stride L*head_dim, row stride head_dim, chunk stride
 * batch*heads*L*head_dim) and write out in the layout the reverse exchange
 * sends.
 *
 * Query row i lies in chunk c = i / L (L = sq_local / n_q_chunks) and has
 * global position q_chunk_pos[c] + i % L. Key row j lies in KV chunk
 * c = j / Lkv (Lkv = skv / n_kv_chunks) and has global position
 * kv_chunk_pos[c] + j % Lkv. With causal != 0, key j is visible to query i iff
 * pos(j) <= pos(i) (the diagonal included); with causal == 0 every key is
 * visible. One KV chunk is the natural order (keys at kv_chunk_pos[0],
 * kv_chunk_pos[0]+1, ...). Several KV chunks describe K/V in any chunk order,
 * for example straight from a Head-Tail all-gather, where rank r contributes
 * its chunks r and 2cp-1-r ([Trainer-CP] §4.4 zigzag order): kv_chunk_pos =
 * {0, (2cp-1)L, L, (2cp-2)L, ...}. The result does not depend on the order;
 * dk/dv rows follow the k/v rows (storage order). KV chunk positions must be
 * pairwise disjoint ranges. Query head h reads KV head h / (hq / hkv) (contiguous GQA groups,
 * [CP-migration] §9.2).
 *
 * Packed variable-length sequences ([FLA-CP] §3.1, §3.3: a global cu_seqlens
 * split across ranks): with n_docs > 0 the global positions are cut into
 * sequences starting at doc_starts[0] < doc_starts[1] < ... (a cu_seqlens
 * without its final total; positions before doc_starts[0] form one more
 * sequence), and key j is visible to query i only if it also lies in the
 * query's sequence. Requires causal != 0 and one KV chunk. The library keeps
 * only the boundaries the share can meet (per query chunk: the last start at
 * or before it, every start inside it, the first start after it); more than
 * CP_ATTN_MAX_DOC_BOUNDS of them is CP_ATTN_ERR_UNSUPPORTED.
 *
 * A user attention mask ([CP-migration] §8: merged with the CP mask, never
 * replacing it): with attn_mask != NULL and mask_additive == 0, key j is
 * visible to query i only if also attn_mask[b][h][i][j] != 0 (bytes; i the
 * local row, j the key row); with mask_additive == 1 the float32 value
 * a = attn_mask[b][h][i][j] is added to softmax_scale * q.k, and a value
 * a <= CP_ATTN_MASK_HIDE (-inf, -1e9, the float32 minimum, ...) hides the key.
 * Finite values above it are biases; the stated precision holds for
 * |a| < 1e4, larger positive values and NaN are outside the supported range.
 * Requires one KV chunk and no packed sequences; the pointer and strides must
 * be multiples of 4 bytes (16 for an additive mask). The mask is read by
 * the kernels during the call's work on the stream; the caller keeps it alive
 * like the other device buffers. With bf16 a first kernel packs the mask
 * into bit tables in the workspace; an additive mask whose values are all 0
 * or hiding (a padding mask) is then applied through them, bitwise as the
 * boolean mask it encodes, the kernel finding so on the device.
 *
 * The LSE of query i is the natural log of the sum, over its visible keys j,
 * of exp(softmax_scale * q_i.k_j + a_ij), with a_ij the additive mask value
 * (0 without an additive mask); a row with no visible key gets out = 0 and
 * lse = -inf.
 */
typedef struct cp_attn_desc {
  int32_t abi_version;         /* must be CP_ATTN_ABI_VERSION */
  int32_t dtype;               /* cp_attn_dtype */
  int32_t batch, hq, hkv;      /* hq % hkv == 0 */
  int32_t head_dim;            /* bf16: 64 or 128; fp32: 64 or 128 */
  int64_t sq_local;            /* local query rows (all chunks) */
  int64_t skv;                 /* gathered key/value rows */
  int32_t n_q_chunks;          /* 1..CP_ATTN_MAX_Q_CHUNKS, equal lengths */
  const int64_t *q_chunk_pos;  /* host array [n_q_chunks]: global position of each chunk's row 0 */
  int32_t n_kv_chunks;         /* 1..CP_ATTN_MAX_KV_CHUNKS, equal lengths; with more than one, */
                               /* skv / n_kv_chunks must be a multiple of CP_ATTN_KV_CHUNK_ALIGN */
  const int64_t *kv_chunk_pos; /* host array [n_kv_chunks]: global position of each KV chunk's row 0 */
  int32_t layout;              /* cp_attn_layout: contiguous needs 1 Q chunk, head_tail needs 2 */
  int32_t causal;              /* 1: global-position causal mask, 0: no mask */
  float softmax_scale;         /* scale applied to q.k, finite and > 0 (1/sqrt(head_dim) is SDPA's default) */
  int64_t q_strides[3];        /* batch, head, row strides of q (elements) */
  int64_t kv_strides[3];       /* batch, head, row strides of k and v (elements) */
  int64_t o_strides[3];        /* batch, head, row strides of out, dout and dq (elements) */
                               /* all strides >= 0, multiples of 16 bytes; row strides < 2^24 */
  int32_t n_docs;              /* 0: one sequence; > 0: packed sequences (needs causal, one KV chunk) */
  const int64_t *doc_starts;   /* host array [n_docs]: strictly increasing global start positions, >= 0 */
  const void *attn_mask;       /* NULL, or DEVICE [batch][hq][sq_local][skv] mask of mask_additive's kind */
  int64_t mask_strides[3];     /* batch, head, row strides of attn_mask in bytes (0 broadcasts; row stride < 32 MiB); key stride 1 */
  int32_t mask_additive;       /* 0: bytes, nonzero = may attend; 1: float32 added to the scaled score */
  int64_t chunk_strides[3];    /* q, k/v, out/dout/dq: elements from one chunk's row 0 to the next */
                               /* chunk's (Q chunks for q and out, KV chunks for k/v); 0: the rows */
                               /* follow on (chunk length x row stride). Multiples of 16 bytes, >= 0. */
} cp_attn_desc;

/* ABI version of the loaded library (CP_ATTN_ABI_VERSION of its build). A
 * descriptor whose abi_version differs is rejected (CP_ATTN_ERR_ABI), in line
 * with the fail-fast rule of [CP-migration] §13.2. */
int32_t cp_attn_abi_version(void);

/* Human-readable text of a status code ([CP-migration] §13.2: every rejected
 * configuration is reported with its reason); never NULL, static storage. */
const char *cp_attn_error_string(int32_t status);

/*
 * Global chunk positions of CP rank `cp_rank` of `cp_size` over a sequence of
 * `s_global` tokens ([CP-migration] §8 offset table; [FLA-CP] §3.2):
 *   contiguous: one chunk at cp_rank * s_global / cp_size of length s_global / cp_size;
 *   head_tail : two chunks of length L = s_global / (2 cp_size) at
 *               cp_rank * L (front) and (2 cp_size - 1 - cp_rank) * L (back).
 * Outputs: q_chunk_pos[0..n-1] (the caller provides room for 2), *n_q_chunks,
 * *chunk_len. Returns CP_ATTN_ERR_DIVISIBILITY when s_global is not a multiple
 * of cp_size (contiguous) or 2*cp_size (head_tail) ([Trainer-CP] §4.2,
 * [FLA-CP] §3.3), CP_ATTN_ERR_BAD_SHAPE for cp_size < 1 or a rank out of range.
 * Host only; no GPU needed.
 */
int32_t cp_attn_share_positions(int32_t layout, int64_t s_global, int32_t cp_size,
                                int32_t cp_rank, int64_t *q_chunk_pos,
                                int32_t *n_q_chunks, int64_t *chunk_len);

/* Validate a descriptor (host only; no GPU needed). Checks everything that
 * does not need device pointers: the fail-fast checks of [CP-migration] §13.2
 * (shape and layout errors are reported before any work, never worked around)
 * and the divisibility and chunk rules of [Trainer-CP] §4.2 / [FLA-CP] §3.3.
 * Returns CP_ATTN_OK or the first failing check's status (see cp_attn_status):
 * ABI, UNSUPPORTED (dtype, head_dim, sizes >= 2^31, row strides >= 2^24, KV
 * chunk length), BAD_SHAPE, BAD_LAYOUT, BAD_POSITIONS, NULL_PTR (host arrays),
 * ALIGNMENT (strides, mask pointer). `desc` is read only during the call. */
int32_t cp_attn_validate(const cp_attn_desc *desc);

/* Number of visible (query, key) pairs per (batch, query head) of the share:
 * the causal work that FLOP counts are based on, under the global-position
 * causal mask ([CP-migration] §8), the KV chunk table and the packed
 * sequences ([FLA-CP] §3.3). Equal for every rank of a Head-Tail split
 * ([Trainer-CP] §0, Head-Tail: each rank gets the same causal work). Errors:
 * cp_attn_validate's, NULL_PTR for `pairs`. Host only. */
int32_t cp_attn_share_pairs(const cp_attn_desc *desc, int64_t *pairs);

/* Bytes of device workspace cp_attn_fwd (backward == 0) or cp_attn_bwd
 * (backward != 0) needs for this descriptor; may be 0. With a user mask
 * (bf16) both hold the mask as row bits, one 64-bit word per query row,
 * 64-key tile and mask batch/head (an eighth of a boolean mask's bytes),
 * and for an additive mask 256 bytes more for the flag that says whether its
 * values are only 0 and hiding ones; the forward needs nothing else. The
 * backward's also holds the per-row statistics of the recompute-based
 * gradient of [CP-migration] §6.1 (-Delta and LSE*log2(e)), for shares whose
 * key tiles are split over several workgroups their float32 partial dK/dV,
 * and with a user mask its column bits too: one 64-bit word per key, 64-row
 * query tile and mask batch/head. Errors: cp_attn_validate's, NULL_PTR for
 * `bytes`. Host only. */
int32_t cp_attn_workspace_bytes(const cp_attn_desc *desc, int32_t backward, size_t *bytes);

/* Work-list statistics of the forward tile scheduler (host only), for tests
 * and reports: number of work items (one workgroup each), the KV tiles they
 * visit in total (per KV chunk, the prefix the item's last row can see; with
 * packed sequences, from the first row's sequence start on), and the tile
 * shape. The scheduler maps both Head-Tail chunks ([Trainer-CP] §4.4) and
 * their causal KV ranges ([CP-migration] §8) onto one launch. Errors:
 * cp_attn_validate's, NULL_PTR for `stats`. */
typedef struct cp_attn_plan_stats {
  int64_t work_items;
  int64_t kv_tile_visits;      /* summed over work items */
  int64_t masked_tile_visits;  /* visits that need an element-wise mask */
  int32_t block_q_rows;        /* query rows per work item (per head) */
  int32_t block_kv_rows;       /* keys per KV tile */
  int32_t heads_per_item;      /* query heads of one GQA group packed in a work item */
} cp_attn_plan_stats;
int32_t cp_attn_plan_stats_fwd(const cp_attn_desc *desc, cp_attn_plan_stats *stats);

/*
 * Forward of the share: out = softmax(scale * q k^T, masked) v and the LSE.
 * This is the local-Q / gathered-K/V attention call of [CP-migration] §6.1
 * (and of §6.2 / §6.3 on head-sliced inputs), under the global-position
 * causal mask of §8 and the GQA head mapping of §9.2; the Head-Tail share's
 * two chunks ([Trainer-CP] §4.4) are computed in one call.
 * q, k, v: device pointers of `dtype`, caller-owned, read only; out: device,
 * `dtype`, o_strides, written; lse: device float32 [batch, hq, sq_local]
 * contiguous, written. Pointers must be 16-byte aligned (lse 4-byte).
 * The workspace (cp_attn_workspace_bytes with backward == 0) is caller-owned
 * device memory, 16-byte aligned, whose contents on entry do not matter; only
 * a bf16 share with a user mask needs one (it holds the mask as row bits,
 * packed by a first kernel), else workspace may be NULL. Returns
 * CP_ATTN_OK once the kernels are enqueued on `stream`; validation errors
 * (cp_attn_validate's, NULL_PTR, ALIGNMENT, UNSUPPORTED for a bit table of
 * 2^32 words or more) and CP_ATTN_ERR_WORKSPACE (needed and NULL or too
 * small) return before anything is enqueued or written; CP_ATTN_ERR_HIP if a
 * launch fails.
 * Deterministic: the same inputs give bitwise the same outputs.
 */
int32_t cp_attn_fwd(const cp_attn_desc *desc, const void *q, const void *k, const void *v,
                    void *out, float *lse, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * Backward of the share for the loss sum(dout * out):
 *   dq [batch, hq, sq_local, head_dim] of `dtype` (o_strides);
 *   dk, dv [batch, hkv, skv, head_dim] float32 contiguous: this share's
 *   PARTIAL gradients over the gathered K/V, to be summed across ranks by a
 *   reduce-scatter ([CP-migration] §6.1 backward). Key rows no query of the
 *   share can see are written as zeros.
 * out and lse are the forward's outputs for the same inputs. q, k, v, out,
 * lse, dout: device, caller-owned, read only; dq, dk, dv: device, written.
 * The workspace (cp_attn_workspace_bytes with backward != 0) is caller-owned
 * device memory; its contents on entry do not matter. Returns CP_ATTN_OK once
 * the kernels are enqueued on `stream`; validation errors (as cp_attn_fwd)
 * and CP_ATTN_ERR_WORKSPACE (workspace NULL or too small) return before
 * anything is enqueued or written; CP_ATTN_ERR_HIP if a launch fails.
 * Deterministic: split key tiles add their partial sums in a fixed order.
 */
int32_t cp_attn_bwd(const cp_attn_desc *desc, const void *q, const void *k, const void *v,
                    const void *out, const float *lse, const void *dout,
                    void *dq, float *dk, float *dv, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * cp_attn_bwd ([CP-migration] §6.1 backward) with its phases bracketed by
 * caller-owned HIP events, for per-kernel timing on the caller's stream. `events` holds n_events
 * hipEvent_t handles (n_events must be 4, or events NULL and n_events 0,
 * which makes this call identical to cp_attn_bwd). They are recorded on
 * `stream` before phase 1 and after phases 1, 2 and 3:
 *   bf16: 1 = Delta pre-pass, 2 = dK/dV kernel, 3 = dQ kernel;
 *   fp32: 1 = Delta + dQ kernel, 2 = dK/dV kernel, 3 = nothing.
 * A phase with no work still records its events. Results are bitwise those
 * of cp_attn_bwd. Errors as cp_attn_bwd; CP_ATTN_ERR_NULL_PTR when
 * n_events is 4 and an event is NULL, CP_ATTN_ERR_BAD_SHAPE for any other
 * n_events. Events are not recorded when validation fails.
 */
int32_t cp_attn_bwd_timed(const cp_attn_desc *desc, const void *q, const void *k, const void *v,
                          const void *out, const float *lse, const void *dout,
                          void *dq, float *dk, float *dv, void *workspace, size_t workspace_bytes,
                          void *stream, void *const *events, int32_t n_events);

/*
 * cp_attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation. Same arguments and errors as
 * cp_attn_bwd, and the same results: dq bitwise; dk and dv up to the order
 * of float32 additions (cp_attn_bwd may split a key tile's queries over
 * several workgroups and add their partial sums; this entry point never
 * splits). The backward's per-row statistics (-Delta and
 * LSE * log2(e)) live in a fixed scratch array inside the library instead
 * (2 x CP_ATTN_NOALLOC_MAX_ROWS float32, 16 MiB, held by every GPU the
 * library runs on until the process ends). Calls no allocating routine; the
 * first call on a device looks up that device's array once.
 * batch * hq * sq_local above CP_ATTN_NOALLOC_MAX_ROWS, or a share whose
 * workspace (cp_attn_workspace_bytes without split key tiles, e.g. with the
 * bit tables of a large user mask) exceeds the 16 MiB, returns
 * CP_ATTN_ERR_SCRATCH_LIMIT before anything is enqueued. `stream`'s device
 * (the current device for NULL) selects the array. Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (different streams,
 * or host threads) race and must be serialised by the caller; calls in order
 * on one stream are safe (each call rewrites every row it reads).
 */
#define CP_ATTN_NOALLOC_MAX_ROWS (1 << 21)
int32_t cp_attn_bwd_noalloc(const cp_attn_desc *desc, const void *q, const void *k, const void *v,
                            const void *out, const float *lse, const void *dout,
                            void *dq, float *dk, float *dv, void *stream);

/* ------------------------------------------------------------------------
 * Ulysses exchange: the local steps on either side of the all-to-all
 * ([CP-migration] §6.2: Q/K/V [B, N, S/P, D] are split by head and exchanged
 * into [B, N/P, S, D], the output goes back by the inverse exchange; §6.3 runs
 * the same exchange inside the Hybrid's cp_ulysses sub-group). The collective
 * (an all_to_all_single over the u ranks of the group) moves block p of every
 * rank's send buffer to rank p, where it lands as block "source rank". These
 * functions are the re-layouts around it; they do not communicate.
 * ------------------------------------------------------------------------ */
typedef enum {
  CP_ATTN_ULYSSES_SEQ_TO_HEAD_PACK = 0,    /* src x,      dst blocks */
  CP_ATTN_ULYSSES_SEQ_TO_HEAD_UNPACK = 1,  /* src blocks, dst y      */
  CP_ATTN_ULYSSES_HEAD_TO_SEQ_PACK = 2,    /* src y,      dst blocks */
  CP_ATTN_ULYSSES_HEAD_TO_SEQ_UNPACK = 3   /* src blocks, dst x      */
} cp_attn_ulysses_step;

/*
 * Tensors, element type `dtype` (cp_attn_dtype), head_dim contiguous:
 *   x       [batch, u*heads, rows, head_dim]   a rank's sequence shard, every head
 *   y       [batch, heads, u*rows, head_dim]   its head shard over the group's sequence
 *   blocks  [u, batch, heads, rows, head_dim]  contiguous; block p goes to / came from rank p
 * Steps (p < u, b < batch, h < heads, t < rows):
 *   SEQ_TO_HEAD_PACK    blocks[p][b][h][t] = x[b][p*heads + h][t]
 *   SEQ_TO_HEAD_UNPACK  y[b][h][p*rows + t] = blocks[p][b][h][t]
 *   HEAD_TO_SEQ_PACK    blocks[p][b][h][t] = y[b][h][p*rows + t]
 *   HEAD_TO_SEQ_UNPACK  x[b][p*heads + h][t] = blocks[p][b][h][t]
 * `strides` are the (batch, head, row) strides in ELEMENTS of the x or y side
 * the step names (host array, read during the call); the blocks side is
 * contiguous. Every row is copied bit-exactly; work is enqueued on `stream`
 * (hipStream_t, NULL = default stream). The caller owns both buffers, which
 * must not overlap. Errors (nothing is enqueued): CP_ATTN_ERR_BAD_LAYOUT
 * (unknown step), CP_ATTN_ERR_BAD_SHAPE (u, batch or heads < 1, rows < 0,
 * negative strides, overlapping buffers), CP_ATTN_ERR_UNSUPPORTED (dtype;
 * head_dim * element size not a power of two in [16, 4096] bytes; rows >= 2^31),
 * CP_ATTN_ERR_NULL_PTR, CP_ATTN_ERR_ALIGNMENT (pointers or strides not 16-byte
 * multiples), CP_ATTN_ERR_HIP.
 */
int32_t cp_attn_ulysses_relayout(int32_t step, int32_t dtype, int32_t u, int32_t batch,
                                 int32_t heads, int64_t rows, int32_t head_dim,
                                 const void *src, void *dst, const int64_t *strides,
                                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */
