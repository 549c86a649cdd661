// Ulysses exchange re-layouts: the local steps on either side of the
// sequence<->head all-to-all ("新流程 CP 多通信模式迁移设计方案" §6.2 Pure
// Ulysses, §6.3 Hybrid). A rank's sequence shard x [B, u*H, L, D] is cut by
// head into u blocks [u][B, H, L, D], one per peer; after the collective the
// blocks received (one per source rank) are laid end to end along the
// sequence as the head shard y [B, H, u*L, D]. The inverse exchange of the
// output runs the same two steps the other way round.
//
// All four steps are one strided copy of whole rows: an index (p, b, h, t)
// names a row of D elements on both sides, and each side maps it to a byte
// offset with its own four strides. The copy is bound by HBM bandwidth (it
// reads and writes every byte once), so the kernel moves 16-byte vectors,
// rows stay contiguous along (t, d) on both sides (every wavefront reads and
// writes whole 256-byte or longer runs), each thread keeps four loads in
// flight before it stores, and loads and stores are non-temporal (every byte
// is touched once; measured about 5 % faster than cached accesses).
#include <hip/hip_runtime.h>

#include "cp_attn.h"
#include "gfx950_common.h"

namespace cpattn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // rows per thread per pass (loads in flight)

struct RelayoutParams {
  const char *src;
  char *dst;
  int64_t s[4];   // byte strides of (block p, batch, head, row) on the source side
  int64_t d[4];   // and on the destination side
  int32_t heads;
  int32_t rows;
  int32_t vpr_log2;   // 16-byte vectors per row = 1 << vpr_log2
};

// blockIdx.z: block p; blockIdx.y: batch * heads + head; blockIdx.x: a run of
// kUnroll * (kThreads >> vpr_log2) rows of that (p, b, h) slab.
__global__ void __launch_bounds__(kThreads) relayout_kernel(const RelayoutParams p) {
  const int q = blockIdx.z;
  const int b = blockIdx.y / p.heads;
  const int h = blockIdx.y - b * p.heads;
  const char *src = p.src + q * p.s[0] + b * p.s[1] + h * p.s[2];
  char *dst = p.dst + q * p.d[0] + b * p.d[1] + h * p.d[2];
  const int v = threadIdx.x & ((1 << p.vpr_log2) - 1);   // vector within the row
  const int rpb = kThreads >> p.vpr_log2;                  // rows per pass of the block
  const int r0 = blockIdx.x * (kUnroll * rpb) + (threadIdx.x >> p.vpr_log2);
  u32x4 val[kUnroll];
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int t = r0 + k * rpb;
    if (t < p.rows) val[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + t * p.s[3] + 16 * v));
  }
#pragma unroll
  for (int k = 0; k < kUnroll; ++k) {
    const int t = r0 + k * rpb;
    if (t < p.rows) __builtin_nontemporal_store(val[k], reinterpret_cast<u32x4 *>(dst + t * p.d[3] + 16 * v));
  }
}

// Largest byte offset touched + 1 of a side with the given strides.
int64_t extent(const int64_t st[4], int u, int batch, int heads, int64_t rows, int64_t row_bytes) {
  return (u - 1) * st[0] + (batch - 1) * st[1] + (heads - 1) * st[2] + (rows - 1) * st[3] + row_bytes;
}

}  // namespace
}  // namespace cpattn

using namespace cpattn;

extern "C" int32_t cp_attn_ulysses_relayout(int32_t step, int32_t dtype, int32_t u, int32_t batch,
                                            int32_t heads, int64_t rows, int32_t head_dim,
                                            const void *src, void *dst, const int64_t *strides,
                                            void *stream) {
  if (step < CP_ATTN_ULYSSES_SEQ_TO_HEAD_PACK || step > CP_ATTN_ULYSSES_HEAD_TO_SEQ_UNPACK)
    return CP_ATTN_ERR_BAD_LAYOUT;
  if (dtype != CP_ATTN_BF16 && dtype != CP_ATTN_FP32) return CP_ATTN_ERR_UNSUPPORTED;
  if (u < 1 || batch < 1 || heads < 1 || rows < 0 || head_dim < 1) return CP_ATTN_ERR_BAD_SHAPE;
  if (rows >= (int64_t(1) << 31)) return CP_ATTN_ERR_UNSUPPORTED;
  const int64_t el = dtype == CP_ATTN_BF16 ? 2 : 4;
  const int64_t row_bytes = head_dim * el;
  if (row_bytes < 16 || row_bytes > 4096 || (row_bytes & (row_bytes - 1)) != 0) return CP_ATTN_ERR_UNSUPPORTED;
  if (!strides) return CP_ATTN_ERR_NULL_PTR;
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0) return CP_ATTN_ERR_BAD_SHAPE;
    if ((strides[i] * el) % 16 != 0) return CP_ATTN_ERR_ALIGNMENT;
  }
  if (rows == 0) return CP_ATTN_OK;
  if (!src || !dst) return CP_ATTN_ERR_NULL_PTR;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u))
    return CP_ATTN_ERR_ALIGNMENT;

  // Byte strides of (p, b, h, t) on each side.
  const int64_t blk[4] = {batch * heads * rows * row_bytes, heads * rows * row_bytes, rows * row_bytes, row_bytes};
  const int64_t sb = strides[0] * el, sh = strides[1] * el, st = strides[2] * el;
  const int64_t xs[4] = {heads * sh, sb, sh, st};    // x [b][p*heads + h][t]
  const int64_t ys[4] = {rows * st, sb, sh, st};     // y [b][h][p*rows + t]
  const int64_t *s_src, *s_dst;
  switch (step) {
    case CP_ATTN_ULYSSES_SEQ_TO_HEAD_PACK: s_src = xs; s_dst = blk; break;
    case CP_ATTN_ULYSSES_SEQ_TO_HEAD_UNPACK: s_src = blk; s_dst = ys; break;
    case CP_ATTN_ULYSSES_HEAD_TO_SEQ_PACK: s_src = ys; s_dst = blk; break;
    default: s_src = blk; s_dst = xs; break;
  }
  // The buffers must not overlap (byte ranges from each side's extent).
  const char *a = static_cast<const char *>(src), *c = static_cast<const char *>(dst);
  const int64_t ea = extent(s_src, u, batch, heads, rows, row_bytes);
  const int64_t ec = extent(s_dst, u, batch, heads, rows, row_bytes);
  if (a < c + ec && c < a + ea) return CP_ATTN_ERR_BAD_SHAPE;

  RelayoutParams p;
  p.src = a;
  p.dst = static_cast<char *>(dst);
  for (int i = 0; i < 4; ++i) {
    p.s[i] = s_src[i];
    p.d[i] = s_dst[i];
  }
  p.heads = heads;
  p.rows = (int32_t)rows;
  int lg = 0;
  while ((int64_t(16) << lg) < row_bytes) ++lg;
  p.vpr_log2 = lg;
  const int64_t rows_per_block = (int64_t)kUnroll * (kThreads >> lg);
  const dim3 grid((unsigned)((rows + rows_per_block - 1) / rows_per_block), (unsigned)(batch * heads),
                  (unsigned)u);
  hipLaunchKernelGGL(relayout_kernel, grid, dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? CP_ATTN_OK : CP_ATTN_ERR_HIP;
}
