// cp_attn_bwd_noalloc: the share's backward without a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The backward's scratch is its per-row statistics: -Delta and LSE *
// log2(e), each [batch, hq, sq_local] float32, and with a user mask the
// mask's bit tables (the workspace of cp_attn_bwd, less the partial dK/dV
// of split key tiles, which this entry point never splits). Here it lives in
// a file-scope device array, `scratch`, of a fixed size; each GPU the library runs on holds its own copy of it until the
// process ends. Host code never passes the array's name to a kernel (in host
// code it is a stand-in, not a device address): the device address is looked
// up once per device with hipGetSymbolAddress and kept in a table.
#include <hip/hip_runtime.h>

#include <mutex>

#include "cp_attn.h"
#include "plan.h"

namespace {

// -Delta and LSE * log2(e) for up to CP_ATTN_NOALLOC_MAX_ROWS rows each, every
// array starting on a 256-byte boundary (the layout cp_attn_bwd gives its
// workspace); a share's bit tables follow its statistics when all fit.
constexpr size_t kStatBytes = ((size_t)CP_ATTN_NOALLOC_MAX_ROWS * 4 + 255) & ~(size_t)255;
constexpr size_t kScratchBytes = 2 * kStatBytes;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];   // device address of `scratch` per device ordinal (NULL: not looked up yet)

// Device address of this device's `scratch`, looked up on the first call on
// the device with that device current. Returns NULL on a HIP error.
void *scratch_of(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev]) return g_scratch[dev];
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return nullptr;
  if (prev != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (prev != dev) (void)hipSetDevice(prev);
  if (e != hipSuccess || !ptr) return nullptr;
  g_scratch[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" int32_t cp_attn_bwd_noalloc(const cp_attn_desc *desc, const void *q, const void *k,
                                       const void *v, const void *out, const float *lse,
                                       const void *dout, void *dq, float *dk, float *dv,
                                       void *stream) {
  const int32_t st = cp_attn_validate(desc);
  if (st) return st;
  const int64_t rows = (int64_t)desc->batch * desc->hq * desc->sq_local;
  if (rows > CP_ATTN_NOALLOC_MAX_ROWS || cpattn::bwd_workspace_bytes(desc, false) > kScratchBytes)
    return CP_ATTN_ERR_SCRATCH_LIMIT;
  if (rows == 0 && desc->skv == 0) return CP_ATTN_OK;
  int dev = -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return CP_ATTN_ERR_HIP;
  void *ws = scratch_of(dev);
  if (!ws) return CP_ATTN_ERR_HIP;
  // The statistics pass writes every row of both arrays before the main
  // kernels read them, so nothing needs clearing between calls. Key tiles are
  // never split here (the scratch holds no partial dK/dV).
  return cpattn::bwd_run(desc, q, k, v, out, lse, dout, dq, dk, dv, ws, kScratchBytes, stream, nullptr, 0,
                         false);
}
