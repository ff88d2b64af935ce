// noalloc.hip -- rvq_encode without a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The workspace is a file-scope device array, `scratch`, of kScratchBytes.
// In host code that name is only a host-side stand-in, so its device
// address is looked up once per device (with that device current, on the
// device's first call) and that address is what the encoder receives.
// Every call on one device shares that device's array: calls that overlap
// on one GPU (two streams, two threads) race and must not be issued.  The
// encoder writes every part of its workspace before reading it, so nothing
// needs clearing between calls.
#include <mutex>

#include "rvq.h"
#include "common.h"

namespace rvq {
rvq_status fail(rvq_status st, const char *fmt, ...);
}

namespace {

constexpr size_t kScratchBytes = (size_t)256 << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

rvq_status scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return rvq::fail(RVQ_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return rvq::fail(RVQ_ERR_UNSUPPORTED, "device %d above the %d devices supported", dev,
                     kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return rvq::fail(RVQ_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return RVQ_OK;
}

}  // namespace

extern "C" rvq_status rvq_encode_noalloc(const void *x, rvq_dtype x_dtype, int64_t n, int32_t d,
                                         const float *codebooks, const void *prepared, int32_t L,
                                         int32_t K, int32_t *ids, float *residual_out,
                                         hipStream_t stream) {
  size_t need = 0;
  rvq_status st = rvq_encode_workspace_size(n, d, L, K, &need);
  if (st != RVQ_OK) return st;
  if (need > kScratchBytes)
    return rvq::fail(RVQ_ERR_UNSUPPORTED,
                     "rvq_encode_noalloc: n=%lld rows of d=%d with L=%d, K=%d need a %zu-byte "
                     "workspace, above its %zu-byte scratch; call rvq_encode with a workspace",
                     (long long)n, d, L, K, need, kScratchBytes);
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != RVQ_OK) return st;
  return rvq_encode(x, x_dtype, n, d, codebooks, prepared, L, K, ids, residual_out, ws,
                    kScratchBytes, stream);
}
