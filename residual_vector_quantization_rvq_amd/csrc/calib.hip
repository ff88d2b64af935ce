// calib.hip -- the matrix cores' achievable bf16 rate on the running chip.
//
// A measurement aid for the distance stage, not a step of the path.  The
// published dense bf16 peak assumes the nominal 2.4 GHz clock; the clock the
// chip holds under a full matrix load depends on how much the operands
// switch.  This kernel issues only v_mfma_f32_32x32x16_bf16 (the encoder's
// instruction) on register operands, one wave per SIMD, four independent
// accumulator chains per wave and no memory traffic inside the timed loop,
// on random or on all-zero operands.
#include <vector>

#include "rvq.h"
#include "common.h"

namespace rvq {
rvq_status fail(rvq_status st, const char *fmt, ...);
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
// flops of one v_mfma_f32_32x32x16_bf16: 32 x 32 outputs, 16 products each
constexpr double kFlopsPerMfma = 2.0 * 32 * 32 * 16;
constexpr int kMfmaPerIter = 8;

// The 32-bit finalizer of MurmurHash3 (fmix32), as published.
__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// Two bf16 values from 32 random bits: random sign, magnitude in
// [0.25, 4) (exponent 2^-2 .. 2^1), random 7-bit mantissa.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t h) {
  const uint32_t lo = ((h & 1u) << 15) | ((125u + ((h >> 1) & 3u)) << 7) | ((h >> 3) & 0x7fu);
  const uint32_t hi =
      (((h >> 10) & 1u) << 15) | ((125u + ((h >> 11) & 3u)) << 7) | ((h >> 13) & 0x7fu);
  return lo | (hi << 16);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
mfma_rate_kernel(int iters, int zero, uint64_t *clocks, float *sink) {
  const uint32_t t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wa[k] = zero ? 0u : bf16_pair(fmix32(t * 32u + (uint32_t)(i * 8 + k)));
      wb[k] = zero ? 0u : bf16_pair(fmix32(t * 32u + (uint32_t)(i * 8 + 4 + k)));
    }
    __builtin_memcpy(&a[i], wa, 16);
    __builtin_memcpy(&b[i], wb, 16);
  }
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaPerIter / 4; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], c[i], 0, 0, 0);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[i][e];
  sink[t] = s;  // keeps the loop's results live
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" size_t rvq_mfma_rate_workspace_size(int32_t blocks) {
  return blocks > 0 ? (size_t)blocks * (2 * sizeof(uint64_t) + kThreads * sizeof(float)) : 0;
}

extern "C" rvq_status rvq_mfma_rate(int32_t blocks, int32_t iters, int32_t zero_operands,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream,
                                    double *tflops, double *clock_ghz) {
  if (blocks < 1 || blocks > 65536)
    return rvq::fail(RVQ_ERR_INVALID_ARGUMENT, "blocks = %d outside 1 .. 65536", blocks);
  if (iters < 10 || iters > 10000000)
    return rvq::fail(RVQ_ERR_INVALID_ARGUMENT, "iters = %d outside 10 .. 10^7", iters);
  if (!workspace || !tflops || !clock_ghz)
    return rvq::fail(RVQ_ERR_INVALID_ARGUMENT, "null workspace or output pointer");
  if ((uintptr_t)workspace % 8 != 0)
    return rvq::fail(RVQ_ERR_INVALID_ARGUMENT, "workspace must be 8-byte aligned");
  if (workspace_bytes < rvq_mfma_rate_workspace_size(blocks))
    return rvq::fail(RVQ_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, %zu needed",
                     workspace_bytes, rvq_mfma_rate_workspace_size(blocks));
  uint64_t *clocks = static_cast<uint64_t *>(workspace);
  float *sink = reinterpret_cast<float *>(clocks + 2 * (size_t)blocks);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  // a short run first, so that the timed one starts from a loaded chip
  if (e == hipSuccess) {
    mfma_rate_kernel<<<dim3(blocks), dim3(kThreads), 0, stream>>>(iters / 10, zero_operands != 0,
                                                                  clocks, sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, stream);
  if (e == hipSuccess) {
    mfma_rate_kernel<<<dim3(blocks), dim3(kThreads), 0, stream>>>(iters, zero_operands != 0,
                                                                  clocks, sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, stream);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  std::vector<uint64_t> host;
  if (e == hipSuccess) {
    host.resize(2 * (size_t)blocks);
    e = hipMemcpy(host.data(), clocks, host.size() * sizeof(uint64_t), hipMemcpyDeviceToHost);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return rvq::fail(RVQ_ERR_HIP, "mfma rate: %s", hipGetErrorString(e));
  // s_memtime counts shader clocks, s_memrealtime a constant 100 MHz
  double ticks = 0.0, real = 0.0;
  for (int i = 0; i < blocks; ++i) {
    ticks += (double)host[2 * i];
    real += (double)host[2 * i + 1];
  }
  const double waves = (double)blocks * (kThreads / 64);
  const double flops = waves * (double)iters * kMfmaPerIter * kFlopsPerMfma;
  *tflops = ms > 0.f ? flops / ((double)ms * 1e-3) / 1e12 : 0.0;
  *clock_ghz = real > 0.0 ? ticks / (real / 100e6) / 1e9 : 0.0;
  return RVQ_OK;
}
