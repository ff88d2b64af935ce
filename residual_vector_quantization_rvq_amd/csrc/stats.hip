// stats.hip -- per-level codeword usage counts and mean squared residual.
//
// Visual token counts and codeword usage matter for the pages' offline
// preprocessing and load balancing ("LongCat-2.5 Native Multimodality for
// Agentic Tasks", "Visual Primitive Modeling", paragraph "Offline Visual
// Preprocessing"); the mean squared residual after each level measures how
// much detail each level adds ("LongCat-2.5 Open Source Release ...", "02
// Visual Coding and 3D").  Both are exact or fixed-order reductions: counts
// are integers, and the fp64 sums are reduced in an order that depends only
// on n, so results are bitwise reproducible.
#include "common.h"

namespace rvq {

namespace {

constexpr int kHistLdsMaxK = 16384;  // LDS counters: K * 4 bytes <= 64 KB

int64_t hist_chunks(int64_t n, int L) {
  int64_t c = ceil_div(n, 8192);
  const int64_t cap = L >= 1024 ? 1 : 1024 / L;
  if (c > cap) c = cap;
  if (c < 1) c = 1;
  return c;
}

}  // namespace

// Workgroup (chunk, level): LDS counters for one level over a chunk of rows.
__global__ __launch_bounds__(256) void hist_partial_kernel(const int32_t *__restrict__ ids,
                                                           int64_t n, int L, int K,
                                                           int64_t rows_per_chunk,
                                                           uint32_t *__restrict__ partial,
                                                           uint32_t *__restrict__ bad) {
  extern __shared__ uint32_t cnt[];
  const int l = blockIdx.x % L;
  const int64_t chunk = blockIdx.x / L;
  for (int k = threadIdx.x; k < K; k += 256) cnt[k] = 0;
  __syncthreads();
  const int64_t r0 = chunk * rows_per_chunk;
  int64_t r1 = r0 + rows_per_chunk;
  if (r1 > n) r1 = n;
  uint32_t nbad = 0;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += 256) {
    const int id = ids[r * L + l];
    if (id >= 0 && id < K)
      atomicAdd(&cnt[id], 1u);
    else
      ++nbad;
  }
  if (bad) {
    const unsigned long long m = __ballot(nbad != 0);
    if (m) {
      uint32_t s = nbad;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
      if ((threadIdx.x & 63) == 0) atomicAdd(bad, s);
    }
  }
  __syncthreads();
  uint32_t *dst = partial + ((int64_t)chunk * L + l) * K;
  for (int k = threadIdx.x; k < K; k += 256) dst[k] = cnt[k];
}

// hist[l][k] = sum over chunks of partial[chunk][l][k], chunks in order.
__global__ __launch_bounds__(256) void hist_reduce_kernel(const uint32_t *__restrict__ partial,
                                                          int64_t chunks, int L, int K,
                                                          int64_t *__restrict__ hist) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)L * K) return;
  int64_t s = 0;
  for (int64_t c = 0; c < chunks; ++c) s += partial[c * L * K + e];
  hist[e] = s;
}

__global__ __launch_bounds__(256) void fill_zero_i64_kernel(int64_t *__restrict__ p, int64_t count) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < count) p[e] = 0;
}

// Large-K path: integer atomics straight into the int64 counts.
__global__ __launch_bounds__(256) void hist_atomic_kernel(const int32_t *__restrict__ ids,
                                                          int64_t n, int L, int K,
                                                          int64_t *__restrict__ hist,
                                                          uint32_t *__restrict__ bad) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n * L) return;
  const int l = (int)(e % L);
  const int id = ids[e];
  if (id >= 0 && id < K)
    atomicAdd(reinterpret_cast<unsigned long long *>(hist + (int64_t)l * K + id), 1ull);
  else if (bad)
    atomicAdd(bad, 1u);
}

size_t hist_partial_bytes(int64_t n, int L, int K) {
  if (K > kHistLdsMaxK) return 0;
  return (size_t)hist_chunks(n, L) * (size_t)L * (size_t)K * sizeof(uint32_t);
}

hipError_t launch_hist(const int32_t *ids, int64_t n, int L, int K, int64_t *hist,
                       uint32_t *partial, uint32_t *bad, hipStream_t s) {
  const int64_t lk = (int64_t)L * K;
  if (K <= kHistLdsMaxK) {
    const int64_t chunks = hist_chunks(n, L);
    const int64_t rpc = ceil_div(n > 0 ? n : 1, chunks);
    hist_partial_kernel<<<dim3((unsigned)(chunks * L)), dim3(256), (size_t)K * sizeof(uint32_t), s>>>(
        ids, n, L, K, rpc, partial, bad);
    hist_reduce_kernel<<<dim3((unsigned)ceil_div(lk, 256)), dim3(256), 0, s>>>(partial, chunks, L,
                                                                              K, hist);
  } else {
    fill_zero_i64_kernel<<<dim3((unsigned)ceil_div(lk, 256)), dim3(256), 0, s>>>(hist, lk);
    if (n > 0)
      hist_atomic_kernel<<<dim3((unsigned)ceil_div(n * L, 256)), dim3(256), 0, s>>>(ids, n, L, K,
                                                                                   hist, bad);
  }
  return hipGetLastError();
}

// One wave per row, 4 rows per workgroup.  Each lane walks its columns,
// subtracting the row's codewords level by level in fp32 and accumulating
// the squared residual of every level in fp64; the wave then sums lanes in
// a fixed butterfly, and the workgroup sums its 4 rows in wave order.
constexpr int kMsrLevelChunk = 16;

__global__ __launch_bounds__(256) void msr_rows_kernel(const void *__restrict__ x, int x_bf16,
                                                       const int32_t *__restrict__ ids, int64_t n,
                                                       int d, const float *__restrict__ cb, int L,
                                                       int K, double *__restrict__ partial,
                                                       uint32_t *__restrict__ bad) {
  __shared__ double rowsum[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const bool live = row < n;
  const int32_t *rid = ids + (live ? row : 0) * L;
  if (live && bad) {
    const int my_id = lane < L ? rid[lane] : 0;
    const unsigned long long m = __ballot(my_id < 0 || my_id >= K);
    if (lane == 0 && m) atomicAdd(bad, (uint32_t)__popcll(m));
  }
  for (int lc = 0; lc < L; lc += kMsrLevelChunk) {
    double sq[kMsrLevelChunk];
#pragma unroll
    for (int u = 0; u < kMsrLevelChunk; ++u) sq[u] = 0.0;
    if (live) {
      for (int i = lane; i < d; i += 64) {
        float r = x_bf16 ? bf16_bits_to_f32(((const uint16_t *)x)[row * d + i])
                         : ((const float *)x)[row * d + i];
        for (int l = 0; l < lc; ++l) {
          const int id = rid[l];
          if (id >= 0 && id < K) r -= cb[((int64_t)l * K + id) * d + i];
        }
#pragma unroll
        for (int u = 0; u < kMsrLevelChunk; ++u) {
          const int l = lc + u;
          if (l < L) {
            const int id = rid[l];
            if (id >= 0 && id < K) r -= cb[((int64_t)l * K + id) * d + i];
            sq[u] += (double)r * (double)r;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kMsrLevelChunk; ++u) {
      const double t = wave_sum_f64(sq[u]);
      if (lane == 0 && lc + u < L) rowsum[wave][lc + u] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x < L) {
    const int l = threadIdx.x;
    double s = rowsum[0][l];
    s += rowsum[1][l];
    s += rowsum[2][l];
    s += rowsum[3][l];
    partial[(int64_t)blockIdx.x * L + l] = s;
  }
}

// msr[l] = (sum of the workgroup partials) / n; thread t sums partials
// t, t+256, ... in order, then a fixed tree over the 256 threads.
__global__ __launch_bounds__(256) void msr_final_kernel(const double *__restrict__ partial,
                                                        int64_t nblocks, int L, int64_t n,
                                                        double *__restrict__ msr) {
  __shared__ double sh[256];
  for (int l = 0; l < L; ++l) {
    double s = 0.0;
    for (int64_t b = threadIdx.x; b < nblocks; b += 256) s += partial[b * L + l];
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) msr[l] = n > 0 ? sh[0] / (double)n : 0.0;
    __syncthreads();
  }
}

size_t msr_partial_bytes(int64_t n, int L) {
  const int64_t blocks = n > 0 ? ceil_div(n, 4) : 1;
  return (size_t)blocks * (size_t)L * sizeof(double);
}

hipError_t launch_msr(const void *x, bool x_bf16, const int32_t *ids, int64_t n, int d,
                      const float *cb, int L, int K, double *msr, double *partial, uint32_t *bad,
                      hipStream_t s) {
  const int64_t blocks = n > 0 ? ceil_div(n, 4) : 0;
  if (blocks > 0)
    msr_rows_kernel<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(x, x_bf16 ? 1 : 0, ids, n, d, cb,
                                                                 L, K, partial, bad);
  msr_final_kernel<<<dim3(1), dim3(256), 0, s>>>(partial, blocks, L, n, msr);
  return hipGetLastError();
}

}  // namespace rvq
