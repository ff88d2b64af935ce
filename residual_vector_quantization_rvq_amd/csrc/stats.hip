// stats.hip -- per-level codeword usage counts and mean squared residual.
//
// Visual token counts and codeword usage matter for the pages' offline
// preprocessing and load balancing ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
// "Visual Primitive Modeling", paragraph "Offline Visual Preprocessing");
// the mean squared residual after each level measures how much detail each
// level adds ("LongCat-2.5 Open Source Release: Meituan's 1.6T Multimodal
// Agent Model with 1M Context", "02 Visual Coding and 3D").  Both are exact or fixed-order reductions: counts
// are integers, and the fp64 sums are reduced in an order that depends only
// on n, so results are bitwise reproducible.
//
// The mean-squared-residual pass gathers every level's codeword of every
// row, which is exactly what decoding needs; with an output buffer it also
// writes the full reconstruction (sum of the codewords in level order, in
// fp32, skipping out-of-range IDs), bit for bit what the decode kernel
// writes, so decode and statistics of the same IDs cost one gather pass.
#include "common.h"

namespace rvq {

namespace {

constexpr int kHistLdsMaxK = 16384;  // LDS counters: K * 4 bytes <= 64 KB
// All levels in one workgroup: L * K 16-bit counters, two to a 32-bit LDS
// word (128 KB), over chunks of at most 65535 rows so no counter overflows.
constexpr int kHistPackedMaxLK = 65536;
constexpr int64_t kHistPackedRows = 65535;

int64_t hist_packed_chunks(int64_t n) {
  int64_t c = ceil_div(n, 512);   // at least 512 rows per workgroup
  if (c > 256) c = 256;           // about one workgroup per compute unit
  const int64_t need = ceil_div(n, kHistPackedRows);
  if (c < need) c = need;
  if (c < 1) c = 1;
  return c;
}

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

// Workgroup per chunk of rows, every level: the chunk's IDs are read once,
// contiguously, and counted in 16-bit LDS counters of (level, codeword);
// partial[chunk] receives the counter words as they are.  The counters take
// 128 KB, so one workgroup fills a compute unit: 16 waves, each thread
// with eight loads in flight before its atomics.
constexpr int kHistPackedThreads = 1024;
__global__ __launch_bounds__(kHistPackedThreads) void hist_packed_kernel(
    const int32_t *__restrict__ ids, int64_t n, int L, int K, int64_t rows_per_chunk,
    uint32_t *__restrict__ partial, uint32_t *__restrict__ bad) {
  constexpr int T = kHistPackedThreads, U = 8;
  __shared__ uint32_t cnt[kHistPackedMaxLK / 2];
  const int words = (L * K + 1) >> 1;
  for (int w = threadIdx.x; w < words; w += T) cnt[w] = 0;
  __syncthreads();
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_chunk;
  int64_t r1 = r0 + rows_per_chunk;
  if (r1 > n) r1 = n;
  const int32_t *src = ids + r0 * L;
  // (rows_per_chunk * L < 2^32 - 2^16: at most 65535 rows and L <= 65536)
  const uint32_t count = r1 > r0 ? (uint32_t)((r1 - r0) * L) : 0u;
  uint32_t nbad = 0;
  // the level of element e is e % L, carried along as e steps by T
  const uint32_t step = (uint32_t)T % (uint32_t)L;
  uint32_t l = threadIdx.x % (uint32_t)L;
  for (uint32_t base = threadIdx.x; base < count; base += T * U) {
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = base + u * T < count ? src[base + u * T] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * T < count) {
        if (v[u] >= 0 && v[u] < K) {
          const uint32_t c = l * (uint32_t)K + (uint32_t)v[u];
          atomicAdd(&cnt[c >> 1], 1u << ((c & 1u) << 4));
        } else {
          ++nbad;
        }
      }
      l += step;
      if (l >= (uint32_t)L) l -= (uint32_t)L;
    }
  }
  if (bad) {
    const unsigned long long m = __ballot(nbad != 0);
    if (m) {
      uint32_t t = nbad;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
      if ((threadIdx.x & 63) == 0) atomicAdd(bad, t);
    }
  }
  __syncthreads();
  uint32_t *dst = partial + (int64_t)blockIdx.x * words;
  for (int w = threadIdx.x; w < words; w += T) dst[w] = cnt[w];
}

// hist[l][k] = sum over chunks of the 16-bit counter (l, k) of partial[chunk].
// A workgroup takes 16 counter words (32 counters): thread (g, w) sums word
// w of chunks g, g + 16, ..., then the 16 partial sums of each word are
// added in LDS (integers: the order does not matter).
__global__ __launch_bounds__(256) void hist_packed_reduce_kernel(
    const uint32_t *__restrict__ partial, int64_t chunks, int L, int K,
    int64_t *__restrict__ hist) {
  __shared__ int64_t lo_sum[16][16], hi_sum[16][16];
  const int wl = threadIdx.x & 15, g = threadIdx.x >> 4;
  const int64_t lk = (int64_t)L * K;
  const int64_t words = (lk + 1) >> 1;
  const int64_t w = (int64_t)blockIdx.x * 16 + wl;
  int64_t lo = 0, hi = 0;
  if (w < words) {
#pragma unroll 8
    for (int64_t c = g; c < chunks; c += 16) {
      const uint32_t v = partial[c * words + w];
      lo += v & 0xffffu;
      hi += v >> 16;
    }
  }
  lo_sum[g][wl] = lo;
  hi_sum[g][wl] = hi;
  __syncthreads();
  if (g == 0 && w < words) {
    for (int j = 1; j < 16; ++j) {
      lo += lo_sum[j][wl];
      hi += hi_sum[j][wl];
    }
    hist[2 * w] = lo;
    if (2 * w + 1 < lk) hist[2 * w + 1] = hi;
  }
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
  if ((int64_t)L * K <= kHistPackedMaxLK)
    return (size_t)hist_packed_chunks(n) * (size_t)(((int64_t)L * K + 1) >> 1) * sizeof(uint32_t);
  if (K > kHistLdsMaxK) return 0;
  return (size_t)hist_chunks(n, L) * (size_t)L * (size_t)K * sizeof(uint32_t);
}

hipError_t launch_hist(const int32_t *ids, int64_t n, int L, int K, int64_t *hist,
                       uint32_t *partial, uint32_t *bad, hipStream_t s) {
  const int64_t lk = (int64_t)L * K;
  if (lk <= kHistPackedMaxLK) {
    const int64_t chunks = hist_packed_chunks(n);
    const int64_t rpc = ceil_div(n > 0 ? n : 1, chunks);
    hist_packed_kernel<<<dim3((unsigned)chunks), dim3(kHistPackedThreads), 0, s>>>(
        ids, n, L, K, rpc, partial, bad);
    hist_packed_reduce_kernel<<<dim3((unsigned)ceil_div((lk + 1) >> 1, 16)), dim3(256), 0, s>>>(
        partial, chunks, L, K, hist);
  } else if (K <= kHistLdsMaxK) {
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

// Each workgroup takes kMsrRowsPerBlock consecutive rows; wave w takes rows
// w, w+4, ... of them.  A lane owns float4 column groups of its row (scalar
// columns when d is not a multiple of 4), subtracts the row's codewords
// level by level in fp32, with the gathers of up to kMsrLevelChunk levels
// in flight, and accumulates each level's squared residual in fp64 over its
// rows in order.  The wave then sums lanes in a fixed butterfly and the
// workgroup sums its waves in order, so every sum's order depends only on n.
// An out-of-range ID adds nothing (the histogram pass counts it).
// Levels past kMsrLevelChunk are done in further passes that recompute the
// residual prefix.
constexpr int kMsrRowsPerBlock = 32;
constexpr int kMsrLevelChunk = 8;

__device__ __forceinline__ float4 load_x4(const void *x, bool x_bf16, int64_t row, int d4, int i4) {
  if (x_bf16) {
    const uint2 b = reinterpret_cast<const uint2 *>(x)[row * d4 + i4];
    return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                       __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u));
  }
  return reinterpret_cast<const float4 *>(x)[row * d4 + i4];
}

__device__ __forceinline__ double sq4(double acc, float4 r) {
  acc = fma((double)r.x, (double)r.x, acc);
  acc = fma((double)r.y, (double)r.y, acc);
  acc = fma((double)r.z, (double)r.z, acc);
  return fma((double)r.w, (double)r.w, acc);
}

// Decoded output of the fused pass: OUT 0 none, 1 fp32, 2 bf16 (rounded to
// nearest even); stored non-temporally like the decode kernel's.
typedef float msr_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t msr_u32x2 __attribute__((ext_vector_type(2)));
template <int OUT>
__device__ __forceinline__ void store_dec4(void *out, int64_t row, int d4, int i4, float4 v) {
  if constexpr (OUT == 1) {
    const msr_f32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<msr_f32x4 *>(out) + row * d4 + i4);
  } else if constexpr (OUT == 2) {
    const uint32_t lo = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
    const msr_u32x2 w = {lo, hi};
    __builtin_nontemporal_store(w, reinterpret_cast<msr_u32x2 *>(out) + row * d4 + i4);
  }
}
template <int OUT>
__device__ __forceinline__ void store_dec1(void *out, int64_t i, float v) {
  if constexpr (OUT == 1) reinterpret_cast<float *>(out)[i] = v;
  else if constexpr (OUT == 2) reinterpret_cast<uint16_t *>(out)[i] = f32_to_bf16_bits(v);
}

template <bool VEC, int OUT>
__global__ __launch_bounds__(256) void msr_rows_kernel(const void *__restrict__ x, int x_bf16,
                                                       const int32_t *__restrict__ ids, int64_t n,
                                                       int d, const float *__restrict__ cb, int L,
                                                       int K, double *__restrict__ partial,
                                                       int64_t nblocks, void *__restrict__ out) {
  __shared__ double wsum[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t r0 = (int64_t)blockIdx.x * kMsrRowsPerBlock;
  const int d4 = d >> 2;
  const float4 *cb4 = reinterpret_cast<const float4 *>(cb);
  for (int lc = 0; lc < L; lc += kMsrLevelChunk) {
    double sq[kMsrLevelChunk];
#pragma unroll
    for (int u = 0; u < kMsrLevelChunk; ++u) sq[u] = 0.0;
    for (int j = wave; j < kMsrRowsPerBlock; j += 4) {
      const int64_t row = r0 + j;  // wave-uniform
      if (row >= n) break;
      const int32_t *rid = ids + row * L;
      // the decoded row (sum of the codewords in level order) is complete
      // in the last level chunk
      const bool dec = OUT != 0 && lc + kMsrLevelChunk >= L;
      if constexpr (VEC) {
        for (int i4 = lane; i4 < d4; i4 += 64) {
          float4 r = load_x4(x, x_bf16, row, d4, i4);
          float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
          for (int l = 0; l < lc; ++l) {
            const int id = rid[l];
            if (id >= 0 && id < K) {
              const float4 c = cb4[((int64_t)l * K + id) * d4 + i4];
              r.x -= c.x; r.y -= c.y; r.z -= c.z; r.w -= c.w;
              if (OUT != 0) { acc.x += c.x; acc.y += c.y; acc.z += c.z; acc.w += c.w; }
            }
          }
          float4 v[kMsrLevelChunk];
          bool ok[kMsrLevelChunk];
#pragma unroll
          for (int u = 0; u < kMsrLevelChunk; ++u) {
            const int l = lc + u;
            const int id = l < L ? rid[l] : -1;  // uniform load
            ok[u] = id >= 0 && id < K;
            v[u] = ok[u] ? cb4[((int64_t)l * K + id) * d4 + i4] : make_float4(0.f, 0.f, 0.f, 0.f);
          }
#pragma unroll
          for (int u = 0; u < kMsrLevelChunk; ++u) {
            if (lc + u < L) {
              r.x -= v[u].x; r.y -= v[u].y; r.z -= v[u].z; r.w -= v[u].w;
              sq[u] = sq4(sq[u], r);
              if (OUT != 0 && ok[u]) {
                acc.x += v[u].x; acc.y += v[u].y; acc.z += v[u].z; acc.w += v[u].w;
              }
            }
          }
          if (dec) store_dec4<OUT>(out, row, d4, i4, acc);
        }
      } else {
        for (int i = lane; i < d; i += 64) {
          float r = x_bf16 ? bf16_bits_to_f32(((const uint16_t *)x)[row * d + i])
                           : ((const float *)x)[row * d + i];
          float acc = 0.f;
          for (int l = 0; l < lc; ++l) {
            const int id = rid[l];
            if (id >= 0 && id < K) {
              const float c = cb[((int64_t)l * K + id) * d + i];
              r -= c;
              if (OUT != 0) acc += c;
            }
          }
#pragma unroll
          for (int u = 0; u < kMsrLevelChunk; ++u) {
            const int l = lc + u;
            if (l < L) {
              const int id = rid[l];
              if (id >= 0 && id < K) {
                const float c = cb[((int64_t)l * K + id) * d + i];
                r -= c;
                if (OUT != 0) acc += c;
              }
              sq[u] = fma((double)r, (double)r, sq[u]);
            }
          }
          if (dec) store_dec1<OUT>(out, row * d + i, acc);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kMsrLevelChunk; ++u) {
      const double t = wave_sum_f64(sq[u]);
      if (lane == 0 && lc + u < L) wsum[wave][lc + u] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x < L) {
    const int l = threadIdx.x;
    double s = wsum[0][l];
    s += wsum[1][l];
    s += wsum[2][l];
    s += wsum[3][l];
    partial[(int64_t)l * nblocks + blockIdx.x] = s;
  }
}

// msr[l] = (sum of the workgroup partials) / n, partials stored level-major;
// workgroup l: thread t sums partials t, t+256, ... in order, then a fixed
// tree over the 256 threads.
__global__ __launch_bounds__(256) void msr_final_kernel(const double *__restrict__ partial,
                                                        int64_t nblocks, int64_t n,
                                                        double *__restrict__ msr) {
  __shared__ double sh[256];
  const int l = blockIdx.x;
  double s = 0.0;
  for (int64_t b = threadIdx.x; b < nblocks; b += 256) s += partial[(int64_t)l * nblocks + b];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) msr[l] = n > 0 ? sh[0] / (double)n : 0.0;
}

size_t msr_partial_bytes(int64_t n, int L) {
  const int64_t blocks = n > 0 ? ceil_div(n, kMsrRowsPerBlock) : 1;
  return (size_t)blocks * (size_t)L * sizeof(double);
}

hipError_t launch_msr(const void *x, bool x_bf16, const int32_t *ids, int64_t n, int d,
                      const float *cb, int L, int K, double *msr, double *partial, void *out,
                      int out_kind, hipStream_t s) {
  const int64_t blocks = n > 0 ? ceil_div(n, kMsrRowsPerBlock) : 0;
  // float4 columns need d % 4 == 0 and 16-byte (fp32) / 8-byte (bf16) row starts,
  // which an aligned base pointer then gives for every row; rows that start
  // less aligned (a slice of a larger batch) take the per-element path
  const bool vec = (d & 3) == 0 && ((uintptr_t)x & (x_bf16 ? 7 : 15)) == 0;
  if (blocks > 0) {
    const dim3 grid((unsigned)blocks), block(256);
#define RVQ_MSR(V, O)                                                                    \
  msr_rows_kernel<V, O><<<grid, block, 0, s>>>(x, x_bf16 ? 1 : 0, ids, n, d, cb, L, K, \
                                               partial, blocks, out)
    if (vec) {
      if (out_kind == 1) RVQ_MSR(true, 1);
      else if (out_kind == 2) RVQ_MSR(true, 2);
      else RVQ_MSR(true, 0);
    } else {
      if (out_kind == 1) RVQ_MSR(false, 1);
      else if (out_kind == 2) RVQ_MSR(false, 2);
      else RVQ_MSR(false, 0);
    }
#undef RVQ_MSR
  }
  msr_final_kernel<<<dim3((unsigned)L), dim3(256), 0, s>>>(partial, blocks, n, msr);
  return hipGetLastError();
}

}  // namespace rvq
