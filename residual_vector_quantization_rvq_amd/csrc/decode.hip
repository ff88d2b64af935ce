// decode.hip -- token IDs back to vectors by summing the chosen codewords.
//
// "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", Figure 1: the
// discrete token sequences are reconstructed; with residual quantization
// the reconstruction from levels 0..levels-1 is the sum of the chosen
// codewords (prefix sums give the coarse-to-fine reconstructions of "02
// Visual Coding and 3D" in "LongCat-2.5 Open Source Release: Meituan's 1.6T
// Multimodal Agent Model with 1M Context").
//
// HBM/MALL-bound gather-sum.  One wave per row (per part of a row when the
// rows are too few to fill the GPU): the row's IDs are read as
// wave-uniform values, and every lane sums its float4 columns over the
// levels in level order in fp32, issuing the gathers of 8 levels before
// adding them.  Output rows are written with non-temporal stores so the
// output stream does not evict the codebook from the caches.
#include "common.h"

namespace rvq {

namespace {

typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store_out(float *o, int64_t i4, float4 v) {
  const nt_f32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nt_f32x4 *>(o) + i4);
}
__device__ __forceinline__ void store_out(uint16_t *o, int64_t i4, float4 v) {
  const uint32_t lo = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
  const nt_u32x2 w = {lo, hi};
  __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x2 *>(o) + i4);
}
__device__ __forceinline__ void store_out1(float *o, int64_t i, float v) { o[i] = v; }
__device__ __forceinline__ void store_out1(uint16_t *o, int64_t i, float v) {
  o[i] = f32_to_bf16_bits(v);
}

}  // namespace

// A wave takes columns [part * span, (part + 1) * span) of one row (float4
// columns when d % 4 == 0, else single ones); span covers the whole row
// unless rows are too few to fill the GPU, when a row is split over several
// waves.  Every element is the same level-order sum either way.
template <typename OutT>
__global__ __launch_bounds__(256) void decode_kernel(const int32_t *__restrict__ ids, int64_t n,
                                                     const float *__restrict__ cb, int L, int K,
                                                     int d, int levels, OutT *__restrict__ out,
                                                     uint32_t *__restrict__ bad, int parts,
                                                     int span) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * 4 + wave;  // wave-uniform
  const int64_t row = gw / parts;
  const int part = (int)(gw - row * parts);
  if (row >= n) return;
  const int32_t *rid = ids + row * L;
  if (bad && part == 0) {  // count out-of-range IDs once per row (levels <= 64, checked on the host)
    const int my_id = lane < levels ? rid[lane] : 0;
    const unsigned long long bad_mask = __ballot(my_id < 0 || my_id >= K);
    if (lane == 0 && bad_mask) atomicAdd(bad, (uint32_t)__popcll(bad_mask));
  }

  if ((d & 3) == 0) {
    const int d4 = d >> 2;
    const int c1 = min(d4, (part + 1) * span);
    const float4 *cb4 = reinterpret_cast<const float4 *>(cb);
    for (int i4 = part * span + lane; i4 < c1; i4 += 64) {
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int l0 = 0; l0 < levels; l0 += 8) {
        float4 v[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int l = l0 + u;
          const int id = l < levels ? rid[l] : -1;  // uniform load
          ok[u] = id >= 0 && id < K;
          v[u] = ok[u] ? cb4[((int64_t)l * K + id) * d4 + i4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (ok[u]) {  // level order; skipped levels add nothing
            acc.x += v[u].x;
            acc.y += v[u].y;
            acc.z += v[u].z;
            acc.w += v[u].w;
          }
        }
      }
      store_out(out + row * d, i4, acc);
    }
  } else {
    const int c1 = min(d, (part + 1) * span);
    for (int i = part * span + lane; i < c1; i += 64) {
      float acc = 0.f;
      for (int l = 0; l < levels; ++l) {
        const int id = rid[l];
        if (id >= 0 && id < K) acc += cb[((int64_t)l * K + id) * d + i];
      }
      store_out1(out + row * d, i, acc);
    }
  }
}

hipError_t launch_decode(const int32_t *ids, int64_t n, const float *cb, int L, int K, int d,
                         int levels, void *out, bool out_bf16, uint32_t *bad, hipStream_t s) {
  if (n == 0) return hipSuccess;
  // columns per row in the kernel's units; with fewer than 8 waves per
  // compute unit's worth of rows, split rows into 64-column parts
  const int cols = (d & 3) == 0 ? d >> 2 : d;
  const int whole = (int)ceil_div(cols, 64);
  const int parts = n >= 8 * 1024 ? 1 : whole;
  const int span = (int)ceil_div(cols, parts);
  const dim3 grid((unsigned)ceil_div(n * parts, 4)), block(256);
  if (out_bf16)
    decode_kernel<uint16_t><<<grid, block, 0, s>>>(ids, n, cb, L, K, d, levels, (uint16_t *)out,
                                                   bad, parts, span);
  else
    decode_kernel<float><<<grid, block, 0, s>>>(ids, n, cb, L, K, d, levels, (float *)out, bad,
                                                parts, span);
  return hipGetLastError();
}

}  // namespace rvq
