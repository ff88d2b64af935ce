// prep.hip -- codebook preparation and residual initialisation.
//
// The tokenizer is fixed ("LongCat-2.5 Native Multimodality for Agentic
// Tasks", "Visual Primitive Modeling", paragraph "Offline Visual
// Preprocessing"), so the per-codeword data the distance kernel needs is
// derived once per codebook set: ||c||^2 in fp32 and a bf16 copy of every
// codeword, zero-padded to a multiple of the stage width in the feature
// dimension and to a whole number of codeword tiles (padded codewords get
// an infinite norm, so their score is +inf and they are never chosen).
#include "common.h"

namespace rvq {

// One wave per (level, padded codeword).  HBM-bound: reads d*4 bytes and
// writes Dp*2 + 4 bytes per codeword.
__global__ __launch_bounds__(256) void prepare_kernel(const float *__restrict__ cb, int L, int K,
                                                      int d, int Kp, int Dp,
                                                      float *__restrict__ norms,
                                                      uint16_t *__restrict__ cbh) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)L * Kp) return;
  const int l = (int)(w / Kp);
  const int k = (int)(w % Kp);
  uint16_t *dst = cbh + w * Dp;
  if (k >= K) {
    for (int i = lane; i < Dp; i += 64) dst[i] = 0;
    if (lane == 0) norms[w] = __builtin_inff();
    return;
  }
  const float *src = cb + ((int64_t)l * K + k) * d;
  float acc = 0.f;
  for (int i = lane; i < Dp; i += 64) {
    float v = i < d ? src[i] : 0.f;
    acc = fmaf(v, v, acc);
    dst[i] = f32_to_bf16_bits(v);
  }
  acc = wave_sum_f32(acc);
  if (lane == 0) norms[w] = acc;
}

hipError_t launch_prepare(const float *cb, int L, int K, int d, float *norms, uint16_t *cbh,
                          hipStream_t s) {
  const int Kp = (int)padded_k(K), Dp = (int)padded_d(d);
  const int64_t waves = (int64_t)L * Kp;
  prepare_kernel<<<dim3((unsigned)ceil_div(waves, 4)), dim3(256), 0, s>>>(cb, L, K, d, Kp, Dp,
                                                                         norms, cbh);
  return hipGetLastError();
}

// r32 = fp32(x) [n][d];  r16 = bf16(x) [n][Dp], zero-padded.  One wave per row.
__global__ __launch_bounds__(256) void init_residual_kernel(const void *__restrict__ x, int x_bf16,
                                                            int64_t n, int d, int Dp,
                                                            float *__restrict__ r32,
                                                            uint16_t *__restrict__ r16) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  for (int i = lane; i < Dp; i += 64) {
    float v = 0.f;
    if (i < d) {
      v = x_bf16 ? bf16_bits_to_f32(((const uint16_t *)x)[row * d + i])
                 : ((const float *)x)[row * d + i];
      r32[row * d + i] = v;
    }
    r16[row * Dp + i] = f32_to_bf16_bits(v);
  }
}

hipError_t launch_init_residual(const void *x, bool x_bf16, int64_t n, int d, int Dp, float *r32,
                                uint16_t *r16, hipStream_t s) {
  if (n == 0) return hipSuccess;
  init_residual_kernel<<<dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, s>>>(x, x_bf16 ? 1 : 0, n,
                                                                           d, Dp, r32, r16);
  return hipGetLastError();
}

}  // namespace rvq
