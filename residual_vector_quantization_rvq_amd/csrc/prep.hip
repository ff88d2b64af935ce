// prep.hip -- codebook preparation.
//
// The tokenizer is fixed ("LongCat-2.5 Native Multimodality for Agentic
// Tasks", "Visual Primitive Modeling", paragraph "Offline Visual
// Preprocessing"), so the data the distance sweep streams is derived once
// per codebook set: ||c||^2 in fp32 and the fragment-ordered bf16 stream of
// -2c with the norm k-step (layout in common.h).
#include "common.h"

namespace rvq {

// norms[l][k] = ||c_{l,k}||^2 in fp32: lane-strided partial sums, then a
// fixed butterfly.  One wave per (level, padded codeword); padding gets
// kPadNorm.
__global__ __launch_bounds__(256) void norms_kernel(const float *__restrict__ cb, int L, int K,
                                                    int d, int Kp, float *__restrict__ norms) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= (int64_t)L * Kp) return;
  const int l = (int)(w / Kp);
  const int k = (int)(w % Kp);
  if (k >= K) {
    if (lane == 0) norms[w] = kPadNorm;
    return;
  }
  const float *src = cb + ((int64_t)l * K + k) * d;
  float acc = 0.f;
  for (int i = lane; i < d; i += 64) acc = fmaf(src[i], src[i], acc);
  acc = wave_sum_f32(acc);
  if (lane == 0) norms[w] = acc;
}

// One thread per 16-byte chunk of the stream.  Writes are contiguous; each
// group of 256 threads reads 32 codewords x 64 features.
__global__ __launch_bounds__(256) void stream_kernel(const float *__restrict__ cb,
                                                     const float *__restrict__ norms, int L, int K,
                                                     int d, int Kp, int S,
                                                     uint4 *__restrict__ stream) {
  const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int T = Kp / kTileCw;
  const int64_t per_tile = 256 + (int64_t)S * 1024;
  if (chunk >= (int64_t)L * T * per_tile) return;
  const int64_t lt = chunk / per_tile;
  const int c = (int)(chunk % per_tile);
  const int l = (int)(lt / T);
  const int t = (int)(lt % T);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (c < 256) {
    const int j = c >> 6, lane = c & 63;
    if (lane < 32) {
      const int k = t * kTileCw + j * 32 + lane;
      const float nv = norms[(int64_t)l * Kp + k];
      const uint16_t hi = f32_to_bf16_bits(nv);
      const uint16_t lo = k < K ? f32_to_bf16_bits(nv - bf16_bits_to_f32(hi)) : (uint16_t)0;
      w[0] = (uint32_t)hi | ((uint32_t)lo << 16);
    }
  } else {
    const int c2 = c - 256;
    const int s = c2 >> 10, rem = c2 & 1023;
    const int j = rem >> 8, ks = (rem >> 6) & 3, lane = rem & 63;
    const int k = t * kTileCw + j * 32 + (lane & 31);
    const int d0 = s * kStageCols + ks * 16 + (lane >> 5) * 8;
    if (k < K) {
      const float *src = cb + ((int64_t)l * K + k) * d;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float a = d0 + e < d ? -2.0f * src[d0 + e] : 0.f;
        const float b = d0 + e + 1 < d ? -2.0f * src[d0 + e + 1] : 0.f;
        w[e >> 1] = (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
      }
    }
  }
  stream[chunk] = make_uint4(w[0], w[1], w[2], w[3]);
}

// fp32 codebook copy with row stride dp and zero padding.
__global__ __launch_bounds__(256) void pad_codebook_kernel(const float *__restrict__ cb,
                                                           int64_t rows, int d, int dp,
                                                           float *__restrict__ out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= rows * dp) return;
  const int64_t r = e / dp;
  const int i = (int)(e % dp);
  out[e] = i < d ? cb[r * d + i] : 0.f;
}

hipError_t launch_prepare(const float *cb, int L, int K, int d, float *norms, uint8_t *stream,
                          float *cbpad, int dp, hipStream_t s) {
  if (cbpad) {
    const int64_t rows = (int64_t)L * K;
    pad_codebook_kernel<<<dim3((unsigned)ceil_div(rows * dp, 256)), dim3(256), 0, s>>>(cb, rows, d,
                                                                                      dp, cbpad);
  }
  const int Kp = (int)padded_k(K), S = (int)(padded_d(d) / kStageCols);
  const int64_t waves = (int64_t)L * Kp;
  norms_kernel<<<dim3((unsigned)ceil_div(waves, 4)), dim3(256), 0, s>>>(cb, L, K, d, Kp, norms);
  const int64_t chunks = stream_bytes(L, K, d) / 16;
  stream_kernel<<<dim3((unsigned)ceil_div(chunks, 256)), dim3(256), 0, s>>>(
      cb, norms, L, K, d, Kp, S, reinterpret_cast<uint4 *>(stream));
  return hipGetLastError();
}

}  // namespace rvq
