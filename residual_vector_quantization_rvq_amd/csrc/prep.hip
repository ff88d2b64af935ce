// prep.hip -- codebook preparation (one pass over the fp32 codebooks).
//
// The tokenizer is fixed ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
// "Visual Primitive Modeling", paragraph "Offline Visual Preprocessing"), so
// the data the distance sweep streams is derived once per codebook set:
// ||c||^2 in fp32 and the fragment-ordered bf16 stream of -2c with the norm
// k-step (layout in common.h).
#include "common.h"

namespace rvq {

// One workgroup per (level, 128-codeword tile), one pass over the tile's
// codewords.  Wave j takes sub-tile j (32 codewords); lane L takes codeword
// j*32 + L%32 and half h = L/32 of every k-step, i.e. exactly the 16-byte
// chunks it writes into the stream (features s*64 + ks*16 + h*8 .. +7 of
// stage s, k-step ks), so each wave writes 1 KB contiguous per k-step.  The
// lane sums the squares of its features in increasing order (fmaf), and
// ||c||^2 = (half 0) + (half 1).  Padded codewords (index >= K) are zero
// with norm kPadNorm.  The tile's largest ||c||^2 and ||c - bf16(c)||^2 over
// its real codewords go to tstat (terms of the encoder's band bound).
__global__ __launch_bounds__(256) void prepare_tile_kernel(const float *__restrict__ cb, int L,
                                                           int K, int d, int Kp, int S,
                                                           float *__restrict__ norms,
                                                           uint4 *__restrict__ stream,
                                                           float *__restrict__ tstat) {
  __shared__ float red[2][4];
  const int T = Kp / kTileCw;
  const int l = blockIdx.x / T, t = blockIdx.x % T;
  const int lane = threadIdx.x & 63;
  const int j = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int k = t * kTileCw + j * 32 + (lane & 31);
  const bool real = k < K;
  const float *src = cb + ((int64_t)l * K + (real ? k : 0)) * d;
  const bool vec = (d & 3) == 0;
  uint4 *tile = stream + ((int64_t)l * T + t) * (tile_bytes(S) / 16);
  float acc = 0.f, dacc = 0.f;
  // two stages (eight k-steps) per pass: all sixteen loads are issued before
  // the first is used; the squares are still summed in feature order
  for (int s0 = 0; s0 < S; s0 += 2) {
    float v[8][8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + (u >> 2), ks = u & 3;
      const int d0 = s * kStageCols + ks * 16 + h * 8;
      if (s < S && real && vec && d0 + 8 <= d) {
        const float4 a = *reinterpret_cast<const float4 *>(src + d0);
        const float4 b = *reinterpret_cast<const float4 *>(src + d0 + 4);
        v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
        v[u][4] = b.x; v[u][5] = b.y; v[u][6] = b.z; v[u][7] = b.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[u][e] = (s < S && real && d0 + e < d) ? src[d0 + e] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + (u >> 2), ks = u & 3;
      if (s >= S) break;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        acc = fmaf(v[u][e], v[u][e], acc);
        acc = fmaf(v[u][e + 1], v[u][e + 1], acc);
        const float r0 = v[u][e] - bf16_bits_to_f32(f32_to_bf16_bits(v[u][e]));
        const float r1 = v[u][e + 1] - bf16_bits_to_f32(f32_to_bf16_bits(v[u][e + 1]));
        dacc = fmaf(r0, r0, dacc);
        dacc = fmaf(r1, r1, dacc);
        w[e >> 1] = (uint32_t)f32_to_bf16_bits(-2.0f * v[u][e]) |
                    ((uint32_t)f32_to_bf16_bits(-2.0f * v[u][e + 1]) << 16);
      }
      tile[256 + s * 1024 + (j * 4 + ks) * 64 + lane] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
  const float other = __shfl_xor(acc, 32, 64);
  const float nv = real ? (h ? other + acc : acc + other) : kPadNorm;
  uint32_t w0 = 0u;
  if (h == 0) {
    const uint16_t hi = f32_to_bf16_bits(nv);
    const uint16_t lo = real ? f32_to_bf16_bits(nv - bf16_bits_to_f32(hi)) : (uint16_t)0;
    w0 = (uint32_t)hi | ((uint32_t)lo << 16);
    norms[(int64_t)l * Kp + k] = nv;
  }
  tile[j * 64 + lane] = make_uint4(w0, 0u, 0u, 0u);
  // tile maxima over real codewords (both halves hold the same codeword
  // total, so the halves' maxima agree on the norm)
  float m0 = real ? nv : 0.f;
  float m1 = real ? dacc + __shfl_xor(dacc, 32, 64) : 0.f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
    m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
  }
  if (lane == 0) {
    red[0][j] = m0;
    red[1][j] = m1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    tstat[((int64_t)l * T + t) * 2] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    tstat[((int64_t)l * T + t) * 2 + 1] =
        fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  }
}

// lstat[l] = (max ||c||^2, max ||c - bf16(c)||^2, 0, 0) over level l's tiles.
__global__ __launch_bounds__(256) void level_stat_kernel(const float *__restrict__ tstat, int T,
                                                         float *__restrict__ lstat) {
  __shared__ float red[2][4];
  const int l = blockIdx.x;
  float m0 = 0.f, m1 = 0.f;
  for (int t = threadIdx.x; t < T; t += 256) {
    m0 = fmaxf(m0, tstat[((int64_t)l * T + t) * 2]);
    m1 = fmaxf(m1, tstat[((int64_t)l * T + t) * 2 + 1]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, off, 64));
    m1 = fmaxf(m1, __shfl_xor(m1, off, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = m0;
    red[1][threadIdx.x >> 6] = m1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    lstat[l * 4] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    lstat[l * 4 + 1] = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
    lstat[l * 4 + 2] = 0.f;
    lstat[l * 4 + 3] = 0.f;
  }
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
                          float *cbpad, int dp, float *tstat, float *lstat, hipStream_t s) {
  if (cbpad) {
    const int64_t rows = (int64_t)L * K;
    pad_codebook_kernel<<<dim3((unsigned)ceil_div(rows * dp, 256)), dim3(256), 0, s>>>(cb, rows, d,
                                                                                      dp, cbpad);
  }
  const int Kp = (int)padded_k(K), S = (int)(padded_d(d) / kStageCols);
  // rows wider than the sweep holds are encoded in exact fp32: the padded
  // copy is all they use
  if (S == 0) return hipGetLastError();
  const int64_t tiles = (int64_t)L * (Kp / kTileCw);
  prepare_tile_kernel<<<dim3((unsigned)tiles), dim3(256), 0, s>>>(
      cb, L, K, d, Kp, S, norms, reinterpret_cast<uint4 *>(stream), tstat);
  level_stat_kernel<<<dim3((unsigned)L), dim3(256), 0, s>>>(tstat, Kp / kTileCw, lstat);
  return hipGetLastError();
}

}  // namespace rvq
