// wide.hip -- the encoder for rows wider than the matrix-core sweep holds.
//
// The RVQ step is the same as everywhere else in the library: at each level
// the nearest codeword of the residual, its index recorded, the residual
// reduced by it ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
// "Visual Primitive Modeling", paragraph "Discrete Native Resolution Vision
// Transformer"; "LongCat-2.5 Open Source Release: Meituan's 1.6T Multimodal
// Agent Model with 1M Context", "02 Visual Coding and 3D").  The sweep keeps
// a row's bf16 features resident in registers, which bounds it at 1280
// features; wider rows come here.  This path computes every distance
// exactly in fp32, sum over features of (r_i - c_i)^2, with no screening,
// so no band and no exact scans afterwards are needed.  It runs on the
// vector ALUs, one launch per level.
//
// A workgroup owns 64 rows and sweeps the level's codewords 64 at a time;
// thread (ty, tx) = (tid / 16, tid % 16) accumulates the 4 x 4 distances of
// rows 4 ty .. +3 and codewords 4 tx .. +3 of the tile.  Features come
// through LDS 16 at a time (a chunk), transposed so that a thread reads its
// four rows and its four codewords of one feature as two 16-byte words.  A
// distance is summed chunk by chunk: within a chunk over its 16 features in
// increasing order with fmaf from zero, then added to the running sum, so
// its value depends only on the row and the codeword (batch invariance).
// The smallest distance wins, the lower index on a tie.
#include "common.h"

namespace rvq {

namespace {

constexpr int kWRows = 64;    // rows per workgroup
constexpr int kWCw = 64;      // codewords per tile
constexpr int kWChunk = 16;   // features per LDS chunk
constexpr int kWPad = 4;      // LDS row padding (floats)

__device__ __forceinline__ bool lex_less(float d, int i, float bd, int bi) {
  return d < bd || (d == bd && i < bi);
}

__device__ void wide_update(const EncodeArgs &a, int level, int64_t row0, const int *win, int f4b,
                            int f4e);

// With slices > 1 the level's codewords are split over `slices`
// workgroups per 64-row block (slice sl takes codewords sl * slice_cw ..
// +slice_cw - 1) and each writes its rows' (distance, index) minimum to the
// split plan's records; wide_merge_kernel then picks each row's winner.
__global__ __launch_bounds__(256) void wide_level_kernel(EncodeArgs a, int level, int slices,
                                                         int slice_cw) {
  __shared__ __align__(16) float rs[kWChunk][kWRows + kWPad];  // [feature][row]
  __shared__ __align__(16) float cs[kWChunk][kWCw + kWPad];    // [feature][codeword]
  __shared__ float red_d[kWRows][16];
  __shared__ int red_i[kWRows][16];
  __shared__ int win[kWRows];

  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int64_t row0 = (int64_t)(blockIdx.x / slices) * kWRows;
  const int sl = blockIdx.x % slices;
  const int k_begin = sl * slice_cw;
  const int k_end = min(a.K, k_begin + slice_cw);
  const int dp = a.dp;
  const float *src = level == 0 ? a.src0 : (level & 1) ? a.rbuf[1] : a.rbuf[0];
  const float *cb_l = a.cb + (int64_t)level * a.K * dp;
  // this thread's piece of each chunk load: row / codeword tid / 4,
  // features 4 (tid % 4) .. +3 of the chunk
  const int lr = tid >> 2, lq = tid & 3;
  const int64_t lrow = row0 + lr;
  const bool lrow_ok = lrow < a.n;
  const float *rsrc = src + (lrow_ok ? lrow : 0) * dp + lq * 4;

  float bd[4];
  int bi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bd[i] = __builtin_inff();
    bi[i] = 0x7fffffff;
  }
  for (int c0 = k_begin; c0 < k_end; c0 += kWCw) {
    const int lcw = c0 + lr;
    const bool lcw_ok = lcw < k_end;
    const float *csrc = cb_l + (int64_t)(lcw_ok ? lcw : 0) * dp + lq * 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
    for (int f0 = 0; f0 < dp; f0 += kWChunk) {
      const float4 rv = lrow_ok ? *reinterpret_cast<const float4 *>(rsrc + f0)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 cv = lcw_ok ? *reinterpret_cast<const float4 *>(csrc + f0)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
      __syncthreads();  // every thread is done with the previous chunk
      rs[lq * 4 + 0][lr] = rv.x;
      rs[lq * 4 + 1][lr] = rv.y;
      rs[lq * 4 + 2][lr] = rv.z;
      rs[lq * 4 + 3][lr] = rv.w;
      cs[lq * 4 + 0][lr] = cv.x;
      cs[lq * 4 + 1][lr] = cv.y;
      cs[lq * 4 + 2][lr] = cv.z;
      cs[lq * 4 + 3][lr] = cv.w;
      __syncthreads();
      float p[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[i][j] = 0.f;
#pragma unroll
      for (int f = 0; f < kWChunk; ++f) {
        const float4 r4 = *reinterpret_cast<const float4 *>(&rs[f][ty * 4]);
        const float4 c4 = *reinterpret_cast<const float4 *>(&cs[f][tx * 4]);
        const float r[4] = {r4.x, r4.y, r4.z, r4.w};
        const float c[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float t = r[i] - c[j];
            p[i][j] = fmaf(t, t, p[i][j]);
          }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __fadd_rn(acc[i][j], p[i][j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = c0 + tx * 4 + j;
      if (k < k_end) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (lex_less(acc[i][j], k, bd[i], bi[i])) {
            bd[i] = acc[i][j];
            bi[i] = k;
          }
      }
    }
  }
  // the row's winner over the 16 threads that share it
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red_d[ty * 4 + i][tx] = bd[i];
    red_i[ty * 4 + i][tx] = bi[i];
  }
  __syncthreads();
  if (tid < kWRows) {
    float d = red_d[tid][0];
    int k = red_i[tid][0];
    for (int t = 1; t < 16; ++t)
      if (lex_less(red_d[tid][t], red_i[tid][t], d, k)) {
        d = red_d[tid][t];
        k = red_i[tid][t];
      }
    const int64_t row = row0 + tid;
    if (slices > 1) {
      if (row < a.n)
        reinterpret_cast<int2 *>(a.part)[row * slices + sl] = make_int2(__float_as_int(d), k);
    } else {
      // finite inputs always give a valid codeword
      k = (k >= 0 && k < a.K) ? k : 0;
      win[tid] = k;
      if (row < a.n) {
        a.ids[row * a.L + level] = k;
        a.aux[row * a.L + level] = kAuxOk;
      }
    }
  }
  if (slices > 1) return;
  __syncthreads();
  wide_update(a, level, row0, win, 0, a.dp >> 2);
}

// Each row's winner over the slices' minima ((distance, index) order), its
// ID, and the next level's residual.  Workgroup b takes the rows of block
// b / fsplit and features (in float4) [f4b, f4e) of part b % fsplit of the
// row; four threads share a row's minima, and part 0 writes the IDs.
__global__ __launch_bounds__(256) void wide_merge_kernel(EncodeArgs a, int level, int slices,
                                                         int fsplit) {
  __shared__ int win[kWRows];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)(blockIdx.x / fsplit) * kWRows;
  const int fs = blockIdx.x % fsplit;
  const int r = tid >> 2, q = tid & 3;
  const int64_t row = row0 + r;
  float d = __builtin_inff();
  int k = 0x7fffffff;
  if (row < a.n) {
    const int2 *pm = reinterpret_cast<const int2 *>(a.part) + row * slices;
    for (int t = q; t < slices; t += 4) {
      const int2 e = pm[t];
      if (lex_less(__int_as_float(e.x), e.y, d, k)) {
        d = __int_as_float(e.x);
        k = e.y;
      }
    }
  }
  // (a total order: the minimum does not depend on how it is reduced)
#pragma unroll
  for (int off = 1; off < 4; off <<= 1) {
    const float od = __shfl_xor(d, off, 64);
    const int ok = __shfl_xor(k, off, 64);
    if (lex_less(od, ok, d, k)) {
      d = od;
      k = ok;
    }
  }
  if (q == 0) {
    k = (k >= 0 && k < a.K) ? k : 0;
    win[r] = k;
    if (row < a.n && fs == 0) {
      a.ids[row * a.L + level] = k;
      a.aux[row * a.L + level] = kAuxOk;
    }
  }
  __syncthreads();
  const int dp4 = a.dp >> 2;
  const int per = (dp4 + fsplit - 1) / fsplit;
  const int f4b = fs * per;
  wide_update(a, level, row0, win, f4b, min(dp4, f4b + per));
}

__device__ void wide_update(const EncodeArgs &a, int level, int64_t row0, const int *win, int f4b,
                            int f4e) {
  const int tid = threadIdx.x;
  const int dp = a.dp;
  const float *src = level == 0 ? a.src0 : (level & 1) ? a.rbuf[1] : a.rbuf[0];
  const float *cb_l = a.cb + (int64_t)level * a.K * dp;
  // r - c of the winner, the next level's residual (rows of stride dp)
  float *dst = level == a.L - 1 ? a.res_final : (level & 1) ? a.rbuf[0] : a.rbuf[1];
  if (dst == nullptr) return;
  const int w4 = f4e - f4b;
  for (int e = tid; e < kWRows * w4; e += 256) {
    const int rr = e / w4, f4 = f4b + e % w4;
    const int64_t row = row0 + rr;
    if (row >= a.n) continue;
    const float4 r = reinterpret_cast<const float4 *>(src + row * dp)[f4];
    const float4 c = reinterpret_cast<const float4 *>(cb_l + (int64_t)win[rr] * dp)[f4];
    reinterpret_cast<float4 *>(dst + row * dp)[f4] =
        make_float4(r.x - c.x, r.y - c.y, r.z - c.z, r.w - c.w);
  }
}

}  // namespace

int wide_slices(int64_t n, int K, int num_cus) {
  // enough workgroups to fill the GPU twice over, in whole 64-codeword
  // tiles, within the split plan's records (int2 per row and slice), which
  // the workspace holds only for row counts that some device may split
  if (n <= 0 || !split_possible(n)) return 1;
  const int64_t blocks = ceil_div(n, kWRows);
  const int64_t units = ceil_div((int64_t)K, kWCw);
  int64_t want = ceil_div(2 * (int64_t)num_cus, blocks);
  const int64_t room = split_records(n, K) * kRecF4 * 16 / (n * (int64_t)sizeof(int2));
  want = want < units ? want : units;
  want = want < room ? want : room;
  if (want <= 1) return 1;
  const int64_t per = ceil_div(units, want);
  return (int)ceil_div(units, per);
}

hipError_t launch_wide(const EncodeArgs &a, int slices, hipEvent_t *ev, hipStream_t s) {
  hipError_t e;
  const int64_t blocks = ceil_div(a.n, kWRows);
  const int units = (int)ceil_div((int64_t)a.K, kWCw);
  const int slice_cw = (int)ceil_div(units, slices) * kWCw;
  for (int l = 0; l < a.L; ++l) {
    if (ev && (e = hipEventRecord(ev[2 * l], s)) != hipSuccess) return e;
    wide_level_kernel<<<dim3((unsigned)(blocks * slices)), dim3(256), 0, s>>>(a, l, slices,
                                                                             slice_cw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev && (e = hipEventRecord(ev[2 * l + 1], s)) != hipSuccess) return e;
    if (slices > 1) {
      // about 512 workgroups for the merge and the residual update
      const int64_t dp4 = a.dp >> 2;
      int64_t fsplit = ceil_div(512, blocks);
      fsplit = fsplit < dp4 ? fsplit : dp4;
      wide_merge_kernel<<<dim3((unsigned)(blocks * fsplit)), dim3(256), 0, s>>>(a, l, slices,
                                                                              (int)fsplit);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace rvq
