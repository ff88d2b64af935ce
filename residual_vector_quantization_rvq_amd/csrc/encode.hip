// encode.hip -- encoder planning, input staging and dispatch over the
// instantiated stage counts (the kernels are in encode_impl.h).
#include "encode_impl.h"

namespace rvq {

// fp32 copy of the input rows with stride dp and zero padding (bf16 input,
// or a width that is not a multiple of 8).  One wave per row.
__global__ __launch_bounds__(256) void stage_input_kernel(const void *__restrict__ x, int x_bf16,
                                                          int64_t n, int d, int dp,
                                                          float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  for (int i = lane; i < dp; i += 64) {
    float v = 0.f;
    if (i < d)
      v = x_bf16 ? bf16_bits_to_f32(((const uint16_t *)x)[row * d + i]) : ((const float *)x)[row * d + i];
    out[row * dp + i] = v;
  }
}

// residual_out [n][d] from the fused encoder's fragment-major residual: one
// workgroup per block of 32 rows; the 16-byte run of lane L in k-step ks,
// half q holds row 32*blk + L%32, features ks*16 + (L/32)*8 + q*4 .. +3.
__global__ __launch_bounds__(256) void unfragment_kernel(const float *__restrict__ fm, int64_t n,
                                                         int d, int dp, float *__restrict__ out) {
  const int64_t blk = blockIdx.x;
  const int runs = (dp >> 4) * 2 * 64;  // 16-byte runs in a block
  const float *src = fm + blk * 32 * dp;
  for (int i = threadIdx.x; i < runs; i += 256) {
    const int lane = i & 63, q = (i >> 6) & 1, ks = i >> 7;
    const int64_t row = blk * 32 + (lane & 31);
    if (row >= n) continue;
    const float4 v = *reinterpret_cast<const float4 *>(src + (int64_t)i * 4);
    const int f0 = ks * 16 + (lane >> 5) * 8 + q * 4;
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (f0 + k < d) out[row * d + f0 + k] = e[k];
  }
}

// bf16 B-fragments of the level-0 rows (split mode), from the fp32 rows of
// stride dp: one thread per 16-byte piece, piece (b, ks, L) holding features
// ks*16 + (L/32)*8 .. +7 of row 32 b + L%32 (zeros for rows past n, up to
// the end of the last 128-row block).
__global__ __launch_bounds__(256) void fragment_rows_kernel(const float *__restrict__ src,
                                                            int64_t n, int dp,
                                                            uint4 *__restrict__ frag,
                                                            int64_t pieces) {
  const int64_t o = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (o >= pieces) return;
  const int lane = (int)(o & 63);
  const int ksp = dp >> 4;
  const int64_t rest = o >> 6;
  const int ks = (int)(rest % ksp);
  const int64_t row = (rest / ksp) * 32 + (lane & 31);
  u32x4 q = {0u, 0u, 0u, 0u};
  if (row < n) {
    float v[8];
    read8(src, row, dp, ks * 16 + (lane >> 5) * 8, true, v);
    q = to_bf16x8(v);
  }
  frag[o] = make_uint4(q[0], q[1], q[2], q[3]);
}

// residual_out [n][d] from the padded fp32 residual [n][dp].
__global__ __launch_bounds__(256) void unpad_kernel(const float *__restrict__ src, int64_t n,
                                                    int d, int dp, float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  for (int i = lane; i < d; i += 64) out[row * d + i] = src[row * dp + i];
}

EncodePlan plan_encode(int64_t n, int d, int K, int num_cus) {
  EncodePlan p{};
  p.stages = (int)(padded_d(d) / kStageCols);
  p.tiles = (int)(padded_k(K) / kTileCw);
  p.row_blocks = (int)ceil_div(n, kRowsPerWG);
  const int cus = num_cus > 0 ? num_cus : 256;
  p.fused = (int64_t)p.row_blocks * 10 >= (int64_t)cus * 6;
  if (p.fused) {
    p.splits = 1;
    p.tiles_per_split = p.tiles;
  } else {
    const int want = (int)ceil_div(2 * cus, p.row_blocks);
    const int splits = want < p.tiles ? want : p.tiles;
    p.tiles_per_split = (int)ceil_div(p.tiles, splits);
    p.splits = (int)ceil_div(p.tiles, p.tiles_per_split);
  }
  return p;
}

#define RVQ_DECLARE(NS) \
  extern template hipError_t launch_stage_count<NS>(const EncodePlan &, const EncodeArgs &, \
                                                    hipEvent_t *, hipStream_t);
RVQ_FOR_EACH_STAGE_COUNT(RVQ_DECLARE)
#undef RVQ_DECLARE

hipError_t launch_stages(const EncodePlan &p, const EncodeArgs &a, hipEvent_t *events,
                         hipStream_t s) {
  switch (p.stages) {
#define RVQ_CASE(NS) \
  case NS:           \
    return launch_stage_count<NS>(p, a, events, s);
    RVQ_FOR_EACH_STAGE_COUNT(RVQ_CASE)
#undef RVQ_CASE
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_encode(const EncodePlan &p, const EncodeArgs &a_in, hipEvent_t *events,
                         hipStream_t s) {
  if (a_in.n == 0) return hipSuccess;
  EncodeArgs a = a_in;
  const unsigned row_waves = (unsigned)ceil_div(a.n, 4);
  a.x16 = nullptr;
  // rows read with 16-byte accesses must start 16-byte aligned; others (a
  // slice of a larger batch, say) go through the staging copy
  const bool x_al = ((uintptr_t)a.x & 15) == 0;
  if (p.fused && a.x_bf16 && a.dp == a.d && x_al) {
    // level 0 of the fused encoder reads the bf16 rows directly
    a.x16 = (const uint16_t *)a.x;
    a.src0 = nullptr;
  } else if (a.x_bf16 || a.dp != a.d || !x_al) {
    stage_input_kernel<<<dim3(row_waves), dim3(256), 0, s>>>(a.x, a.x_bf16, a.n, a.d, a.dp,
                                                           a.rbuf[0]);
    a.src0 = a.rbuf[0];
  } else {
    a.src0 = (const float *)a.x;
  }
  // The last level reads rbuf[(L-1) & 1] and writes the final residual to
  // rbuf[L & 1]: fragment-major in fused mode (converted afterwards), rows of
  // stride dp in split mode (written straight to the caller's buffer when
  // d == dp and the buffer is 16-byte aligned).
  float *final_buf = a.rbuf[a.L & 1];
  const bool out_al = ((uintptr_t)a.residual_out & 15) == 0;
  const bool convert = a.residual_out && (p.fused || a.dp != a.d || !out_al);
  a.res_final = convert ? final_buf : a.residual_out;
  if (!p.fused) {
    // every block a sweep workgroup reads (4 per 128 rows)
    const int64_t pieces = ceil_div(a.n, kRowsPerWG) * 4 * (a.dp >> 4) * 64;
    fragment_rows_kernel<<<dim3((unsigned)ceil_div(pieces, 256)), dim3(256), 0, s>>>(
        a.src0, a.n, a.dp, a.xfrag, pieces);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_stages(p, a, events, s);
  if (e != hipSuccess || !convert) return e;
  if (p.fused)
    unfragment_kernel<<<dim3((unsigned)ceil_div(a.n, 32)), dim3(256), 0, s>>>(final_buf, a.n, a.d,
                                                                          a.dp, a.residual_out);
  else
    unpad_kernel<<<dim3(row_waves), dim3(256), 0, s>>>(final_buf, a.n, a.d, a.dp,
                                                       a.residual_out);
  return hipGetLastError();
}

}  // namespace rvq
