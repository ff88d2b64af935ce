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
  if (p.fused && a.x_bf16 && a.dp == a.d && (a.L > 1 || a.residual_out)) {
    // level 0 of the fused encoder reads the bf16 rows directly
    a.x16 = (const uint16_t *)a.x;
    a.src0 = nullptr;
  } else if (a.x_bf16 || a.dp != a.d) {
    stage_input_kernel<<<dim3(row_waves), dim3(256), 0, s>>>(a.x, a.x_bf16, a.n, a.d, a.dp,
                                                           a.rbuf[0]);
    a.src0 = a.rbuf[0];
  } else {
    a.src0 = (const float *)a.x;
  }
  // the last level reads rbuf[(L-1) & 1] and writes the final residual to
  // the caller's buffer, or (padded width) to the other buffer first
  const bool unpad = a.residual_out && a.dp != a.d;
  float *padded_final = a.rbuf[a.L & 1];
  a.res_final = unpad ? padded_final : a.residual_out;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_stages(p, a, events, s);
  if (e != hipSuccess || !unpad) return e;
  unpad_kernel<<<dim3(row_waves), dim3(256), 0, s>>>(padded_final, a.n, a.d, a.dp,
                                                     a.residual_out);
  return hipGetLastError();
}

}  // namespace rvq
