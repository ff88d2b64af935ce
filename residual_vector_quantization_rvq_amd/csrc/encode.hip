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

// Band inputs of the level-0 rows for split mode (the fused encoder forms
// them while building its fragments): sum bf16(v)^2 and sum (v - bf16(v))^2
// of each half, over features ks*16 + h*8 + e in order with fmaf, then
// half 0 + half 1, as every encoder kernel sums them.  One wave per row:
// every lane rounds its features into LDS, then lane 2q + h runs the chain
// of sum q of half h, so one instruction stream serves all four chains.
__global__ __launch_bounds__(256) void row_stats_kernel(const float *__restrict__ src, int64_t n,
                                                        int dp, float2 *__restrict__ rstat) {
  __shared__ float4 area[4][2][kMaxStages * kStageCols / 4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n) return;
  const int dp4 = dp >> 2;
  const float4 *rs = reinterpret_cast<const float4 *>(src + row * dp);
  for (int i = lane; i < dp4; i += 64) {
    const float4 t = rs[i];
    const float4 b = make_float4(bf16_bits_to_f32(f32_to_bf16_bits(t.x)),
                                 bf16_bits_to_f32(f32_to_bf16_bits(t.y)),
                                 bf16_bits_to_f32(f32_to_bf16_bits(t.z)),
                                 bf16_bits_to_f32(f32_to_bf16_bits(t.w)));
    area[wave][0][i] = b;
    area[wave][1][i] = make_float4(t.x - b.x, t.y - b.y, t.z - b.z, t.w - b.w);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float acc = 0.f;
  if (lane < 4) {
    const float4 *tl = &area[wave][lane >> 1][(lane & 1) * 2];
    const int kend = dp >> 4;
#pragma unroll 4
    for (int ks = 0; ks < kend; ++ks) {
      const float4 ta = tl[ks * 4], tb = tl[ks * 4 + 1];
      const float tv[8] = {ta.x, ta.y, ta.z, ta.w, tb.x, tb.y, tb.z, tb.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(tv[e], tv[e], acc);
    }
  }
  const float rb0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 0));
  const float rb1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 1));
  const float dr0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 2));
  const float dr1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), 3));
  if (lane == 0) rstat[row] = make_float2(rb0 + rb1, dr0 + dr1);
}

// Levels whose candidate band could not be shown complete (repair code
// kAuxScan, rare: a band list overflowed, or two blocks each held two keys
// inside the band) are taken again by an exact scan: the nearest codeword
// under the rescoring's own fp32 distance (two half sums in feature order,
// half 0 + half 1) over all K, the lower index on a tie.  One workgroup per
// 256 rows finds its rows with such a level and redoes each one: the
// residual is rebuilt from the row and its IDs with the encoder's fp32
// subtractions, and once an ID changes every later level is scanned too.
// Changed IDs, and the final residual when the caller asked for it, are
// rewritten.
__global__ __launch_bounds__(256) void repair_kernel(EncodeArgs a) {
  __shared__ float res[kMaxStages * kStageCols];
  __shared__ int rows[256];
  __shared__ int nrows;
  __shared__ float wd[4];
  __shared__ int wi[4];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 256;
  if (tid == 0) nrows = 0;
  __syncthreads();
  {
    const int64_t row = r0 + tid;
    bool f = false;
    if (row < a.n)
      for (int l = 0; l < a.L; ++l) f |= a.aux[row * a.L + l] == kAuxScan;
    if (f) rows[atomicAdd(&nrows, 1)] = tid;
  }
  __syncthreads();
  const int nr = nrows;
  const int nks = a.dp >> 4;
  for (int q = 0; q < nr; ++q) {
    const int64_t row = r0 + rows[q];
    for (int i = tid; i < a.dp; i += 256) {
      float v = 0.f;
      if (i < a.d)
        v = a.x_bf16 ? bf16_bits_to_f32(((const uint16_t *)a.x)[row * a.d + i])
                     : ((const float *)a.x)[row * a.d + i];
      res[i] = v;
    }
    __syncthreads();
    bool changed = false;
    for (int l = 0; l < a.L; ++l) {
      const float *cb_l = a.cb + (int64_t)l * a.K * a.dp;
      int id = a.ids[row * a.L + l];
      if (changed || a.aux[row * a.L + l] == kAuxScan) {
        float bd = __builtin_inff();
        int bi = kNoIndex;
        for (int k = tid; k < a.K; k += 256) {
          const float *c = cb_l + (int64_t)k * a.dp;
          float p0 = 0.f, p1 = 0.f;
          for (int ks = 0; ks < nks; ++ks) {
            float x0[8], x1[8];
            read8(c, 0, a.dp, ks * 16, true, x0);
            read8(c, 0, a.dp, ks * 16 + 8, true, x1);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float t = res[ks * 16 + e] - x0[e];
              const float u = res[ks * 16 + 8 + e] - x1[e];
              p0 = fmaf(t, t, p0);
              p1 = fmaf(u, u, p1);
            }
          }
          const float dk = p0 + p1;
          if (lex_lt(dk, k, bd, bi)) {
            bd = dk;
            bi = k;
          }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float od = __shfl_xor(bd, off, 64);
          const int oi = __shfl_xor(bi, off, 64);
          if (lex_lt(od, oi, bd, bi)) {
            bd = od;
            bi = oi;
          }
        }
        if ((tid & 63) == 0) {
          wd[tid >> 6] = bd;
          wi[tid >> 6] = bi;
        }
        __syncthreads();
        bd = wd[0];
        bi = wi[0];
        for (int w = 1; w < 4; ++w)
          if (lex_lt(wd[w], wi[w], bd, bi)) {
            bd = wd[w];
            bi = wi[w];
          }
        if (bi != id) {
          changed = true;
          if (tid == 0) a.ids[row * a.L + l] = bi;
          id = bi;
        }
      }
      for (int i = tid; i < a.dp; i += 256) res[i] = res[i] - cb_l[(int64_t)id * a.dp + i];
      __syncthreads();
    }
    if (changed && a.residual_out)
      for (int i = tid; i < a.d; i += 256) a.residual_out[row * a.d + i] = res[i];
    __syncthreads();
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

bool split_possible(int64_t n) { return ceil_div(n, kRowsPerWG) * 10 < (int64_t)kPlanMaxCus * 6; }

int64_t split_records(int64_t n, int K) {
  const int64_t rb = ceil_div(n, kRowsPerWG);
  const int64_t tiles = padded_k(K) / kTileCw;
  const int64_t want = ceil_div(2 * (int64_t)kPlanMaxCus, rb > 0 ? rb : 1);
  return n * (want < tiles ? want : tiles) * 2;
}

EncodePlan plan_encode(int64_t n, int d, int K, int num_cus) {
  EncodePlan p{};
  p.stages = (int)(padded_d(d) / kStageCols);
  p.tiles = (int)(padded_k(K) / kTileCw);
  p.row_blocks = (int)ceil_div(n, kRowsPerWG);
  int cus = num_cus > 0 ? num_cus : 256;
  cus = cus < kPlanMaxCus ? cus : kPlanMaxCus;
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
    row_stats_kernel<<<dim3(row_waves), dim3(256), 0, s>>>(a.src0, a.n, a.dp, a.rstat);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_stages(p, a, events, s);
  if (e != hipSuccess) return e;
  if (convert) {
    if (p.fused)
      unfragment_kernel<<<dim3((unsigned)ceil_div(a.n, 32)), dim3(256), 0, s>>>(
          final_buf, a.n, a.d, a.dp, a.residual_out);
    else
      unpad_kernel<<<dim3(row_waves), dim3(256), 0, s>>>(final_buf, a.n, a.d, a.dp,
                                                         a.residual_out);
  }
  repair_kernel<<<dim3((unsigned)ceil_div(a.n, 256)), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace rvq
