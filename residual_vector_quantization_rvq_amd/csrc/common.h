// common.h -- shared device helpers and launcher prototypes for the RVQ library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Sentinel index of an empty top-2 slot; never a valid codeword index.
constexpr int kNoIndex = 0x7fffffff;

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  __bf16 h = (__bf16)v;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Lexicographic order on (score, index): smaller score first, lower index
// on equal scores.  A total order on finite scores, so every merge of top-2
// lists below gives the same result whatever the merge order.
__device__ __forceinline__ bool lex_lt(float sa, int ia, float sb, int ib) {
  return sa < sb || (sa == sb && ia < ib);
}

// Merge candidate list (t1 <= t2) into running list (s1 <= s2), keeping the
// two smallest under lex_lt.  Indices in the two lists must be distinct.
__device__ __forceinline__ void merge_top2(float &s1, int &i1, float &s2, int &i2,
                                           float t1, int j1, float t2, int j2) {
  if (lex_lt(t1, j1, s1, i1)) {
    bool keep_s1 = lex_lt(s1, i1, t2, j2);
    s2 = keep_s1 ? s1 : t2;
    i2 = keep_s1 ? i1 : j2;
    s1 = t1;
    i1 = j1;
  } else if (lex_lt(t1, j1, s2, i2)) {
    s2 = t1;
    i2 = j1;
  }
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// ---- tiling constants of the distance kernel (shared with host sizing) ----
constexpr int kTileCodewords = 256;  // codewords per tile (MFMA M side)
constexpr int kTileRows = 128;       // rows per tile (MFMA N side)
constexpr int kStageCols = 32;       // feature columns per LDS stage
constexpr int kNumXcd = 8;           // workgroups are dispatched round-robin over 8 XCDs

// Padded sizes of the prepared codebook.
inline int64_t padded_k(int64_t K) { return round_up(K, kTileCodewords); }
inline int64_t padded_d(int64_t d) { return round_up(d, kStageCols); }

// ---- host-side launchers (return hipGetLastError of their launches) ----
hipError_t launch_prepare(const float *cb, int L, int K, int d, float *norms, uint16_t *cbh,
                          hipStream_t s);
hipError_t launch_init_residual(const void *x, bool x_bf16, int64_t n, int d, int Dp, float *r32,
                                uint16_t *r16, hipStream_t s);

struct DistPlan {
  int ktiles;      // codeword tiles per level
  int tiles_per_wg;
  int splits;      // partial top-2 lists per row = ceil(ktiles / tiles_per_wg)
  int row_blocks;
  int group;       // row blocks per L2-sharing group
  int per_xcd;     // workgroups per XCD
  int grid;
};
DistPlan plan_distance(int64_t n, int K, int num_cus);
hipError_t launch_distance_top2(const DistPlan &p, const uint16_t *r16, int64_t n, int Dp,
                                const uint16_t *cbh_l, const float *norms_l, float4 *part,
                                hipStream_t s);
hipError_t launch_rescore_update(const float4 *part, int splits, int64_t n, int d, int Dp, int K,
                                 int L, int level, const float *cb_l, const float *r_in,
                                 float *r_out, uint16_t *r16, bool write_r16, int32_t *ids,
                                 hipStream_t s);
hipError_t launch_decode(const int32_t *ids, int64_t n, const float *cb, int L, int K, int d,
                         int levels, void *out, bool out_bf16, uint32_t *bad, hipStream_t s);
size_t hist_partial_bytes(int64_t n, int L, int K);
hipError_t launch_hist(const int32_t *ids, int64_t n, int L, int K, int64_t *hist,
                       uint32_t *partial, uint32_t *bad, hipStream_t s);
size_t msr_partial_bytes(int64_t n, int L);
hipError_t launch_msr(const void *x, bool x_bf16, const int32_t *ids, int64_t n, int d,
                      const float *cb, int L, int K, double *msr, double *partial, uint32_t *bad,
                      hipStream_t s);

}  // namespace rvq
