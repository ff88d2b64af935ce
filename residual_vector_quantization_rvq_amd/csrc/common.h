// common.h -- shared device helpers and launcher prototypes for the RVQ library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rvq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Sentinel index of an empty (key, index) slot; never a valid codeword index.
constexpr int kNoIndex = 0x7fffffff;

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  __bf16 h = (__bf16)v;  // round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Lexicographic order on (score, index): smaller score first, lower index
// on equal scores.  A total order on finite scores, so every merge of
// (key, index) minima gives the same result whatever the merge order.
__device__ __forceinline__ bool lex_lt(float sa, int ia, float sb, int ib) {
  return sa < sb || (sa == sb && ia < ib);
}

// Merge candidate list (t1 <= t2) into running list (s1 <= s2), keeping the
// two smallest under lex_lt.  Indices in the two lists must be distinct.
__device__ __forceinline__ void merge_top2(float &s1, int &i1, float &s2, int &i2,
                                           float t1, int j1, float t2, int j2) {
  // selects only: written as two branches through references, the list is
  // kept in scratch memory
  const bool first = lex_lt(t1, j1, s1, i1);   // t1 becomes the best
  const bool keep1 = lex_lt(s1, i1, t2, j2);   // ... and s1 or t2 the second
  const bool second = lex_lt(t1, j1, s2, i2);  // else t1 may become the second
  const float n2 = first ? (keep1 ? s1 : t2) : (second ? t1 : s2);
  const int m2 = first ? (keep1 ? i1 : j2) : (second ? j1 : i2);
  s1 = first ? t1 : s1;
  i1 = first ? j1 : i1;
  s2 = n2;
  i2 = m2;
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

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// ---- prepared codebook stream (shared by every encode kernel) ----
// Codewords are grouped in tiles of 128 and features in stages of 64.  For
// level l and tile t the stream holds
//   [norm k-step: 4 blocks][stage 0: 16 blocks] ... [stage S-1: 16 blocks]
// where a block is 1 KB = one MFMA A-fragment of v_mfma_f32_32x32x16_bf16
// for a sub-tile j (32 codewords) and a k-step ks (16 features):
//   lane L holds 8 bf16 values -2*c[t*128 + j*32 + L%32][s*64 + ks*16 + (L/32)*8 + e].
// Stage blocks are ordered (j, ks).  Norm block j: lanes L < 32 hold
// [hi, lo, 0 x 6] with hi = bf16(||c||^2), lo = bf16(||c||^2 - hi) for
// codeword t*128 + j*32 + L; lanes >= 32 hold zeros.  Multiplied by a
// B-fragment of ones in the same two positions, the norm k-step adds
// ||c||^2 to the accumulator, so a sweep accumulates the score
// ||c||^2 - 2 r.c directly.  Padded codewords (index >= K) are zero
// vectors with norm kPadNorm, so their score is huge and finite.
constexpr int kTileCw = 128;
constexpr int kStageCols = 64;
constexpr int kBlockBytes = 1024;
constexpr int kStageBytes = 16 * kBlockBytes;
constexpr int kNormBytes = 4 * kBlockBytes;
constexpr int kRowsPerWG = 128;      // 4 waves x 32 rows
constexpr int kMaxStages = 20;       // features <= 1280
// Wider rows (up to this many features) take the exact fp32 encoder (wide.hip).
constexpr int kWideMaxD = 8192;
constexpr float kPadNorm = 3.0e38f;

// Stage counts (features / 64) with an instantiated encoder; a width is
// padded with zeros up to the next one (zero features change no distance).
#define RVQ_FOR_EACH_STAGE_COUNT(X) X(1) X(2) X(4) X(8) X(12) X(16) X(18) X(20)
constexpr int kStageCounts[] = {1, 2, 4, 8, 12, 16, 18, 20};
__host__ __device__ inline int stages_for(int64_t d) {
  const int s = (int)ceil_div(d, kStageCols);
  for (int c : kStageCounts)
    if (c >= s) return c;
  return 0;
}
// The instantiated stage count below S (0 for the smallest): a row encoded
// with S stages is wider than 64 * prev_stage_count(S) features, so its first
// 4 * prev_stage_count(S) k-steps of 16 features are all inside the row.
__host__ __device__ constexpr int prev_stage_count(int S) {
  int p = 0;
  for (int c : kStageCounts) {
    if (c >= S) return p;
    p = c;
  }
  return p;
}
__host__ __device__ inline int64_t padded_k(int64_t K) { return round_up(K, kTileCw); }
__host__ __device__ inline int64_t padded_d(int64_t d) { return (int64_t)stages_for(d) * kStageCols; }
__host__ __device__ inline int64_t tile_bytes(int stages) { return kNormBytes + (int64_t)stages * kStageBytes; }
__host__ __device__ inline int64_t stream_bytes(int L, int64_t K, int64_t d) {
  return (int64_t)L * (padded_k(K) / kTileCw) * tile_bytes((int)(padded_d(d) / kStageCols));
}

// ---- candidate band of the encoder ----
// The bf16 screening key of codeword k, key_k, lies near the exact score
// t_k = ||c_k||^2 - 2 r.c_k of the fp32 residual r.  With r_b = bf16(r),
// dr = r - r_b, dc_k = c_k - bf16(c_k), the identity
//   r.c - r_b.bf16(c) = dr.c + r_b.dc
// splits the screening error into a residual-rounding and a codeword-rounding
// part.  Per row and level the encoder uses the bound
//   E = min(5 sigma, E_cs) + E_acc + E_norm + E_tag,
//   sigma = 2 sqrt((||dr||^2 cmax + ||r_b||^2 dmax) / d)   (error scale of a
//           typical codeword: rounding errors of independent features),
//   E_cs  = 2 (sqrt(||dr||^2 cmax) + sqrt(||r_b||^2 dmax))  (Cauchy-Schwarz,
//           a worst case; smaller than 5 sigma only for d < about 25),
//   E_acc = min(d + 2, 5 sqrt(d + 2)) 2^-23 T,  T = 2 sqrt(||r_b||^2 cmax) + cmax
//           (fp32 accumulation on the matrix cores),
//   E_norm = ((d/2 + 1) 2^-24 + 2^-17) cmax   (fp32 norm chain, hi + lo split),
//   E_tag = 2^-18 T                           (5 tag bits of the key),
// with cmax = max_k ||c_k||^2 and dmax = max_k ||dc_k||^2 of the level.  Every
// codeword whose key is within
//   band = max(0, 2 E - 0.5e-4 ||r_b||^2)
// of the smallest key is rescored exactly in fp32.  If the nearest codeword
// k* is more than 1e-4 ||r||^2 closer than every other, then
// key_k* <= t_k* + E <= t_k1 - 1e-4 ||r||^2 + E <= key_min + band, so k* is
// a candidate, and the fp32 rescoring then orders it first.
// Written with explicitly rounded operations so that every kernel computes
// the same bits from the same inputs.
constexpr float kBandZ = 5.0f;
__device__ __forceinline__ float screen_band(float rbn2, float drn2, float cmax, float dmax, int d) {
  const float fd = (float)d;
  const float a = __fmul_rn(drn2, cmax);
  const float b = __fmul_rn(rbn2, dmax);
  const float sig = __fmul_rn(2.f, __fsqrt_rn(__fdiv_rn(__fadd_rn(a, b), fd)));
  const float ecs = __fmul_rn(2.f, __fadd_rn(__fsqrt_rn(a), __fsqrt_rn(b)));
  const float escr = fminf(__fmul_rn(kBandZ, sig), ecs);
  const float tsum = __fadd_rn(__fmul_rn(2.f, __fsqrt_rn(__fmul_rn(rbn2, cmax))), cmax);
  const float nacc = fminf(__fadd_rn(fd, 2.f), __fmul_rn(kBandZ, __fsqrt_rn(__fadd_rn(fd, 2.f))));
  const float eacc = __fmul_rn(__fmul_rn(nacc, 0x1p-23f), tsum);
  const float enorm =
      __fmul_rn(__fadd_rn(__fmul_rn(__fadd_rn(__fmul_rn(0.5f, fd), 1.f), 0x1p-24f), 0x1p-17f), cmax);
  const float etag = __fmul_rn(0x1p-18f, tsum);
  const float e = __fmul_rn(__fadd_rn(__fadd_rn(escr, eacc), __fadd_rn(enorm, etag)), 1.0f + 0x1p-10f);
  return fmaxf(0.f, __fsub_rn(__fmul_rn(2.f, e), __fmul_rn(0.5e-4f, rbn2)));
}

// Per-lane candidate list of the sweep: blocks of 64 codewords whose
// smallest key came within the band of the running minimum.
constexpr int kList = 6;
// Split-mode record per (row, split, lane half), in float4 units: [cnt, 0,
// 0, 0], then up to kList list entries [k1, k2, base, 0]
constexpr int kRecF4 = 1 + kList;
// Candidates the encoder rescores per row and level (the smallest key's
// codeword included); a level with more is left to the exact scan.
constexpr int kMaxRescore = 6;
// repair codes per (row, level): kAuxOk when the band was complete; kAuxScan
// when it may not have been (the list overflowed, or two blocks each held
// two keys inside the band), so that the level is taken again by an exact
// fp32 scan
constexpr int kAuxOk = -1;
constexpr int kAuxScan = -2;

// ---- host-side launchers (return hipGetLastError of their launches) ----
// lstat [L][4]: max ||c||^2 and max ||c - bf16(c)||^2 of each level (the
// band bound's codebook terms); tstat [L][tiles][2] the per-tile maxima.
hipError_t launch_prepare(const float *cb, int L, int K, int d, float *norms, uint8_t *stream,
                          float *cbpad, int dp, float *tstat, float *lstat, hipStream_t s);

struct EncodePlan {
  bool fused;          // all levels in one launch
  int stages;          // feature stages (d padded to 64)
  int tiles;           // codeword tiles per level
  int row_blocks;
  int splits;          // split mode: workgroups per row block per level
  int tiles_per_split;
};
// The planner assumes at most this many compute units, so that workspace
// sizes (which do not know the device) bound every plan.
constexpr int kPlanMaxCus = 1024;
EncodePlan plan_encode(int64_t n, int d, int K, int num_cus);
// Whether some device may run n rows in split mode, and the split-mode
// records such a plan may write.
bool split_possible(int64_t n);
int64_t split_records(int64_t n, int K);
struct EncodeArgs {
  const void *x;        // caller's rows [n][d], fp32 or bf16
  int x_bf16;
  int64_t n;
  int d;                // true width
  int dp;               // row stride seen by the sweep: d rounded up to 16
  const uint8_t *stream;
  int L, K;
  const float *cb;      // fp32 codebooks with row stride dp
  float *rbuf[2];       // fp32 residuals [n][dp]: level l reads rbuf[l & 1], writes rbuf[(l+1) & 1]
  float *residual_out;  // caller's [n][d] output or null
  int32_t *ids;
  float4 *part;         // split mode: kRecF4 float4 per (row, split, lane half)
  const float *lstat;   // [L][4] codebook terms of the band bound
  float2 *rstat;        // split mode: (||r_b||^2, ||dr||^2) per row of the level's residual
  int32_t *aux;         // [n][L] repair codes (kAuxOk, kAuxScan)
  // Split mode: bf16 B-fragments of the rows the next sweep reads (the
  // input, then each level's residual), in blocks of 32 rows: the 16 bytes
  // of lane L for k-step ks of block b are at ((b * dp/16 + ks) * 64 + L),
  // holding features ks*16 + (L/32)*8 .. +7 of row 32 b + L%32.
  uint4 *xfrag;
  // set by launch_encode
  const float *src0;    // level-0 rows, fp32 stride dp (x itself or a staged copy)
  const uint16_t *x16;  // fused mode with bf16 rows of stride dp: level 0 reads them directly
  float *res_final;     // where the last level writes its residual (or null)
};
// The exact fp32 encoder of rows wider than the sweep holds: per level one
// distance launch (events: 2 L, around each) over `slices` codeword slices,
// then (slices > 1) a merge launch; rows of stride dp in rbuf.
int wide_slices(int64_t n, int K, int num_cus);
hipError_t launch_wide(const EncodeArgs &a, int slices, hipEvent_t *events, hipStream_t s);
hipError_t launch_encode(const EncodePlan &p, const EncodeArgs &a, hipEvent_t *events,
                         hipStream_t s);

hipError_t launch_embed(const int32_t *ids, const uint8_t *is_visual, int64_t T, int L,
                        const void *text, int64_t V, const void *vis, int K, int D, bool tab_bf16,
                        void *out, bool out_bf16, uint32_t *bad, hipStream_t s);
hipError_t launch_decode(const int32_t *ids, int64_t n, const float *cb, int L, int K, int d,
                         int levels, void *out, bool out_bf16, uint32_t *bad, hipStream_t s);
size_t hist_partial_bytes(int64_t n, int L, int K);
hipError_t launch_hist(const int32_t *ids, int64_t n, int L, int K, int64_t *hist,
                       uint32_t *partial, uint32_t *bad, hipStream_t s);
size_t msr_partial_bytes(int64_t n, int L);
// out_kind 0: statistics only; 1 / 2: also write the full decode of the
// rows to out as fp32 / bf16.
hipError_t launch_msr(const void *x, bool x_bf16, const int32_t *ids, int64_t n, int d,
                      const float *cb, int L, int K, double *msr, double *partial, void *out,
                      int out_kind, hipStream_t s);

}  // namespace rvq
