// encode.hip -- one level of greedy residual vector quantization.
//
// Method: "LongCat-2.5 Native Multimodality for Agentic Tasks", section
// "Visual Primitive Modeling", paragraph "Discrete Native Resolution Vision
// Transformer" (RVQ on native-resolution features) and "LongCat-2.5 Open
// Source Release ...", section "02 Visual Coding and 3D" (detail added level
// by level).  Per level and row r the nearest codeword under the squared
// Euclidean distance ||r||^2 - 2 r.c + ||c||^2 is chosen; ||r||^2 is the
// same for every codeword, so codewords are ranked by the score
// ||c||^2 - 2 r.c.
//
// Two kernels per level:
//   distance_top2_kernel  dense contraction of bf16 residual rows with the
//       bf16 codebook on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32
//       accumulation over the whole feature dimension, which is never split
//       across workgroups), with a fused epilogue that keeps each row's two
//       best (score, index) pairs.  Each workgroup covers one block of rows
//       and a range of codeword tiles and writes one top-2 list per row.
//   rescore_update_kernel  merges a row's top-2 lists, rescores the two
//       candidates exactly in fp32 (sum of squared differences), picks the
//       smaller (lower index on a tie), writes the ID, subtracts the chosen
//       fp32 codeword from the fp32 residual and refreshes the bf16 copy the
//       next level's contraction reads.
// Scores depend only on (row, codeword) -- one MFMA shape, one feature
// order -- so a row's IDs never depend on the other rows of the batch.
#include "common.h"

namespace rvq {

namespace {

constexpr int BM = kTileCodewords;  // 256 codewords per tile
constexpr int BN = kTileRows;       // 128 rows per tile
constexpr int BK = kStageCols;      // 32 feature columns per stage
constexpr int LDS_ROW = BK + 8;     // bf16 per LDS row: 80 B, conflict-free 16-B reads
constexpr int NT = 256;             // 4 waves: 2 (codeword halves) x 2 (row halves)

// Workgroup id -> (row block, split).  Workgroups are dispatched round-robin
// over the 8 XCDs, each with its own L2; the linear order below gives every
// XCD a contiguous range of tiles, and inside it tiles come in groups of
// `group` row blocks x all splits, row block fastest, so the workgroups
// running together on one XCD share row blocks and codeword tiles in L2.
__device__ __forceinline__ bool tile_of(int bid, int n_rb, int S, int group, int per_xcd, int &rb,
                                        int &split) {
  const int xcd = bid % kNumXcd;
  const int j = bid / kNumXcd;
  const int64_t t = (int64_t)xcd * per_xcd + j;
  const int64_t total = (int64_t)n_rb * S;
  if (j >= per_xcd || t >= total) return false;
  const int64_t gsz = (int64_t)group * S;
  const int g = (int)(t / gsz);
  const int within = (int)(t % gsz);
  const int rows_in_group = min(group, n_rb - g * group);
  split = within / rows_in_group;
  rb = g * group + within % rows_in_group;
  return true;
}

}  // namespace

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void distance_top2_kernel(
    const uint16_t *__restrict__ r16, int64_t n, int Dp, const uint16_t *__restrict__ cbh,
    const float *__restrict__ norms, int ktiles, int T, int S, int n_rb, int group, int per_xcd,
    float4 *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * LDS_ROW];
  __shared__ float4 norm_s[BM / 4];
  __shared__ float4 xchg[BN];

  int rb, split;
  if (!tile_of(blockIdx.x, n_rb, S, group, per_xcd, rb, split)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;   // codewords wm*128 .. +127 of the tile
  const int wn = wave >> 1;  // rows wn*64 .. +63 of the block
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int64_t row0 = (int64_t)rb * BN;

  // Global -> LDS copy assignment: 16 B per chunk, 4 chunks per 64-B row segment.
  // A (codebook tile): 1024 chunks, 4 per thread.  B (rows): 512 chunks, 2 per thread.
  const uint16_t *bsrc[2];
  int b_lds[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + NT * j;
    const int r = c >> 2;
    int64_t gr = row0 + r;
    if (gr > n - 1) gr = n - 1;  // ragged tail: reuse the last row, result discarded
    bsrc[j] = r16 + gr * Dp + (c & 3) * 8;
    b_lds[j] = r * LDS_ROW + (c & 3) * 8;
  }
  int a_off[4], a_lds[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + NT * j;
    a_off[j] = (c >> 2) * Dp + (c & 3) * 8;
    a_lds[j] = (c >> 2) * LDS_ROW + (c & 3) * 8;
  }

  float s1[2], s2[2];
  int i1[2], i2[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s1[t] = s2[t] = __builtin_inff();
    i1[t] = i2[t] = kNoIndex;
  }

  const int nst = Dp / BK;
  for (int tt = 0; tt < T; ++tt) {
    const int kt = split * T + tt;
    if (kt >= ktiles) break;
    const uint16_t *cbt = cbh + (int64_t)kt * BM * Dp;
    __syncthreads();  // previous tile's epilogue has finished with norm_s
    if (tid < BM / 4) norm_s[tid] = reinterpret_cast<const float4 *>(norms + (int64_t)kt * BM)[tid];

    f32x16 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

    uint4 ra[4], rbv[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) ra[j] = *reinterpret_cast<const uint4 *>(cbt + a_off[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) rbv[j] = *reinterpret_cast<const uint4 *>(bsrc[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4 *>(&As[0][a_lds[j]]) = ra[j];
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<uint4 *>(&Bs[0][b_lds[j]]) = rbv[j];
    __syncthreads();

    for (int s = 0; s < nst; ++s) {
      const int cur = s & 1;
      if (s + 1 < nst) {
        const int d0 = (s + 1) * BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) ra[j] = *reinterpret_cast<const uint4 *>(cbt + a_off[j] + d0);
#pragma unroll
        for (int j = 0; j < 2; ++j) rbv[j] = *reinterpret_cast<const uint4 *>(bsrc[j] + d0);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 af[4], bfr[2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = *reinterpret_cast<const bf16x8 *>(
              &As[cur][(wm * 128 + mt * 32 + l32) * LDS_ROW + ks * 16 + hi * 8]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bfr[nt] = *reinterpret_cast<const bf16x8 *>(
              &Bs[cur][(wn * 64 + nt * 32 + l32) * LDS_ROW + ks * 16 + hi * 8]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
      }
      if (s + 1 < nst) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4 *>(&As[cur ^ 1][a_lds[j]]) = ra[j];
#pragma unroll
        for (int j = 0; j < 2; ++j) *reinterpret_cast<uint4 *>(&Bs[cur ^ 1][b_lds[j]]) = rbv[j];
      }
      __syncthreads();
    }

    // Epilogue.  Accumulator element i of tile (mt, nt) holds codeword
    // (i/4)*8 + hi*4 + i%4 of the 32-codeword M tile for row l32 of the N
    // tile; visiting (mt, i) in order visits this lane's codewords in
    // increasing index order, so a strict '<' keeps the lower index on ties.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cw_local = wm * 128 + mt * 32 + g * 8 + hi * 4;
        const float4 nv = norm_s[cw_local >> 2];
        const float nvq[4] = {nv.x, nv.y, nv.z, nv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cw = kt * BM + cw_local + q;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const float sc = fmaf(-2.0f, acc[mt][nt][g * 4 + q], nvq[q]);
            const bool lt2 = sc < s2[nt];
            const bool lt1 = sc < s1[nt];
            const float ns2 = lt1 ? s1[nt] : (lt2 ? sc : s2[nt]);
            const int ni2 = lt1 ? i1[nt] : (lt2 ? cw : i2[nt]);
            s1[nt] = lt1 ? sc : s1[nt];
            i1[nt] = lt1 ? cw : i1[nt];
            s2[nt] = ns2;
            i2[nt] = ni2;
          }
        }
      }
    }
  }

  // Merge the two lanes that hold the same row (lane and lane ^ 32).
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const float t1 = __shfl_xor(s1[nt], 32, 64);
    const int j1 = __shfl_xor(i1[nt], 32, 64);
    const float t2 = __shfl_xor(s2[nt], 32, 64);
    const int j2 = __shfl_xor(i2[nt], 32, 64);
    merge_top2(s1[nt], i1[nt], s2[nt], i2[nt], t1, j1, t2, j2);
  }
  // Merge the two waves that hold the same rows (codeword halves wm = 0, 1).
  if (wm == 1 && hi == 0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      xchg[wn * 64 + nt * 32 + l32] =
          make_float4(s1[nt], __int_as_float(i1[nt]), s2[nt], __int_as_float(i2[nt]));
  }
  __syncthreads();
  if (wm == 0 && hi == 0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float4 o = xchg[wn * 64 + nt * 32 + l32];
      merge_top2(s1[nt], i1[nt], s2[nt], i2[nt], o.x, __float_as_int(o.y), o.z,
                 __float_as_int(o.w));
      const int64_t row = row0 + wn * 64 + nt * 32 + l32;
      if (row < n)
        part[row * S + split] =
            make_float4(s1[nt], __int_as_float(i1[nt]), s2[nt], __int_as_float(i2[nt]));
    }
  }
}

DistPlan plan_distance(int64_t n, int K, int num_cus) {
  DistPlan p{};
  p.ktiles = (int)ceil_div(K, BM);
  p.row_blocks = (int)ceil_div(n, BN);
  // Two workgroups fit per CU (60 KB of LDS each).  Pick the number of
  // codeword tiles per workgroup that keeps the last round of workgroups
  // fullest, preferring more tiles per workgroup on a tie (fewer partial
  // top-2 lists to merge).
  const int64_t slots = (int64_t)2 * (num_cus > 0 ? num_cus : 256);
  double best_eff = -1.0;
  int best_t = 1;
  for (int t = 1; t <= p.ktiles; t *= 2) {
    const int64_t wgs = (int64_t)p.row_blocks * ceil_div(p.ktiles, t);
    const int64_t rounds = ceil_div(wgs, slots);
    const double eff = (double)wgs / (double)(rounds * slots) *
                       ((double)p.ktiles / (double)(ceil_div(p.ktiles, t) * t));
    if (eff > best_eff + 0.02) {
      best_eff = eff;
      best_t = t;
    } else if (eff >= best_eff - 0.02 && wgs >= 4 * slots) {
      best_t = t;
      if (eff > best_eff) best_eff = eff;
    }
  }
  p.tiles_per_wg = best_t;
  p.splits = (int)ceil_div(p.ktiles, best_t);
  p.group = 8;
  const int64_t total = (int64_t)p.row_blocks * p.splits;
  p.per_xcd = (int)ceil_div(total, kNumXcd);
  p.grid = p.per_xcd * kNumXcd;
  return p;
}

hipError_t launch_distance_top2(const DistPlan &p, const uint16_t *r16, int64_t n, int Dp,
                                const uint16_t *cbh_l, const float *norms_l, float4 *part,
                                hipStream_t s) {
  if (n == 0) return hipSuccess;
  distance_top2_kernel<<<dim3(p.grid), dim3(NT), 0, s>>>(r16, n, Dp, cbh_l, norms_l, p.ktiles,
                                                         p.tiles_per_wg, p.splits, p.row_blocks,
                                                         p.group, p.per_xcd, part);
  return hipGetLastError();
}

// One wave per row.  Memory-bound: reads the row's top-2 lists, its fp32
// residual and two fp32 codewords; writes the new residual (fp32 and bf16)
// and one ID.
__global__ __launch_bounds__(256) void rescore_update_kernel(
    const float4 *__restrict__ part, int S, int64_t n, int d, int Dp, int K, int L, int level,
    const float *__restrict__ cb_l, const float *r_in, float *r_out, uint16_t *__restrict__ r16,
    int write_r16, int32_t *__restrict__ ids) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;

  float s1 = __builtin_inff(), s2 = __builtin_inff();
  int i1 = kNoIndex, i2 = kNoIndex;
  for (int j = lane; j < S; j += 64) {
    const float4 p = part[row * S + j];
    merge_top2(s1, i1, s2, i2, p.x, __float_as_int(p.y), p.z, __float_as_int(p.w));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float t1 = __shfl_xor(s1, off, 64);
    const int j1 = __shfl_xor(i1, off, 64);
    const float t2 = __shfl_xor(s2, off, 64);
    const int j2 = __shfl_xor(i2, off, 64);
    // Lists from different lanes can hold the same index only if both are
    // empty slots; merge_top2 keeps the result well-defined either way.
    merge_top2(s1, i1, s2, i2, t1, j1, t2, j2);
  }
  const bool v1 = i1 >= 0 && i1 < K;
  const bool v2 = i2 >= 0 && i2 < K && i2 != i1;
  const int c1 = v1 ? i1 : 0;  // a finite input always yields a valid first candidate
  const int c2 = v2 ? i2 : c1;

  const float *r = r_in + row * d;
  const float *C1 = cb_l + (int64_t)c1 * d;
  const float *C2 = cb_l + (int64_t)c2 * d;
  float d1 = 0.f, d2 = 0.f;
  for (int i = lane; i < d; i += 64) {
    const float rv = r[i];
    const float a = rv - C1[i];
    const float b = rv - C2[i];
    d1 = fmaf(a, a, d1);
    d2 = fmaf(b, b, d2);
  }
  d1 = wave_sum_f32(d1);
  d2 = wave_sum_f32(d2);
  const int id = (v2 && (d2 < d1 || (d2 == d1 && c2 < c1))) ? c2 : c1;
  if (lane == 0) ids[row * L + level] = id;

  const float *C = cb_l + (int64_t)id * d;
  float *ro = r_out + row * d;
  for (int i = lane; i < d; i += 64) {
    const float v = r[i] - C[i];
    ro[i] = v;
    if (write_r16) r16[row * Dp + i] = f32_to_bf16_bits(v);
  }
}

hipError_t launch_rescore_update(const float4 *part, int splits, int64_t n, int d, int Dp, int K,
                                 int L, int level, const float *cb_l, const float *r_in,
                                 float *r_out, uint16_t *r16, bool write_r16, int32_t *ids,
                                 hipStream_t s) {
  if (n == 0) return hipSuccess;
  rescore_update_kernel<<<dim3((unsigned)ceil_div(n, 4)), dim3(256), 0, s>>>(
      part, splits, n, d, Dp, K, L, level, cb_l, r_in, r_out, r16, write_r16 ? 1 : 0, ids);
  return hipGetLastError();
}

}  // namespace rvq
