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

// ---- exact scans of the levels the sweep could not show complete ----
//
// A level with repair code kAuxScan (rare: a band list overflowed, or two
// blocks each held two keys inside the band) is taken again by an exact
// scan: the nearest codeword under the rescoring's own fp32 distance (two
// half sums in feature order, half 0 + half 1) over all K, the lower index
// on a tie.  The residual a scan needs is rebuilt from the row and its IDs
// with the encoder's fp32 subtractions.  Two kernels:
//   repair_list_kernel, one workgroup per 256 rows, lists the block's
//     flagged (row, level) entries in row, then level order (a block with
//     more than kRepairList entries is redone there, row by row);
//   repair_scan_kernel, a fixed grid, scans every listed entry in slices of
//     kRepairSlice codewords, one item per (entry, slice) spread over the
//     grid.  Each item's nearest goes into the entry's 64-bit key (distance
//     bits, then index: distances are not negative, so the unsigned minimum
//     is the lexicographic one).  The workgroup that finishes a block's last
//     item then redoes the block's rows: a flagged level takes its key's
//     index unless an earlier ID of the row changed; once an ID changes,
//     every later level is scanned whole, since its residual is no longer
//     the one the sweep and the keys saw.
// Changed IDs are rewritten, and so is the final residual of a row with a
// changed ID when the caller asked for it.
//
// Both kernels run after the sweep and the residual conversion, when the
// two residual buffers hold nothing live, and keep their lists there:
// rbuf[1] the listed count of each block, rbuf[0] an area of
// kRepairAreaBytes per block (ticket, keys, entries).  Each buffer holds
// round_up(n, 128) rows of at least 16 floats, at least 8 KiB per block.
constexpr int kRepairList = 448;
constexpr int kRepairSlice = 256;
constexpr int kRepairAreaBytes = 8192;
constexpr int kRepairKeysOff = 64;
constexpr int kRepairRowOff = kRepairKeysOff + kRepairList * 8;
constexpr int kRepairLevOff = kRepairRowOff + kRepairList * 4;
static_assert(kRepairLevOff + kRepairList * 4 <= kRepairAreaBytes, "repair area too small");
constexpr int kRepairChunk = 4096;  // block counts the scan kernel reads per pass, 16 a thread
constexpr unsigned kRepairGrid = 512;

struct RepairArea {
  unsigned *ticket;          // items of the block finished
  unsigned long long *keys;  // per entry: (distance bits << 32) | index
  int *row;                  // per entry: row within the block
  int *lev;                  // per entry: level
};

__device__ __forceinline__ RepairArea repair_area(const EncodeArgs &a, int64_t b) {
  char *p = (char *)a.rbuf[0] + b * kRepairAreaBytes;
  return {(unsigned *)p, (unsigned long long *)(p + kRepairKeysOff), (int *)(p + kRepairRowOff),
          (int *)(p + kRepairLevOff)};
}

// Exact fp32 distance of codeword c to the row res (in LDS): half 0
// (features ks*16 + e) and half 1 (ks*16 + 8 + e), each summed in feature
// order with fmaf, then half 0 + half 1, the rescoring's order.  Loads go
// eight k-steps at a time, all issued before their sums.
__device__ __forceinline__ float exact_dist(const float *c, const float *res, int nks) {
  float p0 = 0.f, p1 = 0.f;
  constexpr int G = 8;
  int ks = 0;
  for (; ks + G <= nks; ks += G) {
    float x0[G][8], x1[G][8];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      read8(c, 0, 0, (ks + u) * 16, true, x0[u]);
      read8(c, 0, 0, (ks + u) * 16 + 8, true, x1[u]);
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = res[(ks + u) * 16 + e] - x0[u][e];
        const float v = res[(ks + u) * 16 + 8 + e] - x1[u][e];
        p0 = fmaf(t, t, p0);
        p1 = fmaf(v, v, p1);
      }
    }
  }
  for (; ks < nks; ++ks) {
    float x0[8], x1[8];
    read8(c, 0, 0, ks * 16, true, x0);
    read8(c, 0, 0, ks * 16 + 8, true, x1);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float t = res[ks * 16 + e] - x0[e];
      const float v = res[ks * 16 + 8 + e] - x1[e];
      p0 = fmaf(t, t, p0);
      p1 = fmaf(v, v, p1);
    }
  }
  return p0 + p1;
}

// The nearest to res of codewords k0 + tid, k0 + tid + 256, ... below k1 of
// one level (the lower index on a tie), over the workgroup: every thread
// returns it.  Called by all 256 threads.
__device__ void wg_nearest(const float *cb_l, int dp, const float *res, int k0, int k1,
                           float *wd, int *wi, float &bd, int &bi) {
  const int tid = threadIdx.x;
  const int nks = dp >> 4;
  bd = __builtin_inff();
  bi = kNoIndex;
  for (int k = k0 + tid; k < k1; k += 256) {
    const float dk = exact_dist(cb_l + (int64_t)k * dp, res, nks);
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
  __syncthreads();
}

// res (LDS, dp floats) = the residual of a row entering level l: the row
// (zero past d) minus the chosen codewords of levels 0 .. l-1, in level
// order.  Each thread builds its own features; a barrier follows.
__device__ void row_residual(const EncodeArgs &a, int64_t row, int l, float *res) {
  const int32_t *id = a.ids + row * a.L;
  for (int i = threadIdx.x; i < a.dp; i += 256) {
    float v = 0.f;
    if (i < a.d)
      v = a.x_bf16 ? bf16_bits_to_f32(((const uint16_t *)a.x)[row * a.d + i])
                   : ((const float *)a.x)[row * a.d + i];
    int j = 0;
    for (; j + 4 <= l; j += 4) {
      float c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) c[u] = a.cb[((int64_t)(j + u) * a.K + id[j + u]) * a.dp + i];
#pragma unroll
      for (int u = 0; u < 4; ++u) v = v - c[u];
    }
    for (; j < l; ++j) v = v - a.cb[((int64_t)j * a.K + id[j]) * a.dp + i];
    res[i] = v;
  }
  __syncthreads();
}

// Redo one row level by level.  keys: the nearest of each flagged level of
// the row from the parallel scan, in level order, or null to scan every
// flagged level here.  The residual (res, LDS) is built only once a scan
// or a changed ID needs it, and then kept level by level.  A result outside
// [0, K) (only NaN distances give one) leaves the ID as the sweep chose it.
// flags: 256 ints of LDS for the row's repair codes.
__device__ void fix_row(const EncodeArgs &a, int64_t row, const unsigned long long *keys,
                        float *res, int *flags, float *wd, int *wi) {
  const int tid = threadIdx.x;
  bool changed = false, have = false;
  int q = 0;
  for (int l0 = 0; l0 < a.L; l0 += 256) {
    const int nl = a.L - l0 < 256 ? a.L - l0 : 256;
    __syncthreads();
    if (tid < nl) flags[tid] = a.aux[row * a.L + l0 + tid] == kAuxScan ? 1 : 0;
    __syncthreads();
    for (int t = 0; t < nl; ++t) {
      const int l = l0 + t;
      const bool flagged = flags[t] != 0;
      const float *cb_l = a.cb + (int64_t)l * a.K * a.dp;
      int id = -1;
      if (changed || flagged) {
        id = a.ids[row * a.L + l];
        int bi;
        if (!changed && keys) {
          bi = (int)(unsigned)__hip_atomic_load(keys + q, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        } else {
          if (!have) {
            row_residual(a, row, l, res);
            have = true;
          }
          float bd;
          wg_nearest(cb_l, a.dp, res, 0, a.K, wd, wi, bd, bi);
        }
        q += flagged ? 1 : 0;
        if (bi >= 0 && bi < a.K && bi != id) {
          if (!have) {
            row_residual(a, row, l, res);
            have = true;
          }
          changed = true;
          if (tid == 0) a.ids[row * a.L + l] = bi;
          id = bi;
        }
      }
      if (have) {
        if (id < 0) id = a.ids[row * a.L + l];
        for (int i = tid; i < a.dp; i += 256) res[i] = res[i] - cb_l[(int64_t)id * a.dp + i];
        __syncthreads();
      }
    }
  }
  if (changed && a.residual_out)
    for (int i = tid; i < a.d; i += 256) a.residual_out[row * a.d + i] = res[i];
  __syncthreads();
}

// Exclusive prefix of v over the 256 threads, and the total.
__device__ __forceinline__ int wg_exclusive_sum(int v, int *wsum, int &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = incl - v;
  total = 0;
  for (int w = 0; w < 4; ++w) {
    base += w < wave ? wsum[w] : 0;
    total += wsum[w];
  }
  __syncthreads();
  return base;
}

__global__ __launch_bounds__(256) void repair_list_kernel(EncodeArgs a) {
  __shared__ float res[kMaxStages * kStageCols];
  __shared__ int flagged[256];
  __shared__ int lvflags[256];
  __shared__ int wsum[4];
  __shared__ float wd[4];
  __shared__ int wi[4];
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t row = b * 256 + tid;
  // flagged levels per row, from the block's codes read as one contiguous
  // run (16-byte loads: the run starts 1 KiB-aligned)
  flagged[tid] = 0;
  __syncthreads();
  {
    const int64_t rows = a.n - b * 256 < 256 ? a.n - b * 256 : 256;
    const int64_t m = rows * a.L;
    const int32_t *ax = a.aux + b * 256 * a.L;
    for (int64_t i = tid; i < (m >> 2); i += 256) {
      const int4 v = reinterpret_cast<const int4 *>(ax)[i];
      const int e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (e[u] == kAuxScan) atomicAdd(&flagged[(int)((i * 4 + u) / a.L)], 1);
    }
    for (int64_t i = (m & ~(int64_t)3) + tid; i < m; i += 256)
      if (ax[i] == kAuxScan) atomicAdd(&flagged[(int)(i / a.L)], 1);
  }
  __syncthreads();
  const int c = flagged[tid];
  int total;
  const int base = wg_exclusive_sum(c, wsum, total);
  if (tid == 0) ((int *)a.rbuf[1])[b] = total <= kRepairList ? total : 0;
  if (total == 0) return;
  if (total <= kRepairList) {
    const RepairArea ar = repair_area(a, b);
    if (tid == 0) *ar.ticket = 0u;
    if (c > 0)
      for (int l = 0, q = base; l < a.L; ++l)
        if (a.aux[row * a.L + l] == kAuxScan) {
          ar.keys[q] = ~0ull;
          ar.row[q] = tid;
          ar.lev[q] = l;
          ++q;
        }
    return;
  }
  // more entries than a block lists: this workgroup redoes its rows
  for (int r = 0; r < 256; ++r)
    if (flagged[r] > 0) fix_row(a, b * 256 + r, nullptr, res, lvflags, wd, wi);
}

__global__ __launch_bounds__(256) void repair_scan_kernel(EncodeArgs a, int64_t nb, int slices) {
  __shared__ float res[kMaxStages * kStageCols];
  __shared__ int pre[kRepairChunk + 1];
  __shared__ int lvflags[256];
  __shared__ int wsum[4];
  __shared__ float wd[4];
  __shared__ int wi[4];
  __shared__ int last;
  const int tid = threadIdx.x;
  const int *bcnt = (const int *)a.rbuf[1];
  const int64_t G = gridDim.x;
  int64_t E = 0;  // entries listed by the blocks before this pass's
  for (int64_t c0 = 0; c0 < nb; c0 += kRepairChunk) {
    // pre[i]: entries of blocks c0 .. c0+i-1; pre[kRepairChunk]: the pass's
    int v[16], t = 0;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int64_t b = c0 + tid * 16 + u;
      v[u] = b < nb ? bcnt[b] : 0;
      t += v[u];
    }
    int total;
    int acc = wg_exclusive_sum(t, wsum, total);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      pre[tid * 16 + u] = acc;
      acc += v[u];
    }
    if (tid == 0) pre[kRepairChunk] = total;
    __syncthreads();
    // items (entry, slice) of this pass, entry-major, dealt round robin
    const int64_t lo = E * slices, hi = (E + total) * slices;
    for (int64_t it = lo + (((int64_t)blockIdx.x - lo % G) + G) % G; it < hi; it += G) {
      const int e = (int)(it / slices - E);
      const int s = (int)(it % slices);
      // the block of entry e: the last bl with pre[bl] <= e
      int bl = 0;
#pragma unroll
      for (int step = kRepairChunk / 2; step > 0; step >>= 1)
        if (pre[bl + step] <= e) bl += step;
      const int64_t b = c0 + bl;
      const int j = e - pre[bl];
      const int cnt = pre[bl + 1] - pre[bl];
      const RepairArea ar = repair_area(a, b);
      const int l = ar.lev[j];
      row_residual(a, b * 256 + ar.row[j], l, res);
      float bd;
      int bi;
      const int k0 = s * kRepairSlice;
      const int k1 = a.K - k0 < kRepairSlice ? a.K : k0 + kRepairSlice;
      wg_nearest(a.cb + (int64_t)l * a.K * a.dp, a.dp, res, k0, k1, wd, wi, bd, bi);
      if (tid == 0) {
        atomicMin(ar.keys + j, ((unsigned long long)__float_as_uint(bd) << 32) | (unsigned)bi);
        __threadfence();
        last = atomicAdd(ar.ticket, 1u) + 1u == (unsigned)cnt * (unsigned)slices;
      }
      __syncthreads();
      if (last) {
        // every item of block b is in: redo its rows
        __threadfence();
        for (int q = 0; q < cnt;) {
          const int r = ar.row[q];
          fix_row(a, b * 256 + r, ar.keys + q, res, lvflags, wd, wi);
          while (q < cnt && ar.row[q] == r) ++q;
        }
      }
      __syncthreads();
    }
    E += total;
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
  // (stages == 0: rows wider than the sweep holds, for the exact fp32 encoder)
  p.fused = p.stages > 0 && (int64_t)p.row_blocks * 10 >= (int64_t)cus * 6;
  if (p.stages == 0) {
    // wide rows: codeword slices of the exact fp32 encoder
    p.splits = wide_slices(n, K, cus);
    p.tiles_per_split = p.tiles;
  } else if (p.fused) {
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
  if (p.stages == 0) {
    // rows wider than the sweep holds: exact fp32 distances, nothing to
    // rescan afterwards
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_wide(a, p.splits, events, s);
    if (e != hipSuccess) return e;
    if (convert)
      unpad_kernel<<<dim3(row_waves), dim3(256), 0, s>>>(final_buf, a.n, a.d, a.dp,
                                                         a.residual_out);
    return hipGetLastError();
  }
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
  const int64_t nb = ceil_div(a.n, 256);
  repair_list_kernel<<<dim3((unsigned)nb), dim3(256), 0, s>>>(a);
  repair_scan_kernel<<<dim3(kRepairGrid), dim3(256), 0, s>>>(a, nb,
                                                            (int)ceil_div(a.K, kRepairSlice));
  return hipGetLastError();
}

}  // namespace rvq
