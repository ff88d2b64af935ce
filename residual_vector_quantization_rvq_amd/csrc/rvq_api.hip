// rvq_api.hip -- the C ABI declared in include/rvq.h.
//
// Host side only: argument validation (before any HIP call), workspace
// layout, kernel planning and the per-level launch sequence of the encoder.
// Everything is enqueued on the caller's stream; nothing is allocated.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "rvq.h"
#include "common.h"

using namespace rvq;

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace rvq {
// Records the message that rvq_last_error returns (per thread) and returns
// st; shared by the library's host sources.
rvq_status fail(rvq_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
rvq_status fail(rvq_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
}  // namespace rvq

namespace {

rvq_status hip_fail(hipError_t e, const char *what) {
  return fail(RVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxRows = (int64_t)1 << 25;  // one wave per row: grid work-items < 2^32
constexpr int kMaxLevelsGather = 64;            // decode / statistics: IDs of a row in one wave

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

rvq_status check_shape(int64_t n, int32_t d, int32_t L, int32_t K) {
  if (n < 0) return fail(RVQ_ERR_INVALID_ARGUMENT, "n must be >= 0 (got %lld)", (long long)n);
  if (d < 1) return fail(RVQ_ERR_INVALID_ARGUMENT, "d must be >= 1 (got %d)", d);
  if (L < 1) return fail(RVQ_ERR_INVALID_ARGUMENT, "L must be >= 1 (got %d)", L);
  if (K < 1) return fail(RVQ_ERR_INVALID_ARGUMENT, "K must be >= 1 (got %d)", K);
  if (K > INT32_MAX - kTileCw)
    return fail(RVQ_ERR_UNSUPPORTED, "K too large (got %d)", K);
  if (n > kMaxRows)
    return fail(RVQ_ERR_UNSUPPORTED, "n above %lld rows per call (got %lld)", (long long)kMaxRows,
                (long long)n);
  if (stream_bytes(L, K, d) > ((int64_t)1 << 40))
    return fail(RVQ_ERR_UNSUPPORTED, "codebook too large");
  return RVQ_OK;
}

rvq_status need(const void *p, const char *name, size_t align) {
  if (!p) return fail(RVQ_ERR_INVALID_ARGUMENT, "%s must not be NULL", name);
  if (!aligned(p, align))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "%s must be %zu-byte aligned", name, align);
  return RVQ_OK;
}

#define RVQ_TRY(expr)                     \
  do {                                    \
    rvq_status _st = (expr);              \
    if (_st != RVQ_OK) return _st;        \
  } while (0)

#define HIP_TRY(expr, what)               \
  do {                                    \
    hipError_t _e = (expr);               \
    if (_e != hipSuccess) return hip_fail(_e, what); \
  } while (0)

// Row stride of the fp32 rows and codewords the encoder reads.
int32_t row_stride(int32_t d) { return (int32_t)round_up(d, 16); }

// Prepared buffer: norms [L][Kp] fp32, the fragment stream, the codebook
// terms of the band bound (per tile [L][tiles][2], per level [L][4]) and
// (only when d is not a multiple of 16) an fp32 copy of the codebooks with
// stride dp.
struct PreparedLayout {
  size_t norms_off, stream_off, tstat_off, lstat_off, cbpad_off, total;
};
PreparedLayout prepared_layout(int32_t L, int32_t K, int32_t d) {
  PreparedLayout p;
  p.norms_off = 0;
  p.stream_off = align256((size_t)L * (size_t)padded_k(K) * sizeof(float));
  p.tstat_off = p.stream_off + align256((size_t)stream_bytes(L, K, d));
  p.lstat_off = p.tstat_off + align256((size_t)L * (size_t)(padded_k(K) / kTileCw) * 2 * sizeof(float));
  p.cbpad_off = p.lstat_off + align256((size_t)L * 4 * sizeof(float));
  const int32_t dp = row_stride(d);
  p.total = p.cbpad_off + (dp != d ? align256((size_t)L * K * dp * sizeof(float)) : 0);
  return p;
}

struct EncodeLayout {
  size_t r0_off, r1_off, aux_off, part_off, frag_off, rstat_off, total;
};
// Workspace: two fp32 residual buffers [n][dp] (level l reads one and
// writes the other), the repair codes [n][L] and, when some device may run
// the split plan for n rows, its records (kRecF4 float4 per row, split and
// row half, for the largest split count), the bf16 B-fragments of the rows
// the next sweep reads [n][dp] and the rows' band inputs [n] float2.
EncodeLayout encode_layout(int64_t n, int32_t d, int32_t L, int32_t K) {
  EncodeLayout w;
  // rows rounded up to whole workgroups: the fused encoder keeps residuals
  // in fragment-major blocks of 32 rows, one set of 4 per workgroup
  const size_t rbytes =
      align256((size_t)round_up(n, kRowsPerWG) * row_stride(d) * sizeof(float));
  w.r0_off = 0;
  w.r1_off = rbytes;
  w.aux_off = 2 * rbytes;
  w.part_off = w.aux_off + align256((size_t)n * L * sizeof(int32_t));
  const bool split = split_possible(n);
  w.frag_off =
      w.part_off + (split ? align256((size_t)split_records(n, K) * kRecF4 * sizeof(float4)) : 0);
  w.rstat_off =
      w.frag_off + (split ? align256((size_t)round_up(n, kRowsPerWG) * row_stride(d) * 2) : 0);
  w.total = w.rstat_off + (split ? align256((size_t)n * sizeof(float2)) : 0);
  if (w.total == 0) w.total = 256;
  return w;
}

int num_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 256;
  return cus > 0 ? cus : 256;
}

rvq_status check_encode_width(int32_t d, int32_t K);

}  // namespace

extern "C" {

const char *rvq_status_string(rvq_status s) {
  switch (s) {
    case RVQ_OK: return "RVQ_OK";
    case RVQ_ERR_INVALID_ARGUMENT: return "RVQ_ERR_INVALID_ARGUMENT";
    case RVQ_ERR_UNSUPPORTED: return "RVQ_ERR_UNSUPPORTED";
    case RVQ_ERR_WORKSPACE_TOO_SMALL: return "RVQ_ERR_WORKSPACE_TOO_SMALL";
    case RVQ_ERR_HIP: return "RVQ_ERR_HIP";
  }
  return "RVQ_ERR_UNKNOWN";
}

const char *rvq_last_error(void) { return g_err; }

namespace {
rvq_status check_encode_width(int32_t d, int32_t K) {
  // d <= 1280: the matrix-core sweep; up to kWideMaxD: the exact fp32 encoder
  if (stages_for(d) == 0 && d > kWideMaxD)
    return fail(RVQ_ERR_UNSUPPORTED, "encode supports d <= %d (got %d)", kWideMaxD, d);
  // the fused update addresses a level's codewords with 32-bit lane offsets
  if ((int64_t)K * row_stride(d) * (int64_t)sizeof(float) > (int64_t)UINT32_MAX)
    return fail(RVQ_ERR_UNSUPPORTED, "encode supports K * d below 2^30 per level (got K=%d, d=%d)",
                K, d);
  return RVQ_OK;
}
}  // namespace

rvq_status rvq_prepared_size(int32_t L, int32_t K, int32_t d, size_t *bytes) {
  RVQ_TRY(check_shape(0, d, L, K));
  RVQ_TRY(check_encode_width(d, K));
  if (!bytes) return fail(RVQ_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  *bytes = prepared_layout(L, K, d).total;
  return RVQ_OK;
}

rvq_status rvq_prepare_codebooks(const float *codebooks, int32_t L, int32_t K, int32_t d,
                                 void *prepared, size_t prepared_bytes, hipStream_t stream) {
  RVQ_TRY(check_shape(0, d, L, K));
  RVQ_TRY(check_encode_width(d, K));
  RVQ_TRY(need(codebooks, "codebooks", 16));
  RVQ_TRY(need(prepared, "prepared", 256));
  const PreparedLayout pl = prepared_layout(L, K, d);
  if (prepared_bytes < pl.total)
    return fail(RVQ_ERR_WORKSPACE_TOO_SMALL, "prepared buffer needs %zu bytes (got %zu)", pl.total,
                prepared_bytes);
  char *base = (char *)prepared;
  const int32_t dp = row_stride(d);
  HIP_TRY(launch_prepare(codebooks, L, K, d, (float *)(base + pl.norms_off),
                         (uint8_t *)(base + pl.stream_off),
                         dp != d ? (float *)(base + pl.cbpad_off) : nullptr, dp,
                         (float *)(base + pl.tstat_off), (float *)(base + pl.lstat_off), stream),
          "codebook preparation launch");
  return RVQ_OK;
}

rvq_status rvq_encode_workspace_size(int64_t n, int32_t d, int32_t L, int32_t K, size_t *bytes) {
  RVQ_TRY(check_shape(n, d, L, K));
  RVQ_TRY(check_encode_width(d, K));
  if (!bytes) return fail(RVQ_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  *bytes = encode_layout(n, d, L, K).total;
  return RVQ_OK;
}

rvq_status rvq_encode_profiled(const void *x, rvq_dtype x_dtype, int64_t n, int32_t d,
                               const float *codebooks, const void *prepared, int32_t L, int32_t K,
                               int32_t *ids, float *residual_out, void *workspace,
                               size_t workspace_bytes, hipStream_t stream, hipEvent_t *events,
                               int32_t *launches) {
  RVQ_TRY(check_shape(n, d, L, K));
  RVQ_TRY(check_encode_width(d, K));
  if (x_dtype != RVQ_F32 && x_dtype != RVQ_BF16)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown x_dtype %d", (int)x_dtype);
  RVQ_TRY(need(codebooks, "codebooks", 16));
  RVQ_TRY(need(prepared, "prepared", 256));
  if (n > 0) {
    RVQ_TRY(need(x, "x", x_dtype == RVQ_BF16 ? 2 : 4));
    RVQ_TRY(need(ids, "ids", 4));
    if (residual_out && !aligned(residual_out, 4))
      return fail(RVQ_ERR_INVALID_ARGUMENT, "residual_out must be 4-byte aligned");
  }
  const EncodeLayout wl = encode_layout(n, d, L, K);
  RVQ_TRY(need(workspace, "workspace", 256));
  if (workspace_bytes < wl.total)
    return fail(RVQ_ERR_WORKSPACE_TOO_SMALL, "encode workspace needs %zu bytes (got %zu)",
                wl.total, workspace_bytes);
  if (launches) *launches = 0;
  if (n == 0) return RVQ_OK;

  const PreparedLayout pl = prepared_layout(L, K, d);
  char *ws = (char *)workspace;
  EncodeArgs a;
  a.x = x;
  a.x_bf16 = x_dtype == RVQ_BF16 ? 1 : 0;
  a.n = n;
  a.d = d;
  a.dp = row_stride(d);
  a.stream = (const uint8_t *)prepared + pl.stream_off;
  a.L = L;
  a.K = K;
  a.cb = a.dp != d ? (const float *)((const char *)prepared + pl.cbpad_off) : codebooks;
  a.rbuf[0] = (float *)(ws + wl.r0_off);
  a.rbuf[1] = (float *)(ws + wl.r1_off);
  a.residual_out = residual_out;
  a.ids = ids;
  a.part = (float4 *)(ws + wl.part_off);
  a.xfrag = (uint4 *)(ws + wl.frag_off);
  a.lstat = (const float *)((const char *)prepared + pl.lstat_off);
  a.rstat = (float2 *)(ws + wl.rstat_off);
  a.aux = (int32_t *)(ws + wl.aux_off);
  const EncodePlan plan = plan_encode(n, d, K, num_cus());
  HIP_TRY(launch_encode(plan, a, events, stream), "encode launch");
  if (launches) *launches = plan.fused ? 1 : L;
  return RVQ_OK;
}

rvq_status rvq_encode(const void *x, rvq_dtype x_dtype, int64_t n, int32_t d,
                      const float *codebooks, const void *prepared, int32_t L, int32_t K,
                      int32_t *ids, float *residual_out, void *workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return rvq_encode_profiled(x, x_dtype, n, d, codebooks, prepared, L, K, ids, residual_out,
                             workspace, workspace_bytes, stream, nullptr, nullptr);
}

rvq_status rvq_decode(const int32_t *ids, int64_t n, const float *codebooks, int32_t L, int32_t K,
                      int32_t d, int32_t levels, void *out, rvq_dtype out_dtype, uint32_t *bad_ids,
                      hipStream_t stream) {
  RVQ_TRY(check_shape(n, d, L, K));
  if (L > kMaxLevelsGather)
    return fail(RVQ_ERR_UNSUPPORTED, "decode supports L <= %d (got %d)", kMaxLevelsGather, L);
  if (levels < 0 || levels > L)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "levels must be in [0, L] (got %d)", levels);
  if (out_dtype != RVQ_F32 && out_dtype != RVQ_BF16)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown out_dtype %d", (int)out_dtype);
  RVQ_TRY(need(codebooks, "codebooks", 16));
  if (n > 0) {
    RVQ_TRY(need(ids, "ids", 4));
    RVQ_TRY(need(out, "out", 16));
  }
  if (bad_ids && !aligned(bad_ids, 4))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "bad_ids must be 4-byte aligned");
  if (n == 0) return RVQ_OK;
  HIP_TRY(launch_decode(ids, n, codebooks, L, K, d, levels, out, out_dtype == RVQ_BF16, bad_ids,
                        stream),
          "decode_kernel launch");
  return RVQ_OK;
}

rvq_status rvq_embed_tokens(const int32_t *ids, const uint8_t *is_visual, int64_t T, int32_t L,
                            const void *text_table, int64_t V, const void *level_tables,
                            int32_t K, int32_t D, rvq_dtype table_dtype, void *out,
                            rvq_dtype out_dtype, uint32_t *bad_ids, hipStream_t stream) {
  if (T < 0) return fail(RVQ_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %lld)", (long long)T);
  if (L < 1 || K < 1 || D < 1 || V < 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "need L, K, D >= 1 and V >= 0 (got %d, %d, %d, %lld)",
                L, K, D, (long long)V);
  if (L > kMaxLevelsGather)
    return fail(RVQ_ERR_UNSUPPORTED, "embedding supports L <= %d (got %d)", kMaxLevelsGather, L);
  if (T > kMaxRows)
    return fail(RVQ_ERR_UNSUPPORTED, "T above %lld tokens per call (got %lld)",
                (long long)kMaxRows, (long long)T);
  if (table_dtype != RVQ_F32 && table_dtype != RVQ_BF16)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown table_dtype %d", (int)table_dtype);
  if (out_dtype != RVQ_F32 && out_dtype != RVQ_BF16)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown out_dtype %d", (int)out_dtype);
  RVQ_TRY(need(level_tables, "level_tables", 16));
  if (V > 0) RVQ_TRY(need(text_table, "text_table", 16));
  if (T > 0) {
    RVQ_TRY(need(ids, "ids", 4));
    RVQ_TRY(need(out, "out", 16));
  }
  if (bad_ids && !aligned(bad_ids, 4))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "bad_ids must be 4-byte aligned");
  if (T == 0) return RVQ_OK;
  HIP_TRY(launch_embed(ids, is_visual, T, L, V > 0 ? text_table : nullptr, V, level_tables, K, D,
                       table_dtype == RVQ_BF16, out, out_dtype == RVQ_BF16, bad_ids, stream),
          "embed_kernel launch");
  return RVQ_OK;
}

rvq_status rvq_level_stats_workspace_size(int64_t n, int32_t L, int32_t K, int32_t d,
                                          int32_t with_msr, size_t *bytes) {
  RVQ_TRY(check_shape(n, with_msr ? d : 1, L, K));
  if (!bytes) return fail(RVQ_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  size_t total = align256(hist_partial_bytes(n, L, K));
  if (with_msr) total += align256(msr_partial_bytes(n, L));
  *bytes = total > 0 ? total : 256;
  return RVQ_OK;
}

rvq_status rvq_level_stats(const int32_t *ids, int64_t n, int32_t L, int32_t K, int64_t *hist,
                           const void *x, rvq_dtype x_dtype, int32_t d, const float *codebooks,
                           double *msr, uint32_t *bad_ids, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  const bool with_msr = msr != nullptr;
  RVQ_TRY(check_shape(n, with_msr ? d : 1, L, K));
  if (L > kMaxLevelsGather)
    return fail(RVQ_ERR_UNSUPPORTED, "level statistics support L <= %d (got %d)",
                kMaxLevelsGather, L);
  RVQ_TRY(need(hist, "hist", 8));
  if (n > 0) RVQ_TRY(need(ids, "ids", 4));
  if (with_msr) {
    if (x_dtype != RVQ_F32 && x_dtype != RVQ_BF16)
      return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown x_dtype %d", (int)x_dtype);
    RVQ_TRY(need(codebooks, "codebooks", 16));
    RVQ_TRY(need(msr, "msr", 8));
    if (n > 0) RVQ_TRY(need(x, "x", x_dtype == RVQ_BF16 ? 2 : 4));
  }
  if (bad_ids && !aligned(bad_ids, 4))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "bad_ids must be 4-byte aligned");
  size_t need_bytes = 0;
  RVQ_TRY(rvq_level_stats_workspace_size(n, L, K, d, with_msr ? 1 : 0, &need_bytes));
  RVQ_TRY(need(workspace, "workspace", 256));
  if (workspace_bytes < need_bytes)
    return fail(RVQ_ERR_WORKSPACE_TOO_SMALL, "level-stats workspace needs %zu bytes (got %zu)",
                need_bytes, workspace_bytes);
  char *ws = (char *)workspace;
  uint32_t *hpart = (uint32_t *)ws;
  double *mpart = (double *)(ws + align256(hist_partial_bytes(n, L, K)));
  HIP_TRY(launch_hist(ids, n, L, K, hist, hpart, bad_ids, stream), "histogram launch");
  if (with_msr)
    HIP_TRY(launch_msr(x, x_dtype == RVQ_BF16, ids, n, d, codebooks, L, K, msr, mpart, nullptr,
                       0, stream),
            "msr launch");
  return RVQ_OK;
}

rvq_status rvq_decode_level_stats(const int32_t *ids, int64_t n, const float *codebooks,
                                  int32_t L, int32_t K, int32_t d, void *out, rvq_dtype out_dtype,
                                  int64_t *hist, const void *x, rvq_dtype x_dtype, double *msr,
                                  uint32_t *bad_ids, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  RVQ_TRY(check_shape(n, d, L, K));
  if (L > kMaxLevelsGather)
    return fail(RVQ_ERR_UNSUPPORTED, "level statistics support L <= %d (got %d)",
                kMaxLevelsGather, L);
  if (out_dtype != RVQ_F32 && out_dtype != RVQ_BF16)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown out_dtype %d", (int)out_dtype);
  if (x_dtype != RVQ_F32 && x_dtype != RVQ_BF16)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown x_dtype %d", (int)x_dtype);
  RVQ_TRY(need(codebooks, "codebooks", 16));
  RVQ_TRY(need(hist, "hist", 8));
  RVQ_TRY(need(msr, "msr", 8));
  if (n > 0) {
    RVQ_TRY(need(ids, "ids", 4));
    RVQ_TRY(need(out, "out", 16));
    RVQ_TRY(need(x, "x", x_dtype == RVQ_BF16 ? 2 : 4));
  }
  if (bad_ids && !aligned(bad_ids, 4))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "bad_ids must be 4-byte aligned");
  size_t need_bytes = 0;
  RVQ_TRY(rvq_level_stats_workspace_size(n, L, K, d, 1, &need_bytes));
  RVQ_TRY(need(workspace, "workspace", 256));
  if (workspace_bytes < need_bytes)
    return fail(RVQ_ERR_WORKSPACE_TOO_SMALL, "level-stats workspace needs %zu bytes (got %zu)",
                need_bytes, workspace_bytes);
  char *ws = (char *)workspace;
  uint32_t *hpart = (uint32_t *)ws;
  double *mpart = (double *)(ws + align256(hist_partial_bytes(n, L, K)));
  HIP_TRY(launch_hist(ids, n, L, K, hist, hpart, bad_ids, stream), "histogram launch");
  HIP_TRY(launch_msr(x, x_dtype == RVQ_BF16, ids, n, d, codebooks, L, K, msr, mpart, out,
                     out_dtype == RVQ_BF16 ? 2 : 1, stream),
          "decode and msr launch");
  return RVQ_OK;
}

}  // extern "C"
