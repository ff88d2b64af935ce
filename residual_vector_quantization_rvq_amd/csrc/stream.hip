// stream.hip -- encode host-resident rows chunk by chunk, overlapping the
// copies with the encoder: the offline tokenisation pass.
//
// "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", paragraph "Offline
// Visual Preprocessing": the visual tokenizer is fixed, so the token IDs are
// computed ahead of training and cached.  The rows of such a pass live in
// host memory and are far larger than one encoder call needs, so they go
// through the device in chunks: while chunk c is encoded on the caller's
// stream, chunk c+1 is copied in on one copy stream and the IDs of chunk c-1
// are copied out on another; events order the three streams, and each
// buffer is double-buffered.  The encoder is batch-invariant, so the IDs
// are bit for bit those of one rvq_encode call over all rows.
//
// Host code only; the device work is rvq_encode's.
#include <cstring>

#include "rvq.h"

namespace rvq {
rvq_status fail(rvq_status st, const char *fmt, ...);
}
using namespace rvq;

namespace {

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

// workspace: row buffers x[2] (sized for 4-byte features), ID buffers id[2],
// then the encoder's workspace for chunk_rows rows
struct Layout {
  size_t x[2], id[2], enc, enc_bytes, total;
};

rvq_status layout(int64_t chunk_rows, int32_t d, int32_t L, int32_t K, Layout *o) {
  if (chunk_rows < 1)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "chunk_rows must be >= 1 (got %lld)",
                (long long)chunk_rows);
  size_t enc = 0;
  const rvq_status st = rvq_encode_workspace_size(chunk_rows, d, L, K, &enc);
  if (st != RVQ_OK) return st;
  const size_t xb = al256((size_t)chunk_rows * (size_t)d * 4);
  const size_t ib = al256((size_t)chunk_rows * (size_t)L * 4);
  o->x[0] = 0;
  o->x[1] = xb;
  o->id[0] = 2 * xb;
  o->id[1] = 2 * xb + ib;
  o->enc = 2 * xb + 2 * ib;
  o->enc_bytes = enc;
  o->total = o->enc + enc;
  return RVQ_OK;
}

// Streams and events of one call, synchronised and released on every exit
// path (the caller may free its buffers as soon as the call returns).
struct Pipeline {
  hipStream_t compute = nullptr, h2d = nullptr, d2h = nullptr;
  hipEvent_t start = nullptr, loaded[2] = {}, encoded[2] = {}, stored[2] = {};
  ~Pipeline() {
    if (h2d) hipStreamSynchronize(h2d);
    if (d2h) hipStreamSynchronize(d2h);
    if (compute || start) hipStreamSynchronize(compute);
    for (hipEvent_t e : {start, loaded[0], loaded[1], encoded[0], encoded[1], stored[0], stored[1]})
      if (e) hipEventDestroy(e);
    if (h2d) hipStreamDestroy(h2d);
    if (d2h) hipStreamDestroy(d2h);
  }
};

#define STREAM_HIP(call, what)                                                        \
  do {                                                                                \
    const hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) return fail(RVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)

struct CacheSink {
  const char *path;
  int64_t n, chunk_rows;
  int32_t L, K;
  rvq_status status;
};

int append_to_cache(void *user, int64_t chunk, int64_t /*row0*/, int64_t /*rows*/,
                    const int32_t *ids) {
  CacheSink *s = static_cast<CacheSink *>(user);
  s->status = rvq_idcache_append(s->path, s->n, s->L, s->K, s->chunk_rows, chunk, ids);
  return s->status != RVQ_OK;
}

}  // namespace

extern "C" {

rvq_status rvq_stream_workspace_size(int64_t chunk_rows, int32_t d, int32_t L, int32_t K,
                                     size_t *bytes) {
  if (!bytes) return fail(RVQ_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
  Layout lo;
  const rvq_status st = layout(chunk_rows, d, L, K, &lo);
  if (st != RVQ_OK) return st;
  *bytes = lo.total;
  return RVQ_OK;
}

rvq_status rvq_stream_encode(const void *x_host, rvq_dtype x_dtype, int64_t n, int32_t d,
                             const float *codebooks, const void *prepared, int32_t L, int32_t K,
                             int32_t *ids_host, int64_t chunk_rows, int64_t first_chunk,
                             int64_t max_chunks, rvq_chunk_callback on_chunk, void *user,
                             void *workspace, size_t workspace_bytes, hipStream_t stream,
                             int64_t *chunks_done) {
  if (!chunks_done) return fail(RVQ_ERR_INVALID_ARGUMENT, "chunks_done must not be NULL");
  if (n < 0) return fail(RVQ_ERR_INVALID_ARGUMENT, "n must be >= 0 (got %lld)", (long long)n);
  if (x_dtype != RVQ_F32 && x_dtype != RVQ_BF16)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "unknown x_dtype %d", (int)x_dtype);
  Layout lo;
  rvq_status st = layout(chunk_rows, d, L, K, &lo);
  if (st != RVQ_OK) return st;
  if (first_chunk < 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "first_chunk must be >= 0 (got %lld)",
                (long long)first_chunk);
  if (n > 0 && (!x_host || !ids_host))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "x_host and ids_host must not be NULL");
  if (!workspace || ((uintptr_t)workspace & 255))
    return fail(RVQ_ERR_INVALID_ARGUMENT, "workspace must be non-NULL and 256-byte aligned");
  if (workspace_bytes < lo.total)
    return fail(RVQ_ERR_WORKSPACE_TOO_SMALL, "stream workspace needs %zu bytes (got %zu)",
                lo.total, workspace_bytes);
  const int64_t nchunks = (n + chunk_rows - 1) / chunk_rows;
  int64_t last = nchunks;  // one past the last chunk to run
  if (max_chunks > 0 && first_chunk < nchunks && max_chunks < nchunks - first_chunk)
    last = first_chunk + max_chunks;
  *chunks_done = first_chunk < nchunks ? first_chunk : nchunks;
  if (first_chunk >= last) return RVQ_OK;

  const size_t esize = x_dtype == RVQ_BF16 ? 2 : 4;
  char *ws = static_cast<char *>(workspace);
  const char *xh = static_cast<const char *>(x_host);
  Pipeline p;
  p.compute = stream;
  STREAM_HIP(hipStreamCreateWithFlags(&p.h2d, hipStreamNonBlocking), "copy stream");
  STREAM_HIP(hipStreamCreateWithFlags(&p.d2h, hipStreamNonBlocking), "copy stream");
  STREAM_HIP(hipEventCreateWithFlags(&p.start, hipEventDisableTiming), "event");
  for (int b = 0; b < 2; ++b) {
    STREAM_HIP(hipEventCreateWithFlags(&p.loaded[b], hipEventDisableTiming), "event");
    STREAM_HIP(hipEventCreateWithFlags(&p.encoded[b], hipEventDisableTiming), "event");
    STREAM_HIP(hipEventCreateWithFlags(&p.stored[b], hipEventDisableTiming), "event");
  }
  // the copies follow whatever the caller queued before this call
  STREAM_HIP(hipEventRecord(p.start, stream), "event record");
  STREAM_HIP(hipStreamWaitEvent(p.h2d, p.start, 0), "stream wait");
  STREAM_HIP(hipStreamWaitEvent(p.d2h, p.start, 0), "stream wait");

  auto rows_of = [&](int64_t c) { return c + 1 < nchunks ? chunk_rows : n - c * chunk_rows; };
  // host side of chunk c: wait for its IDs, then report them
  auto finish = [&](int64_t c) -> int {
    const hipError_t e = hipEventSynchronize(p.stored[c & 1]);
    if (e != hipSuccess) {
      st = fail(RVQ_ERR_HIP, "IDs copy: %s", hipGetErrorString(e));
      return 1;
    }
    *chunks_done = c + 1;
    if (on_chunk && on_chunk(user, c, c * chunk_rows, rows_of(c), ids_host + c * chunk_rows * L))
      return 1;
    return 0;
  };

  for (int64_t c = first_chunk; c < last; ++c) {
    const int b = (int)(c & 1);
    const int64_t rows = rows_of(c), row0 = c * chunk_rows;
    const bool reuse = c - first_chunk >= 2;  // buffers b last held chunk c-2
    // copy in (after chunk c-2's encode has read the row buffer)
    if (reuse) STREAM_HIP(hipStreamWaitEvent(p.h2d, p.encoded[b], 0), "stream wait");
    STREAM_HIP(hipMemcpyAsync(ws + lo.x[b], xh + (size_t)row0 * d * esize,
                              (size_t)rows * d * esize, hipMemcpyHostToDevice, p.h2d),
               "rows copy");
    STREAM_HIP(hipEventRecord(p.loaded[b], p.h2d), "event record");
    // encode (after the rows are in and chunk c-2's IDs have left the ID buffer)
    STREAM_HIP(hipStreamWaitEvent(stream, p.loaded[b], 0), "stream wait");
    if (reuse) STREAM_HIP(hipStreamWaitEvent(stream, p.stored[b], 0), "stream wait");
    st = rvq_encode(ws + lo.x[b], x_dtype, rows, d, codebooks, prepared, L, K,
                    reinterpret_cast<int32_t *>(ws + lo.id[b]), nullptr, ws + lo.enc,
                    lo.enc_bytes, stream);
    if (st != RVQ_OK) return st;
    STREAM_HIP(hipEventRecord(p.encoded[b], stream), "event record");
    // copy the IDs out
    STREAM_HIP(hipStreamWaitEvent(p.d2h, p.encoded[b], 0), "stream wait");
    STREAM_HIP(hipMemcpyAsync(ids_host + row0 * L, ws + lo.id[b], (size_t)rows * L * 4,
                              hipMemcpyDeviceToHost, p.d2h),
               "IDs copy");
    STREAM_HIP(hipEventRecord(p.stored[b], p.d2h), "event record");
    // chunk c-1 is reported while chunk c runs
    if (c > first_chunk && finish(c - 1)) return st;
  }
  finish(last - 1);
  return st;
}

rvq_status rvq_stream_encode_to_cache(const char *path, const void *x_host, rvq_dtype x_dtype,
                                      int64_t n, int32_t d, const float *codebooks,
                                      const void *prepared, int32_t L, int32_t K,
                                      int32_t *ids_host, int64_t chunk_rows, int64_t max_chunks,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream,
                                      int64_t *chunks_done) {
  if (!chunks_done) return fail(RVQ_ERR_INVALID_ARGUMENT, "chunks_done must not be NULL");
  int64_t have = 0;
  rvq_status st = rvq_idcache_resume(path, n, L, K, chunk_rows, &have);
  if (st != RVQ_OK) return st;
  CacheSink sink{path, n, chunk_rows, L, K, RVQ_OK};
  st = rvq_stream_encode(x_host, x_dtype, n, d, codebooks, prepared, L, K, ids_host, chunk_rows,
                         have, max_chunks, append_to_cache, &sink, workspace, workspace_bytes,
                         stream, chunks_done);
  if (st == RVQ_OK && sink.status != RVQ_OK) {
    // the append that failed did not land
    *chunks_done = *chunks_done > 0 ? *chunks_done - 1 : 0;
    return sink.status;
  }
  return st;
}

}  // extern "C"
