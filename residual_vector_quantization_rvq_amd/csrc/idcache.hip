// idcache.hip -- resumable on-disk cache of token IDs, written chunk by chunk.
//
// "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", paragraph "Offline
// Visual Preprocessing": the visual tokenizer is fixed, so the visual token
// IDs are computed ahead of training and cached offline.  This file holds
// such a cache: IDs [n][L] of n rows, produced in chunks of chunk_rows rows,
// appended as each chunk completes, so an interrupted tokenisation resumes
// after its last complete chunk.
//
// Host code only (no device work).  Format, little-endian:
//   header (64 bytes): "RVQIDC01", n (i64), L (i32), K (i32), chunk_rows
//     (i64), CRC-32 of the 32 bytes before it (u32), zeros;
//   record c (chunks in order 0, 1, ...): c (i64), rows (i64), the chunk's
//     IDs rows x L (i32), CRC-32 of everything before it in the record (u32),
//     4 zero bytes.
// A record that is short or whose CRC does not match ends the valid prefix.
// CRC-32 is the IEEE 802.3 one (reflected polynomial 0xEDB88320, initial
// value and final XOR 0xFFFFFFFF).
#include <cerrno>
#include <cstdio>
#include <cstring>
#include <vector>

#include <unistd.h>

#include "rvq.h"

namespace rvq {

rvq_status fail(rvq_status st, const char *fmt, ...);

namespace {

constexpr char kMagic[8] = {'R', 'V', 'Q', 'I', 'D', 'C', '0', '1'};
constexpr int64_t kHeaderBytes = 64;

struct CrcTable {
  uint32_t t[256];
  constexpr CrcTable() : t() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t c = i;
      for (int k = 0; k < 8; ++k) c = (c & 1u) ? (0xEDB88320u ^ (c >> 1)) : (c >> 1);
      t[i] = c;
    }
  }
};
constexpr CrcTable kCrc{};

// running CRC-32: pass the previous return value (0 to start)
uint32_t crc32_update(uint32_t crc, const void *data, size_t bytes) {
  const uint8_t *p = static_cast<const uint8_t *>(data);
  uint32_t c = ~crc;
  for (size_t i = 0; i < bytes; ++i) c = kCrc.t[(c ^ p[i]) & 0xFFu] ^ (c >> 8);
  return ~c;
}

struct Geometry {
  int64_t n, chunk_rows, nchunks;
  int32_t L, K;
  int64_t rows_of(int64_t c) const {
    const int64_t r = n - c * chunk_rows;
    return r < chunk_rows ? r : chunk_rows;
  }
  int64_t record_bytes(int64_t rows) const { return 16 + rows * L * 4 + 8; }
  // byte offset of record c (all earlier chunks are full)
  int64_t offset_of(int64_t c) const { return kHeaderBytes + c * record_bytes(chunk_rows); }
};

rvq_status check_geometry(int64_t n, int32_t L, int32_t K, int64_t chunk_rows, Geometry *g) {
  if (n < 0 || L < 1 || K < 1 || chunk_rows < 1)
    return fail(RVQ_ERR_INVALID_ARGUMENT,
                "ID cache: need n >= 0, L >= 1, K >= 1, chunk_rows >= 1 (got %lld, %d, %d, %lld)",
                (long long)n, L, K, (long long)chunk_rows);
  if (chunk_rows > ((int64_t)1 << 40) / L)
    return fail(RVQ_ERR_UNSUPPORTED, "ID cache: chunk too large");
  g->n = n;
  g->L = L;
  g->K = K;
  g->chunk_rows = chunk_rows;
  g->nchunks = (n + chunk_rows - 1) / chunk_rows;
  return RVQ_OK;
}

void make_header(const Geometry &g, uint8_t (&h)[kHeaderBytes]) {
  std::memset(h, 0, sizeof(h));
  std::memcpy(h, kMagic, 8);
  std::memcpy(h + 8, &g.n, 8);
  std::memcpy(h + 16, &g.L, 4);
  std::memcpy(h + 20, &g.K, 4);
  std::memcpy(h + 24, &g.chunk_rows, 8);
  const uint32_t crc = crc32_update(0, h, 32);
  std::memcpy(h + 32, &crc, 4);
}

struct File {
  FILE *f = nullptr;
  ~File() {
    if (f) std::fclose(f);
  }
};

// Reads and checks record c at the current position; on success the IDs go
// to ids (when non-null) and true is returned.
bool read_record(FILE *f, const Geometry &g, int64_t c, int32_t *ids, std::vector<uint8_t> &buf) {
  const int64_t rows = g.rows_of(c);
  const size_t bytes = (size_t)g.record_bytes(rows);
  buf.resize(bytes);
  if (std::fread(buf.data(), 1, bytes, f) != bytes) return false;
  int64_t rc, rr;
  std::memcpy(&rc, buf.data(), 8);
  std::memcpy(&rr, buf.data() + 8, 8);
  if (rc != c || rr != rows) return false;
  const size_t body = 16 + (size_t)rows * g.L * 4;
  uint32_t crc;
  std::memcpy(&crc, buf.data() + body, 4);
  if (crc != crc32_update(0, buf.data(), body)) return false;
  if (ids) std::memcpy(ids, buf.data() + 16, (size_t)rows * g.L * 4);
  return true;
}

// Opens an existing cache, checks its header against g and counts the
// valid records; returns the byte length of the valid prefix in *valid_bytes.
rvq_status scan(const char *path, const Geometry &g, int32_t *ids, int64_t *chunks,
                int64_t *valid_bytes, bool *exists) {
  File fh;
  fh.f = std::fopen(path, "rb");
  *exists = fh.f != nullptr;
  *chunks = 0;
  *valid_bytes = 0;
  if (!fh.f) return RVQ_OK;
  uint8_t h[kHeaderBytes], want[kHeaderBytes];
  if (std::fread(h, 1, kHeaderBytes, fh.f) != (size_t)kHeaderBytes)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: short header", path);
  make_header(g, want);
  if (std::memcmp(h, kMagic, 8) != 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: not an ID cache", path);
  if (std::memcmp(h, want, kHeaderBytes) != 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT,
                "ID cache %s: header does not match n, L, K and chunk_rows of this call", path);
  std::vector<uint8_t> buf;
  int64_t c = 0;
  while (c < g.nchunks &&
         read_record(fh.f, g, c, ids ? ids + c * g.chunk_rows * g.L : nullptr, buf))
    ++c;
  *chunks = c;
  *valid_bytes = g.offset_of(c);
  return RVQ_OK;
}

}  // namespace

}  // namespace rvq

using namespace rvq;

extern "C" {

rvq_status rvq_idcache_resume(const char *path, int64_t n, int32_t L, int32_t K,
                              int64_t chunk_rows, int64_t *chunks_done) {
  if (!path || !chunks_done)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache: path and chunks_done must not be NULL");
  Geometry g;
  rvq_status st = check_geometry(n, L, K, chunk_rows, &g);
  if (st != RVQ_OK) return st;
  int64_t chunks, valid;
  bool exists;
  st = scan(path, g, nullptr, &chunks, &valid, &exists);
  if (st != RVQ_OK) return st;
  if (!exists) {
    File fh;
    fh.f = std::fopen(path, "wb");
    if (!fh.f) return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: %s", path, std::strerror(errno));
    uint8_t h[kHeaderBytes];
    make_header(g, h);
    if (std::fwrite(h, 1, kHeaderBytes, fh.f) != (size_t)kHeaderBytes || std::fflush(fh.f) != 0)
      return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: write failed", path);
    *chunks_done = 0;
    return RVQ_OK;
  }
  // drop a torn or corrupt tail so that appends continue the valid prefix
  if (truncate(path, (off_t)valid) != 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: truncate failed: %s", path,
                std::strerror(errno));
  *chunks_done = chunks;
  return RVQ_OK;
}

rvq_status rvq_idcache_append(const char *path, int64_t n, int32_t L, int32_t K,
                              int64_t chunk_rows, int64_t chunk, const int32_t *ids) {
  if (!path || !ids) return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache: path and ids must not be NULL");
  Geometry g;
  rvq_status st = check_geometry(n, L, K, chunk_rows, &g);
  if (st != RVQ_OK) return st;
  if (chunk < 0 || chunk >= g.nchunks)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache: chunk %lld outside [0, %lld)",
                (long long)chunk, (long long)g.nchunks);
  File fh;
  fh.f = std::fopen(path, "r+b");
  if (!fh.f) return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: %s", path, std::strerror(errno));
  uint8_t h[kHeaderBytes], want[kHeaderBytes];
  make_header(g, want);
  if (std::fread(h, 1, kHeaderBytes, fh.f) != (size_t)kHeaderBytes ||
      std::memcmp(h, want, kHeaderBytes) != 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: header does not match", path);
  if (std::fseek(fh.f, 0, SEEK_END) != 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: seek failed", path);
  const long end = std::ftell(fh.f);
  if (end != (long)g.offset_of(chunk))
    return fail(RVQ_ERR_INVALID_ARGUMENT,
                "ID cache %s: chunk %lld appended out of order (the file holds %ld bytes)", path,
                (long long)chunk, end);
  const int64_t rows = g.rows_of(chunk);
  const size_t body = 16 + (size_t)rows * L * 4;
  std::vector<uint8_t> rec((size_t)g.record_bytes(rows), 0);
  std::memcpy(rec.data(), &chunk, 8);
  std::memcpy(rec.data() + 8, &rows, 8);
  std::memcpy(rec.data() + 16, ids, (size_t)rows * L * 4);
  const uint32_t crc = crc32_update(0, rec.data(), body);
  std::memcpy(rec.data() + body, &crc, 4);
  if (std::fwrite(rec.data(), 1, rec.size(), fh.f) != rec.size() || std::fflush(fh.f) != 0)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: write failed", path);
  return RVQ_OK;
}

rvq_status rvq_idcache_read(const char *path, int64_t n, int32_t L, int32_t K, int64_t chunk_rows,
                            int32_t *ids, int64_t *chunks_done) {
  if (!path || !chunks_done)
    return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache: path and chunks_done must not be NULL");
  if (n > 0 && !ids) return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache: ids must not be NULL");
  Geometry g;
  rvq_status st = check_geometry(n, L, K, chunk_rows, &g);
  if (st != RVQ_OK) return st;
  int64_t chunks, valid;
  bool exists;
  st = scan(path, g, ids, &chunks, &valid, &exists);
  if (st != RVQ_OK) return st;
  if (!exists) return fail(RVQ_ERR_INVALID_ARGUMENT, "ID cache %s: no such file", path);
  *chunks_done = chunks;
  return RVQ_OK;
}

}  // extern "C"
