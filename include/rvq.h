/*
 * rvq.h -- C ABI of the MI355X (gfx950) residual vector quantization library.
 *
 * What the library computes.  Visual feature vectors become multi-level
 * discrete token IDs by residual vector quantization (RVQ): at each level
 * the nearest codeword of that level's codebook is chosen, its index is
 * recorded, and it is subtracted so the residual passes on to the next
 * level ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型", section
 * "Visual Primitive Modeling", paragraph "Discrete Native Resolution Vision
 * Transformer"; "LongCat-2.5 Open Source Release: Meituan's 1.6T Multimodal
 * Agent Model with 1M Context", section "02 Visual Coding and 3D": detail is
 * added level by level).  Token IDs are turned
 * back into vectors by summing the chosen codewords (same blog, Figure 1:
 * the token sequences are reconstructed).  The tokenizer is fixed and its
 * IDs are precomputed offline (same blog, paragraph "Offline Visual
 * Preprocessing"), so encoding here is a deterministic, batch-invariant
 * function of (row, codebooks): a row's IDs do not depend on the other rows
 * in the call or on its position.
 *
 * Readings taken where the pages are silent: the distance is the squared
 * Euclidean distance; there is one [K][d] codebook per level; search is
 * greedy level by level; among codewords at the same distance the lower
 * index wins.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers are device memory owned by the
 *     caller (any allocator).  The library allocates no device memory and
 *     keeps no global mutable state; scratch memory is a caller-provided
 *     workspace.  (The host-side ID cache uses short-lived host buffers, and
 *     the streaming encoder creates and destroys its own copy streams and
 *     events within the call.)
 *   - All arrays are dense and row-major.  Codebooks are [L][K][d] fp32;
 *     token IDs are [n][L] int32 (level-minor); rows are [n][d].
 *   - Work is enqueued on `stream` and the call returns without waiting.
 *     Concurrent calls on different streams must use different workspaces.
 *   - The device entry points issue only kernel launches on `stream` (no
 *     memset, copy, allocation or host synchronisation), so a caller may
 *     capture them in a HIP graph; the streaming encoder is the exception.
 *   - Arguments are validated on the host before any HIP call; a non-OK
 *     status means nothing was enqueued, except RVQ_ERR_HIP, which reports
 *     a failed launch (the stream may then hold part of the work).
 *   - n == 0 is a valid no-op (outputs of size zero; hist and msr are still
 *     written for level statistics).
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified
 *     but every memory access stays in bounds.
 */
#ifndef RVQ_H
#define RVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rvq_status {
    RVQ_OK = 0,
    RVQ_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misaligned pointer */
    RVQ_ERR_UNSUPPORTED = 2,        /* valid request outside what the library supports */
    RVQ_ERR_WORKSPACE_TOO_SMALL = 3,
    RVQ_ERR_HIP = 4                 /* a HIP launch failed */
} rvq_status;

typedef enum rvq_dtype {
    RVQ_F32 = 0,
    RVQ_BF16 = 1
} rvq_dtype;

/* Static text for a status code. */
const char *rvq_status_string(rvq_status s);

/* Detail of the last non-OK status returned on the calling host thread
 * (thread-local, overwritten by the next failing call). */
const char *rvq_last_error(void);

/* ------------------------------------------------------------------------
 * Codebook preparation (once per fixed codebook set).
 *
 * The tokenizer is fixed ("Offline Visual Preprocessing"), so per-codeword
 * data derived from the codebooks is computed once and reused by every
 * encode call: the squared norms ||c||^2 in fp32 and a bf16 copy of the
 * codewords in the layout the distance kernel reads.
 * ---------------------------------------------------------------------- */

/* Bytes of the prepared buffer for L levels of K codewords of dimension d. */
rvq_status rvq_prepared_size(int32_t L, int32_t K, int32_t d, size_t *bytes);

/*
 * codebooks : device, [L][K][d] fp32, 16-byte aligned.
 * prepared  : device, >= rvq_prepared_size bytes, 256-byte aligned.  For
 *             d <= 1280 fully overwritten; for wider rows only an fp32 copy
 *             of the codebooks with rows padded to a multiple of 16 is
 *             written (when d is not one), the only part the exact fp32
 *             encoder reads.  Owned by the caller; pass it to rvq_encode with
 *             the same codebooks, L, K and d (not checked: a buffer prepared
 *             from other codebooks gives wrong IDs, never a fault).
 */
rvq_status rvq_prepare_codebooks(const float *codebooks, int32_t L, int32_t K, int32_t d,
                                 void *prepared, size_t prepared_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Encode: greedy multi-level nearest-codeword search with residual update.
 *
 * Per level l and row r the nearest codeword under ||r - c||^2 is chosen,
 * its index recorded, and it is subtracted from the fp32 residual, which
 * feeds the next level.
 *
 * Rows of at most 1280 features: the codewords are ranked by the score
 * ||c||^2 - 2 r.c (||r||^2 is the same for every codeword), with the dot
 * products taken on the matrix cores from bf16 copies of r and c with fp32
 * accumulation.  Per row and level the encoder bounds how far this
 * screening can move a score (from the row's and the level's rounding
 * terms: the residual's and the codewords' bf16 rounding, the fp32
 * accumulation, the hi/lo split of ||c||^2 and the tag bits of the ranking
 * keys), and every codeword whose key lies within the resulting band of the
 * smallest key is rescored exactly in fp32 as sum_i (r_i - c_i)^2; the
 * smallest distance wins.  A level whose candidates cannot all be kept
 * (a crowded band) is rescanned exactly over all K codewords after the
 * distance launch.  So the nearest codeword is returned wherever it beats
 * every other by more than 1e-4 ||r||^2.  (The bound treats the rounding
 * errors of different features as independent, a reading of the typical
 * case; its Cauchy-Schwarz worst case is used where it is smaller, at
 * widths below about 25.)
 *
 * Rows of 1281 to 8192 features: every distance sum_i (r_i - c_i)^2 is
 * computed exactly in fp32 on the vector ALUs, with no screening (slower).
 *
 * On both paths, among codewords at the same fp32 distance the lower index
 * wins (duplicated codewords return the lowest index), and a row's IDs and
 * fp32 residual depend only on the row and the codebooks, not on the other
 * rows of the call or on its position.
 * ---------------------------------------------------------------------- */

/* Workspace bytes needed by rvq_encode for n rows. */
rvq_status rvq_encode_workspace_size(int64_t n, int32_t d, int32_t L, int32_t K, size_t *bytes);

/*
 * x            : device, [n][d] rows in x_dtype (fp32 or bf16), aligned to
 *                the element size; rows that do not start 16-byte aligned
 *                (e.g. a slice of a larger batch) are first copied to the
 *                workspace.
 * codebooks    : device, [L][K][d] fp32 (the exact values used for rescoring
 *                and for the residual update), 16-byte aligned.
 * prepared     : device, filled by rvq_prepare_codebooks for these codebooks.
 * ids          : device, [n][L] int32 output; ids[row*L + l] in [0, K).
 * residual_out : device, [n][d] fp32 output x - sum_l codebooks[l][ids[l]],
 *                or NULL when not wanted.  4-byte aligned (16-byte alignment
 *                can save a final copy).
 * d            : 1..8192 (RVQ_ERR_UNSUPPORTED above).  Up to 1280 a row's
 *                features stay resident in registers during the matrix-core
 *                sweep; wider rows take the exact fp32 path.  One level of
 *                codewords, K x (d rounded up to 16) fp32, must be below
 *                4 GiB (RVQ_ERR_UNSUPPORTED otherwise; the same checks apply
 *                to rvq_prepared_size, rvq_prepare_codebooks and
 *                rvq_encode_workspace_size).
 * workspace    : device, >= rvq_encode_workspace_size bytes, 256-byte
 *                aligned; contents on entry are ignored.
 */
rvq_status rvq_encode(const void *x, rvq_dtype x_dtype, int64_t n, int32_t d,
                      const float *codebooks, const void *prepared, int32_t L, int32_t K,
                      int32_t *ids, float *residual_out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Same as rvq_encode, and additionally times the distance stage with
 * caller-created events (hipEventCreate).  The encoder runs either one
 * launch for all levels (enough rows to fill the GPU: the launch includes
 * each level's rescoring and residual update) or one distance launch per
 * level (few rows, or rows wider than 1280 features).  events[2*i] is recorded on `stream` immediately before
 * and events[2*i + 1] immediately after distance launch i; `events` must
 * hold 2*L events, or be NULL to record nothing.  *launches (may be NULL)
 * receives the number of launches recorded (1 or L; 0 when n == 0).
 */
rvq_status rvq_encode_profiled(const void *x, rvq_dtype x_dtype, int64_t n, int32_t d,
                               const float *codebooks, const void *prepared, int32_t L, int32_t K,
                               int32_t *ids, float *residual_out,
                               void *workspace, size_t workspace_bytes, hipStream_t stream,
                               hipEvent_t *events, int32_t *launches);

/* ------------------------------------------------------------------------
 * Decode: out[row] = sum_{l < levels} codebooks[l][ids[row*L + l]], summed in
 * fp32 in level order, then stored as fp32 or rounded to nearest-even bf16.
 * `levels` in [0, L] reconstructs from the first `levels` levels only
 * (coarse-to-fine; levels == L is the full reconstruction).
 *
 * ids       : device, [n][L] int32.  An ID outside [0, K) contributes
 *             nothing and is counted in *bad_ids.
 * codebooks : device, [L][K][d] fp32, 16-byte aligned.
 * out       : device, [n][d] in out_dtype, 16-byte aligned.
 * bad_ids   : device uint32 counter incremented by the number of out-of-range
 *             IDs seen, or NULL.  The caller zeroes it.
 * ---------------------------------------------------------------------- */
rvq_status rvq_decode(const int32_t *ids, int64_t n, const float *codebooks,
                      int32_t L, int32_t K, int32_t d, int32_t levels,
                      void *out, rvq_dtype out_dtype, uint32_t *bad_ids, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Level statistics.
 *   hist[l][k] = number of rows whose level-l ID is k (exact integer count;
 *                out-of-range IDs are not counted and go to *bad_ids).
 *   msr[l]     = mean over rows of ||x_row - sum_{j <= l} codebooks[j][ids[row][j]]||^2,
 *                the mean squared residual left after levels 0..l (an
 *                out-of-range ID subtracts nothing).  Per-row residuals are
 *                fp32, squared norms and the mean are fp64, reduced in an
 *                order that depends only on n (bitwise reproducible).
 * Each out-of-range ID is counted once in *bad_ids per call.
 * ---------------------------------------------------------------------- */

/* Workspace bytes needed by rvq_level_stats (with_msr != 0 when msr is requested). */
rvq_status rvq_level_stats_workspace_size(int64_t n, int32_t L, int32_t K, int32_t d,
                                          int32_t with_msr, size_t *bytes);

/*
 * ids       : device, [n][L] int32.
 * hist      : device, [L][K] int64 output, fully overwritten.  Required.
 * msr       : device, [L] fp64 output, or NULL to compute the counts only.
 *             With n == 0 it is all zeros.
 * x         : device, [n][d] rows (x_dtype), aligned to the element size;
 *             required when msr is non-NULL and n > 0, ignored otherwise.
 *             Rows that do not start 16-byte (fp32) or 8-byte (bf16)
 *             aligned, or d not a multiple of 4, take a per-element path:
 *             the counts are the same and msr may differ in the last bits
 *             of its fp64 sum.
 * codebooks : device, [L][K][d] fp32; required when msr is non-NULL.
 * bad_ids   : as for rvq_decode.
 * workspace : device, >= rvq_level_stats_workspace_size bytes, 256-byte aligned.
 */
rvq_status rvq_level_stats(const int32_t *ids, int64_t n, int32_t L, int32_t K, int64_t *hist,
                           const void *x, rvq_dtype x_dtype, int32_t d, const float *codebooks,
                           double *msr, uint32_t *bad_ids,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode and level statistics of the same IDs in one pass.
 *
 * Produces exactly (bit for bit) what rvq_decode with levels == L followed by
 * rvq_level_stats with msr would: out[row] = sum of the row's codewords in
 * level order (fp32, out-of-range IDs skipped, stored as out_dtype), hist and
 * msr as defined above.  The msr pass already gathers every level's codeword
 * of every row, so the decode costs only its output writes.  Each
 * out-of-range ID is counted once in *bad_ids.
 *
 * Arguments are those of rvq_decode and rvq_level_stats; x, msr and out are
 * required (n > 0), and the workspace is sized by
 * rvq_level_stats_workspace_size(n, L, K, d, 1).
 * ---------------------------------------------------------------------- */
rvq_status rvq_decode_level_stats(const int32_t *ids, int64_t n, const float *codebooks,
                                  int32_t L, int32_t K, int32_t d, void *out, rvq_dtype out_dtype,
                                  int64_t *hist, const void *x, rvq_dtype x_dtype, double *msr,
                                  uint32_t *bad_ids, void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/* ------------------------------------------------------------------------
 * Unified token embedding of a mixed text / visual sequence.
 *
 * Visual signals are multi-level discrete tokens that the backbone takes in
 * the same token format as text, and the visual codebook embeddings are
 * learned jointly with the backbone ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
 * section "Visual Primitive Modeling", paragraph "Native
 * Visual Representation").  Token t of a sequence of T tokens becomes one
 * row of D values:
 *   visual token: out[t] = sum over l of level_tables[l][ids[t][l]], added
 *                 in fp32 in level order (bit for bit rvq_decode's sum when
 *                 the tables are fp32); an out-of-range ID adds nothing;
 *   text token:   out[t] = text_table[ids[t][0]] (ids[t][1..L-1] are not
 *                 read); an out-of-range ID gives a row of zeros.
 * bf16 outputs are the fp32 values rounded to nearest even.  Each
 * out-of-range ID that is read is counted once in *bad_ids.
 *
 * ids          : device, [T][L] int32.
 * is_visual    : device, [T] uint8, nonzero for a visual token; NULL means
 *                every token is visual.
 * text_table   : device, [V][D] in table_dtype, 16-byte aligned; may be NULL
 *                when V == 0 (every text ID is then out of range).
 * level_tables : device, [L][K][D] in table_dtype, 16-byte aligned.
 * table_dtype  : RVQ_F32 or RVQ_BF16 (both tables).
 * out          : device, [T][D] in out_dtype (RVQ_F32 or RVQ_BF16), 16-byte
 *                aligned, fully overwritten.
 * bad_ids      : device uint32 counter (added to), or NULL.
 * Limits: 1 <= L <= 64 (RVQ_ERR_UNSUPPORTED above), K >= 1, D >= 1, V >= 0.
 * ---------------------------------------------------------------------- */
rvq_status rvq_embed_tokens(const int32_t *ids, const uint8_t *is_visual, int64_t T, int32_t L,
                            const void *text_table, int64_t V, const void *level_tables,
                            int32_t K, int32_t D, rvq_dtype table_dtype, void *out,
                            rvq_dtype out_dtype, uint32_t *bad_ids, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Resumable ID cache (host files).
 *
 * The visual tokenizer is fixed, so token IDs are computed ahead of time
 * and cached offline ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
 * paragraph "Offline Visual Preprocessing").  An ID cache file holds the
 * IDs [n][L] of n rows in chunks of chunk_rows rows (the last chunk may be
 * shorter), appended in chunk order, each with a CRC-32, so that an
 * interrupted writer resumes after its last complete chunk.  Host code
 * only: these calls make no HIP call and touch no device memory; each
 * opens and closes the file.  Errors (bad arguments, I/O failure, a header
 * that does not match) return RVQ_ERR_INVALID_ARGUMENT.
 * ---------------------------------------------------------------------- */

/* Creates the file (header only) when it does not exist.  Otherwise checks
 * that its header matches (n, L, K, chunk_rows), cuts off a torn or corrupt
 * tail, and reports in *chunks_done how many leading chunks it holds. */
rvq_status rvq_idcache_resume(const char *path, int64_t n, int32_t L, int32_t K,
                              int64_t chunk_rows, int64_t *chunks_done);

/* Appends chunk `chunk`: its rows x L IDs from host memory.  The file must
 * hold exactly chunks 0 .. chunk-1. */
rvq_status rvq_idcache_append(const char *path, int64_t n, int32_t L, int32_t K,
                              int64_t chunk_rows, int64_t chunk, const int32_t *ids);

/* Reads the valid leading chunks into ids (host, [n][L]; the rows of
 * missing chunks are left as they are) and reports their count. */
rvq_status rvq_idcache_read(const char *path, int64_t n, int32_t L, int32_t K,
                            int64_t chunk_rows, int32_t *ids, int64_t *chunks_done);

/* ------------------------------------------------------------------------
 * Streaming encode of host-resident rows (the offline tokenisation pass).
 *
 * Token IDs are computed ahead of training and cached ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
 * paragraph "Offline Visual Preprocessing").  rvq_stream_encode encodes rows [0, n) of a host array
 * in chunks of chunk_rows rows: while chunk c is encoded on `stream`, chunk
 * c+1 is copied in and the IDs of chunk c-1 are copied out, each on a copy
 * stream of its own that the call creates (default priority) and destroys,
 * ordered by events.  The IDs are bit for bit those of one rvq_encode call
 * over all n rows (the encoder is batch-invariant).  The call is
 * synchronous: it returns when its chunks are done and every stream it used
 * is idle.
 * ---------------------------------------------------------------------- */

/* Called on the calling thread once chunk `chunk` (rows row0 .. row0+rows-1)
 * has its IDs in host memory at `ids` ([rows][L]).  A nonzero return stops
 * the call after this chunk (which counts as done). */
typedef int (*rvq_chunk_callback)(void *user, int64_t chunk, int64_t row0, int64_t rows,
                                  const int32_t *ids);

/* Device workspace bytes for rvq_stream_encode with chunks of chunk_rows rows:
 * two row buffers, two ID buffers and rvq_encode's workspace. */
rvq_status rvq_stream_workspace_size(int64_t chunk_rows, int32_t d, int32_t L, int32_t K,
                                     size_t *bytes);

/*
 * x_host      : host, [n][d] rows (x_dtype).  Pinned memory (hipHostMalloc)
 *               lets the copies overlap the encoder; pageable memory works,
 *               with copies that may not overlap.
 * codebooks, prepared, L, K : as for rvq_encode (device).
 * ids_host    : host, [n][L] int32 output; chunks not run are left as they are.
 * chunk_rows  : rows per chunk (>= 1); chunk c holds rows c*chunk_rows ...
 * first_chunk : the first chunk to run (earlier ones are skipped: resume).
 * max_chunks  : run at most this many chunks (<= 0: all that remain).
 * on_chunk    : callback per finished chunk, or NULL; user is passed to it.
 * workspace   : device, >= rvq_stream_workspace_size bytes, 256-byte aligned.
 * stream      : the stream the encoder runs on; work the caller queued on it
 *               before the call is done before the first copy.
 * chunks_done : out: chunks 0 .. *chunks_done - 1 are done (those before
 *               first_chunk included), also when an error is returned.
 */
rvq_status rvq_stream_encode(const void *x_host, rvq_dtype x_dtype, int64_t n, int32_t d,
                             const float *codebooks, const void *prepared, int32_t L, int32_t K,
                             int32_t *ids_host, int64_t chunk_rows, int64_t first_chunk,
                             int64_t max_chunks, rvq_chunk_callback on_chunk, void *user,
                             void *workspace, size_t workspace_bytes, hipStream_t stream,
                             int64_t *chunks_done);

/* rvq_stream_encode into a resumable ID cache file: rvq_idcache_resume on
 * `path`, then the chunks the file does not hold yet (at most max_chunks of
 * them), each appended to the file as it finishes.  Rerun after an
 * interruption to continue.  *chunks_done: the chunks the file holds. */
rvq_status rvq_stream_encode_to_cache(const char *path, const void *x_host, rvq_dtype x_dtype,
                                      int64_t n, int32_t d, const float *codebooks,
                                      const void *prepared, int32_t L, int32_t K,
                                      int32_t *ids_host, int64_t chunk_rows, int64_t max_chunks,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream,
                                      int64_t *chunks_done);

/* ------------------------------------------------------------------------
 * rvq_encode with no workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The workspace is the library's own
 * file-scope device array of 256 MiB (268,435,456 bytes; one on every
 * device the library runs on, held until the process ends): enough for one
 * image of up to 84 x 84 patches (7,056 rows) at d = 1152, L = 8,
 * K = 8192.  Arguments, layouts, results and errors are rvq_encode's; a call
 * whose workspace (rvq_encode_workspace_size) exceeds the array returns
 * RVQ_ERR_UNSUPPORTED before any HIP call.  No hipMalloc or hipFree.  The
 * device address of the array is looked up on a device's first call (with
 * that device current).  Every call on one device shares the array: calls
 * that overlap on one GPU (several streams or threads) race, and must not
 * be made.
 * ---------------------------------------------------------------------- */
rvq_status rvq_encode_noalloc(const void *x, rvq_dtype x_dtype, int64_t n, int32_t d,
                              const float *codebooks, const void *prepared, int32_t L, int32_t K,
                              int32_t *ids, float *residual_out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Token-count-aware packing across data-parallel ranks (host code).
 *
 * With the visual tokenizer out of the training graph, every sample's
 * image-token count is known when batches are packed, so the share of
 * visual tokens on each data-parallel rank can be kept close to the
 * batch's ("LongCat-2.5 Released", section 4 "Infrastructure: Under 80 GB
 * Per Card", "Supernode-aware parallelism", last paragraph; "LongCat-2.5
 * 发布：面向智能体任务的原生多模态大模型", "Supernode-Aware Parallelism",
 * last paragraph).  The pages state the goal only; the objective is this
 * library's reading of it.  Sample i has t_i text and v_i image tokens,
 * n_i = t_i + v_i; the batch has N = sum n_i tokens, V = sum v_i of them
 * visual, p = V / N.  Rank r receives N_r tokens, V_r of them visual, and
 * at most `capacity` tokens.  The planner minimises
 *     max_r |V_r - p N_r|      (the rank's tokens beyond the batch's
 *                               modality proportion),
 * then max_r N_r, computing the excesses exactly in integers
 * (N (V_r - p N_r) = sum over the rank of v_i N - V n_i).
 *
 * text_tokens, image_tokens: host arrays [samples], each >= 0, at most
 * 2^30 tokens in all.  ranks >= 1.  Inputs of at most exact_max samples
 * are solved exactly (exhaustive search with a bound; keep exact_max small,
 * about 12: the search is exponential); larger ones by a greedy
 * assignment (samples by decreasing modality excess, each to the rank
 * that keeps its excess smallest) followed by moves and swaps that lower
 * the largest excess.  rank_of (host, [samples]) receives each sample's
 * rank.  summary (host, [3], or NULL): max_r |sum of v_i N - V n_i| (the
 * objective times N), N, and max_r N_r.  Returns RVQ_ERR_INVALID_ARGUMENT
 * for bad arguments and RVQ_ERR_UNSUPPORTED when a sample exceeds the
 * capacity, the samples do not fit, or the counts are too large.  No HIP
 * call; thread-safe.
 * ---------------------------------------------------------------------- */
rvq_status rvq_pack_ranks(const int64_t *text_tokens, const int64_t *image_tokens,
                          int64_t samples, int32_t ranks, int64_t capacity, int32_t exact_max,
                          int32_t *rank_of, int64_t *summary);

/* ------------------------------------------------------------------------
 * Measurement aid: the matrix cores' achievable bf16 rate.
 *
 * Not a step of the path.  The published dense bf16 peak assumes the
 * nominal clock; under a full matrix load the chip holds a clock that
 * depends on how much the operands switch.  rvq_mfma_rate runs a
 * register-only loop of v_mfma_f32_32x32x16_bf16 (the instruction of the
 * encoder's distance stage) on `blocks` workgroups of four waves (use one
 * per compute unit: one wave per SIMD), four independent accumulator chains
 * per wave, `iters` iterations of eight instructions, no memory traffic in
 * the loop.  zero_operands != 0 uses all-zero operands, otherwise random
 * bf16 values (random sign, magnitude in [0.25, 4), random mantissa).
 * A short untimed run precedes the timed one.
 *
 * workspace: device memory of at least rvq_mfma_rate_workspace_size(blocks)
 * bytes, 8-byte aligned (per-workgroup clock readings and a result sink).
 * tflops (host) receives the timed launch's rate from HIP events; clock_ghz
 * (host) the shader clock over the loop (s_memtime ticks over
 * s_memrealtime's 100 MHz, averaged over workgroups).  Unlike the other
 * device entry points this call waits for its work and copies the clock
 * readings to the host.  Returns RVQ_ERR_INVALID_ARGUMENT for blocks
 * outside 1 .. 65536, iters outside 10 .. 10^7 or a null or misaligned
 * pointer, RVQ_ERR_WORKSPACE_TOO_SMALL, or RVQ_ERR_HIP.
 * ---------------------------------------------------------------------- */
size_t rvq_mfma_rate_workspace_size(int32_t blocks);
rvq_status rvq_mfma_rate(int32_t blocks, int32_t iters, int32_t zero_operands, void *workspace,
                         size_t workspace_bytes, hipStream_t stream, double *tflops,
                         double *clock_ghz);

#ifdef __cplusplus
}
#endif

#endif /* RVQ_H */
