/*
 * rvq_oracle.c -- plain fp64 CPU oracle for residual vector quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  The product (the HIP library) never links,
 * loads or calls this file; only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no code with the GPU
 * path.
 *
 * What is computed (the method as the pages describe it, written out as
 * its plain definition):
 *   - "LongCat-2.5 发布：面向智能体任务的原生多模态大模型", section
 *     "Visual Primitive Modeling", paragraph "Discrete Native Resolution
 *     Vision Transformer": visual features become multi-level discrete
 *     tokens by residual vector quantization (RVQ).
 *   - "LongCat-2.5 Open Source Release: Meituan's 1.6T Multimodal Agent
 *     Model with 1M Context", section "02 Visual Coding and 3D": the
 *     quantizer adds detail level by level.  Read as greedy RVQ:
 *     at level l pick the codeword of codebook l nearest to the current
 *     residual, record its index, subtract it, pass the residual on.
 *   - Same blog, Figure 1: token sequences are reconstructed; the plainest
 *     reconstruction is the sum of the chosen codewords.
 *   - Same blog, paragraph "Offline Visual Preprocessing": the tokenizer
 *     is fixed, so encoding is a deterministic function of its inputs.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   distance = squared Euclidean distance; one [K, D] codebook per level;
 *   ties go to the lowest codeword index; the "gap" of a decision is the
 *   second-smallest distance over k != chosen minus the smallest.
 *
 * Arithmetic: every value is fp64; every sum over the feature dimension is
 * a sequential loop i = 0..d-1; no blocking, no reordering, no fast-math.
 * Rows are independent, so OpenMP splits the row loop only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

static int bad_shape(int64_t n, int32_t d, int32_t L, int32_t K)
{
    return n < 0 || d < 1 || L < 1 || K < 1;
}

/* Squared Euclidean distance, sequential sum over i. */
static double sqdist(const double *a, const double *b, int32_t d)
{
    double s = 0.0;
    for (int32_t i = 0; i < d; ++i) {
        double t = a[i] - b[i];
        s += t * t;
    }
    return s;
}

static double sqnorm(const double *a, int32_t d)
{
    double s = 0.0;
    for (int32_t i = 0; i < d; ++i) s += a[i] * a[i];
    return s;
}

/* Index of the smallest value; the first one on exact ties. */
static int32_t first_argmin(const double *v, int32_t K)
{
    int32_t best = 0;
    for (int32_t k = 1; k < K; ++k)
        if (v[k] < v[best]) best = k;
    return best;
}

/*
 * Greedy RVQ encode.
 *   x   [n][d]    input rows (fp64)
 *   cb  [L][K][d] one codebook per level
 * Outputs (any may be NULL except ids):
 *   ids [n][L]  chosen codeword per level
 *   gap [n][L]  min_{k != id} dist_k - dist_id  (+inf when K == 1)
 *   rn2 [n][L]  squared norm of the residual entering level l
 *   ms  [n][L]  squared norm of the residual after level l
 *   res [n][d]  final residual x - sum_l cb[l][ids[l]]
 */
int rvq_oracle_encode(const double *x, int64_t n, int32_t d,
                      const double *cb, int32_t L, int32_t K,
                      int32_t *ids, double *gap, double *rn2, double *ms,
                      double *res, int32_t threads)
{
    if (bad_shape(n, d, L, K) || (n > 0 && (!x || !cb || !ids))) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
    {
        double *r = (double *)malloc(sizeof(double) * (size_t)d);
        double *dist = (double *)malloc(sizeof(double) * (size_t)K);
        if (!r || !dist) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        }
#pragma omp barrier
        if (err == ORACLE_OK) {
#pragma omp for schedule(dynamic, 1)
            for (int64_t row = 0; row < n; ++row) {
                memcpy(r, x + row * d, sizeof(double) * (size_t)d);
                for (int32_t l = 0; l < L; ++l) {
                    const double *C = cb + (int64_t)l * K * d;
                    if (rn2) rn2[row * L + l] = sqnorm(r, d);
                    for (int32_t k = 0; k < K; ++k) dist[k] = sqdist(r, C + (int64_t)k * d, d);
                    int32_t id = first_argmin(dist, K);
                    if (gap) {
                        double second = INFINITY;
                        for (int32_t k = 0; k < K; ++k)
                            if (k != id && dist[k] < second) second = dist[k];
                        gap[row * L + l] = second - dist[id];
                    }
                    ids[row * L + l] = id;
                    const double *c = C + (int64_t)id * d;
                    for (int32_t i = 0; i < d; ++i) r[i] = r[i] - c[i];
                    if (ms) ms[row * L + l] = sqnorm(r, d);
                }
                if (res) memcpy(res + row * d, r, sizeof(double) * (size_t)d);
            }
        }
        free(r);
        free(dist);
    }
    return err;
}

/*
 * Decode: out[n][d] = sum_{l < levels} cb[l][ids[n][l]], summed in level
 * order in fp64.  levels <= L lets a caller reconstruct from a prefix of
 * the levels (coarse-to-fine).  Returns ORACLE_ERR_ARG on an ID outside
 * [0, K).
 */
int rvq_oracle_decode(const int32_t *ids, int64_t n, const double *cb,
                      int32_t L, int32_t K, int32_t d, int32_t levels,
                      double *out, int32_t threads)
{
    if (bad_shape(n, d, L, K) || levels < 0 || levels > L) return ORACLE_ERR_ARG;
    if (n > 0 && (!ids || !cb || !out)) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n * L; ++i)
        if (ids[i] < 0 || ids[i] >= K) return ORACLE_ERR_ARG;
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t row = 0; row < n; ++row) {
        double *o = out + row * d;
        for (int32_t i = 0; i < d; ++i) o[i] = 0.0;
        for (int32_t l = 0; l < levels; ++l) {
            const double *c = cb + ((int64_t)l * K + ids[row * L + l]) * d;
            for (int32_t i = 0; i < d; ++i) o[i] = o[i] + c[i];
        }
    }
    return ORACLE_OK;
}

/*
 * Unified token embedding of a mixed sequence ("LongCat-2.5 发布：面向智能体任务的原生多模态大模型",
 * section "Visual Primitive Modeling":
 * visual tokens are multi-level discrete tokens handled in one token format
 * with text, and the visual codebook embeddings are learned with the
 * backbone).  A visual token t takes the sum over levels, in level order,
 * of row ids[t][l] of level l's embedding table vis[L][K][D]; a text token
 * takes row ids[t][0] of text[V][D] (ids[t][1..L-1] unused).  is_visual
 * may be null: every token is visual.  Returns ORACLE_ERR_ARG on an ID out
 * of range.
 */
int rvq_oracle_embed(const int32_t *ids, const uint8_t *is_visual, int64_t T, int32_t L,
                     const double *text, int64_t V, const double *vis, int32_t K, int32_t D,
                     double *out, int32_t threads)
{
    if (bad_shape(T, D, L, K) || V < 0) return ORACLE_ERR_ARG;
    if (T > 0 && (!ids || !vis || !out)) return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < T; ++t) {
        if (is_visual && !is_visual[t]) {
            if (ids[t * L] < 0 || (int64_t)ids[t * L] >= V || !text) return ORACLE_ERR_ARG;
        } else {
            for (int32_t l = 0; l < L; ++l)
                if (ids[t * L + l] < 0 || ids[t * L + l] >= K) return ORACLE_ERR_ARG;
        }
    }
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel for num_threads(threads) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double *o = out + t * D;
        if (is_visual && !is_visual[t]) {
            const double *e = text + (int64_t)ids[t * L] * D;
            for (int32_t i = 0; i < D; ++i) o[i] = e[i];
        } else {
            for (int32_t i = 0; i < D; ++i) o[i] = 0.0;
            for (int32_t l = 0; l < L; ++l) {
                const double *e = vis + ((int64_t)l * K + ids[t * L + l]) * D;
                for (int32_t i = 0; i < D; ++i) o[i] = o[i] + e[i];
            }
        }
    }
    return ORACLE_OK;
}

/* Per-level usage counts: hist[l][k] = #{n : ids[n][l] == k}. */
int rvq_oracle_hist(const int32_t *ids, int64_t n, int32_t L, int32_t K, int64_t *hist)
{
    if (n < 0 || L < 1 || K < 1 || !hist || (n > 0 && !ids)) return ORACLE_ERR_ARG;
    memset(hist, 0, sizeof(int64_t) * (size_t)L * (size_t)K);
    for (int64_t row = 0; row < n; ++row)
        for (int32_t l = 0; l < L; ++l) {
            int32_t id = ids[row * L + l];
            if (id < 0 || id >= K) return ORACLE_ERR_ARG;
            hist[(int64_t)l * K + id] += 1;
        }
    return ORACLE_OK;
}

/*
 * Squared residual per row and level along the given IDs:
 *   ms[n][l] = || x[n] - sum_{j <= l} cb[j][ids[n][j]] ||^2
 * The mean over rows (the per-level mean squared residual) is taken by the
 * caller in a fixed sequential order.
 */
int rvq_oracle_row_sq_residual(const double *x, const int32_t *ids, int64_t n,
                               int32_t d, const double *cb, int32_t L, int32_t K,
                               double *ms, int32_t threads)
{
    if (bad_shape(n, d, L, K)) return ORACLE_ERR_ARG;
    if (n > 0 && (!x || !ids || !cb || !ms)) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n * L; ++i)
        if (ids[i] < 0 || ids[i] >= K) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
    {
        double *r = (double *)malloc(sizeof(double) * (size_t)d);
        if (!r) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        }
#pragma omp barrier
        if (err == ORACLE_OK) {
#pragma omp for schedule(static)
            for (int64_t row = 0; row < n; ++row) {
                memcpy(r, x + row * d, sizeof(double) * (size_t)d);
                for (int32_t l = 0; l < L; ++l) {
                    const double *c = cb + ((int64_t)l * K + ids[row * L + l]) * d;
                    for (int32_t i = 0; i < d; ++i) r[i] = r[i] - c[i];
                    ms[row * L + l] = sqnorm(r, d);
                }
            }
        }
        free(r);
    }
    return err;
}

/*
 * Teacher-forced check along given IDs (e.g. IDs produced elsewhere):
 * rho_0 = x, rho_{l+1} = rho_l - cb[l][ids[l]].  For every (n, l):
 *   excess[n][l] = dist(rho_l, cb[l][ids[l]]) - min_k dist(rho_l, cb[l][k])
 *   rho2[n][l]   = ||rho_l||^2
 * excess == 0 means the given ID is a nearest codeword of the residual it
 * was chosen for.
 */
int rvq_oracle_teacher_forced(const double *x, const int32_t *ids, int64_t n,
                              int32_t d, const double *cb, int32_t L, int32_t K,
                              double *excess, double *rho2, int32_t threads)
{
    if (bad_shape(n, d, L, K)) return ORACLE_ERR_ARG;
    if (n > 0 && (!x || !ids || !cb || !excess || !rho2)) return ORACLE_ERR_ARG;
    for (int64_t i = 0; i < n * L; ++i)
        if (ids[i] < 0 || ids[i] >= K) return ORACLE_ERR_ARG;
    int err = ORACLE_OK;
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
    {
        double *r = (double *)malloc(sizeof(double) * (size_t)d);
        double *dist = (double *)malloc(sizeof(double) * (size_t)K);
        if (!r || !dist) {
#pragma omp atomic write
            err = ORACLE_ERR_NOMEM;
        }
#pragma omp barrier
        if (err == ORACLE_OK) {
#pragma omp for schedule(dynamic, 1)
            for (int64_t row = 0; row < n; ++row) {
                memcpy(r, x + row * d, sizeof(double) * (size_t)d);
                for (int32_t l = 0; l < L; ++l) {
                    const double *C = cb + (int64_t)l * K * d;
                    rho2[row * L + l] = sqnorm(r, d);
                    for (int32_t k = 0; k < K; ++k) dist[k] = sqdist(r, C + (int64_t)k * d, d);
                    int32_t given = ids[row * L + l];
                    excess[row * L + l] = dist[given] - dist[first_argmin(dist, K)];
                    const double *c = C + (int64_t)given * d;
                    for (int32_t i = 0; i < d; ++i) r[i] = r[i] - c[i];
                }
            }
        }
        free(r);
        free(dist);
    }
    return err;
}
