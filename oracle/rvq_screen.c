/*
 * rvq_screen.c -- the encoder's codeword decision taken at the precision the
 * GPU encoder takes it in, for the CPU test oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  The product (the HIP library) never links,
 * loads or calls this file; only the test suite does.  It shares no code
 * with the GPU path: it is written from the arithmetic the encoder's
 * contract states (bf16 screening of ||r - c||^2, the two best screened
 * codewords rescored in fp32, fp32 residual), not from the kernels.
 *
 * Why it exists.  The method picks, at each level, the codeword nearest to
 * the residual ("LongCat-2.5 Native Multimodality for Agentic Tasks",
 * section "Visual Primitive Modeling"; "LongCat-2.5 Open Source Release
 * ...", section "02 Visual Coding and 3D").  Floating point decides that
 * integer, so a test must compare both sides at one precision.  The fp64
 * oracle (rvq_oracle.c) gives the exact nearest codeword; this file gives
 * the decision of the encoder's own procedure:
 *
 *   1. residual r in fp32: r_0 = x, r_{l+1} = fl32(r_l - c) per feature;
 *   2. codeword norm nv = ||c||^2 in fp32: the features split in two halves
 *      by bit 3 of their index (f & 8), each half an fmaf chain in
 *      increasing feature order from 0, nv = half 0 + half 1; nv is then
 *      carried as two bf16 numbers hi = bf16(nv), lo = bf16(nv - hi);
 *   3. screening score S_k = hi + lo - 2 sum_f bf16(r_f) bf16(c_kf), whose
 *      exact value is formed here in fp64 (every product is exact);
 *   4. the two codewords of smallest screening score are rescored as
 *      sum_f fl32(r_f - c_f)^2, same two-half fmaf chains as in 2, and the
 *      smaller wins, the lower index on a tie; with K = 1 codeword 0 wins.
 *
 * What is not reproduced bit for bit: the GPU accumulates step 3 in fp32 on
 * the matrix cores in an order that is not part of the contract, and ranks
 * scores with their 5 lowest mantissa bits replaced by a tag.  Both are
 * bounded: the GPU's key for codeword k lies within
 *     delta_k = g T_k + 2^-18 (|S_k| + g T_k) + (d + 2) 2^-52 T_k
 * of S_k, with T_k = |hi| + |lo| + 2 sum_f |bf16(r_f) bf16(c_kf)|,
 * g = n u / (1 - n u), n = d + 2 roundings and u = 2^-23 (a unit roundoff
 * that also covers truncating rather than rounding adders); the last term
 * bounds this file's own fp64 sum.  A pair {a, b} can be the GPU's top two
 * exactly when some choice of keys within those bounds puts both below
 * every other codeword (ties may go either way); the admissible IDs of a
 * decision are the rescoring winners of its admissible pairs.  Nearly every
 * decision has one admissible ID.
 *
 * Arithmetic: fp32 steps use C float arithmetic and fmaf (correctly
 * rounded), built with FP contraction off; screening sums are sequential
 * fp64 loops.  Rows are independent, so OpenMP splits the row loop only.
 *
 * Pins (tests/test_oracle_screen.py): bf16 rounding against torch's
 * conversion; the norm chain against exact integer sums and the fp32
 * error bound; with data whose bf16 copies are exact and whose gaps exceed
 * the bounds, ids and residuals equal the fp64 oracle's; a hand-worked
 * three-codeword case where screening ranks the nearest codeword third;
 * the admissible set always holds the unperturbed decision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define SCREEN_OK 0
#define SCREEN_ERR_ARG 1
#define SCREEN_ERR_NOMEM 2
#define SCREEN_ERR_CROWD 3   /* more near-equal scores than MAX_NEAR */
#define SCREEN_ERR_FOLLOW 4  /* a followed id outside [0, K) */

#define MAX_NEAR 64

/* float -> nearest bf16 value (ties to even), returned as a float; finite
 * inputs.  bf16 keeps the upper 16 bits of the fp32 encoding. */
static float bf16_round(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    float o;
    memcpy(&o, &u, 4);
    return o;
}

/* sum_f v_f^2 in fp32: two fmaf chains over the halves f & 8 == 0 and
 * f & 8 == 8, each in increasing f, then added. */
static float sq_chain(const float *v, int32_t d)
{
    float h[2] = {0.0f, 0.0f};
    for (int32_t f = 0; f < d; ++f) {
        const int b = (f >> 3) & 1;
        h[b] = fmaf(v[f], v[f], h[b]);
    }
    return h[0] + h[1];
}

/* Per codebook: hi + lo of each codeword norm and the bf16 copy. */
struct prepared {
    double *hilo;  /* [L][K] hi + lo (exact in fp64) */
    double *habs;  /* [L][K] |hi| + |lo| */
    float *bc;     /* [L][K][d] bf16(c) */
};

static void prepare(const float *cb, int32_t L, int32_t K, int32_t d, struct prepared *p)
{
    for (int64_t k = 0; k < (int64_t)L * K; ++k) {
        const float *c = cb + k * d;
        const float nv = sq_chain(c, d);
        const float hi = bf16_round(nv);
        const float lo = bf16_round(nv - hi);
        p->hilo[k] = (double)hi + (double)lo;
        p->habs[k] = fabs((double)hi) + fabs((double)lo);
        for (int32_t f = 0; f < d; ++f) p->bc[k * d + f] = bf16_round(c[f]);
    }
}

/* Exact screening score of one codeword (step 3) and the bound on how far
 * the GPU's ranking key can lie from it. */
static void score_and_bound(const float *br, const float *bc, double hilo, double habs, int32_t d,
                            double *S, double *D)
{
    const double u = ldexp(1.0, -23);
    const double nr = (double)d + 2.0;
    const double g = nr * u / (1.0 - nr * u);
    double s = 0.0, a = 0.0;
    for (int32_t f = 0; f < d; ++f) {
        const double q = (double)br[f] * (double)bc[f];
        s += q;
        a += fabs(q);
    }
    const double sk = hilo - 2.0 * s;
    const double tk = habs + 2.0 * a;
    *S = sk;
    *D = g * tk + ldexp(fabs(sk) + g * tk, -18) + nr * ldexp(tk, -52);
}

/* Exact fp32 rescoring distance of residual r to codeword c. */
static float rescore(const float *r, const float *c, float *t, int32_t d)
{
    for (int32_t f = 0; f < d; ++f) t[f] = r[f] - c[f];
    return sq_chain(t, d);
}

/* Winner of a rescored pair: smaller distance, lower index on a tie. */
static int32_t pair_winner(int32_t a, float da, int32_t b, float db)
{
    if (da < db) return a;
    if (db < da) return b;
    return a < b ? a : b;
}

/*
 * One decision.  r: fp32 residual, br: its bf16 copy.  Writes the
 * unperturbed choice to *own (the winner of the two smallest exact scores,
 * lower index first among equal scores), the admissible IDs to win[0..*nw).
 * Scratch: S, D [K] doubles, t [d] floats.
 */
static int decide(const float *r, const float *br, const float *cbl, const struct prepared *p,
                  int64_t off, int32_t K, int32_t d, double *S, double *D, float *t,
                  int32_t *own, int32_t *win, int32_t *nw)
{
    if (K == 1) {
        *own = 0;
        win[0] = 0;
        *nw = 1;
        return SCREEN_OK;
    }
    int32_t b1 = -1, b2 = -1;  /* two smallest (S, index) */
    for (int32_t k = 0; k < K; ++k) {
        score_and_bound(br, p->bc + (off + k) * (int64_t)d, p->hilo[off + k], p->habs[off + k],
                        d, &S[k], &D[k]);
        const double sk = S[k];
        if (b1 < 0 || sk < S[b1]) {
            b2 = b1;
            b1 = k;
        } else if (b2 < 0 || sk < S[b2]) {
            b2 = k;
        }
    }
    const float *c1 = cbl + (int64_t)b1 * d, *c2 = cbl + (int64_t)b2 * d;
    *own = pair_winner(b1, rescore(r, c1, t, d), b2, rescore(r, c2, t, d));

    /* second smallest upper end S + D: no codeword whose lower end lies
     * above it can be among the top two */
    double u1 = INFINITY, u2 = INFINITY;
    for (int32_t k = 0; k < K; ++k) {
        const double hi = S[k] + D[k];
        if (hi < u1) {
            u2 = u1;
            u1 = hi;
        } else if (hi < u2) {
            u2 = hi;
        }
    }
    int32_t near[MAX_NEAR];
    int32_t m = 0;
    for (int32_t k = 0; k < K; ++k) {
        if (S[k] - D[k] <= u2) {
            if (m == MAX_NEAR) return SCREEN_ERR_CROWD;
            near[m++] = k;
        }
    }
    float dist[MAX_NEAR];
    for (int32_t i = 0; i < m; ++i) dist[i] = rescore(r, cbl + (int64_t)near[i] * d, t, d);
    *nw = 0;
    for (int32_t i = 0; i < m; ++i) {
        for (int32_t j = i + 1; j < m; ++j) {
            const int32_t a = near[i], b = near[j];
            const double top = fmax(S[a] - D[a], S[b] - D[b]);
            int ok = 1;
            for (int32_t q = 0; q < m && ok; ++q) {
                const int32_t k = near[q];
                if (k != a && k != b && S[k] + D[k] < top) ok = 0;
            }
            if (!ok) continue;
            const int32_t w = pair_winner(a, dist[i], b, dist[j]);
            int seen = 0;
            for (int32_t q = 0; q < *nw; ++q) seen |= win[q] == w;
            if (!seen) win[(*nw)++] = w;
        }
    }
    return SCREEN_OK;
}

/*
 * Greedy encode with the encoder's decision procedure.
 *   x      [n][d] fp32 input rows (bf16 inputs passed as their fp32 values)
 *   cb     [L][K][d] fp32 codebooks
 *   follow [n][L] or NULL.  NULL: each level takes the unperturbed decision.
 *          Otherwise each level takes follow's ID (it must lie in [0, K))
 *          and reports whether that ID was admissible.
 * Outputs (any may be NULL):
 *   ids        [n][L] the IDs taken
 *   n_options  [n][L] number of admissible IDs of the decision (>= 1)
 *   admissible [n][L] 1 if the ID taken is admissible (always 1 without follow)
 *   res        [n][d] fp32 residual after the L levels
 * Returns 0, or an error code above.
 */
int rvq_oracle_screen_encode(const float *x, int64_t n, int32_t d, const float *cb, int32_t L,
                             int32_t K, const int32_t *follow, int32_t *ids, int32_t *n_options,
                             uint8_t *admissible, float *res, int32_t threads)
{
    if (n < 0 || d < 1 || L < 1 || K < 1 || (n > 0 && (!x || !cb))) return SCREEN_ERR_ARG;
    if (n == 0) return SCREEN_OK;
    struct prepared p;
    const size_t lk = (size_t)L * K;
    p.hilo = malloc(lk * sizeof(double));
    p.habs = malloc(lk * sizeof(double));
    p.bc = malloc(lk * (size_t)d * sizeof(float));
    int err = SCREEN_OK;
    if (!p.hilo || !p.habs || !p.bc) {
        err = SCREEN_ERR_NOMEM;
        goto out;
    }
    prepare(cb, L, K, d, &p);
    if (threads < 1) threads = omp_get_max_threads();
#pragma omp parallel num_threads(threads)
    {
        float *r = malloc((size_t)d * sizeof(float));
        float *br = malloc((size_t)d * sizeof(float));
        float *t = malloc((size_t)d * sizeof(float));
        double *S = malloc((size_t)K * sizeof(double));
        double *D = malloc((size_t)K * sizeof(double));
        if (!r || !br || !t || !S || !D) {
#pragma omp atomic write
            err = SCREEN_ERR_NOMEM;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t row = 0; row < n; ++row) {
                memcpy(r, x + row * d, (size_t)d * sizeof(float));
                for (int32_t l = 0; l < L; ++l) {
                    for (int32_t f = 0; f < d; ++f) br[f] = bf16_round(r[f]);
                    const int64_t off = (int64_t)l * K;
                    const float *cbl = cb + off * d;
                    int32_t own, nw, win[MAX_NEAR];
                    const int e = decide(r, br, cbl, &p, off, K, d, S, D, t, &own, win, &nw);
                    if (e != SCREEN_OK) {
#pragma omp atomic write
                        err = e;
                        break;
                    }
                    int32_t take = own;
                    uint8_t ok = 1;
                    if (follow) {
                        take = follow[row * L + l];
                        if (take < 0 || take >= K) {
#pragma omp atomic write
                            err = SCREEN_ERR_FOLLOW;
                            break;
                        }
                        ok = 0;
                        for (int32_t q = 0; q < nw; ++q) ok |= win[q] == take;
                    }
                    if (ids) ids[row * L + l] = take;
                    if (n_options) n_options[row * L + l] = nw;
                    if (admissible) admissible[row * L + l] = ok;
                    const float *c = cbl + (int64_t)take * d;
                    for (int32_t f = 0; f < d; ++f) r[f] = r[f] - c[f];
                }
                if (res) memcpy(res + row * d, r, (size_t)d * sizeof(float));
            }
        }
        free(r);
        free(br);
        free(t);
        free(S);
        free(D);
    }
out:
    free(p.hilo);
    free(p.habs);
    free(p.bc);
    return err;
}

/* out[i] = the bf16 rounding of v[i] (as a float), i < n. */
int rvq_oracle_screen_round_bf16(const float *v, int64_t n, float *out)
{
    if (n < 0 || (n > 0 && (!v || !out))) return SCREEN_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_round(v[i]);
    return SCREEN_OK;
}

/* out[i] = the fp32 two-half chain sum of squares of row i of v [n][d]
 * (step 2: the codeword norm; step 4 applies it to r - c). */
int rvq_oracle_screen_sq_chain(const float *v, int64_t n, int32_t d, float *out)
{
    if (n < 0 || d < 1 || (n > 0 && (!v || !out))) return SCREEN_ERR_ARG;
    for (int64_t i = 0; i < n; ++i) out[i] = sq_chain(v + i * d, d);
    return SCREEN_OK;
}

/* Screening scores of rows r [n][d] (fp32) against one codebook cb [K][d]:
 * S [n][K] the exact score of step 3, D [n][K] the bound on the GPU's key. */
int rvq_oracle_screen_scores(const float *r, int64_t n, int32_t d, const float *cb, int32_t K,
                             double *S, double *D)
{
    if (n < 0 || d < 1 || K < 1 || (n > 0 && (!r || !cb || !S || !D))) return SCREEN_ERR_ARG;
    if (n == 0) return SCREEN_OK;
    struct prepared p;
    p.hilo = malloc((size_t)K * sizeof(double));
    p.habs = malloc((size_t)K * sizeof(double));
    p.bc = malloc((size_t)K * (size_t)d * sizeof(float));
    float *br = malloc((size_t)d * sizeof(float));
    int err = SCREEN_OK;
    if (!p.hilo || !p.habs || !p.bc || !br) {
        err = SCREEN_ERR_NOMEM;
    } else {
        prepare(cb, 1, K, d, &p);
        for (int64_t i = 0; i < n; ++i) {
            for (int32_t f = 0; f < d; ++f) br[f] = bf16_round(r[i * d + f]);
            for (int32_t k = 0; k < K; ++k)
                score_and_bound(br, p.bc + (int64_t)k * d, p.hilo[k], p.habs[k], d,
                                &S[i * K + k], &D[i * K + k]);
        }
    }
    free(p.hilo);
    free(p.habs);
    free(p.bc);
    free(br);
    return err;
}
