/*
 * CPU oracle for the routed 4-bit MoE expert FFN (switch-GLU with a tanh-GELU
 * product, "GeGLU").
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * Everything is the plain definition, written out in IEEE double:
 *
 *   route   counts, exclusive offsets, and a stable counting sort of the flat
 *           assignment index a = t*k + j by expert id: the "sorted indices"
 *           that the Layr-Labs/mlx PR #4 page ("What") feeds its expert-tile
 *           kernel.
 *   tiles   per expert, runs of at most bm_big sorted rows; a run of at most
 *           bm_small rows is marked bm_small: the page's "BM32 expert tiles,
 *           BM16 fallback rows" ("What"), emitted in expert order as its
 *           scan-plus-upper-bound builder produces them.
 *   weight  W[e,n,c] = S[e,n,c/gs] * q + B[e,n,c/gs], q the 4-bit code of
 *           element c (low nibble first in each uint32 word): the affine
 *           4-bit, group-size-64 format of the PR #4 page ("What"), with the
 *           scale and bias widened before use (mlx-node PR #168 page: the
 *           sidecars are promoted to f32 "either way").  Group sizes 32 and
 *           128 and 8-bit codes (4 per word, low byte first) are the same
 *           affine format at other geometries; the pages use only 4-bit, 64.
 *   gate|up g = x . W_gu[e, n, :], u = x . W_gu[e, I+n, :]  (PR #168 page:
 *           one packed "MLP gate|up" projection split in two halves).
 *   GeGLU   h = gelu_tanh(g) * u, with
 *           gelu_tanh(v) = 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
 *           (SwiftLM issue #236, "Still missing": activation(xGate) * xUp with
 *           activation = geluApproximate).
 *   SwiGLU  h = silu(g) * u, silu(v) = v / (1 + exp(-v)), when act = 1 (the
 *           SwiGLU product of SwiftLM issue #236, "What #27 set out to do" (2)
 *           and "Already on main"; mlx-node PR #168's MoE switch GLU).  The
 *           pages do not spell out SiLU; this is its usual definition.
 *   down    y[a, m] = W_d[e, m, :] . h
 *   combine out[t, m] = sum_j w[t, j] * y[t*k + j, m]  (SwiftLM issue #236
 *           "Already on main": weightedExpertSum; PR #4 "Measured standing":
 *           the direct weighted unsort back to token order).
 *
 * oracle_ffn_all computes the same sums for a whole batch, expert by expert
 * (each expert's matrices dequantised once), in the same order, so its
 * results are the same bits as oracle_ffn_tokens'.
 *
 * Expert ids outside [0, E) are not routed: they are counted, placed after all
 * valid rows in the sorted order (ascending a), get no tile, and contribute
 * zero to the combine.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_ALLOC (-2)

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only; results do not depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------- route */

int oracle_route(const int32_t* ids, int64_t A, int32_t E,
                 int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* inv_perm, int32_t* n_invalid) {
    if (A < 0 || E <= 0 || (A > 0 && (!ids || !perm || !inv_perm)) || !counts ||
        !offsets || !n_invalid)
        return ORACLE_ERR_ARG;
    int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!fill) return ORACLE_ERR_ALLOC;
    for (int32_t e = 0; e < E; ++e) counts[e] = 0;
    int32_t bad = 0;
    for (int64_t a = 0; a < A; ++a) {
        int32_t e = ids[a];
        if (e >= 0 && e < E)
            counts[e] += 1;
        else
            bad += 1;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t bad_fill = 0;
    for (int64_t a = 0; a < A; ++a) {
        int32_t e = ids[a];
        int32_t s;
        if (e >= 0 && e < E)
            s = offsets[e] + fill[e]++;
        else
            s = offsets[E] + bad_fill++;
        perm[s] = (int32_t)a;
        inv_perm[a] = s;
    }
    *n_invalid = bad;
    free(fill);
    return ORACLE_OK;
}

/* tiles: 4 int32 per tile {expert, row_begin, row_count, bm}. */
int oracle_tiles(const int32_t* counts, const int32_t* offsets, int32_t E,
                 int32_t bm_big, int32_t bm_small, int32_t* tiles,
                 int64_t max_tiles, int32_t* num_tiles) {
    if (!counts || !offsets || E <= 0 || bm_big <= 0 || bm_small <= 0 ||
        bm_small > bm_big || !num_tiles)
        return ORACLE_ERR_ARG;
    int64_t nt = 0;
    for (int32_t e = 0; e < E; ++e) {
        for (int32_t done = 0; done < counts[e]; done += bm_big) {
            int32_t rows = counts[e] - done;
            if (rows > bm_big) rows = bm_big;
            if (nt < max_tiles && tiles) {
                tiles[4 * nt + 0] = e;
                tiles[4 * nt + 1] = offsets[e] + done;
                tiles[4 * nt + 2] = rows;
                tiles[4 * nt + 3] = (rows <= bm_small) ? bm_small : bm_big;
            }
            ++nt;
        }
    }
    *num_tiles = (int32_t)nt;
    return nt <= max_tiles ? ORACLE_OK : ORACLE_ERR_ARG;
}

/* ------------------------------------------------------------- weights */

/* The code of column c in one packed row: bits = 4, 8 codes per word, low
 * nibble first; bits = 8, 4 codes per word, low byte first. */
static int32_t code_at(const uint32_t* packed_row, int64_t c, int32_t bits) {
    const int64_t per_word = 32 / bits;
    const uint32_t word = packed_row[c / per_word];
    const uint32_t mask = (1u << bits) - 1u;
    return (int32_t)((word >> (bits * (c % per_word))) & mask);
}

/* Dequantised weight W[e, n, c] of a [E, rows, K] matrix of bits-wide codes. */
double oracle_weight(const uint32_t* P, const uint16_t* S, const uint16_t* B,
                     int64_t rows, int64_t K, int32_t gs, int32_t bits, int64_t e,
                     int64_t n, int64_t c) {
    const int64_t row = e * rows + n;
    const int64_t groups = K / gs;
    double s = bf16_value(S[row * groups + c / gs]);
    double b = bf16_value(B[row * groups + c / gs]);
    return s * (double)code_at(P + row * (K * bits / 32), c, bits) + b;
}

double oracle_gelu_tanh(double v) {
    const double k0 = sqrt(2.0 / M_PI);
    return 0.5 * v * (1.0 + tanh(k0 * (v + 0.044715 * v * v * v)));
}

double oracle_silu(double v) { return v / (1.0 + exp(-v)); }

/* dot(W[e, n, :], v) over K columns, v in double. */
static double row_dot(const uint32_t* P, const uint16_t* S, const uint16_t* B,
                      int64_t rows, int64_t K, int32_t gs, int32_t bits, int64_t e,
                      int64_t n, const double* v) {
    double acc = 0.0;
    for (int64_t c = 0; c < K; ++c)
        acc += oracle_weight(P, S, B, rows, K, gs, bits, e, n, c) * v[c];
    return acc;
}

/* ------------------------------------------------------------- forward */

/*
 * Expert FFN for the listed tokens.  For list entry i (token t = tokens[i])
 * and slot j, assignment a = t*k + j is stored at row r = i*k + j of
 *   h   [ntok*k, I]  act(g) * u, act = gelu_tanh (act 0) or silu (act 1)
 *                    (NULL to skip)
 *   y   [ntok*k, H]  unweighted expert output (NULL to skip)
 *   out [ntok, H]    sum_j w[t, j] * y[t*k+j] (NULL to skip)
 * Rows of an assignment with an out-of-range expert id are zero.
 */
int oracle_ffn_tokens(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I,
                      int32_t gs, int32_t bits, const uint16_t* x, const int32_t* ids,
                      const float* w, const uint32_t* w_gu, const uint16_t* s_gu,
                      const uint16_t* b_gu, const uint32_t* w_d,
                      const uint16_t* s_d, const uint16_t* b_d,
                      const int32_t* tokens, int32_t ntok, int32_t act, double* h,
                      double* y, double* out) {
    if (act != 0 && act != 1) return ORACLE_ERR_ARG;
    if (T < 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0 || gs <= 0 || H % gs ||
        I % gs || H % 8 || I % 8 || (bits != 4 && bits != 8) || ntok < 0 ||
        (ntok > 0 && !tokens))
        return ORACLE_ERR_ARG;
    for (int32_t i = 0; i < ntok; ++i)
        if (tokens[i] < 0 || tokens[i] >= T) return ORACLE_ERR_ARG;
    const int64_t n_rows = (int64_t)ntok * k;
    double* yy = (double*)calloc((size_t)(n_rows > 0 ? n_rows : 1) * (size_t)H,
                                 sizeof(double));
    if (!yy) return ORACLE_ERR_ALLOC;
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t t = tokens[r / k];
        const int64_t a = t * k + (r % k);
        const int32_t e = ids[a];
        double* xv = (double*)malloc(sizeof(double) * (size_t)H);
        double* hv = (double*)malloc(sizeof(double) * (size_t)I);
        if (!xv || !hv) {
            failed = 1;
            free(xv);
            free(hv);
            continue;
        }
        for (int64_t c = 0; c < H; ++c) xv[c] = bf16_value(x[t * H + c]);
        if (e >= 0 && e < E) {
            for (int64_t n = 0; n < I; ++n) {
                double g = row_dot(w_gu, s_gu, b_gu, 2 * (int64_t)I, H, gs, bits, e, n, xv);
                double u = row_dot(w_gu, s_gu, b_gu, 2 * (int64_t)I, H, gs, bits, e, I + n, xv);
                hv[n] = (act ? oracle_silu(g) : oracle_gelu_tanh(g)) * u;
            }
            for (int64_t m = 0; m < H; ++m)
                yy[r * H + m] = row_dot(w_d, s_d, b_d, H, I, gs, bits, e, m, hv);
        } else {
            for (int64_t n = 0; n < I; ++n) hv[n] = 0.0;
        }
        if (h) memcpy(h + r * I, hv, sizeof(double) * (size_t)I);
        free(xv);
        free(hv);
    }
    if (failed) {
        free(yy);
        return ORACLE_ERR_ALLOC;
    }
    if (y) memcpy(y, yy, sizeof(double) * (size_t)n_rows * (size_t)H);
    if (out) {
        for (int64_t i = 0; i < ntok; ++i) {
            const int64_t t = tokens[i];
            for (int64_t m = 0; m < H; ++m) {
                double acc = 0.0;
                for (int64_t j = 0; j < k; ++j) {
                    const int32_t e = ids[t * k + j];
                    if (e < 0 || e >= E) continue;
                    acc += (double)w[t * k + j] * yy[(i * k + j) * H + m];
                }
                out[i * H + m] = acc;
            }
        }
    }
    free(yy);
    return ORACLE_OK;
}

/*
 * The same expert FFN for every assignment of the batch, organised by expert
 * so that a large batch finishes in seconds: each expert's matrices are
 * dequantised once (W = S * q + B, the values oracle_weight gives), then
 * every dot product is the same plain sum over the columns in ascending
 * order as in oracle_ffn_tokens, so the results are bit-identical to it.
 * Only the loop order differs: for each expert, output neuron n runs over
 * all of the expert's assignments (ascending a) while row n of the matrix is
 * at hand.
 *   h   [T*k, I]  flat order a = t*k + j (NULL to skip)
 *   y   [T*k, H]  unweighted expert output, flat order (NULL to skip)
 *   out [T, H]    sum_j w[t, j] * y[t*k+j] (NULL to skip)
 * Rows of an assignment with an out-of-range expert id are zero.
 */
int oracle_ffn_all(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I, int32_t gs,
                   int32_t bits, const uint16_t* x, const int32_t* ids, const float* w,
                   const uint32_t* w_gu, const uint16_t* s_gu, const uint16_t* b_gu,
                   const uint32_t* w_d, const uint16_t* s_d, const uint16_t* b_d,
                   int32_t act, double* h, double* y, double* out) {
    if (act != 0 && act != 1) return ORACLE_ERR_ARG;
    if (T < 0 || k <= 0 || E <= 0 || H <= 0 || I <= 0 || gs <= 0 || H % gs ||
        I % gs || H % 8 || I % 8 || (bits != 4 && bits != 8))
        return ORACLE_ERR_ARG;
    const int64_t A = (int64_t)T * k;
    const size_t nA = (size_t)(A > 0 ? A : 1);
    double* xv = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * (size_t)H);
    double* hh = (double*)calloc(nA * (size_t)I, sizeof(double));
    double* yy = (double*)calloc(nA * (size_t)H, sizeof(double));
    double* wgu = (double*)malloc(sizeof(double) * 2 * (size_t)I * (size_t)H);
    double* wd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)I);
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * nA);
    if (!xv || !hh || !yy || !wgu || !wd || !rows) {
        free(xv); free(hh); free(yy); free(wgu); free(wd); free(rows);
        return ORACLE_ERR_ALLOC;
    }
    for (int64_t i = 0; i < (int64_t)T * H; ++i) xv[i] = bf16_value(x[i]);
    for (int32_t e = 0; e < E; ++e) {
        int64_t n_rows = 0;
        for (int64_t a = 0; a < A; ++a)
            if (ids[a] == e) rows[n_rows++] = a;
        if (n_rows == 0) continue;
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < 2 * (int64_t)I; ++n)
            for (int64_t c = 0; c < H; ++c)
                wgu[n * H + c] = oracle_weight(w_gu, s_gu, b_gu, 2 * (int64_t)I, H, gs, bits, e, n, c);
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < H; ++m)
            for (int64_t c = 0; c < I; ++c)
                wd[m * I + c] = oracle_weight(w_d, s_d, b_d, H, I, gs, bits, e, m, c);
#pragma omp parallel for schedule(dynamic, 8)
        for (int64_t n = 0; n < I; ++n) {
            const double* wg = wgu + n * H;
            const double* wu = wgu + (I + n) * H;
            for (int64_t r = 0; r < n_rows; ++r) {
                const int64_t a = rows[r];
                const double* xr = xv + (a / k) * H;
                double g = 0.0, u = 0.0;
                for (int64_t c = 0; c < H; ++c) g += wg[c] * xr[c];
                for (int64_t c = 0; c < H; ++c) u += wu[c] * xr[c];
                hh[a * I + n] = (act ? oracle_silu(g) : oracle_gelu_tanh(g)) * u;
            }
        }
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t m = 0; m < H; ++m) {
            const double* wm = wd + m * I;
            for (int64_t r = 0; r < n_rows; ++r) {
                const int64_t a = rows[r];
                const double* hr = hh + a * I;
                double acc = 0.0;
                for (int64_t c = 0; c < I; ++c) acc += wm[c] * hr[c];
                yy[a * H + m] = acc;
            }
        }
    }
    if (out) {
#pragma omp parallel for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int64_t m = 0; m < H; ++m) {
                double acc = 0.0;
                for (int64_t j = 0; j < k; ++j) {
                    const int32_t e = ids[t * k + j];
                    if (e < 0 || e >= E) continue;
                    acc += (double)w[t * k + j] * yy[(t * k + j) * H + m];
                }
                out[t * H + m] = acc;
            }
        }
    }
    if (h) memcpy(h, hh, sizeof(double) * (size_t)A * (size_t)I);
    if (y) memcpy(y, yy, sizeof(double) * (size_t)A * (size_t)H);
    free(xv); free(hh); free(yy); free(wgu); free(wd); free(rows);
    return ORACLE_OK;
}

/*
 * The down projection alone, for rows whose h is given: row r (expert
 * experts[r]) gets y[r, m] = sum_n W_d[e, m, n] * h[r, n], summed over n in
 * ascending order, and yabs[r, m] = sum_n |W_d[e, m, n] * h[r, n]| (the sum of
 * the terms' magnitudes, which bounds the rounding error of any fp32
 * evaluation of the same sum; NULL to skip).  Rows of an out-of-range expert
 * are zero.
 */
int oracle_down_rows(int32_t E, int32_t H, int32_t I, int32_t gs, int32_t bits,
                     const uint32_t* w_d, const uint16_t* s_d, const uint16_t* b_d,
                     const int32_t* experts, int64_t n_rows, const double* h, double* y,
                     double* yabs) {
    if (E <= 0 || H <= 0 || I <= 0 || gs <= 0 || I % gs || I % 8 || n_rows < 0 ||
        (bits != 4 && bits != 8) || (n_rows > 0 && (!experts || !h || !y)))
        return ORACLE_ERR_ARG;
    double* wd = (double*)malloc(sizeof(double) * (size_t)H * (size_t)I);
    int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n_rows > 0 ? n_rows : 1));
    if (!wd || !rows) {
        free(wd);
        free(rows);
        return ORACLE_ERR_ALLOC;
    }
    for (int64_t i = 0; i < n_rows * H; ++i) {
        y[i] = 0.0;
        if (yabs) yabs[i] = 0.0;
    }
    for (int32_t e = 0; e < E; ++e) {
        int64_t cnt = 0;
        for (int64_t r = 0; r < n_rows; ++r)
            if (experts[r] == e) rows[cnt++] = r;
        if (cnt == 0) continue;
#pragma omp parallel for schedule(static)
        for (int64_t m = 0; m < H; ++m)
            for (int64_t c = 0; c < I; ++c)
                wd[m * I + c] = oracle_weight(w_d, s_d, b_d, H, I, gs, bits, e, m, c);
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t m = 0; m < H; ++m) {
            const double* wm = wd + m * I;
            for (int64_t i = 0; i < cnt; ++i) {
                const int64_t r = rows[i];
                const double* hr = h + r * I;
                double acc = 0.0, mag = 0.0;
                for (int64_t c = 0; c < I; ++c) {
                    acc += wm[c] * hr[c];
                    mag += fabs(wm[c] * hr[c]);
                }
                y[r * H + m] = acc;
                if (yabs) yabs[r * H + m] = mag;
            }
        }
    }
    free(wd);
    free(rows);
    return ORACLE_OK;
}

/* ------------------------------------------------------------- router */

/*
 * Softmax top-k routing of one logits row per token, in double: the k largest
 * logits (ties to the lower expert id), in order of descending logit, with
 * weights exp(l_i - m) / sum over the k chosen of exp(l_j - m), m the largest
 * logit.  That is the softmax over all E experts renormalised over the chosen
 * k: the full softmax denominator cancels.  The pages do not define the
 * router; this is the usual top-k softmax gate with renormalised weights (the
 * fused top-k candidate selection of the mlx-node PR #168 page is its nearest
 * relative there).
 */
int oracle_router_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                       int32_t* ids, double* weights) {
    if (T < 0 || E <= 0 || k <= 0 || k > E || (T > 0 && (!logits || !ids || !weights)))
        return ORACLE_ERR_ARG;
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        int32_t* id = ids + t * k;
        /* selection: repeatedly take the largest remaining logit, lowest id on ties */
        for (int32_t j = 0; j < k; ++j) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int32_t i = 0; i < j; ++i) taken |= (id[i] == e);
                if (taken) continue;
                if (best < 0 || (double)l[e] > (double)l[best]) best = e;
            }
            id[j] = best;
        }
        const double m = (double)l[id[0]];
        double sum = 0.0;
        for (int32_t j = 0; j < k; ++j) sum += exp((double)l[id[j]] - m);
        for (int32_t j = 0; j < k; ++j) weights[t * k + j] = exp((double)l[id[j]] - m) / sum;
    }
    return ORACLE_OK;
}
