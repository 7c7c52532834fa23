/*
 * oracle.c -- plain, slow, fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  The library never calls, links or loads this
 * file; only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with
 * the HIP kernels, and includes nothing from them.
 *
 * What it computes is the plain definition, not the tiled algorithm: the
 * pages state that the tiled method reaches the same result as standard
 * attention up to floating-point rounding ("FlashAttention." plate, section
 * "Never write the scores"; "FlashAttention: Fast and Memory-Efficient Exact
 * Attention with IO-Awareness", DarcStar commentary, which says the tiled
 * result equals the standard one).
 * Standard attention is spelled out in the opening of the "FlashAttention."
 * plate: S = Q K^T, a row softmax of S, then P V.  Every step below follows
 * that order, one query row at a time, in double precision, with libm's
 * exp() and log().
 *
 * Readings of points the pages leave open (all listed in the design notes):
 *   - scale multiplies the scores before the softmax (the pages use
 *     1/sqrt(d); the caller passes the value it wants);
 *   - a masked score is -infinity; key j is visible to query i under the
 *     causal mask iff j <= i;
 *   - a block mask entry mask[i/mb][j/mb] == 0 masks the whole tile
 *     (block-sparse attention skips the tiles that are not relevant:
 *     "Flash Attention: IO-Aware Attention Computation", paragraph on
 *     block-sparse attention);
 *   - a row with every score masked has O = 0 and LSE = -infinity;
 *   - LSE is the natural log-sum-exp of the scaled, masked scores;
 *   - the backward pass is derived by calculus from the forward definition
 *     (the pages only say the scores are recomputed, "Never write the
 *     scores").
 *
 * Parity pins: see tests/test_oracle.py (brute force in 40-digit decimal,
 * torch fp64 library routines, closed forms, invariants, central finite
 * differences).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* Visibility of key j to query i under the causal flag and the tile mask. */
static int visible(long i, long j, int causal, const unsigned char *mask,
                   int mb, long nkb)
{
    if (causal && j > i)
        return 0;
    if (mask && !mask[(i / mb) * nkb + (j / mb)])
        return 0;
    return 1;
}

static double dot(const double *a, const double *b, int d)
{
    double acc = 0.0;
    for (int c = 0; c < d; ++c)
        acc += a[c] * b[c];
    return acc;
}

/*
 * Softmax row of query i of one head: fills p[j] = P_ij (0 where masked)
 * and returns LSE_i.  Follows the definition: scores s_j = scale * q_i . k_j,
 * masked scores -inf, m = max_j s_j, p_j = exp(s_j - m), l = sum_j p_j,
 * P_ij = p_j / l, LSE_i = m + ln l.  A fully masked row gives P = 0 and
 * LSE = -inf.
 */
static double softmax_row(const double *qi, const double *K, long N, int d,
                          double scale, long i, int causal,
                          const unsigned char *mask, int mb, long nkb,
                          double *p)
{
    double m = -INFINITY;
    for (long j = 0; j < N; ++j) {
        if (visible(i, j, causal, mask, mb, nkb)) {
            p[j] = scale * dot(qi, K + j * d, d);
            if (p[j] > m)
                m = p[j];
        } else {
            p[j] = -INFINITY;
        }
    }
    if (m == -INFINITY) {
        for (long j = 0; j < N; ++j)
            p[j] = 0.0;
        return -INFINITY;
    }
    double l = 0.0;
    for (long j = 0; j < N; ++j) {
        p[j] = (p[j] == -INFINITY) ? 0.0 : exp(p[j] - m);
        l += p[j];
    }
    for (long j = 0; j < N; ++j)
        p[j] /= l;
    return m + log(l);
}

static int check_args(const void *a, const void *b, const void *c, long nheads,
                      long N, int d, const unsigned char *mask, int mb)
{
    if (!a || !b || !c || nheads < 0 || N < 0 || d <= 0)
        return -1;
    if (mask && mb <= 0)
        return -1;
    return 0;
}

/*
 * Forward: O = softmax(scale * Q K^T  (+ masks)) V and LSE, for `nheads`
 * independent heads laid out contiguously as [nheads][N][d] (O the same,
 * LSE [nheads][N]).  The tile mask, if given, is [ceil(N/mb)][ceil(N/mb)]
 * bytes and is shared by every head.  Work is split over (head, row) pairs;
 * nthreads <= 0 means OpenMP's default.  Returns 0, or -1 on bad arguments
 * or allocation failure.
 */
int oracle_forward(const double *q, const double *k, const double *v,
                   double *o, double *lse, long nheads, long N, int d,
                   double scale, int causal, const unsigned char *mask,
                   int mb, int nthreads)
{
    if (check_args(q, k, v, nheads, N, d, mask, mb) || !o || !lse)
        return -1;
    const long nkb = mask ? (N + mb - 1) / mb : 0;
    const long total = nheads * N;
    int failed = 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!p) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long r = 0; r < total; ++r) {
                const long h = r / N, i = r % N;
                const double *K = k + h * N * d, *V = v + h * N * d;
                double *oi = o + r * d;
                lse[r] = softmax_row(q + r * d, K, N, d, scale, i, causal,
                                     mask, mb, nkb, p);
                for (int c = 0; c < d; ++c)
                    oi[c] = 0.0;
                for (long j = 0; j < N; ++j) {
                    if (p[j] == 0.0)
                        continue;
                    for (int c = 0; c < d; ++c)
                        oi[c] += p[j] * V[j * d + c];
                }
            }
            free(p);
        }
    }
    return failed ? -1 : 0;
}

/*
 * Backward of L(Q,K,V) with upstream gradient dO = dL/dO, derived from the
 * forward definition (the chain rule through P = softmax(S), S = scale*QK^T):
 *
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . V_j
 *   D_i   = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij K_j
 *   dK_j  = scale * sum_i dS_ij Q_i
 *
 * P is recomputed from Q and K here (never taken from the GPU).  The pass
 * runs in two sweeps so every output element has one owner: a row sweep that
 * produces dQ_i, LSE_i and D_i, then a column sweep that produces dK_j and
 * dV_j, in which P_ij = exp(s_ij - LSE_i) (the same quantity as the row
 * softmax, by the definition of LSE).  lse_out and delta_out ([nheads][N])
 * are optional outputs of LSE and D.  Returns 0, or -1 on bad arguments or
 * allocation failure.
 */
int oracle_backward(const double *q, const double *k, const double *v,
                    const double *dout, double *dq, double *dk, double *dv,
                    double *lse_out, double *delta_out, long nheads, long N,
                    int d, double scale, int causal, const unsigned char *mask,
                    int mb, int nthreads)
{
    if (check_args(q, k, v, nheads, N, d, mask, mb) || !dout || !dq || !dk ||
        !dv)
        return -1;
    const long nkb = mask ? (N + mb - 1) / mb : 0;
    const long total = nheads * N;
    double *lse = (double *)malloc(sizeof(double) * (size_t)(total > 0 ? total : 1));
    double *D = (double *)malloc(sizeof(double) * (size_t)(total > 0 ? total : 1));
    if (!lse || !D) {
        free(lse);
        free(D);
        return -1;
    }
    int failed = 0;
    if (nthreads <= 0)
        nthreads = omp_get_max_threads();

    /* Row sweep: P_i, dP_i, D_i, dS_i, dQ_i. */
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
        if (!p || !dp) {
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long r = 0; r < total; ++r) {
                const long h = r / N, i = r % N;
                const double *K = k + h * N * d, *V = v + h * N * d;
                const double *doi = dout + r * d;
                lse[r] = softmax_row(q + r * d, K, N, d, scale, i, causal,
                                     mask, mb, nkb, p);
                double Di = 0.0;
                for (long j = 0; j < N; ++j) {
                    dp[j] = (p[j] == 0.0) ? 0.0 : dot(doi, V + j * d, d);
                    Di += p[j] * dp[j];
                }
                D[r] = Di;
                double *dqi = dq + r * d;
                for (int c = 0; c < d; ++c)
                    dqi[c] = 0.0;
                for (long j = 0; j < N; ++j) {
                    if (p[j] == 0.0)
                        continue;
                    const double dsij = p[j] * (dp[j] - Di);
                    for (int c = 0; c < d; ++c)
                        dqi[c] += scale * dsij * K[j * d + c];
                }
            }
        }
        free(p);
        free(dp);
    }

    /* Column sweep: dV_j and dK_j, with P_ij = exp(s_ij - LSE_i). */
    if (!failed) {
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 16)
        for (long r = 0; r < total; ++r) {
            const long h = r / N, j = r % N;
            const double *Q = q + h * N * d, *dO = dout + h * N * d;
            const double *kj = k + r * d, *vj = v + r * d;
            const double *L = lse + h * N, *Dh = D + h * N;
            double *dkj = dk + r * d, *dvj = dv + r * d;
            for (int c = 0; c < d; ++c) {
                dkj[c] = 0.0;
                dvj[c] = 0.0;
            }
            for (long i = 0; i < N; ++i) {
                if (!visible(i, j, causal, mask, mb, nkb) || L[i] == -INFINITY)
                    continue;
                const double pij = exp(scale * dot(Q + i * d, kj, d) - L[i]);
                const double dpij = dot(dO + i * d, vj, d);
                const double dsij = pij * (dpij - Dh[i]);
                for (int c = 0; c < d; ++c) {
                    dvj[c] += pij * dO[i * d + c];
                    dkj[c] += scale * dsij * Q[i * d + c];
                }
            }
        }
    }
    if (!failed && lse_out)
        memcpy(lse_out, lse, sizeof(double) * (size_t)total);
    if (!failed && delta_out)
        memcpy(delta_out, D, sizeof(double) * (size_t)total);
    free(lse);
    free(D);
    return failed ? -1 : 0;
}

/* Number of OpenMP threads the oracle uses by default. */
int oracle_max_threads(void) { return omp_get_max_threads(); }
