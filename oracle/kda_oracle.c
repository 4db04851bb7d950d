/*
 * CPU ORACLE for the gated delta-rule (Kimi Delta Attention) forward pass.
 * TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
 * baseline call this; the product path never does.
 *
 * Plain fp64, token by token, no blocking and no reordering beyond what the
 * definition states.  What it computes (per sequence n and head h):
 *
 *   The state is a fixed-size matrix S (d_k x d_v) that takes the place of a
 *   growing key/value cache, updated token by token by the delta rule; beta
 *   sets how strongly a token writes and alpha how much of the state is
 *   forgotten, and alpha is clamped to [e^-5, 1]
 *   ("Kimi K3 Open Model Surpasses Closed GPT and Anthropic Systems on
 *   Independent Benchmarks", worldcybernews, second paragraph).
 *
 *   Reading of that description used here (the gated delta rule with a
 *   per-key-channel forget gate applied before the delta correction):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 *   with alpha_t = exp(clamp(g_t, -5, 0)) per key channel, g = log alpha given
 *   as input, and beta_t one scalar per (token, head).  Evaluated as
 *     S <- Diag(alpha_t) S;  w = S^T k_t;  S <- S + k_t (beta_t (v_t - w))^T;
 *     o_t = S^T q_t,
 *   which is the same matrix expression multiplied out.
 *
 * Columns of S evolve independently (column j of S_t depends only on column j
 * of S_{t-1} and on v_t[j]), so the oracle can compute any subset of d_v
 * columns exactly; that is how full-size workloads are sampled.
 *
 * Threads split the work over (sequence, head, block of columns); every task
 * runs the plain recurrence on its own columns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_COL_BLOCK 16

/* alpha = exp(clamp(g, -5, 0)): the forget gate kept inside [e^-5, 1]. */
static double forget_gate(double g) {
    double x = g;
    if (x < -5.0) x = -5.0;
    if (x > 0.0) x = 0.0;
    return exp(x);
}

/*
 * q, k: [total, H, Dk] double; v: [total, H, Dv] double;
 * g: [total, H, Dk] double (log alpha, clamped here); beta: [total, H] double;
 * s0: [N, H, Dk, Dv] double or NULL (zero state);
 * cu_seqlens: [N+1] int64, sequence n covers tokens cu[n] .. cu[n+1]-1;
 * cols: [ncols] d_v column indices to compute (each in [0, Dv));
 * o: [total, H, ncols] double; s_final: [N, H, Dk, ncols] double or NULL.
 * Returns 0, or -1 on a bad argument.
 */
int kda_oracle_forward(const double* q, const double* k, const double* v, const double* g, const double* beta,
                       const double* s0, const int64_t* cu_seqlens, int64_t N, int64_t H, int64_t Dk,
                       int64_t Dv, const int32_t* cols, int64_t ncols, double* o, double* s_final,
                       int nthreads) {
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || ncols < 0 || !cu_seqlens || (ncols > 0 && !cols)) return -1;
    for (int64_t c = 0; c < ncols; ++c)
        if (cols[c] < 0 || cols[c] >= Dv) return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (ncols == 0 || N == 0) return 0;

    int64_t nblk = (ncols + ORACLE_COL_BLOCK - 1) / ORACLE_COL_BLOCK;
    int64_t ntask = N * H * nblk;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
        int64_t n = task / (H * nblk);
        int64_t h = (task / nblk) % H;
        int64_t b = task % nblk;
        int64_t c0 = b * ORACLE_COL_BLOCK;
        int64_t nc = ncols - c0 < ORACLE_COL_BLOCK ? ncols - c0 : ORACLE_COL_BLOCK;

        double* S = (double*)malloc(sizeof(double) * (size_t)(Dk * nc));
        double* alpha = (double*)malloc(sizeof(double) * (size_t)Dk);
        double w[ORACLE_COL_BLOCK], u[ORACLE_COL_BLOCK];
        if (!S || !alpha) {
            free(S); free(alpha);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
            continue;
        }
        /* S <- S0 (or zero) */
        for (int64_t i = 0; i < Dk; ++i)
            for (int64_t j = 0; j < nc; ++j)
                S[i * nc + j] = s0 ? s0[((n * H + h) * Dk + i) * Dv + cols[c0 + j]] : 0.0;

        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const double* qt = q + (t * H + h) * Dk;
            const double* kt = k + (t * H + h) * Dk;
            const double* vt = v + (t * H + h) * Dv;
            const double* gt = g + (t * H + h) * Dk;
            double bt = (double)beta[t * H + h];
            for (int64_t i = 0; i < Dk; ++i) alpha[i] = forget_gate(gt[i]);
            /* forget: S <- Diag(alpha) S */
            for (int64_t i = 0; i < Dk; ++i)
                for (int64_t j = 0; j < nc; ++j) S[i * nc + j] *= alpha[i];
            /* prediction of v from the decayed state: w = S^T k */
            for (int64_t j = 0; j < nc; ++j) w[j] = 0.0;
            for (int64_t i = 0; i < Dk; ++i)
                for (int64_t j = 0; j < nc; ++j) w[j] += (double)kt[i] * S[i * nc + j];
            /* delta write: S <- S + k (beta (v - w))^T */
            for (int64_t j = 0; j < nc; ++j) u[j] = bt * ((double)vt[cols[c0 + j]] - w[j]);
            for (int64_t i = 0; i < Dk; ++i)
                for (int64_t j = 0; j < nc; ++j) S[i * nc + j] += (double)kt[i] * u[j];
            /* read-out from the updated state: o = S^T q */
            double* ot = o + (t * H + h) * ncols + c0;
            for (int64_t j = 0; j < nc; ++j) ot[j] = 0.0;
            for (int64_t i = 0; i < Dk; ++i)
                for (int64_t j = 0; j < nc; ++j) ot[j] += (double)qt[i] * S[i * nc + j];
        }
        if (s_final)
            for (int64_t i = 0; i < Dk; ++i)
                for (int64_t j = 0; j < nc; ++j)
                    s_final[((n * H + h) * Dk + i) * ncols + c0 + j] = S[i * nc + j];
        free(S);
        free(alpha);
    }
    return bad ? -2 : 0;
}

int kda_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
