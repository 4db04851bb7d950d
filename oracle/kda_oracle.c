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

/*
 * Gradients of the same recurrence (reverse mode, written out by hand from the forward steps
 * above; the pages give no backward pass).  For a loss L with dL/do = d_o and dL/dS_T = d_sfinal
 * (NULL = 0), per token t from last to first, with dS = dL/dS_t:
 *     dS += q_t do_t^T;               dq_t = S_t do_t
 *     du = dS^T k_t;                  dk_t = dS u_t                 (S_t = S~ + k_t u_t^T)
 *     dbeta_t = du . (v_t - w);       dv_t = beta_t du;  dw = -beta_t du
 *     dS~ = dS + k_t dw^T;            dk_t += S~ dw                 (w = S~^T k_t)
 *     dalpha_i = sum_j dS~_ij S_{t-1,ij};  dS_{t-1} = Diag(alpha) dS~   (S~ = Diag(alpha) S_{t-1})
 *     dg_i = dalpha_i alpha_i if -5 <= g_i <= 0, else 0   (the clamp passes the gradient on [-5, 0])
 * and ds0 = dS after the first token.  States are recomputed from checkpoints every
 * ORACLE_CKPT tokens with the forward steps above (the same operations, so the same values).
 *
 * q, k, g: [total, H, Dk]; v: [total, H, Dv]; beta: [total, H] (double);
 * s0: [N, H, Dk, Dv] or NULL; d_o: [total, H, Dv]; d_sfinal: [N, H, Dk, Dv] or NULL;
 * outputs dq, dk, dg: [total, H, Dk]; dv: [total, H, Dv]; dbeta: [total, H]; ds0: [N, H, Dk, Dv].
 */
#define ORACLE_CKPT 64

/* one forward token step on the full state; keeps alpha, w, u for the backward step */
static void oracle_step(const double* qt, const double* kt, const double* vt, const double* gt, double bt,
                        double* S, int64_t Dk, int64_t Dv, double* alpha, double* w, double* u) {
    (void)qt;
    for (int64_t i = 0; i < Dk; ++i) alpha[i] = forget_gate(gt[i]);
    for (int64_t i = 0; i < Dk; ++i)
        for (int64_t j = 0; j < Dv; ++j) S[i * Dv + j] *= alpha[i];
    for (int64_t j = 0; j < Dv; ++j) w[j] = 0.0;
    for (int64_t i = 0; i < Dk; ++i)
        for (int64_t j = 0; j < Dv; ++j) w[j] += kt[i] * S[i * Dv + j];
    for (int64_t j = 0; j < Dv; ++j) u[j] = bt * (vt[j] - w[j]);
    for (int64_t i = 0; i < Dk; ++i)
        for (int64_t j = 0; j < Dv; ++j) S[i * Dv + j] += kt[i] * u[j];
}

int kda_oracle_backward(const double* q, const double* k, const double* v, const double* g, const double* beta,
                        const double* s0, const double* d_o, const double* d_sfinal, const int64_t* cu_seqlens,
                        int64_t N, int64_t H, int64_t Dk, int64_t Dv, double* dq, double* dk, double* dv,
                        double* dg, double* dbeta, double* ds0, int nthreads) {
    if (N < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || !cu_seqlens) return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    int64_t ntask = N * H;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t task = 0; task < ntask; ++task) {
        int64_t n = task / H, h = task % H;
        int64_t t0 = cu_seqlens[n], T = cu_seqlens[n + 1] - t0;
        int64_t nck = (T + ORACLE_CKPT - 1) / ORACLE_CKPT;
        size_t SS = (size_t)(Dk * Dv);
        double* ck = (double*)malloc(sizeof(double) * SS * (size_t)(nck > 0 ? nck : 1));
        double* blk = (double*)malloc(sizeof(double) * SS * (ORACLE_CKPT + 1));
        double* dS = (double*)malloc(sizeof(double) * SS);
        double* dSt = (double*)malloc(sizeof(double) * SS);
        double* al = (double*)malloc(sizeof(double) * (size_t)Dk * ORACLE_CKPT);
        double* wv = (double*)malloc(sizeof(double) * (size_t)Dv * ORACLE_CKPT);
        double* uv = (double*)malloc(sizeof(double) * (size_t)Dv * ORACLE_CKPT);
        double* du = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* dw = (double*)malloc(sizeof(double) * (size_t)Dv);
        if (!ck || !blk || !dS || !dSt || !al || !wv || !uv || !du || !dw) {
            free(ck); free(blk); free(dS); free(dSt); free(al); free(wv); free(uv); free(du); free(dw);
#ifdef _OPENMP
#pragma omp atomic write
#endif
            bad = 1;
            continue;
        }
        /* forward: checkpoints of the state at tokens 0, CKPT, 2 CKPT, ... */
        double* S = blk;
        for (size_t e = 0; e < SS; ++e) S[e] = s0 ? s0[(n * H + h) * SS + e] : 0.0;
        for (int64_t t = 0; t < T; ++t) {
            if (t % ORACLE_CKPT == 0) memcpy(ck + (t / ORACLE_CKPT) * SS, S, sizeof(double) * SS);
            int64_t tt = t0 + t;
            oracle_step(q + (tt * H + h) * Dk, k + (tt * H + h) * Dk, v + (tt * H + h) * Dv,
                        g + (tt * H + h) * Dk, beta[tt * H + h], S, Dk, Dv, al, wv, uv);
        }
        /* backward */
        for (size_t e = 0; e < SS; ++e) dS[e] = d_sfinal ? d_sfinal[(n * H + h) * SS + e] : 0.0;
        for (int64_t b = nck - 1; b >= 0; --b) {
            int64_t tb = b * ORACLE_CKPT, nb = T - tb < ORACLE_CKPT ? T - tb : ORACLE_CKPT;
            /* states S_{tb} .. S_{tb+nb} of this block: blk[s] = state after s tokens of the block */
            memcpy(blk, ck + b * SS, sizeof(double) * SS);
            for (int64_t s = 0; s < nb; ++s) {
                int64_t tt = t0 + tb + s;
                memcpy(blk + (s + 1) * SS, blk + s * SS, sizeof(double) * SS);
                oracle_step(q + (tt * H + h) * Dk, k + (tt * H + h) * Dk, v + (tt * H + h) * Dv,
                            g + (tt * H + h) * Dk, beta[tt * H + h], blk + (s + 1) * SS, Dk, Dv,
                            al + s * Dk, wv + s * Dv, uv + s * Dv);
            }
            for (int64_t s = nb - 1; s >= 0; --s) {
                int64_t tt = t0 + tb + s;
                const double* qt = q + (tt * H + h) * Dk;
                const double* kt = k + (tt * H + h) * Dk;
                const double* vt = v + (tt * H + h) * Dv;
                const double* gt = g + (tt * H + h) * Dk;
                const double* dot = d_o + (tt * H + h) * Dv;
                double bt = beta[tt * H + h];
                const double* Sprev = blk + s * SS;       /* S_{t-1} */
                const double* Scur = blk + (s + 1) * SS;  /* S_t */
                const double* a = al + s * Dk;
                const double* w = wv + s * Dv;
                const double* u = uv + s * Dv;
                double* dqt = dq + (tt * H + h) * Dk;
                double* dkt = dk + (tt * H + h) * Dk;
                double* dvt = dv + (tt * H + h) * Dv;
                double* dgt = dg + (tt * H + h) * Dk;
                /* read-out o_t = S_t^T q_t */
                for (int64_t i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < Dv; ++j) {
                        dS[i * Dv + j] += qt[i] * dot[j];
                        acc += Scur[i * Dv + j] * dot[j];
                    }
                    dqt[i] = acc;
                }
                /* write S_t = S~ + k u^T */
                for (int64_t j = 0; j < Dv; ++j) du[j] = 0.0;
                for (int64_t i = 0; i < Dk; ++i) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < Dv; ++j) {
                        du[j] += dS[i * Dv + j] * kt[i];
                        acc += dS[i * Dv + j] * u[j];
                    }
                    dkt[i] = acc;
                }
                /* u = beta (v - w) */
                double db = 0.0;
                for (int64_t j = 0; j < Dv; ++j) {
                    db += du[j] * (vt[j] - w[j]);
                    dvt[j] = bt * du[j];
                    dw[j] = -bt * du[j];
                }
                dbeta[tt * H + h] = db;
                /* w = S~^T k, S~ = Diag(alpha) S_{t-1} */
                for (int64_t i = 0; i < Dk; ++i) {
                    double acc = 0.0, da = 0.0;
                    for (int64_t j = 0; j < Dv; ++j) {
                        double St = a[i] * Sprev[i * Dv + j];
                        double d = dS[i * Dv + j] + kt[i] * dw[j];
                        acc += St * dw[j];
                        da += d * Sprev[i * Dv + j];
                        dSt[i * Dv + j] = a[i] * d;
                    }
                    dkt[i] += acc;
                    dgt[i] = (gt[i] >= -5.0 && gt[i] <= 0.0) ? da * a[i] : 0.0;
                }
                memcpy(dS, dSt, sizeof(double) * SS);
            }
        }
        if (ds0)
            memcpy(ds0 + (n * H + h) * SS, dS, sizeof(double) * SS);
        free(ck); free(blk); free(dS); free(dSt); free(al); free(wv); free(uv); free(du); free(dw);
    }
    return bad ? -2 : 0;
}
