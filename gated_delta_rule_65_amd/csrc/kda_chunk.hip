// Chunked gated delta-rule forward pass for gfx950.
//
// Recurrence ("Kimi K3 Open Model Surpasses Closed GPT and Anthropic Systems on
// Independent Benchmarks", worldcybernews, second paragraph; read as the gated
// delta rule with a per-key-channel forget gate):
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t,
//     a_t = exp(clamp(g_t, -5, 0)).
// The third paragraph of that page describes processing the tokens of a chunk in
// parallel and carrying the state across chunks.  Multiplying the recurrence out
// over a chunk of C = 64 tokens (G = running sum of clamped g inside the chunk,
// gamma_r = exp(G_r) per key channel) gives, exactly up to rounding:
//     A_ri = b_r sum_c k_rc k_ic e^{G_rc - G_ic}   (i < r)      M = I + A
//     P_ri =     sum_c q_rc k_ic e^{G_rc - G_ic}   (i <= r)
//     U  = M^{-1} Diag(b) (V - (gamma*K) S)                     (C x Dv)
//     O  = (gamma*Q) S + P U
//     S' = Diag(gamma_C) S + (e^{G_C - G} * K)^T U
// Columns of S evolve independently, so a workgroup owns a 32-column slice of
// one head's state and walks its chunks in order; all contractions run on MFMA.
//
// Exponent range.  The clamp bounds every g by 5 in magnitude, so inside a
// 16-token sub-block the running sum stays within [-80, 0] and e^{+-80} is a
// normal float (and bf16).  Every factor is therefore formed relative to a
// sub-block boundary: per element E = e^{Gloc} and 1/E, per sub-block and
// channel the decays between boundaries; no exponent ever exceeds 80 in size,
// and a factor that underflows multiplies a quantity that is itself below
// e^-87.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kSlice = 32;  // state columns per workgroup

template <int DK>
struct ChunkLds {
    static constexpr int PK = DK + 4;  // padded row of DK floats
    static constexpr int P64 = 68;     // padded row of 64 floats
    static constexpr int PV = 36;      // padded row of the value slice
    static constexpr int S = 0;                          // S^T       [32][PK]
    static constexpr int KBT = S + kSlice * PK;          // Kbar^T    [DK][P64]
    static constexpr int COL = KBT + DK * P64;           // k*F rows of sub-blocks 0..2 [48][PK]
    static constexpr int A = COL + 48 * PK;              // b_r * A   [64][P64]
    static constexpr int T = A + 64 * P64;               // M^{-1}    [64][P64]
    static constexpr int P = T + 64 * P64;               // P         [64][P64]
    static constexpr int X = P + 64 * P64;               // (b(V-KS))^T [32][P64]
    static constexpr int U = X + kSlice * P64;           // U^T       [32][P64]
    static constexpr int V = U + kSlice * P64;           // V slice   [64][PV]
    static constexpr int GT = V + kChunk * PV;           // sub-block sums of g [4][DK]
    static constexpr int GC = GT + 4 * DK;               // gamma_C   [DK]
    static constexpr int BETA = GC + DK;                 // b         [64]
    static constexpr int TOTAL = BETA + kChunk;
    // decay tables, overlaid on X/U (free until the chain step)
    static constexpr int TPW = X;           // e^{sum_{J<w} Gt_J}  [4][DK]
    static constexpr int TAF = TPW + 4 * DK;  // e^{sum_{J>w} Gt_J}  [4][DK]
    static constexpr int TBT = TAF + 4 * DK;  // e^{Gt_w}            [4][DK]
    static constexpr int TD = TBT + 4 * DK;   // e^{sum_{I<J<R} Gt_J} for (I,R) = (0,2),(1,3),(0,3)  [3][DK]
    static_assert(TD + 3 * DK <= V, "decay tables overflow");
    static constexpr int Z = COL;             // solve temporaries [3][16][17], overlaid on COL
    static_assert(3 * 16 * 17 <= 48 * PK, "solve scratch overflow");
    static_assert(TOTAL * 4 <= 160 * 1024, "LDS budget");
};

template <int DK, bool F32>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, const void* __restrict__ vv,
    const float* __restrict__ g, const float* __restrict__ beta, const float* s0, float* __restrict__ o,
    float* s_final, const int32_t* __restrict__ cu_seqlens, int64_t T_fixed, int64_t total, int64_t N, int H,
    int Dv) {
    using In = typename std::conditional<F32, float, uint16_t>::type;
    using Fr = Frag<F32>;
    using L = ChunkLds<DK>;
    constexpr int KS = DK / 32;   // 32-wide reduction steps over the key dimension
    constexpr int CBW = DK / 64;  // 16-row channel blocks of S owned by each wave
    constexpr int PK = L::PK, P64 = L::P64, PV = L::PV;

    const In* __restrict__ q = static_cast<const In*>(qv);
    const In* __restrict__ k = static_cast<const In*>(kv);
    const In* __restrict__ v = static_cast<const In*>(vv);

    __shared__ __align__(16) float smem[L::TOTAL];
    float* sS = smem + L::S;
    float* sKbT = smem + L::KBT;
    float* sCol = smem + L::COL;
    float* sA = smem + L::A;
    float* sT = smem + L::T;
    float* sP = smem + L::P;
    float* sX = smem + L::X;
    float* sU = smem + L::U;
    float* sV = smem + L::V;
    float* sGt = smem + L::GT;
    float* sGC = smem + L::GC;
    float* sBeta = smem + L::BETA;
    float* tPw = smem + L::TPW;
    float* tAf = smem + L::TAF;
    float* tBt = smem + L::TBT;
    float* tD = smem + L::TD;
    float* sZ = smem + L::Z;

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;

    // Workgroup -> (sequence, head, column slice).  Workgroups are handed to the
    // 8 XCDs round-robin; all slices of one (sequence, head) get the same XCD so
    // that their identical q/k/g reads hit that XCD's L2.
    const int NS = Dv / kSlice;
    const int64_t pairs = N * (int64_t)H;
    const int64_t bid = blockIdx.x;
    const int64_t loc = bid >> 3;
    const int sl = (int)(loc % NS);
    const int64_t pr = (loc / NS) * 8 + (bid & 7);
    if (pr >= pairs) return;
    const int64_t n = pr / H;
    const int h = (int)(pr % H);
    int64_t start, end;
    if (cu_seqlens) {
        start = min<int64_t>(max<int64_t>(cu_seqlens[n], 0), total);
        end = min<int64_t>(max<int64_t>(cu_seqlens[n + 1], start), total);
    } else {
        start = n * T_fixed;
        end = start + T_fixed;
    }
    const int col0 = sl * kSlice;

    // Zero T and P once: their blocks above the diagonal are never written.
    for (int e = tid; e < 64 * P64; e += 256) {
        sT[e] = 0.f;
        sP[e] = 0.f;
    }

    // ---- initial state: wave w owns channel blocks cb = w*CBW + i, both 16-column halves
    f32x4_t accS[CBW][2];
#pragma unroll
    for (int ci = 0; ci < CBW; ++ci) {
        const int cb = w * CBW + ci;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c = 16 * cb + 4 * cg + jj;
                accS[ci][nb][jj] = s0 ? s0[((n * H + h) * DK + c) * (int64_t)Dv + col0 + 16 * nb + m] : 0.f;
            }
            *reinterpret_cast<float4*>(&sS[(16 * nb + m) * PK + 16 * cb + 4 * cg]) =
                make_float4(accS[ci][nb][0], accS[ci][nb][1], accS[ci][nb][2], accS[ci][nb][3]);
        }
    }
    __syncthreads();

    const int r = 16 * w + m;  // this lane's token row inside the chunk (phase A layout)

    for (int64_t t0 = start; t0 < end; t0 += kChunk) {
        const int nt = (int)min<int64_t>(kChunk, end - t0);
        const bool rv = r < nt;

        // ---------------- phase A: loads, clamp, sub-block prefix sums of g
        float qf[KS][8], kf[KS][8], gl[KS][8];
        {
            const int64_t base = ((t0 + r) * H + h) * (int64_t)DK;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                if (rv) {
                    load8_as_float(q + base + 32 * s + 8 * cg, qf[s]);
                    load8_as_float(k + base + 32 * s + 8 * cg, kf[s]);
                    load8_as_float(g + base + 32 * s + 8 * cg, gl[s]);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) qf[s][j] = kf[s][j] = gl[s][j] = 0.f;
                }
            }
        }
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                gl[s][j] = row16_inclusive_scan(fminf(fmaxf(gl[s][j], -5.f), 0.f));
        if (m == 15) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float* dst = &sGt[w * DK + 32 * s + 8 * cg];
                *reinterpret_cast<float4*>(dst) = make_float4(gl[s][0], gl[s][1], gl[s][2], gl[s][3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(gl[s][4], gl[s][5], gl[s][6], gl[s][7]);
            }
        }
        {   // value slice [64 tokens][32 columns] and beta
            const int vr = tid >> 2, vc = (tid & 3) * 8;
            float vx[8];
            if (vr < nt) {
                load8_as_float(v + ((t0 + vr) * H + h) * (int64_t)Dv + col0 + vc, vx);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) vx[j] = 0.f;
            }
            *reinterpret_cast<float4*>(&sV[vr * PV + vc]) = make_float4(vx[0], vx[1], vx[2], vx[3]);
            *reinterpret_cast<float4*>(&sV[vr * PV + vc + 4]) = make_float4(vx[4], vx[5], vx[6], vx[7]);
            if (tid < kChunk) sBeta[tid] = tid < nt ? beta[(t0 + tid) * H + h] : 0.f;
        }
        __syncthreads();

        // ---------------- decay tables per (sub-block, channel)
        if (tid < DK) {
            const int c = tid;
            const float G0 = sGt[c], G1 = sGt[DK + c], G2 = sGt[2 * DK + c], G3 = sGt[3 * DK + c];
            tPw[c] = 1.f;
            tPw[DK + c] = __expf(G0);
            tPw[2 * DK + c] = __expf(G0 + G1);
            tPw[3 * DK + c] = __expf(G0 + G1 + G2);
            tAf[c] = __expf(G1 + G2 + G3);
            tAf[DK + c] = __expf(G2 + G3);
            tAf[2 * DK + c] = __expf(G3);
            tAf[3 * DK + c] = 1.f;
            tBt[c] = __expf(G0);
            tBt[DK + c] = __expf(G1);
            tBt[2 * DK + c] = __expf(G2);
            tBt[3 * DK + c] = __expf(G3);
            tD[c] = __expf(G1);            // (I=0, R=2)
            tD[DK + c] = __expf(G2);       // (I=1, R=3)
            tD[2 * DK + c] = __expf(G1 + G2);  // (I=0, R=3)
            sGC[c] = __expf(G0 + G1 + G2 + G3);
        }
        __syncthreads();

        // ---------------- per-element factors and operands (rows of sub-block w)
        Fr fQt[KS], fKt[KS], fqE[KS], fkE[KS], fkd[KS];
        float qE[KS][8], kE[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int c0 = 32 * s + 8 * cg;
            float pw[8], af[8], bt[8];
            lds_read8(&tPw[w * DK + c0], pw);
            lds_read8(&tAf[w * DK + c0], af);
            lds_read8(&tBt[w * DK + c0], bt);
            float xq[8], xk[8], xkd[8], xkf[8], xkb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float E = __expf(gl[s][j]);    // e^{G_r - G_start(w)} in [e^-80, 1]
                const float Ei = __expf(-gl[s][j]);  // its inverse, <= e^80
                const float gam = pw[j] * E;         // e^{G_r}
                const float F = bt[j] * Ei;          // e^{G_end(w) - G_r} in [e^-80, 1]
                xq[j] = qf[s][j] * gam;
                xk[j] = kf[s][j] * gam;
                qE[s][j] = qf[s][j] * E;
                kE[s][j] = kf[s][j] * E;
                xkd[j] = kf[s][j] * Ei;
                xkf[j] = kf[s][j] * F;
                xkb[j] = kf[s][j] * (af[j] * F);     // e^{G_C - G_r} k_r
            }
            fQt[s].set(xq);
            fKt[s].set_hi_only(xk);
            fqE[s].set(qE[s]);
            fkE[s].set_hi_only(kE[s]);
            fkd[s].set(xkd);
            if (w < 3) {
                float* dst = &sCol[r * PK + c0];
                *reinterpret_cast<float4*>(dst) = make_float4(xkf[0], xkf[1], xkf[2], xkf[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(xkf[4], xkf[5], xkf[6], xkf[7]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) sKbT[(c0 + j) * P64 + r] = xkb[j];
        }
        __syncthreads();

        // ---------------- decay-folded Gram blocks (w, I), I <= w
        for (int I = 0; I <= w; ++I) {
            f32x4_t accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
            if (I == w) {
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    accA = mma_fast(accA, fkE[s], fkd[s]);
                    accP = mma_full(accP, fqE[s], fkd[s]);
                }
            } else {
                const int dsel = (w - I == 2) ? (I == 0 ? 0 : 1) : 2;  // only read when w - I >= 2
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int c0 = 32 * s + 8 * cg;
                    float cx[8];
                    lds_read8(&sCol[(16 * I + m) * PK + c0], cx);
                    Fr colf;
                    colf.set(cx);
                    if (w - I >= 2) {
                        float d[8], rk[8], rq[8];
                        lds_read8(&tD[dsel * DK + c0], d);
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            rk[j] = kE[s][j] * d[j];
                            rq[j] = qE[s][j] * d[j];
                        }
                        Fr rkf, rqf;
                        rkf.set_hi_only(rk);
                        rqf.set(rq);
                        accA = mma_fast(accA, rkf, colf);
                        accP = mma_full(accP, rqf, colf);
                    } else {
                        accA = mma_fast(accA, fkE[s], colf);
                        accP = mma_full(accP, fqE[s], colf);
                    }
                }
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 4 * cg + jj;  // row inside the sub-block
                const int gr = 16 * w + rr, gi = 16 * I + m;
                float a = accA[jj], pv = accP[jj];
                if (I == w) {
                    if (m >= rr) a = 0.f;
                    if (m > rr) pv = 0.f;
                }
                sA[gr * P64 + gi] = a * sBeta[gr];
                sP[gr * P64 + gi] = pv;
            }
        }
        __syncthreads();

        // ---------------- M^{-1} = (I + A)^{-1}: diagonal sub-blocks by forward substitution
        if (lane < 16) {
            const int cidx = lane;
            const float* Ab = &sA[(16 * w) * P64 + 16 * w];
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < rr; ++j) acc = fmaf(Ab[rr * P64 + j], x[j], acc);
                x[rr] = (rr == cidx) ? 1.f : (rr < cidx ? 0.f : -acc);
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) sT[(16 * w + rr) * P64 + 16 * w + cidx] = x[rr];
        }
        __syncthreads();
        // off-diagonal sub-blocks, by distance d = R - I:
        //   N_RI = -N_RR * sum_{J=I}^{R-1} A_RJ N_JI
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            const int nblk = 4 - d;
            for (int e = tid; e < nblk * 256; e += 256) {
                const int b = e >> 8, i = (e >> 4) & 15, j = e & 15;
                const int R = d + b, I = R - d;
                float acc = 0.f;
                for (int J = I; J < R; ++J)
#pragma unroll
                    for (int kk = 0; kk < 16; ++kk)
                        acc = fmaf(sA[(16 * R + i) * P64 + 16 * J + kk], sT[(16 * J + kk) * P64 + 16 * I + j], acc);
                sZ[(b * 16 + i) * 17 + j] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nblk * 256; e += 256) {
                const int b = e >> 8, i = (e >> 4) & 15, j = e & 15;
                const int R = d + b, I = R - d;
                float acc = 0.f;
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    acc = fmaf(sT[(16 * R + i) * P64 + 16 * R + kk], sZ[(b * 16 + kk) * 17 + j], acc);
                sT[(16 * R + i) * P64 + 16 * I + j] = -acc;
            }
            __syncthreads();
        }

        // ---------------- chain 1: X = b (V - Kt S), O1 = Qt S
        f32x4_t accO[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x4_t accX = {0.f, 0.f, 0.f, 0.f};
            accO[nb] = accX;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float sx[8];
                lds_read8(&sS[(16 * nb + m) * PK + 32 * s + 8 * cg], sx);
                Fr sf;
                sf.set(sx);
                accX = mma_fast(accX, fKt[s], sf);
                accO[nb] = mma_full(accO[nb], fQt[s], sf);
            }
            float xv[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 16 * w + 4 * cg + jj;
                xv[jj] = sBeta[rr] * (sV[rr * PV + 16 * nb + m] - accX[jj]);
            }
            *reinterpret_cast<float4*>(&sX[(16 * nb + m) * P64 + 16 * w + 4 * cg]) =
                make_float4(xv[0], xv[1], xv[2], xv[3]);
        }
        __syncthreads();

        // ---------------- chain 2: U = M^{-1} X   (rows of sub-block w)
        const int nk = (w >= 2) ? 2 : 1;  // 32-token steps that reach the diagonal
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x4_t accU = {0.f, 0.f, 0.f, 0.f};
            for (int kb = 0; kb < nk; ++kb) {
                float tx[8], xx[8];
                lds_read8(&sT[(16 * w + m) * P64 + 32 * kb + 8 * cg], tx);
                lds_read8(&sX[(16 * nb + m) * P64 + 32 * kb + 8 * cg], xx);
                Fr tf, xf;
                tf.set(tx);
                xf.set(xx);
                accU = mma_full(accU, tf, xf);
            }
            *reinterpret_cast<float4*>(&sU[(16 * nb + m) * P64 + 16 * w + 4 * cg]) =
                make_float4(accU[0], accU[1], accU[2], accU[3]);
        }
        __syncthreads();

        // ---------------- chain 3: O = O1 + P U (store), S = gamma_C S + Kbar^T U
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x4_t acc = accO[nb];
            for (int kb = 0; kb < nk; ++kb) {
                float px[8], ux[8];
                lds_read8(&sP[(16 * w + m) * P64 + 32 * kb + 8 * cg], px);
                lds_read8(&sU[(16 * nb + m) * P64 + 32 * kb + 8 * cg], ux);
                Fr pf, uf;
                pf.set(px);
                uf.set(ux);
                acc = mma_full(acc, pf, uf);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 16 * w + 4 * cg + jj;
                if (rr < nt) o[((t0 + rr) * H + h) * (int64_t)Dv + col0 + 16 * nb + m] = acc[jj];
            }
        }
#pragma unroll
        for (int ci = 0; ci < CBW; ++ci) {
            const int cb = w * CBW + ci;
            float gc[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) gc[jj] = sGC[16 * cb + 4 * cg + jj];
            Fr af[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float kx[8];
                lds_read8(&sKbT[(16 * cb + m) * P64 + 32 * kb + 8 * cg], kx);
                af[kb].set(kx);
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                f32x4_t acc;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[jj] = accS[ci][nb][jj] * gc[jj];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    float ux[8];
                    lds_read8(&sU[(16 * nb + m) * P64 + 32 * kb + 8 * cg], ux);
                    Fr uf;
                    uf.set(ux);
                    acc = mma_full(acc, af[kb], uf);
                }
                accS[ci][nb] = acc;
                *reinterpret_cast<float4*>(&sS[(16 * nb + m) * PK + 16 * cb + 4 * cg]) =
                    make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }
        __syncthreads();
    }

    if (s_final) {
#pragma unroll
        for (int ci = 0; ci < CBW; ++ci) {
            const int cb = w * CBW + ci;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int c = 16 * cb + 4 * cg + jj;
                    s_final[((n * H + h) * DK + c) * (int64_t)Dv + col0 + 16 * nb + m] = accS[ci][nb][jj];
                }
        }
    }
}

int64_t chunk_grid_size(int64_t N, int H, int Dv) {
    const int64_t pairs = N * (int64_t)H;
    return ((pairs + 7) / 8) * 8 * (Dv / kSlice);
}

template <int DK, bool F32>
static hipError_t launch_dk(const ChunkArgs& a, hipStream_t st) {
    const int64_t grid = chunk_grid_size(a.N, a.H, a.Dv);
    hipLaunchKernelGGL((chunk_fwd_kernel<DK, F32>), dim3((unsigned)grid), dim3(256), 0, st, a.q, a.k, a.v, a.g,
                       a.beta, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t st) {
    if (a.Dk == 128) return a.f32 ? launch_dk<128, true>(a, st) : launch_dk<128, false>(a, st);
    return a.f32 ? launch_dk<64, true>(a, st) : launch_dk<64, false>(a, st);
}

}  // namespace kda
