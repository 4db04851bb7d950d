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
//
// Work split inside a workgroup (4 waves, one per SIMD): wave w owns tokens
// 16w..16w+15 of the chunk for the per-element work and the Gram rows, column
// block w of M^{-1}, and channel rows 32w..32w+31 (16w..16w+15 for Dk=64) of the
// state.  The next chunk's inputs are loaded into registers while the current
// chunk is computed.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kSlice = 32;  // state columns per workgroup

template <int DK, bool F32>
struct ChunkLds {
    using MS = LMat<F32, kSlice, DK>;   // S^T          [n][c]
    using MKB = LMat<F32, DK, kChunk>;  // Kbar^T       [c][t]
    using MCOL = LMat<true, 48, DK>;    // fp32 k * e^{G_end(blk) - G}, sub-blocks 0..2  [t][c]
    using MN = LMat<F32, 64, 64>;       // M^{-1}       [t][t]
    using MP = LMat<F32, 64, 64>;       // P            [t][t]
    using MX = LMat<F32, kSlice, 64>;   // (b (V - Kt S))^T  [n][t]
    using MU = LMat<F32, kSlice, 64>;   // U^T          [n][t]
    static constexpr int S = 0;
    static constexpr int KB = S + MS::BYTES;
    static constexpr int COL = KB + MKB::BYTES;
    static constexpr int N = COL + MCOL::BYTES;
    static constexpr int P = N + MN::BYTES;
    static constexpr int X = P + MP::BYTES;
    static constexpr int U = X + MX::BYTES;
    static constexpr int A = U;                       // fp32 b_r A_ri [64][68], shares space with U
    static constexpr int UA_BYTES = (MU::BYTES > 64 * 68 * 4) ? MU::BYTES : 64 * 68 * 4;
    static constexpr int D = U + UA_BYTES;            // fp32 diagonal inverses [4][16][17]
    static constexpr int TAB = D + 4 * 16 * 17 * 4;   // fp32 decay tables [15][DK]
    static constexpr int GT = TAB + 15 * DK * 4;      // fp32 sub-block sums of g (log2 units) [4][DK]
    static constexpr int GC = GT + 4 * DK * 4;        // fp32 gamma_C [DK]
    static constexpr int BETA = GC + DK * 4;          // fp32 b [64]
    static constexpr int TOTAL = BETA + 64 * 4;
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
    // rows of sub-block 3 as Gram row operands (q e^{Gloc}, k e^{Gloc}) for the waves that take
    // Gram blocks (3,0) and (3,1); they live in the M^{-1} planes, which are free until the
    // inverse is formed
    using MR = LMat<F32, 16, DK>;
    static constexpr int RQ = N;
    static constexpr int RK = N + MR::BYTES;
    static_assert(2 * MR::BYTES <= MN::BYTES, "row-operand overlay");
};

// Row block W of a chunk (rows 16W..16W+15), one pass over the key channels:
//   Gram blocks:  A_ri = b_r sum_c kE_rc col_ic (one pass, strictly lower in the diagonal block),
//                 P_ri = sum_c qE_rc col_ic (full precision, lower in the diagonal block),
//     with kE = k e^{Gloc}, qE = q e^{Gloc}; col = k e^{-Gloc} on the diagonal block, and for a
//     block I below it the LDS rows k_i e^{G_end(I) - G_i} times e^{G_start(R) - G_end(I)}
//     (both factors <= 1);
//   chain 1:  X = b (V - Kt S) (one pass), O1 = Qt S (full), with Qt = q e^{G}, Kt = k e^{G}.
// The ten Gram blocks are shared out 2/3/3/2: wave 3 keeps (3,2) and (3,3); blocks (3,0) and
// (3,1) go to waves 0 and 1, which read sub-block 3's row operands from LDS.
// X goes to LDS (transposed, for U = M^{-1} X), A and P to LDS, O1 stays in accO.
template <int W, int DK, bool F32>
__device__ __forceinline__ void gram_chain1(const Raw8<F32>* pq, const Raw8<F32>* pk, const float (*E)[8],
                                            const float (*Ei)[8], const float* tPw, const char* pCol,
                                            const float* tD, const char* pS, const char* pRQ, const char* pRK,
                                            const float* sBeta, const float (*vD)[4], float* sA, char* pP,
                                            char* pX, f32x4_t* accO, float rq, float rk, int m, int cg) {
    using Fr = Frag<F32>;
    constexpr int KS = DK / 32;
    constexpr int IMIN = (W == 3) ? 2 : 0;  // first own Gram block of this row block
    constexpr bool FOREIGN = (W < 2);       // also takes block (3, W)
    f32x4_t accA[W + 1], accP[W + 1], accX[2], accAf, accPf;
#pragma unroll
    for (int I = 0; I <= W; ++I) accA[I] = accP[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    accAf = accPf = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) accX[nb] = accO[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int c0 = 32 * s + 8 * cg;
        float qf[8], kf[8], pw[8], x1[8], x2[8], x3[8];
        raw8_to_float<F32>(pq[s], qf);
        raw8_to_float<F32>(pk[s], kf);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            qf[j] *= rq;
            kf[j] *= rk;
        }
        lds_read8(&tPw[W * DK + c0], pw);
        Fr fqE, fkE, fkd, fQt, fKt;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x1[j] = qf[j] * E[s][j];
            x2[j] = kf[j] * E[s][j];
            x3[j] = kf[j] * Ei[s][j];
        }
        fqE.set(x1);
        fkE.set_hi_only(x2);
        fkd.set(x3);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x1[j] *= pw[j];  // q e^{G}
            x2[j] *= pw[j];  // k e^{G}
        }
        fQt.set(x1);
        fKt.set_hi_only(x2);
        // chain 1
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            const Fr sf = lds_frag<F32, kSlice, DK>(pS, 16 * nb + m, c0);
            accX[nb] = mma_fast(accX[nb], fKt, sf);
            accO[nb] = mma_full(accO[nb], fQt, sf);
        }
        // own Gram blocks below the diagonal
#pragma unroll
        for (int I = IMIN; I < W; ++I) {
            float cx[8];
            lds_read8(reinterpret_cast<const float*>(pCol) + (16 * I + m) * (DK + 4) + c0, cx);
            if constexpr (W >= 2) {
                if (W - I >= 2) {
                    const int dsel = (W - I == 3) ? 2 : I;  // (0,2)->0, (1,3)->1, (0,3)->2
                    float d[8];
                    lds_read8(&tD[dsel * DK + c0], d);
#pragma unroll
                    for (int j = 0; j < 8; ++j) cx[j] *= d[j];
                }
            }
            Fr colf;
            colf.set(cx);
            accA[I] = mma_fast(accA[I], fkE, colf);
            accP[I] = mma_full(accP[I], fqE, colf);
        }
        // diagonal block
        accA[W] = mma_fast(accA[W], fkE, fkd);
        accP[W] = mma_full(accP[W], fqE, fkd);
        // block (3, W) with sub-block 3's row operands
        if constexpr (FOREIGN) {
            float cx[8], d[8];
            lds_read8(reinterpret_cast<const float*>(pCol) + (16 * W + m) * (DK + 4) + c0, cx);
            lds_read8(&tD[(W == 0 ? 2 : 1) * DK + c0], d);  // e^{G_start(3) - G_end(W)}
#pragma unroll
            for (int j = 0; j < 8; ++j) cx[j] *= d[j];
            Fr colf;
            colf.set(cx);
            const Fr rq = lds_frag<F32, 16, DK>(pRQ, m, c0);
            const Fr rk = lds_frag<F32, 16, DK>(pRK, m, c0);
            accAf = mma_fast(accAf, rk, colf);
            accPf = mma_full(accPf, rq, colf);
        }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        f32x4_t xv;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int rr = 16 * W + 4 * cg + jj;
            xv[jj] = sBeta[rr] * (vD[nb][jj] - accX[nb][jj]);
        }
        lds_store4<F32, kSlice, 64>(pX, 16 * nb + m, 16 * W + 4 * cg, xv);
    }
#pragma unroll
    for (int I = IMIN; I <= W; ++I) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int rr = 4 * cg + jj;  // row inside the sub-block
            const int gr = 16 * W + rr, gi = 16 * I + m;
            float a = accA[I][jj], pv = accP[I][jj];
            if (I == W) {
                if (m >= rr) a = 0.f;
                if (m > rr) pv = 0.f;
            }
            sA[gr * 68 + gi] = a * sBeta[gr];
            lds_store1<F32, 64, 64>(pP, gr, gi, pv);
        }
    }
    if constexpr (FOREIGN) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int gr = 48 + 4 * cg + jj, gi = 16 * W + m;
            sA[gr * 68 + gi] = accAf[jj] * sBeta[gr];
            lds_store1<F32, 64, 64>(pP, gr, gi, accPf[jj]);
        }
    }
}

template <int DK, bool F32, bool PRO>
__global__ __launch_bounds__(256, 1) void chunk_fwd_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, const void* __restrict__ vv,
    const void* __restrict__ gv, const void* __restrict__ bv, const float* s0, float* __restrict__ o,
    float* s_final, const int32_t* __restrict__ cu_seqlens, int64_t T_fixed, int64_t total, int64_t N, int H,
    int Dv, Prologue pro) {
    // input prologue; PRO = false compiles the plain form (fp32 log alpha and beta, q and k as given)
    const Prologue pf{PRO && pro.g_bf16, PRO && pro.g_logit, PRO && pro.b_bf16, PRO && pro.b_logit,
                      PRO && pro.l2norm};
    using In = typename std::conditional<F32, float, uint16_t>::type;
    using Fr = Frag<F32>;
    using L = ChunkLds<DK, F32>;
    constexpr int KS = DK / 32;   // 32-wide reduction steps over the key dimension
    constexpr int CBW = DK / 64;  // 16-row channel blocks of S owned by each wave

    const In* __restrict__ q = static_cast<const In*>(qv);
    const In* __restrict__ k = static_cast<const In*>(kv);
    const In* __restrict__ v = static_cast<const In*>(vv);

    __shared__ __align__(16) char smem[L::TOTAL];
    char* pS = smem + L::S;
    char* pKB = smem + L::KB;
    char* pCol = smem + L::COL;
    char* pN = smem + L::N;
    char* pP = smem + L::P;
    char* pX = smem + L::X;
    char* pU = smem + L::U;
    float* sA = reinterpret_cast<float*>(smem + L::A);
    float* sD = reinterpret_cast<float*>(smem + L::D);
    float* tPw = reinterpret_cast<float*>(smem + L::TAB);  // e^{sum_{J<w} Gt_J}      [4][DK]
    float* tAf = tPw + 4 * DK;                              // e^{sum_{J>w} Gt_J}      [4][DK]
    float* tBt = tAf + 4 * DK;                              // e^{Gt_w}                [4][DK]
    float* tD = tBt + 4 * DK;                               // e^{sum_{I<J<R} Gt_J}, (I,R) = (0,2),(1,3),(0,3)
    float* sGt = reinterpret_cast<float*>(smem + L::GT);
    float* sGC = reinterpret_cast<float*>(smem + L::GC);
    float* sBeta = reinterpret_cast<float*>(smem + L::BETA);

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

    // M^{-1} and P are lower triangular: zero their planes once, the blocks above
    // the diagonal are never written.
    lds_zero<F32, 64, 64>(pN, tid, 256);
    lds_zero<F32, 64, 64>(pP, tid, 256);

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
            lds_store4<F32, kSlice, DK>(pS, 16 * nb + m, 16 * cb + 4 * cg, accS[ci][nb]);
        }
    }

    const int r = 16 * w + m;  // this lane's token row inside the chunk (per-element layout)

    // ---- prefetch registers: this lane's q/k/g row pieces, its 8 entries of the value
    // slice in MFMA result layout (rows 16w+4cg+jj, column 16nb+m), one beta.  Rows past
    // the end of the sequence are loaded from its last row (always valid memory) and
    // zeroed when consumed, so no load has to be waited for before it is used.
    Raw8<F32> pq[KS], pk[KS];
    Raw8<true> pg[KS];
    In pv[2][4];
    float pb = 0.f;
    // The next chunk's loads are issued in four parts spread over the current chunk,
    // so that the waves of all workgroups do not hit the memory system in one burst.
    // Addresses: a per-lane pointer fixed for the whole sequence plus a 64-bit chunk offset
    // (wave-uniform) plus a 32-bit row offset (row < 64, row stride < 2^25 elements).
    const uint32_t rs_k = (uint32_t)H * DK, rs_v = (uint32_t)H * (uint32_t)Dv;
    const In* __restrict__ q_l = q + (int64_t)h * DK + 8 * cg;
    const In* __restrict__ k_l = k + (int64_t)h * DK + 8 * cg;
    const int64_t g_l = (int64_t)h * DK + 8 * cg;  // element offset into g (fp32 or bf16)
    const In* __restrict__ v_l = v + (int64_t)h * Dv + col0 + m;

    float* __restrict__ o_l = o + (int64_t)h * Dv + col0 + m;
    auto prefetch_part = [&](int part, int64_t t0, int nt) {
        const int64_t cq = t0 * (int64_t)rs_k;
        const uint32_t rq = (uint32_t)min(r, nt - 1) * rs_k;
        if (part == 0) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const int64_t e = g_l + cq + rq + 32 * s;
                if (pf.g_bf16) pg[s].a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(gv) + e);
                else load_raw8(static_cast<const float*>(gv) + e, pg[s]);
            }
        } else if (part == 1) {
#pragma unroll
            for (int s = 0; s < KS; ++s) load_raw8(k_l + cq + rq + 32 * s, pk[s]);
        } else if (part == 2) {
#pragma unroll
            for (int s = 0; s < KS; ++s) load_raw8(q_l + cq + rq + 32 * s, pq[s]);
        } else {
            const int64_t cv = t0 * (int64_t)rs_v;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint32_t rv = (uint32_t)min(16 * w + 4 * cg + jj, nt - 1) * rs_v;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) pv[nb][jj] = v_l[cv + rv + 16 * nb];
            }
            pb = load1_gate(bv, t0 * H + h + (uint32_t)min(tid & 63, nt - 1) * (uint32_t)H, pf.b_bf16);
        }
    };
    auto prefetch = [&](int64_t t0, int nt) {
        for (int part = 0; part < 4; ++part) prefetch_part(part, t0, nt);
    };
    if (start < end) prefetch(start, (int)min<int64_t>(kChunk, end - start));
    lds_barrier();

    f32x4_t oPrev[2];  // output rows of the last chunk computed (rows 16w+4cg+jj, column 16nb+m)
    auto store_o = [&](int64_t tc, int ntc) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 16 * w + 4 * cg + jj;
                if (rr < ntc) o_l[tc * (int64_t)rs_v + (uint32_t)rr * rs_v + 16 * nb] = oPrev[nb][jj];
            }
    };

    for (int64_t t0 = start; t0 < end; t0 += kChunk) {
        const int nt = (int)min<int64_t>(kChunk, end - t0);

        // ---------------- phase A: take the prefetched chunk (rows >= nt contribute nothing:
        // q = k = v = 0, g = 0, beta = 0)
        const bool rv = r < nt;
        // next chunk to prefetch; on the last chunk the current one is read again, so the
        // loads need no branch (which would cost exact wait counts on the loads in flight)
        const bool more = t0 + kChunk < end;
        const int64_t t0_next = more ? t0 + kChunk : t0;
        const int nt_next = more ? (int)min<int64_t>(kChunk, end - t0 - kChunk) : nt;
        float gl[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s) {  // clamped log alpha in log2 units; 0 past the end
            if (pf.g_bf16) {
                Raw8<false> t;
                t.a = pg[s].a;
                raw8_to_float<false>(t, gl[s]);
            } else {
                raw8_to_float<true>(pg[s], gl[s]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) gl[s][j] = rv ? gate_log2(gl[s][j], pf.g_logit) : 0.f;
        }
        float vD[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float x;
                if constexpr (F32) x = pv[nb][jj];
                else x = bf16_bits_to_float(pv[nb][jj]);
                vD[nb][jj] = (16 * w + 4 * cg + jj < nt) ? x : 0.f;
            }
        const float bval = (tid < nt) ? beta_value(pb, pf.b_logit) : 0.f;
        if (tid < kChunk) sBeta[tid] = bval;
        prefetch_part(3, t0_next, nt_next);  // v and beta of the next chunk

        // inclusive sums over each 16-token sub-block
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int j = 0; j < 8; ++j) gl[s][j] = row16_inclusive_scan(gl[s][j]);
        if (m == 15) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float* dst = &sGt[w * DK + 32 * s + 8 * cg];
                *reinterpret_cast<float4*>(dst) = make_float4(gl[s][0], gl[s][1], gl[s][2], gl[s][3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(gl[s][4], gl[s][5], gl[s][6], gl[s][7]);
            }
        }
        lds_barrier();  // (1)

        // ---------------- decay tables per (sub-block, channel)
        if (tid < DK) {
            const int c = tid;
            const float G0 = sGt[c], G1 = sGt[DK + c], G2 = sGt[2 * DK + c], G3 = sGt[3 * DK + c];
            tPw[c] = 1.f;
            tPw[DK + c] = __builtin_amdgcn_exp2f(G0);
            tPw[2 * DK + c] = __builtin_amdgcn_exp2f(G0 + G1);
            tPw[3 * DK + c] = __builtin_amdgcn_exp2f(G0 + G1 + G2);
            tAf[c] = __builtin_amdgcn_exp2f(G1 + G2 + G3);
            tAf[DK + c] = __builtin_amdgcn_exp2f(G2 + G3);
            tAf[2 * DK + c] = __builtin_amdgcn_exp2f(G3);
            tAf[3 * DK + c] = 1.f;
            tBt[c] = __builtin_amdgcn_exp2f(G0);
            tBt[DK + c] = __builtin_amdgcn_exp2f(G1);
            tBt[2 * DK + c] = __builtin_amdgcn_exp2f(G2);
            tBt[3 * DK + c] = __builtin_amdgcn_exp2f(G3);
            tD[c] = __builtin_amdgcn_exp2f(G1);                 // (I=0, R=2)
            tD[DK + c] = __builtin_amdgcn_exp2f(G2);            // (I=1, R=3)
            tD[2 * DK + c] = __builtin_amdgcn_exp2f(G1 + G2);   // (I=0, R=3)
            sGC[c] = __builtin_amdgcn_exp2f(G0 + G1 + G2 + G3);
        }
        lds_barrier();  // (2)

        // ---------------- per-element decay factors; column operands of the Gram blocks below
        // the diagonal and Kbar^T go to LDS.  Rows past the end of the sequence need no
        // masking beyond g = 0 and b = 0: their rows of A are zero, so their rows of
        // M^{-1} are unit rows and their pseudo-values U = b(V - Kt S) = 0.
        float rq = 1.f, rk = 1.f;  // 1/||q_r||, 1/||k_r|| when q and k are scaled to unit length
        if (pf.l2norm) {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float qf[8], kf[8];
                raw8_to_float<F32>(pq[s], qf);
                raw8_to_float<F32>(pk[s], kf);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    sq = fmaf(qf[j], qf[j], sq);
                    sk = fmaf(kf[j], kf[j], sk);
                }
            }
            rq = rnorm_lanes4(sq);
            rk = rnorm_lanes4(sk);
        }
        float Ei[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int c0 = 32 * s + 8 * cg;
            float af[8], bt[8], kf[8], xkf[8], xkb[8];
            lds_read8(&tAf[w * DK + c0], af);
            lds_read8(&tBt[w * DK + c0], bt);
            raw8_to_float<F32>(pk[s], kf);
#pragma unroll
            for (int j = 0; j < 8; ++j) kf[j] *= rk;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float E = __builtin_amdgcn_exp2f(gl[s][j]);   // e^{G_r - G_start(w)} in [e^-80, 1]
                Ei[s][j] = __builtin_amdgcn_exp2f(-gl[s][j]);       // its inverse, <= e^80
                gl[s][j] = E;
                xkf[j] = kf[j] * (bt[j] * Ei[s][j]);                // k e^{G_end(w) - G_r}, factor in [e^-80, 1]
                xkb[j] = xkf[j] * af[j];                            // k e^{G_C - G_r}
            }
            if (w < 3) {
                lds_store8<true, 48, DK>(pCol, r, c0, xkf);
            } else {
                float qf[8], xqe[8], xke[8];
                raw8_to_float<F32>(pq[s], qf);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    xqe[j] = (qf[j] * rq) * gl[s][j];
                    xke[j] = kf[j] * gl[s][j];
                }
                lds_store8<F32, 16, DK>(smem + L::RQ, m, c0, xqe);
                lds_store8<F32, 16, DK>(smem + L::RK, m, c0, xke);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) lds_store1<F32, DK, kChunk>(pKB, c0 + j, r, xkb[j]);
        }
        // output rows of the previous chunk, kept in registers until this chunk's inputs
        // have been consumed, so that later waits on loads never have to count these stores
        if (t0 > start) store_o(t0 - kChunk, kChunk);
        lds_barrier();  // (3)

        // ---------------- Gram row block w and chain 1, sharing one pass over the key channels:
        //   A = b (kE . col^T) strictly lower (one pass), P = qE . col^T lower (full),
        //   X = b (V - Kt S) (one pass), O1 = Qt S (full).
        // Each wave runs a copy specialised for its sub-block so that its independent
        // accumulations interleave.
        f32x4_t accO[2];
        switch (w) {
            case 0: gram_chain1<0, DK, F32>(pq, pk, gl, Ei, tPw, pCol, tD, pS, smem + L::RQ, smem + L::RK, sBeta, vD, sA, pP, pX, accO, rq, rk, m, cg); break;
            case 1: gram_chain1<1, DK, F32>(pq, pk, gl, Ei, tPw, pCol, tD, pS, smem + L::RQ, smem + L::RK, sBeta, vD, sA, pP, pX, accO, rq, rk, m, cg); break;
            case 2: gram_chain1<2, DK, F32>(pq, pk, gl, Ei, tPw, pCol, tD, pS, smem + L::RQ, smem + L::RK, sBeta, vD, sA, pP, pX, accO, rq, rk, m, cg); break;
            default: gram_chain1<3, DK, F32>(pq, pk, gl, Ei, tPw, pCol, tD, pS, smem + L::RQ, smem + L::RK, sBeta, vD, sA, pP, pX, accO, rq, rk, m, cg); break;
        }

        lds_barrier();  // (4)
        prefetch_part(0, t0_next, nt_next);  // g of the next chunk


        // ---------------- diagonal blocks of M^{-1} = (I + A)^{-1}: forward substitution,
        // one column per lane (lanes 0..15 of wave w, block w)
        if (lane < 16) {
            const int cidx = lane;
            const float* Ab = &sA[(16 * w) * 68 + 16 * w];
            float x[16];
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < rr; ++j) acc[j & 3] = fmaf(Ab[rr * 68 + j], x[j], acc[j & 3]);
                const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
                x[rr] = (rr == cidx) ? 1.f : (rr < cidx ? 0.f : -sum);
            }
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) sD[(w * 16 + rr) * 17 + cidx] = x[rr];
        }
        lds_barrier();  // (5)
        prefetch_part(1, t0_next, nt_next);  // k of the next chunk

        // ---------------- column block I = w of M^{-1}:  N_II = D_I,
        //   N_RI = -D_R sum_{J=I}^{R-1} A_RJ N_JI,  R = I+1..3  (fp32 MFMA, 16x16x4).
        // A 16x16 result in registers (lane: column m, rows 4cg..4cg+3) is used
        // directly as the B operand of the next product, reduction index 4cg+j
        // in MFMA number j.
        {
            const int I = w;
            // blocks above the diagonal were overwritten by the row-operand overlay: zero them
#pragma unroll
            for (int R = 0; R < 3; ++R) {
                if (R >= I) continue;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) lds_store1<F32, 64, 64>(pN, 16 * R + 4 * cg + jj, 16 * I + m, 0.f);
            }
            f32x4_t Nr[4];
#pragma unroll
            for (int R = 0; R < 4; ++R) Nr[R] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                if (R < I) continue;
                f32x4_t nv;
                if (R == I) {
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) nv[jj] = sD[(I * 16 + 4 * cg + jj) * 17 + m];
                } else {
                    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int J = 0; J < 3; ++J) {
                        if (J < I || J >= R) continue;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            z = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * R + m) * 68 + 16 * J + 4 * cg + j],
                                                                     Nr[J][j], z, 0, 0, 0);
                    }
                    f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sD[(R * 16 + m) * 17 + 4 * cg + j], z[j], y, 0, 0,
                                                                 0);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) nv[jj] = -y[jj];
                }
                Nr[R] = nv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) lds_store1<F32, 64, 64>(pN, 16 * R + 4 * cg + jj, 16 * I + m, nv[jj]);
            }
        }
        lds_barrier();  // (6)
        prefetch_part(2, t0_next, nt_next);  // q of the next chunk

        // ---------------- chain 2: U = M^{-1} X   (rows of sub-block w)
        const int nk = (w >= 2) ? 2 : 1;  // 32-token steps that reach the diagonal
        {
            f32x4_t accU[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb >= nk) continue;
                const Fr tf = lds_frag<F32, 64, 64>(pN, 16 * w + m, 32 * kb + 8 * cg);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const Fr xf = lds_frag<F32, kSlice, 64>(pX, 16 * nb + m, 32 * kb + 8 * cg);
                    accU[nb] = mma_full(accU[nb], tf, xf);
                }
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) lds_store4<F32, kSlice, 64>(pU, 16 * nb + m, 16 * w + 4 * cg, accU[nb]);
        }
        lds_barrier();  // (8)

        // ---------------- chain 3: O = O1 + P U (store), S = gamma_C S + Kbar^T U
        {
            Fr uf[2][2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) uf[nb][kb] = lds_frag<F32, kSlice, 64>(pU, 16 * nb + m, 32 * kb + 8 * cg);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb >= nk) continue;
                const Fr pf = lds_frag<F32, 64, 64>(pP, 16 * w + m, 32 * kb + 8 * cg);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) accO[nb] = mma_full(accO[nb], pf, uf[nb][kb]);
            }
#pragma unroll
            for (int ci = 0; ci < CBW; ++ci) {
                const int cb = w * CBW + ci;
                float gc[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) gc[jj] = sGC[16 * cb + 4 * cg + jj];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) accS[ci][nb][jj] *= gc[jj];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const Fr af = lds_frag<F32, DK, kChunk>(pKB, 16 * cb + m, 32 * kb + 8 * cg);
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) accS[ci][nb] = mma_full(accS[ci][nb], af, uf[nb][kb]);
                }
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) lds_store4<F32, kSlice, DK>(pS, 16 * nb + m, 16 * cb + 4 * cg, accS[ci][nb]);
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) oPrev[nb] = accO[nb];
        }
        lds_barrier();  // (9)
    }
    if (start < end) {
        const int64_t t_last = start + ((end - start - 1) / kChunk) * kChunk;
        store_o(t_last, (int)(end - t_last));
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
    if (any_prologue(a.pro))
        hipLaunchKernelGGL((chunk_fwd_kernel<DK, F32, true>), dim3((unsigned)grid), dim3(256), 0, st, a.q, a.k, a.v,
                           a.g, a.beta, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv, a.pro);
    else
        hipLaunchKernelGGL((chunk_fwd_kernel<DK, F32, false>), dim3((unsigned)grid), dim3(256), 0, st, a.q, a.k, a.v,
                           a.g, a.beta, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv, a.pro);
    return hipGetLastError();
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t st) {
    if (a.Dk == 128) return a.f32 ? launch_dk<128, true>(a, st) : launch_dk<128, false>(a, st);
    return a.f32 ? launch_dk<64, true>(a, st) : launch_dk<64, false>(a, st);
}

}  // namespace kda
