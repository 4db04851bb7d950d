// Two-kernel chunked forward pass for gfx950 (used when the caller passes a workspace).
//
// The chunked form of the gated delta rule ("Kimi K3 Open Model Surpasses Closed
// GPT and Anthropic Systems on Independent Benchmarks", worldcybernews, second and
// third paragraphs; kda_chunk.hip derives the equations) splits into work that
// does not depend on the carried state S and a short state-dependent chain.  With
// G the running sum of the clamped gates inside a chunk (log2 units), Qt = e^G q,
// Kt = e^G k, Kbar = e^{G_C - G} k, M = I + A and P the decay-folded Gram blocks:
//
//   per chunk, state independent:  Qt, Kt, Kbar^T, M^{-1} Diag(b), P, gamma_C = e^{G_C}
//   per chunk, state dependent:    X = V - Kt S,  U = M^{-1} Diag(b) X,
//                                  O = Qt S + P U,  S' = Diag(gamma_C) S + Kbar^T U
//
// prep_kernel computes the first line for every (chunk, head) at once, one
// workgroup each and two per CU, and stores the operands in MFMA fragment order:
// each stored fragment is one 1 KiB plane per 64 lanes, so every load of the chain
// kernel is a fully contiguous 1 KiB request.  chain_kernel walks the chunks of one
// (sequence, head, 32-column slice) in order and only runs the products of the
// second line, with three workgroup barriers per chunk; each chunk's operands are
// loaded during the previous chunk, once the products that read the registers they
// replace have completed (the Qt steps right after their last read).  The backward
// pass's state-only form (mode 3) stores B = Kbar^T M^{-1} Diag(b) in Kbar^T's place
// and updates S' = Diag(gamma_C) S + B X, so U leaves the carried chain: two
// barriers per chunk.
#include <algorithm>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC = 64;  // tokens per chunk
constexpr int kS = 32;  // state columns per chain workgroup
constexpr int kChainThreads = 512;  // chain workgroup: eight waves

// ---------------------------------------------------------------------------- fragments in HBM
// A fragment (eight values per lane, see Frag) is stored as two planes of
// 64 lanes x 16 B: bf16 hi and bf16 lo (split policy) or fp32 values 0-3 and
// 4-7 (fp32 policy).  A hi-only fragment of the split policy has one plane.
// Records are written with non-temporal stores: they are read back only after the
// whole preparation pass, and write-back of cached record lines would otherwise
// overlap the chain kernel's reads.
constexpr int kPlane = 1024;

template <bool F32>
__device__ __forceinline__ void gfrag_store(char* grp, int lane, const Frag<F32>& f) {
    if constexpr (F32) {
        __builtin_nontemporal_store(f32x4_t{f.v[0], f.v[1], f.v[2], f.v[3]}, reinterpret_cast<f32x4_t*>(grp + lane * 16));
        __builtin_nontemporal_store(f32x4_t{f.v[4], f.v[5], f.v[6], f.v[7]},
                                    reinterpret_cast<f32x4_t*>(grp + kPlane + lane * 16));
    } else {
        __builtin_nontemporal_store(f.hi, reinterpret_cast<bf16x8_t*>(grp + lane * 16));
        __builtin_nontemporal_store(f.lo, reinterpret_cast<bf16x8_t*>(grp + kPlane + lane * 16));
    }
}

template <bool F32>
__device__ __forceinline__ void gfrag_store_hi(char* grp, int lane, const Frag<F32>& f) {
    if constexpr (F32) gfrag_store<true>(grp, lane, f);
    else __builtin_nontemporal_store(f.hi, reinterpret_cast<bf16x8_t*>(grp + lane * 16));
}

template <bool F32>
__device__ __forceinline__ Frag<F32> gfrag_load(const char* grp, int lane) {
    Frag<F32> f;
    if constexpr (F32) {
        const float4 a = *reinterpret_cast<const float4*>(grp + lane * 16);
        const float4 b = *reinterpret_cast<const float4*>(grp + kPlane + lane * 16);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    } else {
        f.hi = *reinterpret_cast<const bf16x8_t*>(grp + lane * 16);
        f.lo = *reinterpret_cast<const bf16x8_t*>(grp + kPlane + lane * 16);
    }
    return f;
}

// Split policy: only the hi plane (the fragment feeds one-pass products only).
template <bool F32>
__device__ __forceinline__ Frag<F32> gfrag_load_hi(const char* grp, int lane) {
    if constexpr (F32) {
        return gfrag_load<true>(grp, lane);
    } else {
        Frag<false> f;
        f.hi = *reinterpret_cast<const bf16x8_t*>(grp + lane * 16);
        f.lo = f.hi;  // never read by a one-pass product
        return f;
    }
}

// Row blocks of M^{-1} and P are lower triangular: row block w (16 rows) meets
// 32-wide column steps kb < nk(w); the six (w, kb) pairs are stored in order.
__host__ __device__ constexpr int steps_of(int w) { return w >= 2 ? 2 : 1; }
__host__ __device__ constexpr int pair_of(int w, int kb) { return w < 2 ? w : 2 * w - 2 + kb; }

// Operand record of one (chunk, head): byte offsets of its parts.  KT2: Kt has both planes (the fp32
// policy, and the split policy of the backward's state pass, whose products all run in full precision).
template <int DK, bool F32, bool KT2 = F32>
struct Rec {
    static constexpr int KS = DK / 32;                      // 32-channel steps
    static constexpr int KT_PLANES = KT2 ? 2 : 1;
    static constexpr int64_t QT = 0;                        // Qt rows:    [w 4][s KS], 2 planes
    static constexpr int64_t KT = QT + 4 * KS * 2 * kPlane;  // Kt rows:    [w 4][s KS], KT_PLANES
    static constexpr int64_t KB = KT + 4 * KS * KT_PLANES * kPlane;  // Kbar^T rows (B = Kbar^T M^{-1} Diag(b) in
                                                                     // the backward's records): [c-block DK/16][kb 2], 2 planes
    static constexpr int64_t NM = KB + (DK / 16) * 2 * 2 * kPlane;   // M^{-1} Diag(b): [pair 6], 2 planes
    static constexpr int64_t PM = NM + 6 * 2 * kPlane;               // P:            [pair 6], 2 planes
    static constexpr int64_t GC = PM + 6 * 2 * kPlane;               // gamma_C fp32 [DK]
    static constexpr int64_t BYTES = GC + DK * 4;
    static_assert(BYTES % 256 == 0, "records stay 256-byte aligned");
};

struct SeqRange {
    int64_t start, end;
};

// Tokens of sequence n: from the offsets, or T_fixed tokens starting at n * T_stride (T_stride =
// T_fixed for a whole batch; larger when a call covers a window of each sequence).
__device__ __forceinline__ SeqRange seq_range(const int32_t* cu, int64_t n, int64_t T_fixed, int64_t T_stride,
                                              int64_t total) {
    SeqRange s;
    if (cu) {
        s.start = min<int64_t>(max<int64_t>(cu[n], 0), total);
        s.end = min<int64_t>(max<int64_t>(cu[n + 1], s.start), total);
    } else {
        s.start = n * T_stride;
        s.end = s.start + T_fixed;
    }
    return s;
}

// Chunk slot of chunk j of sequence n: n * ceil(T/64) + j for equal lengths;
// floor(cu[n]/64) + n + j for packed sequences (unique, below floor(total/64) + N).
__device__ __forceinline__ int64_t slot_of(const int32_t* cu, int64_t n, int64_t j, int64_t T_fixed, int64_t start) {
    if (cu) return start / kC + n + j;
    return n * ((T_fixed + kC - 1) / kC) + j;
}

}  // namespace

// ============================================================================ prep kernel

template <int DK, bool F32>
struct PrepLds {
    using MKB = LMat<F32, DK, kC>;                       // Kbar^T staging [c][t]
    static constexpr int COL = 0;                         // fp32 Gram column operands, sub-blocks 0..2 [48][DK+4]
    static constexpr int PM = COL + 48 * (DK + 4) * 4;    // fp32 P [64][68]
    static constexpr int KB = 0;                          // Kbar^T, over COL and PM once both are read
    static constexpr int A0 = PM + 64 * 68 * 4;
    static constexpr int A = A0 > MKB::BYTES ? A0 : MKB::BYTES;  // fp32 b_r A_ri [64][68], then M^{-1} Diag(b)
    static constexpr int D = A + 64 * 68 * 4;             // fp32 diagonal inverses [4][16][17]
    static constexpr int TAB = D + 4 * 16 * 17 * 4;       // fp32 tables [15][DK]
    static constexpr int GT = TAB + 15 * DK * 4;          // fp32 sub-block sums (log2) [4][DK]
    static constexpr int BETA = GT + 4 * DK * 4;          // fp32 b [64]
    static constexpr int TOTAL = BETA + 64 * 4;
    static_assert(TOTAL <= 80 * 1024, "two prep workgroups per CU");
};

// Gram row block W (rows 16W..16W+15), all column blocks I <= W: A (one pass) into sA,
// scaled by b_r and strictly lower on the diagonal block; P (full precision) into sP,
// lower with diagonal; blocks I > W of both are zero.
// gAbar (backward form only): the unscaled strictly lower A, row-major [64][64]; the blocks right of
// the diagonal block are not written (their readers take them as zero).
template <int W, int DK, bool F32, bool BWD>
__device__ __forceinline__ void prep_gram(const float (*qf)[8], const float (*kf)[8], const float (*E)[8],
                                          const float (*Ei)[8], const float* sCol, const float* tD,
                                          const float* sBeta, float* sA, float* sP, float* gAbar, int m, int cg) {
    using Fr = Frag<F32>;
    constexpr int KS = DK / 32;
    f32x4_t accA[W + 1], accP[W + 1];
#pragma unroll
    for (int I = 0; I <= W; ++I) accA[I] = accP[I] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int c0 = 32 * s + 8 * cg;
        float x1[8], x2[8], x3[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            x1[j] = qf[s][j] * E[s][j];
            x2[j] = kf[s][j] * E[s][j];
            x3[j] = kf[s][j] * Ei[s][j];
        }
        Fr fqE, fkE, fkd;
        fqE.set(x1);
        if constexpr (BWD) fkE.set(x2);
        else fkE.set_hi_only(x2);
        fkd.set(x3);
#pragma unroll
        for (int I = 0; I < W; ++I) {
            float cx[8];
            lds_read8(sCol + (16 * I + m) * (DK + 4) + c0, cx);
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
            accA[I] = BWD ? mma_full(accA[I], fkE, colf) : mma_fast(accA[I], fkE, colf);
            accP[I] = mma_full(accP[I], fqE, colf);
        }
        accA[W] = BWD ? mma_full(accA[W], fkE, fkd) : mma_fast(accA[W], fkE, fkd);
        accP[W] = mma_full(accP[W], fqE, fkd);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int rr = 4 * cg + jj;
            const int gr = 16 * W + rr, gi = 16 * I + m;
            float a = 0.f, pv = 0.f;
            if (I <= W) {
                a = accA[I][jj];
                pv = accP[I][jj];
                if (I == W) {
                    if (m >= rr) a = 0.f;
                    if (m > rr) pv = 0.f;
                }
            }
            sA[gr * 68 + gi] = a * sBeta[gr];
            sP[gr * 68 + gi] = pv;
            if constexpr (BWD) {
                if (I <= W) gAbar[gr * 64 + gi] = a;
            }
        }
    }
}

// F32: precision policy of the records (fp32 MFMA operands, else split bf16); IN_F32: q/k input type.
// BWD: also write the backward pass's operands (BwdRec: the reverse chain's fragments, the gradient kernel's
// fp32 operands) to brecs, and leave out the Qt and P fragments of the record (only the state-only chain
// reads these records).
template <int DK, bool F32, bool PRO, bool IN_F32 = F32, bool BWD = false>
__global__ __launch_bounds__(256, 2) void prep_kernel(const void* __restrict__ qv, const void* __restrict__ kv,
                                                      const void* __restrict__ gv, const void* __restrict__ bv,
                                                      const int32_t* __restrict__ cu_seqlens, int64_t T_fixed,
                                                      int64_t T_stride, int64_t total, int64_t N, int H, Prologue pro,
                                                      char* __restrict__ ws, float* __restrict__ brecs = nullptr) {
    using In = typename std::conditional<IN_F32, float, uint16_t>::type;
    using Fr = Frag<F32>;
    using L = PrepLds<DK, F32>;
    // input prologue; PRO = false compiles the plain form (fp32 log alpha and beta, q and k as given)
    const Prologue pf{PRO && pro.g_bf16, PRO && pro.g_logit, PRO && pro.b_bf16, PRO && pro.b_logit,
                      PRO && pro.l2norm};
    using R = Rec<DK, F32, F32 || BWD>;
    constexpr int KS = DK / 32;
    const In* __restrict__ q = static_cast<const In*>(qv);
    const In* __restrict__ k = static_cast<const In*>(kv);

    __shared__ __align__(16) char smem[L::TOTAL];
    float* sCol = reinterpret_cast<float*>(smem + L::COL);
    float* sP = reinterpret_cast<float*>(smem + L::PM);
    char* pKB = smem + L::KB;
    float* sA = reinterpret_cast<float*>(smem + L::A);
    float* sD = reinterpret_cast<float*>(smem + L::D);
    float* tPw = reinterpret_cast<float*>(smem + L::TAB);   // e^{sum_{J<w} Gt_J}     [4][DK]
    float* tBt = tPw + 4 * DK;                              // e^{Gt_w}               [4][DK]
    float* tD = tBt + 4 * DK;                               // e^{sum_{I<J<R} Gt_J}   [3][DK]
    float* tAf = tD + 3 * DK;                               // e^{sum_{J>w} Gt_J}     [4][DK]
    float* sGt = reinterpret_cast<float*>(smem + L::GT);
    float* sBeta = reinterpret_cast<float*>(smem + L::BETA);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);

    // (slot) -> (sequence n, chunk j)
    int64_t n, j;
    if (cu_seqlens) {
        int64_t lo = 0, hi = N - 1;  // largest n with floor(cu[n]/64) + n <= slot
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            const int64_t f = min<int64_t>(max<int64_t>(cu_seqlens[mid], 0), total) / kC + mid;
            if (f <= slot) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        j = slot - (min<int64_t>(max<int64_t>(cu_seqlens[n], 0), total) / kC + n);
    } else {
        const int64_t nch = (T_fixed + kC - 1) / kC;
        n = slot / nch;
        j = slot % nch;
    }
    const SeqRange sr = seq_range(cu_seqlens, n, T_fixed, T_stride, total);
    const int64_t t0 = sr.start + j * kC;
    if (j < 0 || t0 >= sr.end) return;  // unused slot
    const int nt = (int)min<int64_t>(kC, sr.end - t0);
    char* rec = ws + (slot * H + h) * R::BYTES;
    using BR = BwdRec<DK>;
    float* brec = BWD ? brecs + (slot * H + h) * (int64_t)BR::FLOATS : nullptr;

    // ---- rows of sub-block w; running gate sums inside the sub-block (log2)
    const int r = 16 * w + m;
    const bool rv = r < nt;
    const int64_t base = ((t0 + min(r, nt - 1)) * H + h) * (int64_t)DK + 8 * cg;
    // beta first: its LDS store then waits for this one load, not for the rows below
    float braw = 0.f;
    if (tid < kC) braw = load1_gate(bv, (t0 + min(tid, nt - 1)) * H + h, pf.b_bf16);
    // the gates first: the running sums below start while q and k are still arriving
    float qf[KS][8], kf[KS][8], gl[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) load8_gate(gv, base + 32 * s, pf.g_bf16, gl[s]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        load8_as_float(q + base + 32 * s, qf[s]);
        load8_as_float(k + base + 32 * s, kf[s]);
    }
    if (tid < kC) sBeta[tid] = tid < nt ? beta_value(braw, pf.b_logit) : 0.f;
    if (pf.l2norm) {  // unit q and k rows: each row lives in lanes m, m+16, m+32, m+48
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                sq = fmaf(qf[s][jj], qf[s][jj], sq);
                sk = fmaf(kf[s][jj], kf[s][jj], sk);
            }
        const float rq = rnorm_lanes4(sq), rk = rnorm_lanes4(sk);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                qf[s][jj] *= rq;
                kf[s][jj] *= rk;
            }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            gl[s][jj] = row16_inclusive_scan(rv ? gate_log2(gl[s][jj], pf.g_logit) : 0.f);
    if (m == 15) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float* dst = &sGt[w * DK + 32 * s + 8 * cg];
            *reinterpret_cast<float4*>(dst) = make_float4(gl[s][0], gl[s][1], gl[s][2], gl[s][3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(gl[s][4], gl[s][5], gl[s][6], gl[s][7]);
        }
    }
    lds_barrier();  // (1)

    // ---- per-channel tables; gamma_C to the record
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
        tD[c] = __builtin_amdgcn_exp2f(G1);
        tD[DK + c] = __builtin_amdgcn_exp2f(G2);
        tD[2 * DK + c] = __builtin_amdgcn_exp2f(G1 + G2);
        const float GC = ((G0 + G1) + G2) + G3;
        reinterpret_cast<float*>(rec + R::GC)[c] = __builtin_amdgcn_exp2f(GC);
        if constexpr (BWD) brec[BR::GM + c] = __builtin_amdgcn_exp2f(GC);
    }
    lds_barrier();  // (2)

    // ---- Qt, Kt to the record; Gram factors E = e^{Gloc}, Ei = e^{-Gloc}; column operands to LDS
    // (two exponentials per element: the sub-block offsets come from the per-channel tables).
    // Backward form: Qt^T and -Kt^T fragments too, 64 channels at a time, transposed through the P
    // and A areas ([64][68] fp32 each, not written before the Gram products)
    float E[KS][8], Ei[KS][8];
    constexpr int HALVES = BWD ? DK / 64 : 1;
#pragma unroll
    for (int hf = 0; hf < HALVES; ++hf) {
#pragma unroll
        for (int s = hf * (KS / HALVES); s < (hf + 1) * (KS / HALVES); ++s) {
            const int c0 = 32 * s + 8 * cg;
            float pw[8], bt[8], xq[8], xk[8], xc[8];
            lds_read8(&tPw[w * DK + c0], pw);
            lds_read8(&tBt[w * DK + c0], bt);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                E[s][jj] = __builtin_amdgcn_exp2f(gl[s][jj]);
                Ei[s][jj] = __builtin_amdgcn_exp2f(-gl[s][jj]);
                const float gam = pw[jj] * E[s][jj];  // e^{G_r}
                xq[jj] = qf[s][jj] * gam;
                xk[jj] = kf[s][jj] * gam;
                xc[jj] = kf[s][jj] * (bt[jj] * Ei[s][jj]);  // k e^{G_end(w) - G_r}
            }
            Fr fq, fk;
            fq.set(xq);
            if constexpr (BWD) fk.set(xk);
            else fk.set_hi_only(xk);
            if constexpr (!BWD) gfrag_store<F32>(rec + R::QT + (w * KS + s) * 2 * kPlane, lane, fq);  // the state-only chain reads no Qt
            if constexpr (R::KT_PLANES == 2) gfrag_store<F32>(rec + R::KT + (w * KS + s) * 2 * kPlane, lane, fk);
            else gfrag_store_hi<F32>(rec + R::KT + (w * KS + s) * kPlane, lane, fk);
            if constexpr (BWD) {  // Qt^T, -Kt^T [c - 64 hf][r] (rows past the end as zeros)
                const float z = rv ? 1.f : 0.f;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    sP[(c0 + jj - 64 * hf) * 68 + r] = z * xq[jj];
                    sA[(c0 + jj - 64 * hf) * 68 + r] = -z * xk[jj];
                }
            }
            if (w < 3) {
                float* dst = sCol + r * (DK + 4) + c0;
                *reinterpret_cast<float4*>(dst) = make_float4(xc[0], xc[1], xc[2], xc[3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(xc[4], xc[5], xc[6], xc[7]);
            }
        }
        if constexpr (BWD) {  // wave w: matrix w / 2, channel blocks 2 (w % 2) and 2 (w % 2) + 1 of the half
            lds_barrier();  // (3a)
            const float* stg = (w < 2) ? sP : sA;
            char* dstb = reinterpret_cast<char*>(brec + ((w < 2) ? BR::QTF : BR::KTF));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int cbl = 2 * (w & 1) + (i >> 1), s2 = i & 1;
                float x[8];
                lds_read8(&stg[(16 * cbl + m) * 68 + 32 * s2 + 8 * cg], x);
                Fr f;
                f.set(x);
                gfrag_store<F32>(dstb + ((4 * hf + cbl) * 2 + s2) * 2 * kPlane, lane, f);
            }
            if (hf + 1 < HALVES) lds_barrier();  // (3b) the next half goes over the same areas
        }
    }
    lds_barrier();  // (3)

    switch (w) {
        case 0: prep_gram<0, DK, F32, BWD>(qf, kf, E, Ei, sCol, tD, sBeta, sA, sP, brec + BR::AB, m, cg); break;
        case 1: prep_gram<1, DK, F32, BWD>(qf, kf, E, Ei, sCol, tD, sBeta, sA, sP, brec + BR::AB, m, cg); break;
        case 2: prep_gram<2, DK, F32, BWD>(qf, kf, E, Ei, sCol, tD, sBeta, sA, sP, brec + BR::AB, m, cg); break;
        default: prep_gram<3, DK, F32, BWD>(qf, kf, E, Ei, sCol, tD, sBeta, sA, sP, brec + BR::AB, m, cg); break;
    }
    lds_barrier();  // (4)

    // ---- diagonal blocks of M^{-1} = (I + A)^{-1}: forward substitution, one column per lane
    if (lane < 16) {
        const int cidx = lane;
        const float* Ab = &sA[(16 * w) * 68 + 16 * w];
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < rr; ++jj) acc[jj & 3] = fmaf(Ab[rr * 68 + jj], x[jj], acc[jj & 3]);
            const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            x[rr] = (rr == cidx) ? 1.f : (rr < cidx ? 0.f : -sum);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sD[(w * 16 + rr) * 17 + cidx] = x[rr];
    }
    // ---- P rows of block w to the record
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (BWD || kb >= steps_of(w)) continue;  // the state-only chain reads no P
        float x[8];
        lds_read8(&sP[r * 68 + 32 * kb + 8 * cg], x);
        Fr f;
        f.set(x);
        gfrag_store<F32>(rec + R::PM + pair_of(w, kb) * 2 * kPlane, lane, f);
    }
    if constexpr (BWD) {  // P^T fragments of row block w: columns of P (the zero block of w >= 2 left out)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 < (w >> 1)) continue;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sP[(32 * s2 + 8 * cg + e) * 68 + 16 * w + m];
            Fr f;
            f.set(x);
            gfrag_store<F32>(reinterpret_cast<char*>(brec + BR::PTF) + BR::tri(w, s2) * 2 * kPlane, lane, f);
        }
        if (tid < kC) brec[BR::BT + tid] = sBeta[tid];
    }
    lds_barrier();  // (5)

    // ---- column block I = w of M^{-1}: N_II = D_I, N_RI = -D_R sum_{J=I}^{R-1} A_RJ N_JI (fp32 MFMA);
    // each 16x16 result (lane: column m, rows 4cg..4cg+3) feeds the next product as B operand
    f32x4_t Nr[4];
    {
        const int I = w;
#pragma unroll
        for (int R_ = 0; R_ < 4; ++R_) {
            f32x4_t nv = {0.f, 0.f, 0.f, 0.f};
            if (R_ == I) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) nv[jj] = sD[(I * 16 + 4 * cg + jj) * 17 + m];
            } else if (R_ > I) {
                f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int J = 0; J < 3; ++J) {
                    if (J < I || J >= R_) continue;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        z = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * R_ + m) * 68 + 16 * J + 4 * cg + jj],
                                                                 Nr[J][jj], z, 0, 0, 0);
                }
                f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(sD[(R_ * 16 + m) * 17 + 4 * cg + jj], z[jj], y, 0, 0, 0);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) nv[jj] = -y[jj];
            }
            Nr[R_] = nv;
        }
    }
    if constexpr (BWD) {  // column block w of M^{-1}, as rows of (M^{-1})^T (its zero blocks above the
                          // diagonal block are not written; their readers take them as zero)
#pragma unroll
        for (int R_ = 0; R_ < 4; ++R_)
            if (R_ >= w)
                *reinterpret_cast<float4*>(brec + BR::MIT + (16 * w + m) * 64 + 16 * R_ + 4 * cg) =
                    make_float4(Nr[R_][0], Nr[R_][1], Nr[R_][2], Nr[R_][3]);
    }
    // ---- Kbar = e^{G_C - G} k staged transposed ([c][t]) over the Gram operands and P
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int c0 = 32 * s + 8 * cg;
        float bt[8], af[8];
        lds_read8(&tBt[w * DK + c0], bt);
        lds_read8(&tAf[w * DK + c0], af);
        float kb8[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float kbar = (kf[s][jj] * (bt[jj] * Ei[s][jj])) * af[jj];  // k e^{G_C - G_r}
            lds_store1<F32, DK, kC>(pKB, c0 + jj, r, kbar);
            kb8[jj] = rv ? kbar : 0.f;
        }
        if constexpr (BWD) {  // this lane's piece of the Kb fragment (row block w, step s)
            Fr f;
            f.set(kb8);
            gfrag_store<F32>(reinterpret_cast<char*>(brec + BR::KBF) + (w * KS + s) * 2 * kPlane, lane, f);
        }
    }
    lds_barrier();  // (6)

    // ---- M^{-1} Diag(b) over A (A is no longer read); Kbar^T fragments to the record
    {
        const float bcol = sBeta[16 * w + m];
#pragma unroll
        for (int R_ = 0; R_ < 4; ++R_)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) sA[(16 * R_ + 4 * cg + jj) * 68 + 16 * w + m] = Nr[R_][jj] * bcol;
    }
    if constexpr (!BWD) {
#pragma unroll
        for (int i = 0; i < DK / 32; ++i) {  // (c-block, kb) groups w, w+4, ...
            const int gidx = w + 4 * i;
            const int cb = gidx >> 1, kb = gidx & 1;
            const Fr f = lds_frag<F32, DK, kC>(pKB, 16 * cb + m, 32 * kb + 8 * cg);
            gfrag_store<F32>(rec + R::KB + (cb * 2 + kb) * 2 * kPlane, lane, f);
        }
    }
    lds_barrier();  // (7)

    if constexpr (BWD) {
        // The state-only chain updates S' = Diag(gamma_C) S + B X with B = Kbar^T M^{-1} Diag(b)
        // (= Kbar^T U / X: U = M^{-1} Diag(b) X), so its carried step needs X only.  B [DK][64] as
        // fragments in Kbar^T's place: wave w takes channel blocks (DK/64) w .. and both token steps.
        // Two 16x16 results per fragment, their result rows permuted so that a lane ends up with the
        // eight consecutive columns 32 kb + 8 cg .. of its fragment row: result row i of tile T is
        // column 32 kb + 8 (i / 4) + 4 T + i % 4.  N is lower triangular (with zero rows and columns
        // past the chunk's end), so the contraction starts at token 32 kb.
#pragma unroll
        for (int i = 0; i < DK / 32; ++i) {
            const int cb = (DK / 64) * w + (i >> 1), kb = i & 1;
            f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                if (s2 < kb) continue;
                const Fr kf8 = lds_frag<F32, DK, kC>(pKB, 16 * cb + m, 32 * s2 + 8 * cg);
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    const int j = 32 * kb + 8 * (m >> 2) + 4 * T + (m & 3);
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = sA[(32 * s2 + 8 * cg + e) * 68 + j];
                    Fr nf;
                    nf.set(x);
                    acc[T] = mma_full(acc[T], nf, kf8);
                }
            }
            float x[8];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                x[jj] = acc[0][jj];
                x[4 + jj] = acc[1][jj];
            }
            Fr f;
            f.set(x);
            gfrag_store<F32>(rec + R::KB + (cb * 2 + kb) * 2 * kPlane, lane, f);
        }
    }

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb >= steps_of(w)) continue;
        float x[8];
        lds_read8(&sA[r * 68 + 32 * kb + 8 * cg], x);
        Fr f;
        f.set(x);
        gfrag_store<F32>(rec + R::NM + pair_of(w, kb) * 2 * kPlane, lane, f);
    }
    if constexpr (BWD) {  // (M^{-1} Diag(b))^T fragments of row block w: columns of M^{-1} Diag(b) (zero block left out)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 < (w >> 1)) continue;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = sA[(32 * s2 + 8 * cg + e) * 68 + 16 * w + m];
            Fr f;
            f.set(x);
            gfrag_store<F32>(reinterpret_cast<char*>(brec + BR::NTF) + BR::tri(w, s2) * 2 * kPlane, lane, f);
        }
    }
}

// ============================================================================ chain kernel

template <int DK, bool F32>
struct ChainLds {
    using MS = LMat<F32, kS, DK>;  // S^T  [n][c]
    using MX = LMat<F32, kS, kC>;  // X^T, U^T  [n][t]
    static constexpr int S = 0;
    static constexpr int X = S + MS::BYTES;
    static constexpr int U = X + MX::BYTES;
    static constexpr int O = U + MX::BYTES;     // fp32 output rows [64][kS + 4] on their way to HBM
    static constexpr int V = O + 64 * (kS + 4) * 4;  // v rows [64][kS] (input type) on their way from HBM
    static constexpr int TOTAL = V + 64 * kS * 4;
    // mode 3 (state only): X rows over O, then U rows [64][kS + 4] and the chunk-start state rows
    // [DK][kS + 4], fp32, on their way to HBM as whole 128-byte rows
    static constexpr int FU = TOTAL;
    static constexpr int FS = FU + 64 * (kS + 4) * 4;
    static constexpr int TOTAL_ST = FS + DK * (kS + 4) * 4;
};

// Operands of one chunk for one wave of the chain kernel.  A state wave (row block rb) holds the rows
// of rb of Kt and M^{-1} Diag(b) and its v rows; an output wave (row block rb) the rows of rb of Qt and
// P; both hold the Kbar^T rows and gamma_C entries of their S tiles' channel block.
template <int DK, bool F32, bool IN_F32>
struct ChainStateOps {
    Frag<F32> fK[DK / 32], fN[2], fKB[2];
    float4 gC;
    uint4 vraw[IN_F32 ? 2 : 1];  // this lane's 16-byte pieces of the wave's v rows
};
template <int DK, bool F32>
struct ChainOutOps {
    Frag<F32> fQ[DK / 32], fP[2], fKB[2];
    float4 gC;
};

// SO (state only, modes 1 and 3): the output products, their operands and the o traffic are compiled
// out.  F32: precision policy of the records; IN_F32: type of v; ST: mode 3's stores are compiled in.
//
// Eight waves, two per SIMD, so that one wave's LDS and MFMA latencies overlap the other's work.
// State waves 0-3 (row block rb = w) compute X = V - Kt S and U = M^{-1} Diag(b) X for the 16 rows
// of rb and all 32 columns; output waves 4-7 (rb = w - 4) compute O = Qt S + P U for the same rows,
// Qt S spread over the first two phases.  Every wave also updates DK / 64 of the (16-channel block,
// 16-column half) tiles of S in the third phase (mode 3: in the second, from X and B, while the state
// waves form U for the stores).  Both kinds of wave pass the same three (mode 3: two) barriers
// per chunk.
template <int DK, bool F32, bool SO, bool IN_F32 = F32, bool ST = false>
__global__ __launch_bounds__(kChainThreads, SO && !F32 && !ST ? 4 : 1) void chain_kernel(const void* __restrict__ vv, const float* s0,
                                                                 float* __restrict__ o, float* s_final,
                                                                 const int32_t* __restrict__ cu_seqlens,
                                                                 int64_t T_fixed, int64_t T_stride, int64_t total,
                                                                 int64_t N, int H,
                                                                 int Dv, ChainMode cm,
                                                                 const char* ws) {  // not restrict: keeps the loads of the next chunk where they are written
    using In = typename std::conditional<IN_F32, float, uint16_t>::type;
    using Fr = Frag<F32>;
    using L = ChainLds<DK, F32>;
    using R = Rec<DK, F32, F32 || ST>;
    constexpr int KS = DK / 32;
    constexpr int KH = KS / 2;                      // Qt S steps in the first phase (the rest in the second)
    constexpr int TPW = DK / 64;                    // S tiles per wave (all in one channel block)
    constexpr int VPL = 16 / (int)sizeof(In);       // v values per 16-byte lane load
    const In* __restrict__ v = static_cast<const In*>(vv);

    __shared__ __align__(16) char smem[ST ? L::TOTAL_ST : L::TOTAL];
    char* pS = smem + L::S;
    char* pX = smem + L::X;
    char* pU = smem + L::U;
    float* sO = reinterpret_cast<float*>(smem + L::O);
    In* sV = reinterpret_cast<In*>(smem + L::V);
    constexpr int FLD = kS + 4;  // row stride of the mode-3 fp32 tiles
    float* fX = reinterpret_cast<float*>(smem + L::O);  // mode 3 only (SO: no output rows)
    float* fU = reinterpret_cast<float*>(smem + (ST ? L::FU : 0));
    float* fS = reinterpret_cast<float*>(smem + (ST ? L::FS : 0));

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    const int rb = w & 3;
    const int cbw = (w * TPW) >> 1;                            // channel block of this wave's S tiles
    auto nbt = [&](int i) { return (w * TPW + i) & 1; };      // column half of S tile i
    const int NV = Dv / kS;                                // value-column slices
    const int NS = cm.mode == 1 ? NV + DK / kS : NV;       // + identity-column slices in mode 1
    const int segs = cm.mode == 1 ? cm.P - 1 : (cm.mode == 2 ? cm.P : 1);
    const int64_t items = N * (int64_t)H * segs;
    const int64_t bid = blockIdx.x;
    const int64_t loc = bid >> 3;
    const int sl = (int)(loc % NS);
    const int64_t pr = (loc / NS) * 8 + (bid & 7);  // slices of one item on one XCD
    if (pr >= items) return;
    const int64_t n = cm.order ? (int64_t)cm.order[pr / ((int64_t)H * segs)] : pr / ((int64_t)H * segs);
    const int h = (int)((pr / segs) % H);
    const int p = (int)(pr % segs);
    const SeqRange sr = seq_range(cu_seqlens, n, T_fixed, T_stride, total);
    const int64_t start = sr.start, end = sr.end;
    const int64_t nall = (end - start + kC - 1) / kC;
    const bool split = cm.mode == 1 || cm.mode == 2;
    const int64_t jbeg = split ? min<int64_t>(p * cm.L, nall) : 0;
    const int64_t jend = split ? min<int64_t>((p + 1) * cm.L, nall) : nall;
    const bool ident = sl >= NV;                           // identity columns (mode 1)
    const int col0 = ident ? 0 : sl * kS;                  // value columns read (v) by this slice
    const int colx = sl * kS;                              // column of this slice in sx rows (mode 1)
    const float vscale = ident ? 0.f : 1.f;                // V = 0 for the identity columns
    const int nk = steps_of(rb);

    // state of this slice at the segment start (its source chosen once, so that the loads of all of a
    // wave's elements are issued together) / its destination
    // (mode 2 reads every segment's initial state from sfold, p = 0 included, where the fold kernel
    // copied s0: s0 is then read by no launch that also writes s_final, which may alias it)
    const float* const s_src = cm.mode == 1 ? nullptr
                               : (cm.mode == 2 ? cm.sfold + (((n * H + h) * (int64_t)cm.P + p) * DK) * Dv
                                               : (s0 ? s0 + (n * H + h) * (int64_t)DK * Dv : nullptr));

    float* const sdst = cm.mode == 1 ? cm.sx + (pr * DK) * (int64_t)(Dv + DK)
                                     : ((cm.mode == 0 || p == cm.P - 1) && s_final
                                            ? s_final + (n * H + h) * (int64_t)DK * Dv : nullptr);
    const int ld_dst = cm.mode == 1 ? Dv + DK : Dv;
    const int col_dst = cm.mode == 1 ? colx : col0;

    // initial state of this wave's tiles
    f32x4_t accS[TPW];
    if (cm.mode == 1) {  // zero value columns; the identity on the identity columns
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c = 16 * cbw + 4 * cg + jj, col = col0 + 16 * nbt(i) + m;
                accS[i][jj] = ident && c == colx - Dv + col - col0 ? 1.f : 0.f;
            }
    } else if (s_src) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                accS[i][jj] = s_src[(16 * cbw + 4 * cg + jj) * (int64_t)Dv + col0 + 16 * nbt(i) + m];
    } else {
#pragma unroll
        for (int i = 0; i < TPW; ++i) accS[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) lds_store4<F32, kS, DK>(pS, 16 * nbt(i) + m, 16 * cbw + 4 * cg, accS[i]);
    auto tile_state = [&]() {  // mode 3: this wave's S tiles to the fp32 state rows
        if constexpr (ST) {
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) fS[(16 * cbw + 4 * cg + jj) * FLD + 16 * nbt(i) + m] = accS[i][jj];
        }
    };
    tile_state();

    auto record = [&](int64_t jc) -> const char* {
        return ws + (slot_of(cu_seqlens, n, jc, T_fixed, start) * H + h) * R::BYTES;
    };
    auto chunk_start = [&](int64_t jc) { return start + jc * kC; };
    auto chunk_len = [&](int64_t jc) { return (int)min<int64_t>(kC, end - chunk_start(jc)); };
    // the chunk after jc, or jc again after the last one
    auto next_chunk = [&](int64_t jc) { return jc + 1 < jend ? jc + 1 : jc; };

    // third phase, both kinds of wave: S = gamma_C S + Kbar^T U on this wave's tiles (mode 3, second
    // phase: S = gamma_C S + B X, B = Kbar^T M^{-1} Diag(b) from the record, ub = X^T)
    auto update_state = [&](const Fr (&uf)[2][2], const Fr (&fKB)[2], float4 gC, const char* ub) {
        const float gcv[4] = {gC.x, gC.y, gC.z, gC.w};
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) accS[i][jj] *= gcv[jj];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if constexpr (TPW == 2) {  // tile i is column half i
                    accS[i] = mma_full(accS[i], fKB[kb], uf[i][kb]);
                } else {
                    const Fr u = lds_frag<F32, kS, kC>(ub, 16 * nbt(i) + m, 32 * kb + 8 * cg);
                    accS[i] = mma_full(accS[i], fKB[kb], u);
                }
            }
        }
    };
    auto store_state = [&]() {
#pragma unroll
        for (int i = 0; i < TPW; ++i) lds_store4<F32, kS, DK>(pS, 16 * nbt(i) + m, 16 * cbw + 4 * cg, accS[i]);
        tile_state();
    };
    auto read_u = [&](Fr (&uf)[2][2], const char* ub) {
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) uf[hb][kb] = lds_frag<F32, kS, kC>(ub, 16 * hb + m, 32 * kb + 8 * cg);
    };
    auto load_kb = [&](Fr (&fKB)[2], float4& gC, const char* rec) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) fKB[kb] = gfrag_load<F32>(rec + R::KB + (cbw * 2 + kb) * 2 * kPlane, lane);
        gC = *reinterpret_cast<const float4*>(rec + R::GC + (16 * cbw + 4 * cg) * 4);
    };
    // mode 3, every thread: rows of a staged fp32 tile to memory, eight lanes per 128-byte row
    // (ROWS a multiple of 64: unrolled, so that the compiler counts every store)
    auto store_rows = [&](float* dst, const float* tile, auto rows) {
        constexpr int ROWS = decltype(rows)::value;
        static_assert(ROWS % (kChainThreads / 8) == 0, "whole passes");
#pragma unroll
        for (int k = 0; k < ROWS / (kChainThreads / 8); ++k) {
            const int r = (tid >> 3) + k * (kChainThreads / 8);
            const float4 x = *reinterpret_cast<const float4*>(&tile[r * FLD + 4 * (tid & 7)]);
            st_nt4(dst + r * (int64_t)Dv + 4 * (tid & 7), x.x, x.y, x.z, x.w);
        }
    };
    auto store_start_state = [&](int64_t jc) {  // mode 3: the state at the start of chunk jc
        if constexpr (ST)
            store_rows(cm.sx + (slot_of(cu_seqlens, n, jc, T_fixed, start) * H + h) * (int64_t)DK * Dv + col0, fS, std::integral_constant<int, DK>{});
    };
    auto store_x = [&](int64_t jc) {  // mode 3: X rows of chunk jc (staged in phase 1)
        if constexpr (ST)
            store_rows(cm.xu + (slot_of(cu_seqlens, n, jc, T_fixed, start) * H + h) * 128 * (int64_t)Dv + col0, fX, std::integral_constant<int, 64>{});
    };
    auto store_u = [&](int64_t jc) {  // mode 3: U rows of chunk jc (staged in phase 2, stored in the next step)
        if constexpr (ST)
            store_rows(cm.xu + ((slot_of(cu_seqlens, n, jc, T_fixed, start) * H + h) * 128 + 64) * (int64_t)Dv + col0,
                       fU, std::integral_constant<int, 64>{});
    };

    if (w < 4) {
        // ======================= state waves: X and U of row block rb
        using Ops = ChainStateOps<DK, F32, IN_F32>;
        constexpr int VLPR = kS / VPL;        // lanes per v row slice (bf16: 4, fp32: 8)
        constexpr int VROWS = 64 / VLPR;      // v rows per load (bf16: 16, fp32: 8)
        constexpr int VLOADS = 16 / VROWS;    // loads per lane (bf16: 1, fp32: 2)
        const uint32_t rs_v = (uint32_t)H * (uint32_t)Dv;
        const int vrow = 16 * rb + lane / VLPR, vpiece = lane % VLPR;
        const In* __restrict__ v_l = v + (int64_t)h * Dv + col0 + vpiece * VPL;

        auto load_k = [&](Ops& d, const char* rec, int s) {
            if constexpr (R::KT_PLANES == 2) d.fK[s] = gfrag_load<F32>(rec + R::KT + (rb * KS + s) * 2 * kPlane, lane);
            else d.fK[s] = gfrag_load_hi<F32>(rec + R::KT + (rb * KS + s) * kPlane, lane);
        };
        auto load_nv = [&](Ops& d, const char* rec, int64_t jc) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)  // blocks 0, 1 stop at token 31: their second step repeats the first
                d.fN[kb] = gfrag_load<F32>(rec + R::NM + pair_of(rb, min(kb, nk - 1)) * 2 * kPlane, lane);
            const int64_t t0 = chunk_start(jc);
            const int nt = chunk_len(jc);
#pragma unroll
            for (int i = 0; i < VLOADS; ++i) {
                const uint32_t rvo = (uint32_t)min(vrow + i * VROWS, nt - 1) * rs_v;
                d.vraw[i] = *reinterpret_cast<const uint4*>(v_l + t0 * (int64_t)rs_v + rvo);
            }
        };
        auto step = [&](Ops& cur, Ops& nxt, int64_t jc) {
            const int nt = chunk_len(jc);
            const int64_t jn = next_chunk(jc);
            const char* recn = record(jn);
            store_start_state(jc);
            if constexpr (ST) {
                if (jc > jbeg) store_u(jc - 1);  // staged in the previous step's second phase
            }
#pragma unroll
            for (int i = 0; i < VLOADS; ++i)
                *reinterpret_cast<uint4*>(&sV[(vrow + i * VROWS) * kS + vpiece * VPL]) = cur.vraw[i];

            // ---- phase 1:  X = V - Kt S (one pass)
            f32x4_t accX[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    accX[nb] = ST ? mma_full(accX[nb], cur.fK[s], lds_frag<F32, kS, DK>(pS, 16 * nb + m, 32 * s + 8 * cg))
                                  : mma_fast(accX[nb], cur.fK[s], lds_frag<F32, kS, DK>(pS, 16 * nb + m, 32 * s + 8 * cg));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                f32x4_t xv;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const In raw = sV[(16 * rb + 4 * cg + jj) * kS + 16 * nb + m];
                    float vj;
                    if constexpr (IN_F32) vj = raw;
                    else vj = bf16_bits_to_float(raw);
                    xv[jj] = vscale * vj - accX[nb][jj];
                }
                lds_store4<F32, kS, kC>(pX, 16 * nb + m, 16 * rb + 4 * cg, xv);
                if constexpr (ST) {  // rows past the end stored as zeros
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int row = 16 * rb + 4 * cg + jj;
                        fX[row * FLD + 16 * nb + m] = row < nt ? xv[jj] : 0.f;
                    }
                }
            }
            // the next chunk's Kt rows: requested only now, when the products that read this chunk's
            // copy (whose registers they may take) have completed, so the requests do not stall
#pragma unroll
            for (int s = 0; s < KS; ++s) load_k(nxt, recn, s);
            lds_barrier();  // (1)
            store_x(jc);

            // ---- phase 2:  U = M^{-1} Diag(b) X
            f32x4_t accU[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb >= nk) continue;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    accU[nb] = mma_full(accU[nb], cur.fN[kb], lds_frag<F32, kS, kC>(pX, 16 * nb + m, 32 * kb + 8 * cg));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                if constexpr (ST) {  // U is only stored: the state update below takes X
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) fU[(16 * rb + 4 * cg + jj) * FLD + 16 * nb + m] = accU[nb][jj];
                } else {
                    lds_store4<F32, kS, kC>(pU, 16 * nb + m, 16 * rb + 4 * cg, accU[nb]);
                }
            }
            load_nv(nxt, recn, jn);  // after the products that read this chunk's M^{-1} rows
            if constexpr (!ST) {
                lds_barrier();  // (2)
                store_u(jc);
            }

            // ---- phase 3 (mode 3: still the second phase):  S tiles
            Fr uf[2][2];
            read_u(uf, ST ? pX : pU);
            update_state(uf, cur.fKB, cur.gC, ST ? pX : pU);
            store_state();
            load_kb(nxt.fKB, nxt.gC, recn);  // after the tile products that read this chunk's copy
            lds_barrier();  // (3)
        };
        Ops opsA, opsB;
        if (jbeg < jend) {
            const char* rec = record(jbeg);
#pragma unroll
            for (int s = 0; s < KS; ++s) load_k(opsA, rec, s);
            load_nv(opsA, rec, jbeg);
            load_kb(opsA.fKB, opsA.gC, rec);
        }
        lds_barrier();
        // two chunks per iteration, so that the operand sets alternate without copies
        int64_t jc = jbeg;
        for (; jc + 1 < jend; jc += 2) {
            step(opsA, opsB, jc);
            step(opsB, opsA, jc + 1);
        }
        if (jc < jend) step(opsA, opsB, jc);
    } else {
        // ======================= output waves: O of row block rb (and S tiles)
        using Ops = ChainOutOps<DK, F32>;
        const uint32_t rs_o = (uint32_t)H * (uint32_t)Dv;
        float* __restrict__ o_l = o + (int64_t)h * Dv + col0 + (lane & 7) * 4;

        auto load_q = [&](Ops& d, const char* rec, int s) {
            if constexpr (!SO) d.fQ[s] = gfrag_load<F32>(rec + R::QT + (rb * KS + s) * 2 * kPlane, lane);
        };
        auto load_p = [&](Ops& d, const char* rec) {
            if constexpr (!SO) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    d.fP[kb] = gfrag_load<F32>(rec + R::PM + pair_of(rb, min(kb, nk - 1)) * 2 * kPlane, lane);
            }
        };
        // o rows of a finished chunk: D-layout registers -> LDS -> whole row slices (this wave's rows only)
        auto stage_o = [&](const f32x4_t (&accO)[2]) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sO[(16 * rb + 4 * cg + jj) * (kS + 4) + 16 * nb + m] = accO[nb][jj];
        };
        auto store_o = [&](int64_t tc, int ntc) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int rr = 16 * rb + 8 * half + (lane >> 3);
                const float4 x = *reinterpret_cast<const float4*>(&sO[rr * (kS + 4) + (lane & 7) * 4]);
                if (rr < ntc)  // o is not read again by this call: streamed past the caches
                    __builtin_nontemporal_store(f32x4_t{x.x, x.y, x.z, x.w},
                                                reinterpret_cast<f32x4_t*>(o_l + (tc + rr) * (int64_t)rs_o));
            }
        };
        auto step = [&](Ops& cur, Ops& nxt, int64_t jc) {
            const int64_t jn = next_chunk(jc);
            const char* recn = record(jn);
            store_start_state(jc);
            if constexpr (ST) {
                if (jc > jbeg) store_u(jc - 1);  // staged in the previous step's second phase
            }

            // ---- phase 1:  O = Qt S, first half of the channels
            f32x4_t accO[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            if constexpr (!SO) {
#pragma unroll
                for (int s = 0; s < KH; ++s) {
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        accO[nb] = mma_full(accO[nb], cur.fQ[s], lds_frag<F32, kS, DK>(pS, 16 * nb + m, 32 * s + 8 * cg));
                    load_q(nxt, recn, s);
                }
                if (jc > jbeg) store_o(chunk_start(jc) - kC, kC);
            }
            lds_barrier();  // (1)
            store_x(jc);

            // ---- phase 2:  second half of the channels (S is rewritten only in phase 3)
            if constexpr (!SO) {
#pragma unroll
                for (int s = KH; s < KS; ++s) {
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        accO[nb] = mma_full(accO[nb], cur.fQ[s], lds_frag<F32, kS, DK>(pS, 16 * nb + m, 32 * s + 8 * cg));
                    load_q(nxt, recn, s);
                }
            }
            if constexpr (!ST) {
                lds_barrier();  // (2)
                store_u(jc);
            }

            // ---- phase 3 (mode 3: the second phase):  O += P U, S tiles
            Fr uf[2][2];
            read_u(uf, ST ? pX : pU);
            if constexpr (!SO) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (kb >= nk) continue;
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) accO[nb] = mma_full(accO[nb], cur.fP[kb], uf[nb][kb]);
                }
            }
            update_state(uf, cur.fKB, cur.gC, ST ? pX : pU);
            store_state();
            load_kb(nxt.fKB, nxt.gC, recn);  // after the tile products that read this chunk's copy
            if constexpr (!SO) {
                stage_o(accO);
                load_p(nxt, recn);  // after the P U products that read this chunk's copy
            }
            lds_barrier();  // (3)
        };
        Ops opsA, opsB;
        if (jbeg < jend) {
            const char* rec = record(jbeg);
#pragma unroll
            for (int s = 0; s < KS; ++s) load_q(opsA, rec, s);
            load_p(opsA, rec);
            load_kb(opsA.fKB, opsA.gC, rec);
        }
        lds_barrier();
        // two chunks per iteration, so that the operand sets alternate without copies
        int64_t jc = jbeg;
        for (; jc + 1 < jend; jc += 2) {
            step(opsA, opsB, jc);
            step(opsB, opsA, jc + 1);
        }
        if (jc < jend) step(opsA, opsB, jc);
        if (!SO && jbeg < jend) store_o(chunk_start(jend - 1), chunk_len(jend - 1));
    }
    if constexpr (ST) {  // the last chunk's U rows, staged before the last barrier
        if (jbeg < jend) store_u(jend - 1);
    }

    if (sdst) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                sdst[(16 * cbw + 4 * cg + jj) * (int64_t)ld_dst + col_dst + 16 * nbt(i) + m] = accS[i][jj];
    }
}

// ============================================================================ segment fold

// Initial states of the segments of a split sequence, one workgroup per (sequence, head,
// 32-column slice): S_in(0) = s0 (or 0), S_in(p+1) = Phi_p S_in(p) + S0_p for p < P - 1, written
// to sfold [n][h][p][Dk][Dv] (p = 0 included).  fp32 throughout; the running state stays in LDS.
// Each step is a [Dk x Dk] x [Dk x 32] product on fp32 MFMA (16x16x4): wave w owns result rows
// 16 RT w .. as 16x16 tiles (row tile rt, column tile ct); MFMA number t of a tile contracts channel
// (Dk/4) g + t in lane group g, so each lane reads one run of Dk/4 channels of its Phi row.  The next
// step's Phi rows are requested while the current step's products run.
template <int DK>
__global__ __launch_bounds__(256) void fold_kernel(const float* s0, const float* __restrict__ sx,
                                                   float* __restrict__ sfold, int H, int Dv, int P) {
    constexpr int RT = DK / 64;   // row tiles per wave (4 waves x RT x 16 rows = DK)
    constexpr int KPL = DK / 4;   // channels contracted by one lane group
    constexpr int NQ = KPL / 4;   // float4 runs of a lane's Phi row
    constexpr int SST = kS + 1;
    __shared__ float sS[DK * SST];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, g = lane >> 4;
    const int NV = Dv / kS;
    const int64_t item = blockIdx.x / NV;  // n * H + h
    const int col0 = (int)(blockIdx.x % NV) * kS;
    const int64_t ldx = Dv + DK;
    // S_in(0): to LDS and to sfold[p = 0]
    float* const dst0 = sfold + (item * P * DK) * (int64_t)Dv + col0;
    for (int e = tid; e < DK * kS; e += 256) {
        const int c = e / kS, j = e % kS;
        const float x = s0 ? s0[(item * DK + c) * (int64_t)Dv + col0 + j] : 0.f;
        sS[c * SST + j] = x;
        dst0[c * Dv + j] = x;
    }
    // Phi rows of this lane: row 16 (RT w + rt) + m, channels KPL g + 0..KPL-1 (NQ float4 per row tile)
    float4 ph[RT][NQ];
    auto load_phi = [&](int p) {
        const float* X = sx + ((item * (P - 1) + p) * DK) * ldx + Dv;  // Phi_p [Dk][Dk] at column Dv
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                ph[rt][q] = *reinterpret_cast<const float4*>(X + (16 * (RT * w + rt) + m) * ldx + KPL * g + 4 * q);
    };
    if (P > 1) load_phi(0);
    __syncthreads();
    for (int p = 0; p + 1 < P; ++p) {
        const float* S0p = sx + ((item * (P - 1) + p) * DK) * ldx + col0;  // S0_p [Dk][Dv] at column 0
        f32x4_t acc[RT][2];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[rt][ct][i] = S0p[(16 * (RT * w + rt) + 4 * g + i) * ldx + 16 * ct + m];
        float4 cur[RT][NQ];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int q = 0; q < NQ; ++q) cur[rt][q] = ph[rt][q];
        if (p + 2 < P) load_phi(p + 1);
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = 4 * q + u;
                const float b0 = sS[(KPL * g + t) * SST + m], b1 = sS[(KPL * g + t) * SST + 16 + m];
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const float av = u == 0 ? cur[rt][q].x : (u == 1 ? cur[rt][q].y : (u == 2 ? cur[rt][q].z : cur[rt][q].w));
                    acc[rt][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b0, acc[rt][0], 0, 0, 0);
                    acc[rt][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b1, acc[rt][1], 0, 0, 0);
                }
            }
        __syncthreads();  // every lane has read S_in(p)
        float* dst = sfold + ((item * P + p + 1) * DK) * (int64_t)Dv + col0;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * (RT * w + rt) + 4 * g + i;
                    sS[r * SST + 16 * ct + m] = acc[rt][ct][i];
                    dst[r * Dv + 16 * ct + m] = acc[rt][ct][i];
                }
        __syncthreads();
    }
}

// ============================================================================ host side

static int64_t seq_stride(const ChunkArgs& a) { return a.T_stride > 0 ? a.T_stride : a.T_fixed; }

int64_t chunk_slots(const ChunkArgs& a) {
    if (a.cu_seqlens) return a.total / kC + a.N;
    return a.N * ((a.T_fixed + kC - 1) / kC);
}

int64_t chunk_record_bytes(int Dk, bool f32) {
    if (Dk == 128) return f32 ? Rec<128, true>::BYTES : Rec<128, false>::BYTES;
    return f32 ? Rec<64, true>::BYTES : Rec<64, false>::BYTES;
}

// Segments of the split-T path: equal-length sequences whose chain would occupy fewer than half
// of 256 workgroup slots are cut into P segments so that the output pass has about 256
// workgroups, each segment at least 64 chunks long.  (A fixed target keeps the workspace size a
// function of the arguments alone.)
int chunk_segments(const ChunkArgs& a) {
    if (a.cu_seqlens) return 1;
    constexpr int64_t kTarget = 256;
    const int64_t slices = a.N * a.H * (a.Dv / kS);
    if (slices * 2 > kTarget) return 1;
    int64_t P = kTarget / slices;
    const int64_t nch = (a.T_fixed + kC - 1) / kC;
    if (P > nch / 64) P = nch / 64;
    return P >= 2 ? (int)P : 1;
}

static int64_t records_bytes(const ChunkArgs& a) { return chunk_slots(a) * a.H * chunk_record_bytes(a.Dk, a.f32); }

// split-T state areas: segment maps [N][H][P-1][Dk][Dv + Dk], segment initial states [N][H][P][Dk][Dv]
static int64_t segment_bytes(const ChunkArgs& a, int P) {
    if (P < 2) return 0;
    return a.N * a.H * (int64_t)a.Dk * 4 * ((P - 1) * (int64_t)(a.Dv + a.Dk) + P * (int64_t)a.Dv);
}

// packed sequences: their order, longest first, for the chain's dispatch [N] int32
static int64_t order_bytes(const ChunkArgs& a) { return a.cu_seqlens ? ((a.N * 4 + 255) / 256) * 256 : 0; }

// bf16 inputs take the fp16-operand path of kda_fwd16.hip; fp32 inputs the fp32 records here.
int64_t chunk_workspace_bytes(const ChunkArgs& a) {
    if (!a.f32) return chunk16_workspace_bytes(a);
    return records_bytes(a) + segment_bytes(a, chunk_segments(a)) + order_bytes(a);
}

// Packed sequences sorted by length, longest first (ties by index): order[rank] = n.  The chain
// kernel's workgroups start in that order, so the longest chains do not trail at the end of the grid.
// One workgroup per 256 sequences; the lengths are staged in LDS (up to kOrderMax sequences; beyond
// that the order is the identity).
constexpr int kOrderMax = 4096;
__global__ __launch_bounds__(256) void seq_order_kernel(const int32_t* __restrict__ cu, int64_t N, int64_t total,
                                                        int32_t* __restrict__ order) {
    __shared__ int32_t sl[kOrderMax];
    const int64_t i = blockIdx.x * 256 + threadIdx.x;
    if (N > kOrderMax) {
        if (i < N) order[i] = (int32_t)i;
        return;
    }
    auto len = [&](int64_t j) {
        const int64_t s0 = min<int64_t>(max<int64_t>(cu[j], 0), total);
        return (int32_t)(min<int64_t>(max<int64_t>(cu[j + 1], s0), total) - s0);
    };
    for (int64_t j = threadIdx.x; j < N; j += 256) sl[j] = len(j);
    __syncthreads();
    if (i >= N) return;
    const int32_t li = sl[i];
    int32_t rank = 0;
    for (int j = 0; j < (int)N; ++j) rank += (sl[j] > li) || (sl[j] == li && j < (int)i);
    order[rank] = (int32_t)i;
}

static int64_t chain_grid(int64_t items, int slices) { return ((items + 7) / 8) * 8 * slices; }

hipError_t launch_seq_order(const int32_t* cu, int64_t N, int64_t total, int32_t* order, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, cu, N, total, order);
    return hipGetLastError();
}

hipError_t launch_fold(int Dk, const float* s0, const float* sx, float* sfold, int64_t items, int H, int Dv, int P,
                       hipStream_t st) {
    const dim3 grid((unsigned)(items * (Dv / kS)));
    if (Dk == 128) hipLaunchKernelGGL((fold_kernel<128>), grid, dim3(256), 0, st, s0, sx, sfold, H, Dv, P);
    else hipLaunchKernelGGL((fold_kernel<64>), grid, dim3(256), 0, st, s0, sx, sfold, H, Dv, P);
    return hipGetLastError();
}

template <int DK, bool F32>
static hipError_t launch_two(const ChunkArgs& a, void* ws, hipStream_t st, bool allow_split = true) {
    const int64_t prep_grid = chunk_slots(a) * a.H;
    if (prep_grid > 0 && any_prologue(a.pro))
        hipLaunchKernelGGL((prep_kernel<DK, F32, true>), dim3((unsigned)prep_grid), dim3(256), 0, st, a.q, a.k, a.g,
                           a.beta, a.cu_seqlens, a.T_fixed, seq_stride(a), a.total, a.N, a.H, a.pro, static_cast<char*>(ws));
    else if (prep_grid > 0)
        hipLaunchKernelGGL((prep_kernel<DK, F32, false>), dim3((unsigned)prep_grid), dim3(256), 0, st, a.q, a.k, a.g,
                           a.beta, a.cu_seqlens, a.T_fixed, seq_stride(a), a.total, a.N, a.H, a.pro, static_cast<char*>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int P = allow_split ? chunk_segments(a) : 1;
    const int NV = a.Dv / kS;
    if (P < 2) {
        ChainMode cm{0, 1, 0, nullptr, nullptr};
        if (a.cu_seqlens && a.N > 0) {
            int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + records_bytes(a));
            hipLaunchKernelGGL(seq_order_kernel, dim3((unsigned)((a.N + 255) / 256)), dim3(256), 0, st, a.cu_seqlens,
                               a.N, a.total, order);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            cm.order = order;
        }
        hipLaunchKernelGGL((chain_kernel<DK, F32, false>), dim3((unsigned)chain_grid(a.N * a.H, NV)), dim3(kChainThreads), 0, st,
                           a.v, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, seq_stride(a), a.total, a.N, a.H, a.Dv, cm,
                           static_cast<const char*>(ws));
        return hipGetLastError();
    }
    // split-T: segment maps, fold, outputs
    const int64_t nch = (a.T_fixed + kC - 1) / kC;
    const int64_t L = (nch + P - 1) / P;
    float* sx = reinterpret_cast<float*>(static_cast<char*>(ws) + records_bytes(a));
    float* sfold = sx + a.N * a.H * (int64_t)(P - 1) * a.Dk * (a.Dv + a.Dk);
    const ChainMode c1{1, P, L, sx, nullptr};
    hipLaunchKernelGGL((chain_kernel<DK, F32, true>), dim3((unsigned)chain_grid(a.N * a.H * (P - 1), NV + DK / kS)),
                       dim3(kChainThreads), 0, st, a.v, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, seq_stride(a), a.total, a.N,
                       a.H, a.Dv, c1, static_cast<const char*>(ws));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((fold_kernel<DK>), dim3((unsigned)(a.N * a.H * NV)), dim3(256), 0, st, a.s0, sx, sfold, a.H,
                       a.Dv, P);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const ChainMode c2{2, P, L, nullptr, sfold};
    hipLaunchKernelGGL((chain_kernel<DK, F32, false>), dim3((unsigned)chain_grid(a.N * a.H * P, NV)), dim3(kChainThreads), 0, st,
                       a.v, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, seq_stride(a), a.total, a.N, a.H, a.Dv, c2,
                       static_cast<const char*>(ws));
    return hipGetLastError();
}

// States at every chunk start, for the backward pass: split-bf16 records with every product in three
// passes (Kt with both planes, the Gram of k included; fp32 states and accumulators) for both input
// types.  prep into `recs` (chunk_slots(a) * H records of chunk_record_bytes(Dk, true)) and the plain
// backward operands into `brecs`, then the state-only chain in mode 3 writing `states` [slot][h][Dk][Dv]
// and X, U of every chunk to `xu` [slot][h][2][64][Dv].
template <int DK, bool IN_F32>
static hipError_t launch_states(const ChunkArgs& a, void* recs, float* brecs, float* states, float* xu,
                                hipStream_t st) {
    const int64_t prep_grid = chunk_slots(a) * a.H;
    if (prep_grid > 0)
        hipLaunchKernelGGL((prep_kernel<DK, false, false, IN_F32, true>), dim3((unsigned)prep_grid), dim3(256), 0, st,
                           a.q, a.k, a.g, a.beta, a.cu_seqlens, a.T_fixed, seq_stride(a), a.total, a.N, a.H, a.pro,
                           static_cast<char*>(recs), brecs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const ChainMode cm{3, 1, 0, states, nullptr, xu};
    hipLaunchKernelGGL((chain_kernel<DK, false, true, IN_F32, true>), dim3((unsigned)chain_grid(a.N * a.H, a.Dv / kS)),
                       dim3(kChainThreads), 0, st, a.v, a.s0, (float*)nullptr, (float*)nullptr, a.cu_seqlens, a.T_fixed, seq_stride(a), a.total,
                       a.N, a.H, a.Dv, cm, static_cast<const char*>(recs));
    return hipGetLastError();
}

int64_t chunk_states_record_bytes(int Dk) { return chunk_record_bytes(Dk, true); }

hipError_t launch_chunk_states(const ChunkArgs& a, void* recs, float* brecs, float* states, float* xu,
                               hipStream_t st) {
    if (a.Dk == 128)
        return a.f32 ? launch_states<128, true>(a, recs, brecs, states, xu, st)
                     : launch_states<128, false>(a, recs, brecs, states, xu, st);
    return a.f32 ? launch_states<64, true>(a, recs, brecs, states, xu, st)
                 : launch_states<64, false>(a, recs, brecs, states, xu, st);
}

hipError_t launch_chunk_fwd_two_pass(const ChunkArgs& a, void* ws, hipStream_t st) {
    if (!a.f32) return launch_chunk_fwd16(a, ws, st, true);
    return a.Dk == 128 ? launch_two<128, true>(a, ws, st) : launch_two<64, true>(a, ws, st);
}

// ---------------------------------------------------------------------------- T-windows in a fixed scratch
// Each window covers tokens [t0, t0 + W*64) of every sequence: its pointers are offset by t0 tokens,
// its sequences start T tokens apart (T_stride) and are at most W*64 tokens long (T_fixed), so the
// records of one window occupy B * W * H record slots.  The chain carries the state from window to
// window in fp32 exactly as it does from chunk to chunk (read at a workgroup's start, written at its
// end), so the results equal those of the whole-sequence call bit for bit.
static int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t chunk_window_state_bytes(const ChunkArgs& a) {
    return a.s_final ? 0 : round256(a.N * a.H * (int64_t)a.Dk * a.Dv * 4);
}

int64_t chunk_window_chunks(const ChunkArgs& a, int64_t scratch_bytes) {
    const int64_t per_chunk = a.N * a.H * (a.f32 ? chunk_record_bytes(a.Dk, true) : chunk16_record_bytes(a.Dk));
    const int64_t room = scratch_bytes - chunk_window_state_bytes(a);
    if (per_chunk <= 0 || room < per_chunk) return 0;
    const int64_t nch = (a.T_fixed + kC - 1) / kC;
    return std::min<int64_t>(room / per_chunk, std::max<int64_t>(nch, 1));
}

hipError_t launch_chunk_fwd_windows(const ChunkArgs& a, char* scratch, int64_t scratch_bytes, hipStream_t st) {
    const int64_t W = chunk_window_chunks(a, scratch_bytes);
    if (W <= 0 || a.cu_seqlens || a.T_fixed <= 0) return hipErrorInvalidValue;
    float* carry = a.s_final ? a.s_final : reinterpret_cast<float*>(scratch);
    char* recs = scratch + chunk_window_state_bytes(a);
    const int64_t qk_es = a.f32 ? 4 : 2, g_es = a.pro.g_bf16 ? 2 : 4, b_es = a.pro.b_bf16 ? 2 : 4;
    for (int64_t t0 = 0; t0 < a.T_fixed; t0 += W * kC) {
        ChunkArgs w = a;
        w.T_fixed = std::min<int64_t>(W * kC, a.T_fixed - t0);
        w.T_stride = a.T_fixed;
        const int64_t tk = t0 * a.H;  // token offset times heads
        w.q = static_cast<const char*>(a.q) + tk * a.Dk * qk_es;
        w.k = static_cast<const char*>(a.k) + tk * a.Dk * qk_es;
        w.v = static_cast<const char*>(a.v) + tk * a.Dv * qk_es;
        w.g = static_cast<const char*>(a.g) + tk * a.Dk * g_es;
        w.beta = static_cast<const char*>(a.beta) + tk * b_es;
        w.o = a.o + tk * a.Dv;
        w.s0 = t0 == 0 ? a.s0 : carry;
        w.s_final = carry;
        hipError_t e;
        if (!a.f32) e = launch_chunk_fwd16(w, recs, st, false);
        else e = a.Dk == 128 ? launch_two<128, true>(w, recs, st, false) : launch_two<64, true>(w, recs, st, false);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace kda
