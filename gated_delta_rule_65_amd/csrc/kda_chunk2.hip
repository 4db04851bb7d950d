// Two-kernel chunked forward pass for gfx950 (used when the caller passes a workspace).
//
// The chunked form of the gated delta rule ("Kimi K3 Open Model Surpasses Closed
// GPT and Anthropic Systems on Independent Benchmarks", worldcybernews, second and
// third paragraphs; see kda_chunk.hip for the equations) splits into work that does
// not depend on the carried state S and a short state-dependent chain:
//
//   state independent, per chunk:  G (running sum of clamped g, log2 units),
//       A and P (decay-folded Gram blocks), M^{-1} = (I + A)^{-1}
//   state dependent, per chunk:    X = b (V - (e^G k) S),  U = M^{-1} X,
//       O = (e^G q) S + P U,  S' = Diag(e^{G_C}) S + (e^{G_C - G} k)^T U
//
// prep_kernel runs the first part for every (chunk, head) at once, one workgroup
// each and two workgroups per CU, and writes G, M^{-1} and P to the workspace.
// chain_kernel walks the chunks of one (sequence, head, 32-column slice) in order
// and only runs the state-dependent products, with four barriers per chunk.
//
// Workspace record per (chunk slot, head): G fp32 [64][Dk]; then M^{-1} and P as
// [64][64] planes (bf16 hi, bf16 lo for bf16 inputs; fp32 for fp32 inputs).
// Chunk slots: equal-length sequences use n * ceil(T/64) + j; packed sequences use
// floor(cu[n]/64) + n + j, which is unique and below floor(total/64) + N.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC = 64;      // tokens per chunk
constexpr int kS = 32;      // state columns per chain workgroup
constexpr float kL2e = 1.4426950408889634f;

template <int DK>
__host__ __device__ constexpr int64_t record_bytes() {
    return 64 * DK * 4 + 2 * 64 * 64 * 4;
}

// Sequence range and chunk slot of (sequence n, chunk j).
struct SeqRange {
    int64_t start, end;
};

__device__ __forceinline__ SeqRange seq_range(const int32_t* cu, int64_t n, int64_t T_fixed, int64_t total) {
    SeqRange s;
    if (cu) {
        s.start = min<int64_t>(max<int64_t>(cu[n], 0), total);
        s.end = min<int64_t>(max<int64_t>(cu[n + 1], s.start), total);
    } else {
        s.start = n * T_fixed;
        s.end = s.start + T_fixed;
    }
    return s;
}

__device__ __forceinline__ int64_t slot_of(const int32_t* cu, int64_t n, int64_t j, int64_t T_fixed, int64_t start) {
    if (cu) return start / kC + n + j;
    return n * ((T_fixed + kC - 1) / kC) + j;
}

// 16-bit / 32-bit stores of one element of a [64][64] plane pair.
template <bool F32>
__device__ __forceinline__ void ws_store1(char* planes, int row, int col, float x) {
    if constexpr (F32) {
        reinterpret_cast<float*>(planes)[row * 64 + col] = x;
    } else {
        __bf16* p = reinterpret_cast<__bf16*>(planes);
        const __bf16 h = (__bf16)x;
        p[row * 64 + col] = h;
        p[4096 + row * 64 + col] = (__bf16)(x - (float)h);
    }
}

// MFMA operand fragment (eight consecutive columns of one row) of a [64][64] plane pair.
template <bool F32>
__device__ __forceinline__ Frag<F32> ws_frag(const char* planes, int row, int col) {
    Frag<F32> f;
    if constexpr (F32) {
        const float* p = reinterpret_cast<const float*>(planes) + row * 64 + col;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    } else {
        const __bf16* p = reinterpret_cast<const __bf16*>(planes) + row * 64 + col;
        f.hi = *reinterpret_cast<const bf16x8_t*>(p);
        f.lo = *reinterpret_cast<const bf16x8_t*>(p + 4096);
    }
    return f;
}

}  // namespace

// ============================================================================ prep kernel

template <int DK>
struct PrepLds {
    static constexpr int COL = 0;                            // fp32 k e^{G_end(blk)-G}, sub-blocks 0..2 [48][DK+4]
    static constexpr int A = COL + 48 * (DK + 4) * 4;        // fp32 b_r A_ri [64][68]
    static constexpr int D = A + 64 * 68 * 4;                // fp32 diagonal inverses [4][16][17]
    static constexpr int TAB = D + 4 * 16 * 17 * 4;          // fp32 tables [11][DK]
    static constexpr int GT = TAB + 11 * DK * 4;             // fp32 sub-block sums (log2) [4][DK]
    static constexpr int BETA = GT + 4 * DK * 4;             // fp32 b [64]
    static constexpr int TOTAL = BETA + 64 * 4;
    static_assert(TOTAL <= 80 * 1024, "two prep workgroups per CU");
};

// Gram row block W (rows 16W..16W+15): A (one pass) into sA (scaled by b_r, strictly lower on
// the diagonal block), P (full precision) stored to the workspace planes, all blocks I <= W.
template <int W, int DK, bool F32>
__device__ __forceinline__ void prep_gram(const float (*qf)[8], const float (*kf)[8], const float (*E)[8],
                                          const float (*Ei)[8], const float* sCol, const float* tD,
                                          const float* sBeta, float* sA, char* wsP, int m, int cg) {
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
        fkE.set_hi_only(x2);
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
            accA[I] = mma_fast(accA[I], fkE, colf);
            accP[I] = mma_full(accP[I], fqE, colf);
        }
        accA[W] = mma_fast(accA[W], fkE, fkd);
        accP[W] = mma_full(accP[W], fqE, fkd);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int rr = 4 * cg + jj;
            const int gr = 16 * W + rr, gi = 16 * I + m;
            if (I <= W) {
                float a = accA[I][jj], pv = accP[I][jj];
                if (I == W) {
                    if (m >= rr) a = 0.f;
                    if (m > rr) pv = 0.f;
                }
                sA[gr * 68 + gi] = a * sBeta[gr];
                ws_store1<F32>(wsP, gr, gi, pv);
            } else {
                ws_store1<F32>(wsP, gr, gi, 0.f);
            }
        }
    }
}

template <int DK, bool F32>
__global__ __launch_bounds__(256, 2) void prep_kernel(const void* __restrict__ qv, const void* __restrict__ kv,
                                                      const float* __restrict__ g, const float* __restrict__ beta,
                                                      const int32_t* __restrict__ cu_seqlens, int64_t T_fixed,
                                                      int64_t total, int64_t N, int H, char* __restrict__ ws) {
    using In = typename std::conditional<F32, float, uint16_t>::type;
    using L = PrepLds<DK>;
    constexpr int KS = DK / 32;
    constexpr int64_t RB = record_bytes<DK>();
    const In* __restrict__ q = static_cast<const In*>(qv);
    const In* __restrict__ k = static_cast<const In*>(kv);

    __shared__ __align__(16) char smem[L::TOTAL];
    float* sCol = reinterpret_cast<float*>(smem + L::COL);
    float* sA = reinterpret_cast<float*>(smem + L::A);
    float* sD = reinterpret_cast<float*>(smem + L::D);
    float* tCum = reinterpret_cast<float*>(smem + L::TAB);  // sum_{J<w} Gt_J (log2)  [4][DK]
    float* tBt = tCum + 4 * DK;                             // e^{Gt_w}               [4][DK]
    float* tD = tBt + 4 * DK;                               // e^{sum_{I<J<R} Gt_J}   [3][DK]
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
    const SeqRange sr = seq_range(cu_seqlens, n, T_fixed, total);
    const int64_t t0 = sr.start + j * kC;
    if (j < 0 || t0 >= sr.end) return;  // unused slot
    const int nt = (int)min<int64_t>(kC, sr.end - t0);
    char* rec = ws + (slot * H + h) * RB;
    float* wsG = reinterpret_cast<float*>(rec);
    char* wsN = rec + 64 * DK * 4;
    char* wsP = wsN + 64 * 64 * 4;

    const int r = 16 * w + m;
    const bool rv = r < nt;
    const int64_t base = ((t0 + min(r, nt - 1)) * H + h) * (int64_t)DK + 8 * cg;
    float qf[KS][8], kf[KS][8], gl[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        load8_as_float(q + base + 32 * s, qf[s]);
        load8_as_float(k + base + 32 * s, kf[s]);
        load8_as_float(g + base + 32 * s, gl[s]);
    }
    if (tid < kC) sBeta[tid] = (tid < nt) ? beta[(t0 + tid) * H + h] : 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            gl[s][jj] = row16_inclusive_scan(rv ? __builtin_amdgcn_fmed3f(gl[s][jj], -5.f, 0.f) * kL2e : 0.f);
    if (m == 15) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float* dst = &sGt[w * DK + 32 * s + 8 * cg];
            *reinterpret_cast<float4*>(dst) = make_float4(gl[s][0], gl[s][1], gl[s][2], gl[s][3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(gl[s][4], gl[s][5], gl[s][6], gl[s][7]);
        }
    }
    lds_barrier();
    if (tid < DK) {
        const int c = tid;
        const float G0 = sGt[c], G1 = sGt[DK + c], G2 = sGt[2 * DK + c], G3 = sGt[3 * DK + c];
        tCum[c] = 0.f;
        tCum[DK + c] = G0;
        tCum[2 * DK + c] = G0 + G1;
        tCum[3 * DK + c] = G0 + G1 + G2;
        tBt[c] = __builtin_amdgcn_exp2f(G0);
        tBt[DK + c] = __builtin_amdgcn_exp2f(G1);
        tBt[2 * DK + c] = __builtin_amdgcn_exp2f(G2);
        tBt[3 * DK + c] = __builtin_amdgcn_exp2f(G3);
        tD[c] = __builtin_amdgcn_exp2f(G1);
        tD[DK + c] = __builtin_amdgcn_exp2f(G2);
        tD[2 * DK + c] = __builtin_amdgcn_exp2f(G1 + G2);
    }
    lds_barrier();

    // per-element factors; G to the workspace; Gram column operands to LDS
    float Ei[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int c0 = 32 * s + 8 * cg;
        float cum[8], bt[8], gout[8], xkf[8];
        lds_read8(&tCum[w * DK + c0], cum);
        lds_read8(&tBt[w * DK + c0], bt);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            gout[jj] = cum[jj] + gl[s][jj];
            const float E = __builtin_amdgcn_exp2f(gl[s][jj]);
            Ei[s][jj] = __builtin_amdgcn_exp2f(-gl[s][jj]);
            gl[s][jj] = E;
            xkf[jj] = kf[s][jj] * (bt[jj] * Ei[s][jj]);
        }
        float* gdst = wsG + r * DK + c0;
        *reinterpret_cast<float4*>(gdst) = make_float4(gout[0], gout[1], gout[2], gout[3]);
        *reinterpret_cast<float4*>(gdst + 4) = make_float4(gout[4], gout[5], gout[6], gout[7]);
        if (w < 3) {
            float* dst = sCol + r * (DK + 4) + c0;
            *reinterpret_cast<float4*>(dst) = make_float4(xkf[0], xkf[1], xkf[2], xkf[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(xkf[4], xkf[5], xkf[6], xkf[7]);
        }
    }
    lds_barrier();

    switch (w) {
        case 0: prep_gram<0, DK, F32>(qf, kf, gl, Ei, sCol, tD, sBeta, sA, wsP, m, cg); break;
        case 1: prep_gram<1, DK, F32>(qf, kf, gl, Ei, sCol, tD, sBeta, sA, wsP, m, cg); break;
        case 2: prep_gram<2, DK, F32>(qf, kf, gl, Ei, sCol, tD, sBeta, sA, wsP, m, cg); break;
        default: prep_gram<3, DK, F32>(qf, kf, gl, Ei, sCol, tD, sBeta, sA, wsP, m, cg); break;
    }
    lds_barrier();

    // diagonal blocks of M^{-1} = (I + A)^{-1}: forward substitution, one column per lane
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
    lds_barrier();

    // column block I = w of M^{-1}: N_II = D_I, N_RI = -D_R sum_{J=I}^{R-1} A_RJ N_JI (fp32 MFMA),
    // each 16x16 result (lane: column m, rows 4cg..4cg+3) feeding the next product as B operand
    {
        const int I = w;
        f32x4_t Nr[4];
#pragma unroll
        for (int R = 0; R < 4; ++R) Nr[R] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int R = 0; R < 4; ++R) {
            f32x4_t nv = {0.f, 0.f, 0.f, 0.f};
            if (R == I) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) nv[jj] = sD[(I * 16 + 4 * cg + jj) * 17 + m];
            } else if (R > I) {
                f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int J = 0; J < 3; ++J) {
                    if (J < I || J >= R) continue;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        z = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[(16 * R + m) * 68 + 16 * J + 4 * cg + jj],
                                                                 Nr[J][jj], z, 0, 0, 0);
                }
                f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    y = __builtin_amdgcn_mfma_f32_16x16x4f32(sD[(R * 16 + m) * 17 + 4 * cg + jj], z[jj], y, 0, 0, 0);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) nv[jj] = -y[jj];
            }
            Nr[R] = nv;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ws_store1<F32>(wsN, 16 * R + 4 * cg + jj, 16 * I + m, nv[jj]);
        }
    }
}

// ============================================================================ chain kernel

template <int DK, bool F32>
struct ChainLds {
    using MS = LMat<F32, kS, DK>;   // S^T           [n][c]
    using MKB = LMat<F32, DK, kC>;  // Kbar^T        [c][t]
    using MX = LMat<F32, kS, kC>;   // (b(V - Kt S))^T [n][t]
    using MU = LMat<F32, kS, kC>;   // U^T           [n][t]
    static constexpr int S = 0;
    static constexpr int KB = S + MS::BYTES;
    static constexpr int X = KB + MKB::BYTES;
    static constexpr int U = X + MX::BYTES;
    static constexpr int GCL = U + MU::BYTES;   // fp32 G_C (log2) [DK]
    static constexpr int GC = GCL + DK * 4;     // fp32 gamma_C    [DK]
    static constexpr int BETA = GC + DK * 4;    // fp32 b          [64]
    static constexpr int TOTAL = BETA + 64 * 4;
    static_assert(TOTAL <= 96 * 1024, "chain LDS");
};

template <int DK, bool F32>
__global__ __launch_bounds__(256, 1) void chain_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, const void* __restrict__ vv,
    const float* __restrict__ beta, const float* s0, float* __restrict__ o, float* s_final,
    const int32_t* __restrict__ cu_seqlens, int64_t T_fixed, int64_t total, int64_t N, int H, int Dv,
    const char* __restrict__ ws) {
    using In = typename std::conditional<F32, float, uint16_t>::type;
    using Fr = Frag<F32>;
    using L = ChainLds<DK, F32>;
    constexpr int KS = DK / 32;
    constexpr int CBW = DK / 64;
    constexpr int64_t RB = record_bytes<DK>();
    const In* __restrict__ q = static_cast<const In*>(qv);
    const In* __restrict__ k = static_cast<const In*>(kv);
    const In* __restrict__ v = static_cast<const In*>(vv);

    __shared__ __align__(16) char smem[L::TOTAL];
    char* pS = smem + L::S;
    char* pKB = smem + L::KB;
    char* pX = smem + L::X;
    char* pU = smem + L::U;
    float* sGCl = reinterpret_cast<float*>(smem + L::GCL);
    float* sGC = reinterpret_cast<float*>(smem + L::GC);
    float* sBeta = reinterpret_cast<float*>(smem + L::BETA);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    const int NS = Dv / kS;
    const int64_t pairs = N * (int64_t)H;
    const int64_t bid = blockIdx.x;
    const int64_t loc = bid >> 3;
    const int sl = (int)(loc % NS);
    const int64_t pr = (loc / NS) * 8 + (bid & 7);  // slices of one head on one XCD
    if (pr >= pairs) return;
    const int64_t n = pr / H;
    const int h = (int)(pr % H);
    const SeqRange sr = seq_range(cu_seqlens, n, T_fixed, total);
    const int64_t start = sr.start, end = sr.end;
    const int col0 = sl * kS;

    // initial state (wave w: channel blocks w*CBW.., both 16-column halves)
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
            lds_store4<F32, kS, DK>(pS, 16 * nb + m, 16 * cb + 4 * cg, accS[ci][nb]);
        }
    }

    const int r = 16 * w + m;
    const int nk = (w >= 2) ? 2 : 1;  // 32-token steps of M^{-1} / P rows that reach the diagonal
    const uint32_t rs_k = (uint32_t)H * DK, rs_v = (uint32_t)H * (uint32_t)Dv;
    const In* __restrict__ q_l = q + (int64_t)h * DK + 8 * cg;
    const In* __restrict__ k_l = k + (int64_t)h * DK + 8 * cg;
    const In* __restrict__ v_l = v + (int64_t)h * Dv + col0 + m;
    const float* __restrict__ b_l = beta + h;
    float* __restrict__ o_l = o + (int64_t)h * Dv + col0 + m;

    // prefetch registers for one chunk
    Raw8<F32> pq[KS], pk[KS];
    Raw8<true> pg[KS];
    In pv[2][4];
    float pb = 0.f;
    Fr pN[2], pP[2];
    auto prefetch = [&](int64_t t0, int nt, int64_t jc) {
        const char* rec = ws + (slot_of(cu_seqlens, n, jc, T_fixed, start) * H + h) * RB;
        const float* G = reinterpret_cast<const float*>(rec) + r * DK + 8 * cg;
        const int64_t cq = t0 * (int64_t)rs_k;
        const uint32_t rq = (uint32_t)min(r, nt - 1) * rs_k;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            load_raw8(G + 32 * s, pg[s]);
            load_raw8(q_l + cq + rq + 32 * s, pq[s]);
            load_raw8(k_l + cq + rq + 32 * s, pk[s]);
        }
        const int64_t cv = t0 * (int64_t)rs_v;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const uint32_t rvo = (uint32_t)min(16 * w + 4 * cg + jj, nt - 1) * rs_v;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) pv[nb][jj] = v_l[cv + rvo + 16 * nb];
        }
        pb = b_l[t0 * H + (uint32_t)min(tid & 63, nt - 1) * (uint32_t)H];
        const char* planesN = rec + 64 * DK * 4;
        const char* planesP = planesN + 64 * 64 * 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // rows 16w..16w+15 only reach tokens below 32*nk; the other step is not needed
            const int kk = min(kb, nk - 1);
            pN[kb] = ws_frag<F32>(planesN, r, 32 * kk + 8 * cg);
            pP[kb] = ws_frag<F32>(planesP, r, 32 * kk + 8 * cg);
        }
    };

    f32x4_t oPrev[2];
    auto store_o = [&](int64_t tc, int ntc) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 16 * w + 4 * cg + jj;
                if (rr < ntc) o_l[tc * (int64_t)rs_v + (uint32_t)rr * rs_v + 16 * nb] = oPrev[nb][jj];
            }
    };

    if (start < end) prefetch(start, (int)min<int64_t>(kC, end - start), 0);
    lds_barrier();

    int64_t jc = 0;
    for (int64_t t0 = start; t0 < end; t0 += kC, ++jc) {
        const int nt = (int)min<int64_t>(kC, end - t0);
        const bool more = t0 + kC < end;
        const int64_t t0n = more ? t0 + kC : t0;
        const int ntn = more ? (int)min<int64_t>(kC, end - t0 - kC) : nt;
        const int64_t jn = more ? jc + 1 : jc;

        // ---- take this chunk's prefetched inputs
        float G[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s) raw8_to_float<true>(pg[s], G[s]);
        float vD[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if constexpr (F32) vD[nb][jj] = pv[nb][jj];
                else vD[nb][jj] = bf16_bits_to_float(pv[nb][jj]);
            }
        Fr fN[2], fP[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            fN[kb] = pN[kb];
            fP[kb] = pP[kb];
        }
        const float bval = (tid < nt) ? pb : 0.f;
        if (tid < kC) sBeta[tid] = bval;
        if (r == 63) {  // the chunk's total decay per channel (G of its last row)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                float* dst = &sGCl[32 * s + 8 * cg];
                *reinterpret_cast<float4*>(dst) = make_float4(G[s][0], G[s][1], G[s][2], G[s][3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(G[s][4], G[s][5], G[s][6], G[s][7]);
            }
        }
        lds_barrier();  // (1)

        // ---- operands and chain 1:  X = b (V - Kt S) (one pass), O1 = Qt S (full)
        float qf[KS][8], kf[KS][8];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            raw8_to_float<F32>(pq[s], qf[s]);
            raw8_to_float<F32>(pk[s], kf[s]);
        }
        if (tid < DK) sGC[tid] = __builtin_amdgcn_exp2f(sGCl[tid]);
        prefetch(t0n, ntn, jn);  // next chunk (the current one again on the last chunk)
        f32x4_t accO[2], accX[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) accX[nb] = accO[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const int c0 = 32 * s + 8 * cg;
            float gc[8], xq[8], xk[8], xb[8];
            lds_read8(&sGCl[c0], gc);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const float gam = __builtin_amdgcn_exp2f(G[s][jj]);            // e^{G_r}
                const float gbar = __builtin_amdgcn_exp2f(gc[jj] - G[s][jj]);  // e^{G_C - G_r}
                xq[jj] = qf[s][jj] * gam;
                xk[jj] = kf[s][jj] * gam;
                xb[jj] = kf[s][jj] * gbar;
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) lds_store1<F32, DK, kC>(pKB, c0 + jj, r, xb[jj]);
            Fr fQt, fKt;
            fQt.set(xq);
            fKt.set_hi_only(xk);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const Fr sf = lds_frag<F32, kS, DK>(pS, 16 * nb + m, c0);
                accX[nb] = mma_fast(accX[nb], fKt, sf);
                accO[nb] = mma_full(accO[nb], fQt, sf);
            }
        }
        if (t0 > start) store_o(t0 - kC, kC);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            f32x4_t xv;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int rr = 16 * w + 4 * cg + jj;
                xv[jj] = sBeta[rr] * (vD[nb][jj] - accX[nb][jj]);
            }
            lds_store4<F32, kS, kC>(pX, 16 * nb + m, 16 * w + 4 * cg, xv);
        }
        lds_barrier();  // (2)

        // ---- chain 2: U = M^{-1} X (rows of sub-block w)
        {
            f32x4_t accU[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb >= nk) continue;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const Fr xf = lds_frag<F32, kS, kC>(pX, 16 * nb + m, 32 * kb + 8 * cg);
                    accU[nb] = mma_full(accU[nb], fN[kb], xf);
                }
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) lds_store4<F32, kS, kC>(pU, 16 * nb + m, 16 * w + 4 * cg, accU[nb]);
        }
        lds_barrier();  // (3)

        // ---- chain 3: O = O1 + P U, S = gamma_C S + Kbar^T U
        {
            Fr uf[2][2];
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) uf[nb][kb] = lds_frag<F32, kS, kC>(pU, 16 * nb + m, 32 * kb + 8 * cg);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb >= nk) continue;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) accO[nb] = mma_full(accO[nb], fP[kb], uf[nb][kb]);
            }
#pragma unroll
            for (int ci = 0; ci < CBW; ++ci) {
                const int cb = w * CBW + ci;
                float gcv[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) gcv[jj] = sGC[16 * cb + 4 * cg + jj];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) accS[ci][nb][jj] *= gcv[jj];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const Fr af = lds_frag<F32, DK, kC>(pKB, 16 * cb + m, 32 * kb + 8 * cg);
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) accS[ci][nb] = mma_full(accS[ci][nb], af, uf[nb][kb]);
                }
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) lds_store4<F32, kS, DK>(pS, 16 * nb + m, 16 * cb + 4 * cg, accS[ci][nb]);
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) oPrev[nb] = accO[nb];
        }
        lds_barrier();  // (4)
    }
    if (start < end) {
        const int64_t t_last = start + ((end - start - 1) / kC) * kC;
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

// ============================================================================ host side

int64_t chunk_slots(const ChunkArgs& a) {
    if (a.cu_seqlens) return a.total / kC + a.N;
    return a.N * ((a.T_fixed + kC - 1) / kC);
}

int64_t chunk_workspace_bytes(const ChunkArgs& a) {
    const int64_t rb = a.Dk == 128 ? record_bytes<128>() : record_bytes<64>();
    return chunk_slots(a) * a.H * rb;
}

template <int DK, bool F32>
static hipError_t launch_two(const ChunkArgs& a, void* ws, hipStream_t st) {
    const int64_t prep_grid = chunk_slots(a) * a.H;
    if (prep_grid > 0)
        hipLaunchKernelGGL((prep_kernel<DK, F32>), dim3((unsigned)prep_grid), dim3(256), 0, st, a.q, a.k, a.g, a.beta,
                           a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, static_cast<char*>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t grid = chunk_grid_size(a.N, a.H, a.Dv);
    hipLaunchKernelGGL((chain_kernel<DK, F32>), dim3((unsigned)grid), dim3(256), 0, st, a.q, a.k, a.v, a.beta, a.s0,
                       a.o, a.s_final, a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv,
                       static_cast<const char*>(ws));
    return hipGetLastError();
}

hipError_t launch_chunk_fwd_two_pass(const ChunkArgs& a, void* ws, hipStream_t st) {
    if (a.Dk == 128) return a.f32 ? launch_two<128, true>(a, ws, st) : launch_two<128, false>(a, ws, st);
    return a.f32 ? launch_two<64, true>(a, ws, st) : launch_two<64, false>(a, ws, st);
}

}  // namespace kda
