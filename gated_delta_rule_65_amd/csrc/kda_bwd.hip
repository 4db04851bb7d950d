// Backward pass of the gated delta rule for gfx950: gradients of the outputs o and of the final
// state with respect to q, k, v, g (log alpha, before the clamp), beta and the initial state.
// The pages describe the forward recurrence only ("Kimi K3 Open Model Surpasses Closed GPT and
// Anthropic Systems on Independent Benchmarks", worldcybernews, second paragraph); the gradients
// below are derived from the chunked form of that recurrence (kda_chunk.hip).
//
// Forward per chunk (C = 64 tokens, S the state at the chunk start, G the running sum of the
// clamped log gates inside the chunk, Gam = e^G, Gbar = e^{G_C - G}, gamma = e^{G_C}):
//   Qt = Gam q, Kt = Gam k, Kb = Gbar k,
//   Abar_ri = sum_c k_rc k_ic e^{G_rc - G_ic} (i < r),  P_ri = sum_c q_rc k_ic e^{G_rc - G_ic} (i <= r),
//   Minv = (I + Diag(b) Abar)^{-1},  X = V - Kt S,  U = Minv Diag(b) X,
//   O = Qt S + P U,  S' = Diag(gamma) S + Kb^T U.
// Backward, given dO and dS' (the gradient at the chunk end):
//   dU = P^T dO + Kb dS',  dX = Diag(b) Minv^T dU,  dV = dX,
//   dS = Qt^T dO + Diag(gamma) dS' - Kt^T dX                     (carried to the previous chunk)
//   dQt = dO S^T, dKt = -dX S^T, dKb = U dS'^T, dgamma = rowsum(S o dS'),
//   dP = tril(dO U^T), dN = tril(dU X^T) for N = Minv Diag(b):
//     db_i += sum_r dN_ri Minv_ri,  dM = -Minv^T (dN Diag(b)) Minv^T,
//     dAbar = strict_tril(Diag(b) dM),  db_r += sum_{i<r} dM_ri Abar_ri,
//   then through Abar, P, Qt, Kt, Kb and gamma to q, k and G, and from G to g by a reverse
//   running sum inside the chunk (the clamp passes the gradient where -5 <= g <= 0).
//
// Qt, Kt, Kb, P, Minv, Abar, gamma, b per (chunk, head) and the state at every chunk start come from
// the forward pass's prep kernel in its backward form and its chain kernel in mode 3, both with fp32
// records (launch_chunk_states).  Then three kernels, fp32 arithmetic, 256 threads each:
//   bwd_dstates_kernel per (sequence, head, 32 state columns), chunks in reverse: dS' of every chunk, ds0
//   bwd_grad_a_kernel  per (chunk, head): dv and the sums over value columns (dQt, dKt, dKb, dP, dN, dgamma)
//   bwd_grad_b_kernel  per (chunk, head): through the inverse, the decayed Gram blocks and the gates
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kBC = 64;  // tokens per chunk
constexpr int kBS = 32;  // state columns per chain workgroup

template <int DK>
using BRec = BwdRec<DK>;
// Per (chunk, head) output of bwd_grad_a (float offsets).
template <int DK>
struct GRec {
    static constexpr int DQT = 0, DKT = 64 * DK, DKB = 128 * DK, DP = 192 * DK, DN = DP + 4096, DGM = DN + 4096,
                         FLOATS = DGM + DK;
    static_assert(FLOATS % 64 == 0, "records stay 256-byte aligned");
};

struct BSeq {
    int64_t start, end;
};

__device__ __forceinline__ BSeq bseq(const int32_t* cu, int64_t n, int64_t T_fixed, int64_t total) {
    BSeq s;
    if (cu) {
        s.start = min<int64_t>(max<int64_t>(cu[n], 0), total);
        s.end = min<int64_t>(max<int64_t>(cu[n + 1], s.start), total);
    } else {
        s.start = n * T_fixed;
        s.end = s.start + T_fixed;
    }
    return s;
}

// chunk slot of chunk j of sequence n (as in the forward workspace)
__device__ __forceinline__ int64_t bslot(const int32_t* cu, int64_t n, int64_t j, int64_t T_fixed, int64_t start) {
    if (cu) return start / kBC + n + j;
    return n * ((T_fixed + kBC - 1) / kBC) + j;
}

// slot -> (sequence, chunk); false for an unused slot
__device__ __forceinline__ bool slot_chunk(const int32_t* cu, int64_t slot, int64_t T_fixed, int64_t total, int64_t N,
                                           int64_t& n, int64_t& t0, int& nt) {
    int64_t j;
    if (cu) {
        int64_t lo = 0, hi = N - 1;  // largest n with floor(cu[n]/64) + n <= slot
        while (lo < hi) {
            const int64_t mid = (lo + hi + 1) >> 1;
            const int64_t f = min<int64_t>(max<int64_t>(cu[mid], 0), total) / kBC + mid;
            if (f <= slot) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
        j = slot - (min<int64_t>(max<int64_t>(cu[n], 0), total) / kBC + n);
    } else {
        const int64_t nch = (T_fixed + kBC - 1) / kBC;
        n = slot / nch;
        j = slot % nch;
    }
    const BSeq sr = bseq(cu, n, T_fixed, total);
    t0 = sr.start + j * kBC;
    if (j < 0 || t0 >= sr.end) return false;
    nt = (int)min<int64_t>(kBC, sr.end - t0);
    return true;
}

template <bool F32>
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
    if constexpr (F32) return static_cast<const float*>(p)[i];
    else return bf16_bits_to_float(static_cast<const uint16_t*>(p)[i]);
}

// chain workgroups: the slices of one (sequence, head) sit on one XCD
__device__ __forceinline__ bool chain_item(int64_t items, int NS, int64_t& pr, int& sl) {
    const int64_t bid = blockIdx.x;
    const int64_t loc = bid >> 3;
    sl = (int)(loc % NS);
    pr = (loc / NS) * 8 + (bid & 7);
    return pr < items;
}

}  // namespace

// ============================================================================ state gradients, in reverse

template <int DK>
__global__ __launch_bounds__(256, 1) void bwd_dstates_kernel(const float* __restrict__ d_o,
                                                             const float* __restrict__ d_sfinal, float* ds0,
                                                             const int32_t* __restrict__ cu, int64_t T_fixed,
                                                             int64_t total, int64_t N, int H, int Dv,
                                                             const float* __restrict__ recs,
                                                             float* __restrict__ dstates) {
    using R = BRec<DK>;
    constexpr int LD = DK + 1;
    constexpr int TPC = 256 / DK, CPT = kBS / TPC;
    __shared__ float sD[DK * kBS], sO[64 * kBS], sDU[64 * kBS], sDX[64 * kBS], sM1[64 * LD], sM2[64 * LD],
        sMI[64 * 65], sB[64], sGm[DK];
    const int tid = threadIdx.x;
    int64_t pr;
    int sl;
    if (!chain_item(N * (int64_t)H, Dv / kBS, pr, sl)) return;
    const int64_t n = pr / H;
    const int h = (int)(pr % H);
    const BSeq sr = bseq(cu, n, T_fixed, total);
    const int64_t nch = (sr.end - sr.start + kBC - 1) / kBC;
    const int col0 = sl * kBS;

    for (int e = tid; e < DK * kBS; e += 256) {
        const int c = e / kBS, jj = e % kBS;
        sD[e] = d_sfinal ? d_sfinal[((n * H + h) * DK + c) * (int64_t)Dv + col0 + jj] : 0.f;
    }
    __syncthreads();
    const int xr = tid >> 2, xj = (tid & 3) * 8;
    const int sc = tid / TPC, sj = (tid % TPC) * CPT;
    for (int64_t jc = nch - 1; jc >= 0; --jc) {
        const int64_t slot = bslot(cu, n, jc, T_fixed, sr.start);
        const float* rec = recs + (slot * H + h) * (int64_t)R::FLOATS;
        float* dst = dstates + (slot * H + h) * (int64_t)DK * Dv;
        const int64_t t0 = sr.start + jc * kBC;
        const int nt = (int)min<int64_t>(kBC, sr.end - t0);
        for (int e = tid; e < DK * kBS; e += 256) dst[(e / kBS) * (int64_t)Dv + col0 + e % kBS] = sD[e];
        for (int e = tid; e < 64 * kBS; e += 256) {
            const int r = e / kBS;
            sO[e] = r < nt ? d_o[((t0 + r) * H + h) * (int64_t)Dv + col0 + e % kBS] : 0.f;
        }
        for (int e = tid; e < 64 * DK; e += 256) sM1[(e / DK) * LD + e % DK] = rec[R::KB + e];
        for (int e = tid; e < 4096; e += 256) {
            sM2[(e >> 6) * 65 + (e & 63)] = rec[R::PM + e];
            sMI[(e >> 6) * 65 + (e & 63)] = rec[R::MI + e];
        }
        if (tid < 64) sB[tid] = rec[R::BT + tid];
        if (tid < DK) sGm[tid] = rec[R::GM + tid];
        __syncthreads();
        {  // dU = P^T dO + Kb dS'
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int r = xr; r < 64; ++r) {
                const float p = sM2[r * 65 + xr];
#pragma unroll
                for (int m = 0; m < 8; ++m) acc[m] = fmaf(p, sO[r * kBS + xj + m], acc[m]);
            }
            for (int c = 0; c < DK; ++c) {
                const float kb = sM1[xr * LD + c];
#pragma unroll
                for (int m = 0; m < 8; ++m) acc[m] = fmaf(kb, sD[c * kBS + xj + m], acc[m]);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) sDU[xr * kBS + xj + m] = acc[m];
        }
        __syncthreads();
        {  // dX = Diag(b) Minv^T dU
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int r = xr; r < 64; ++r) {
                const float mi = sMI[r * 65 + xr];
#pragma unroll
                for (int m = 0; m < 8; ++m) acc[m] = fmaf(mi, sDU[r * kBS + xj + m], acc[m]);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) sDX[xr * kBS + xj + m] = sB[xr] * acc[m];
        }
        for (int e = tid; e < 64 * DK; e += 256) {  // Kb and P were last read before the barrier above
            sM1[(e / DK) * LD + e % DK] = rec[R::QT + e];
            sM2[(e / DK) * LD + e % DK] = rec[R::KT + e];
        }
        __syncthreads();
        {  // dS = Diag(gamma) dS' + Qt^T dO - Kt^T dX
            float acc[CPT];
#pragma unroll
            for (int m = 0; m < CPT; ++m) acc[m] = sGm[sc] * sD[sc * kBS + sj + m];
            for (int r = 0; r < 64; ++r) {
                const float qt = sM1[r * LD + sc], kt = sM2[r * LD + sc];
#pragma unroll
                for (int m = 0; m < CPT; ++m)
                    acc[m] = fmaf(qt, sO[r * kBS + sj + m], fmaf(-kt, sDX[r * kBS + sj + m], acc[m]));
            }
#pragma unroll
            for (int m = 0; m < CPT; ++m) sD[sc * kBS + sj + m] = acc[m];
        }
        __syncthreads();
    }
    if (ds0)
        for (int e = tid; e < DK * kBS; e += 256)
            ds0[((n * H + h) * DK + e / kBS) * (int64_t)Dv + col0 + e % kBS] = sD[e];
}

// ============================================================================ sums over the value columns

// Per (chunk, head): X, U, dU, dX per 16-column tile of the state, dv, and the products summed over
// all value columns: dQt = dO S^T, dKt = -dX S^T, dKb = U dS'^T (64 x DK), dP = dO U^T,
// dN = dU X^T (64 x 64), dgamma = rowsum(S o dS').  Tiles are stored column-major ([j][row]) so
// that the accumulations read whole rows of them.
template <int DK, bool F32>
__global__ __launch_bounds__(256, 1) void bwd_grad_a_kernel(const void* __restrict__ vv, const float* __restrict__ d_o,
                                                            const int32_t* __restrict__ cu, int64_t T_fixed,
                                                            int64_t total, int64_t N, int H, int Dv,
                                                            const float* __restrict__ recs,
                                                            const float* __restrict__ states,
                                                            const float* __restrict__ dstates,
                                                            float* __restrict__ grads, float* __restrict__ dv) {
    using R = BRec<DK>;
    using GR = GRec<DK>;
    constexpr int LD = DK + 1;  // [64][DK] operands
    constexpr int LT = DK + 4;  // [16][DK] state tiles
    constexpr int LR = 68;      // [16][64] token tiles
    constexpr int CPT = DK / 16;
    __shared__ __align__(16) float sKt[64 * LD], sKb[64 * LD], sP[64 * 65], sMI[64 * 65], sB[64];
    __shared__ __align__(16) float sST[16 * LT], sDST[16 * LT], sOT[16 * LR], sXT[16 * LR], sUT[16 * LR],
        sDUT[16 * LR], sDXT[16 * LR];
    const int tid = threadIdx.x;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    int64_t n, t0;
    int nt;
    if (!slot_chunk(cu, slot, T_fixed, total, N, n, t0, nt)) return;
    const float* rec = recs + (slot * H + h) * (int64_t)R::FLOATS;
    const float* Sg = states + (slot * H + h) * (int64_t)DK * Dv;
    const float* dSg = dstates + (slot * H + h) * (int64_t)DK * Dv;
    float* out = grads + (slot * H + h) * (int64_t)GR::FLOATS;

    for (int e = tid; e < 64 * DK; e += 256) {
        sKt[(e / DK) * LD + e % DK] = rec[R::KT + e];
        sKb[(e / DK) * LD + e % DK] = rec[R::KB + e];
    }
    for (int e = tid; e < 4096; e += 256) {
        sP[(e >> 6) * 65 + (e & 63)] = rec[R::PM + e];
        sMI[(e >> 6) * 65 + (e & 63)] = rec[R::MI + e];
    }
    if (tid < 64) sB[tid] = rec[R::BT + tid];

    const int ar = 4 * (tid >> 4), ac = CPT * (tid & 15), ai = 4 * (tid & 15);  // accumulator block
    const int xr = tid >> 2, xj = 4 * (tid & 3);                              // tile products: row, 4 columns
    float aQ[4][CPT], aK[4][CPT], aB[4][CPT], aP[4][4], aN[4][4], aG = 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < CPT; ++b) aQ[a][b] = aK[a][b] = aB[a][b] = 0.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) aP[a][b] = aN[a][b] = 0.f;
    }

    for (int j0 = 0; j0 < Dv; j0 += 16) {
        for (int e = tid; e < DK * 16; e += 256) {
            const int c = e >> 4, jj = e & 15;
            sST[jj * LT + c] = Sg[c * (int64_t)Dv + j0 + jj];
            sDST[jj * LT + c] = dSg[c * (int64_t)Dv + j0 + jj];
        }
        for (int e = tid; e < 64 * 16; e += 256) {
            const int r = e >> 4, jj = e & 15;
            const int64_t idx = ((t0 + r) * H + h) * (int64_t)Dv + j0 + jj;
            sOT[jj * LR + r] = r < nt ? d_o[idx] : 0.f;
            sXT[jj * LR + r] = r < nt ? load_in<F32>(vv, idx) : 0.f;
        }
        __syncthreads();
        {  // X = V - Kt S
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < DK; ++c) {
                const float kt = sKt[xr * LD + c];
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] = fmaf(kt, sST[(xj + m) * LT + c], acc[m]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) sXT[(xj + m) * LR + xr] -= acc[m];
        }
        __syncthreads();
        {  // U = Minv Diag(b) X;  dU = P^T dO + Kb dS'
            float u[4] = {0.f, 0.f, 0.f, 0.f}, du[4] = {0.f, 0.f, 0.f, 0.f};
            for (int i = 0; i <= xr; ++i) {
                const float wgt = sMI[xr * 65 + i] * sB[i];
#pragma unroll
                for (int m = 0; m < 4; ++m) u[m] = fmaf(wgt, sXT[(xj + m) * LR + i], u[m]);
            }
            for (int r = xr; r < 64; ++r) {
                const float p = sP[r * 65 + xr];
#pragma unroll
                for (int m = 0; m < 4; ++m) du[m] = fmaf(p, sOT[(xj + m) * LR + r], du[m]);
            }
            for (int c = 0; c < DK; ++c) {
                const float kb = sKb[xr * LD + c];
#pragma unroll
                for (int m = 0; m < 4; ++m) du[m] = fmaf(kb, sDST[(xj + m) * LT + c], du[m]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                sUT[(xj + m) * LR + xr] = u[m];
                sDUT[(xj + m) * LR + xr] = du[m];
            }
        }
        __syncthreads();
        {  // dX = Diag(b) Minv^T dU = dV
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            for (int r = xr; r < 64; ++r) {
                const float mi = sMI[r * 65 + xr];
#pragma unroll
                for (int m = 0; m < 4; ++m) acc[m] = fmaf(mi, sDUT[(xj + m) * LR + r], acc[m]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const float x = sB[xr] * acc[m];
                sDXT[(xj + m) * LR + xr] = x;
                if (xr < nt) dv[((t0 + xr) * H + h) * (int64_t)Dv + j0 + xj + m] = x;
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int jj = 0; jj < 16; ++jj) {
            float o4[4], x4[4], u4[4], du4[4], s[CPT], ds[CPT], uI[4], xI[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                o4[a] = sOT[jj * LR + ar + a];
                x4[a] = sDXT[jj * LR + ar + a];
                u4[a] = sUT[jj * LR + ar + a];
                du4[a] = sDUT[jj * LR + ar + a];
                uI[a] = sUT[jj * LR + ai + a];
                xI[a] = sXT[jj * LR + ai + a];
            }
#pragma unroll
            for (int b = 0; b < CPT; ++b) {
                s[b] = sST[jj * LT + ac + b];
                ds[b] = sDST[jj * LT + ac + b];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
#pragma unroll
                for (int b = 0; b < CPT; ++b) {
                    aQ[a][b] = fmaf(o4[a], s[b], aQ[a][b]);
                    aK[a][b] = fmaf(-x4[a], s[b], aK[a][b]);
                    aB[a][b] = fmaf(u4[a], ds[b], aB[a][b]);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    aP[a][b] = fmaf(o4[a], uI[b], aP[a][b]);
                    aN[a][b] = fmaf(du4[a], xI[b], aN[a][b]);
                }
            }
        }
        if (tid < DK)
            for (int jj = 0; jj < 16; ++jj) aG = fmaf(sST[jj * LT + tid], sDST[jj * LT + tid], aG);
        __syncthreads();
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
            const int e = (ar + a) * DK + ac + b;
            out[GR::DQT + e] = aQ[a][b];
            out[GR::DKT + e] = aK[a][b];
            out[GR::DKB + e] = aB[a][b];
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            out[GR::DP + (ar + a) * 64 + ai + b] = aP[a][b];
            out[GR::DN + (ar + a) * 64 + ai + b] = aN[a][b];
        }
    }
    if (tid < DK) out[GR::DGM + tid] = aG;
}

// ============================================================================ to dq, dk, dg, db

template <int DK, bool F32>
__global__ __launch_bounds__(256, 1) void bwd_grad_b_kernel(const void* __restrict__ qv, const void* __restrict__ kv,
                                                            const float* __restrict__ g,
                                                            const int32_t* __restrict__ cu, int64_t T_fixed,
                                                            int64_t total, int64_t N, int H,
                                                            const float* __restrict__ recs,
                                                            const float* __restrict__ grads, float* __restrict__ dq,
                                                            float* __restrict__ dk, float* __restrict__ dg,
                                                            float* __restrict__ dbeta) {
    using R = BRec<DK>;
    using GR = GRec<DK>;
    constexpr int LD = DK + 4;
    constexpr int CPT = DK / 16;
    __shared__ __align__(16) float sq[64 * LD], sk[64 * LD], sG[64 * LD], sM1[64 * 65], sM2[64 * 65],
        sM3[64 * 65], sB[64], sDB[64];
    const int tid = threadIdx.x;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    int64_t n, t0;
    int nt;
    if (!slot_chunk(cu, slot, T_fixed, total, N, n, t0, nt)) return;
    const float* rec = recs + (slot * H + h) * (int64_t)R::FLOATS;
    const float* gin = grads + (slot * H + h) * (int64_t)GR::FLOATS;

    // ---- through N = Minv Diag(b) and Minv = M^{-1}
    for (int e = tid; e < 4096; e += 256) {
        const int r = e >> 6, i = e & 63;
        sM1[r * 65 + i] = i <= r ? gin[GR::DN + e] : 0.f;  // dN (N is lower triangular)
        sM2[r * 65 + i] = rec[R::MI + e];                   // Minv
    }
    if (tid < 64) sB[tid] = rec[R::BT + tid];
    __syncthreads();
    float dbn = 0.f;
    if (tid < 64)
        for (int r = tid; r < 64; ++r) dbn = fmaf(sM1[r * 65 + tid], sM2[r * 65 + tid], dbn);
    __syncthreads();
    for (int e = tid; e < 4096; e += 256) sM1[(e >> 6) * 65 + (e & 63)] *= sB[e & 63];  // dMinv = dN Diag(b)
    __syncthreads();
    const int xr = tid >> 2, xs = 16 * (tid & 3);
    {  // T1 = dMinv Minv^T
        float acc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[m] = 0.f;
        for (int i = 0; i < 64; ++i) {
            const float d = sM1[xr * 65 + i];
#pragma unroll
            for (int m = 0; m < 16; ++m) acc[m] = fmaf(d, sM2[(xs + m) * 65 + i], acc[m]);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) sM3[xr * 65 + xs + m] = acc[m];
    }
    __syncthreads();
    {  // dM = -Minv^T T1
        float acc[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) acc[m] = 0.f;
        for (int r = 0; r < 64; ++r) {
            const float mi = sM2[r * 65 + xr];
#pragma unroll
            for (int m = 0; m < 16; ++m) acc[m] = fmaf(mi, sM3[r * 65 + xs + m], acc[m]);
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) sM1[xr * 65 + xs + m] = -acc[m];
    }
    __syncthreads();
    for (int e = tid; e < 4096; e += 256) {
        const int r = e >> 6, i = e & 63;
        sM3[r * 65 + i] = rec[R::AB + e];                   // Abar
        sM2[r * 65 + i] = i <= r ? gin[GR::DP + e] : 0.f;   // dP (P is lower triangular with the diagonal)
    }
    __syncthreads();
    if (tid < 64) {  // db from M = I + Diag(b) Abar, then dAbar = strict_tril(Diag(b) dM)
        const int r = tid;
        float dbm = 0.f;
        for (int i = 0; i < r; ++i) dbm = fmaf(sM1[r * 65 + i], sM3[r * 65 + i], dbm);
        sDB[r] = dbn + dbm;
        for (int i = 0; i < 64; ++i) sM1[r * 65 + i] = i < r ? sB[r] * sM1[r * 65 + i] : 0.f;
    }
    // ---- q, k and the running gate sums
    for (int e = tid; e < 64 * DK; e += 256) {
        const int r = e / DK, c = e % DK;
        float x = 0.f, y = 0.f, z = 0.f;
        if (r < nt) {
            const int64_t idx = ((t0 + r) * H + h) * (int64_t)DK + c;
            x = load_in<F32>(qv, idx);
            y = load_in<F32>(kv, idx);
            z = fminf(fmaxf(g[idx], -5.f), 0.f);
        }
        sq[r * LD + c] = x;
        sk[r * LD + c] = y;
        sG[r * LD + c] = z;
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
        for (int r = 0; r < 64; ++r) {
            acc += sG[r * LD + tid];
            sG[r * LD + tid] = acc;
        }
    }
    __syncthreads();

    // ---- decayed Gram blocks: thread block rows ar..ar+3, channels ac..ac+CPT-1
    const int ar = 4 * (tid >> 4), ac = CPT * (tid & 15);
    float Gr[4][CPT], aq[4][CPT], ak1[4][CPT], ak2[4][CPT];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
            Gr[a][b] = sG[(ar + a) * LD + ac + b];
            aq[a][b] = ak1[a][b] = ak2[a][b] = 0.f;
        }
    // rows r of this thread against every column i <= r: dq (P), dk (Abar) of row r
    for (int i = 0; i < 64; ++i) {
        float ki[CPT], Gi[CPT];
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
            ki[b] = sk[i * LD + ac + b];
            Gi[b] = sG[i * LD + ac + b];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float dp = sM2[(ar + a) * 65 + i], da = sM1[(ar + a) * 65 + i];  // zero unless i <= r
#pragma unroll
            for (int b = 0; b < CPT; ++b) {
                const float ke = ki[b] * __expf(fminf(Gr[a][b] - Gi[b], 0.f));
                aq[a][b] = fmaf(dp, ke, aq[a][b]);
                ak1[a][b] = fmaf(da, ke, ak1[a][b]);
            }
        }
    }
    // rows of this thread as the column index i against every row r >= i: dk of row i
    for (int r = 0; r < 64; ++r) {
        float kr[CPT], qr[CPT], Grr[CPT];
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
            kr[b] = sk[r * LD + ac + b];
            qr[b] = sq[r * LD + ac + b];
            Grr[b] = sG[r * LD + ac + b];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float dp = sM2[r * 65 + ar + a], da = sM1[r * 65 + ar + a];  // zero unless r >= i
#pragma unroll
            for (int b = 0; b < CPT; ++b) {
                const float e = __expf(fminf(Grr[b] - Gr[a][b], 0.f));
                ak2[a][b] = fmaf(fmaf(da, kr[b], dp * qr[b]), e, ak2[a][b]);
            }
        }
    }
    // ---- own elements: dq, dk, and dG into LDS (after every thread has read q, k, G)
    float dG[4][CPT], colp[CPT];
#pragma unroll
    for (int b = 0; b < CPT; ++b) colp[b] = 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int r = ar + a;
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
            const int c = ac + b;
            const float Gc = sG[63 * LD + c];
            const float gam = __expf(Gr[a][b]), gbar = __expf(Gc - Gr[a][b]);
            const float qx = sq[r * LD + c], kx = sk[r * LD + c];
            const float dQt = gin[GR::DQT + r * DK + c], dKt = gin[GR::DKT + r * DK + c];
            const float dKb = gin[GR::DKB + r * DK + c];
            const float dqv = fmaf(gam, dQt, aq[a][b]);
            const float dkv = fmaf(gam, dKt, fmaf(gbar, dKb, ak1[a][b] + ak2[a][b]));
            dG[a][b] = qx * (gam * dQt + aq[a][b]) + kx * (gam * dKt - gbar * dKb + ak1[a][b] - ak2[a][b]);
            colp[b] = fmaf(kx * gbar, dKb, colp[b]);
            if (r < nt) {
                const int64_t idx = ((t0 + r) * H + h) * (int64_t)DK + c;
                dq[idx] = dqv;
                dk[idx] = dkv;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < CPT; ++b) sq[(ar + a) * LD + ac + b] = dG[a][b];
#pragma unroll
    for (int b = 0; b < CPT; ++b) sM3[(tid >> 4) * DK + ac + b] = colp[b];  // [16 row blocks][DK]
    __syncthreads();
    // ---- G to g: reverse running sum plus the chunk-end term; the clamp's mask
    if (tid < DK) {
        const int c = tid;
        float acc = rec[R::GM + c] * gin[GR::DGM + c];  // gamma dgamma
        for (int rb = 0; rb < 16; ++rb) acc += sM3[rb * DK + c];
        for (int r = 63; r >= 0; --r) {
            acc += sq[r * LD + c];
            if (r < nt) {
                const int64_t idx = ((t0 + r) * H + h) * (int64_t)DK + c;
                const float gr = g[idx];
                dg[idx] = (gr >= -5.f && gr <= 0.f) ? acc : 0.f;
            }
        }
    }
    if (tid < nt) dbeta[(t0 + tid) * H + h] = sDB[tid];
}

// ============================================================================ host side

int64_t bwd_slots(const BwdArgs& a) {
    if (a.cu_seqlens) return a.total / kBC + a.N;
    return a.N * ((a.T_fixed + kBC - 1) / kBC);
}

static int64_t bwd_rec_floats(int Dk) { return Dk == 128 ? BRec<128>::FLOATS : BRec<64>::FLOATS; }
static int64_t bwd_grad_floats(int Dk) { return Dk == 128 ? GRec<128>::FLOATS : GRec<64>::FLOATS; }

// [records][states][state gradients][column sums], each per (slot, head)
int64_t bwd_workspace_bytes(const BwdArgs& a) {
    const int64_t per = bwd_rec_floats(a.Dk) + 2 * (int64_t)a.Dk * a.Dv + bwd_grad_floats(a.Dk);
    return bwd_slots(a) * a.H * per * 4;
}


template <int DK, bool F32>
static hipError_t launch_bwd_dk(const BwdArgs& a, void* ws, hipStream_t st) {
    const int64_t ch = bwd_slots(a) * a.H;
    float* recs = static_cast<float*>(ws);
    float* states = recs + ch * (int64_t)BRec<DK>::FLOATS;
    float* dstates = states + ch * (int64_t)DK * a.Dv;
    float* grads = dstates + ch * (int64_t)DK * a.Dv;
    const int64_t items = a.N * (int64_t)a.H;
    const int NS = a.Dv / kBS;
    const unsigned chain = (unsigned)(((items + 7) / 8) * 8 * NS);
    if (ch > 0) {
        // the forward pass's preparation (fp32 records, plus the plain operands `recs`) and its
        // state-only chain give the chunk-start states; the fragment records borrow the column-sum
        // area, which bwd_grad_a writes only later
        const ChunkArgs fa{a.q, a.k, a.v, a.g, a.beta, a.s0, nullptr, nullptr, a.cu_seqlens, a.T_fixed, a.total,
                           a.N, a.H, a.Dk, a.Dv, a.f32, Prologue{false, false, false, false, false}};
        if ((int64_t)GRec<DK>::FLOATS * 4 < chunk_states_record_bytes(DK)) return hipErrorInvalidValue;
        const hipError_t e = launch_chunk_states(fa, grads, recs, states, st);
        if (e != hipSuccess) return e;
    }
    // with no chunks at all this only passes d_sfinal (or zeros) through to ds0
    hipLaunchKernelGGL((bwd_dstates_kernel<DK>), dim3(chain), dim3(256), 0, st, a.d_o, a.d_sfinal, a.ds0,
                       a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv, recs, dstates);
    if (ch > 0) {
        hipLaunchKernelGGL((bwd_grad_a_kernel<DK, F32>), dim3((unsigned)ch), dim3(256), 0, st, a.v, a.d_o,
                           a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv, recs, states, dstates, grads, a.dv);
        hipLaunchKernelGGL((bwd_grad_b_kernel<DK, F32>), dim3((unsigned)ch), dim3(256), 0, st, a.q, a.k, a.g,
                           a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, recs, grads, a.dq, a.dk, a.dg, a.dbeta);
    }
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, void* ws, hipStream_t st) {
    if (a.Dk == 128) return a.f32 ? launch_bwd_dk<128, true>(a, ws, st) : launch_bwd_dk<128, false>(a, ws, st);
    return a.f32 ? launch_bwd_dk<64, true>(a, ws, st) : launch_bwd_dk<64, false>(a, ws, st);
}

}  // namespace kda
