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
// Qt, Kt, Kb, P, Minv, Abar, gamma, b per (chunk, head) (fp32) and the state at every chunk start come
// from the forward pass's prep kernel in its backward form and its chain kernel in mode 3, on split-bf16
// records with every product in three passes (launch_chunk_states).  Then three kernels, fp32
// accumulation (the column sums as three-pass split-bf16 products, the others on fp32 MFMA):
//   bwd_dstates_kernel per (sequence, head, 32 state columns), chunks in reverse: dS', dU, dX of every
//                      chunk, dv = dX, ds0
//   bwd_colsum_kernel  per (chunk, head): the sums over value columns (dQt, dKt, dKb, dP, dN, dgamma)
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
// Per (chunk, head) output of bwd_colsum (float offsets).
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

// x where keep holds, else +0.  A bit mask rather than a select, so that a value loaded early is
// not turned back into a load on the kept branch only (which would wait for every later load).
__device__ __forceinline__ float keep_if(float x, bool keep) {
    return __uint_as_float(__float_as_uint(x) & (keep ? 0xffffffffu : 0u));
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

// One workgroup of 1024 threads (16 waves) per (sequence, head, 32 state columns) walks the chunks
// backwards on MFMA (F32: fp32 products, else split bf16):
//   dU = P^T dO + Kb dS',  dX = Diag(b) Minv^T dU,  dS = Diag(gamma) dS' + Qt^T dO - Kt^T dX.
// Waves 0-7 own one 16x16 tile of dU and dX each; every wave (Dk = 128) or waves 0-7 (Dk = 64) own
// one 16x16 tile of dS, which stays in their registers from chunk to chunk.  dS' (the gradient at
// the chunk end) goes to dstates, dU and dX to dudx, dX to dv.  The operands are read with 16-byte
// loads into registers one phase ahead of their use and staged in LDS in operand order (rows, then
// the contracted index), so that each MFMA fragment is one row read.
template <int DK, bool F32>
__global__ __launch_bounds__(1024, 1) void bwd_dstates_kernel(const float* __restrict__ d_o,
                                                              const float* __restrict__ d_sfinal, float* ds0,
                                                              const int32_t* __restrict__ cu, int64_t T_fixed,
                                                              int64_t total, int64_t N, int H, int Dv,
                                                              const float* __restrict__ recs,
                                                              float* __restrict__ dstates, float* __restrict__ dudx,
                                                              float* __restrict__ dv) {
    using R = BRec<DK>;
    using Fr = Frag<F32>;
    using MTT = LMat<F32, 64, 64>;   // P^T, Minv^T  [i][r]
    using MKB = LMat<F32, 64, DK>;   // Kb           [i][c]
    using MQT = LMat<F32, DK, 64>;   // Qt^T, -Kt^T  [c][r]
    using MOT = LMat<F32, kBS, 64>;  // dO^T, dU^T, dX^T [j][r]
    using MDS = LMat<F32, kBS, DK>;  // dS'^T [j][c]
    constexpr int NT = 1024;
    constexpr int AB1 = MTT::BYTES + MKB::BYTES, AB2 = 2 * MQT::BYTES;
    constexpr int A_BYTES = AB1 > AB2 ? AB1 : AB2;  // P^T + Kb (for dU), then Qt^T + -Kt^T (for dS)
    constexpr int O_MT = A_BYTES, O_OT = O_MT + MTT::BYTES, O_DS = O_OT + MOT::BYTES, O_DU = O_DS + MDS::BYTES,
                  O_DX = O_DU + MOT::BYTES, O_B = O_DX + MOT::BYTES, O_G = O_B + 256, TOTAL = O_G + DK * 4;
    constexpr int KQ = 64 * DK / 4 / NT;  // 16-byte pieces per thread of a [64][DK] operand
    __shared__ __align__(16) char smem[TOTAL];
    char* pPT = smem;
    char* pKB = smem + MTT::BYTES;
    char* pQT = smem;
    char* pKT = smem + MQT::BYTES;
    char* pMT = smem + O_MT;
    char* pOT = smem + O_OT;
    char* pDS = smem + O_DS;
    char* pDU = smem + O_DU;
    char* pDX = smem + O_DX;
    float* sB = reinterpret_cast<float*>(smem + O_B);
    float* sG = reinterpret_cast<float*>(smem + O_G);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    int64_t pr;
    int sl;
    if (!chain_item(N * (int64_t)H, Dv / kBS, pr, sl)) return;
    const int64_t n = pr / H;
    const int h = (int)(pr % H);
    const BSeq sr = bseq(cu, n, T_fixed, total);
    const int64_t nch = (sr.end - sr.start + kBC - 1) / kBC;
    const int col0 = sl * kBS;

    const bool uwave = w < 8;                         // owns a tile of dU and dX
    const int rb = (w >> 1) & 3, nb = w & 1;          // that tile: rows 16rb.., columns 16nb..
    const int s0u = rb >= 2 ? 1 : 0;                  // P^T, Minv^T rows 16rb.. vanish below column 32 s0u
    const bool swave = w < DK / 8;                    // owns a tile of dS
    const int cb = w >> 1;                            // that tile: rows 16cb.., columns 16nb..

    // dS' in the owners' registers (D layout: rows 16cb + 4cg + jj, column 16nb + m) and in LDS
    f32x4_t dS = {0.f, 0.f, 0.f, 0.f};
    if (swave) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            dS[jj] = d_sfinal ? d_sfinal[((n * H + h) * DK + 16 * cb + 4 * cg + jj) * (int64_t)Dv + col0 + 16 * nb + m]
                              : 0.f;
        lds_store4<F32, kBS, DK>(pDS, 16 * nb + m, 16 * cb + 4 * cg, dS);
    }

    float4 rPT, rMT, rKB[KQ], rQT[KQ], rKT[KQ];
    float2 rO;
    float rB = 0.f, rG = 0.f;
    const int orow = tid >> 4, ocol = 2 * (tid & 15);  // this thread's two dO values
    auto rec_of = [&](int64_t jc) {
        return recs + (bslot(cu, n, jc, T_fixed, sr.start) * H + h) * (int64_t)R::FLOATS;
    };
    auto load_a = [&](int64_t jc) {  // P^T, Minv^T, Kb, dO, b, gamma of chunk jc
        const float* rec = rec_of(jc);
        rPT = reinterpret_cast<const float4*>(rec + R::PMT)[tid];
        rMT = reinterpret_cast<const float4*>(rec + R::MIT)[tid];
#pragma unroll
        for (int q = 0; q < KQ; ++q) rKB[q] = reinterpret_cast<const float4*>(rec + R::KB)[tid + q * NT];
        const int64_t t0 = sr.start + jc * kBC;
        const int nt = (int)min<int64_t>(kBC, sr.end - t0);
        rO = orow < nt ? *reinterpret_cast<const float2*>(d_o + ((t0 + orow) * H + h) * (int64_t)Dv + col0 + ocol)
                       : make_float2(0.f, 0.f);
        if (tid < 64) rB = rec[R::BT + tid];
        if (tid < DK) rG = rec[R::GM + tid];
    };
    auto load_c = [&](int64_t jc) {  // Qt^T, Kt^T of chunk jc
        const float* rec = rec_of(jc);
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            rQT[q] = reinterpret_cast<const float4*>(rec + R::QTT)[tid + q * NT];
            rKT[q] = reinterpret_cast<const float4*>(rec + R::KTT)[tid + q * NT];
        }
    };
    auto f4 = [](float4 x, float sgn) { return f32x4_t{sgn * x.x, sgn * x.y, sgn * x.z, sgn * x.w}; };

    if (nch > 0) load_a(nch - 1);
    for (int64_t jc = nch - 1; jc >= 0; --jc) {
        const int64_t slot = bslot(cu, n, jc, T_fixed, sr.start);
        const int64_t t0 = sr.start + jc * kBC;
        const int nt = (int)min<int64_t>(kBC, sr.end - t0);
        if (swave) {  // dS' of this chunk
            float* dst = dstates + (slot * H + h) * (int64_t)DK * Dv + col0 + 16 * nb + m;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) st_nt(&dst[(16 * cb + 4 * cg + jj) * (int64_t)Dv], dS[jj]);
        }
        // stage P^T, Minv^T, Kb, dO^T, b, gamma (the previous chunk's dS phase has finished: barrier)
        lds_store4<F32, 64, 64>(pPT, (4 * tid) >> 6, (4 * tid) & 63, f4(rPT, 1.f));
        lds_store4<F32, 64, 64>(pMT, (4 * tid) >> 6, (4 * tid) & 63, f4(rMT, 1.f));
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            const int e = 4 * (tid + q * NT);
            lds_store4<F32, 64, DK>(pKB, e / DK, e % DK, f4(rKB[q], 1.f));
        }
        lds_store1<F32, kBS, 64>(pOT, ocol, orow, rO.x);
        lds_store1<F32, kBS, 64>(pOT, ocol + 1, orow, rO.y);
        if (tid < 64) sB[tid] = rB;
        if (tid < DK) sG[tid] = rG;
        load_c(jc);
        __syncthreads();
        if (jc > 0) load_a(jc - 1);

        f32x4_t accU = {0.f, 0.f, 0.f, 0.f};
        if (uwave) {  // dU = P^T dO + Kb dS'
            for (int s = s0u; s < 2; ++s)
                accU = mma_full(accU, lds_frag<F32, 64, 64>(pPT, 16 * rb + m, 32 * s + 8 * cg),
                                lds_frag<F32, kBS, 64>(pOT, 16 * nb + m, 32 * s + 8 * cg));
#pragma unroll
            for (int s = 0; s < DK / 32; ++s)
                accU = mma_full(accU, lds_frag<F32, 64, DK>(pKB, 16 * rb + m, 32 * s + 8 * cg),
                                lds_frag<F32, kBS, DK>(pDS, 16 * nb + m, 32 * s + 8 * cg));
            lds_store4<F32, kBS, 64>(pDU, 16 * nb + m, 16 * rb + 4 * cg, accU);
        }
        __syncthreads();
        if (uwave) {  // dX = Diag(b) Minv^T dU; dU, dX of the chunk and dv = dX
            f32x4_t accX = {0.f, 0.f, 0.f, 0.f};
            for (int s = s0u; s < 2; ++s)
                accX = mma_full(accX, lds_frag<F32, 64, 64>(pMT, 16 * rb + m, 32 * s + 8 * cg),
                                lds_frag<F32, kBS, 64>(pDU, 16 * nb + m, 32 * s + 8 * cg));
            float* du_o = dudx + (slot * H + h) * 128 * (int64_t)Dv + col0 + 16 * nb + m;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * rb + 4 * cg + jj;
                accX[jj] *= sB[i];
                st_nt(&du_o[i * (int64_t)Dv], accU[jj]);
                st_nt(&du_o[(64 + i) * (int64_t)Dv], accX[jj]);
                if (i < nt) st_nt(&dv[((t0 + i) * H + h) * (int64_t)Dv + col0 + 16 * nb + m], accX[jj]);
            }
            lds_store4<F32, kBS, 64>(pDX, 16 * nb + m, 16 * rb + 4 * cg, accX);
        }
        __syncthreads();  // P^T and Kb are no longer read: Qt^T and -Kt^T go over them
#pragma unroll
        for (int q = 0; q < KQ; ++q) {
            const int e = 4 * (tid + q * NT);
            lds_store4<F32, DK, 64>(pQT, e / 64, e % 64, f4(rQT[q], 1.f));
            lds_store4<F32, DK, 64>(pKT, e / 64, e % 64, f4(rKT[q], -1.f));
        }
        __syncthreads();
        if (swave) {  // dS = Diag(gamma) dS' + Qt^T dO - Kt^T dX
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dS[jj] *= sG[16 * cb + 4 * cg + jj];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                dS = mma_full(dS, lds_frag<F32, DK, 64>(pQT, 16 * cb + m, 32 * s + 8 * cg),
                              lds_frag<F32, kBS, 64>(pOT, 16 * nb + m, 32 * s + 8 * cg));
                dS = mma_full(dS, lds_frag<F32, DK, 64>(pKT, 16 * cb + m, 32 * s + 8 * cg),
                              lds_frag<F32, kBS, 64>(pDX, 16 * nb + m, 32 * s + 8 * cg));
            }
            lds_store4<F32, kBS, DK>(pDS, 16 * nb + m, 16 * cb + 4 * cg, dS);
        }
        __syncthreads();
    }
    if (ds0 && swave)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            ds0[((n * H + h) * DK + 16 * cb + 4 * cg + jj) * (int64_t)Dv + col0 + 16 * nb + m] = dS[jj];
}

// ============================================================================ sums over the value columns

// Eight consecutive fp32 values of a row-major matrix as a split-bf16 MFMA fragment: lane l takes row
// row0 + l%16 and columns k0 + 8(l/16) .. +7.  The same fragment serves as the A operand of rows of
// the matrix and as the B operand of its columns (both contract over the stored column index).
__device__ __forceinline__ Frag<false> frag_rows(const float* base, int64_t ld, int row0, int k0, int m, int cg,
                                                 float x[8]) {
    load8_as_float(base + (row0 + m) * ld + k0 + 8 * cg, x);
    Frag<false> f;
    f.set(x);
    return f;
}

// Per (chunk, head): the products summed over the value columns, all contracting over the stored
// column index of row-major operands:
//   dQt = dO S^T, dKt = -dX S^T, dKb = U dS'^T (64 x DK);  dP = dO U^T, dN = dU X^T (64 x 64);
//   dgamma = rowsum(S o dS').  Split-bf16 three-pass products; wave w owns rows 16w..16w+15.
// Per 32-column step the operands every wave needs (S and dS' rows, U and X rows) are read from
// memory once per workgroup, split once and staged in LDS; the next step's pieces are requested
// while the current step's products run.  A wave's own rows (dO, dX, U, dU) come straight from memory.
template <int DK>
struct ColsumLds {
    using MS = LMat<false, DK, 32>;  // S, dS' column step [c][n]
    using MR = LMat<false, 64, 32>;  // U, X column step [t][n]
    static constexpr int S = 0, DS = S + MS::BYTES, U = DS + MS::BYTES, X = U + MR::BYTES, TOTAL = X + MR::BYTES;
};

template <int DK>
__global__ __launch_bounds__(256, 2) void bwd_colsum_kernel(const float* __restrict__ d_o,
                                                            const int32_t* __restrict__ cu, int64_t T_fixed,
                                                            int64_t total, int64_t N, int H, int Dv,
                                                            const float* __restrict__ states,
                                                            const float* __restrict__ dstates,
                                                            const float* __restrict__ xu,
                                                            const float* __restrict__ dudx,
                                                            float* __restrict__ grads) {
    using GR = GRec<DK>;
    using L = ColsumLds<DK>;
    constexpr int CB = DK / 16;
    constexpr int PS = DK / 8;  // S / dS' values staged per thread per step (32 DK / 256)
    __shared__ __align__(16) char smem[L::TOTAL];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    int64_t n, t0;
    int nt;
    if (!slot_chunk(cu, slot, T_fixed, total, N, n, t0, nt)) return;
    const int64_t ch = slot * H + h;
    const float* S = states + ch * DK * (int64_t)Dv;
    const float* dS = dstates + ch * DK * (int64_t)Dv;
    const float* X = xu + ch * 128 * (int64_t)Dv;
    const float* U = X + 64 * (int64_t)Dv;
    const float* dU = dudx + ch * 128 * (int64_t)Dv;
    const float* dX = dU + 64 * (int64_t)Dv;
    // dO rows of this wave: tokens past the end read the last token and count as zero
    const int orow = 16 * w + m;
    const float* dO = d_o + ((t0 + min(orow, nt - 1)) * H + h) * (int64_t)Dv;
    const float omask = orow < nt ? 1.f : 0.f;
    // staging pieces: S and dS' rows sr (PS columns from sc), U and X rows ur (8 columns from uc)
    const int sr = (tid * PS) / 32, sc = (tid * PS) % 32, ur = tid >> 2, uc = 8 * (tid & 3);
    float vS[PS], vD[PS], vU[8], vX[8];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int j = 0; j < PS; j += 4) {
            const float4 a = *reinterpret_cast<const float4*>(S + sr * (int64_t)Dv + k0 + sc + j);
            const float4 b = *reinterpret_cast<const float4*>(dS + sr * (int64_t)Dv + k0 + sc + j);
            vS[j] = a.x; vS[j + 1] = a.y; vS[j + 2] = a.z; vS[j + 3] = a.w;
            vD[j] = b.x; vD[j + 1] = b.y; vD[j + 2] = b.z; vD[j + 3] = b.w;
        }
        load8_as_float(U + ur * (int64_t)Dv + k0 + uc, vU);
        load8_as_float(X + ur * (int64_t)Dv + k0 + uc, vX);
    };

    f32x4_t aQ[CB], aK[CB], aB[CB], aP[4], aN[4];
#pragma unroll
    for (int i = 0; i < CB; ++i) aQ[i] = aK[i] = aB[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) aP[i] = aN[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float dgam = 0.f;  // partial row sum of S o dS' for row sr

    fetch(0);
    for (int k0 = 0; k0 < Dv; k0 += 32) {
        __syncthreads();  // the previous step's fragments have been read
#pragma unroll
        for (int j = 0; j < PS; j += 8) {
            lds_store8<false, DK, 32>(smem + L::S, sr, sc + j, vS + j);
            lds_store8<false, DK, 32>(smem + L::DS, sr, sc + j, vD + j);
        }
#pragma unroll
        for (int j = 0; j < PS; ++j) dgam = fmaf(vS[j], vD[j], dgam);
        lds_store8<false, 64, 32>(smem + L::U, ur, uc, vU);
        lds_store8<false, 64, 32>(smem + L::X, ur, uc, vX);
        __syncthreads();
        if (k0 + 32 < Dv) fetch(k0 + 32);

        float x[8];
        load8_as_float(dO + k0 + 8 * cg, x);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] *= omask;
        Frag<false> fO;
        fO.set(x);
        const Frag<false> fX = frag_rows(dX, Dv, 16 * w, k0, m, cg, x);
        const Frag<false> fU = frag_rows(U, Dv, 16 * w, k0, m, cg, x);
        const Frag<false> fdU = frag_rows(dU, Dv, 16 * w, k0, m, cg, x);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            const Frag<false> fS = lds_frag<false, DK, 32>(smem + L::S, 16 * cb + m, 8 * cg);
            const Frag<false> fdS = lds_frag<false, DK, 32>(smem + L::DS, 16 * cb + m, 8 * cg);
            aQ[cb] = mma_full(aQ[cb], fO, fS);
            aK[cb] = mma_full(aK[cb], fX, fS);
            aB[cb] = mma_full(aB[cb], fU, fdS);
        }
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            aP[ib] = mma_full(aP[ib], fO, lds_frag<false, 64, 32>(smem + L::U, 16 * ib + m, 8 * cg));
            aN[ib] = mma_full(aN[ib], fdU, lds_frag<false, 64, 32>(smem + L::X, 16 * ib + m, 8 * cg));
        }
    }
    float* out = grads + ch * (int64_t)GR::FLOATS;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * cg + i;
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
            st_nt(&out[GR::DQT + r * DK + 16 * cb + m], aQ[cb][i]);
            st_nt(&out[GR::DKT + r * DK + 16 * cb + m], -aK[cb][i]);
            st_nt(&out[GR::DKB + r * DK + 16 * cb + m], aB[cb][i]);
        }
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
            st_nt(&out[GR::DP + r * 64 + 16 * ib + m], aP[ib][i]);
            st_nt(&out[GR::DN + r * 64 + 16 * ib + m], aN[ib][i]);
        }
    }
    // dgamma: the 32 / PS threads of a row are adjacent
#pragma unroll
    for (int off = 1; off < 32 / PS; off <<= 1) dgam += __shfl_xor(dgam, off);
    if (sc == 0) st_nt(&out[GR::DGM + sr], dgam);
}

// ============================================================================ to dq, dk, dg, db

// Per (chunk, head), 1024 threads: through N = Minv Diag(b) and Minv = (I + Diag(b) Abar)^{-1} to db and
// dAbar, then through the decayed Gram blocks Abar and P, Qt, Kt, Kb and gamma to dq, dk and dG, and
// from G to dg.  Thread t owns row t/16 and channels (t%16)*DK/16 .. of the token-by-channel tensors.
template <int DK, bool F32>
__global__ __launch_bounds__(1024, 1) void bwd_grad_b_kernel(const void* __restrict__ qv,
                                                             const void* __restrict__ kv,
                                                             const float* __restrict__ g,
                                                             const int32_t* __restrict__ cu, int64_t T_fixed,
                                                             int64_t total, int64_t N, int H,
                                                             const float* __restrict__ recs,
                                                             const float* __restrict__ grads,
                                                             float* __restrict__ dq, float* __restrict__ dk,
                                                             float* __restrict__ dg, float* __restrict__ dbeta) {
    using R = BRec<DK>;
    using GR = GRec<DK>;
    constexpr int NT = 1024;
    constexpr int LD = DK + 4;
    constexpr int CPT = DK / 16;
    __shared__ __align__(16) float sq[64 * LD], sk[64 * LD], sG[64 * LD], sM1[64 * 65], sM2[64 * 65],
        sM3[64 * 65], sB[64], sDB[64], sGb[5 * DK], sFf[6 * DK], sDf[4 * DK];
    __shared__ uint32_t sMk[64 * DK / 32];  // bit set: g outside [-5, 0] (its gradient is zero)
    const int tid = threadIdx.x;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    int64_t n, t0;
    int nt;
    if (!slot_chunk(cu, slot, T_fixed, total, N, n, t0, nt)) return;
    const float* rec = recs + (slot * H + h) * (int64_t)R::FLOATS;
    const float* gin = grads + (slot * H + h) * (int64_t)GR::FLOATS;

    // ---- every global operand of the chunk is requested up front (the phases below are short and
    // would otherwise each wait out a full memory latency): four elements of each 64x64 block per
    // thread, and one piece of eight q, k, g channels per thread (8 DK <= 1024 pieces)
    static_assert(4096 % NT == 0 && 8 * DK <= NT, "one piece per thread");
    constexpr int EPT = 4096 / NT;
    // (in the order they are consumed: the first phase waits only for b, dN and Minv)
    const float vb = tid < 64 ? rec[R::BT + tid] : 0.f;
    float vN[EPT], vM[EPT], vA[EPT], vP[EPT];
#pragma unroll
    for (int a = 0; a < EPT; ++a) {
        vN[a] = gin[GR::DN + tid + a * NT];
        vM[a] = rec[R::MIT + tid + a * NT];
    }
#pragma unroll
    for (int a = 0; a < EPT; ++a) {
        vA[a] = rec[R::AB + tid + a * NT];
        vP[a] = gin[GR::DP + tid + a * NT];
    }
    const bool has8 = tid < 8 * DK;
    const int r8 = (8 * tid) / DK, c8 = (8 * tid) % DK;
    Raw8<F32> xq8, xk8;
    float4 zg[2];
    if (has8) {
        const int64_t idx = ((t0 + min(r8, nt - 1)) * H + h) * (int64_t)DK + c8;
        if constexpr (F32) {
            load_raw8(static_cast<const float*>(qv) + idx, xq8);
            load_raw8(static_cast<const float*>(kv) + idx, xk8);
        } else {
            load_raw8(static_cast<const uint16_t*>(qv) + idx, xq8);
            load_raw8(static_cast<const uint16_t*>(kv) + idx, xk8);
        }
        zg[0] = *reinterpret_cast<const float4*>(g + idx);
        zg[1] = *reinterpret_cast<const float4*>(g + idx + 4);
    }
    const float vgd = rec[R::GM + tid % DK] * gin[GR::DGM + tid % DK];  // gamma dgamma of channel tid % DK

    // ---- through N = Minv Diag(b) and Minv = M^{-1}
#pragma unroll
    for (int a = 0; a < EPT; ++a) {
        const int e = tid + a * NT, r = e >> 6, i = e & 63;
        sM1[r * 65 + i] = keep_if(vN[a], i <= r);  // dN (N is lower triangular)
        sM2[i * 65 + r] = vM[a];                 // Minv (from its transpose)
    }
    if (tid < 64) sB[tid] = vb;
    for (int e = tid; e < 64 * DK / 32; e += NT) sMk[e] = 0u;
    __syncthreads();
    {  // db from N: column sums of dN o Minv, 16 partial sums of 4 rows per column
        const int i = tid & 63, r0 = 4 * (tid >> 6);
        float p = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) p = fmaf(sM1[(r0 + a) * 65 + i], sM2[(r0 + a) * 65 + i], p);
        sM3[(tid >> 6) * 64 + i] = p;
    }
    __syncthreads();
    float dbn = 0.f;
    if (tid < 64)
        for (int rg = 0; rg < 16; ++rg) dbn += sM3[rg * 64 + tid];
    __syncthreads();
    for (int e = tid; e < 4096; e += NT) sM1[(e >> 6) * 65 + (e & 63)] *= sB[e & 63];  // dMinv = dN Diag(b)
    __syncthreads();
    // T1 = dMinv Minv^T, then dM = -Minv^T T1, on fp32 MFMA: wave wv computes the 16x16 tile
    // (row block wv / 4, column block wv % 4) of each; MFMA number kk takes reduction index
    // 4 kk + lane / 16 in both operands
    {
        const int wv = tid >> 6, mm = tid & 15, cq = (tid >> 4) & 3, X = wv >> 2, S = wv & 3;
        f32x4_t t1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int i = 4 * kk + cq;
            t1 = __builtin_amdgcn_mfma_f32_16x16x4f32(sM1[(16 * X + mm) * 65 + i], sM2[(16 * S + mm) * 65 + i], t1,
                                                      0, 0, 0);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sM3[(16 * X + 4 * cq + jj) * 65 + 16 * S + mm] = t1[jj];
        __syncthreads();
        f32x4_t dm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int r = 4 * kk + cq;
            dm = __builtin_amdgcn_mfma_f32_16x16x4f32(sM2[r * 65 + 16 * X + mm], sM3[r * 65 + 16 * S + mm], dm, 0, 0,
                                                      0);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sM1[(16 * X + 4 * cq + jj) * 65 + 16 * S + mm] = -dm[jj];
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < EPT; ++a) {
        const int e = tid + a * NT, r = e >> 6, i = e & 63;
        sM3[r * 65 + i] = vA[a];                 // Abar
        sM2[r * 65 + i] = keep_if(vP[a], i <= r);  // dP (P is lower triangular with the diagonal)
    }
    __syncthreads();
    if (tid < 64) sDB[tid] = dbn;
    {  // db from M = I + Diag(b) Abar (row sums over 16 lanes), then dAbar = strict_tril(Diag(b) dM)
        const int r = tid >> 4, i0 = 4 * (tid & 15);
        float p = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int i = i0 + a;
            const float dm = sM1[r * 65 + i];
            if (i < r) p = fmaf(dm, sM3[r * 65 + i], p);
            sM1[r * 65 + i] = i < r ? sB[r] * dm : 0.f;
        }
        p += __shfl_xor(p, 1);
        p += __shfl_xor(p, 2);
        p += __shfl_xor(p, 4);
        p += __shfl_xor(p, 8);
        __syncthreads();  // sDB holds the column part
        if ((tid & 15) == 0) sDB[r] += p;
    }
    // ---- q, k and the clamped gates to LDS (the piece loaded at the start).  At DK = 128 the piece
    // of thread t is exactly its own elements of the final step (row t/16, channels 8 (t%16)..), so
    // q and k stay in registers for it.
    constexpr bool OWN8 = 8 * DK == NT;
    float qown[CPT], kown[CPT];
    if (has8) {
        float x[8], y[8];
        raw8_to_float<F32>(xq8, x);
        raw8_to_float<F32>(xk8, y);
        const float z[8] = {zg[0].x, zg[0].y, zg[0].z, zg[0].w, zg[1].x, zg[1].y, zg[1].z, zg[1].w};
        const int r = r8, c = c8;
        const float msk = r < nt ? 1.f : 0.f;
        uint32_t bits = 0u;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            sq[r * LD + c + jj] = msk * x[jj];
            sk[r * LD + c + jj] = msk * y[jj];
            sG[r * LD + c + jj] = msk * fminf(fmaxf(z[jj], -5.f), 0.f);
            bits |= (z[jj] < -5.f || z[jj] > 0.f) ? (1u << jj) : 0u;
            if constexpr (OWN8) {
                qown[jj] = msk * x[jj];
                kown[jj] = msk * y[jj];
            }
        }
        atomicOr(&sMk[r * (DK / 32) + c / 32], bits << (c % 32));
    }
    __syncthreads();
    // running sums down each channel: segments of SEG rows per thread, then the segment offsets
    constexpr int NSEG = NT / DK, SEG = 64 / NSEG;
    const int sc_ = tid % DK, sg_ = tid / DK;
    {
        float acc = 0.f;
#pragma unroll
        for (int r = SEG * sg_; r < SEG * sg_ + SEG; ++r) {
            acc += sG[r * LD + sc_];
            sG[r * LD + sc_] = acc;
        }
    }
    __syncthreads();
    {
        float off = 0.f;
        for (int s2 = 0; s2 < sg_; ++s2) off += sG[(SEG * s2 + SEG - 1) * LD + sc_];
        __syncthreads();  // every offset read before any is changed
#pragma unroll
        for (int r = SEG * sg_; r < SEG * sg_ + SEG; ++r) sG[r * LD + sc_] += off;
    }
    __syncthreads();

    // ---- decay factors by 16-token sub-block (as in the forward pass): with Gs_R the running sum
    // before block R and Ge_I the one at the end of block I, for token r in block R and i in I <= R
    //   e^{G_r - G_i} = A1_r * F_RI * B1_i  (I < R),   A1_r * D_R * B1_i  (I = R),
    // A1_r = e^{G_r - Gs_R} <= 1, B1_i = e^{Ge_I - G_i} <= 1, F_RI = e^{Gs_R - Ge_I} <= 1,
    // D_R = e^{Gs_R - Ge_R} <= e^80: no exponential per term, none that overflows.
    if (tid < DK) {
        const int c = tid;
        float gb[5];
        gb[0] = 0.f;
#pragma unroll
        for (int b = 1; b < 5; ++b) gb[b] = sG[(16 * b - 1) * LD + c];
#pragma unroll
        for (int b = 0; b < 5; ++b) sGb[b * DK + c] = gb[b];
#pragma unroll
        for (int R_ = 0; R_ < 4; ++R_) {
            sDf[R_ * DK + c] = __expf(gb[R_] - gb[R_ + 1]);
#pragma unroll
            for (int I = 0; I < R_; ++I) sFf[(R_ * (R_ - 1) / 2 + I) * DK + c] = __expf(gb[R_] - gb[I + 1]);
        }
    }
    const int ar = tid >> 4, ac = CPT * (tid & 15), blk = ar >> 4;  // one row; a wave's rows share a block
    float Gr[CPT];
#pragma unroll
    for (int b = 0; b < CPT; ++b) Gr[b] = sG[ar * LD + ac + b];
    __syncthreads();
    // own elements -> tables: sq = q A1, sk = k A1, sG = k B1
#pragma unroll
    for (int b = 0; b < CPT; ++b) {
        const int e = ar * LD + ac + b;
        const float a1 = __expf(Gr[b] - sGb[blk * DK + ac + b]);
        const float b1 = __expf(sGb[(blk + 1) * DK + ac + b] - Gr[b]);
        const float kx = sk[e];
        sq[e] *= a1;
        sk[e] = kx * a1;
        sG[e] = kx * b1;
    }
    __syncthreads();

    // the column-sum gradients of this thread's own elements, loaded while the products below run
    float pQt[CPT], pKt[CPT], pKb[CPT];
#pragma unroll
    for (int b = 0; b < CPT; b += 4) {
        const float* base = gin + ar * DK + ac + b;
        const float4 u = *reinterpret_cast<const float4*>(base + GR::DQT);
        const float4 v4 = *reinterpret_cast<const float4*>(base + GR::DKT);
        const float4 w4 = *reinterpret_cast<const float4*>(base + GR::DKB);
        pQt[b] = u.x; pQt[b + 1] = u.y; pQt[b + 2] = u.z; pQt[b + 3] = u.w;
        pKt[b] = v4.x; pKt[b + 1] = v4.y; pKt[b + 2] = v4.z; pKt[b + 3] = v4.w;
        pKb[b] = w4.x; pKb[b + 1] = w4.y; pKb[b + 2] = w4.z; pKb[b + 3] = w4.w;
    }

    // ---- the decayed Gram contractions on fp32 MFMA (16x16x4).  Wave wv owns the (row block R,
    // 16-channel block cb) pairs below and, for each, three 16x16 results at rows 16R.. and
    // channels 16cb.. (F_RR = D_R):
    //   aq  = sum_{I <= R} F_RI o (dP[R, I] (k B1)[I])          (for dq)
    //   ak1 = sum_{I <= R} F_RI o (dAbar[R, I] (k B1)[I])       (for dk)
    //   ak2 = sum_{R2 >= R} F_{R2, R} o (dAbar[R2, R]^T (k A1)[R2] + dP[R2, R]^T (q A1)[R2])
    // The decay factor depends only on the channel (the result's column), so it scales each block
    // pair's product as a whole.  MFMA number kk takes reduction index 4 kk + lane / 16 in both
    // operands; every pair costs 8 (R + 1) + 8 (4 - R) = 40 products.
    constexpr int NCB = DK / 16, PPW = 4 * NCB / 16;  // pairs per wave
    const int wv = tid >> 6, mm = tid & 15, cq = (tid >> 4) & 3;
    f32x4_t oq[PPW], ok1[PPW], ok2[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int cb = wv % NCB, R = wv / NCB + p * (16 / NCB);
        const int c = 16 * cb + mm;
        f32x4_t aQ = {0.f, 0.f, 0.f, 0.f}, aK = {0.f, 0.f, 0.f, 0.f}, aK2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int I = 0; I <= R; ++I) {
            f32x4_t tq = {0.f, 0.f, 0.f, 0.f}, tk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int i = 16 * I + 4 * kk + cq;
                const float bv = sG[i * LD + c];
                tq = __builtin_amdgcn_mfma_f32_16x16x4f32(sM2[(16 * R + mm) * 65 + i], bv, tq, 0, 0, 0);
                tk = __builtin_amdgcn_mfma_f32_16x16x4f32(sM1[(16 * R + mm) * 65 + i], bv, tk, 0, 0, 0);
            }
            const float f = I < R ? sFf[(R * (R - 1) / 2 + I) * DK + c] : sDf[R * DK + c];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                aQ[jj] = fmaf(f, tq[jj], aQ[jj]);
                aK[jj] = fmaf(f, tk[jj], aK[jj]);
            }
        }
#pragma unroll 1
        for (int R2 = R; R2 < 4; ++R2) {
            f32x4_t t2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int r = 16 * R2 + 4 * kk + cq;
                t2 = __builtin_amdgcn_mfma_f32_16x16x4f32(sM1[r * 65 + 16 * R + mm], sk[r * LD + c], t2, 0, 0, 0);
                t2 = __builtin_amdgcn_mfma_f32_16x16x4f32(sM2[r * 65 + 16 * R + mm], sq[r * LD + c], t2, 0, 0, 0);
            }
            const float f = R2 > R ? sFf[(R2 * (R2 - 1) / 2 + R) * DK + c] : sDf[R * DK + c];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) aK2[jj] = fmaf(f, t2[jj], aK2[jj]);
        }
        oq[p] = aQ;
        ok1[p] = aK;
        ok2[p] = aK2;
    }
    __syncthreads();  // every operand has been read: sq, sk, sG take the three results
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int cb = wv % NCB, R = wv / NCB + p * (16 / NCB);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int e = (16 * R + 4 * cq + jj) * LD + 16 * cb + mm;
            sq[e] = oq[p][jj];
            sk[e] = ok1[p][jj];
            sG[e] = ok2[p][jj];
        }
    }
    __syncthreads();
    float aq[CPT], ak1[CPT], ak2[CPT];
#pragma unroll
    for (int b = 0; b < CPT; ++b) {
        const int e = ar * LD + ac + b;
        aq[b] = sq[e];
        ak1[b] = sk[e];
        ak2[b] = sG[e];
    }
    // ---- own elements: dq, dk, and dG (after every thread has read the tables)
    float dG[CPT], colp[CPT];
    {
        const int r = ar;
        float qx[CPT], kx[CPT];
        if constexpr (OWN8) {
#pragma unroll
            for (int b = 0; b < CPT; ++b) {
                qx[b] = qown[b];
                kx[b] = kown[b];
            }
        } else {
            const int64_t idx0 = ((t0 + min(r, nt - 1)) * H + h) * (int64_t)DK + ac;
#pragma unroll
            for (int b = 0; b < CPT; ++b) {
                qx[b] = r < nt ? load_in<F32>(qv, idx0 + b) : 0.f;
                kx[b] = r < nt ? load_in<F32>(kv, idx0 + b) : 0.f;
            }
        }
        float gs[CPT], ge[CPT], gc[CPT], dqv[CPT], dkv[CPT];  // running sums at the block start / end, G_C
#pragma unroll
        for (int b = 0; b < CPT; b += 4) {
            const float4 u = *reinterpret_cast<const float4*>(&sGb[blk * DK + ac + b]);
            const float4 v4 = *reinterpret_cast<const float4*>(&sGb[(blk + 1) * DK + ac + b]);
            const float4 w4 = *reinterpret_cast<const float4*>(&sGb[4 * DK + ac + b]);
            gs[b] = u.x; gs[b + 1] = u.y; gs[b + 2] = u.z; gs[b + 3] = u.w;
            ge[b] = v4.x; ge[b + 1] = v4.y; ge[b + 2] = v4.z; ge[b + 3] = v4.w;
            gc[b] = w4.x; gc[b + 1] = w4.y; gc[b + 2] = w4.z; gc[b + 3] = w4.w;
        }
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
            const float a1 = __expf(Gr[b] - gs[b]);
            const float b1 = __expf(ge[b] - Gr[b]);
            const float q_ = a1 * aq[b], k1 = a1 * ak1[b], k2 = b1 * ak2[b];
            const float gam = __expf(Gr[b]), gbar = __expf(gc[b] - Gr[b]);
            const float dQt = pQt[b], dKt = pKt[b], dKb = pKb[b];
            dqv[b] = fmaf(gam, dQt, q_);
            dkv[b] = fmaf(gam, dKt, fmaf(gbar, dKb, k1 + k2));
            dG[b] = qx[b] * (gam * dQt + q_) + kx[b] * (gam * dKt - gbar * dKb + k1 - k2);
            colp[b] = kx[b] * gbar * dKb;
        }
        if (r < nt) {
            const int64_t idx = ((t0 + r) * H + h) * (int64_t)DK + ac;
#pragma unroll
            for (int b = 0; b < CPT; b += 4) {
                st_nt4(dq + idx + b, dqv[b], dqv[b + 1], dqv[b + 2], dqv[b + 3]);
                st_nt4(dk + idx + b, dkv[b], dkv[b + 1], dkv[b + 2], dkv[b + 3]);
            }
        }
    }
    // the four rows of a wave summed for the chunk-end column term
#pragma unroll
    for (int b = 0; b < CPT; ++b) {
        colp[b] += __shfl_xor(colp[b], 16);
        colp[b] += __shfl_xor(colp[b], 32);
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < CPT; ++b) sq[ar * LD + ac + b] = dG[b];
    if ((tid & 63) < 16)
#pragma unroll
        for (int b = 0; b < CPT; ++b) sM3[(tid >> 6) * DK + ac + b] = colp[b];  // [16 waves][DK]
    __syncthreads();
    // ---- G to g: reverse running sum (segments as above) plus the chunk-end term; the clamp's mask
    {
        const int c = sc_;
        float acc = 0.f;
#pragma unroll
        for (int r = SEG * sg_ + SEG - 1; r >= SEG * sg_; --r) {
            acc += sq[r * LD + c];
            sq[r * LD + c] = acc;
        }
    }
    __syncthreads();
    {
        const int c = sc_;
        float off = vgd;  // gamma dgamma (c = tid % DK)
        for (int wv = 0; wv < 16; ++wv) off += sM3[wv * DK + c];
        for (int s2 = sg_ + 1; s2 < NSEG; ++s2) off += sq[(SEG * s2) * LD + c];
#pragma unroll
        for (int r = SEG * sg_; r < SEG * sg_ + SEG; ++r) {
            if (r < nt) {
                const bool outside = (sMk[r * (DK / 32) + c / 32] >> (c % 32)) & 1u;
                dg[((t0 + r) * H + h) * (int64_t)DK + c] = outside ? 0.f : sq[r * LD + c] + off;
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

// [records][states][state gradients][column sums][X, U][dU, dX], each per (slot, head)
int64_t bwd_workspace_bytes(const BwdArgs& a) {
    const int64_t per = bwd_rec_floats(a.Dk) + 2 * (int64_t)a.Dk * a.Dv + bwd_grad_floats(a.Dk) + 4 * 64 * (int64_t)a.Dv;
    return bwd_slots(a) * a.H * per * 4;
}


template <int DK, bool F32>
static hipError_t launch_bwd_dk(const BwdArgs& a, void* ws, hipStream_t st) {
    const int64_t ch = bwd_slots(a) * a.H;
    float* recs = static_cast<float*>(ws);
    float* states = recs + ch * (int64_t)BRec<DK>::FLOATS;
    float* dstates = states + ch * (int64_t)DK * a.Dv;
    float* grads = dstates + ch * (int64_t)DK * a.Dv;
    float* xu = grads + ch * (int64_t)GRec<DK>::FLOATS;
    float* dudx = xu + ch * 128 * (int64_t)a.Dv;
    const int64_t items = a.N * (int64_t)a.H;
    const int NS = a.Dv / kBS;
    const unsigned chain = (unsigned)(((items + 7) / 8) * 8 * NS);
    if (ch > 0) {
        // the forward pass's preparation (fp32 records, plus the plain operands `recs`) and its
        // state-only chain give the chunk-start states and X, U; the fragment records borrow the
        // column-sum area, which bwd_colsum writes only later
        const ChunkArgs fa{a.q, a.k, a.v, a.g, a.beta, a.s0, nullptr, nullptr, a.cu_seqlens, a.T_fixed, a.total,
                           a.N, a.H, a.Dk, a.Dv, a.f32, Prologue{false, false, false, false, false}};
        if ((int64_t)GRec<DK>::FLOATS * 4 < chunk_states_record_bytes(DK)) return hipErrorInvalidValue;
        const hipError_t e = launch_chunk_states(fa, grads, recs, states, xu, st);
        if (e != hipSuccess) return e;
    }
    // with no chunks at all this only passes d_sfinal (or zeros) through to ds0
    hipLaunchKernelGGL((bwd_dstates_kernel<DK, true>), dim3(chain), dim3(1024), 0, st, a.d_o, a.d_sfinal, a.ds0,
                       a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv, recs, dstates, dudx, a.dv);
    if (ch > 0) {
        hipLaunchKernelGGL((bwd_colsum_kernel<DK>), dim3((unsigned)ch), dim3(256), 0, st, a.d_o, a.cu_seqlens,
                           a.T_fixed, a.total, a.N, a.H, a.Dv, states, dstates, xu, dudx, grads);
        hipLaunchKernelGGL((bwd_grad_b_kernel<DK, F32>), dim3((unsigned)ch), dim3(1024), 0, st, a.q, a.k, a.g,
                           a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, recs, grads, a.dq, a.dk, a.dg, a.dbeta);
    }
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, void* ws, hipStream_t st) {
    if (a.Dk == 128) return a.f32 ? launch_bwd_dk<128, true>(a, ws, st) : launch_bwd_dk<128, false>(a, ws, st);
    return a.f32 ? launch_bwd_dk<64, true>(a, ws, st) : launch_bwd_dk<64, false>(a, ws, st);
}

}  // namespace kda
