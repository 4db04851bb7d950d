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
// Per (chunk, head), the reverse chain's operands Qt^T, -Kt^T, Kb, P^T, (Minv Diag(b))^T as split-bf16
// MFMA fragments, the gradient kernel's Minv, Abar, gamma, b in fp32, and the state at every chunk
// start and X, U of every chunk come from the forward pass's prep kernel in its backward form and its
// chain kernel in mode 3,
// on split-bf16 records with every product in three passes (launch_chunk_states).  Then two kernels, fp32
// accumulation (the reverse chain, the column sums and the decayed Gram contractions as three-pass
// split-bf16 products, the products through the inverse on fp32 MFMA):
//   bwd_dstates_kernel per (sequence, head, 32 state columns), chunks in reverse: dS' and dU of every
//                      chunk, dv = dX (which the gradient kernel reads back), ds0
//   bwd_grad_kernel    per (chunk, head): the sums over value columns (dQt, dKt, dKb, dP, dN, dgamma),
//                      kept in LDS, then through the inverse, the decayed Gram blocks and the gates
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kBC = 64;  // tokens per chunk
constexpr int kBS = 32;  // state columns per chain workgroup

template <int DK>
using BRec = BwdRec<DK>;

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

// Two consecutive elements (columns col, col + 1; col even) of one row of a split-bf16 LDS matrix.
template <int ROWS, int COLS>
__device__ __forceinline__ void lds_store2(char* base, int row, int col, float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    using M = LMat<false, ROWS, COLS>;
    const __bf16 ha = (__bf16)a, hb = (__bf16)b;
    const bf16x2_t hi = {ha, hb}, lo = {(__bf16)(a - (float)ha), (__bf16)(b - (float)hb)};
    __bf16* p = reinterpret_cast<__bf16*>(base) + row * M::STRIDE + col;
    *reinterpret_cast<bf16x2_t*>(p) = hi;
    *reinterpret_cast<bf16x2_t*>(p + M::PLANE) = lo;
}

// A split-bf16 MFMA fragment of a record: a plane of 64 lanes x 16 B of bf16 hi, then one of bf16 lo.
__device__ __forceinline__ Frag<false> rec_frag(const float* p, int lane) {
    Frag<false> f;
    f.hi = reinterpret_cast<const bf16x8_t*>(p)[lane];
    f.lo = reinterpret_cast<const bf16x8_t*>(p + 256)[lane];
    return f;
}

// One workgroup per (sequence, head, 32 state columns) walks the chunks backwards on split-bf16 MFMA:
//   dU = P^T dO + Kb dS',  dX = N^T dU,  dS = Diag(gamma) dS' + Qt^T dO - Kt^T dX   (N = Minv Diag(b)).
// Waves 0-3 (U waves) own rows 16w.. of dU and dX; waves 4.. (S waves) own rows 16(w-4).. of dS,
// which stays in their registers from chunk to chunk; each wave covers both 16-column tiles of its
// rows.  A wave loads the fragments of P^T, Kb, N^T (U) or Qt^T, -Kt^T (S) that it multiplies
// straight from the record into registers, one chunk ahead (each a contiguous 1 KiB request per
// plane), so each record is read once per workgroup and the products take only the operands shared
// between waves from LDS: dO^T, dS'^T, dU^T, dX^T.  Three barriers per chunk:
//   (1) U: dU -> LDS                        S: dS' to memory; dS = Diag(gamma) dS' + Qt^T dO
//   (2) U: dX -> LDS
//   (3) U: dU, dv = dX to memory;           S: dS -= Kt^T dX; dS' of the next chunk -> LDS
//          dO^T of the next chunk -> LDS
// The results also pass through fp32 tiles in LDS, so that each goes to memory as whole 128-byte rows.
// Every chunk issues the same memory instructions in the same order (the loads past either end
// are clamped to an existing chunk, never skipped, and the first chunk is peeled off the loop), so
// the compiler's wait counts are exact and no wait for a load also waits for a store.
template <int DK>
__global__ __launch_bounds__(64 * (4 + DK / 16), 1) void bwd_dstates_kernel(
    const float* __restrict__ d_o, const float* __restrict__ d_sfinal, float* ds0, const int32_t* __restrict__ cu,
    int64_t T_fixed, int64_t total, int64_t N, int H, int Dv, const float* __restrict__ recs,
    float* __restrict__ dstates, float* __restrict__ du, float* __restrict__ dv, float* __restrict__ trash) {
    using R = BRec<DK>;
    using Fr = Frag<false>;
    using MOT = LMat<false, kBS, 64>;  // dO^T, dU^T, dX^T [j][r]
    using MDS = LMat<false, kBS, DK>;  // dS'^T [j][c]
    constexpr int KS = DK / 32;
    constexpr int FS = kBS + 4;  // fp32 row stride of the tiles on their way to memory
    __shared__ __align__(16) char smem[3 * MOT::BYTES + MDS::BYTES + (DK + 128) * FS * 4];
    char* pOT = smem;
    char* pDU = smem + MOT::BYTES;
    char* pDX = smem + 2 * MOT::BYTES;
    char* pDS = smem + 3 * MOT::BYTES;
    float* fDS = reinterpret_cast<float*>(smem + 3 * MOT::BYTES + MDS::BYTES);  // dS' [DK][FS] fp32
    float* fDU = fDS + DK * FS;                                                 // dU [64][FS]
    float* fDX = fDU + 64 * FS;                                                 // dX [64][FS]

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    int64_t pr;
    int sl;
    if (!chain_item(N * (int64_t)H, Dv / kBS, pr, sl)) return;
    const int64_t n = pr / H;
    const int h = (int)(pr % H);
    const BSeq sr = bseq(cu, n, T_fixed, total);
    const int64_t nch = (sr.end - sr.start + kBC - 1) / kBC;
    const int col0 = sl * kBS;
    auto rec_of = [&](int64_t jc) {
        return recs + (bslot(cu, n, jc, T_fixed, sr.start) * H + h) * (int64_t)R::FLOATS;
    };

    if (w < 4) {  // ------------------------------------------------------------------ U waves
        const int rb = w;
        Fr fP[2], fK[KS], fN[2];
        float4 o0, o1;
        const int p = tid >> 3, q = tid & 7;  // dO staging: rows 2p, 2p + 1, columns 4q .. 4q + 3
        int ont = 0;                          // valid rows of the chunk whose dO is in o0, o1
        auto load_o = [&](int64_t jc) {
            const int64_t t0 = sr.start + jc * kBC;
            ont = (int)min<int64_t>(kBC, sr.end - t0);
            const float* base = d_o + (int64_t)h * Dv + col0 + 4 * q;
            o0 = *reinterpret_cast<const float4*>(base + (t0 + min(2 * p, ont - 1)) * H * (int64_t)Dv);
            o1 = *reinterpret_cast<const float4*>(base + (t0 + min(2 * p + 1, ont - 1)) * H * (int64_t)Dv);
        };
        auto stage_o = [&]() {  // dO^T (rows past the end as zeros)
            const float4 a = 2 * p < ont ? o0 : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 b = 2 * p + 1 < ont ? o1 : make_float4(0.f, 0.f, 0.f, 0.f);
            lds_store2<kBS, 64>(pOT, 4 * q + 0, 2 * p, a.x, b.x);
            lds_store2<kBS, 64>(pOT, 4 * q + 1, 2 * p, a.y, b.y);
            lds_store2<kBS, 64>(pOT, 4 * q + 2, 2 * p, a.z, b.z);
            lds_store2<kBS, 64>(pOT, 4 * q + 3, 2 * p, a.w, b.w);
        };
        if (nch > 0) {
            const float* rec = rec_of(nch - 1);
#pragma unroll
            for (int s = 0; s < 2; ++s) fP[s] = rec_frag(rec + R::PTF + R::tri(rb, s) * R::FRAG, lane);
#pragma unroll
            for (int s = 0; s < KS; ++s) fK[s] = rec_frag(rec + R::KBF + (rb * KS + s) * R::FRAG, lane);
#pragma unroll
            for (int s = 0; s < 2; ++s) fN[s] = rec_frag(rec + R::NTF + R::tri(rb, s) * R::FRAG, lane);
            load_o(nch - 1);
            stage_o();
            load_o(nch > 1 ? nch - 2 : 0);
        }
        lds_barrier();
        auto chunk = [&](int64_t jc) {
            const float* recn = rec_of(jc > 0 ? jc - 1 : 0);  // operands of the next chunk
            const int64_t slot = bslot(cu, n, jc, T_fixed, sr.start);
            const int64_t t0 = sr.start + jc * kBC;
            const int nt = (int)min<int64_t>(kBC, sr.end - t0);
            // (1) dU = P^T dO + Kb dS'
            f32x4_t aU[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s = 0; s < 2; ++s) {  // (row blocks 2, 3: step 0 is zero, its registers hold step 1)
                const Fr a = s < (rb >> 1) ? Fr{} : fP[s];
                fP[s] = rec_frag(recn + R::PTF + R::tri(rb, s) * R::FRAG, lane);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    aU[nb] = mma_full(aU[nb], a, lds_frag<false, kBS, 64>(pOT, 16 * nb + m, 32 * s + 8 * cg));
            }
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const Fr a = fK[s];
                fK[s] = rec_frag(recn + R::KBF + (rb * KS + s) * R::FRAG, lane);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    aU[nb] = mma_full(aU[nb], a, lds_frag<false, kBS, DK>(pDS, 16 * nb + m, 32 * s + 8 * cg));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                lds_store4<false, kBS, 64>(pDU, 16 * nb + m, 16 * rb + 4 * cg, aU[nb]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) fDU[(16 * rb + 4 * cg + jj) * FS + 16 * nb + m] = aU[nb][jj];
            }
            lds_barrier();  // (1)
            // (2) dX = N^T dU
            f32x4_t aX[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const Fr a = s < (rb >> 1) ? Fr{} : fN[s];
                fN[s] = rec_frag(recn + R::NTF + R::tri(rb, s) * R::FRAG, lane);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    aX[nb] = mma_full(aX[nb], a, lds_frag<false, kBS, 64>(pDU, 16 * nb + m, 32 * s + 8 * cg));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                lds_store4<false, kBS, 64>(pDX, 16 * nb + m, 16 * rb + 4 * cg, aX[nb]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) fDX[(16 * rb + 4 * cg + jj) * FS + 16 * nb + m] = aX[nb][jj];
            }
            lds_barrier();  // (2)
            // (3) dU and dX = dv of the chunk to memory, whole 128-byte rows (eight lanes a row); dO^T of
            // the next chunk (every read of this chunk's dO^T is behind barrier 1)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int i = (tid >> 3) + 32 * hh, c4 = 4 * (tid & 7);
                const float4 u = *reinterpret_cast<const float4*>(&fDU[i * FS + c4]);
                const float4 x = *reinterpret_cast<const float4*>(&fDX[i * FS + c4]);
                st_nt4(du + ((slot * H + h) * 64 + i) * (int64_t)Dv + col0 + c4, u.x, u.y, u.z, u.w);
                // rows past the end (zero: b vanishes there) go to the trash row, never read
                st_nt4(i < nt ? dv + ((t0 + i) * H + h) * (int64_t)Dv + col0 + c4 : trash + col0 + c4, x.x, x.y, x.z, x.w);
            }
            stage_o();
            load_o(jc > 1 ? jc - 2 : 0);
            lds_barrier();  // (3)
        };
        if (nch > 0) {  // the first chunk peeled: the loop is entered only after one whole chunk
            chunk(nch - 1);
            for (int64_t jc = nch - 2; jc >= 0; --jc) chunk(jc);
        }
    } else {  // ------------------------------------------------------------------------ S waves
        const int cb = w - 4;
        Fr fQ[2], fK[2];
        float4 g4;
        // dS' in registers (D layout: rows 16cb + 4cg + jj, columns 16nb + m) and in LDS
        f32x4_t acc[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                acc[nb][jj] = d_sfinal ? d_sfinal[((n * H + h) * DK + 16 * cb + 4 * cg + jj) * (int64_t)Dv + col0 +
                                                  16 * nb + m]
                                       : 0.f;
            lds_store4<false, kBS, DK>(pDS, 16 * nb + m, 16 * cb + 4 * cg, acc[nb]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) fDS[(16 * cb + 4 * cg + jj) * FS + 16 * nb + m] = acc[nb][jj];
        }
        if (nch > 0) {
            const float* rec = rec_of(nch - 1);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                fQ[s] = rec_frag(rec + R::QTF + (cb * 2 + s) * R::FRAG, lane);
                fK[s] = rec_frag(rec + R::KTF + (cb * 2 + s) * R::FRAG, lane);
            }
            g4 = *reinterpret_cast<const float4*>(rec + R::GM + 16 * cb + 4 * cg);
        }
        lds_barrier();
        auto chunk = [&](int64_t jc) {
            const float* recn = rec_of(jc > 0 ? jc - 1 : 0);
            const int64_t slot = bslot(cu, n, jc, T_fixed, sr.start);
            // dS' of this chunk (the gradient at its end) to memory, whole 128-byte rows from its fp32 tile
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c = ((tid - 256) >> 3) + (DK / 2) * hh, c4 = 4 * (tid & 7);
                const float4 d = *reinterpret_cast<const float4*>(&fDS[c * FS + c4]);
                st_nt4(dstates + ((slot * H + h) * DK + c) * (int64_t)Dv + col0 + c4, d.x, d.y, d.z, d.w);
            }
            // (1) dS = Diag(gamma) dS' + Qt^T dO
            const float gg[4] = {g4.x, g4.y, g4.z, g4.w};
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) acc[nb][jj] *= gg[jj];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const Fr a = fQ[s];
                fQ[s] = rec_frag(recn + R::QTF + (cb * 2 + s) * R::FRAG, lane);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[nb] = mma_full(acc[nb], a, lds_frag<false, kBS, 64>(pOT, 16 * nb + m, 32 * s + 8 * cg));
            }
            g4 = *reinterpret_cast<const float4*>(recn + R::GM + 16 * cb + 4 * cg);
            lds_barrier();  // (1)
            lds_barrier();  // (2)
            // (3) dS -= Kt^T dX; dS' of the next chunk to LDS (every read of dS'^T is behind barrier 1)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const Fr a = fK[s];
                fK[s] = rec_frag(recn + R::KTF + (cb * 2 + s) * R::FRAG, lane);
#pragma unroll
                for (int nb = 0; nb < 2; ++nb)
                    acc[nb] = mma_full(acc[nb], a, lds_frag<false, kBS, 64>(pDX, 16 * nb + m, 32 * s + 8 * cg));
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                lds_store4<false, kBS, DK>(pDS, 16 * nb + m, 16 * cb + 4 * cg, acc[nb]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) fDS[(16 * cb + 4 * cg + jj) * FS + 16 * nb + m] = acc[nb][jj];
            }
            lds_barrier();  // (3)
        };
        if (nch > 0) {  // the first chunk peeled: the loop is entered only after one whole chunk
            chunk(nch - 1);
            for (int64_t jc = nch - 2; jc >= 0; --jc) chunk(jc);
        }
        if (ds0) {
            float* d0 = ds0 + (n * H + h) * (int64_t)DK * Dv + col0;  // uniform base, small per-lane offsets
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) d0[(16 * cb + 4 * cg + jj) * Dv + 16 * nb + m] = acc[nb][jj];
        }
    }
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

// Per (chunk, head), the products summed over the value columns, all contracting over the stored
// column index of row-major operands:
//   dQt = dO S^T, dKt = -dX S^T, dKb = U dS'^T (64 x DK);  dP = dO U^T, dN = dU X^T (64 x 64);
//   dgamma = rowsum(S o dS').
// Split-bf16 three-pass products on the gradient kernel's 16 waves: the four waves of row block rb
// (w & 3) take dQt, dKt, dKb, and dP with dN respectively (w >> 2).  Per 32-column step every operand
// (S, dS', dO, dX, U, X, dU) is read from memory once per workgroup, one step ahead, split once and
// staged in LDS, one after the other from the start of sq (over sq, sk, sG and, at Dk = 64, sM1 and
// part of sM2: none of them holds anything yet), so the products of a step wait for no memory request.  The results land in LDS
// for the phases that follow: dQt in sq, dKt in sk, dKb in sG (rows [64][LD]), dN in sM1 and dP in sM3
// ([64][65]), and gamma o dgamma (gamma from `gam`) in sGam.
template <int DK>
__device__ __forceinline__ void colsum_to_lds(const float* __restrict__ d_o, int64_t t0, int nt, int H, int h,
                                              int Dv, const float* __restrict__ S, const float* __restrict__ dS,
                                              const float* __restrict__ X, const float* __restrict__ dU,
                                              const float* __restrict__ dv, const float* __restrict__ gam, float* sq, float* sk, float* sG,
                                              float* sM1, float* sM3, float* sGam, int tid) {
    using MS = LMat<false, DK, 32>;  // S, dS' column step [c][n]
    using MR = LMat<false, 64, 32>;  // U, X, dO, dX, dU column step [t][n]
    constexpr int LD = DK + 4;
    constexpr int CB = DK / 16;
    const float* U = X + 64 * (int64_t)Dv;
    char* pS = reinterpret_cast<char*>(sq);
    char* pD = pS + MS::BYTES;
    char* pU = pD + MS::BYTES;
    char* pX = pU + MR::BYTES;
    char* pO = pX + MR::BYTES;
    char* pDX = pO + MR::BYTES;
    char* pDU = pDX + MR::BYTES;
    const int w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    const int rb = w & 3, role = w >> 2;
    // staging pieces of four values, columns 4 (tid % 8) of the step: S and dS' row tid / 8 (threads
    // below 8 DK); row (tid % 512) / 8 of U or X (threads below / from 512) and of dO or dX (likewise);
    // dU row tid / 8 (threads below 512).  dO and dX (= dv, written by the reverse chain) rows past the
    // end read the last token and count as zero.
    const bool hasS = tid < 8 * DK, lo = tid < 512;
    const int srow = tid >> 3, scol = 4 * (tid & 7), urow = (tid & 511) >> 3;
    const float gam_row = hasS && (tid & 7) == 0 ? gam[srow] : 0.f;  // gamma of row srow, for its writer
    const float* UX = lo ? U : X;
    const float* OD = (lo ? d_o : dv) + ((t0 + min(urow, nt - 1)) * H + h) * (int64_t)Dv - urow * (int64_t)Dv;
    const float omask = urow >= nt ? 0.f : 1.f;
    char* pUX = lo ? pU : pX;
    char* pOD = lo ? pO : pDX;
    float4 vS = make_float4(0.f, 0.f, 0.f, 0.f), vD = vS, vR = vS, vO = vS, vW = vS;
    auto fetch_sd = [&](int k0) {
        if (hasS) {
            vS = *reinterpret_cast<const float4*>(S + srow * (int64_t)Dv + k0 + scol);
            vD = *reinterpret_cast<const float4*>(dS + srow * (int64_t)Dv + k0 + scol);
        }
    };
    auto fetch_rows = [&](int k0) {
        vR = *reinterpret_cast<const float4*>(UX + urow * (int64_t)Dv + k0 + scol);
        vO = *reinterpret_cast<const float4*>(OD + urow * (int64_t)Dv + k0 + scol);
        if (lo) vW = *reinterpret_cast<const float4*>(dU + urow * (int64_t)Dv + k0 + scol);
    };
    // one set of accumulator tiles for every role: CB tiles of dQt, dKt or dKb, or dN (0..3) and dP (4..7)
    constexpr int NACC = CB > 8 ? CB : 8;
    f32x4_t acc[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float dgam = 0.f;
    fetch_sd(0);
    fetch_rows(0);
    for (int k0 = 0; k0 < Dv; k0 += 32) {
        __syncthreads();  // the previous step's fragments have been read
        if (hasS) {
            lds_store4<false, DK, 32>(pS, srow, scol, f32x4_t{vS.x, vS.y, vS.z, vS.w});
            lds_store4<false, DK, 32>(pD, srow, scol, f32x4_t{vD.x, vD.y, vD.z, vD.w});
            dgam = fmaf(vS.x, vD.x, fmaf(vS.y, vD.y, fmaf(vS.z, vD.z, fmaf(vS.w, vD.w, dgam))));
        }
        if (k0 + 32 < Dv) fetch_sd(k0 + 32);  // the next step's pieces as soon as these are staged
        lds_store4<false, 64, 32>(pUX, urow, scol, f32x4_t{vR.x, vR.y, vR.z, vR.w});
        lds_store4<false, 64, 32>(pOD, urow, scol, f32x4_t{omask * vO.x, omask * vO.y, omask * vO.z, omask * vO.w});
        if (lo) lds_store4<false, 64, 32>(pDU, urow, scol, f32x4_t{vW.x, vW.y, vW.z, vW.w});
        if (k0 + 32 < Dv) fetch_rows(k0 + 32);
        __syncthreads();

        // Loops fully unrolled, so that the accumulator tiles are named registers (a loop index into
        // acc[] makes the compiler move each tile through indexed register moves around its products);
        // the scheduling barrier after each tile keeps its fragment read in place, so that the reads are
        // not all hoisted ahead (which runs out of registers).
        const int ar = 16 * rb + m;
        if (role == 3) {
            const Frag<false> fO = lds_frag<false, 64, 32>(pO, ar, 8 * cg);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                acc[4 + ib] = mma_full(acc[4 + ib], fO, lds_frag<false, 64, 32>(pU, 16 * ib + m, 8 * cg));
                __builtin_amdgcn_sched_barrier(0);
            }
            const Frag<false> fdU = lds_frag<false, 64, 32>(pDU, ar, 8 * cg);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                acc[ib] = mma_full(acc[ib], fdU, lds_frag<false, 64, 32>(pX, 16 * ib + m, 8 * cg));
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            const Frag<false> fr = lds_frag<false, 64, 32>(role == 0 ? pO : (role == 1 ? pDX : pU), ar, 8 * cg);
            const char* pB = role == 2 ? pD : pS;
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                acc[cb] = mma_full(acc[cb], fr, lds_frag<false, DK, 32>(pB, 16 * cb + m, 8 * cg));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // dgamma: the eight threads of a row are adjacent lanes
    dgam += __shfl_xor(dgam, 1);
    dgam += __shfl_xor(dgam, 2);
    dgam += __shfl_xor(dgam, 4);
    __syncthreads();  // every staged operand has been read
    if (hasS && (tid & 7) == 0) sGam[srow] = gam_row * dgam;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int r = 16 * rb + 4 * cg + jj;
        if (role == 3) {
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                sM1[r * 65 + 16 * ib + m] = acc[ib][jj];      // dN
                sM3[r * 65 + 16 * ib + m] = acc[4 + ib][jj];  // dP
            }
        } else {
            float* dst = role == 0 ? sq : (role == 1 ? sk : sG);
            const float sgn = role == 1 ? -1.f : 1.f;  // dKt = -dX S^T
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) dst[r * LD + 16 * cb + m] = sgn * acc[cb][jj];
        }
    }
    __syncthreads();
}

// A [64][DK] fp32 token-by-channel table staged channel-major as split bf16 over its own area: a
// plane of bf16 hi, then one of bf16 lo, each [DK][64]; the 8-byte groups of four tokens of row c
// are swizzled by c % 16, so that sixteen consecutive rows read at one token offset hit distinct banks.
__device__ __forceinline__ int tst_index(int c, int t) { return c * 64 + 4 * ((t >> 2) ^ (c & 15)) + (t & 3); }

// Four consecutive reduction-index values of a v_mfma_f32_16x16x16_bf16 operand, split.
struct Frag4 {
    bf16x4_t hi, lo;
};
__device__ __forceinline__ Frag4 split4(float a, float b, float c, float d) {
    const float x[4] = {a, b, c, d};
    Frag4 f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const __bf16 h = (__bf16)x[j];
        f.hi[j] = h;
        f.lo[j] = (__bf16)(x[j] - (float)h);
    }
    return f;
}
// acc += A * B with the split (three-pass) policy: lane l holds A[l % 16][4 (l / 16) ..] and
// B[4 (l / 16) ..][l % 16] of the 16x16x16 product.
__device__ __forceinline__ f32x4_t mma16(f32x4_t acc, const Frag4& a, const Frag4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
}
// Stage the EPS tokens r0 .. r0 + EPS - 1 (a multiple of four) of channel c.
template <int DK, int EPS>
__device__ __forceinline__ void tstage(float* base, int c, int r0, const float* x) {
    __bf16* p = reinterpret_cast<__bf16*>(base);
#pragma unroll
    for (int g = 0; g < EPS / 4; ++g) {
        const Frag4 f = split4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]);
        const int idx = tst_index(c, r0 + 4 * g);
        *reinterpret_cast<bf16x4_t*>(p + idx) = f.hi;
        *reinterpret_cast<bf16x4_t*>(p + DK * 64 + idx) = f.lo;
    }
}
// The lower 16x16 blocks (R, I <= R; block R (R + 1) / 2 + I) of dP and dAbar staged as split bf16:
// arrays 0, 1 hold the blocks of dP, dAbar as [row][column], arrays 2, 3 as [column][row]; each block
// a plane of 256 bf16 hi, then 256 lo.  Row `row`, columns 4 cq .. 4 cq + 3 of block bb of array arr.
__device__ __forceinline__ Frag4 gblk(const float* base, int arr, int bb, int row, int cq) {
    const __bf16* p = reinterpret_cast<const __bf16*>(base) + (arr * 10 + bb) * 512 + row * 16 + 4 * cq;
    return Frag4{*reinterpret_cast<const bf16x4_t*>(p), *reinterpret_cast<const bf16x4_t*>(p + 256)};
}
// Tokens t0 .. t0 + 3 (t0 a multiple of four) of channel c of a staged table.
template <int DK>
__device__ __forceinline__ Frag4 tfrag(const float* base, int c, int t0) {
    const __bf16* p = reinterpret_cast<const __bf16*>(base);
    const int idx = tst_index(c, t0);
    return Frag4{*reinterpret_cast<const bf16x4_t*>(p + idx), *reinterpret_cast<const bf16x4_t*>(p + DK * 64 + idx)};
}

// Per (chunk, head), 1024 threads: first the sums over the value columns (colsum_to_lds), then through
// N = Minv Diag(b) and Minv = (I + Diag(b) Abar)^{-1} to db and dAbar, then through the decayed Gram
// blocks Abar and P, Qt, Kt, Kb and gamma to dq, dk and dG, and from G to dg.  Thread t owns row t/16
// and channels (t%16)*DK/16 .. of the token-by-channel tensors.
template <int DK, bool F32>
__global__ __launch_bounds__(1024, 1) void bwd_grad_kernel(const void* __restrict__ qv,
                                                           const void* __restrict__ kv,
                                                           const float* __restrict__ g,
                                                           const float* __restrict__ d_o,
                                                           const int32_t* __restrict__ cu, int64_t T_fixed,
                                                           int64_t total, int64_t N, int H, int Dv,
                                                           const float* __restrict__ recs,
                                                           const float* __restrict__ states,
                                                           const float* __restrict__ dstates,
                                                           const float* __restrict__ xu,
                                                           const float* __restrict__ du,
                                                           const float* __restrict__ dv,
                                                           float* __restrict__ dq, float* __restrict__ dk,
                                                           float* __restrict__ dg, float* __restrict__ dbeta) {
    using R = BRec<DK>;
    constexpr int NT = 1024;
    constexpr int LD = DK + 4;
    constexpr int CPT = DK / 16;
    // one block, in this order, so that the column sums can stage their operands across the first
    // areas (colsum_to_lds)
    constexpr int O_Q = 0, O_K = O_Q + 64 * LD, O_G = O_K + 64 * LD, O_M1 = O_G + 64 * LD, O_M2 = O_M1 + 64 * 65,
                  O_M3 = O_M2 + 64 * 65, O_B = O_M3 + 64 * 65, O_DB = O_B + 64, O_GB = O_DB + 64, O_FF = O_GB + 5 * DK,
                  O_DF = O_FF + 6 * DK, O_MK = O_DF + 4 * DK, O_GD = O_MK + 64 * DK / 32, FLOATS = O_GD + DK;
    __shared__ __align__(16) float smem[FLOATS];
    float *sq = smem + O_Q, *sk = smem + O_K, *sG = smem + O_G, *sM1 = smem + O_M1, *sM2 = smem + O_M2,
          *sM3 = smem + O_M3, *sB = smem + O_B, *sDB = smem + O_DB, *sGb = smem + O_GB, *sFf = smem + O_FF,
          *sDf = smem + O_DF;
    uint32_t* sMk = reinterpret_cast<uint32_t*>(smem + O_MK);  // bit set: g outside [-5, 0] (its gradient is zero)
    float* sGd = smem + O_GD;                                  // gamma o dgamma per channel
    static_assert(O_M3 * 4 >= 2 * LMat<false, DK, 32>::BYTES + 5 * LMat<false, 64, 32>::BYTES,
                  "the column sums' staging ends before sM3");
    const int tid = threadIdx.x;
    const int64_t slot = blockIdx.x / H;
    const int h = (int)(blockIdx.x % H);
    int64_t n, t0;
    int nt;
    if (!slot_chunk(cu, slot, T_fixed, total, N, n, t0, nt)) return;
    const int64_t ch = slot * H + h;
    const float* rec = recs + ch * (int64_t)R::FLOATS;

    // ---- the records' operands of the later phases are requested up front, to arrive while the
    // column sums run: four elements of each 64x64 block per thread, only those inside the triangle that
    // can be nonzero (i >= r of Minv^T, i < r of Abar; the preparation leaves the blocks outside it
    // unwritten)
    static_assert(4096 % NT == 0 && 8 * DK <= NT, "one piece per thread");
    constexpr int EPT = 4096 / NT;
    const float vb = tid < 64 ? rec[R::BT + tid] : 0.f;
    float vN[EPT], vM[EPT], vA[EPT], vP[EPT];
#pragma unroll
    for (int a = 0; a < EPT; ++a) {
        const int e = tid + a * NT, r = e >> 6, i = e & 63;
        vM[a] = i >= r ? rec[R::MIT + e] : 0.f;
    }
#pragma unroll
    for (int a = 0; a < EPT; ++a) {
        const int e = tid + a * NT, r = e >> 6, i = e & 63;
        vA[a] = i < r ? rec[R::AB + e] : 0.f;
    }

    // ---- the sums over the value columns, into LDS
    colsum_to_lds<DK>(d_o, t0, nt, H, h, Dv, states + ch * DK * (int64_t)Dv, dstates + ch * DK * (int64_t)Dv,
                      xu + ch * 128 * (int64_t)Dv, du + ch * 64 * (int64_t)Dv, dv, rec + R::GM, sq, sk, sG, sM1, sM3,
                      sGd, tid);
    // this thread's pieces of them: dN and dP elements as in the loads above, and its own elements of
    // dQt, dKt, dKb (row tid / 16, channels (tid % 16) DK / 16 ..)
#pragma unroll
    for (int a = 0; a < EPT; ++a) {
        const int e = tid + a * NT;
        vN[a] = sM1[(e >> 6) * 65 + (e & 63)];
        vP[a] = sM3[(e >> 6) * 65 + (e & 63)];
    }
    float pQt[CPT], pKt[CPT], pKb[CPT];
    {
        const int e0 = (tid >> 4) * LD + CPT * (tid & 15);
#pragma unroll
        for (int b = 0; b < CPT; ++b) {
            pQt[b] = sq[e0 + b];
            pKt[b] = sk[e0 + b];
            pKb[b] = sG[e0 + b];
        }
    }
    __syncthreads();  // read before the phases below reuse these areas
    // q, k and g: one piece of eight channels per thread (first needed a few phases below)
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


    // ---- the decayed Gram contractions on split-bf16 MFMA (16x16x16, three passes).  Wave wv owns
    // the (row block R, 16-channel block cb) pairs below and, for each, three 16x16 results at rows
    // 16R.. and channels 16cb.. (F_RR = D_R):
    //   aq  = sum_{I <= R} F_RI o (dP[R, I] (k B1)[I])                             (for dq)
    //   ak1 = sum_{I <= R} F_RI o (dAbar[R, I] (k B1)[I])                          (for dk)
    //   ak2 = sum_{R2 >= R} F_{R2, R} o (dAbar[R2, R]^T (k A1)[R2] + dP[R2, R]^T (q A1)[R2])
    // The decay factor depends only on the channel (the result's column), so it scales each block
    // pair's product as a whole.  Every operand is split once and staged with the reduction index
    // innermost: k B1, k A1, q A1 as [channel][token] over sG, sk, sq; the ten lower 16x16 blocks of
    // dP and dAbar, as they are and transposed, over sM1 .. sM3 (gblk).
    constexpr int NCB = DK / 16, PPW = 4 * NCB / 16;  // pairs per wave
    constexpr int EPS = 64 * DK / NT;                  // staged table elements per thread
    constexpr int NBI = 4 * 10 * 64;                   // block pieces: (array, block, row, four columns)
    static_assert(4 * 10 * 1024 <= 3 * 65 * 64 * 4, "the staged blocks fit sM1 .. sM3");
    {
        float xb[3][4];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int it = tid + u * NT;
            if (it < NBI) {
                const int arr = it / 640, bb = (it >> 6) % 10, rr = (it >> 2) & 15, g = it & 3;
                const int R = bb >= 6 ? 3 : (bb >= 3 ? 2 : (bb >= 1 ? 1 : 0)), I = bb - R * (R + 1) / 2;
                const float* src = (arr & 1) ? sM1 : sM2;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xb[u][j] = arr < 2 ? src[(16 * R + rr) * 65 + 16 * I + 4 * g + j]
                                       : src[(16 * R + 4 * g + j) * 65 + 16 * I + rr];
            }
        }
        __syncthreads();  // dP and dAbar read before their blocks go over them
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int it = tid + u * NT;
            if (it < NBI) {
                const Frag4 f = split4(xb[u][0], xb[u][1], xb[u][2], xb[u][3]);
                __bf16* d = reinterpret_cast<__bf16*>(sM1) + (it >> 6) * 512 + ((it >> 2) & 15) * 16 + 4 * (it & 3);
                *reinterpret_cast<bf16x4_t*>(d) = f.hi;
                *reinterpret_cast<bf16x4_t*>(d + 256) = f.lo;
            }
        }
        const int c = tid % DK, r0 = EPS * (tid / DK);
        float xg[EPS], xk[EPS], xq[EPS];
#pragma unroll
        for (int e = 0; e < EPS; ++e) {
            xg[e] = sG[(r0 + e) * LD + c];
            xk[e] = sk[(r0 + e) * LD + c];
            xq[e] = sq[(r0 + e) * LD + c];
        }
        __syncthreads();  // every fp32 table element read before the split copies go over them
        tstage<DK, EPS>(sG, c, r0, xg);
        tstage<DK, EPS>(sk, c, r0, xk);
        tstage<DK, EPS>(sq, c, r0, xq);
    }
    __syncthreads();
    const int wv = tid >> 6, mm = tid & 15, cq = (tid >> 4) & 3;
    f32x4_t oq[PPW], ok1[PPW], ok2[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int cb = wv % NCB, R = wv / NCB + p * (16 / NCB);
        const int c = 16 * cb + mm;  // this lane's result channel and B-operand channel
        const f32x4_t z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4_t aQ = z4, aK = z4, aK2 = z4;
#pragma unroll 1
        for (int I = 0; I <= R; ++I) {
            const int bb = R * (R + 1) / 2 + I;
            const Frag4 b = tfrag<DK>(sG, c, 16 * I + 4 * cq);
            const f32x4_t tq = mma16(z4, gblk(sM1, 0, bb, mm, cq), b);
            const f32x4_t tk = mma16(z4, gblk(sM1, 1, bb, mm, cq), b);
            const float f = I < R ? sFf[(R * (R - 1) / 2 + I) * DK + c] : sDf[R * DK + c];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                aQ[jj] = fmaf(f, tq[jj], aQ[jj]);
                aK[jj] = fmaf(f, tk[jj], aK[jj]);
            }
        }
#pragma unroll 1
        for (int R2 = R; R2 < 4; ++R2) {
            const int bb = R2 * (R2 + 1) / 2 + R;
            const f32x4_t t2 = mma16(mma16(z4, gblk(sM1, 3, bb, mm, cq), tfrag<DK>(sk, c, 16 * R2 + 4 * cq)),
                                     gblk(sM1, 2, bb, mm, cq), tfrag<DK>(sq, c, 16 * R2 + 4 * cq));
            const float f = R2 > R ? sFf[(R2 * (R2 - 1) / 2 + R) * DK + c] : sDf[R * DK + c];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) aK2[jj] = fmaf(f, t2[jj], aK2[jj]);
        }
        oq[p] = aQ;
        ok1[p] = aK;
        ok2[p] = aK2;
    }
    __syncthreads();  // every operand has been read: sq, sk, sG take the three results ([token][channel])
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
        float off = sGd[c];  // gamma dgamma
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
// the state recompute's fragment records, in floats (their bytes are a multiple of 256)
static int64_t bwd_frag_floats(int Dk) { return chunk_states_record_bytes(Dk) / 4; }

// [records][states][state gradients][fragment records][X, U][dU], each per (slot, head), then one trash
// row of Dv floats (256-byte granules) for the reverse chain's stores past the end of a sequence
int64_t bwd_workspace_bytes(const BwdArgs& a) {
    const int64_t per = bwd_rec_floats(a.Dk) + 2 * (int64_t)a.Dk * a.Dv + bwd_frag_floats(a.Dk) + 3 * 64 * (int64_t)a.Dv;
    return bwd_slots(a) * a.H * per * 4 + (4 * (int64_t)a.Dv + 255) / 256 * 256;
}


template <int DK, bool F32>
static hipError_t launch_bwd_dk(const BwdArgs& a, void* ws, hipStream_t st) {
    const int64_t ch = bwd_slots(a) * a.H;
    float* recs = static_cast<float*>(ws);
    float* states = recs + ch * (int64_t)BRec<DK>::FLOATS;
    float* dstates = states + ch * (int64_t)DK * a.Dv;
    float* frecs = dstates + ch * (int64_t)DK * a.Dv;
    float* xu = frecs + ch * bwd_frag_floats(DK);
    float* du = xu + ch * 128 * (int64_t)a.Dv;
    float* trash = du + ch * 64 * (int64_t)a.Dv;
    const int64_t items = a.N * (int64_t)a.H;
    const int NS = a.Dv / kBS;
    const unsigned chain = (unsigned)(((items + 7) / 8) * 8 * NS);
    if (ch > 0) {
        // the forward pass's preparation (fragment records `frecs`, plus the plain operands `recs`)
        // and its state-only chain give the chunk-start states and X, U
        const ChunkArgs fa{a.q, a.k, a.v, a.g, a.beta, a.s0, nullptr, nullptr, a.cu_seqlens, a.T_fixed, a.total,
                           a.N, a.H, a.Dk, a.Dv, a.f32, Prologue{false, false, false, false, false}};
        const hipError_t e = launch_chunk_states(fa, frecs, recs, states, xu, st);
        if (e != hipSuccess) return e;
    }
    // with no chunks at all this only passes d_sfinal (or zeros) through to ds0
    hipLaunchKernelGGL((bwd_dstates_kernel<DK>), dim3(chain), dim3(64 * (4 + DK / 16)), 0, st, a.d_o, a.d_sfinal, a.ds0,
                       a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv, recs, dstates, du, a.dv, trash);
    if (ch > 0) {
        hipLaunchKernelGGL((bwd_grad_kernel<DK, F32>), dim3((unsigned)ch), dim3(1024), 0, st, a.q, a.k, a.g, a.d_o,
                           a.cu_seqlens, a.T_fixed, a.total, a.N, a.H, a.Dv, recs, states, dstates, xu, du, a.dv, a.dq,
                           a.dk, a.dg, a.dbeta);
    }
    return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, void* ws, hipStream_t st) {
    if (a.Dk == 128) return a.f32 ? launch_bwd_dk<128, true>(a, ws, st) : launch_bwd_dk<128, false>(a, ws, st);
    return a.f32 ? launch_bwd_dk<64, true>(a, ws, st) : launch_bwd_dk<64, false>(a, ws, st);
}

}  // namespace kda
