// Two-kernel chunked forward pass for bf16 inputs on gfx950, with fp16 matrix-core operands.
//
// The chunked form of the gated delta rule ("Kimi K3 Open Model Surpasses Closed GPT and Anthropic
// Systems on Independent Benchmarks", worldcybernews, second and third paragraphs; kda_chunk.hip
// derives it) is rearranged so that the state-dependent part of a chunk is two products long.
// With G the running sum of the clamped gates inside a chunk, Qt = e^G q, Kt = e^G k,
// Kbar = e^{G_C - G} k, M = I + A and P the decay-folded Gram blocks, and
//     N  = M^{-1} Diag(b),   W = N Kt,   Qh = Qt - P W   (= Qt - (P N) Kt),
// one chunk is, exactly up to rounding,
//     U0 = N V,   U = U0 - W S,   O = Qh S + P U0,   S' = Diag(gamma_C) S + Kbar^T U.
// O needs only the chunk's initial state, so the carried chain is U, then S'.
//
// prep16_kernel computes, per (chunk, head), -W, Qh, Kbar^T (fp16), N and P (fp16 hi + lo) and
// gamma_C, and stores them in matrix-core operand order.  chain16_kernel carries the state of one
// (sequence, head, 32-column slice) through the chunks with two workgroup barriers per chunk: U (state
// waves), then the state tiles (all waves).  The rest fills the gaps: the state waves stage V and form
// U0 of the next chunk; the output waves form Qh S after the state tiles and add P U0 in the next
// chunk's first phase.
//
// Channel order.  Within each 32-channel step, lane group g of an operand fragment holds the
// channels 32s + 4g + {0..3} and 32s + 16 + 4g + {0..3} (pi order).  A 16x16 product result holds,
// per lane, 4 consecutive rows of one column; computing W^T and Qh^T (channels as rows) therefore
// leaves two adjacent channel tiles of a token's row in exactly one pi-order fragment, so the prep
// stores them without a pass through LDS.  The chain keeps the state in LDS in the same order.
//
// Precision.  Every product accumulates in fp32; the state is carried in fp32.  -W, Qh, Kbar, S and
// U enter the products as fp16 (11 significant bits); N, P and U0 as fp16 hi + lo pairs (about 21
// bits); V as fp16, exactly (a bf16 value times a power of two is an fp16 value while in range).
// Range: the operands built from q, k and g scale with |q| |k| and |k|^2 (every decay factor is at
// most 1), which unit-norm keys and queries keep far inside fp16; V and S carry the caller's scale,
// so the chain runs on V 2^-e and S 2^-e with a per-chunk power-of-two e chosen from their maxima
// (range_exp below) and scales o and the final state back.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr int kC = 64;            // tokens per chunk
constexpr int kS = 32;            // state columns per chain workgroup
constexpr int kThreads = 576;     // chain workgroup: eight computing waves and one prefetching wave
constexpr int kThreadsSO = 512;   // state-only chain: the eight computing waves, two workgroups per CU
constexpr int kPl = 1024;         // one fragment plane: 64 lanes x 16 bytes

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// pi position p = 32s + 8g + 4h + j  <->  channel 32s + 16h + 4g + j
__host__ __device__ constexpr int pos_chan(int p) {
    return (p & ~31) + 16 * ((p >> 2) & 1) + 4 * ((p >> 3) & 3) + (p & 3);
}

__device__ __forceinline__ f32x4_t mma16(f32x4_t acc, f16x8_t a, f16x8_t b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f16x8_t to_h8(const float x[8]) {
    f16x8_t r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)x[j];
    return r;
}
__device__ __forceinline__ void to_h8_split(const float x[8], f16x8_t& hi, f16x8_t& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const _Float16 h = (_Float16)x[j];
        hi[j] = h;
        lo[j] = (_Float16)(x[j] - (float)h);
    }
}
__device__ __forceinline__ void gst_h8(char* grp, int lane, f16x8_t f) {
    __builtin_nontemporal_store(f, reinterpret_cast<f16x8_t*>(grp + lane * 16));
}
__device__ __forceinline__ f16x8_t gld_h8(const char* grp, int lane) {
    return *reinterpret_cast<const f16x8_t*>(grp + lane * 16);
}
__device__ __forceinline__ f16x8_t lds_h8(const _Float16* p) { return *reinterpret_cast<const f16x8_t*>(p); }

// Range of the fp16 state and values.  The recurrence is linear in (V, S0) jointly, so the chain may
// run on V 2^-e and S 2^-e and scale o and the final state back by 2^e.  Each chunk's e is the
// smallest e >= 0 that keeps below 2^6 the max|v| of that chunk and of the one before it, and below
// 2^10 the state's max as last measured (after the chunk before the previous one); e falls again
// when the magnitudes do, so that values after a decayed spike do not sink into fp16's subnormals.
// Inputs in the usual range keep e = 0 and are computed exactly as without it.
// range_exp(m, lg, off) is the smallest e >= 0 with m 2^(off - e) < 2^lg, capped at 100.
constexpr int kMaxRangeExp = 100;
__device__ __forceinline__ int range_exp(float m, int lg, int off = 0) {
    const int bexp = (int)((__float_as_uint(m) >> 23) & 0xff);  // m < 2^(bexp - 126)
    return min(max(bexp - 126 - lg + off, 0), kMaxRangeExp);
}
__device__ __forceinline__ float pow2i(int e) { return __int_as_float((127 + e) << 23); }  // 2^e, |e| <= 126
// Maximum over the wave of x >= 0 (compared as bit patterns): row reductions with DPP row shifts (lanes
// shifted in from outside the row read 0), then the four row results.
__device__ __forceinline__ float wave_max(float x) {
    uint32_t u = __float_as_uint(x);
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x111, 0xf, 0xf, true));  // row_shr:1
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x112, 0xf, 0xf, true));  // row_shr:2
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x114, 0xf, 0xf, true));  // row_shr:4
    u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x118, 0xf, 0xf, true));  // row_shr:8
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)u, 15);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)u, 31);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)u, 47);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)u, 63);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// Row blocks of N and P are lower triangular: row block w meets 32-wide token steps kb < steps_of(w);
// the six (w, kb) pairs are stored in order.
__host__ __device__ constexpr int steps_of(int w) { return w >= 2 ? 2 : 1; }
__host__ __device__ constexpr int pair_of(int w, int kb) { return w < 2 ? w : 2 * w - 2 + kb; }

// Operand record of one (chunk, head).
template <int DK>
struct Rec16 {
    static constexpr int KS = DK / 32;
    static constexpr int64_t W = 0;                             // -W rows:     [rb 4][s KS], fp16, pi order
    static constexpr int64_t QH = W + 4 * KS * kPl;             // Qh rows:     [rb 4][s KS], fp16, pi order
    static constexpr int64_t KB = QH + 4 * KS * kPl;            // Kbar^T rows: [cb DK/16][kb 2], fp16
    static constexpr int64_t NM = KB + (DK / 16) * 2 * kPl;     // N rows:      [pair 6][hi, lo]
    static constexpr int64_t PM = NM + 6 * 2 * kPl;             // P rows:      [pair 6][hi, lo]
    static constexpr int64_t GC = PM + 6 * 2 * kPl;             // gamma_C fp32 [DK], channel order
    static constexpr int64_t BYTES = GC + DK * 4;
    static_assert(BYTES % 256 == 0, "records stay 256-byte aligned");
};

struct SeqRange {
    int64_t start, end;
};

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

// Chunk slot of chunk j of sequence n: n * ceil(T/64) + j for equal lengths; floor(cu[n]/64) + n + j
// for packed sequences (unique, below floor(total/64) + N).
__device__ __forceinline__ int64_t slot_of(const int32_t* cu, int64_t n, int64_t j, int64_t T_fixed, int64_t start) {
    if (cu) return start / kC + n + j;
    return n * ((T_fixed + kC - 1) / kC) + j;
}

// Four consecutive bf16 values (8 bytes) as floats.
__device__ __forceinline__ void bf16x4_to_float(uint2 w, float* x) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
}
// The 8 values of a lane's pi-order fragment: channels c0 .. c0+3 and c0+16 .. c0+19 (c0 = 32s + 4g).
__device__ __forceinline__ void load_pi8_bf16(const uint16_t* p, float x[8]) {
    bf16x4_to_float(*reinterpret_cast<const uint2*>(p), x);
    bf16x4_to_float(*reinterpret_cast<const uint2*>(p + 16), x + 4);
}
__device__ __forceinline__ void load_pi8_gate(const void* g, int64_t idx, bool bf, float x[8]) {
    if (bf) {
        load_pi8_bf16(static_cast<const uint16_t*>(g) + idx, x);
    } else {
        const float* p = static_cast<const float*>(g) + idx;
        const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 16);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

}  // namespace

// ============================================================================ prep kernel

// Lower block-triangular fp32 [64][64] matrix (A, then N; P, then -P N): row block R keeps its 16 (R + 1)
// columns plus 4 of padding, so rows stay 16-byte aligned and 16 rows of one column fall in 16 banks.
__host__ __device__ constexpr int tri_stride(int R) { return 16 * R + 20; }
__host__ __device__ constexpr int tri_base(int R) { return 128 * R * R + 192 * R; }
// element (row 16 R + rr, column c), c < 16 (R + 1)
__host__ __device__ constexpr int tri(int R, int rr, int c) { return tri_base(R) + rr * tri_stride(R) + c; }
constexpr int kTriFloats = tri_base(4);  // 2816

template <int DK>
struct Prep16Lds {
    // The regions live in two phases.  Up to the Gram results: the fp32 Gram column operands of sub-blocks
    // 0..2 [48][DK+4] (pi positions) and row block 3's Gram operands for waves 0 and 1.  From then on:
    // A (later N) and P (later -P N) in block-triangular form, the fp16 staging of Kbar^T and then Kt^T
    // [DK][72], and the diagonal inverses.  The gates' sub-block sums are only read before the column
    // operands are written.  Tables and b live throughout.  At DK = 128 this is 53,248 bytes: three
    // workgroups per CU.
    static constexpr int COL_BYTES = 48 * (DK + 4) * 4;
    static constexpr int ROW3_BYTES = DK / 32 * 3 * 64 * 16;
    static constexpr int STG = 72;                         // halves per row of the fp16 staging [DK][72]
    static constexpr int TRI_BYTES = kTriFloats * 4;
    static constexpr int COL = 0;                          // phase 1: column operands
    static constexpr int ROW3 = COL + COL_BYTES;           // phase 1: row block 3's Gram operands
    static constexpr int GT = 0;                           // before phase 1: sub-block gate sums (log2) [4][DK]
    static constexpr int A = 0;                            // phase 2: b_r A_ri, later N
    static constexpr int PM = A + TRI_BYTES;               // phase 2: P, later -P N (rows of block w by wave w)
    static constexpr int STGO = PM + TRI_BYTES;            // phase 2: fp16 Kbar^T, later Kt^T [DK][72]
    static constexpr int D = STGO + DK * STG * 2;          // phase 2: fp32 diagonal inverses [4][16][17]
    static constexpr int END2 = D + 4 * 16 * 17 * 4;
    static constexpr int END1 = ROW3 + ROW3_BYTES;
    static_assert(ROW3 + ROW3_BYTES <= D, "row block 3's operands stay clear of the diagonal inverses");
    static_assert(GT + 4 * DK * 4 <= COL_BYTES, "the gate sums lie inside the column operands");
    static constexpr int TAB = END1 > END2 ? END1 : END2;  // fp32 tables [15][DK] (pi positions)
    static constexpr int BETA = TAB + 15 * DK * 4;         // fp32 b [64]
    static constexpr int TOTAL = BETA + 64 * 4;
    static_assert(DK != 128 || TOTAL <= 160 * 1024 / 3, "three prep workgroups per CU");
};

// The decay-folded Gram blocks (R, I), I <= R, of A (one bf16 pass; scaled by b_r and strictly lower on
// the diagonal block) and P (three passes; lower with diagonal), in 16x16 blocks.  Row block R's
// operands are q E and k E of its rows (E = e^{Gloc}, the sub-block-relative decay), column block I's
// are k e^{G_end(I) - G} times the decay over the blocks between (sCol, tD) or, on the diagonal,
// k / E of the same rows; all in pi order.  Row block 3 has four blocks and row block 0 one, so the
// work is shared out: wave W computes (W, I) for I <= W except that (3, 0) and (3, 1) go to waves 0
// and 1, which read row block 3's operands from the fragments wave 3 staged in LDS (sRow3).  Results
// stay in registers until every wave has read its operands (the staging lies over sA).
template <int DK>
struct GramOut {
    f32x4_t a[3], p[3];
};
template <int W, int DK>
__device__ __forceinline__ void gram16(const float (*xq)[8], const float (*xk)[8], const float (*x3)[8],
                                       const float* sCol, const float* tD, const bf16x8_t* sRow3, int lane,
                                       int m, int cg, GramOut<DK>& g) {
    using Fr = Frag<false>;
    constexpr int KS = DK / 32;
    constexpr int ILO = W == 3 ? 2 : 0;   // own row block: column blocks ILO..W
    constexpr int NX = W < 2 ? 1 : 0;     // one block of row block 3: (3, W)
#pragma unroll
    for (int i = 0; i < 3; ++i) g.a[i] = g.p[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // column operand of block I for row block R, channels of step s
    auto col = [&](int R, int I, int s, Fr& colf) {
        float cx[8];
        lds_read8(sCol + (16 * I + m) * (DK + 4) + 32 * s + 8 * cg, cx);
        if (R - I >= 2) {
            const int dsel = (R - I == 3) ? 2 : I;  // (0,2)->0, (1,3)->1, (0,3)->2
            float d[8];
            lds_read8(&tD[dsel * DK + 32 * s + 8 * cg], d);
#pragma unroll
            for (int j = 0; j < 8; ++j) cx[j] *= d[j];
        }
        colf.set(cx);
    };
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        Fr fqE, fkE, fkd;
        fqE.set(xq[s]);
        fkE.set_hi_only(xk[s]);
        fkd.set(x3[s]);
#pragma unroll
        for (int I = ILO; I < W; ++I) {
            Fr colf;
            col(W, I, s, colf);
            g.a[I - ILO] = mma_fast(g.a[I - ILO], fkE, colf);
            g.p[I - ILO] = mma_full(g.p[I - ILO], fqE, colf);
        }
        g.a[W - ILO] = mma_fast(g.a[W - ILO], fkE, fkd);
        g.p[W - ILO] = mma_full(g.p[W - ILO], fqE, fkd);
        if constexpr (NX) {
            Fr rq, rk, colf;
            rq.hi = sRow3[(s * 3 + 0) * 64 + lane];
            rq.lo = sRow3[(s * 3 + 1) * 64 + lane];
            rk.hi = sRow3[(s * 3 + 2) * 64 + lane];
            col(3, W, s, colf);
            g.a[W + 1] = mma_fast(g.a[W + 1], rk, colf);
            g.p[W + 1] = mma_full(g.p[W + 1], rq, colf);
        }
    }
}
// Gram results of wave W to sA (times b_r) and sP: its own row block (zeros right of the diagonal block;
// for row block 3 only its blocks 2 and 3) and, for waves 0 and 1, block (3, W).
template <int W, int DK>
__device__ __forceinline__ void gram16_store(const GramOut<DK>& g, const float* sBeta, float* sA, float* sP, int m,
                                             int cg) {
    constexpr int ILO = W == 3 ? 2 : 0;
    auto put = [&](int R, int I, const f32x4_t& a, const f32x4_t& pv, bool diag) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int rr = 4 * cg + jj;
            const int gr = 16 * R + rr, gi = 16 * I + m;
            float av = a[jj], pp = pv[jj];
            if (diag) {
                if (m >= rr) av = 0.f;
                if (m > rr) pp = 0.f;
            }
            sA[tri(R, rr, gi)] = av * sBeta[gr];
            sP[tri(R, rr, gi)] = pp;
        }
    };
#pragma unroll
    for (int I = ILO; I <= W; ++I) put(W, I, g.a[I - ILO], g.p[I - ILO], I == W);
    if constexpr (W < 2) put(3, W, g.a[W + 1], g.p[W + 1], false);
}

// -P N in 16x16 tiles (R, ct), ct <= R: tile (R, ct) = sum_{J=ct}^{R} P_RJ N_Jct (fp32 MFMA, P rows from
// sP, N from sA).  Row block 3 has four tiles of up to four products and row block 0 one, so wave W
// takes (W, ct) for ct <= W except that (3, 0) and (3, 1) go to waves 0 and 1.  Tiles are stored over
// the P rows only after every wave has read them.
template <int W>
__device__ __forceinline__ void pn_tiles(const float* sP, const float* sA, int m, int cg, f32x4_t (&pn)[3]) {
    constexpr int CLO = W == 3 ? 2 : 0;
    auto tile = [&](int R, int ct) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            if (J < ct || J > R) continue;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sP[tri(R, m, 16 * J + 4 * kk + cg)],
                                                           sA[tri(J, 4 * kk + cg, 16 * ct + m)], acc, 0, 0, 0);
        }
        return acc;
    };
#pragma unroll
    for (int ct = CLO; ct <= W; ++ct) pn[ct - CLO] = tile(W, ct);
    if constexpr (W < 2) pn[W + 1] = tile(3, W);
}
template <int W>
__device__ __forceinline__ void pn_store(float* sP, int m, int cg, const f32x4_t (&pn)[3]) {
    constexpr int CLO = W == 3 ? 2 : 0;
    auto put = [&](int R, int ct, const f32x4_t& x) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) sP[tri(R, 4 * cg + jj, 16 * ct + m)] = -x[jj];
    };
#pragma unroll
    for (int ct = CLO; ct <= W; ++ct) put(W, ct, pn[ct - CLO]);
    if constexpr (W < 2) put(3, W, pn[W + 1]);
}

// One workgroup (four waves, wave w = token rows 16w..16w+15) per (chunk, head); three per CU.
template <int DK, bool PRO>
__global__ __launch_bounds__(256, 3) void prep16_kernel(const void* __restrict__ qv, const void* __restrict__ kv,
                                                        const void* __restrict__ gv, const void* __restrict__ bv,
                                                        const int32_t* __restrict__ cu_seqlens, int64_t T_fixed,
                                                        int64_t T_stride, int64_t total, int64_t N, int H,
                                                        Prologue pro, char* __restrict__ ws) {
    using L = Prep16Lds<DK>;
    using R = Rec16<DK>;
    constexpr int KS = DK / 32;
    // input prologue; PRO = false compiles the plain form (fp32 log alpha and beta, q and k as given)
    const Prologue pf{PRO && pro.g_bf16, PRO && pro.g_logit, PRO && pro.b_bf16, PRO && pro.b_logit,
                      PRO && pro.l2norm};
    const uint16_t* __restrict__ q = static_cast<const uint16_t*>(qv);
    const uint16_t* __restrict__ k = static_cast<const uint16_t*>(kv);

    __shared__ __align__(16) char smem[L::TOTAL];
    float* sCol = reinterpret_cast<float*>(smem + L::COL);
    _Float16* sStg = reinterpret_cast<_Float16*>(smem + L::STGO);
    float* sP = reinterpret_cast<float*>(smem + L::PM);
    float* sA = reinterpret_cast<float*>(smem + L::A);
    bf16x8_t* sRow3 = reinterpret_cast<bf16x8_t*>(smem + L::ROW3);
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

    // ---- rows of sub-block w (rows past the end re-read the last row); running gate sums (log2)
    const int r = 16 * w + m;
    const bool rv = r < nt;
    // this lane's 8 columns 32 kb + 8 cg.. of row r of a block-triangular matrix (zeros right of block w)
    auto tri_row8 = [&](const float* t, int kb, float x[8]) {
        const int c0 = 32 * kb + 8 * cg;
        const bool in = c0 < 16 * (w + 1);
        lds_read8(t + tri(w, m, in ? c0 : 0), x);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] = in ? x[jj] : 0.f;
    };
    const int64_t base = ((t0 + min(r, nt - 1)) * H + h) * (int64_t)DK + 4 * cg;
    float braw = 0.f;
    if (tid < kC) braw = load1_gate(bv, (t0 + min(tid, nt - 1)) * H + h, pf.b_bf16);
    float xq[KS][8], xk[KS][8], gl[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) load_pi8_gate(gv, base + 32 * s, pf.g_bf16, gl[s]);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        load_pi8_bf16(q + base + 32 * s, xq[s]);
        load_pi8_bf16(k + base + 32 * s, xk[s]);
    }
    if (tid < kC) sBeta[tid] = tid < nt ? beta_value(braw, pf.b_logit) : 0.f;
    if (pf.l2norm) {  // unit q and k rows: each row lives in lanes m, m+16, m+32, m+48
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                sq = fmaf(xq[s][jj], xq[s][jj], sq);
                sk = fmaf(xk[s][jj], xk[s][jj], sk);
            }
        const float rq = rnorm_lanes4(sq), rk = rnorm_lanes4(sk);
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                xq[s][jj] *= rq;
                xk[s][jj] *= rk;
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

    // ---- per-position tables; gamma_C to the record in channel order
    if (tid < DK) {
        const int p = tid;
        const float G0 = sGt[p], G1 = sGt[DK + p], G2 = sGt[2 * DK + p], G3 = sGt[3 * DK + p];
        tPw[p] = 1.f;
        tPw[DK + p] = __builtin_amdgcn_exp2f(G0);
        tPw[2 * DK + p] = __builtin_amdgcn_exp2f(G0 + G1);
        tPw[3 * DK + p] = __builtin_amdgcn_exp2f(G0 + G1 + G2);
        tAf[p] = __builtin_amdgcn_exp2f(G1 + G2 + G3);
        tAf[DK + p] = __builtin_amdgcn_exp2f(G2 + G3);
        tAf[2 * DK + p] = __builtin_amdgcn_exp2f(G3);
        tAf[3 * DK + p] = 1.f;
        tBt[p] = __builtin_amdgcn_exp2f(G0);
        tBt[DK + p] = __builtin_amdgcn_exp2f(G1);
        tBt[2 * DK + p] = __builtin_amdgcn_exp2f(G2);
        tBt[3 * DK + p] = __builtin_amdgcn_exp2f(G3);
        tD[p] = __builtin_amdgcn_exp2f(G1);
        tD[DK + p] = __builtin_amdgcn_exp2f(G2);
        tD[2 * DK + p] = __builtin_amdgcn_exp2f(G1 + G2);
        const float GC = ((G0 + G1) + G2) + G3;
        reinterpret_cast<float*>(rec + R::GC)[pos_chan(p)] = __builtin_amdgcn_exp2f(GC);
    }
    lds_barrier();  // (2)

    // ---- sub-block-relative factors E = e^{Gloc}: xq <- q E, xk <- k E, x3 = k / E; column operands
    // k e^{G_end(w) - G_r} of sub-blocks 0..2 to LDS
    float x3[KS][8];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int p0 = 32 * s + 8 * cg;
        float bt[8];
        lds_read8(&tBt[w * DK + p0], bt);
        float xc[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const float E = __builtin_amdgcn_exp2f(gl[s][jj]);
            const float Ei = __builtin_amdgcn_exp2f(-gl[s][jj]);
            x3[s][jj] = xk[s][jj] * Ei;
            xq[s][jj] *= E;
            xk[s][jj] *= E;
            xc[jj] = x3[s][jj] * bt[jj];
        }
        if (w < 3) {
            float* dst = sCol + r * (DK + 4) + p0;
            *reinterpret_cast<float4*>(dst) = make_float4(xc[0], xc[1], xc[2], xc[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(xc[4], xc[5], xc[6], xc[7]);
        } else {  // row block 3's Gram operands (q E split, k E high part) for waves 0 and 1
            Frag<false> fq, fk;
            fq.set(xq[s]);
            fk.set_hi_only(xk[s]);
            sRow3[(s * 3 + 0) * 64 + lane] = fq.hi;
            sRow3[(s * 3 + 1) * 64 + lane] = fq.lo;
            sRow3[(s * 3 + 2) * 64 + lane] = fk.hi;
        }
    }
    lds_barrier();  // (3)

    {
        GramOut<DK> go;
        switch (w) {
            case 0: gram16<0, DK>(xq, xk, x3, sCol, tD, sRow3, lane, m, cg, go); break;
            case 1: gram16<1, DK>(xq, xk, x3, sCol, tD, sRow3, lane, m, cg, go); break;
            case 2: gram16<2, DK>(xq, xk, x3, sCol, tD, sRow3, lane, m, cg, go); break;
            default: gram16<3, DK>(xq, xk, x3, sCol, tD, sRow3, lane, m, cg, go); break;
        }
        lds_barrier();  // (3b) the staged operands are read
        switch (w) {
            case 0: gram16_store<0, DK>(go, sBeta, sA, sP, m, cg); break;
            case 1: gram16_store<1, DK>(go, sBeta, sA, sP, m, cg); break;
            case 2: gram16_store<2, DK>(go, sBeta, sA, sP, m, cg); break;
            default: gram16_store<3, DK>(go, sBeta, sA, sP, m, cg); break;
        }
    }
    lds_barrier();  // (4)

    // ---- diagonal blocks of M^{-1} = (I + A)^{-1}: forward substitution, one column per lane
    if (lane < 16) {
        const int cidx = lane;
        const int ast = tri_stride(w);
        const float* Ab = &sA[tri(w, 0, 16 * w)];
        float x[16];
#pragma unroll
        for (int rr = 0; rr < 16; ++rr, Ab += ast) {
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < rr; ++jj) acc[jj & 3] = fmaf(Ab[jj], x[jj], acc[jj & 3]);
            const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            x[rr] = (rr == cidx) ? 1.f : (rr < cidx ? 0.f : -sum);
        }
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) sD[(w * 16 + rr) * 17 + cidx] = x[rr];
    }
    // ---- P rows of block w to the record (fp16 hi + lo)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb >= steps_of(w)) continue;
        float x[8];
        tri_row8(sP, kb, x);
        f16x8_t hi, lo;
        to_h8_split(x, hi, lo);
        char* dst = rec + R::PM + pair_of(w, kb) * 2 * kPl;
        gst_h8(dst, lane, hi);
        gst_h8(dst + kPl, lane, lo);
    }
    lds_barrier();  // (5)

    // ---- column block I = w of M^{-1}: N_II = D_I, N_RI = -D_R sum_{J=I}^{R-1} A_RJ N_JI (fp32 MFMA)
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
                        z = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[tri(R_, m, 16 * J + 4 * cg + jj)],
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
    // ---- Kbar = e^{G_C - G} k staged as fp16 Kbar^T [channel][token] over the column operands
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int p0 = 32 * s + 8 * cg;
        float bt[8], af[8];
        lds_read8(&tBt[w * DK + p0], bt);
        lds_read8(&tAf[w * DK + p0], af);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            sStg[pos_chan(p0 + jj) * L::STG + r] = (_Float16)((x3[s][jj] * bt[jj]) * af[jj]);
    }
    lds_barrier();  // (6)

    // ---- N = M^{-1} Diag(b) over A (A is no longer read); Kbar^T fragments to the record
    {
        const float bcol = sBeta[16 * w + m];
#pragma unroll
        for (int R_ = 0; R_ < 4; ++R_)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                if (R_ >= w) sA[tri(R_, 4 * cg + jj, 16 * w + m)] = Nr[R_][jj] * bcol;
    }
#pragma unroll
    for (int i = 0; i < DK / 32; ++i) {  // (c-block, kb) groups w, w+4, ...
        const int gidx = w + 4 * i;
        const int cb = gidx >> 1, kb = gidx & 1;
        gst_h8(rec + R::KB + (cb * 2 + kb) * kPl, lane, lds_h8(sStg + (16 * cb + m) * L::STG + 32 * kb + 8 * cg));
    }
    lds_barrier();  // (7)

    // ---- N rows of block w to the record; -P N rows of block w over its P rows (fp32 MFMA; only this
    // wave reads or writes them); Kt = e^G k staged as fp16 Kt^T [channel][token]
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        if (kb >= steps_of(w)) continue;
        float x[8];
        tri_row8(sA, kb, x);
        f16x8_t hi, lo;
        to_h8_split(x, hi, lo);
        char* dst = rec + R::NM + pair_of(w, kb) * 2 * kPl;
        gst_h8(dst, lane, hi);
        gst_h8(dst + kPl, lane, lo);
    }
    {
        f32x4_t pn[3];
        switch (w) {
            case 0: pn_tiles<0>(sP, sA, m, cg, pn); break;
            case 1: pn_tiles<1>(sP, sA, m, cg, pn); break;
            case 2: pn_tiles<2>(sP, sA, m, cg, pn); break;
            default: pn_tiles<3>(sP, sA, m, cg, pn); break;
        }
        lds_barrier();  // (7b) every P row is read
        switch (w) {
            case 0: pn_store<0>(sP, m, cg, pn); break;
            case 1: pn_store<1>(sP, m, cg, pn); break;
            case 2: pn_store<2>(sP, m, cg, pn); break;
            default: pn_store<3>(sP, m, cg, pn); break;
        }
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int p0 = 32 * s + 8 * cg;
        float pw[8];
        lds_read8(&tPw[w * DK + p0], pw);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sStg[pos_chan(p0 + jj) * L::STG + r] = (_Float16)(xk[s][jj] * pw[jj]);
    }
    lds_barrier();  // (8)

    // ---- W^T = Kt^T N^T and Qh^T = Qt^T - Kt^T (P N)^T for this wave's tokens (columns), every channel
    // tile (rows); tiles 2s and 2s+1 of a token form its pi-order fragment of step s
    {
        f16x8_t bN[2][2], bC[2][2];  // [kb][hi, lo]: N and -P N rows of this lane's token
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb >= steps_of(w)) continue;
            float x[8];
            tri_row8(sA, kb, x);
            to_h8_split(x, bN[kb][0], bN[kb][1]);
            tri_row8(sP, kb, x);
            to_h8_split(x, bC[kb][0], bC[kb][1]);
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float pw[8];
            lds_read8(&tPw[w * DK + 32 * s + 8 * cg], pw);
            f32x4_t accW[2], accQ[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                accW[hh] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) accQ[hh][jj] = xq[s][4 * hh + jj] * pw[4 * hh + jj];  // Qt
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (kb >= steps_of(w)) continue;
                    const f16x8_t a = lds_h8(sStg + (32 * s + 16 * hh + m) * L::STG + 32 * kb + 8 * cg);
                    accW[hh] = mma16(accW[hh], a, bN[kb][0]);
                    accW[hh] = mma16(accW[hh], a, bN[kb][1]);
                    accQ[hh] = mma16(accQ[hh], a, bC[kb][0]);
                    accQ[hh] = mma16(accQ[hh], a, bC[kb][1]);
                }
            }
            float xw[8], xh[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    xw[4 * hh + jj] = -accW[hh][jj];
                    xh[4 * hh + jj] = accQ[hh][jj];
                }
            gst_h8(rec + R::W + (w * KS + s) * kPl, lane, to_h8(xw));
            gst_h8(rec + R::QH + (w * KS + s) * kPl, lane, to_h8(xh));
        }
    }
}

// ============================================================================ chain kernel

template <int DK>
struct Chain16Lds {
    static constexpr int SST = DK + 8;                      // halves per state column (pi positions)
    static constexpr int TST = 72;                          // halves per column of U^T, U0^T, V^T (tokens)
    static constexpr int S = 0;                             // fp16 S^T [2 bufs][32 cols][SST]
    static constexpr int U = S + 2 * kS * SST * 2;          // fp16 U^T [32][TST]
    static constexpr int U0 = U + kS * TST * 2;             // fp16 U0^T [2 bufs][hi, lo][32][TST]
    static constexpr int V = U0 + 2 * 2 * kS * TST * 2;     // bf16 V^T [32][TST] (as loaded, scaled when read)
    static constexpr int O = V + kS * TST * 2;              // fp32 output rows [64][kS + 4] on their way to HBM
    static constexpr int MX = O + 64 * (kS + 4) * 4;  // fp32 maxima: [12] s0 and V, [2][4] V, [2][8] state
    static constexpr int TOTAL = MX + 36 * 4;
};

// Operands of one chunk.  A state wave (row block rb) holds -W rows of rb and the Kbar^T rows and
// gamma_C of its state tiles, and, for the chunk after, N rows of rb and its pieces of v (U0 of the next
// chunk is formed during this one).  An output wave holds Qh and P rows of rb and its state tiles'
// Kbar^T rows and gamma_C.
template <int DK>
struct StOps16 {
    f16x8_t fW[DK / 32], fKB[2], fN[2][2];
    float4 gC;
    uint4 vraw;
};
template <int DK>
struct OutOps16 {
    f16x8_t fQ[DK / 32], fKB[2], fP[2][2];
    float4 gC;
};

// Modes as the ChainMode of the split-fp32 chain: 0 whole sequences; 1 segment maps (value columns
// from a zero state, identity columns with V = 0; SO compiles the outputs out); 2 segment outputs from
// the folded initial states.
template <int DK, bool SO>
__global__ __launch_bounds__(SO ? kThreadsSO : kThreads, SO ? 4 : 1) void chain16_kernel(const void* __restrict__ vv, const float* s0,
                                                              float* __restrict__ o, float* s_final,
                                                              const int32_t* __restrict__ cu_seqlens, int64_t T_fixed,
                                                              int64_t T_stride, int64_t total, int64_t N, int H,
                                                              int Dv, ChainMode cm,
                                                              const char* ws) {  // not restrict: see kda_chunk2.hip
    using L = Chain16Lds<DK>;
    using R = Rec16<DK>;
    constexpr int KS = DK / 32;
    constexpr int TPW = DK / 64;                    // state tiles per wave (all in one channel block)
    const uint16_t* __restrict__ v = static_cast<const uint16_t*>(vv);

    __shared__ __align__(16) char smem[L::TOTAL];
    _Float16* sS = reinterpret_cast<_Float16*>(smem + L::S);
    _Float16* sU = reinterpret_cast<_Float16*>(smem + L::U);
    _Float16* sU0 = reinterpret_cast<_Float16*>(smem + L::U0);
    uint16_t* sV = reinterpret_cast<uint16_t*>(smem + L::V);
    float* sMx = reinterpret_cast<float*>(smem + L::MX);
    float* sO = reinterpret_cast<float*>(smem + L::O);

    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, m = lane & 15, cg = lane >> 4;
    const bool prefetcher = w == 8;                            // the ninth wave only prefetches records
    const int wt = prefetcher ? 0 : w;
    const int rb = wt & 3;
    const int cbw = (wt * TPW) >> 1;                           // channel block of this wave's state tiles
    auto nbt = [&](int i) { return (wt * TPW + i) & 1; };     // column half of state tile i
    const int NV = Dv / kS;
    const int NS = cm.mode == 1 ? NV + DK / kS : NV;
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
    const bool ident = sl >= NV;
    const int col0 = ident ? 0 : sl * kS;
    const int colx = sl * kS;
    const float vscale = ident ? 0.f : 1.f;
    const int nk = steps_of(rb);

    const float* const s_src = cm.mode == 1 ? nullptr
                               : (cm.mode == 2 ? cm.sfold + (((n * H + h) * (int64_t)cm.P + p) * DK) * Dv
                                               : (s0 ? s0 + (n * H + h) * (int64_t)DK * Dv : nullptr));
    float* const sdst = cm.mode == 1 ? cm.sx + (pr * DK) * (int64_t)(Dv + DK)
                                     : ((cm.mode == 0 || p == cm.P - 1) && s_final
                                            ? s_final + (n * H + h) * (int64_t)DK * Dv : nullptr);
    const int ld_dst = cm.mode == 1 ? Dv + DK : Dv;
    const int col_dst = cm.mode == 1 ? colx : col0;

    // ---- state tiles of this wave (fp32, registers) and their fp16 copy in LDS
    f32x4_t accS[TPW];
    if (prefetcher) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) accS[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    } else if (cm.mode == 1) {  // zero value columns; the identity on the identity columns
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c = 16 * cbw + 4 * cg + jj, col = 16 * nbt(i) + m;
                accS[i][jj] = ident && c == colx - Dv + col ? 1.f : 0.f;
            }
    } else if (s_src) {
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                accS[i][jj] = s_src[(16 * cbw + 4 * cg + jj) * Dv + col0 + 16 * nbt(i) + m];
    } else {
#pragma unroll
        for (int i = 0; i < TPW; ++i) accS[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // a tile's lane holds channels 16cb + 4cg + {0..3}: pi positions 32(cb/2) + 8cg + 4(cb%2) + {0..3}
    const int spos = 32 * (cbw >> 1) + 8 * cg + 4 * (cbw & 1);
    auto store_state = [&](int buf) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            f16x4_t x;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) x[jj] = (_Float16)accS[i][jj];
            *reinterpret_cast<f16x4_t*>(sS + (buf * kS + 16 * nbt(i) + m) * L::SST + spos) = x;
        }
    };
    int e = 0;  // range exponent of the current chunk (uniform over the workgroup)
    if (!prefetcher) {
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) mx = fmaxf(mx, fabsf(accS[i][jj]));
        mx = wave_max(mx);
        if (lane == 0) sMx[w] = mx;
    }
    // Maxima in LDS: sMx[0..7] the initial state's per wave; V of chunk x at 12 + 4 ((x + 1) & 1), per
    // row block; the state after chunk x (in the units of chunk x + 1) at 20 + 8 (x & 1), per wave.
    const int vslot0 = 12 + 4 * (int)((jbeg + 1) & 1);
    // after the first barrier: the range of the first chunk from the initial state and its V; the
    // state's fp16 copy in those units and its maximum there (as the state "after chunk jbeg - 1")
    auto first_range = [&]() {
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, sMx[i]);
        e = range_exp(mx, 10);
        mx = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sMx[vslot0 + i]);
        e = max(e, range_exp(mx, 6));
        if (!prefetcher) {
            const float sc = pow2i(-e);
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) accS[i][jj] *= sc;
            store_state(jbeg & 1);
            if (lane == 0) sMx[20 + 8 * (int)((jbeg + 1) & 1) + w] = sc * sMx[w];
        }
    };

    auto record = [&](int64_t jc) -> const char* {
        return ws + (slot_of(cu_seqlens, n, jc, T_fixed, start) * H + h) * R::BYTES;
    };
    auto chunk_start = [&](int64_t jc) { return start + jc * kC; };
    auto chunk_len = [&](int64_t jc) { return (int)min<int64_t>(kC, end - chunk_start(jc)); };
    auto next_chunk = [&](int64_t jc) { return jc + 1 < jend ? jc + 1 : jc; };

    // S' = Diag(gamma_C) S + Kbar^T U of chunk jc on this wave's tiles, from U^T in LDS; then, in the
    // units of the next chunk (range exponent en), its fp16 copy and its maximum
    auto update_state = [&](const f16x8_t (&fKB)[2], float4 gC, int buf, int en, int64_t jc) {
        const float gcv[4] = {gC.x, gC.y, gC.z, gC.w};
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) accS[i][jj] *= gcv[jj];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                accS[i] = mma16(accS[i], fKB[kb], lds_h8(sU + (16 * nbt(i) + m) * L::TST + 32 * kb + 8 * cg));
        }
        if (en != e) {
            const float sc = pow2i(e - en);
#pragma unroll
            for (int i = 0; i < TPW; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) accS[i][jj] *= sc;
        }
        store_state(buf);
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) mx = fmaxf(mx, fabsf(accS[i][jj]));
        mx = wave_max(mx);
        if (lane == 0) sMx[20 + 8 * (int)(jc & 1) + w] = mx;
    };
    // range exponent of the chunk after jc, in step jc after its first barrier: from the V maxima of
    // chunks jc + 1 (posted in step jc) and jc, and the state maximum after chunk jc - 1 (in units e)
    auto next_range = [&](int64_t jc) {
        const float* ms = sMx + 20 + 8 * (int)((jc + 1) & 1);
        float mv = 0.f, mx = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) mv = fmaxf(mv, sMx[12 + i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) mx = fmaxf(mx, ms[i]);
        return max(range_exp(mv, 6), range_exp(mx, 10, e));
    };
    auto load_kb = [&](f16x8_t (&fKB)[2], float4& gC, const char* rec) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) fKB[kb] = gld_h8(rec + R::KB + (cbw * 2 + kb) * kPl, lane);
        gC = *reinterpret_cast<const float4*>(rec + R::GC + (16 * cbw + 4 * cg) * 4);
    };
    // S fragment (B operand) of pi step s, column half nb
    auto s_frag = [&](int buf, int s, int nb) {
        return lds_h8(sS + (buf * kS + 16 * nb + m) * L::SST + 32 * s + 8 * cg);
    };

    // V of a chunk as fp16 V^T in LDS, and U0 = N V (two passes: N hi, N lo) of row block rb: the state
    // waves form both, for the chunk after the current one
    const uint32_t rs_v = (uint32_t)H * (uint32_t)Dv;
    const int vrow = 16 * rb + (lane >> 2), vpiece = lane & 3;  // 16 rows x 4 pieces of 8 columns
    const uint16_t* __restrict__ v_l = v + (int64_t)h * Dv + col0 + vpiece * 8;

    if (w < 4) {
        // ======================= state waves: U of row block rb, V and U0 of the next chunk
        using Ops = StOps16<DK>;
        auto load_w = [&](Ops& d, const char* rec) {
#pragma unroll
            for (int s = 0; s < KS; ++s) d.fW[s] = gld_h8(rec + R::W + (rb * KS + s) * kPl, lane);
        };
        auto load_n = [&](Ops& d, int64_t jx) {  // N rows of rb of chunk jx
            const char* rec = record(jx);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {  // blocks 0, 1 stop at token 31: their second step repeats the first
                const char* g = rec + R::NM + pair_of(rb, min(kb, nk - 1)) * 2 * kPl;
                d.fN[kb][0] = gld_h8(g, lane);
                d.fN[kb][1] = gld_h8(g + kPl, lane);
            }
        };
        auto load_v = [&](uint4& raw, int64_t jx) {
            const uint32_t rvo = (uint32_t)min(vrow, chunk_len(jx) - 1) * rs_v;
            raw = *reinterpret_cast<const uint4*>(v_l + chunk_start(jx) * (int64_t)rs_v + rvo);
        };
        // V of a chunk to LDS as loaded (bf16, transposed); its largest |value| over this wave's rows
        // posted to sMx[slot]
        auto stage_v = [&](uint4 raw, int slot) {
            const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
            float mx = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sV[(vpiece * 8 + 2 * i) * L::TST + vrow] = (uint16_t)(u[i] & 0xffffu);
                sV[(vpiece * 8 + 2 * i + 1) * L::TST + vrow] = (uint16_t)(u[i] >> 16);
                mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(u[i] << 16)), fabsf(__uint_as_float(u[i] & 0xffff0000u))));
            }
            mx = wave_max(vscale * mx);
            if (lane == 0) sMx[slot] = mx;
        };
        f32x4_t accU0[2];
        // U0 = N V (two passes: N hi, N lo) for rows rb, V in the units of range exponent ev: into accU0
        // and, split, into U0^T buffer buf
        auto form_u0 = [&](const f16x8_t (&fN)[2][2], int buf, int ev) {
            const float sc = vscale * pow2i(-ev);
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (kb >= nk) continue;
                    const uint4 raw = *reinterpret_cast<const uint4*>(sV + (16 * nb + m) * L::TST + 32 * kb + 8 * cg);
                    const uint32_t u[4] = {raw.x, raw.y, raw.z, raw.w};
                    f16x8_t bv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        bv[2 * i] = (_Float16)(sc * __uint_as_float(u[i] << 16));
                        bv[2 * i + 1] = (_Float16)(sc * __uint_as_float(u[i] & 0xffff0000u));
                    }
                    acc = mma16(acc, fN[kb][0], bv);
                    acc = mma16(acc, fN[kb][1], bv);
                }
                accU0[nb] = acc;
                f16x4_t hi, lo;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const _Float16 x = (_Float16)acc[jj];
                    hi[jj] = x;
                    lo[jj] = (_Float16)(acc[jj] - (float)x);
                }
                _Float16* dst = sU0 + ((buf * 2) * kS + 16 * nb + m) * L::TST + 16 * rb + 4 * cg;
                *reinterpret_cast<f16x4_t*>(dst) = hi;
                *reinterpret_cast<f16x4_t*>(dst + kS * L::TST) = lo;
            }
        };
        // Register sets: the set of chunk x holds -W, Kbar^T, gamma_C of chunk x and N of chunk x + 1
        // (loaded one chunk ahead), and v of chunk x + 1 (loaded two chunks ahead, into the set of the
        // same parity right after it is staged).
        auto step = [&](Ops& cur, Ops& nxt, int64_t jc) {
            const int64_t jn = next_chunk(jc);
            const char* recn = record(jn);
            const int b = (int)(jc & 1);

            // ---- phase 1:  U = U0 - W S;  V of the next chunk to LDS
            // v two chunks ahead, first in the step: memory requests complete in order, and the loop's
            // first wait covers every request made before it, so this one (usually an HBM miss) gets a
            // whole step to arrive
            const uint4 vcur = cur.vraw;
            load_v(cur.vraw, next_chunk(next_chunk(jn)));
            f32x4_t accU[2] = {accU0[0], accU0[1]};
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) accU[nb] = mma16(accU[nb], cur.fW[s], s_frag(b, s, nb));
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                f16x4_t x;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) x[jj] = (_Float16)accU[nb][jj];
                *reinterpret_cast<f16x4_t*>(sU + (16 * nb + m) * L::TST + 16 * rb + 4 * cg) = x;
            }
            stage_v(vcur, 12 + 4 * b + rb);  // V of chunk jc + 1
            load_w(nxt, recn);  // after the products that read this chunk's copy
            lds_barrier();  // (1)

            // ---- phase 2:  state tiles;  U0 of the next chunk (both in the next chunk's units)
            const int en = next_range(jc);
            update_state(cur.fKB, cur.gC, b ^ 1, en, jc);
            load_kb(nxt.fKB, nxt.gC, recn);
            form_u0(cur.fN, b ^ 1, en);
            load_n(nxt, next_chunk(jn));  // after the products that read this copy of N
            e = en;
            lds_barrier();  // (2)
        };
        Ops opsA, opsB;
        // U0 of the first chunk; the first chunk's operands, N of the second, v of the second and third
        // (the barriers are passed by every wave whether or not the sequence has chunks)
        if (jbeg < jend) {
            load_n(opsB, jbeg);
            load_v(opsB.vraw, jbeg);
            stage_v(opsB.vraw, vslot0 + rb);
        } else if (lane == 0) {
            sMx[vslot0 + rb] = 0.f;
        }
        lds_barrier();
        first_range();
        if (jbeg < jend) {
            form_u0(opsB.fN, (int)(jbeg & 1), e);
            const char* rec = record(jbeg);
            load_w(opsA, rec);
            load_kb(opsA.fKB, opsA.gC, rec);
            load_n(opsA, next_chunk(jbeg));
            load_v(opsA.vraw, next_chunk(jbeg));
            load_v(opsB.vraw, next_chunk(next_chunk(jbeg)));
        }
        lds_barrier();
        // two chunks per iteration, so that the operand sets alternate without copies
        int64_t jc = jbeg;
        for (; jc + 1 < jend; jc += 2) {
            step(opsA, opsB, jc);
            step(opsB, opsA, jc + 1);
        }
        if (jc < jend) step(opsA, opsB, jc);
    } else if (w < 8) {
        // ======================= output waves: state tiles; O = Qh S (phase 2) + P U0 (next phase 1)
        using Ops = OutOps16<DK>;
        const uint32_t rs_o = (uint32_t)H * (uint32_t)Dv;
        float* __restrict__ o_l = o + (int64_t)h * Dv + col0 + (lane & 7) * 4;

        auto load_q = [&](Ops& d, const char* rec) {
            if constexpr (!SO) {
#pragma unroll
                for (int s = 0; s < KS; ++s) d.fQ[s] = gld_h8(rec + R::QH + (rb * KS + s) * kPl, lane);
            }
        };
        auto load_p = [&](Ops& d, const char* rec) {
            if constexpr (!SO) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const char* g = rec + R::PM + pair_of(rb, min(kb, nk - 1)) * 2 * kPl;
                    d.fP[kb][0] = gld_h8(g, lane);
                    d.fP[kb][1] = gld_h8(g + kPl, lane);
                }
            }
        };
        // O += P U0 of the chunk whose P fragments are given (U0^T buffer buf), then o rows to HBM
        f32x4_t accO[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        float4 ost[2];  // this lane's two o pieces, stored after the step's loads
        auto finish_o = [&](const f16x8_t (&fP)[2][2], int buf) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb >= nk) continue;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const _Float16* u0 = sU0 + ((buf * 2) * kS + 16 * nb + m) * L::TST + 32 * kb + 8 * cg;
                    const f16x8_t uh = lds_h8(u0), ul = lds_h8(u0 + kS * L::TST);
                    accO[nb] = mma16(accO[nb], fP[kb][0], uh);
                    accO[nb] = mma16(accO[nb], fP[kb][0], ul);
                    accO[nb] = mma16(accO[nb], fP[kb][1], uh);
                }
            }
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) sO[(16 * rb + 4 * cg + jj) * (kS + 4) + 16 * nb + m] = accO[nb][jj];
#pragma unroll
            for (int half = 0; half < 2; ++half)  // this wave's own rows: no barrier needed
                ost[half] = *reinterpret_cast<const float4*>(&sO[(16 * rb + 8 * half + (lane >> 3)) * (kS + 4) +
                                                                   (lane & 7) * 4]);
        };
        // o rows of the chunk with range exponent eo, back in the units of the inputs
        auto store_o = [&](int64_t tc, int ntc, int eo) {
            const float sc = pow2i(eo);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int rr = 16 * rb + 8 * half + (lane >> 3);
                if (rr < ntc)  // o is not read again by this call: streamed past the caches
                    __builtin_nontemporal_store(
                        f32x4_t{sc * ost[half].x, sc * ost[half].y, sc * ost[half].z, sc * ost[half].w},
                        reinterpret_cast<f32x4_t*>(o_l + (tc + rr) * (int64_t)rs_o));
            }
        };
        int eprev = 0;  // range exponent of the previous chunk
        auto step = [&](Ops& cur, Ops& nxt, int64_t jc) {
            const int64_t jn = next_chunk(jc);
            const char* recn = record(jn);
            const int b = (int)(jc & 1);

            // ---- phase 1:  O of the previous chunk (its P U0 part) to HBM, stored after the loads
            // (memory requests complete in order: a wait for a load made after a store waits for the store)
            if constexpr (!SO) {
                if (jc > jbeg) finish_o(nxt.fP, b ^ 1);
                load_p(nxt, recn);  // after the products that read the previous chunk's copy
                if (jc > jbeg) store_o(chunk_start(jc - 1), kC, eprev);
            }
            lds_barrier();  // (1)

            // ---- phase 2:  state tiles;  Qh S of this chunk
            const int en = next_range(jc);
            update_state(cur.fKB, cur.gC, b ^ 1, en, jc);
            load_kb(nxt.fKB, nxt.gC, recn);
            if constexpr (!SO) {
                accO[0] = accO[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) accO[nb] = mma16(accO[nb], cur.fQ[s], s_frag(b, s, nb));
                load_q(nxt, recn);
            }
            eprev = e;
            e = en;
            lds_barrier();  // (2)
        };
        Ops opsA, opsB;
        if (jbeg < jend) {
            const char* rec = record(jbeg);
            load_q(opsA, rec);
            load_p(opsA, rec);
            load_kb(opsA.fKB, opsA.gC, rec);
        }
        lds_barrier();  // (the state waves' V of the first chunk)
        first_range();
        lds_barrier();  // (their U0 of the first chunk)
        int64_t jc = jbeg;
        for (; jc + 1 < jend; jc += 2) {
            step(opsA, opsB, jc);
            step(opsB, opsA, jc + 1);
        }
        if (jc < jend) step(opsA, opsB, jc);
        // the last chunk's P U0 (its P fragments are in the set of its parity)
        if constexpr (!SO) {
            if (jbeg < jend) {
                const int64_t jl = jend - 1;
                finish_o(((jl - jbeg) & 1) ? opsB.fP : opsA.fP, (int)(jl & 1));
                store_o(chunk_start(jl), chunk_len(jl), eprev);
            }
        }
    }

    else {
        // ======================= prefetch wave: at the start of each step, this slice's quarter of the
        // 128-byte lines of the next chunk's record into L2, ahead of the other waves' loads of it, which
        // are spread over the step.  One chunk ahead and no further: the four slices of a sequence-head
        // share each record through L2, and a longer distance makes the lines in flight on an XCD
        // outgrow its L2, so that records are fetched from HBM more than once.  Its loads are consumed
        // two steps after they are made: memory requests complete in order, and the computing waves,
        // which wait for their own loads every step, would otherwise wait for these.
        constexpr int kLines = (int)((R::BYTES + 127) / 128);
        uint32_t sink = 0;
        auto touch = [&](int64_t jx, uint32_t (&r)[3]) {
            const char* rec = record(jx);
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int line = (i * 64 + lane) * 4 + (sl & 3);
                r[i] = line < kLines ? *reinterpret_cast<const uint32_t*>(rec + line * 128) : 0u;
            }
        };
        uint32_t rA[3] = {0u, 0u, 0u}, rB[3] = {0u, 0u, 0u};
        auto pstep = [&](uint32_t (&r)[3], int64_t jc) {
            sink |= r[0] | r[1] | r[2];
            touch(min<int64_t>(jc + 1, jend - 1), r);
            lds_barrier();  // (1)
            lds_barrier();  // (2)
        };
        lds_barrier();
        lds_barrier();
        int64_t jc = jbeg;
        for (; jc + 1 < jend; jc += 2) {
            pstep(rA, jc);
            pstep(rB, jc + 1);
        }
        if (jc < jend) pstep(rA, jc);
        sink |= rA[0] | rA[1] | rA[2] | rB[0] | rB[1] | rB[2];
        if (Dv == 7) sO[0] = (float)sink;  // keeps the loads (Dv is 64 or 128)
    }

    if (sdst && !prefetcher) {
        const float sc = pow2i(e);
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                sdst[(16 * cbw + 4 * cg + jj) * ld_dst + col_dst + 16 * nbt(i) + m] = sc * accS[i][jj];  // 32-bit
                // offsets from the uniform base: a 64-bit address kept across the chunk loop spilled
    }
}

// ============================================================================ host side

int64_t chunk16_record_bytes(int Dk) { return Dk == 128 ? Rec16<128>::BYTES : Rec16<64>::BYTES; }

static int64_t slots16(const ChunkArgs& a) {
    if (a.cu_seqlens) return a.total / kC + a.N;
    return a.N * ((a.T_fixed + kC - 1) / kC);
}
static int64_t records16_bytes(const ChunkArgs& a) { return slots16(a) * a.H * chunk16_record_bytes(a.Dk); }
static int64_t segment16_bytes(const ChunkArgs& a, int P) {
    if (P < 2) return 0;
    return a.N * a.H * (int64_t)a.Dk * 4 * ((P - 1) * (int64_t)(a.Dv + a.Dk) + P * (int64_t)a.Dv);
}
static int64_t order16_bytes(const ChunkArgs& a) { return a.cu_seqlens ? ((a.N * 4 + 255) / 256) * 256 : 0; }

// T-windows of long split calls.  A split-T call whose records would exceed the budget runs as
// windows of equal length (at most the budget of records each), each a complete split-T call over its
// tokens with the state carried from window to window in fp32 (s0 of the call, then a carry area or
// s_final, read by the window's fold and written by its last segment), so that the workspace holds the
// records of one window (the million-token call: 9.7 GB of records in one piece, 2.4 GB per window).
// KDA_SPLIT_WINDOW_BYTES (bytes) overrides the budget, for tests of the windowed path at small sizes.
static int64_t split_window_budget() {
    const char* e = getenv("KDA_SPLIT_WINDOW_BYTES");
    if (e && *e) {
        const long long v = atoll(e);
        if (v > 0) return (int64_t)v;
    }
    return int64_t(3) << 30;
}
static int64_t round256_16(int64_t x) { return (x + 255) / 256 * 256; }
// chunks per window, or 0 when the call runs in one piece
static int64_t split_window_chunks16(const ChunkArgs& a) {
    if (a.cu_seqlens || a.T_fixed <= 0 || chunk_segments(a) < 2) return 0;
    const int64_t nch = (a.T_fixed + kC - 1) / kC;
    const int64_t per_chunk = a.N * a.H * chunk16_record_bytes(a.Dk);
    const int64_t wmax = split_window_budget() / per_chunk;
    if (nch <= wmax) return 0;
    const int64_t nwin = (nch + std::max<int64_t>(wmax, 1) - 1) / std::max<int64_t>(wmax, 1);
    return (nch + nwin - 1) / nwin;  // <= wmax (at least one chunk)
}
// the window of W chunks starting at token t0 of every sequence
static ChunkArgs window16(const ChunkArgs& a, int64_t t0, int64_t W) {
    ChunkArgs w = a;
    w.T_fixed = std::min<int64_t>(W * kC, a.T_fixed - t0);
    w.T_stride = a.T_stride > 0 ? a.T_stride : a.T_fixed;
    const int64_t tk = t0 * a.H;  // token offset times heads
    const int64_t g_es = a.pro.g_bf16 ? 2 : 4, b_es = a.pro.b_bf16 ? 2 : 4;
    w.q = static_cast<const char*>(a.q) + tk * a.Dk * 2;
    w.k = static_cast<const char*>(a.k) + tk * a.Dk * 2;
    w.v = static_cast<const char*>(a.v) + tk * a.Dv * 2;
    w.g = static_cast<const char*>(a.g) + tk * a.Dk * g_es;
    w.beta = static_cast<const char*>(a.beta) + tk * b_es;
    w.o = a.o + tk * a.Dv;
    return w;
}
static int64_t window_state_bytes16(const ChunkArgs& a) { return round256_16(a.N * a.H * (int64_t)a.Dk * a.Dv * 4); }

int64_t chunk16_workspace_bytes(const ChunkArgs& a) {
    const int64_t W = split_window_chunks16(a);
    if (W > 0) {
        const ChunkArgs w = window16(a, 0, W);
        return window_state_bytes16(a) + records16_bytes(w) + segment16_bytes(w, chunk_segments(w));
    }
    return records16_bytes(a) + segment16_bytes(a, chunk_segments(a)) + order16_bytes(a);
}

static int64_t grid16(int64_t items, int slices) { return ((items + 7) / 8) * 8 * slices; }

template <int DK>
static hipError_t launch16(const ChunkArgs& a, void* ws, hipStream_t st, bool allow_split) {
    if (allow_split) {
        const int64_t W = split_window_chunks16(a);
        if (W > 0) {  // windows, each a split call of its own
            float* carry = a.s_final ? a.s_final : static_cast<float*>(ws);
            char* wws = static_cast<char*>(ws) + window_state_bytes16(a);
            for (int64_t t0 = 0; t0 < a.T_fixed; t0 += W * kC) {
                ChunkArgs w = window16(a, t0, W);
                w.s0 = t0 == 0 ? a.s0 : carry;
                w.s_final = carry;
                const hipError_t e = launch16<DK>(w, wws, st, true);
                if (e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }
    const int64_t T_stride = a.T_stride > 0 ? a.T_stride : a.T_fixed;
    const int64_t prep_grid = slots16(a) * a.H;
    char* w = static_cast<char*>(ws);
    if (prep_grid > 0 && any_prologue(a.pro))
        hipLaunchKernelGGL((prep16_kernel<DK, true>), dim3((unsigned)prep_grid), dim3(256), 0, st, a.q, a.k, a.g,
                           a.beta, a.cu_seqlens, a.T_fixed, T_stride, a.total, a.N, a.H, a.pro, w);
    else if (prep_grid > 0)
        hipLaunchKernelGGL((prep16_kernel<DK, false>), dim3((unsigned)prep_grid), dim3(256), 0, st, a.q, a.k, a.g,
                           a.beta, a.cu_seqlens, a.T_fixed, T_stride, a.total, a.N, a.H, a.pro, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int P = allow_split ? chunk_segments(a) : 1;
    const int NV = a.Dv / kS;
    if (P < 2) {
        ChainMode cm{0, 1, 0, nullptr, nullptr};
        if (a.cu_seqlens && a.N > 0) {
            int32_t* order = reinterpret_cast<int32_t*>(w + records16_bytes(a));
            if ((e = launch_seq_order(a.cu_seqlens, a.N, a.total, order, st)) != hipSuccess) return e;
            cm.order = order;
        }
        hipLaunchKernelGGL((chain16_kernel<DK, false>), dim3((unsigned)grid16(a.N * a.H, NV)), dim3(kThreads), 0, st,
                           a.v, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, T_stride, a.total, a.N, a.H, a.Dv, cm,
                           static_cast<const char*>(ws));
        return hipGetLastError();
    }
    // split-T: segment maps, fold, outputs
    const int64_t nch = (a.T_fixed + kC - 1) / kC;
    const int64_t Lc = (nch + P - 1) / P;
    float* sx = reinterpret_cast<float*>(w + records16_bytes(a));
    float* sfold = sx + a.N * a.H * (int64_t)(P - 1) * a.Dk * (a.Dv + a.Dk);
    const ChainMode c1{1, P, Lc, sx, nullptr};
    hipLaunchKernelGGL((chain16_kernel<DK, true>), dim3((unsigned)grid16(a.N * a.H * (P - 1), NV + DK / kS)),
                       dim3(kThreadsSO), 0, st, a.v, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, T_stride, a.total,
                       a.N, a.H, a.Dv, c1, static_cast<const char*>(ws));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_fold(DK, a.s0, sx, sfold, a.N * a.H, a.H, a.Dv, P, st)) != hipSuccess) return e;
    const ChainMode c2{2, P, Lc, nullptr, sfold};
    hipLaunchKernelGGL((chain16_kernel<DK, false>), dim3((unsigned)grid16(a.N * a.H * P, NV)), dim3(kThreads), 0, st,
                       a.v, a.s0, a.o, a.s_final, a.cu_seqlens, a.T_fixed, T_stride, a.total, a.N, a.H, a.Dv, c2,
                       static_cast<const char*>(ws));
    return hipGetLastError();
}

hipError_t launch_chunk_fwd16(const ChunkArgs& a, void* ws, hipStream_t st, bool allow_split) {
    return a.Dk == 128 ? launch16<128>(a, ws, st, allow_split) : launch16<64>(a, ws, st, allow_split);
}

}  // namespace kda
