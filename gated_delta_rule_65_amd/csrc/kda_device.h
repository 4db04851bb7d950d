// Device-side helpers for the gfx950 kernels: bf16 conversion, MFMA operand
// fragments with a split-bf16 or fp32 precision policy, and a 16-lane DPP scan.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Eight consecutive input elements (bf16 or fp32) as floats; p must be 16-byte aligned.
__device__ __forceinline__ void load8_as_float(const uint16_t* p, float x[8]) {
    uint4 w = *reinterpret_cast<const uint4*>(p);
    uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(u[i] << 16);
        x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8_as_float(const float* p, float x[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// ---------------------------------------------------------------------------
// Input prologue (the kda_prologue options): element type of the gate and beta
// inputs, their logit forms, and unit-length q/k.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8_gate(const void* p, int64_t idx, bool bf, float x[8]) {
    if (bf) load8_as_float(static_cast<const uint16_t*>(p) + idx, x);
    else load8_as_float(static_cast<const float*>(p) + idx, x);
}
__device__ __forceinline__ float load1_gate(const void* p, int64_t idx, bool bf) {
    return bf ? bf16_bits_to_float(static_cast<const uint16_t*>(p)[idx]) : static_cast<const float*>(p)[idx];
}

// Clamped log alpha in log2 units.  A log-alpha input x gives clamp(x, -5, 0) / ln 2.  A gate logit
// x gives log alpha = -softplus(x), evaluated as -(max(x, 0) + ln(1 + e^{-|x|})) so that neither
// exponential overflows, then the same clamp.
__device__ __forceinline__ float gate_log2(float x, bool logit) {
    constexpr float l2e = 1.4426950408889634f;
    if (!logit) return __builtin_amdgcn_fmed3f(x, -5.f, 0.f) * l2e;
    const float sp2 = fmaxf(x, 0.f) * l2e + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * l2e));
    return __builtin_amdgcn_fmed3f(-sp2, -5.f * l2e, 0.f);
}

// beta from its input: the value itself, or the logistic function 1 / (1 + e^{-x}) of a logit.
__device__ __forceinline__ float beta_value(float x, bool logit) {
    constexpr float l2e = 1.4426950408889634f;
    return logit ? __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * l2e)) : x;
}

// 1/||x|| of a vector whose squared entries are summed in `ss` over lanes l, l^16, l^32, l^48
// (every lane of the group gets the same value); 0 for an all-zero vector.
__device__ __forceinline__ float rnorm_lanes4(float ss) {
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    return ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f;
}

// ---------------------------------------------------------------------------
// MFMA operand fragments.  For v_mfma_f32_16x16x32_bf16 a lane holds eight
// consecutive reduction-index values of one row (A) or one column (B):
// lane l -> row/column l%16, reduction indices 8*(l/16) .. 8*(l/16)+7 of the
// 32-wide step; the 16x16 result gives lane l column l%16, rows 4*(l/16)..+3.
//
// Precision policies:
//   SPLIT (bf16 inputs): each operand is x = hi + lo with hi = bf16(x) and
//     lo = bf16(x - hi); a 3-pass product hi*hi + hi*lo + lo*hi keeps about
//     16 significant bits, a 1-pass product uses hi*hi only.
//   F32 (fp32 inputs): products go through v_mfma_f32_16x16x4_f32; MFMA number
//     j consumes value j of every lane, so the same eight-values-per-lane
//     fragment covers the 32-wide step in 8 instructions.
// ---------------------------------------------------------------------------
template <bool F32>
struct Frag;

template <>
struct Frag<false> {
    bf16x8_t hi, lo;
    // value as float: hi + lo (about 16 significant bits)
    __device__ __forceinline__ void get(float x[8]) const {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)hi[j] + (float)lo[j];
    }
    __device__ __forceinline__ void get_hi(float x[8]) const {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (float)hi[j];
    }
    __device__ __forceinline__ void set(const float x[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __bf16 h = (__bf16)x[j];
            hi[j] = h;
            lo[j] = (__bf16)(x[j] - (float)h);
        }
    }
    __device__ __forceinline__ void set_hi_only(const float x[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) hi[j] = (__bf16)x[j];
    }
};

template <>
struct Frag<true> {
    float v[8];
    __device__ __forceinline__ void get(float x[8]) const {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = v[j];
    }
    __device__ __forceinline__ void get_hi(float x[8]) const { get(x); }
    __device__ __forceinline__ void set(const float x[8]) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = x[j];
    }
    __device__ __forceinline__ void set_hi_only(const float x[8]) { set(x); }
};

// Stores of data that no later access of the same kernel reads: streamed past the caches, so that
// their write-back does not compete with the loads of the kernels that follow.
__device__ __forceinline__ void st_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt4(float* p, float a, float b, float c, float d) {
    __builtin_nontemporal_store(f32x4_t{a, b, c, d}, reinterpret_cast<f32x4_t*>(p));
}

// acc += A * B with the full precision of the policy.
__device__ __forceinline__ f32x4_t mma_full(f32x4_t acc, const Frag<false>& a, const Frag<false>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.lo, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b.hi, acc, 0, 0, 0);
    return acc;
}
__device__ __forceinline__ f32x4_t mma_full(f32x4_t acc, const Frag<true>& a, const Frag<true>& b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
    return acc;
}
// acc += A * B with one bf16 pass (SPLIT) or full fp32 (F32).
__device__ __forceinline__ f32x4_t mma_fast(f32x4_t acc, const Frag<false>& a, const Frag<false>& b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b.hi, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma_fast(f32x4_t acc, const Frag<true>& a, const Frag<true>& b) {
    return mma_full(acc, a, b);
}

// Eight consecutive floats from LDS (16-byte aligned).
__device__ __forceinline__ void lds_read8(const float* p, float x[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// not for its outstanding global loads (which may be prefetches still in flight).
__device__ __forceinline__ void lds_barrier() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16r .. 16r+15),
// Hillis-Steele with row_shr 1, 2, 4, 8; lanes shifted in from outside the row
// contribute 0.
// ---------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_inclusive_scan(float x) {
    x += dpp_row_shr<1>(x);
    x += dpp_row_shr<2>(x);
    x += dpp_row_shr<4>(x);
    x += dpp_row_shr<8>(x);
    return x;
}

// ---------------------------------------------------------------------------
// Matrices in LDS that feed MFMA operands.  SPLIT policy: two planes, bf16 hi
// then bf16 lo, each ROWS x STRIDE; an element is split once, when written.
// F32 policy: one fp32 plane.  Both take 4 bytes per element.  Rows are padded
// so that sixteen lanes reading 16 bytes from sixteen consecutive rows hit
// distinct LDS banks.
// ---------------------------------------------------------------------------
template <bool F32, int ROWS, int COLS>
struct LMat {
    static constexpr int STRIDE = F32 ? COLS + 4 : COLS + 8;
    static constexpr int PLANE = ROWS * STRIDE;
    static constexpr int BYTES = PLANE * 4;
};

template <bool F32, int ROWS, int COLS>
__device__ __forceinline__ Frag<F32> lds_frag(const char* base, int row, int col) {
    using M = LMat<F32, ROWS, COLS>;
    Frag<F32> f;
    if constexpr (F32) {
        const float* p = reinterpret_cast<const float*>(base) + row * M::STRIDE + col;
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
        f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    } else {
        const __bf16* p = reinterpret_cast<const __bf16*>(base) + row * M::STRIDE + col;
        f.hi = *reinterpret_cast<const bf16x8_t*>(p);
        f.lo = *reinterpret_cast<const bf16x8_t*>(p + M::PLANE);
    }
    return f;
}

template <bool F32, int ROWS, int COLS>
__device__ __forceinline__ void lds_store8(char* base, int row, int col, const float x[8]) {
    using M = LMat<F32, ROWS, COLS>;
    if constexpr (F32) {
        float* p = reinterpret_cast<float*>(base) + row * M::STRIDE + col;
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
    } else {
        bf16x8_t hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            __bf16 h = (__bf16)x[j];
            hi[j] = h;
            lo[j] = (__bf16)(x[j] - (float)h);
        }
        __bf16* p = reinterpret_cast<__bf16*>(base) + row * M::STRIDE + col;
        *reinterpret_cast<bf16x8_t*>(p) = hi;
        *reinterpret_cast<bf16x8_t*>(p + M::PLANE) = lo;
    }
}

template <bool F32, int ROWS, int COLS>
__device__ __forceinline__ void lds_store4(char* base, int row, int col, f32x4_t x) {
    using M = LMat<F32, ROWS, COLS>;
    if constexpr (F32) {
        float* p = reinterpret_cast<float*>(base) + row * M::STRIDE + col;
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    } else {
        bf16x4_t hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            __bf16 h = (__bf16)x[j];
            hi[j] = h;
            lo[j] = (__bf16)(x[j] - (float)h);
        }
        __bf16* p = reinterpret_cast<__bf16*>(base) + row * M::STRIDE + col;
        *reinterpret_cast<bf16x4_t*>(p) = hi;
        *reinterpret_cast<bf16x4_t*>(p + M::PLANE) = lo;
    }
}

template <bool F32, int ROWS, int COLS>
__device__ __forceinline__ void lds_store1(char* base, int row, int col, float x) {
    using M = LMat<F32, ROWS, COLS>;
    if constexpr (F32) {
        reinterpret_cast<float*>(base)[row * M::STRIDE + col] = x;
    } else {
        __bf16 h = (__bf16)x;
        __bf16* p = reinterpret_cast<__bf16*>(base) + row * M::STRIDE + col;
        p[0] = h;
        p[M::PLANE] = (__bf16)(x - (float)h);
    }
}

template <bool F32, int ROWS, int COLS>
__device__ __forceinline__ void lds_zero(char* base, int tid, int nthreads) {
    using M = LMat<F32, ROWS, COLS>;
    float4* p = reinterpret_cast<float4*>(base);
    for (int i = tid; i < M::BYTES / 16; i += nthreads) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Eight input elements held raw in registers between their global load and use
// (one 16-byte load for bf16, two for fp32).
template <bool F32>
struct Raw8 {
    uint4 a, b;
};
template <>
struct Raw8<false> {
    uint4 a;
};
__device__ __forceinline__ void load_raw8(const uint16_t* p, Raw8<false>& r) {
    r.a = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void load_raw8(const float* p, Raw8<true>& r) {
    r.a = *reinterpret_cast<const uint4*>(p);
    r.b = *reinterpret_cast<const uint4*>(p + 4);
}
__device__ __forceinline__ void zero_raw8(Raw8<false>& r) { r.a = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_raw8(Raw8<true>& r) { r.a = r.b = make_uint4(0, 0, 0, 0); }
template <bool F32>
__device__ __forceinline__ void raw8_to_float(const Raw8<F32>& r, float x[8]) {
    if constexpr (F32) {
        x[0] = __uint_as_float(r.a.x); x[1] = __uint_as_float(r.a.y);
        x[2] = __uint_as_float(r.a.z); x[3] = __uint_as_float(r.a.w);
        x[4] = __uint_as_float(r.b.x); x[5] = __uint_as_float(r.b.y);
        x[6] = __uint_as_float(r.b.z); x[7] = __uint_as_float(r.b.w);
    } else {
        uint32_t u[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
}
