// Calibration kernels: the achievable HBM copy rate and matrix-core rates of the GPU the library runs
// on, measured by the same process that times the method's kernels.  They compute nothing of the
// method; they bound what its kernels can reach.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

#include "kda_calib.h"
#include "kda_device.h"

namespace {

// Plain streaming copy: each 256-thread block moves one tile of 4 x 256 x 16 bytes, all four
// non-temporal 16-byte loads issued before the stores.  (On MI355X this form measured 6.2 TB/s for a
// 1 GiB copy; a grid-stride loop of single 16-byte copies 5.1 TB/s, eight per thread 4.2 TB/s.)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(256) void copy_kernel(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                   int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * (kCopyUnroll * 256) + threadIdx.x;
    u32x4_t x[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + u * 256;
        if (i < n16) x[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const int64_t i = base + u * 256;
        if (i < n16) __builtin_nontemporal_store(x[u], dst + i);
    }
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Four independent accumulators per wave, `iters` rounds of one MFMA on each; the accumulators are
// summed into out[] so that nothing is dead code.  Operands vary with the lane so that the products
// are not constant-folded.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int64_t iters) {
    const int lane = threadIdx.x & 63;
    bf16x8_t a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1.0f + 0.001f * (float)(lane + j));
        b[j] = (__bf16)(0.5f - 0.001f * (float)(lane - j));
    }
    float sum = 0.f;
    if constexpr (KIND == 0) {  // v_mfma_f32_16x16x32_bf16
        f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
        for (int64_t i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += c0[j] + c1[j] + c2[j] + c3[j];
    } else {  // v_mfma_f32_32x32x16_bf16
        f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
        for (int64_t i = 0; i < iters; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) sum += c0[j] + c1[j] + c2[j] + c3[j];
    }
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

}  // namespace

extern "C" {

int kda_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return 2;
    const int64_t n16 = (int64_t)(bytes / 16);
    if (n16 == 0) return 0;
    const int64_t blocks = (n16 + kCopyUnroll * 256 - 1) / (kCopyUnroll * 256);
    if (blocks > 0x7fffffff) return 2;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

int kda_calib_mfma(float* out, int blocks, int64_t iters, int kind, void* stream) {
    if (!out || blocks < 1 || iters < 1 || (kind != 0 && kind != 1)) return 2;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (kind == 0)
        hipLaunchKernelGGL(mfma_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, out, iters);
    else
        hipLaunchKernelGGL(mfma_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
