// One decoding step of the gated delta rule for gfx950: a single token per
// (sequence, head) against a state S that lives in HBM.
//
// Per head ("Kimi K3 Open Model Surpasses Closed GPT and Anthropic Systems on
// Independent Benchmarks", worldcybernews, second paragraph: the state replaces
// the key/value cache and is updated with the delta rule; read as
// S' = (I - b k k^T) Diag(a) S + b k v^T, o = S'^T q with a = exp(clamp(g,-5,0))):
//     w_j  = sum_i a_i k_i S_ij          (prediction of v from the decayed state)
//     u_j  = b (v_j - w_j)
//     S'_ij = a_i S_ij + k_i u_j
//     o_j  = sum_i q_i S'_ij
// The step is a single streaming pass over S: each element is read once and
// written once with 128-bit accesses, and both column reductions over i stay on
// chip.  A workgroup of 256 threads owns one (sequence, head): thread t covers
// four adjacent columns (one float4) of every (256/(Dv/4))-th row.
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <int DK, int DV, bool F32, bool PRO>
__global__ __launch_bounds__(256) void decode_kernel(const void* __restrict__ qv, const void* __restrict__ kv,
                                                     const void* __restrict__ vv, const void* __restrict__ gv,
                                                     const void* __restrict__ bv, const float* s_in,
                                                     float* s_out, float* __restrict__ o, Prologue pro) {
    using In = typename std::conditional<F32, float, uint16_t>::type;
    // input prologue; PRO = false compiles the plain form (fp32 log alpha and beta, q and k as given)
    const Prologue pf{PRO && pro.g_bf16, PRO && pro.g_logit, PRO && pro.b_bf16, PRO && pro.b_logit,
                      PRO && pro.l2norm};
    constexpr int C4 = DV / 4;     // threads across the columns
    constexpr int RG = 256 / C4;   // row groups
    constexpr int RPT = DK / RG;   // rows per thread
    static_assert(RPT * RG == DK, "row split");

    __shared__ float sk[DK], sa[DK], sq[DK], su[DV], snk[2], snq[2];
    __shared__ float4 sred[RG][C4];

    const In* __restrict__ q = static_cast<const In*>(qv);
    const In* __restrict__ k = static_cast<const In*>(kv);
    const In* __restrict__ v = static_cast<const In*>(vv);
    const int tid = threadIdx.x, c4 = tid % C4, rg = tid / C4;
    const int64_t bh = blockIdx.x;

    // Load order: the token vectors (k, q, g, v, beta; small), then the whole state slice; memory
    // returns in order, so the vectors are waited for without waiting for the state.
    // (every thread loads, at wrapped indices, so that no branch separates these loads from the
    // state loads; only threads tid < DK / tid < C4 use them)
    const int ti = tid % DK, tv = tid % C4;
    const In kr = k[bh * DK + ti], qr = q[bh * DK + ti];
    const float gr = load1_gate(gv, bh * DK + ti, pf.g_bf16), braw = load1_gate(bv, bh, pf.b_bf16);
    In vr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) vr[j] = v[bh * DV + 4 * tv + j];
    __builtin_amdgcn_sched_barrier(0);  // keep the vector loads ahead of the state loads
    const f32x4_t* S = reinterpret_cast<const f32x4_t*>(s_in + bh * (int64_t)DK * DV);
    f32x4_t* So = reinterpret_cast<f32x4_t*>(s_out + bh * (int64_t)DK * DV);
    f32x4_t st[RPT];
#pragma unroll
    for (int mm = 0; mm < RPT; ++mm) st[mm] = __builtin_nontemporal_load(&S[(rg + RG * mm) * C4 + c4]);
    auto tof = [](In x) -> float {
        if constexpr (F32) return x;
        else return bf16_bits_to_float(x);
    };
    // every thread writes (threads beyond DK repeat the values of thread tid % DK): no branch for the
    // compiler to sink the vector loads into
    sk[ti] = tof(kr);
    sq[ti] = tof(qr);
    sa[ti] = pf.g_logit ? __builtin_amdgcn_exp2f(gate_log2(gr, true)) : __expf(fminf(fmaxf(gr, -5.f), 0.f));
    const float b = beta_value(braw, pf.b_logit);
    if (pf.l2norm) {  // squared norms of k and q: waves 0 (and 1) hold every index once
        float k2 = tof(kr) * tof(kr), q2 = tof(qr) * tof(qr);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            k2 += __shfl_xor(k2, off);
            q2 += __shfl_xor(q2, off);
        }
        if ((tid & 63) == 0 && tid < DK) {
            snk[tid >> 6] = k2;
            snq[tid >> 6] = q2;
        }
    }
    __syncthreads();
    float rk = 1.f, rq = 1.f;  // 1/||k||, 1/||q|| when both are scaled to unit length
    if (pf.l2norm) {
        const float k2 = DK == 128 ? snk[0] + snk[1] : snk[0];
        const float q2 = DK == 128 ? snq[0] + snq[1] : snq[0];
        rk = k2 > 0.f ? __builtin_amdgcn_rsqf(k2) : 0.f;
        rq = q2 > 0.f ? __builtin_amdgcn_rsqf(q2) : 0.f;
    }

    float4 wp = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int mm = 0; mm < RPT; ++mm) {
        const int i = rg + RG * mm;
        const float ak = sa[i] * (sk[i] * rk);
        wp.x = fmaf(ak, st[mm][0], wp.x);
        wp.y = fmaf(ak, st[mm][1], wp.y);
        wp.z = fmaf(ak, st[mm][2], wp.z);
        wp.w = fmaf(ak, st[mm][3], wp.w);
    }
    sred[rg][c4] = wp;
    __syncthreads();
    if (tid < C4) {
        float4 acc = sred[0][tid];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            const float4 x = sred[r][tid];
            acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
        }
        su[4 * tid + 0] = b * (tof(vr[0]) - acc.x);
        su[4 * tid + 1] = b * (tof(vr[1]) - acc.y);
        su[4 * tid + 2] = b * (tof(vr[2]) - acc.z);
        su[4 * tid + 3] = b * (tof(vr[3]) - acc.w);
    }
    __syncthreads();
    const float4 u = make_float4(su[4 * c4], su[4 * c4 + 1], su[4 * c4 + 2], su[4 * c4 + 3]);
    float4 op = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int mm = 0; mm < RPT; ++mm) {
        const int i = rg + RG * mm;
        const float a = sa[i], kk = sk[i] * rk, qq = sq[i] * rq;
        f32x4_t x;
        x[0] = fmaf(a, st[mm][0], kk * u.x);
        x[1] = fmaf(a, st[mm][1], kk * u.y);
        x[2] = fmaf(a, st[mm][2], kk * u.z);
        x[3] = fmaf(a, st[mm][3], kk * u.w);
        __builtin_nontemporal_store(x, &So[i * C4 + c4]);
        op.x = fmaf(qq, x[0], op.x);
        op.y = fmaf(qq, x[1], op.y);
        op.z = fmaf(qq, x[2], op.z);
        op.w = fmaf(qq, x[3], op.w);
    }
    sred[rg][c4] = op;
    __syncthreads();
    if (tid < C4) {
        float4 acc = sred[0][tid];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            const float4 x = sred[r][tid];
            acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
        }
        reinterpret_cast<float4*>(o + bh * DV)[tid] = acc;
    }
}

template <int DK, int DV>
static hipError_t launch_dv(const DecodeArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)(a.B * a.H));
    const bool pro = any_prologue(a.pro);
    if (a.f32 && pro)
        hipLaunchKernelGGL((decode_kernel<DK, DV, true, true>), grid, dim3(256), 0, st, a.q, a.k, a.v, a.g, a.beta,
                           a.s_in, a.s_out, a.o, a.pro);
    else if (a.f32)
        hipLaunchKernelGGL((decode_kernel<DK, DV, true, false>), grid, dim3(256), 0, st, a.q, a.k, a.v, a.g, a.beta,
                           a.s_in, a.s_out, a.o, a.pro);
    else if (pro)
        hipLaunchKernelGGL((decode_kernel<DK, DV, false, true>), grid, dim3(256), 0, st, a.q, a.k, a.v, a.g, a.beta,
                           a.s_in, a.s_out, a.o, a.pro);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, false, false>), grid, dim3(256), 0, st, a.q, a.k, a.v, a.g, a.beta,
                           a.s_in, a.s_out, a.o, a.pro);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.Dk == 128) return a.Dv == 128 ? launch_dv<128, 128>(a, st) : launch_dv<128, 64>(a, st);
    return a.Dv == 128 ? launch_dv<64, 128>(a, st) : launch_dv<64, 64>(a, st);
}

}  // namespace kda
