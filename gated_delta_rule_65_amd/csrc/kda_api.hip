// C ABI of the library (declared in include/kda.h): host-side validation,
// error reporting and dispatch to the gfx950 kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kda.h"
#include "kda_launch.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kda_status ok() {
    g_last_error.clear();
    return KDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

kda_status check_head_dims(int H, int Dk, int Dv) {
    if (H < 1 || H > 65536) return fail(KDA_ERR_BAD_SHAPE, "H must be in [1, 65536] (got %d)", H);
    if (Dk != 64 && Dk != 128) return fail(KDA_ERR_BAD_SHAPE, "Dk must be 64 or 128 (got %d)", Dk);
    if (Dv != 64 && Dv != 128) return fail(KDA_ERR_BAD_SHAPE, "Dv must be 64 or 128 (got %d)", Dv);
    return KDA_OK;
}

kda_status check_dtype(kda_dtype dt) {
    if (dt != KDA_F32 && dt != KDA_BF16) return fail(KDA_ERR_BAD_DTYPE, "dtype must be KDA_F32 or KDA_BF16");
    return KDA_OK;
}

struct Ptr {
    const void* p;
    const char* name;
    bool required;
};

kda_status check_ptrs(std::initializer_list<Ptr> ptrs) {
    for (const Ptr& x : ptrs) {
        if (x.required && !x.p) return fail(KDA_ERR_NULL_ARG, "%s is NULL", x.name);
        if (x.p && !aligned16(x.p)) return fail(KDA_ERR_MISALIGNED, "%s is not 16-byte aligned", x.name);
    }
    return KDA_OK;
}

kda_status read_prologue(const kda_prologue* p, kda::Prologue& out) {
    out = kda::Prologue{false, false, false, false, false};
    if (!p) return KDA_OK;
    if (p->g_dtype != KDA_F32 && p->g_dtype != KDA_BF16)
        return fail(KDA_ERR_BAD_DTYPE, "prologue g_dtype must be KDA_F32 or KDA_BF16");
    if (p->beta_dtype != KDA_F32 && p->beta_dtype != KDA_BF16)
        return fail(KDA_ERR_BAD_DTYPE, "prologue beta_dtype must be KDA_F32 or KDA_BF16");
    out.g_bf16 = p->g_dtype == KDA_BF16;
    out.g_logit = p->g_logit != 0;
    out.b_bf16 = p->beta_dtype == KDA_BF16;
    out.b_logit = p->beta_logit != 0;
    out.l2norm = p->qk_l2norm != 0;
    return KDA_OK;
}

kda_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

kda_status run_chunked(const kda::ChunkArgs& a, void* workspace, size_t workspace_bytes, hipStream_t st,
                       const char* what) {
    const int64_t grid = kda::chunk_grid_size(a.N, a.H, a.Dv);
    if (grid > 0x7fffffff) return fail(KDA_ERR_BAD_SHAPE, "%s: %lld sequence-heads exceed the grid limit", what,
                                       (long long)(a.N * a.H));
    if (grid == 0) return ok();
    // without tokens there is nothing to prepare (the workspace size queries return 0 then): the
    // fused kernel passes s0 (or zeros) through to s_final
    if (!workspace || a.total == 0) return launched(kda::launch_chunk_fwd(a, st), what);
    if (kda::chunk_slots(a) * a.H > 0x7fffffffLL)
        return fail(KDA_ERR_BAD_SHAPE, "%s: %lld chunk-heads exceed the grid limit", what,
                    (long long)(kda::chunk_slots(a) * a.H));
    const int64_t need = kda::chunk_workspace_bytes(a);
    if ((uint64_t)need > (uint64_t)workspace_bytes)
        return fail(KDA_ERR_BAD_SHAPE, "%s: workspace holds %llu bytes, %lld needed", what,
                    (unsigned long long)workspace_bytes, (long long)need);
    return launched(kda::launch_chunk_fwd_two_pass(a, workspace, st), what);
}

// ---------------------------------------------------------------------------- fixed scratch
// Device memory of kda_chunk_fwd_noalloc, for callers that cannot allocate: the per-window records
// of the two-kernel path (and the carried state when s_final is NULL).  Every GPU that runs the
// library holds its own copy for the life of the process.  Its address on a device comes from
// hipGetSymbolAddress, looked up once per device with that device current; host code uses only that
// address, never the array's name (which on the host is a stand-in, not a device address).
constexpr int64_t kScratchBytes = int64_t(128) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kda_status scratch_of_current_device(void** out, const char* what) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: hipGetDevice failed: %s", what, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_HIP, "%s: device %d out of range", what, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(KDA_ERR_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", what, dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                 const float* s0, float* o, float* s_final, int64_t B, int64_t T, int H, int Dk,
                                 int Dv, int chunk, kda_dtype dtype, const kda_prologue* prologue, void* stream) {
    const char* what = "kda_chunk_fwd_noalloc";
    kda_status st;
    kda::Prologue pro;
    if ((st = check_dtype(dtype)) != KDA_OK) return st;
    if ((st = read_prologue(prologue, pro)) != KDA_OK) return st;
    if ((st = check_head_dims(H, Dk, Dv)) != KDA_OK) return st;
    if (chunk != 64) return fail(KDA_ERR_BAD_SHAPE, "chunk must be 64 (got %d)", chunk);
    if (B < 0 || T < 0) return fail(KDA_ERR_BAD_SHAPE, "B and T must be >= 0");
    if (T > 0 && B > INT64_MAX / T) return fail(KDA_ERR_BAD_SHAPE, "B*T overflows");
    const bool tokens = B > 0 && T > 0;
    if ((st = check_ptrs({{q, "q", tokens}, {k, "k", tokens}, {v, "v", tokens}, {g, "g", tokens},
                          {beta, "beta", tokens}, {o, "o", tokens}, {s0, "s0", false},
                          {s_final, "s_final", false}})) != KDA_OK)
        return st;
    if (B == 0 || (!tokens && !s_final)) return ok();
    kda::ChunkArgs a{q, k, v, g, beta, s0, o, s_final, nullptr, T, B * T, B, H, Dk, Dv, dtype == KDA_F32, pro};
    const int64_t grid = kda::chunk_grid_size(a.N, a.H, a.Dv);
    if (grid > 0x7fffffff) return fail(KDA_ERR_BAD_SHAPE, "%s: %lld sequence-heads exceed the grid limit", what,
                                       (long long)(a.N * a.H));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (!tokens) return launched(kda::launch_chunk_fwd(a, hs), what);  // s0 (or zeros) to s_final, no scratch
    if (kda::chunk_window_chunks(a, kScratchBytes) < 1)
        return fail(KDA_ERR_BAD_SHAPE,
                    "%s: B*H = %lld sequence-heads need %lld bytes of scratch for one 64-token window; the fixed "
                    "scratch holds %lld",
                    what, (long long)(a.N * a.H),
                    (long long)(kda::chunk_window_state_bytes(a) + kda::chunk_workspace_bytes(
                        kda::ChunkArgs{q, k, v, g, beta, s0, o, s_final, nullptr, 64, B * 64, B, H, Dk, Dv,
                                       dtype == KDA_F32, pro})),
                    (long long)kScratchBytes);
    void* base = nullptr;
    if ((st = scratch_of_current_device(&base, what)) != KDA_OK) return st;
    return launched(kda::launch_chunk_fwd_windows(a, static_cast<char*>(base), kScratchBytes, hs), what);
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* s0, float* o, float* s_final, int64_t B, int64_t T, int H, int Dk, int Dv,
                         int chunk, kda_dtype dtype, const kda_prologue* prologue, void* workspace,
                         size_t workspace_bytes, void* stream) {
    kda_status st;
    kda::Prologue pro;
    if ((st = check_dtype(dtype)) != KDA_OK) return st;
    if ((st = read_prologue(prologue, pro)) != KDA_OK) return st;
    if ((st = check_head_dims(H, Dk, Dv)) != KDA_OK) return st;
    if (chunk != 64) return fail(KDA_ERR_BAD_SHAPE, "chunk must be 64 (got %d)", chunk);
    if (B < 0 || T < 0) return fail(KDA_ERR_BAD_SHAPE, "B and T must be >= 0");
    if (T > 0 && B > INT64_MAX / T) return fail(KDA_ERR_BAD_SHAPE, "B*T overflows");
    const bool tokens = B > 0 && T > 0;
    if ((st = check_ptrs({{q, "q", tokens}, {k, "k", tokens}, {v, "v", tokens}, {g, "g", tokens},
                          {beta, "beta", tokens}, {o, "o", tokens}, {s0, "s0", false},
                          {s_final, "s_final", false}, {workspace, "workspace", false}})) != KDA_OK)
        return st;
    if (B == 0 || (!tokens && !s_final)) return ok();
    kda::ChunkArgs a{q, k, v, g, beta, s0, o, s_final, nullptr, T, B * T, B, H, Dk, Dv, dtype == KDA_F32, pro};
    return run_chunked(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream), "kda_chunk_fwd");
}

kda_status kda_varlen_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const int32_t* cu_seqlens, int64_t N, int64_t total, const float* s0, float* o,
                          float* s_final, int H, int Dk, int Dv, int chunk, kda_dtype dtype,
                          const kda_prologue* prologue, void* workspace, size_t workspace_bytes, void* stream) {
    kda_status st;
    kda::Prologue pro;
    if ((st = check_dtype(dtype)) != KDA_OK) return st;
    if ((st = read_prologue(prologue, pro)) != KDA_OK) return st;
    if ((st = check_head_dims(H, Dk, Dv)) != KDA_OK) return st;
    if (chunk != 64) return fail(KDA_ERR_BAD_SHAPE, "chunk must be 64 (got %d)", chunk);
    if (N < 0 || total < 0) return fail(KDA_ERR_BAD_SHAPE, "N and total must be >= 0");
    if (total > 0x7fffffffLL) return fail(KDA_ERR_BAD_SHAPE, "total exceeds the int32 range of cu_seqlens");
    const bool tokens = total > 0;
    if (N > 0 && !cu_seqlens) return fail(KDA_ERR_NULL_ARG, "cu_seqlens is NULL");
    if ((st = check_ptrs({{q, "q", tokens}, {k, "k", tokens}, {v, "v", tokens}, {g, "g", tokens},
                          {beta, "beta", tokens}, {o, "o", tokens}, {s0, "s0", false},
                          {s_final, "s_final", false}, {workspace, "workspace", false}})) != KDA_OK)
        return st;
    if (N == 0 || (!tokens && !s_final)) return ok();
    kda::ChunkArgs a{q, k, v, g, beta, s0, o, s_final, cu_seqlens, 0, total, N, H, Dk, Dv, dtype == KDA_F32, pro};
    return run_chunked(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream), "kda_varlen_fwd");
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                           const float* s_in, float* s_out, float* o, int64_t B, int H, int Dk, int Dv,
                           kda_dtype dtype, const kda_prologue* prologue, void* stream) {
    kda_status st;
    kda::Prologue pro;
    if ((st = check_dtype(dtype)) != KDA_OK) return st;
    if ((st = read_prologue(prologue, pro)) != KDA_OK) return st;
    if ((st = check_head_dims(H, Dk, Dv)) != KDA_OK) return st;
    if (B < 0) return fail(KDA_ERR_BAD_SHAPE, "B must be >= 0");
    if (B * H > 0x7fffffffLL) return fail(KDA_ERR_BAD_SHAPE, "B*H exceeds the grid limit");
    const bool any = B > 0;
    if ((st = check_ptrs({{q, "q", any}, {k, "k", any}, {v, "v", any}, {g, "g", any}, {beta, "beta", any},
                          {s_in, "s_in", any}, {s_out, "s_out", any}, {o, "o", any}})) != KDA_OK)
        return st;
    if (s_in != s_out && s_in && s_out) {
        const char* a0 = reinterpret_cast<const char*>(s_in);
        const char* b0 = reinterpret_cast<const char*>(s_out);
        const int64_t bytes = B * H * (int64_t)Dk * Dv * 4;
        if (a0 < b0 + bytes && b0 < a0 + bytes)
            return fail(KDA_ERR_BAD_SHAPE, "s_in and s_out overlap without being the same buffer");
    }
    if (!any) return ok();
    kda::DecodeArgs a{q, k, v, g, beta, s_in, s_out, o, B, H, Dk, Dv, dtype == KDA_F32, pro};
    return launched(kda::launch_decode(a, static_cast<hipStream_t>(stream)), "kda_decode_step");
}

static kda_status run_bwd(const kda::BwdArgs& a, void* workspace, size_t workspace_bytes, hipStream_t st,
                          const char* what) {
    if (a.N * (int64_t)a.H > 0x7fffffffLL / 4)
        return fail(KDA_ERR_BAD_SHAPE, "%s: %lld sequence-heads exceed the grid limit", what, (long long)(a.N * a.H));
    if (kda::bwd_slots(a) * a.H > 0x7fffffffLL)
        return fail(KDA_ERR_BAD_SHAPE, "%s: %lld chunk-heads exceed the grid limit", what,
                    (long long)(kda::bwd_slots(a) * a.H));
    const int64_t need = kda::bwd_workspace_bytes(a);
    if (need > 0 && !workspace) return fail(KDA_ERR_NULL_ARG, "%s: workspace is NULL (%lld bytes needed)", what,
                                            (long long)need);
    if ((uint64_t)need > (uint64_t)workspace_bytes)
        return fail(KDA_ERR_BAD_SHAPE, "%s: workspace holds %llu bytes, %lld needed", what,
                    (unsigned long long)workspace_bytes, (long long)need);
    return launched(kda::launch_bwd(a, workspace, st), what);
}

kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* s0, const float* d_o, const float* d_sfinal, float* dq, float* dk, float* dv,
                         float* dg, float* dbeta, float* ds0, int64_t B, int64_t T, int H, int Dk, int Dv, int chunk,
                         kda_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
    kda_status st;
    if ((st = check_dtype(dtype)) != KDA_OK) return st;
    if ((st = check_head_dims(H, Dk, Dv)) != KDA_OK) return st;
    if (chunk != 64) return fail(KDA_ERR_BAD_SHAPE, "chunk must be 64 (got %d)", chunk);
    if (B < 0 || T < 0) return fail(KDA_ERR_BAD_SHAPE, "B and T must be >= 0");
    if (T > 0 && B > INT64_MAX / T) return fail(KDA_ERR_BAD_SHAPE, "B*T overflows");
    const bool tokens = B > 0 && T > 0;
    if ((st = check_ptrs({{q, "q", tokens}, {k, "k", tokens}, {v, "v", tokens}, {g, "g", tokens},
                          {beta, "beta", tokens}, {d_o, "d_o", tokens}, {dq, "dq", tokens}, {dk, "dk", tokens},
                          {dv, "dv", tokens}, {dg, "dg", tokens}, {dbeta, "dbeta", tokens}, {s0, "s0", false},
                          {d_sfinal, "d_sfinal", false}, {ds0, "ds0", false}, {workspace, "workspace", false}})) !=
        KDA_OK)
        return st;
    if (B == 0 || (!tokens && !ds0)) return ok();
    kda::BwdArgs a{q, k, v, g, beta, s0, d_o, d_sfinal, dq, dk, dv, dg, dbeta, ds0, nullptr, T, B * T, B, H, Dk, Dv,
                   dtype == KDA_F32};
    return run_bwd(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream), "kda_chunk_bwd");
}

kda_status kda_varlen_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, int64_t N, int64_t total, const float* s0, const float* d_o,
                          const float* d_sfinal, float* dq, float* dk, float* dv, float* dg, float* dbeta, float* ds0,
                          int H, int Dk, int Dv, int chunk, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* stream) {
    kda_status st;
    if ((st = check_dtype(dtype)) != KDA_OK) return st;
    if ((st = check_head_dims(H, Dk, Dv)) != KDA_OK) return st;
    if (chunk != 64) return fail(KDA_ERR_BAD_SHAPE, "chunk must be 64 (got %d)", chunk);
    if (N < 0 || total < 0) return fail(KDA_ERR_BAD_SHAPE, "N and total must be >= 0");
    if (total > 0x7fffffffLL) return fail(KDA_ERR_BAD_SHAPE, "total exceeds the int32 range of cu_seqlens");
    const bool tokens = total > 0;
    if (N > 0 && !cu_seqlens) return fail(KDA_ERR_NULL_ARG, "cu_seqlens is NULL");
    if ((st = check_ptrs({{q, "q", tokens}, {k, "k", tokens}, {v, "v", tokens}, {g, "g", tokens},
                          {beta, "beta", tokens}, {d_o, "d_o", tokens}, {dq, "dq", tokens}, {dk, "dk", tokens},
                          {dv, "dv", tokens}, {dg, "dg", tokens}, {dbeta, "dbeta", tokens}, {s0, "s0", false},
                          {d_sfinal, "d_sfinal", false}, {ds0, "ds0", false}, {workspace, "workspace", false}})) !=
        KDA_OK)
        return st;
    if (N == 0 || (!tokens && !ds0)) return ok();
    kda::BwdArgs a{q, k, v, g, beta, s0, d_o, d_sfinal, dq, dk, dv, dg, dbeta, ds0, cu_seqlens, 0, total, N, H, Dk,
                   Dv, dtype == KDA_F32};
    return run_bwd(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream), "kda_varlen_bwd");
}

size_t kda_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int H, int Dk, int Dv, kda_dtype dtype) {
    if (B <= 0 || T < 0 || H < 1 || (Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    kda::BwdArgs a{};
    a.f32 = dtype == KDA_F32;
    a.T_fixed = T;
    a.N = B;
    a.total = B * T;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    return (size_t)kda::bwd_workspace_bytes(a);
}

size_t kda_varlen_bwd_workspace_bytes(int64_t N, int64_t total, int H, int Dk, int Dv, kda_dtype dtype) {
    if (N <= 0 || total < 0 || H < 1 || (Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    kda::BwdArgs a{};
    a.f32 = dtype == KDA_F32;
    static const int32_t dummy = 0;
    a.cu_seqlens = &dummy;  // only its presence matters for the size
    a.N = N;
    a.total = total;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    return (size_t)kda::bwd_workspace_bytes(a);
}

size_t kda_chunk_workspace_bytes(int64_t B, int64_t T, int H, int Dk, int Dv, kda_dtype dtype) {
    if (B <= 0 || T <= 0 || H < 1 || (Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    kda::ChunkArgs a{};
    a.f32 = dtype == KDA_F32;
    a.T_fixed = T;
    a.N = B;
    a.total = B * T;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    return (size_t)kda::chunk_workspace_bytes(a);
}

size_t kda_varlen_workspace_bytes(int64_t N, int64_t total, int H, int Dk, int Dv, kda_dtype dtype) {
    if (N <= 0 || total <= 0 || H < 1 || (Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128)) return 0;
    if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
    kda::ChunkArgs a{};
    a.f32 = dtype == KDA_F32;
    static const int32_t dummy = 0;
    a.cu_seqlens = &dummy;  // only its presence matters for the size
    a.N = N;
    a.total = total;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    return (size_t)kda::chunk_workspace_bytes(a);
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

const char* kda_version(void) { return "kda-gfx950 0.4"; }

}  // extern "C"
