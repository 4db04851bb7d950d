// Internal launch interface between the C ABI (kda_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// How the gate and beta inputs are read (kda_prologue of the C ABI): element type, and whether
// they hold logits (log alpha = -softplus(x), beta = sigmoid(b)); l2norm scales q and k to unit
// length per token and head.
struct Prologue {
    bool g_bf16, g_logit, b_bf16, b_logit, l2norm;
};
inline bool any_prologue(const Prologue& p) { return p.g_bf16 || p.g_logit || p.b_bf16 || p.b_logit || p.l2norm; }

struct ChunkArgs {
    const void *q, *k, *v;
    const void *g, *beta;
    const float* s0;
    float *o, *s_final;
    const int32_t* cu_seqlens;  // device offsets, or nullptr for equal-length sequences
    int64_t T_fixed;            // tokens per sequence when cu_seqlens == nullptr
    int64_t total;              // tokens in all sequences
    int64_t N;                  // sequences
    int H, Dk, Dv;
    bool f32;                   // q/k/v are float32 (else bf16)
    Prologue pro;
    int64_t T_stride = 0;       // tokens between sequence starts (equal lengths); 0 = T_fixed
};

struct DecodeArgs {
    const void *q, *k, *v;
    const void *g, *beta;
    const float* s_in;
    float *s_out, *o;
    int64_t B;
    int H, Dk, Dv;
    bool f32;
    Prologue pro;
};

int64_t chunk_grid_size(int64_t N, int H, int Dv);
hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t st);
// Two-kernel path: per-chunk preparation into a workspace, then the state chain.
int64_t chunk_slots(const ChunkArgs& a);
int64_t chunk_workspace_bytes(const ChunkArgs& a);
hipError_t launch_chunk_fwd_two_pass(const ChunkArgs& a, void* ws, hipStream_t st);
// The two-kernel path over T-windows of equal-length sequences, with the records of one window in
// a scratch buffer of fixed size (see chunk_window_chunks) and the state carried between windows
// in fp32 through s_final or, when that is NULL, a state area at the start of the scratch.
int64_t chunk_window_state_bytes(const ChunkArgs& a);
int64_t chunk_window_chunks(const ChunkArgs& a, int64_t scratch_bytes);  // chunks per window; 0: too small
hipError_t launch_chunk_fwd_windows(const ChunkArgs& a, char* scratch, int64_t scratch_bytes, hipStream_t st);
// The state at every chunk start, [slot][h][Dk][Dv] fp32 (fp32 products for either input type),
// X = V - Kt S and U of every chunk, [slot][h][2][64][Dv], and the backward pass's operands: `recs`
// holds chunk_slots(a) * H records of chunk_states_record_bytes(Dk) bytes, `brecs` as many
// BwdRec<Dk> records.
int64_t chunk_states_record_bytes(int Dk);
hipError_t launch_chunk_states(const ChunkArgs& a, void* recs, float* brecs, float* states, float* xu,
                               hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

// Per (chunk, head) operands of the backward pass in plain row-major fp32 (float offsets):
// Qt^T, Kt^T [DK][64]; Kb [64][DK]; P^T, Minv^T [64][64] with Minv = (I + Diag(b) Abar)^{-1};
// Abar [64][64]; gamma [DK]; b [64].  Transposed where the backward products contract over tokens.
// Written by the forward preparation kernel in its backward form, read by the backward kernels.
template <int DK>
struct BwdRec {
    static constexpr int QTT = 0, KTT = 64 * DK, KB = 128 * DK, PMT = 192 * DK, MIT = PMT + 4096,
                         AB = MIT + 4096, GM = AB + 4096, BT = GM + DK, FLOATS = BT + 64;
    static_assert(FLOATS % 64 == 0, "records stay 256-byte aligned");
};

// Backward pass (kda_bwd.hip): gradients of o and the final state.
struct BwdArgs {
    const void *q, *k, *v;
    const float *g, *beta, *s0, *d_o, *d_sfinal;
    float *dq, *dk, *dv, *dg, *dbeta, *ds0;
    const int32_t* cu_seqlens;  // device offsets, or nullptr for equal-length sequences
    int64_t T_fixed, total, N;
    int H, Dk, Dv;
    bool f32;
};
int64_t bwd_slots(const BwdArgs& a);
int64_t bwd_workspace_bytes(const BwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a, void* ws, hipStream_t st);

}  // namespace kda
