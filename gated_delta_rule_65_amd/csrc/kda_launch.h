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

// Long sequences with few heads split the chunk range into P segments of L chunks (the one-GPU
// form of the segment scan the worldcybernews page's third paragraph describes across GPUs):
//   mode 1 (segment maps), items (n, h, p < P-1), (Dv + Dk)/32 column slices: the segment run
//     from a zero state gives S0_p (its Dv value columns); run on the identity with V = 0 it gives
//     the segment's transition Phi_p (Dk more columns).  Both go to sx [item][Dk][Dv + Dk]; no o.
//   mode 2 (outputs), items (n, h, p): segment p from its true initial state, sfold [n][h][p][Dk][Dv]
//     from the fold kernel (which copies s0 into p = 0), o written, s_final from p = P - 1.
//   mode 0: whole sequences (items (n, h)), s0 -> s_final.
//   mode 3: as mode 0, and the state at the start of every chunk goes to sx [slot][h][Dk][Dv]
//     (for the backward pass; compiled state-only with the stores, SO = ST = true).
struct ChainMode {
    int mode;      // 0, 1, 2 or 3
    int P;         // segments per sequence (modes 1, 2)
    int64_t L;     // chunks per segment (modes 1, 2)
    float* sx;     // mode 1 output; mode 3: chunk-start states
    const float* sfold;  // mode 2 input
    float* xu = nullptr;  // mode 3: X and U of every chunk, [slot][h][2][64][Dv] (rows past the end zero)
    const int32_t* order = nullptr;  // packed sequences: item i runs sequence order[i / H] (longest first)
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
// Shared pieces of the two-kernel paths (kda_chunk2.hip): the packed sequences ranked longest first
// (order[rank] = n), and the split-T fold S_in(p+1) = Phi_p S_in(p) + S0_p over `items` = N*H heads.
hipError_t launch_seq_order(const int32_t* cu, int64_t N, int64_t total, int32_t* order, hipStream_t st);
hipError_t launch_fold(int Dk, const float* s0, const float* sx, float* sfold, int64_t items, int H, int Dv, int P,
                       hipStream_t st);
int chunk_segments(const ChunkArgs& a);
// The bf16-input forward with fp16 matrix-core operands (kda_fwd16.hip): record bytes per (chunk, head),
// workspace bytes and launch.
int64_t chunk16_record_bytes(int Dk);
int64_t chunk16_workspace_bytes(const ChunkArgs& a);
hipError_t launch_chunk_fwd16(const ChunkArgs& a, void* ws, hipStream_t st, bool allow_split);

// Per (chunk, head) operands of the backward pass (float offsets).  The reverse state chain's operands
// are MFMA A fragments (split bf16, FRAG floats each: a plane of 64 lanes x 16 B of bf16 hi, then
// one of bf16 lo; lane l holds row 16*block + l%16, contracted indices 32*s + 8*(l/16) .. +7), in
// the order [block][s]:
//   QTF  Qt^T              rows: channels, contracted: tokens   [DK/16][2]
//   KTF  -Kt^T             rows: channels, contracted: tokens   [DK/16][2]
//   KBF  Kb                rows: tokens,   contracted: channels [4][DK/32]
//   PTF  P^T               rows: tokens,   contracted: tokens   [6 pairs]
//   NTF  Diag(b) Minv^T    rows: tokens,   contracted: tokens   [6 pairs]
// (P^T and Minv^T are upper triangular: row blocks 2 and 3 meet only the second step, so the six
// (row block, step) pairs (0,0) (0,1) (1,0) (1,1) (2,1) (3,1) are stored, in that order: tri())
// and the gradient kernel's plain fp32 operands: Minv^T [64][64] with Minv = (I + Diag(b) Abar)^{-1},
// Abar [64][64], gamma [DK], b [64].  Written by the forward preparation kernel in its backward form;
// the six 16x16 blocks of Minv^T below its diagonal blocks and of Abar above them are all zero and are
// not written (the gradient kernel reads only the triangle that can be nonzero).
template <int DK>
struct BwdRec {
    static constexpr int FRAG = 512;
    static constexpr int QTF = 0, KTF = QTF + (DK / 16) * 2 * FRAG, KBF = KTF + (DK / 16) * 2 * FRAG,
                         PTF = KBF + 4 * (DK / 32) * FRAG, NTF = PTF + 6 * FRAG, MIT = NTF + 6 * FRAG,
                         AB = MIT + 4096, GM = AB + 4096, BT = GM + DK, FLOATS = BT + 64;
    static_assert(FLOATS % 64 == 0, "records stay 256-byte aligned");
    // stored pair of (row block rb, step s) of P^T and N^T; for rb >= 2 step 0 (all zero) maps to step 1
    static constexpr int tri(int rb, int s) { return rb < 2 ? 2 * rb + s : 2 + rb; }
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
