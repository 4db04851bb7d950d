/*
 * kda.h — C ABI of the gated delta-rule (Kimi Delta Attention) forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation ("Kimi K3 Open Model Surpasses Closed GPT and Anthropic
 * Systems on Independent Benchmarks", worldcybernews, second paragraph): each
 * head keeps a fixed-size state matrix S (Dk x Dv) in place of a key/value
 * cache; every token updates it with the delta rule, beta being the write
 * strength and alpha the forget gate, and alpha is kept inside [e^-5, 1].
 * Read here as, per token t and head h,
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t,      alpha_t = exp(clamp(g_t, -5, 0))  (per key channel)
 *
 * The third paragraph of the same page describes a kernel that processes the
 * tokens of each chunk in parallel while the state is carried sequentially from
 * chunk to chunk; kda_chunk_fwd and kda_varlen_fwd compute the recurrence that
 * way, 64 tokens at a time, and their results do not depend on the chunk size
 * beyond rounding.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, contiguous, row-major in the
 *    layouts given below, 16-byte aligned.  The caller owns every buffer; the
 *    library allocates nothing and keeps no pointer after a call returns.
 *  - q, k, v use `dtype` (KDA_BF16 or KDA_F32).  By default g (log alpha,
 *    clamped to [-5, 0] by the library) and beta are float32 and used as
 *    given; a kda_prologue (below) can change that.  The states and the output
 *    o are float32.  o is float32 for both input types: rounding it to bf16
 *    would by itself cost up to about 3% of the output RMS on realistic gate
 *    statistics.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *    asynchronous and stream-ordered; nothing here synchronises the device.
 *  - Arguments are validated on the host before any launch.  A non-zero
 *    status means nothing was launched, except KDA_ERR_HIP, which reports a
 *    launch failure.  kda_last_error() returns a message for the last failing
 *    call on the calling thread.  No call aborts or throws.
 *  - Supported head sizes: Dk, Dv in {64, 128}.  chunk must be 64.
 *  - Calls are reentrant; concurrent calls on different streams must not
 *    write the same buffers.
 *
 * Workspace of the prefill entry points
 * -------------------------------------
 * kda_chunk_fwd and kda_varlen_fwd take an optional caller-owned device
 * workspace (16-byte aligned, at least kda_*_workspace_bytes() bytes; no
 * initial contents needed).  With a workspace, one kernel first prepares every
 * (chunk, head) in parallel -- the decay-weighted queries and keys, the lower
 * triangular inverse (I + A)^-1 scaled by beta and the decay-weighted
 * query-key block of the chunk, in matrix-core operand order -- and stores
 * them there; a second kernel then carries the state through the chunks.  With workspace == NULL a single fused kernel does both
 * and nothing extra is needed.  Both give the same results up to rounding.
 * A workspace smaller than required is rejected with KDA_ERR_BAD_SHAPE.
 * The workspace must not be shared by calls that may run concurrently.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * Input prologue: transforms applied to the inputs as the kernels load them, so
 * that raw projections can be fed in without separate passes over HBM, and
 * bf16 gates halve their bytes.  The page cited above fixes only the roles of
 * alpha (forgetting, kept inside [e^-5, 1] against bf16 underflow and overflow)
 * and beta (write strength); the logit forms below are the customary
 * parameterisations of such gates, not something the page states.  Pass NULL
 * for the defaults (all fields zero / KDA_F32):
 *   g_dtype     element type of g (KDA_F32 or KDA_BF16)
 *   g_logit     0: g is log alpha.  Nonzero: g holds gate logits x and
 *               log alpha = -softplus(x) = -ln(1 + e^x); the clamp to [-5, 0]
 *               follows in both cases.
 *   beta_dtype  element type of beta (KDA_F32 or KDA_BF16)
 *   beta_logit  0: beta is used as given.  Nonzero: beta = 1 / (1 + e^-b).
 *   qk_l2norm   nonzero: q and k are scaled to unit L2 norm per token and
 *               head before use (an all-zero vector stays zero).
 * The transforms are evaluated in float32.
 */
typedef struct {
    kda_dtype g_dtype;
    int g_logit;
    kda_dtype beta_dtype;
    int beta_logit;
    int qk_l2norm;
} kda_prologue;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_ARG = 1,   /* a required pointer is NULL */
    KDA_ERR_BAD_SHAPE = 2,  /* unsupported or inconsistent size */
    KDA_ERR_BAD_DTYPE = 3,  /* dtype not KDA_F32 / KDA_BF16 */
    KDA_ERR_MISALIGNED = 4, /* a pointer is not 16-byte aligned */
    KDA_ERR_HIP = 5         /* the HIP runtime reported an error at launch */
} kda_status;

/*
 * Chunked prefill over B sequences of equal length T.
 * Defined by: the worldcybernews page cited above, second paragraph (the
 * recurrence: fixed-size state, delta-rule update with write strength beta and
 * forget gate alpha in [e^-5, 1]) and third paragraph (the tokens of a chunk
 * processed in parallel, the state carried from chunk to chunk; long
 * sequences with few heads are cut into segments whose initial states a
 * prefix scan recovers, the one-GPU form of that paragraph's scan).
 *   q, k : [B, T, H, Dk]  dtype          v : [B, T, H, Dv]  dtype
 *   g    : [B, T, H, Dk]  log alpha, clamped to [-5, 0] inside (float32 unless
 *                         the prologue says otherwise)
 *   beta : [B, T, H]      used as given, not clamped (idem)
 *   prologue : input transforms, or NULL (see kda_prologue)
 *   s0   : [B, H, Dk, Dv] float32 initial state, or NULL for zeros
 *   o    : [B, T, H, Dv]  float32 output (written)
 *   s_final : [B, H, Dk, Dv] float32 final state (written), or NULL
 * T = 0 is allowed: o is untouched and s_final receives s0 (or zeros).
 * s_final may alias s0 (each state is read before it is written).
 * Arithmetic: float32 accumulation and a float32 state throughout.  With a
 * workspace and bf16 inputs the per-chunk operands are fp16 (some as fp16
 * pairs) on the matrix cores; v and the state are scaled by a power of two per
 * chunk so that any magnitude stays in fp16's range, and queries and keys of
 * the method's scale (unit norm, or qk_l2norm) keep the other operands far
 * inside it.  fp32 inputs and the fused kernel (workspace NULL) use split-bf16
 * or fp32 operands.
 * Speed: with workspace NULL the call is one fused kernel that repeats the
 * state-independent work in every 32-column slice, about three times slower
 * than the two-kernel path a workspace enables; a caller that cannot provide a
 * workspace but can serialise its calls on a GPU gets the two-kernel path from
 * kda_chunk_fwd_noalloc.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                         const float* s0, float* o, float* s_final, int64_t B, int64_t T, int H, int Dk,
                         int Dv, int chunk, kda_dtype dtype, const kda_prologue* prologue, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd without any allocation or workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Arguments, layouts, results and
 * errors as for kda_chunk_fwd; the results equal its two-kernel path bit for bit.
 * The library keeps one fixed scratch area of 128 MiB per GPU (a static device
 * array, held from the first call on that GPU until the process ends) and
 * runs the call in windows of W * 64 tokens whose per-chunk records fit there:
 * W = floor((128 MiB - state) / (B * H * record)), with the record size given
 * for kda_chunk_workspace_bytes and state = B*H*Dk*Dv*4 bytes (rounded up to
 * 256) when s_final is NULL, else 0.  Calls with W < 1 (B*H above 1807 at
 * Dk = 128 with bf16 inputs and s_final given, above 960 without) are rejected with
 * KDA_ERR_BAD_SHAPE.  The scratch of the current device is used: `stream`
 * must belong to it.  Every call on a GPU shares that GPU's scratch, so calls
 * that may overlap on one GPU (different streams, or concurrent host threads)
 * race and must be serialised by the caller.  Nothing is allocated, freed or
 * cleared by the library in this call.
 */
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                                 const float* s0, float* o, float* s_final, int64_t B, int64_t T, int H, int Dk,
                                 int Dv, int chunk, kda_dtype dtype, const kda_prologue* prologue, void* stream);

/*
 * Workspace bytes kda_chunk_fwd needs for these sizes (0 if none are needed or
 * the arguments are unsupported): B * ceil(T/64) * H records of
 * 64*Dk*6 (bf16) or 64*Dk*12 (fp32) + 24576 + 4*Dk bytes
 * (72.5 KiB per chunk and head at Dk = 128 with bf16 inputs).  Calls with few
 * state columns in all (2 * B*H*Dv/32 <= 256) and long sequences are cut into
 * P = min(256 / (B*H*Dv/32), ceil(T/64) / 64) >= 2 segments along T; they need
 * B*H*Dk*4*((P-1)*(Dv+Dk) + P*Dv) more bytes for the segment states.
 */
size_t kda_chunk_workspace_bytes(int64_t B, int64_t T, int H, int Dk, int Dv, kda_dtype dtype);

/*
 * Packed variable-length prefill: N independent sequences stored back to back.
 * Defined by: the same second paragraph -- every sequence keeps its own
 * fixed-size state, so packed sequences are independent runs of the
 * recurrence, each starting from its own initial state; chunks as in the
 * third paragraph, starting at each sequence's first token.
 *   q, k, g : [total, H, Dk]; v, o : [total, H, Dv]; beta : [total, H]
 *   (element types and prologue as for kda_chunk_fwd)
 *   cu_seqlens : DEVICE int32 [N+1], non-decreasing, cu_seqlens[0] = 0,
 *                cu_seqlens[N] = total; sequence n is tokens
 *                cu_seqlens[n] .. cu_seqlens[n+1]-1 and starts its own chunks.
 *   s0, s_final : [N, H, Dk, Dv] float32, each may be NULL (zeros / not written).
 * The offsets are read on the device (no host synchronisation); offsets that
 * break the stated invariants give unspecified results for the affected
 * sequences but never access memory outside [0, total) tokens.
 */
kda_status kda_varlen_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                          const int32_t* cu_seqlens, int64_t N, int64_t total, const float* s0, float* o,
                          float* s_final, int H, int Dk, int Dv, int chunk, kda_dtype dtype,
                          const kda_prologue* prologue, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes kda_varlen_fwd needs (0 if none or unsupported sizes): it
 * depends only on N and total, not on the offsets, so a buffer sized once
 * serves every packing of that many tokens: (floor(total/64) + N) * H records
 * of the size given for kda_chunk_workspace_bytes, plus 4*N bytes rounded up to
 * a multiple of 256 (the order, longest first, in which the sequences' state
 * chains are started).
 */
size_t kda_varlen_workspace_bytes(int64_t N, int64_t total, int H, int Dk, int Dv, kda_dtype dtype);

/*
 * One decoding step (one new token per sequence) on B sequences.
 * Defined by: the same second paragraph -- the state matrix takes the place
 * of the key/value cache, so generating a token is one update of S by the
 * recurrence followed by the read-out o = S^T q.
 *   q, k : [B, H, Dk] dtype;  v : [B, H, Dv] dtype
 *   g    : [B, H, Dk] log alpha;  beta : [B, H]  (float32 unless the prologue
 *          says otherwise; prologue as for kda_chunk_fwd, or NULL)
 *   s_in : [B, H, Dk, Dv] float32 state before the token
 *   s_out: [B, H, Dk, Dv] float32 state after the token; s_out == s_in is
 *          allowed (in-place update); partial overlap is not.
 *   o    : [B, H, Dv] float32 output of the token
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                           const float* s_in, float* s_out, float* o, int64_t B, int H, int Dk, int Dv,
                           kda_dtype dtype, const kda_prologue* prologue, void* stream);

/*
 * Gradients of kda_chunk_fwd (no prologue: g is log alpha and beta is used as given, both
 * float32).  Defined by: the forward recurrence of the same second paragraph, differentiated; the
 * pages give no backward pass ("Kimi K3: Open Frontier Intelligence" abstract only ties KDA to
 * training at scale), so every formula here is derived from the forward one.  The pages describe only the forward recurrence; these are its exact derivatives,
 * for a loss L with dL/do = d_o and dL/dS_T = d_sfinal:
 *   d_o      : [B, T, H, Dv] float32;   d_sfinal : [B, H, Dk, Dv] float32, or NULL for zero
 *   dq, dk   : [B, T, H, Dk] float32;   dv : [B, T, H, Dv] float32   (written)
 *   dg       : [B, T, H, Dk] float32, gradient with respect to g before the clamp: zero where
 *              g < -5 or g > 0 (the clamp passes the gradient on [-5, 0])   (written)
 *   dbeta    : [B, T, H] float32 (written)
 *   ds0      : [B, H, Dk, Dv] float32 gradient of the initial state (written), or NULL
 * q, k, v, g, beta, s0 as for kda_chunk_fwd (s0 NULL = zero initial state).  The workspace is
 * required (kda_chunk_bwd_workspace_bytes; no initial contents needed); a NULL or smaller one is
 * rejected.  Accumulation and the carried states are float32; the matrix products run either in
 * float32 or as three-pass split-bf16 products (hi*hi + hi*lo + lo*hi, about 16 significant bits per
 * operand).  T = 0: only ds0 = d_sfinal (or 0).
 */
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* s0, const float* d_o, const float* d_sfinal, float* dq, float* dk, float* dv,
                         float* dg, float* dbeta, float* ds0, int64_t B, int64_t T, int H, int Dk, int Dv, int chunk,
                         kda_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes kda_chunk_bwd needs: B * ceil(T/64) * H records of
 * 4 * (386*Dk + 20544 + 2*Dk*Dv + 192*Dv) bytes (497.25 KiB at Dk = Dv = 128), plus 4*Dv
 * bytes rounded up to a multiple of 256.
 */
size_t kda_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int H, int Dk, int Dv, kda_dtype dtype);

/*
 * Gradients of kda_varlen_fwd (defined as for kda_chunk_bwd, per packed sequence): the packed layouts of kda_varlen_fwd, the outputs as for
 * kda_chunk_bwd ([total, H, D] for the token tensors, [N, H, Dk, Dv] for d_sfinal and ds0).
 */
kda_status kda_varlen_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const int32_t* cu_seqlens, int64_t N, int64_t total, const float* s0, const float* d_o,
                          const float* d_sfinal, float* dq, float* dk, float* dv, float* dg, float* dbeta, float* ds0,
                          int H, int Dk, int Dv, int chunk, kda_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Workspace bytes kda_varlen_bwd needs: (floor(total/64) + N) * H records as above. */
size_t kda_varlen_bwd_workspace_bytes(int64_t N, int64_t total, int H, int Dk, int Dv, kda_dtype dtype);

/* Message describing the last non-OK status returned on this thread ("" if none). */
const char* kda_last_error(void);

/* Library version string. */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
