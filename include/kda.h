/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * The library computes the forward pass of the channel-wise gated delta rule
 * ("Kimi Delta Attention", KDA) and its two special cases:
 *
 *   KDA_GATE_CHANNEL  Kimi Delta Attention: one decay per key channel,
 *                     S~_t = S_{t-1} Diag(alpha_t)
 *                     ("You could have come up with Kimi Delta Attention",
 *                     the five state-update equations at the top; GeekNews
 *                     #31925, section "Kimi Delta Attention: per-channel decay")
 *   KDA_GATE_SCALAR   Gated DeltaNet: one decay per token and head,
 *                     S~_t = alpha_t S_{t-1}
 *                     (GeekNews #31925, section "Gated DeltaNet: forget the
 *                     whole state first")
 *   KDA_GATE_NONE     DeltaNet: no decay
 *                     (GeekNews #31925, section "DeltaNet: write the error,
 *                     not the value")
 *
 * and then, in every mode, per token t of every (batch, head) sequence:
 *   vhat = S~_t k_t ;  e_t = beta_t (v_t - vhat) ;  S_t = S~_t + e_t k_t^T ;
 *   o_t  = S_t (scale * q_t)      (scale is d_k^-1/2 in the article)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Token tensors are contiguous [B, T, heads, D]: q and k are
 *   [B, T, Hqk, Dk], v and o [B, T, H, Dv].  H counts the value heads: every
 *   (batch, value head) pair is one independent recurrence with its own
 *   state, and value head h reads query/key head h / (H / Hqk) (grouped value
 *   heads; GeekNews #31925, section "Fused recurrent kernel for decode":
 *   programs run per sequence and value head).  Hqk = H is the ungrouped
 *   case; H must be a multiple of Hqk.  beta is [B, T, H] float.  Gates are log-gates
 *   g = log(alpha) <= 0 (GeekNews #31925, section "Diagonal-plus-low-rank
 *   transition": implementations store g and use exp(g)) as float:
 *   [B, T, H, Dk] for KDA_GATE_CHANNEL, [B, T, H] for KDA_GATE_SCALAR, and
 *   NULL for KDA_GATE_NONE (per value head).  The recurrent state is stored transposed,
 *   H = S^T, as contiguous float [B, H, Dk, Dv] (row = key channel, column =
 *   value channel), the d_k x d_v layout named in the same summary.
 * dtype.  q, k and v share one storage type `dtype`: KDA_F32 (float) or
 *   KDA_BF16 (bfloat16 bit patterns).  o has its own storage type `o_dtype`
 *   (either one, independently).  The state is float32.  Arithmetic keeps
 *   about float32 accuracy throughout: every product that carries the state
 *   or the output uses float32 operands, or bf16 hi/lo pairs of them on the
 *   matrix cores (see the kernel sources); a bf16 o is the float32 result
 *   rounded to nearest-even at the final store.
 * Pointers.  All tensor pointers are DEVICE pointers owned by the caller.
 *   The library never allocates, frees or synchronises (its one piece of
 *   device memory, the fixed scratch array behind kda_chunk_fwd_noalloc, is
 *   part of its code object and is placed on a device when the library is
 *   loaded there); all work is enqueued
 *   on `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *   is asynchronous with respect to the host.  Pointers must be 16-byte
 *   aligned.  Inputs are not modified except where stated.
 * Shapes.  B, H >= 1, T >= 0 (T = 0 leaves every output untouched except
 *   that kda_chunk_fwd copies the initial state to the final state).
 *   1 <= Hqk <= H with H % Hqk == 0.  Dk in {16, 32, 64, 128} and Dv in
 *   {16, 32, 64, 128, 256}, in any combination; chunk in {16, 32, 64}; T
 *   need not be a multiple of chunk.  One exception: the chunk forward
 *   (kda_chunk_fwd, kda_chunk_fwd_varlen) with float32 operands, chunk 64,
 *   Dk 128 and Dv 256 returns KDA_ERROR_NOT_SUPPORTED (its staging does not
 *   fit a compute unit's LDS; chunk 32 serves that shape).
 * Values.  g must be finite (a hard forget is g = -30, say, not -inf).
 *   Keys are used as given unless KDA_NORMALIZE_QK is passed: the article
 *   assumes unit keys, but nothing else here normalises or checks them.
 *   beta is not clamped.
 * Errors.  Arguments are validated on the host before any HIP call; a bad
 *   argument returns a status and enqueues nothing.  A failed launch returns
 *   KDA_ERROR_HIP.  Nothing is printed and nothing aborts.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_GATE_CHANNEL = 0,
    KDA_GATE_SCALAR = 1,
    KDA_GATE_NONE = 2
} kda_gate_mode;

typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

/*
 * Fused prologue (the `prologue` argument, a bitwise OR of these flags; 0
 * uses q, k, beta and g as given).  Each flag moves one input transform into
 * the kernels, applied to the values as they are loaded:
 *   KDA_NORMALIZE_QK     q and k of every token and query/key head are
 *                        L2-normalised over Dk, x / sqrt(sum x^2 + 1e-6)
 *                        ("You could have come up with Kimi Delta
 *                        Attention", notation note: keys are assumed
 *                        normalised); the query scale applies after it.
 *   KDA_BETA_SIGMOID     beta holds pre-activations b; the write strength
 *                        is sigmoid(b), inside [0, 1] (GeekNews #31925,
 *                        section "DeltaNet: write the error, not the value").
 *   KDA_GATE_LOGSIGMOID  g holds pre-activations a; the retention is
 *                        alpha = sigmoid(a), i.e. g = log(sigmoid(a)) <= 0
 *                        (GeekNews #31925, section "Diagonal-plus-low-rank
 *                        transition": implementations keep g = log alpha).
 */
typedef enum {
    KDA_NORMALIZE_QK = 1,
    KDA_BETA_SIGMOID = 2,
    KDA_GATE_LOGSIGMOID = 4,
    KDA_PROLOGUE_ALL = 7
} kda_prologue;

typedef enum {
    KDA_SUCCESS = 0,
    KDA_ERROR_INVALID_VALUE = 1,  /* NULL required pointer, negative size, bad enum */
    KDA_ERROR_NOT_SUPPORTED = 2,  /* Dk, Dv or chunk outside the supported set     */
    KDA_ERROR_MISALIGNED = 3,     /* a pointer is not 16-byte aligned (cu_seqlens: 4) */
    KDA_ERROR_WORKSPACE = 4,      /* workspace NULL or smaller than required        */
    KDA_ERROR_HIP = 5,            /* the HIP runtime reported an error at launch    */
    KDA_ERROR_SCRATCH = 6         /* kda_chunk_fwd_noalloc: the call needs more
                                     than KDA_NOALLOC_SCRATCH_BYTES of scratch      */
} kda_status;

/*
 * kda_recurrent_step -- the recurrent (token-by-token) form.
 *
 * Runs T >= 1 tokens of every (b, h) sequence in order, starting from and
 * updating `state` IN PLACE; T = 1 is one decode step.  This is the fused
 * recurrent execution of GeekNews #31925, section "Fused recurrent kernel for
 * decode": one workgroup owns one (batch, head) state, streams it once from
 * HBM, applies decay, prediction, correction, the rank-1 write and the read,
 * and writes it back once.
 *
 *   q, k   [B,T,Hqk,Dk] dtype       in
 *   v      [B,T,H,Dv]  dtype        in
 *   g      see "Layout" (float)     in   (NULL iff mode == KDA_GATE_NONE)
 *   beta   [B,T,H]     float        in
 *   state  [B,H,Dk,Dv] float        in/out (S_{t0-1} on entry, S_{t0+T-1} on exit)
 *   o      [B,T,H,Dv]  o_dtype      out  (must not alias any input)
 *   scale  query scale (pass 1/sqrt(Dk) for the article's d_k^-1/2)
 *   prologue  kda_prologue flags (0: inputs used as given)
 */
kda_status kda_recurrent_step(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              float* state, void* o,
                              int B, int T, int H, int Hqk, int Dk, int Dv, float scale,
                              kda_gate_mode mode, kda_dtype dtype, kda_dtype o_dtype,
                              int prologue, void* stream);

/*
 * kda_chunk_fwd_workspace_size -- bytes of device workspace kda_chunk_fwd
 * needs for these arguments (0 when T == 0).  Returns 0 as well for
 * unsupported arguments; kda_chunk_fwd then reports the precise error.
 */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, int chunk,
                                    kda_gate_mode mode, kda_dtype dtype);

/*
 * kda_chunk_fwd -- the chunkwise-parallel form (prefill / training forward).
 *
 * Same mathematics and results (up to rounding) as running
 * kda_recurrent_step over all T tokens (GeekNews #31925, section "Chunkwise
 * KDA: recasting the recurrence as matrix products": per chunk of `chunk`
 * tokens, cumulative log-decay, the strictly lower coupling matrix and a
 * triangular (UT/WY) solve for pseudo-values; then a sequential carry of
 * the state from chunk to chunk, and intra- plus inter-chunk outputs).
 *
 *   q, k, v, g, beta, o   as for kda_recurrent_step
 *   initial_state  [B,H,Dk,Dv] float in, or NULL for a zero state
 *   final_state    [B,H,Dk,Dv] float out, or NULL (not stored); it may be the
 *                  same pointer as initial_state (in-place hand-off)
 *   chunk          16, 32 or 64 tokens
 *   workspace      device buffer of at least
 *                  kda_chunk_fwd_workspace_size(...) bytes, owned by the
 *                  caller, 256-byte aligned; its contents are scratch
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* initial_state, float* final_state, void* o,
                         int B, int T, int H, int Hqk, int Dk, int Dv, int chunk, float scale,
                         kda_gate_mode mode, kda_dtype dtype, kda_dtype o_dtype,
                         int prologue, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, hosts that
 * forbid allocation.  It takes the same arguments as kda_chunk_fwd except
 * the workspace, runs the same kernels and gives the same bits.  Its chunk
 * records live in a fixed device array of KDA_NOALLOC_SCRATCH_BYTES owned
 * by the library: every device the library runs on holds one copy of it
 * until the process ends, and the call itself allocates nothing (the
 * array's device address is looked up once per device, on the first call
 * made with that device current).
 *
 * Limit: a call whose kda_chunk_fwd_workspace_size(...) exceeds
 * KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERROR_SCRATCH and enqueues nothing.
 * 128 MiB holds, e.g., B1 H16 T4096 d128 chunk 64 with bf16 operands
 * (112.5 MiB).
 * Concurrency: all calls on one device share that device's array; calls
 * that overlap in time on one device (different streams or host threads)
 * race on it and give undefined results.  Calls ordered on one stream are
 * safe (each call writes every record it reads).
 * Other errors are those of kda_chunk_fwd.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
kda_status kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const float* g, const float* beta,
                                 const float* initial_state, float* final_state, void* o,
                                 int B, int T, int H, int Hqk, int Dk, int Dv, int chunk,
                                 float scale, kda_gate_mode mode, kda_dtype dtype,
                                 kda_dtype o_dtype, int prologue, void* stream);

/*
 * Packed variable-length batches
 * ------------------------------
 * N independent sequences of different lengths packed along one token axis
 * (GeekNews #31925, section "Fused recurrent kernel for decode": the
 * recurrent form serves decode, short sequences and stateful serving, and
 * different sequences, heads and value tiles run independently).  Token
 * tensors are [T, heads, D] (the dense layout with B = 1), T the total
 * number of packed tokens: q, k [T, Hqk, Dk], v, o [T, H, Dv]; beta is
 * [T, H]; gates [T, H, Dk] or [T, H].  Sequence n holds
 * tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 and has its own state, entry n of
 * a [N, H, Dk, Dv] float state.  Every sequence starts and ends its own
 * recurrence: results equal separate calls, one per sequence.
 *
 * cu_seqlens is a DEVICE array of N + 1 int32, 4-byte aligned, with
 * 0 = cu_seqlens[0] <= cu_seqlens[1] <= ... <= cu_seqlens[N] = T (empty
 * sequences allowed).  Its contents cannot be checked on the host.  The
 * kernels clamp every entry into [0, T], so no access leaves the buffers
 * whatever the array holds. A malformed array gives defined but meaningless
 * results.
 */

/*
 * kda_recurrent_varlen -- kda_recurrent_step over a packed batch: for every
 * sequence n and head h, the tokens of sequence n in order, starting from
 * and updating state[n, h] IN PLACE (an empty sequence leaves it as is).
 *
 *   q, k   [T,Hqk,Dk] dtype  in         v, o  [T,H,Dv]  (o: o_dtype, out)
 *   g, beta as above (float, in)       state [N,H,Dk,Dv] float in/out
 *   cu_seqlens [N+1] int32 device      N >= 0 (N = 0 or T = 0: nothing to do)
 */
kda_status kda_recurrent_varlen(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                float* state, void* o, const int* cu_seqlens,
                                int N, int T, int H, int Hqk, int Dk, int Dv, float scale,
                                kda_gate_mode mode, kda_dtype dtype, kda_dtype o_dtype,
                                int prologue, void* stream);

/*
 * kda_chunk_fwd_varlen_workspace_size -- bytes of device workspace
 * kda_chunk_fwd_varlen needs (0 for unsupported arguments or N = 0).  It
 * depends on N and T only, not on the individual lengths: the chunks of every
 * sequence start at its first token, and there are at most ceil(T/chunk) + N
 * of them.
 */
size_t kda_chunk_fwd_varlen_workspace_size(int N, int T, int H, int Dk, int Dv, int chunk,
                                           kda_gate_mode mode, kda_dtype dtype);

/*
 * kda_chunk_fwd_varlen -- kda_chunk_fwd over a packed batch: every sequence
 * is cut into chunks from its own first token (the last one ragged) and
 * carries its own state from chunk to chunk.
 *
 *   q, k, v, g, beta, o, cu_seqlens   as for kda_recurrent_varlen
 *   initial_state  [N,H,Dk,Dv] float in, or NULL for zero states
 *   final_state    [N,H,Dk,Dv] float out, or NULL; may equal initial_state
 *   chunk, scale, mode, dtype, o_dtype   as for kda_chunk_fwd
 *   workspace      at least kda_chunk_fwd_varlen_workspace_size(...) bytes,
 *                  256-byte aligned, owned by the caller; contents are
 *                  scratch (it also holds the chunk table built from
 *                  cu_seqlens on the device, so the call stays asynchronous)
 */
kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                const float* g, const float* beta,
                                const float* initial_state, float* final_state, void* o,
                                const int* cu_seqlens, int N, int T, int H, int Hqk, int Dk,
                                int Dv, int chunk, float scale, kda_gate_mode mode, kda_dtype dtype,
                                kda_dtype o_dtype, int prologue, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Gradients (training backward)
 * -----------------------------
 * The pages train the method with the chunkwise algorithm (F29 course
 * outline, "Paper: Gated DeltaNet -> Kimi Delta Attention"; GeekNews #31925,
 * section "Fused recurrent kernel for decode": the chunkwise form serves
 * training and prefill).  kda_chunk_bwd returns the gradients of a scalar
 * loss with respect to every input of kda_chunk_fwd, given the gradients of
 * that loss with respect to its outputs, i.e. reverse mode through the same
 * recurrence (results equal, up to rounding, the gradient of the token loop
 * of kda_recurrent_step).  It recomputes what it needs from the inputs (no
 * tensors are saved by the forward call).
 */

/*
 * kda_chunk_bwd_workspace_size -- bytes of device workspace kda_chunk_bwd
 * needs (0 when T == 0 or the arguments are unsupported).  About
 * 4 (2 Dk Dv + 4 chunk Dk + 3 chunk Dv + 3 chunk^2) bytes per (b, h, chunk),
 * plus 8 B T H Dk bytes when Hqk < H.
 */
size_t kda_chunk_bwd_workspace_size(int B, int T, int H, int Hqk, int Dk, int Dv, int chunk,
                                    kda_gate_mode mode, kda_dtype dtype);

/*
 * kda_chunk_bwd -- gradients of the chunkwise form.
 *
 *   q, k, v, g, beta, initial_state   the inputs of the forward call (same
 *                  layouts; initial_state NULL = zero state)
 *   d_o            [B,T,H,Dv] dtype      dL/do, in
 *   d_final_state  [B,H,Dk,Dv] float     dL/d(final state), in, or NULL (zero)
 *   dq, dk         [B,T,Hqk,Dk] grad_dtype  out (grouped value heads: the sum
 *                  over the value heads that read the query/key head)
 *   dv             [B,T,H,Dv] grad_dtype    out
 *   dg             shape of g, float     out (NULL iff mode == KDA_GATE_NONE;
 *                  scalar mode: one value per token and head)
 *   dbeta          [B,T,H] float         out
 *   d_initial_state [B,H,Dk,Dv] float    out, or NULL (not stored); with
 *                  T = 0 it receives d_final_state (zero if NULL)
 *   chunk, scale, mode   as for kda_chunk_fwd (chunk 16, 32 or 64)
 *   dtype          storage type of q, k, v and d_o
 *   grad_dtype     storage type of dq, dk and dv (either one, independently;
 *                  a bf16 gradient is the float32 result rounded to
 *                  nearest-even at the final store)
 *   workspace      at least kda_chunk_bwd_workspace_size(...) bytes,
 *                  256-byte aligned, caller-owned scratch
 *
 * Outputs must not alias inputs or each other.  The fused prologue is
 * forward-only: pass the transformed inputs (and take the prologue's own
 * gradients outside).  Gates are handled over the same range as the
 * forward: any finite g, hard forgets (g = -30, say) included (GeekNews
 * #31925, section "Gated DeltaNet: forget the whole state first").
 */
kda_status kda_chunk_bwd(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* initial_state, const void* d_o,
                         const float* d_final_state, void* dq, void* dk, void* dv, float* dg,
                         float* dbeta, float* d_initial_state, int B, int T, int H, int Hqk,
                         int Dk, int Dv, int chunk, float scale, kda_gate_mode mode,
                         kda_dtype dtype, kda_dtype grad_dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * kda_chunk_bwd_varlen_workspace_size -- bytes of device workspace
 * kda_chunk_bwd_varlen needs (0 for unsupported arguments or N = 0): records
 * for ceil(T / chunk) + N chunks per head, the chunk and sequence tables,
 * and 8 T H Dk bytes when Hqk < H.
 */
size_t kda_chunk_bwd_varlen_workspace_size(int N, int T, int H, int Hqk, int Dk, int Dv, int chunk,
                                           kda_gate_mode mode, kda_dtype dtype);

/*
 * kda_chunk_bwd_varlen -- kda_chunk_bwd over a packed batch (see "Packed
 * variable-length batches"): the gradients of kda_chunk_fwd_varlen.  Every
 * sequence is cut into chunks from its own first token and carries its own
 * state and state gradient; results equal separate kda_chunk_bwd calls, one
 * per sequence.
 *
 *   q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta   packed [T, heads, ...]
 *                  as for kda_recurrent_varlen (no batch axis)
 *   initial_state, d_final_state, d_initial_state   [N,H,Dk,Dv] float or NULL
 *   cu_seqlens     [N+1] int32 device offsets (clamped as for the forward)
 *   the rest       as for kda_chunk_bwd; the workspace holds at least
 *                  kda_chunk_bwd_varlen_workspace_size(...) bytes, 256-byte
 *                  aligned, and also the tables built on the device
 */
kda_status kda_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, const float* initial_state, const void* d_o,
                                const float* d_final_state, void* dq, void* dk, void* dv,
                                float* dg, float* dbeta, float* d_initial_state,
                                const int* cu_seqlens, int N, int T, int H, int Hqk, int Dk,
                                int Dv, int chunk, float scale, kda_gate_mode mode,
                                kda_dtype dtype, kda_dtype grad_dtype, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* kda_status_string(kda_status s);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
