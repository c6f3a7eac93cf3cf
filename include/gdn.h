/*
 * gdn.h -- C ABI of the MI355X (gfx950) gated delta rule library (libgdn.so).
 *
 * The library computes the gated delta rule
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 *
 * ("Hybrid models: what Gated DeltaNet replaces in the KV cache", section "Gated
 * DeltaNet: add decay"; the query reads the updated state, "From Traditional Attention
 * to hybrid ones", section 5) and its per-channel-decay variant KDA
 *
 *     S_t = S_{t-1} Diag(alpha_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *
 * ("From Traditional Attention to hybrid ones", section 7).  The state S is d_v x d_k
 * (row = value channel, column = key channel), kept in fp32.  The gate is passed as
 * log_alpha = g (g = log alpha, "Attention, Part 4", "Where alpha and beta come from").
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers to contiguous row-major arrays with the
 *    layouts given below (the prefill's s_ckpt may also be pinned host memory, see
 *    gdn_chunk_fwd); q, k, v, o, s0, s_final, s_ckpt and state must be 16-byte
 *    aligned.  `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - The caller owns every buffer.  The library allocates nothing, frees nothing and
 *    keeps no pointer after a call returns.  Outputs are overwritten entirely.
 *  - Arguments are validated synchronously on the host before anything is launched;
 *    on any error nothing is launched and the status says why.  Work is enqueued
 *    asynchronously on `stream`; the library never synchronises.  A failed launch
 *    returns GDN_ERROR_HIP.  Apart from the scratch of kda_chunk_fwd_noalloc, the library
 *    holds no mutable global state, so calls from several host threads are safe.
 *  - Device VALUES are not checked.  Preconditions: log_alpha finite and <= 0
 *    (alpha in (0, 1]); beta finite (in (0, 1) on the pages); |q|, |k|, |v| <= 65504
 *    for bf16 inputs (the prefill kernels use half-precision matrix-core operands).
 *    Queries and keys are expected to be L2-normalised by the caller (the plain entry
 *    points do not normalise; gdn_chunk_fwd_ex and gdn_decode_ex can, with qk_l2norm),
 *    but this is not required.  No 1/sqrt(d) scale is applied.
 *    Invalid values give NaN/Inf in the outputs, never a fault.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_VERSION 112 /* 1.1.2 */

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype_t;

typedef enum {
  GDN_SUCCESS = 0,
  GDN_ERROR_INVALID_VALUE = 1, /* NULL / misaligned pointer, bad size, bad ckpt_every, overlap */
  GDN_ERROR_NOT_SUPPORTED = 2, /* (Dk, Dv, chunk, dtype) combination not compiled in */
  GDN_ERROR_HIP = 3            /* a HIP runtime call or kernel launch failed */
} gdn_status_t;

/* Shape and options of one chunkwise prefill call. */
typedef struct {
  int64_t B, H, T;      /* batch, heads, tokens; T >= 0 (T = 0: no outputs but s_final = s0) */
  int64_t Dk, Dv;       /* key / value head dimensions */
  int32_t chunk;        /* tokens per chunk: 16, 32 or 64.  The result does not depend on it
                           beyond rounding: the chunked form is exact ("Hybrid attention",
                           section "Training a recurrence in parallel").  A ragged tail
                           (T % chunk != 0) is handled as if padded with identity steps
                           (beta = 0, log_alpha = 0: "Attention, Part 4", section 6). */
  gdn_dtype_t in_dtype; /* dtype of q, k, v, beta, log_alpha (all the same) */
  gdn_dtype_t out_dtype;/* dtype of o */
  int64_t ckpt_every;   /* 0 = no snapshots; else a positive multiple of `chunk` */
} gdn_chunk_desc_t;

/*
 * Bytes of device workspace that gdn_chunk_fwd / kda_chunk_fwd can use for `d`
 * (is_kda = 0 or 1): B * H * ceil(T / 64) * 65536 for the matrix-core KDA prefill (its
 * two-kernel form, every chunk's record at once), 0 for every other supported combination.
 * A smaller workspace of at least 131072 bytes also works: the two-kernel form then runs in
 * slabs of streams and chunks that fit it.  Errors as for gdn_chunk_fwd's validation.
 */
gdn_status_t gdn_chunk_workspace_size(const gdn_chunk_desc_t* d, int is_kda, size_t* bytes);

/*
 * Chunkwise-parallel prefill of the gated delta rule with initial state, final state
 * and chunk-boundary snapshots.
 *
 * Method: the sequence is cut into chunks of `chunk` tokens; inside a chunk the updates
 * are dense matrix products and a small unit lower-triangular system, and only the
 * state is handed from one chunk to the next ("Hybrid Linear Attention Architecture
 * Design Explained", section 4, cross-chunk state update and intra-chunk output;
 * "Hybrid attention", section "Training a recurrence in parallel"; "Hybrid models...",
 * section "What a recurrent state changes for serving", prefill takes a chunked path).
 * Snapshot n (0-based) is the state after token (n+1)*ckpt_every: the state at a
 * position N cannot be recovered from a later one, so prefix reuse needs a snapshot
 * taken at N ("Hybrid models...", same section, item 1).  Resuming from a snapshot is
 * passing it as s0.
 *
 * Arguments (device pointers):
 *   q, k      [B, H, T, Dk]   in_dtype
 *   v         [B, H, T, Dv]   in_dtype
 *   beta      [B, H, T]       in_dtype
 *   log_alpha [B, H, T]       in_dtype
 *   s0        [B, H, Dv, Dk]  fp32, or NULL for a zero initial state
 *   o         [B, H, T, Dv]   out_dtype, written
 *   s_final   [B, H, Dv, Dk]  fp32, written, or NULL.  May be exactly s0 (updated in
 *                             place); any other overlap with s0 is INVALID_VALUE.
 *   s_ckpt    [B, H, T / ckpt_every, Dv, Dk] fp32, written; required (non-NULL) when
 *                             ckpt_every > 0 and T >= ckpt_every, ignored otherwise.
 *                             Device memory, or pinned host memory (hipHostMalloc): then
 *                             every snapshot is written into host RAM by the kernel as soon
 *                             as the prefill reaches it, so capturing snapshots needs no copy
 *                             and never stalls the prefill ("Hybrid models...", same section,
 *                             item 1: snapshot capture made asynchronous); the host may read
 *                             them once the stream's work has completed.  Pageable host
 *                             memory, or a pointer the HIP runtime cannot describe, is
 *                             INVALID_VALUE.
 *   workspace, workspace_bytes: device workspace, 16-byte aligned, when one is given.
 *                             Only the matrix-core KDA prefill uses one (a 64 KiB record
 *                             per (stream, chunk)): with it, the state-independent tiles of
 *                             every chunk are formed once, in parallel, by a first kernel,
 *                             and a second kernel runs the sequential part from them (same
 *                             results, bit for bit, as without).  With fewer bytes than
 *                             gdn_chunk_workspace_size() the two kernels run slab by slab,
 *                             the state carried between slabs in the workspace.  NULL runs
 *                             the single-kernel form; a non-NULL workspace under 131072
 *                             bytes, or one overlapping o, s0, s_final, s_ckpt or the
 *                             inputs, is INVALID_VALUE.  Everywhere else it is ignored.
 * Supported: Dk == Dv; bf16 inputs with Dk = 128 and chunk = 64 run on the matrix
 * cores; fp32 or bf16 inputs with Dk in {16, 32, 64, 128} and any allowed chunk run on
 * the fp32 vector path.  Other combinations: GDN_ERROR_NOT_SUPPORTED.
 */
gdn_status_t gdn_chunk_fwd(const gdn_chunk_desc_t* d, const void* q, const void* k, const void* v,
                           const void* beta, const void* log_alpha, const float* s0, void* o,
                           float* s_final, float* s_ckpt, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Chunkwise prefill of KDA (per-channel decay): identical to gdn_chunk_fwd except
 *   log_alpha [B, H, T, Dk]   in_dtype: one forget rate per key channel
 * ("Attention, Part 4", section 7; "Hybrid Linear Attention Architecture Design
 * Explained", sections 3.1 and 4 -- the division form of the intra-chunk products needs
 * overflow protection).  The kernels split every decay factor e^{G_r - G_j} at reference
 * points inside the chunk; a 16-token block whose gates are too strong for its half-precision
 * split (or whose rows are too large for it) is detected on the device and computed with all
 * its factors <= 1, its diagonal products in fp32.  Any finite log_alpha <= 0 therefore gives
 * finite results within the usual tolerance; such blocks only cost extra work.
 */
gdn_status_t kda_chunk_fwd(const gdn_chunk_desc_t* d, const void* q, const void* k, const void* v,
                           const void* beta, const void* log_alpha, const float* s0, void* o,
                           float* s_final, float* s_ckpt, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * kda_chunk_fwd without any allocation, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid it).  Same
 * arguments, results and validation as kda_chunk_fwd minus the workspace: the matrix-core
 * two-kernel form runs on a fixed 64 MiB scratch array inside the library (one per GPU, held
 * from the library's first launch on that GPU until the process ends), slab by slab, so any
 * size is accepted and the scratch never needs more.  The library calls no allocator.
 * Every call on a GPU shares that GPU's scratch: calls that overlap in time on one GPU (on
 * different streams, or from several host threads) race and must be serialised by the
 * caller.  The scratch keeps the last call's contents; every byte a call reads from it is
 * written by that call first.  GDN_ERROR_HIP if the runtime cannot give the scratch's
 * device address.
 */
gdn_status_t kda_chunk_fwd_noalloc(const gdn_chunk_desc_t* d, const void* q, const void* k, const void* v,
                                   const void* beta, const void* log_alpha, const float* s0, void* o,
                                   float* s_final, float* s_ckpt, void* stream);

/*
 * Chunkwise prefill of the gated delta rule with parts of the layer around the core fused
 * in (gdn_chunk_fwd otherwise):
 *  - value heads sharing query/key heads: base.H value heads, H_qk query/key heads (base.H
 *    a multiple of H_qk); value head h reads query/key head h / (base.H / H_qk);
 *  - raw_gates = 1: beta and log_alpha carry the layer's raw projections b and a, and the
 *    kernel forms beta = sigmoid(b), log alpha = -exp(A_log) softplus(a + dt_bias)
 *    ("Attention, Part 4", section "Where alpha and beta come from");
 *  - a ragged batch (cu_seqlens != NULL): B sequences of different lengths prefilled in one
 *    call, as a serving engine admits new prompts.  Sequence b holds tokens
 *    cu_seqlens[b] .. cu_seqlens[b+1] - 1 of T = cu_seqlens[B] in all; every per-token
 *    tensor is the concatenation of the sequences, each in the layout below with its own
 *    length (q of sequence b is [H_qk, T_b, Dk], starting at row H_qk * cu_seqlens[b]).
 *
 *   q, k      [B, H_qk, T, Dk]   in_dtype (ragged: H_qk * T rows of Dk, as above)
 *   v         [B, H, T, Dv]; beta, log_alpha [B, H, T] (ragged: H * T rows); s0, o,
 *             s_final, s_ckpt as in gdn_chunk_fwd (o ragged like v)
 *   A_log, dt_bias [H] fp32, required when raw_gates = 1, ignored otherwise
 *   cu_seqlens [B + 1] int32 device array, non-decreasing from 0 to T, or NULL.  Values out
 *             of that order are clamped into [0, T] (a sequence can come out empty), never
 *             used to address outside the tensors.  Snapshots need ckpt_every = 0 here.
 *  - qk_l2norm = 1: every query and key row is scaled to unit length before use,
 *    x / sqrt(sum(x^2) + 1e-6) over its Dk channels ("Attention, Part 4", section 6: the
 *    layer normalises q and k before the memory step); qk_l2norm = 0 uses them as given.
 * Supported on the matrix-core path (bf16 inputs, Dk = Dv = 128, chunk = 64); with
 * H_qk = H, raw_gates = 0, qk_l2norm = 0 and no cu_seqlens every combination gdn_chunk_fwd
 * supports.
 */
typedef struct {
  gdn_chunk_desc_t base;
  int64_t H_qk;
  int32_t raw_gates;
  int32_t qk_l2norm;
} gdn_chunk_ex_desc_t;

gdn_status_t gdn_chunk_fwd_ex(const gdn_chunk_ex_desc_t* d, const void* q, const void* k, const void* v,
                              const void* beta, const void* log_alpha, const float* A_log,
                              const float* dt_bias, const int32_t* cu_seqlens, const float* s0, void* o,
                              float* s_final, float* s_ckpt, void* stream);

/*
 * One recurrent (decode) step of the gated delta rule for every live sequence: each
 * sequence keeps a fixed-size state that is updated in place once per token
 * ("From Traditional Attention to hybrid ones", section "vLLM Storage": the state is
 * fixed per live sequence and updated in place; "Attention, Part 4", section 8).
 *
 *   state     [N, H, Dv, Dk]  fp32, read and overwritten in place
 *   q, k      [N, H, Dk]      in_dtype
 *   v         [N, H, Dv]      in_dtype
 *   beta      [N, H]          in_dtype
 *   log_alpha [N, H]          in_dtype
 *   o         [N, H, Dv]      out_dtype, written
 * N >= 0 (N = 0 or H = 0 is a no-op).  Supported: Dk == Dv in {16, 32, 64, 128}.
 */
gdn_status_t gdn_decode_step(int64_t N, int64_t H, int64_t Dk, int64_t Dv, gdn_dtype_t in_dtype,
                             gdn_dtype_t out_dtype, float* state, const void* q, const void* k,
                             const void* v, const void* beta, const void* log_alpha, void* o,
                             void* stream);

/*
 * Serving-side decode: a window of T tokens for each of N live sequences whose states sit
 * in a pool addressed through a slot table.  It covers
 *  - one decode step per sequence on slot-addressed states (T = 1): the state is fixed per
 *    live sequence and updated in place ("From Traditional Attention to hybrid ones",
 *    section "vLLM Storage");
 *  - verification of T draft tokens without touching the state (write_state = 0), then a
 *    commit of the n_commit[n] accepted ones (write_state = 1): speculative decoding needs
 *    the state from before the draft ("Hybrid models: what Gated DeltaNet replaces in the
 *    KV cache", section "What a recurrent state changes for serving"), and a verified but
 *    rejected token is simply never committed;
 *  - value heads sharing query/key heads (H a multiple of H_qk, value head h reads q/k head
 *    h / (H / H_qk));
 *  - KDA's per-channel decay (kda = 1; "From Traditional Attention to hybrid ones",
 *    section 7);
 *  - the layer's q/k normalisation and gate activations fused in ("Attention, Part 4",
 *    section "Where alpha and beta come from": beta = sigmoid(b), log alpha =
 *    -exp(A_log) softplus(a + dt_bias); queries and keys normalised to length 1, here as
 *    x / sqrt(sum x^2 + 1e-6)).
 *
 *   pool      [P, H, Dv, Dk] fp32; row slots[n] is read, and written when write_state = 1
 *   slots     [N] int32 pool row of sequence n, or NULL for row n (then P >= N).  A
 *             negative row or one >= P skips the sequence: nothing is read or written
 *   q, k      [N, T, H_qk, Dk]   in_dtype (raw when qk_l2norm = 1)
 *   v         [N, T, H, Dv]      in_dtype
 *   beta      [N, T, H]          in_dtype (b when raw_gates = 1)
 *   log_alpha [N, T, H], or [N, T, H, Dk] when kda = 1, in_dtype (a when raw_gates = 1)
 *   A_log, dt_bias [H] fp32, required when raw_gates = 1, ignored otherwise
 *   n_commit  [N] int32 tokens to commit (clamped to 0..T), or NULL for all T; used only
 *             when write_state = 1.  The row becomes the state after those tokens; with 0
 *             it is left as it was.
 *   o         [N, T, H, Dv] out_dtype, output of every token of the window, or NULL (then
 *             the kernel stops after the committed tokens).  Rows of skipped sequences are
 *             not written.
 * Token t of a sequence sees the state after its tokens 0..t-1 of this window.  A window
 * that only verifies (write_state = 0, o given) with kda = 0, Dk = 128, T <= 8, q, k
 * aligned to 4 elements and v to 16 bytes is computed as one chunk of the chunkwise form on
 * the fp32 matrix cores; its outputs agree with the token-by-token result to fp32 rounding,
 * not bit for bit.  Other windows run token by token.
 * A commit without outputs (write_state = 1, o = NULL, scalar gate) carries the product of
 * the decays as a running scale applied once at the store; the committed rows agree with
 * the token-by-token result to fp32 rounding, not bit for bit.
 * Supported:
 * Dk == Dv in {16, 32, 64, 128}; raw_gates with kda is NOT_SUPPORTED.  Two sequences
 * must not share a slot in one call (their writes would race).  N = 0, or o = NULL with
 * write_state = 0, is a no-op.
 */
typedef struct {
  int64_t N, H, H_qk, Dk, Dv, T, P;
  gdn_dtype_t in_dtype;  /* dtype of q, k, v, beta, log_alpha */
  gdn_dtype_t out_dtype; /* dtype of o */
  int32_t kda, qk_l2norm, raw_gates, write_state; /* each 0 or 1 */
} gdn_decode_ex_desc_t;

gdn_status_t gdn_decode_ex(const gdn_decode_ex_desc_t* d, float* pool, const int32_t* slots,
                           const void* q, const void* k, const void* v, const void* beta,
                           const void* log_alpha, const float* A_log, const float* dt_bias,
                           const int32_t* n_commit, void* o, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* gdn_status_string(gdn_status_t s);

/* GDN_VERSION of the built library. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
