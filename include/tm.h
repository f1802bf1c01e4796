/*
 * tm.h -- C ABI of the Titans neural long-term memory on MI355X (gfx950).
 *
 * The memory M is a small MLP without biases (depth weight matrices, SiLU
 * between them) whose weights are written at test time.  Sources: the pages
 * on Titans; "Titans, explained" (vibeengines.com) method steps 1-6 and its
 * extremes paragraph; "Attack of the Titans" (synthesis.ai), Technical
 * Details / Parallel training; the titans-pytorch analysis (hysenlabs.com),
 * section "NeuralMemory as a standalone module".
 *
 *   store   : per chunk of b tokens, every token's surprise (the gradient of
 *             ||M(k_t) - v_t||^2 w.r.t. the weights, taken at the weights the
 *             chunk started with) goes into the momentum
 *             S_t = eta_t S_{t-1} - theta_t grad, then M_t = (1 - alpha_t) M_{t-1} + S_t.
 *   retrieve: y = M(q), a forward pass that writes nothing.
 *   forward : store and retrieve together; the queries of chunk c are read
 *             through the weights after chunk c has been written.  This is the
 *             (retrieved, mem_state) call of NeuralMemory.
 *
 * Conventions shared by every call
 *   - All buffers are device memory allocated by the caller; the library
 *     never allocates device memory.  Every call is asynchronous on `stream`
 *     (a hipStream_t; NULL is the null stream) unless stated otherwise.
 *   - Streams of memory: s = batch_index * heads + head; every stream owns an
 *     independent memory (one copy per sequence and head).
 *   - Token arrays k, v, q, y: [batch][n_tokens][heads][dim], contiguous,
 *     16-byte aligned.  k, v, q are bf16 (TM_BF16) or fp32 (TM_F32); y is fp32.
 *   - Gates theta, eta, alpha: [batch][n_tokens][heads] fp32, 4-byte aligned,
 *     values in [0, 1].
 *   - Weights: row-vector convention y = x W; W_l is [d_in][d_out] row-major.
 *     Layer widths: dim -> hidden -> ... -> hidden -> dim with
 *     hidden = dim * expansion (depth 1: one dim x dim matrix).  P is the
 *     total weight count per stream.
 *   - Precision: TM_BF16 rounds weights, activations and theta-scaled deltas
 *     to bf16 for the matrix cores and accumulates in fp32; TM_F32 runs the
 *     same steps with fp32 operands.  M and S are always kept in fp32.
 *   - Errors: every function returns a tm_status and never throws.  All
 *     argument checks run on the host before anything is launched, so a call
 *     that returns an error has not touched the state.  Non-finite values are
 *     not call errors: they set a sticky flag read by tm_state_check.
 *   - Environment (read once per process): TM_LOG=1 prints each new call
 *     shape's configuration and launch plan to stderr, TM_LOG=2 also graph
 *     captures and replays; TM_XCD_STREAMS=0 and TM_FIRST4=0 turn off,
 *     for comparison, the grouping of a stream's workgroups on one XCD and
 *     the 4-wave first-layer workgroups of small widths (results agree to
 *     rounding); TM_STORE_GROUPS=1, 2, 4 or 8 sets the number of batch
 *     groups (tm_store_groups_enable) where the batch divides by it.
 *   - A state blob may be used by one stream at a time; a ctx is immutable
 *     and may be shared between threads.
 */
#ifndef TM_H
#define TM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TM_OK = 0,
    TM_ERR_INVALID = -1,  /* null/misaligned pointer, non-positive or unsupported size */
    TM_ERR_SHAPE = -2,    /* n_tokens not a multiple of the chunk size */
    TM_ERR_DTYPE = -3,    /* unknown tm_dtype */
    TM_ERR_STATE = -4,    /* state not set up (tm_state_init / tm_state_import) for this
                             configuration, batch and heads, or its header does not match */
    TM_ERR_HIP = -5,      /* a HIP runtime call or launch failed */
    TM_ERR_SCRATCH = -6   /* tm_forward_noalloc: the call needs more workspace than the
                             library's scratch array holds */
} tm_status;

typedef enum { TM_F32 = 0, TM_BF16 = 1 } tm_dtype;

/* When a chunk's queries read the memory in tm_forward_ex. */
typedef enum {
    TM_READ_AFTER_WRITE = 0,   /* through the memory after the chunk's write (tm_forward) */
    TM_READ_BEFORE_WRITE = 1,  /* through the memory the chunk started with */
    TM_READ_PER_TOKEN = 2      /* each query through the memory right after its own token's write */
} tm_read;

typedef struct tm_ctx tm_ctx;

/* Memory configuration.  dim: per-head width, a multiple of 32, 32..1024;
 * depth: number of weight matrices, 1..8; expansion: hidden = dim*expansion
 * (>= 1, ignored for depth 1); chunk: tokens per mini-batch b, 1..64 ("Titans,
 * explained" step 6: within a chunk every gradient is taken at the chunk-start
 * weights).  On success *out owns a ctx to release with tm_destroy. */
tm_status tm_create(int dim, int depth, int expansion, int chunk, tm_ctx** out);
void tm_destroy(tm_ctx* ctx);

/* Weights per stream (P). */
size_t tm_param_count(const tm_ctx* ctx);

/* The configuration ctx was created with (depth 1 reports expansion 1).
 * Any output pointer may be null.  TM_ERR_INVALID for a null ctx. */
tm_status tm_config(const tm_ctx* ctx, int* dim, int* depth, int* expansion, int* chunk);

/* Size in bytes of the opaque state blob for batch*heads streams (fp32 M and
 * S, a bf16 copy of M for the matrix cores, and a header).  0 on bad args. */
size_t tm_state_bytes(const tm_ctx* ctx, int batch, int heads);

/* Scratch bytes tm_store / tm_retrieve / tm_forward need for a call of
 * n_tokens tokens per stream (enough for the call's batch groups, see
 * tm_store_groups_enable).  The workspace holds no data between calls. */
size_t tm_workspace_bytes(const tm_ctx* ctx, int batch, int heads, int n_tokens);

/* M = init_weights (device fp32 [heads][P], canonical layer order, broadcast
 * over the batch), S = 0, position = 0, flag cleared.  state: 256-byte
 * aligned, tm_state_bytes(ctx, batch, heads) bytes.  The library records on
 * the host, per state address, the configuration, batch and heads it was set
 * up for (tm_state_import records them too); tm_store, tm_retrieve,
 * tm_forward, tm_forward_ex and tm_state_export refuse, with TM_ERR_STATE and
 * before any launch, a state address that was never set up or was set up
 * for another configuration, batch or head count.  The record is
 * process-wide, so a state may be used with any ctx of its configuration. */
tm_status tm_state_init(const tm_ctx* ctx, void* state, int batch, int heads,
                        const float* init_weights, void* stream);

/* Store n_tokens tokens per stream ("Titans, explained" steps 2-4 in the
 * chunked form of step 6).  n_tokens must be a multiple of the chunk
 * (TM_ERR_SHAPE otherwise); chunk boundaries are counted from the start of
 * every call, so calls must stay chunk-aligned.  n_tokens == 0 is a no-op
 * that returns TM_OK without examining the token and gate pointers. */
tm_status tm_store(const tm_ctx* ctx, void* state, const void* k, const void* v,
                   const float* theta, const float* eta, const float* alpha,
                   int batch, int heads, int n_tokens, tm_dtype dtype,
                   void* workspace, void* stream);

/* y = M(q) for every query through the current weights (step 5).  The state
 * is not written.  Any n_tokens >= 0 (0: a no-op, as for tm_store).  With
 * bf16 operands, depth 2, dim <= 128 and a hidden width that is a multiple
 * of 64, both layers run in one launch and the workspace is not touched;
 * otherwise passes of up to 2048 rows per stream go layer by layer through
 * it. */
tm_status tm_retrieve(const tm_ctx* ctx, const void* state, const void* q, float* y,
                      int batch, int heads, int n_tokens, tm_dtype dtype,
                      void* workspace, void* stream);

/* Store and retrieve: for each chunk c, store chunk c, then read chunk c's
 * queries through the written memory.  Equivalent to alternating tm_store and
 * tm_retrieve chunk by chunk.  n_tokens == 0 is a no-op, as for tm_store. */
tm_status tm_forward(const tm_ctx* ctx, void* state, const void* k, const void* v,
                     const void* q, const float* theta, const float* eta,
                     const float* alpha, float* y, int batch, int heads,
                     int n_tokens, tm_dtype dtype, void* workspace, void* stream);

/* The backward through the store: gradients of an outer loss through one
 * call of tm_forward (read = TM_READ_AFTER_WRITE) or tm_forward_ex with
 * TM_READ_BEFORE_WRITE, for training a model around the memory
 * ("titans-pytorch analysis", Editorial conclusion: the loss must
 * backpropagate through the memory state; "Titans, explained", step 6: the
 * chunked form is what makes the memory trainable in parallel).  For
 *     L = sum(dy * y) + <dM, M_after> + <dS, S_after>,
 * with y and the state after the call as that call produces them from
 * `state` (the state blob as it was BEFORE the call; read only) and the
 * same k, v, q and gates, it writes
 *     dk, dv, dq = dL/dk, dL/dv, dL/dq   ([batch][n_tokens][heads][dim] fp32),
 *     dtheta, deta, dalpha               ([batch][n_tokens][heads] fp32),
 * and replaces dstate -- on entry (dM, dS), the gradient with respect to
 * the state after the call, canonical fp32 [batch*heads][2P] as
 * tm_state_export lays it out (zeros if the loss does not see that state) --
 * with the gradient with respect to the state before the call, so that a
 * stream of calls is differentiated by calling tm_backward on them in
 * reverse order with one dstate buffer.  dy is fp32 in the token layout.
 * The call recomputes the forward from `state` (every chunk-start state is
 * kept in the workspace) and sweeps the chunks in reverse; all its
 * arithmetic is fp32, whatever dtype k, v, q have (the gradient of the
 * exact function at the given inputs).  workspace: tm_backward_workspace_bytes
 * bytes, 256-byte aligned.  TM_READ_PER_TOKEN gives TM_ERR_INVALID.  Errors
 * as for tm_forward (dstate null or not 16-byte aligned: TM_ERR_INVALID);
 * n_tokens == 0 leaves dstate as it is (the call is the identity). */
tm_status tm_backward(const tm_ctx* ctx, const void* state, const void* k, const void* v,
                      const void* q, const float* theta, const float* eta, const float* alpha,
                      const float* dy, float* dstate, float* dk, float* dv, float* dq,
                      float* dtheta, float* deta, float* dalpha, int batch, int heads,
                      int n_tokens, tm_dtype dtype, tm_read read, void* workspace, void* stream);

/* Workspace bytes of tm_backward for a call of n_tokens per stream: the
 * chunk-start states (n_tokens / chunk + 1 of them, 8P bytes per stream
 * each), the key rows' activations per chunk and the sweep's scratch. */
size_t tm_backward_workspace_bytes(const tm_ctx* ctx, int batch, int heads, int n_tokens);

/* tm_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results as tm_forward, bitwise, but the workspace is
 * a scratch array the library holds in device memory, 32 MiB per GPU, kept
 * from the first call on that GPU until the process ends; the caller passes
 * only the state, inputs and outputs.  A call whose tm_workspace_bytes
 * exceeds 32 MiB (e.g. more than 2 streams of 1024 tokens at dim 384, chunk
 * 64) returns TM_ERR_SCRATCH before any launch.  No hipMalloc, hipFree or
 * other allocating call is made, and calls are launched directly (no graph
 * replay).  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (on different streams, or from several threads) race and must
 * be serialised by the caller.  Everything else as for tm_forward. */
tm_status tm_forward_noalloc(const tm_ctx* ctx, void* state, const void* k, const void* v,
                             const void* q, const float* theta, const float* eta,
                             const float* alpha, float* y, int batch, int heads,
                             int n_tokens, tm_dtype dtype, void* stream);

/* tm_forward with the read order chosen.  TM_READ_BEFORE_WRITE: for each
 * chunk c, chunk c's queries read the memory chunk c started with, then chunk
 * c is stored (the memory-as-context order: "Attack of the Titans", memory as
 * a context, and "Titans, explained" step 8, where a segment's tokens query
 * the memory before it is updated).  Equivalent to alternating tm_retrieve
 * and tm_store chunk by chunk; the state it leaves is bitwise that of
 * tm_forward.  TM_READ_PER_TOKEN: query t (of the chunk holding token t)
 * reads the memory as token t's write left it, within the chunk too: the
 * gradients stay at the chunk-start weights, but the momentum and forgetting
 * have advanced token by token ("Attack of the Titans", the long-term memory
 * section: a linear-attention output is a lookup in a memory updated at
 * every step; Technical Details / Parallel training for the chunking).  It
 * is computed by the dual form: the chunk start's products of the queries
 * plus a causal b x b correction per layer, one extra launch per layer and
 * chunk (and one per call for layer 0's scores).  The last query of each
 * chunk reads what TM_READ_AFTER_WRITE reads.  An unknown read
 * value gives TM_ERR_INVALID; everything else as for tm_forward. */
tm_status tm_forward_ex(const tm_ctx* ctx, void* state, const void* k, const void* v,
                        const void* q, const float* theta, const float* eta,
                        const float* alpha, float* y, int batch, int heads,
                        int n_tokens, tm_dtype dtype, tm_read read, void* workspace,
                        void* stream);

/* The memory's input side ("Titans, explained" steps 1, 4 and 5), from the
 * tokens' model vectors to the keys, values, queries and gates that
 * tm_store / tm_forward take:
 *   p_i = x W_i^T for i = key, value, query (W_i: heads*dim output rows of
 *   model_dim inputs, PyTorch's Linear layout), then a causal depthwise
 *   convolution of every channel over the last conv_len tokens (tap j weighs
 *   the projection j tokens back; no bias, no activation), then keys and
 *   queries l2-normalised per head (norm clamped below at 1e-12); the gates
 *   sigmoid(x w_g + b_g) per head for g = theta, eta, alpha.
 * x: [batch][n_tokens][model_dim] of dtype, 16-byte aligned, model_dim a
 *   multiple of 32.  w_kvq: [3][heads*dim][model_dim] of dtype, 16-byte
 *   aligned.  conv: [3][heads*dim][conv_len] fp32, conv_len 1..4.  w_gate:
 *   [3][heads][model_dim] fp32, 16-byte aligned.  gate_bias: [3] fp32
 *   (device).
 * history: [batch][conv_len-1][3][heads*dim] fp32, the projections of the
 *   stream's last conv_len-1 tokens before this call, oldest first (zeros at
 *   a stream's start); read, then overwritten with those of this call's last
 *   tokens, so consecutive calls equal one long call.  Ignored (may be null)
 *   for conv_len 1.
 * k, v, q: [batch][n_tokens][heads][dim] of dtype; theta, eta, alpha:
 *   [batch][n_tokens][heads] fp32.  Every pointer is a device pointer owned by
 *   the caller.  n_tokens == 0 is a no-op.  Bad sizes, null or misaligned
 *   pointers give TM_ERR_INVALID, a bad dtype TM_ERR_DTYPE, all before any
 *   launch.  Asynchronous on `stream` (two launches; graph replay as for the
 *   calls below). */
tm_status tm_project(const tm_ctx* ctx, const void* x, int model_dim, const void* w_kvq,
                     const float* conv, int conv_len, const float* w_gate,
                     const float* gate_bias, float* history, void* k, void* v, void* q,
                     float* theta, float* eta, float* alpha, int batch, int heads,
                     int n_tokens, tm_dtype dtype, void* stream);

/* Memory-side wiring of memory as a context (MAC: "Titans, explained" step
 * 8; "Attack of the Titans", Technical Details, memory as a context).  A
 * segment's tokens query the memory (tm_retrieve through the memory before
 * the segment is written); the recalled vectors sit between the persistent
 * tokens and the segment in the window attention runs over; the attention
 * output y is written into the memory (tm_project of y, then tm_store) and
 * gates the final output through the memory's read of it (tm_retrieve of y's
 * queries after the write).  Attention and the persistent tokens' values are
 * the caller's.  These two calls are the wiring the memory's own calls do
 * not cover; both only move and multiply elements.
 *
 * tm_mac_window: window [batch][n_persist + 2 seg_len][model_dim] (dtype) =
 *   persistent [n_persist][model_dim] (dtype; shared over the batch), then
 *   recalled [batch][seg_len][model_dim] (fp32, the memory's read of the
 *   segment, rounded to dtype to nearest even), then segment
 *   [batch][seg_len][model_dim] (dtype).  n_persist may be 0 (persistent
 *   may then be null).
 * tm_mac_gate: out [batch][seg_len][model_dim] fp32 = y * mem element-wise,
 *   y the attention output for the segment's positions (dtype), mem the
 *   memory's fp32 read of y.  The pages fix no form for this gate; the
 *   element-wise product of the output and the memory's read of it is the
 *   plainest.
 * model_dim: a positive multiple of 32; seg_len > 0, batch > 0; pointers
 * 16-byte aligned (else TM_ERR_INVALID, bad dtype TM_ERR_DTYPE), all on the
 * host before any launch.  Asynchronous on `stream`; one launch each. */
tm_status tm_mac_window(const void* persistent, int n_persist, const float* recalled,
                        const void* segment, void* window, int batch, int seg_len, int model_dim,
                        tm_dtype dtype, void* stream);
tm_status tm_mac_gate(const void* y, const float* mem, float* out, int batch, int seg_len,
                      int model_dim, tm_dtype dtype, void* stream);

/* Canonical fp32 copy of the state: dst is [batch*heads][2P], per stream
 * M_1..M_L then S_1..S_L, each W_l row-major [d_in][d_out]. */
tm_status tm_state_export(const tm_ctx* ctx, const void* state, int batch, int heads,
                          float* dst, void* stream);

/* Inverse of tm_state_export (rebuilds the bf16 copy, position = 0, flag
 * cleared). */
tm_status tm_state_import(const tm_ctx* ctx, void* state, int batch, int heads,
                          const float* src, void* stream);

/* Synchronous: waits for `stream`, then checks the state header against the
 * ctx, batch and heads (TM_ERR_STATE on mismatch) and reports the sticky
 * non-finite flag and the number of tokens stored since init/import. */
tm_status tm_state_check(const tm_ctx* ctx, const void* state, int batch, int heads,
                         int* nonfinite, long long* position, void* stream);

const char* tm_status_str(tm_status status);

/* Graph replay (on by default, process-wide).  A tm_state_init / tm_store /
 * tm_retrieve / tm_forward / tm_forward_ex / tm_project call whose device,
 * pointers and sizes repeat an earlier call's is captured once into a HIP
 * graph (on a private stream of the ctx) and from then on replayed on the
 * caller's stream, which removes most of the per-kernel launch cost of the
 * chunk loop.  Each ctx keeps its 16 most recent call shapes.  on = 0
 * launches every call directly. */
tm_status tm_graphs_enable(int on);

/* Placement of W_1's update for depth-2 memories; the results are bitwise
 * identical either way (the same products, in the same order).  With
 * on = 1 (the default), when the step launch leaves compute units free, W_1's
 * update runs in workgroups of its own beside the first-layer blocks, and M_1
 * alternates with a second buffer in the workspace over a call's updates; the
 * state holds the final M_1 when the call ends.  on = 0 keeps it in the
 * first-layer blocks, in place.  fp32 calls always update W_1 in place.
 * Process-wide; calls captured into graphs before a change keep the setting
 * they were captured with. */
tm_status tm_w1_split_enable(int on);

/* Batch groups of the chunk loop (tm_store, tm_forward, tm_forward_ex); the
 * results are bitwise identical either way.  With on = 1 (the default), a
 * call of at least 16 streams with an even batch runs its two batch halves
 * as two independent chunk chains, one on the caller's stream and one on a
 * second stream of the ctx (per device and host thread, default priority,
 * forked from and joined back to the caller's stream, so the call stays
 * ordered on `stream`), and each half uses its own half of the workspace:
 * one chain's launches fill the compute units the other's leave idle.
 * on = 0 runs one chain.  tm_forward_noalloc always runs one chain.
 * Process-wide; the setting is part of a call shape's graph key, so a change
 * captures a graph of its own. */
tm_status tm_store_groups_enable(int on);

/* Instrumentation for measuring kernels in place (not part of the method).
 * Kernel classes: 0 coefficient scan (and key transpose), 1 chunk forward
 * products of layers 1.., 2 chunk backward products, 3 none (kept for
 * numbering: the update of layers 1.. runs inside the first-layer step
 * launch), 4 first-layer step (the first layer's update, its in-place
 * backward, and its forward, with the other layers' updates riding in the
 * same launch), 5 the per-token read's products,
 * 6 the input side's projection kernel (tm_project; its history kernel is
 * not timed), 7 the memory-as-context window and gate kernels
 * (tm_mac_window, tm_mac_gate).  While bit c of
 * class_mask is set, every launch of class c is bracketed by a pair of HIP
 * events recorded on its launch stream (mask 0 turns timing off).
 * tm_timing_read waits for the recorded launches and returns, for one class,
 * the summed duration in milliseconds and the number of launches since its
 * last read, then forgets them.  Process-wide. */
tm_status tm_timing_enable(int class_mask);
tm_status tm_timing_read(int kernel_class, double* total_ms, long long* launches);

#ifdef __cplusplus
}
#endif

#endif /* TM_H */
