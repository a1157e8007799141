/*
 * kda.h -- C ABI of the Kimi Delta Attention (KDA) core for AMD Instinct
 * MI355X (gfx950).
 *
 * KDA is a gated delta-rule recurrence whose decay is one value per key
 * channel (the nnterp Kimi-Linear page, KDA description).  Per sequence and
 * head, with state S[dk][dv] (rows are key channels, columns value channels):
 *
 *     k_hat = k / sqrt(sum(k^2) + 1e-6),  q_hat = scale * q / sqrt(sum(q^2) + 1e-6)
 *     S     = diag(exp(g_t)) S
 *     S     = S + beta_t k_hat (v_t - S^T k_hat)^T
 *     o_t   = S^T q_hat
 *
 * The normalisation (eps inside the root), the query-only scale 1/sqrt(dk)
 * and the read-after-update order follow the Ascend model file (its
 * `_l2_normalize` helper and its chunked fallback `_torch_chunk_kda`).  Each
 * kernel takes (q, k, v, g, beta, initial_state) and returns (out,
 * final_state), the interface the nnterp page gives for the chunked prompt
 * kernel and the token-by-token decode kernel.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *     and densely packed, innermost dimension last.  The library allocates
 *     nothing, keeps no state between calls (kda_chunk_fwd_noalloc's device
 *     array aside) and never synchronises `stream`: work is enqueued on it and
 *     the call returns.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and leave every output untouched.  KDA_ERR_HIP reports a failed launch.
 *     kda_last_error() gives a human-readable detail for the calling thread.
 *   - NaN or Inf inputs propagate into the outputs; they are not checked.
 *   - Alignment (checked on the host, KDA_ERR_BAD_SHAPE otherwise): q, k, v,
 *     out, g or the raw gate when it has one value per key channel, every
 *     state buffer, pool and workspace, and the output gate and norm weight
 *     must be 16-byte aligned (the kernels move them in 16-byte pieces); beta
 *     and a per-head g need their element's alignment (4 bytes for float32, 2
 *     for a bf16 raw input) and the int32 index arrays 4 bytes.  Whole rows
 *     sliced from a PyTorch allocation meet this.
 *   - The numeric domain of the chunked kernel: g must be finite and <= 0;
 *     any such g is handled, however strong the decay.  The chunk form needs
 *     exp(G_r - G_i) for i <= r (G: cumulative sum of g inside a chunk of 64
 *     tokens, counted from the start of each sequence).  A chunk and head
 *     whose partial sums of g stay within 60 of a reference token (with bf16
 *     q/k/v and dk = 128: the chunk's token 31; otherwise the start of each
 *     aligned 16-token block) factors it through that token onto MFMA; one
 *     whose decay is steeper takes an exact path that carries
 *     k_i exp(G_r - G_i) down the rows as products of exp(g) <= 1 (more
 *     work per chunk than the factored path).  Decode has no such split.
 *   - With bf16 q/k/v and dk = 128 the chunk pass carries the state and the
 *     per-chunk operands through fp16 (11 significant bits, largest finite
 *     value 65504): |k|, |v| and the entries of the state must stay well
 *     below 1e4 (with qk_l2norm = 0 also |q|).  Values beyond it overflow to
 *     Inf in the result.
 *   - Setting the environment variable KDA_DEBUG=1 makes every call wait for
 *     its own kernels and report their errors (this synchronises the stream).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 6

typedef enum kda_status {
    KDA_OK = 0,
    KDA_ERR_NULL_POINTER = 1, /* a required pointer is NULL                      */
    KDA_ERR_BAD_SHAPE = 2,    /* negative or inconsistent sizes                  */
    KDA_ERR_UNSUPPORTED = 3,  /* valid but not implemented (head size, dtype...) */
    KDA_ERR_WORKSPACE = 4,    /* workspace smaller than the queried size         */
    KDA_ERR_HIP = 5           /* a HIP launch or runtime call failed             */
} kda_status_t;

typedef enum kda_dtype {
    KDA_F32 = 0,  /* IEEE binary32                              */
    KDA_BF16 = 1  /* bfloat16 (upper 16 bits of a binary32)     */
} kda_dtype_t;

/* Problem description shared by both entry points. */
typedef struct kda_problem {
    int64_t total_tokens; /* T: rows of q/k/v/g/beta/out.  Prefill: == cu_seqlens[num_seqs].
                             Decode: == num_seqs (one token per sequence).              */
    int32_t num_seqs;     /* N >= 0.  N == 0 or T == 0 is a no-op that returns KDA_OK.    */
    int32_t num_heads;    /* H >= 1                                                       */
    int32_t head_k;       /* dk; 64 or 128                                                */
    int32_t head_v;       /* dv; must equal dk                                            */
    int32_t qkv_dtype;    /* kda_dtype_t of q, k and v                                    */
    int32_t out_dtype;    /* kda_dtype_t of out                                           */
    float scale;          /* multiplies q after its L2 norm; 1/sqrt(dk) by convention     */
    int32_t qk_l2norm;    /* 1: L2-normalise q and k inside the kernel; 0: use as given   */
    int32_t chunk_size;   /* prefill chunk length; 64 only (0 selects 64)                 */
    int32_t gate_per_head; /* 0: g (or the raw gate) has one value per key channel,
                              [rows, H, dk]; 1: one value per head, [rows, H], the same
                              decay for every channel (the Gated DeltaNet case); the gated
                              calls then take dt_bias as [H]                               */
    int32_t state_layout; /* KDA_STATE_DK_DV (0): every state block (initial, final, decode
                              state, pool slot) is S[dk][dv], dv contiguous; KDA_STATE_DV_DK
                              (1): the transpose S^T[dv][dk], dk contiguous, the layout of
                              the Ascend model file's recurrent cache (`_prefill_flash_kda`
                              reads and scatters it per request).  Same values either way;
                              only the element order within a block changes.  ABI 5.     */
} kda_problem_t;

#define KDA_STATE_DK_DV 0
#define KDA_STATE_DV_DK 1

/*
 * Gate parameters of the *_gated entry points, which take the raw gate and
 * raw beta projections and activate them inside the kernels.  The activation
 * is that of the Ascend model file's gated paths (`_prefill_torch_kda`, the
 * decode branch of the attention forward, and its `_softplus`): for token t,
 * head h, key channel c, with raw gate x and raw beta y,
 *
 *     u    = x[t][h][c] + dt_bias[h][c]
 *     g    = -exp(a_log[h]) * softplus(u)                (has_lower_bound == 0)
 *     g    = lower_bound * sigmoid(exp(a_log[h]) * u)    (has_lower_bound == 1)
 *     beta = sigmoid(y[t][h])
 *
 * with softplus(u) = max(u, 0) + log(1 + exp(-|u|)) and sigmoid(z) =
 * 1 / (1 + exp(-z)), evaluated in float32.  The activated g must meet the
 * numeric domain stated above.
 */
typedef struct kda_gate {
    const float *a_log;      /* [H] float32 (device): the gate scale is exp(a_log[h])   */
    const float *dt_bias;    /* [H, dk] float32 (device); [H] with gate_per_head        */
    int32_t has_lower_bound; /* 0: softplus gate; 1: bounded sigmoid gate               */
    float lower_bound;       /* used when has_lower_bound == 1: finite and <= 0        */
} kda_gate_t;

/* ABI revision of the loaded library; compare with KDA_ABI_VERSION. */
int kda_abi_version(void);

/* Static text for a status code. */
const char *kda_status_string(kda_status_t status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char *kda_last_error(void);

/*
 * Bytes of device workspace kda_chunk_fwd needs for this problem (0 if none).
 * Returns 0 as well for an invalid problem; kda_chunk_fwd then reports why.
 *
 * bf16 q/k/v with dk = dv = 128 runs in two passes: every (chunk, head) pair
 * is prepared independently and its state-independent operands are stored in
 * the workspace, then a short scan carries the state across chunks.  The size
 * is 4 * (2N + 1) bytes (chunk offsets and the order the scan takes the
 * sequences in) rounded up to a multiple of 256, plus
 * 61952 bytes per (chunk, head) for ceil(T / 64) + N chunks (about 0.95 KiB
 * per token and head).  Other configurations keep everything on chip and need 0.
 */
size_t kda_chunk_fwd_workspace_bytes(const kda_problem_t *problem);

/*
 * Chunked prefill over packed variable-length sequences.
 *
 * Defined by the chunk algorithm of the Ascend model file (`_torch_chunk_kda`):
 * tokens are cut into chunks of `chunk_size` per sequence, never straddling a
 * sequence boundary; inside a chunk the delta rule is solved as one unit
 * lower-triangular system, and the state is carried from chunk to chunk.  The
 * result equals the token-by-token recurrence above up to rounding.  Varlen
 * packing follows that file's per-request loop (`_prefill_flash_kda`): the
 * sequences are concatenated and cu_seqlens marks their boundaries; each
 * sequence starts from its own initial state.  A tail chunk shorter than
 * chunk_size behaves as if padded with no-op tokens (k = v = g = beta = 0).
 *
 *   q, k           [T, H, dk]  qkv_dtype
 *   v              [T, H, dv]  qkv_dtype
 *   g              [T, H, dk]  float32, log-decay per key channel (<= 0); [T, H] with
 *                  problem->gate_per_head
 *   beta           [T, H]      float32, in [0, 1]
 *   cu_seqlens     [N + 1]     int32 (device): 0 = cu[0] <= cu[1] <= ... <= cu[N] = T.
 *                  Sequence n is rows cu[n] .. cu[n+1]-1.  Zero-length sequences are
 *                  allowed (their final state is their initial state).  Entries outside
 *                  [0, T] or decreasing pairs make that sequence empty; they never cause
 *                  an out-of-bounds access.
 *   initial_state  [N, H, dk, dv] float32 ([N, H, dv, dk] with KDA_STATE_DV_DK), or NULL for zeros
 *   out            [T, H, dv]  out_dtype (written)
 *   final_state    [N, H, dk, dv] float32 (layout as initial_state; written), or NULL to skip.  May alias
 *                  initial_state exactly (same pointer); partial overlap is undefined.
 *   workspace      device buffer of at least kda_chunk_fwd_workspace_bytes(problem)
 *                  bytes, or NULL when that is 0.  Contents need not be initialised.
 *   stream         a hipStream_t (NULL: the default stream)
 */
kda_status_t kda_chunk_fwd(const kda_problem_t *problem, const void *q, const void *k,
                           const void *v, const float *g, const float *beta,
                           const int32_t *cu_seqlens, const float *initial_state, void *out,
                           float *final_state, void *workspace, size_t workspace_bytes,
                           void *stream);

/*
 * kda_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same computation, arguments and results
 * as kda_chunk_fwd (the same kernels run); the caller still provides q, k,
 * v, g, beta, cu_seqlens, the states and out.
 *
 * The two-pass path's workspace is a device array inside the library,
 * KDA_NOALLOC_SCRATCH_BYTES (128 MiB) on every GPU the library runs on, held
 * until the process ends.  A problem with kda_chunk_fwd_workspace_bytes(problem)
 * above that ((ceil(T / 64) + N) * H beyond about 2,166: one sequence of up to
 * 4,224 tokens at H = 32, or 34,560 at H = 4, fits) fails with
 * KDA_ERR_UNSUPPORTED before anything is enqueued.  No call allocates or frees memory; the first call on
 * each GPU looks up the array's device address (hipGetSymbolAddress), and a
 * failure there is KDA_ERR_HIP.  Nothing in the array needs to start at zero:
 * each call writes what it reads.  Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (two streams, or two host
 * threads) race and give undefined results: serialise them.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
kda_status_t kda_chunk_fwd_noalloc(const kda_problem_t *problem, const void *q, const void *k,
                                   const void *v, const float *g, const float *beta,
                                   const int32_t *cu_seqlens, const float *initial_state, void *out,
                                   float *final_state, void *stream);

/*
 * kda_chunk_fwd with the gate activation fused in: raw_g [T, H, dk] and
 * raw_beta [T, H] are in qkv_dtype (what the gate projections produce) and
 * are turned into g and beta as described at kda_gate_t; gate, a_log and
 * dt_bias must be non-NULL.  Everything else, the workspace included, is as
 * for kda_chunk_fwd.
 */
kda_status_t kda_chunk_fwd_gated(const kda_problem_t *problem, const kda_gate_t *gate, const void *q,
                                 const void *k, const void *v, const void *raw_g, const void *raw_beta,
                                 const int32_t *cu_seqlens, const float *initial_state, void *out,
                                 float *final_state, void *workspace, size_t workspace_bytes,
                                 void *stream);

/*
 * Short causal convolution fused into the prefill.  The Ascend model file's
 * `_forward_core` runs `KimiShortConvolution` over the fused q/k/v
 * projection before the core; kda_chunk_fwd_conv takes that projection
 * before the convolution and applies the convolution (with y * sigmoid(y)
 * when silu = 1) inside the prefill's loads of q, k and v, so the convolved
 * q/k/v are never written to memory.  The convolution is the one
 * kda_short_conv computes (same taps, same state convention, same bf16
 * rounding of its output), so this call's results equal kda_short_conv
 * followed by kda_chunk_fwd on the split output.
 *
 *   kernel_size  K, 1 to 4
 *   silu         1: y * sigmoid(y) after the convolution; 0: none
 *   weight       [K, 3 H d] bf16 (device, 16-byte aligned), tap-major as for
 *                kda_short_conv; channels [0, H d) are q's, then k's, then v's
 *   state_in     [N, K - 1, 3 H d] bf16 (device, 16-byte aligned): each
 *                request's last K - 1 inputs before this call, oldest first;
 *                NULL for zeros
 *   state_out    [N, K - 1, 3 H d] bf16 (device, 16-byte aligned), written
 *                with each request's last K - 1 inputs (its old state followed
 *                by its inputs when it is shorter), each slice after the
 *                call's last read of it; NULL to skip; may equal state_in
 */
typedef struct kda_conv {
    int32_t kernel_size;
    int32_t silu;
    const void *weight;
    const void *state_in;
    void *state_out;
} kda_conv_t;

/*
 * kda_chunk_fwd (gate NULL: g and beta activated, float32) or
 * kda_chunk_fwd_gated (gate non-NULL: raw projections) with the short
 * convolution fused in (kda_conv_t above).
 *
 *   qkv     [T, 3, H, d] bf16: the fused projection before the convolution
 *           (q = qkv[:, 0], k = qkv[:, 1], v = qkv[:, 2]), 16-byte aligned
 *   problem qkv_dtype KDA_BF16 and head_k = head_v = 128 (the Kimi-Linear
 *           shape); anything else is KDA_ERR_UNSUPPORTED (use kda_short_conv
 *           and then kda_chunk_fwd)
 * g, beta, cu_seqlens, the states, out and the workspace (of
 * kda_chunk_fwd_workspace_bytes bytes) are as for kda_chunk_fwd.  Errors are
 * found on the host before any launch.
 */
kda_status_t kda_chunk_fwd_conv(const kda_problem_t *problem, const kda_gate_t *gate, const kda_conv_t *conv,
                                const void *qkv, const void *g, const void *beta, const int32_t *cu_seqlens,
                                const float *initial_state, void *out, float *final_state, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * One decode step: every sequence advances by exactly one token, and its state
 * is updated IN PLACE.  This is the token-by-token form (the nnterp page's
 * decode kernel; the Ascend model file's decode paths update the recurrent
 * cache in place with a per-channel decay `gk`).
 *
 *   q, k    [N, H, dk]  qkv_dtype     (problem->total_tokens must equal N)
 *   v       [N, H, dv]  qkv_dtype
 *   g       [N, H, dk]  float32 ([N, H] with problem->gate_per_head)
 *   beta    [N, H]      float32
 *   state   [N, H, dk, dv] float32 ([N, H, dv, dk] with KDA_STATE_DV_DK), read and overwritten
 *   out     [N, H, dv]  out_dtype (written)
 *   stream  a hipStream_t (NULL: the default stream)
 */
kda_status_t kda_recurrent_step(const kda_problem_t *problem, const void *q, const void *k,
                                const void *v, const float *g, const float *beta, float *state,
                                void *out, void *stream);

/*
 * kda_recurrent_step with the gate activation fused in: raw_g [N, H, dk] and
 * raw_beta [N, H] in qkv_dtype, activated as described at kda_gate_t.
 */
kda_status_t kda_recurrent_step_gated(const kda_problem_t *problem, const kda_gate_t *gate,
                                      const void *q, const void *k, const void *v, const void *raw_g,
                                      const void *raw_beta, float *state, void *out, void *stream);

/*
 * State pool.  The two calls below keep recurrent states in a pool of slots,
 * the way the Ascend model file keeps its recurrent cache: the prefill branch
 * scatters each request's final state into its cache block
 * (`update_mamba_cache`), and the decode branches hand the kernels one state
 * index per token (`ssm_state_indices`, checked against the fixed "Verify"
 * width) and the number of accepted tokens (`num_accepted_tokens`).
 *
 *   state_pool   [num_slots, H, dk, dv] float32 (device; [num_slots, H, dv, dk] with
 *                KDA_STATE_DV_DK), read and written.
 *   A slot index outside [0, num_slots) names no slot: such a state reads as
 *   zero and is not written.  Slots named by different sequences of one call
 *   must be distinct (otherwise the result is undefined).
 */

/*
 * kda_chunk_fwd with the states in a pool: sequence n starts from slot
 * state_slots[n] and its final state is written back to that slot.
 * gate NULL: g [T, H, dk] and beta [T, H] are float32 as for kda_chunk_fwd;
 * otherwise they are the raw projections and are activated as for
 * kda_chunk_fwd_gated.  state_slots [N] int32 (device).  Everything else is
 * as for kda_chunk_fwd, workspace included.
 */
kda_status_t kda_chunk_fwd_pooled(const kda_problem_t *problem, const kda_gate_t *gate, const void *q,
                                  const void *k, const void *v, const void *g, const void *beta,
                                  const int32_t *cu_seqlens, float *state_pool, int32_t num_slots,
                                  const int32_t *state_slots, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Multi-token verify decode over a state pool.  Every sequence advances by
 * exactly `width` tokens, token by token as kda_recurrent_step does.  The
 * pages fix only the interface (one state slot per token, the accepted-token
 * counts); the meaning taken here:
 *   - sequence n starts from the state in slot idx[a - 1], with
 *     idx = state_indices + n * width and a = num_accepted[n] clamped to
 *     [1, width] (a = 1 when num_accepted is NULL);
 *   - after its token t it writes the state to slot idx[t].
 * The starting state is read in full before anything is written, so idx[a-1]
 * may also be a destination.  width = 1 with num_accepted NULL is the plain
 * decode step with the state in slot idx[0].
 *
 *   problem->total_tokens must equal num_seqs * width.
 *   q, k          [N * width, H, dk]  qkv_dtype; sequence n's tokens are rows
 *                 n*width .. n*width + width - 1
 *   v             [N * width, H, dv]  qkv_dtype
 *   g, beta       gate NULL: [N * width, H, dk] and [N * width, H] float32;
 *                 otherwise the raw projections in qkv_dtype, activated as
 *                 described at kda_gate_t
 *   state_indices [N, width] int32 (device)
 *   num_accepted  [N] int32 (device), or NULL
 *   out           [N * width, H, dv]  out_dtype (written)
 */
kda_status_t kda_recurrent_verify(const kda_problem_t *problem, int32_t width, const kda_gate_t *gate,
                                  const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, float *state_pool, int32_t num_slots,
                                  const int32_t *state_indices, const int32_t *num_accepted, void *out,
                                  void *stream);

/*
 * kda_recurrent_verify with the layer's output epilogue fused, as
 * kda_recurrent_step_normed does for one token: the workgroup of a (sequence,
 * head) holds each token's whole output row, and writes
 *     out = o / sqrt(mean(o^2) + norm_eps) * norm_weight * sigmoid(out_gate)
 * in place of o, which never reaches memory (the Ascend model file's
 * `_project_out` norm and gate).  The states written are those of
 * kda_recurrent_verify, bit for bit.
 *
 *   out_gate    [N * width, H, dv] in qkv_dtype (device, 16-byte aligned)
 *   norm_weight [dv] float32 (device, 16-byte aligned); norm_eps finite, >= 0
 * Everything else as kda_recurrent_verify.
 */
kda_status_t kda_recurrent_verify_normed(const kda_problem_t *problem, int32_t width, const kda_gate_t *gate,
                                         const void *q, const void *k, const void *v, const void *g,
                                         const void *beta, float *state_pool, int32_t num_slots,
                                         const int32_t *state_indices, const int32_t *num_accepted,
                                         const void *out_gate, const float *norm_weight, float norm_eps,
                                         void *out, void *stream);

/*
 * kda_recurrent_step (or, with gate non-NULL, kda_recurrent_step_gated) with
 * the layer's output epilogue fused: the workgroup of a (sequence, head) holds
 * its whole output row, so
 *     out = o / sqrt(mean(o^2) + norm_eps) * norm_weight * sigmoid(out_gate)
 * is written in place of o, which never reaches memory (the Ascend model
 * file's `_project_out` norm and gate; see kda_gated_rmsnorm).
 *
 *   gate        NULL: g and beta are activated float32 values; otherwise the raw
 *               projections as for kda_recurrent_step_gated
 *   out_gate    [N, H, dv] in qkv_dtype (device)
 *   norm_weight [dv] float32 (device); norm_eps finite, >= 0
 * Everything else as kda_recurrent_step.
 */
kda_status_t kda_recurrent_step_normed(const kda_problem_t *problem, const kda_gate_t *gate, const void *q,
                                      const void *k, const void *v, const void *g, const void *beta,
                                      float *state, const void *out_gate, const float *norm_weight,
                                      float norm_eps, void *out, void *stream);

/*
 * Short causal convolution before the core (the Ascend model file's
 * `KimiShortConvolution`, run on the fused q/k/v projection): a depthwise
 * causal convolution, one filter of kernel_size taps per channel, per request,
 * with a conv-state cache holding each request's last kernel_size - 1 inputs.
 * With the window w = [state (oldest first), the request's inputs],
 *     y[t, c] = sum_{j < K} weight[j, c] * w[t + j, c]     (the last tap meets the current input)
 * then, with silu = 1, y * sigmoid(y).  The request's last K - 1 inputs (its
 * state followed by its inputs when it is shorter) become its final state; an
 * empty request keeps its state.  Decode is the same call with one token per
 * request (total_tokens == num_seqs).
 *
 *   num_seqs, total_tokens   N >= 0 requests, T >= 0 tokens (N = 0: no-op)
 *   channels      C, a positive multiple of 8 (e.g. 3 * H * d for fused q/k/v)
 *   kernel_size   K, 1 to 4
 *   dtype         kda_dtype_t of x, weight, the states and y
 *   silu          1: apply y * sigmoid(y); 0: none (the page passes the operator
 *                 no activation argument, so both are offered)
 *   x             [T, C] device; cu_seqlens [N + 1] int32 device, 0 = cu[0] <= ... <= cu[N] = T
 *   weight        [K, C] device (tap-major, the layout the page builds for its operator)
 *   state_in      [N, K - 1, C] device, or NULL for zeros
 *   state_out     [N, K - 1, C] device (written), or NULL to skip; may be state_in
 *                 (in place: every request reads its old state before its new state
 *                 is written; each request then runs on one thread per 8 channels,
 *                 token after token, which suits decode and short requests)
 *   y             [T, C] device (written)
 * All device pointers 16-byte aligned (KDA_ERR_BAD_SHAPE otherwise); T <= 2^27 - 1024,
 * N <= 2^23, C <= 2^26 (the launch grid's limits).  Errors are found on the host
 * before any launch.
 */
kda_status_t kda_short_conv(int32_t num_seqs, int64_t total_tokens, int32_t channels, int32_t kernel_size,
                            int32_t dtype, int32_t silu, const void *x, const void *weight,
                            const int32_t *cu_seqlens, const void *state_in, void *state_out, void *y,
                            void *stream);

/*
 * Output epilogue of the layer: gated RMSNorm over the value channels.  The
 * Ascend model file's attention output path (`_project_out`, with the
 * `KimiRMSNorm` o_norm over head_dim) maps each (token, head) row of the core
 * output o, of length dv, to
 *     y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate)
 * with eps inside the root, one weight per value channel and the output-gate
 * projection `gate` of the same shape as o.  Computed in float32 and rounded
 * once to out_dtype (the page rounds its intermediate products to the
 * activation dtype; that is not modelled).
 *
 *   rows      number of (token, head) rows: T * H (>= 0; 0 is a no-op)
 *   head_v    dv, 64 or 128
 *   in_dtype  kda_dtype_t of o and gate; out_dtype that of out
 *   o, gate   [rows, dv] (i.e. [T, H, dv] contiguous), device
 *   weight    [dv] float32, device
 *   eps       finite, >= 0 (the layer's rms_norm_eps)
 *   out       [rows, dv] out_dtype, device; may be o itself when out_dtype ==
 *             in_dtype (each row is read in full before it is written)
 * All pointers 16-byte aligned (KDA_ERR_BAD_SHAPE otherwise).
 * Errors: KDA_ERR_BAD_SHAPE / _UNSUPPORTED / _NULL_POINTER before any launch.
 */
kda_status_t kda_gated_rmsnorm(int64_t rows, int32_t head_v, int32_t in_dtype, int32_t out_dtype, const void *o,
                               const void *gate, const float *weight, float eps, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
