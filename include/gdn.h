/*
 * gdn.h -- C ABI of the gated delta rule (Gated DeltaNet layer core) for
 * AMD Instinct MI355X (gfx950).  Library: libgdn.so.
 *
 * The operation (per batch b and value head h, key head hk = h / (Hv/Hk)):
 *
 *     S_t = g_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = q_scale * S_t^T q_t,            g_t = exp(log_g_t)
 *
 * with q_t, k_t optionally L2-normalised in the kernels (x / max(|x|, 1e-6)).
 * This is the five-step per-token update of "Qwen3.5 Gated Delta Net NKI
 * Kernel for AWS Neuron" (Hugging Face model card), section "How It Works":
 * decay the state, read S^T k, delta = beta (v - read), write k delta^T, and
 * read the output from the updated state.  The same card's "Correctness
 * Contract" fixes log g <= 0 for Qwen gates (nothing is clamped here either)
 * and makes every (batch, head) independent.  Key heads are shared by
 * consecutive groups of Hv/Hk value heads, as in the 16-key / 48-value-head
 * layout of "Add Qwen3.6-27B contrib model with vLLM APC baseline", table
 * "Architecture".
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library allocates no memory, creates no stream or event and keeps no
 *    global state: a call enqueues kernels on the caller's stream only, so
 *    calls on different streams never wait on one another.  The one
 *    exception is gdn_chunk_prefill_noalloc, whose workspace is a fixed
 *    device array of the library (see there).  (The single-token decode
 *    launcher asks the runtime once per process how many of its workgroups
 *    fit on a compute unit and keeps that read-only figure; it sizes the
 *    grid and couples no calls.)
 *  - Tensors are dense, row-major, innermost dimension last, exactly as listed;
 *    no strides.  Every pointer must be 16-byte aligned.
 *  - q, k, v and o share one storage dtype (gdn_problem.dtype).  log_g, beta
 *    and the recurrent states are always fp32.
 *  - hip_stream is a hipStream_t passed as void*; NULL means the null stream.
 *    Work is enqueued asynchronously; the library never synchronises.
 *  - All argument checks run on the host before anything is enqueued: on any
 *    error the call returns a non-zero gdn_status and enqueues nothing.  A
 *    launch failure reported by the HIP runtime returns GDN_ERR_HIP.  Faults
 *    during execution surface at the caller's next synchronisation, as for
 *    any HIP work.
 *  - Results are bitwise deterministic for identical inputs and launch
 *    parameters (no atomics, fixed reduction orders).
 *  - Calls on different streams are independent and thread-safe provided
 *    their output buffers do not overlap.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

typedef enum {
    GDN_DTYPE_F32 = 0,   /* IEEE binary32 */
    GDN_DTYPE_BF16 = 1   /* bfloat16; kernels accumulate in fp32 and round to
                            nearest-even when storing o */
} gdn_dtype;

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
    GDN_ERR_BAD_SHAPE = 2,    /* negative size, Hv % Hk != 0, decode T != 1, ... */
    GDN_ERR_UNSUPPORTED = 3,  /* head dim / chunk / dtype outside the built kernels */
    GDN_ERR_MISALIGNED = 4,   /* a pointer is not 16-byte aligned */
    GDN_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required */
    GDN_ERR_HIP = 6,          /* the HIP runtime refused the launch */
    GDN_ERR_ALIAS = 7,        /* an output overlaps an input it may not alias */
    /* never returned: they make every int32 value a valid gdn_status, so a
     * code from a newer or foreign caller can be passed to gdn_status_string */
    GDN_STATUS_RESERVED_MIN_ = -2147483647 - 1,
    GDN_STATUS_RESERVED_MAX_ = 2147483647
} gdn_status;

/* Per-call sizes and options. */
typedef struct {
    int32_t B;         /* sequences in the batch, >= 0 */
    int32_t T;         /* tokens per sequence in this call, >= 0 (decode: 1) */
    int32_t Hk;        /* key heads (shared by q and k), >= 1 */
    int32_t Hv;        /* value heads, a multiple of Hk */
    int32_t dk;        /* key head dim: 64 or 128 */
    int32_t dv;        /* value head dim: must equal dk */
    int32_t chunk;     /* prefill chunk length C: 16, 32 or 64 (0 selects 64);
                          ignored by decode */
    int32_t dtype;     /* gdn_dtype of q, k, v, o */
    int32_t qk_l2norm; /* 1: L2-normalise q and k per token inside the kernels;
                          0: use them as given */
    float q_scale;     /* multiplies every output (1.0 for the plain rule) */
} gdn_problem;

/*
 * Workspace bytes that gdn_chunk_prefill needs for this problem (0 is
 * possible).  Returns 0 also for an invalid problem; gdn_chunk_prefill reports
 * the error.  The caller allocates the workspace; its contents need no
 * initialisation and are meaningless after the call.  The bf16 MFMA path
 * ("mfma_bf16" below) needs 13568 bytes per (sequence, value head, chunk of
 * 64 tokens) for up to 256 chunks: the chunk's triangular inverse, masked
 * Q K^T and gate vectors, computed in parallel for a piece of chunks before
 * the serial pass over them.  A call longer than 256 chunks runs in pieces
 * of 256 chunks that reuse these records, and the workspace then also holds
 * the state carried between pieces, after the records at the next multiple
 * of 256 bytes (B * Hv * dk * dv * 4 bytes): at most
 * 256 * 13568 * B * Hv + 255 + 65536 * B * Hv bytes whatever T.  A larger
 * workspace is used for longer pieces; the results are bitwise the same for
 * every piece length.
 * gdn_chunk_prefill_onchip needs no workspace.
 */
size_t gdn_chunk_prefill_workspace_bytes(const gdn_problem* problem);

/*
 * Chunked prefill (context encoding) of T tokens for B sequences.
 *
 * Defined by the recurrence above, evaluated chunk-parallel: inside each chunk
 * of C tokens the decay-masked beta K K^T system is solved directly (forward
 * substitution, never a Neumann power series), as in "Qwen3.6: Fused
 * DeltaNet Direct-Solve Follow-Up", sections "Why This Exists" and
 * "Implementation Details"; the state is handed from chunk to chunk in order.
 * A last chunk shorter than C is allowed.  The result equals the token-serial
 * recurrence up to rounding; splitting a sequence at multiples of C across
 * calls (carrying hT into the next h0) gives bitwise the same o and hT.
 *
 *   q, k   [B, T, Hk, dk]   dtype
 *   v      [B, T, Hv, dv]   dtype
 *   log_g  [B, T, Hv]       fp32, natural-log decay (<= 0 for Qwen gates)
 *   beta   [B, T, Hv]       fp32
 *   h0     [B, Hv, dk, dv]  fp32 initial state, or NULL for zeros
 *   hT     [B, Hv, dk, dv]  fp32 final state, or NULL to drop it; may be the
 *                           same pointer as h0 (in-place carry), may not
 *                           otherwise overlap it
 *   o      [B, T, Hv, dv]   dtype, written
 *   workspace / workspace_bytes: see gdn_chunk_prefill_workspace_bytes
 *
 * T == 0 writes hT = h0 (or zeros) and nothing else.
 */
gdn_status gdn_chunk_prefill(const gdn_problem* problem,
                             const void* q, const void* k, const void* v,
                             const float* log_g, const float* beta,
                             const float* h0, float* hT, void* o,
                             void* workspace, size_t workspace_bytes,
                             void* hip_stream);

/*
 * gdn_chunk_prefill that also stores the recurrent state every ckpt_every
 * tokens: the GDN checkpoint slots that hybrid prefix caching restores from.
 * A reusable prefix of a hybrid DeltaNet/attention model needs a recurrent-
 * state checkpoint at its end as well as attention KV hits ("Add Qwen3.6-27B
 * hybrid DeltaNet/GQA contrib model and vLLM serving path", summary), and the
 * serving path commits such checkpoints from chunked prefill into a bank of
 * slots ("Qwen3.6: Fused DeltaNet Direct-Solve Follow-Up", sections "Hybrid
 * APC Runtime", "Qwen Model Execution" and "Memory").
 *
 *   h_ckpt      [B, NCK, Hv, dk, dv] fp32, NCK = ceil(T / ckpt_every), written:
 *               slot j holds the state after min((j + 1) * ckpt_every, T)
 *               tokens of the sequence (the last slot therefore equals hT).
 *               It may not overlap any other argument.  With T == 0 nothing
 *               is written to it and it may be NULL.
 *   ckpt_every  tokens between checkpoints: a positive multiple of the chunk
 *               length the call runs with (problem->chunk, 0 meaning 64);
 *               otherwise GDN_ERR_BAD_SHAPE.
 * Every other argument, check and result is that of gdn_chunk_prefill (same
 * workspace size).  A slot is bitwise the hT of a call that stops at its
 * token, since both run the same chunks in the same order.
 */
gdn_status gdn_chunk_prefill_ckpt(const gdn_problem* problem,
                                  const void* q, const void* k, const void* v,
                                  const float* log_g, const float* beta,
                                  const float* h0, float* hT, void* o,
                                  float* h_ckpt, int32_t ckpt_every,
                                  void* workspace, size_t workspace_bytes,
                                  void* hip_stream);

/*
 * One decode step (one token per sequence) updating the state in place.
 *
 * Evaluates the five steps for a single token with one read and one write of
 * each state: a = S^T k and c = S^T q come from the same pass over the old
 * state, then delta = beta (v - g a), o = q_scale (g c + delta (k . q)), and
 * S <- g S + k delta^T is stored to the same addresses.
 * problem->T must be 1; problem->chunk is ignored.
 *
 *   q, k   [B, Hk, dk]      dtype
 *   v      [B, Hv, dv]      dtype
 *   log_g  [B, Hv]          fp32
 *   beta   [B, Hv]          fp32
 *   state  [B, Hv, dk, dv]  fp32, read and overwritten in place
 *   o      [B, Hv, dv]      dtype, written
 */
gdn_status gdn_decode_step(const gdn_problem* problem,
                           const void* q, const void* k, const void* v,
                           const float* log_g, const float* beta,
                           float* state, void* o, void* hip_stream);

/*
 * Chunked prefill of a packed batch of sequences of different lengths (the
 * continuous-batching form of context encoding, which the serving pages leave
 * to follow-up work: "Add Qwen3.6-27B hybrid DeltaNet/GQA contrib model and
 * vLLM serving path", summary, "Known limitations and follow-ups").  Every
 * sequence is an independent gdn_chunk_prefill: its own chunks (the last one
 * partial), its own initial and final state.
 *
 *   problem->B      number of sequences
 *   problem->T      the longest sequence (sizes the launch and the workspace:
 *                   gdn_chunk_prefill_workspace_bytes(problem) applies)
 *   cu_seqlens      DEVICE int32 [B + 1]: sequence b is tokens
 *                   cu_seqlens[b] .. cu_seqlens[b + 1] - 1 of the token axis;
 *                   0 = cu_seqlens[0] <= ... <= cu_seqlens[B] = total_tokens
 *                   and no sequence longer than problem->T.  These are not
 *                   checked (they live on the device): values outside them are
 *                   clamped into range, so memory stays in bounds, but results
 *                   are then undefined.
 *   total_tokens    length of the token axis, 0 .. 2^31 - 1
 *   q, k            [total_tokens, Hk, dk]  dtype
 *   v               [total_tokens, Hv, dv]  dtype
 *   log_g, beta     [total_tokens, Hv]      fp32
 *   h0, hT          [B, Hv, dk, dv] fp32 (NULL as in gdn_chunk_prefill)
 *   o               [total_tokens, Hv, dv]  dtype; rows outside every
 *                   sequence are left untouched
 * A sequence of length 0 gets hT = h0.  The results of sequence b are bitwise
 * those of gdn_chunk_prefill on that sequence alone.
 */
gdn_status gdn_chunk_prefill_varlen(const gdn_problem* problem, const int32_t* cu_seqlens,
                                    int64_t total_tokens,
                                    const void* q, const void* k, const void* v,
                                    const float* log_g, const float* beta,
                                    const float* h0, float* hT, void* o,
                                    void* workspace, size_t workspace_bytes,
                                    void* hip_stream);

/*
 * gdn_chunk_prefill in a single pass that keeps every per-chunk intermediate
 * on chip: no workspace, nothing written to memory but o, hT and the
 * checkpoint slots.  The pages' context-encoding kernels are organised the
 * same way, the whole chunked forward with its direct triangular solve in one
 * kernel ("Qwen3.6: Fused DeltaNet Direct-Solve Follow-Up", "Implementation
 * Details"; "Add Qwen3.5-2B contrib model", "Description").
 *
 * For bf16 inputs with d = 128 and chunk 64, each workgroup owns 32 state
 * columns of one value head and forms the chunk's gates, decay-masked
 * K K^T, triangular inverse and masked Q K^T itself, beside the serial
 * state update; other supported shapes run the fp32 kernel, which needs no
 * workspace either.  Arguments, checks and results as
 * gdn_chunk_prefill_ckpt (h_ckpt may be NULL with ckpt_every == 0 for no
 * checkpoints).  Splitting a sequence at multiples of the chunk across calls
 * of this entry point gives bitwise the same results; against
 * gdn_chunk_prefill the results agree to rounding, not bitwise (different
 * kernels, different summation orders).  gdn_chunk_prefill is the faster of
 * the two for long calls (the per-chunk work of a value head is repeated in
 * its four column workgroups here); this one is for callers that cannot
 * provide a workspace and for short calls.
 */
gdn_status gdn_chunk_prefill_onchip(const gdn_problem* problem,
                                    const void* q, const void* k, const void* v,
                                    const float* log_g, const float* beta,
                                    const float* h0, float* hT, void* o,
                                    float* h_ckpt, int32_t ckpt_every,
                                    void* hip_stream);

/*
 * gdn_chunk_prefill for callers that cannot allocate device memory: code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, checks, kernels and results are those of
 * gdn_chunk_prefill (bitwise the same outputs), except that the workspace is
 * a fixed array of gdn_chunk_prefill_noalloc_max_workspace() bytes (64 MiB)
 * that the library holds on every GPU it runs on, from module load until the
 * process ends; the call itself allocates nothing.
 *
 *  - A call runs in pieces of as many chunks as the array holds (bitwise
 *    the same results as gdn_chunk_prefill).  A problem for which the array
 *    cannot hold one chunk's records (13568 * B * Hv bytes) plus, when the
 *    call has more than one chunk, the carried state (65536 * B * Hv bytes
 *    after the next multiple of 256) is rejected with GDN_ERR_WORKSPACE
 *    before anything is enqueued: B * Hv up to 4946 for a one-chunk call,
 *    up to 848 otherwise (27B head shape: 48 value heads, so B up to 17).
 *  - Every call on one GPU uses the same array and leaves its contents
 *    behind.  Calls whose kernels may overlap in time on one GPU (different
 *    streams with no ordering between them) race on it and give wrong
 *    results: order them (one stream, or events).
 *  - The stream must belong to the current device (GDN_ERR_UNSUPPORTED
 *    otherwise).  The first call on a device looks up the array's address
 *    (hipGetSymbolAddress; GDN_ERR_HIP if that fails): make it outside graph
 *    capture, then capture freely.
 */
gdn_status gdn_chunk_prefill_noalloc(const gdn_problem* problem,
                                     const void* q, const void* k, const void* v,
                                     const float* log_g, const float* beta,
                                     const float* h0, float* hT, void* o,
                                     void* hip_stream);

/* Size in bytes of gdn_chunk_prefill_noalloc's fixed workspace array. */
size_t gdn_chunk_prefill_noalloc_max_workspace(void);

/*
 * The operations around the recurrence.  "Qwen3.5 Gated Delta Net NKI Kernel
 * for AWS Neuron", section "How It Works", names them (projections, causal
 * conv1d, gating, RMS norm) without formulas, and "Add Qwen3.6-27B hybrid
 * DeltaNet/GQA contrib model and vLLM serving path", section "Summary",
 * checkpoints the convolution state beside the recurrent one.  These are the
 * plain readings of the two that are not projections.
 *
 * gdn_causal_conv1d: depthwise causal convolution over the channel axis of
 * the q, k, v projections (before the recurrence), width K,
 *   y[b,t,c] = act(bias[c] + sum_{j=0}^{K-1} w[c,j] u[b, t-K+1+j, c]),
 * act = SiLU (x / (1 + e^-x)) when silu != 0, else identity; u is x after the
 * carried state: u[b, s, c] = x[b, s, c] for s >= 0, state_in[b, K-1+s, c]
 * for s < 0 (zeros when state_in is NULL).  The new state is the last K-1
 * inputs, state_out[b, i, c] = u[b, T-K+1+i, c].
 *   x, y              [B, T, C]    dtype (gdn_dtype: fp32 or bf16)
 *   weight            [C, K]       fp32; bias [C] fp32 or NULL
 *   state_in/out      [B, K-1, C]  dtype; either may be NULL; state_out may
 *                                  be state_in itself (updated in place)
 * 1 <= K <= 4; C * sizeof(dtype) a multiple of 16; T = 0 only writes the
 * state; at most 65535 x 64 tokens per call and 65535 sequences.  Consecutive
 * calls carrying the state give bitwise the result of one call.  fp32
 * arithmetic, outputs rounded to the dtype.  y may not overlap any input;
 * state_out may not overlap x, y, weight or bias.
 * Errors: GDN_ERR_UNSUPPORTED (dtype, K, C), GDN_ERR_BAD_SHAPE,
 * GDN_ERR_NULL_POINTER, GDN_ERR_MISALIGNED, GDN_ERR_ALIAS, GDN_ERR_HIP.
 */
gdn_status gdn_causal_conv1d(int32_t B, int32_t T, int32_t C, int32_t K, int32_t dtype,
                             const void* x, const float* weight, const float* bias,
                             const void* state_in, void* state_out, void* y, int32_t silu,
                             void* hip_stream);

/*
 * gdn_gated_rmsnorm: the RMS norm and output gate of the recurrence's output,
 * per row of D values (a row = one token of one value head, D = dv):
 *   y[r, i] = x[r, i] / sqrt(mean_i x[r, i]^2 + eps) * weight[i] * silu(z[r, i])
 * (z NULL: no gate).  x, z, y [rows, D] dtype; weight [D] fp32.  D / (16 /
 * sizeof(dtype)) must be a power of two from 2 to 64 (bf16: D = 16 .. 512;
 * fp32: 8 .. 256); rows < 2^32.  y may be x itself (in place); y may not
 * overlap z or weight.  fp32 arithmetic, the row's sum of squares reduced in
 * a fixed order (deterministic).
 * Errors: GDN_ERR_UNSUPPORTED (dtype, D), GDN_ERR_BAD_SHAPE (rows, eps < 0),
 * GDN_ERR_NULL_POINTER, GDN_ERR_MISALIGNED, GDN_ERR_ALIAS, GDN_ERR_HIP.
 */
gdn_status gdn_gated_rmsnorm(int64_t rows, int32_t D, int32_t dtype, const void* x, const void* z,
                             const float* weight, float eps, void* y, void* hip_stream);

/*
 * Multi-token decode: problem->T >= 0 tokens per sequence applied in order to
 * a state that stays on chip for the whole call, for speculative or
 * multi-token-prediction verification and small continuous-batching steps
 * (the serving pages leave continuous batching, speculative decoding and
 * native multi-token prediction to follow-up work: "Add Qwen3.6-27B hybrid
 * DeltaNet/GQA contrib model and vLLM serving path", summary section "Known
 * limitations and follow-ups", and its GitHub page, "Notes and Limitations").
 * Exactly the token recurrence above, one token after another, with the
 * decode step's fused single pass per token.
 *
 *   q, k     [B, T, Hk, dk]   dtype
 *   v        [B, T, Hv, dv]   dtype
 *   log_g    [B, T, Hv]       fp32 (or the raw projection a, see below)
 *   beta     [B, T, Hv]       fp32 (or the raw projection b)
 *   A_log, dt_bias  [Hv] fp32, or both NULL.  When given, log_g and beta hold
 *            the raw projections and the gates are formed as in
 *            gdn_chunk_prefill_gated.  Exactly one of them NULL:
 *            GDN_ERR_NULL_POINTER.
 *   state    [B, Hv, dk, dv]  fp32, read and overwritten in place (the state
 *            after the last token)
 *   o        [B, T, Hv, dv]   dtype, written
 *   states   [B, T, Hv, dk, dv] fp32 state after every token (what a verifier
 *            rolls back to when it accepts only a prefix of the draft), or
 *            NULL.  It may not overlap any other argument.
 * problem->chunk is ignored.  T == 0 leaves everything unchanged.  With T == 1
 * and states == NULL this is gdn_decode_step.
 */
gdn_status gdn_decode_multi(const gdn_problem* problem,
                            const void* q, const void* k, const void* v,
                            const float* log_g, const float* beta,
                            const float* A_log, const float* dt_bias,
                            float* state, void* o, float* states, void* hip_stream);

/*
 * Fused gate prologue.  The two variants below take the gate projections of
 * the model instead of log g and beta, and form the gates inside the kernels:
 *
 *     log g = -exp(A_log[h]) * softplus(a + dt_bias[h]),   beta = sigmoid(b)
 *
 * ("Qwen3.5 Gated Delta Net NKI Kernel for AWS Neuron", section "Correctness
 * Contract", gives this decay law of the Hugging Face Qwen3.5 layer.  The
 * pages do not spell out beta; the logistic of its projection is taken, the
 * plain way to a write strength in (0, 1)).  log g is never positive, so the
 * state never grows.
 * softplus(x) = log(1 + e^x).  This saves writing and reading log g and beta
 * as separate [B, T, Hv] tensors.
 *
 *   a, b           same shapes and dtype as log_g, beta (fp32 [B, T, Hv]
 *                  for prefill, [B, Hv] for decode): the raw projections
 *   A_log, dt_bias [Hv] fp32 per-value-head gate parameters
 *
 * gdn_chunk_prefill_gated: every other argument as gdn_chunk_prefill_ckpt
 * (h_ckpt may be NULL with ckpt_every == 0 for no checkpoints).
 * gdn_decode_step_gated: every other argument as gdn_decode_step.
 * The results equal those of the plain entry points called with the log g and
 * beta above computed in fp32.
 */
gdn_status gdn_chunk_prefill_gated(const gdn_problem* problem,
                                   const void* q, const void* k, const void* v,
                                   const float* a, const float* b,
                                   const float* A_log, const float* dt_bias,
                                   const float* h0, float* hT, void* o,
                                   float* h_ckpt, int32_t ckpt_every,
                                   void* workspace, size_t workspace_bytes,
                                   void* hip_stream);
gdn_status gdn_decode_step_gated(const gdn_problem* problem,
                                 const void* q, const void* k, const void* v,
                                 const float* a, const float* b,
                                 const float* A_log, const float* dt_bias,
                                 float* state, void* o, void* hip_stream);

/*
 * Name of the prefill kernel variant gdn_chunk_prefill launches for this
 * problem (static storage, never NULL): "generic_f32" (fp32 arithmetic, any
 * supported shape), "mfma_bf16" (bf16 MFMA path for bf16 inputs, d = 128,
 * chunk 64: a parallel prep kernel, then the serial scan), or "invalid" when
 * the problem would be rejected.  Pure query:
 * enqueues nothing.  Setting GDN_FORCE_GENERIC=1 in the environment makes
 * every prefill use "generic_f32" (for A/B comparisons of the two kernels).
 */
const char* gdn_chunk_prefill_variant(const gdn_problem* problem);

/* Human-readable text of a status code (static storage, never NULL). */
const char* gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
