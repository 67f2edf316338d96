/*
 * kda.h -- C ABI of libkda.so: Kimi Delta Attention (KDA) prefill and decode
 * on AMD Instinct MI355X (gfx950).
 *
 * KDA is the gated delta rule with per-channel decay behind Kimi K3's
 * linear-attention layers.  Per head, with a dk x dv state S (row = key
 * channel):
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t,        y_t = o_t (.) sigmoid(gate_logit_t)
 * where q, k, v come out of independent short causal depthwise convolutions
 * ("independent Q/K/V short convolutions", "recurrent KDA state", "KDA output
 * gating": implementation list of the forum post "Experimental Native Vulkan
 * Backend for Kimi K3"), q and k are L2-normalised with KDA_L2_EPS
 * ("metrale_model_arch::kimi_k3" API docs, Constants), alpha_t =
 * exp(log_alpha_t) per key channel and beta_t = sigmoid(beta_logit_t).
 *
 * Entry points (one GPU, caller-owned memory, asynchronous on `stream`):
 *   kda_prologue        short conv + activation + L2(q, k) + sigmoid gates
 *   kda_chunk_forward   chunked prefill over packed variable-length sequences
 *                       with fp32 initial/final state (= kda_chunk_prepare
 *                       followed by kda_chunk_scan, also exported)
 *   kda_prefill         the same prefill from raw inputs in two fused stages
 *                       (= kda_prefill_prepare + kda_prefill_scan)
 *   kda_decode_step     one token for a batch of resident states: conv update
 *                       then recurrent step (kimi_k3 API docs, Functions:
 *                       kda_decode_token)
 *   kda_in_projection, kda_out_projection, kda_mixer_prefill
 *                       the mixer's linear maps around the operator
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or keeps them, and keeps no state between calls
 *     except a per-device "is this a gfx950" flag.
 *   - Calls only enqueue kernels on `stream` (a hipStream_t; NULL = the null
 *     stream) and return; results are ready once the caller synchronises.
 *   - Arguments are checked on the host before anything is launched.  On any
 *     error nothing is launched and nothing is written; the return value
 *     says why and kda_last_error_detail() gives a sentence (per thread).
 *     Unsupported inputs are rejected, never approximated.
 *   - Device-side values are not inspected: NaN/Inf propagate and
 *     log_alpha > 0 is outside the method's range (results unspecified).
 *     kda_decode_step skips a row whose slot index is out of range (see
 *     there).
 *   - Layouts are row-major (last index fastest).  Tokens of all sequences
 *     are packed ("THD": [total_tokens, H, d]); sequence n owns tokens
 *     cu_seqlens[n] .. cu_seqlens[n+1]-1 (int32, cu_seqlens[0] = 0,
 *     non-decreasing; empty sequences are allowed).  A batch may hold no
 *     token at all (total_tokens = 0): the per-token arrays ([T][...]) may
 *     then be NULL, and the states and conv caches pass through unchanged.
 *   - Every tensor pointer must be 16-byte aligned.
 *   - dk = dv = d.  kda_prologue and kda_decode_step accept d in
 *     {4, 8, 16, 32, 64, 128}; the chunk path accepts d = 128 and bf16 only.
 *   - Conv weights: [3][H*d][conv_k] fp32, stream order q, k, v; tap
 *     conv_k-1 multiplies the current token; no bias.  Conv cache:
 *     [n][3][conv_k-1][H*d] fp32, the conv_k-1 raw inputs that precede the
 *     next token of sequence/slot n, oldest first.  Both the conv cache and
 *     the recurrent state are fp32 read-modify-write buffers, as the kimi_k3
 *     API docs describe its per-sequence KdaState.
 *   - Recurrent state: [n][H][d][d] fp32, S[key channel][value channel].
 *   - Thread-safe; calls on different streams may overlap as long as they
 *     do not write the same buffers.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,       /* a size is <= 0 / inconsistent (e.g. total_tokens != cu_seqlens[n]) */
    KDA_ERR_DTYPE = 3,       /* dtype not one of kda_dtype */
    KDA_ERR_UNSUPPORTED = 4, /* valid but not implemented here (d, conv_k, dtype on the chunk path,
                                device architecture other than gfx950) */
    KDA_ERR_SEQLENS = 5,     /* cu_seqlens[0] != 0 or decreasing */
    KDA_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than kda_chunk_workspace_bytes() */
    KDA_ERR_ALIGN = 7,       /* a tensor pointer is not 16-byte aligned */
    KDA_ERR_HIP = 8          /* the HIP runtime reported an error (see kda_last_error_detail) */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;
typedef enum { KDA_ACT_NONE = 0, KDA_ACT_SILU = 1 } kda_act;

/* Geometry and scalars shared by all calls.  The pages give production KDA
 * geometry as head dim 128 and conv kernel 4 (kimi_k3 API docs, struct
 * KdaConfig); they do not print KDA_L2_EPS's value (1e-6 is used by the
 * workloads here).  `scale` multiplies o_t (1.0 reproduces the bare
 * recurrence; dk^-0.5 is the usual attention scaling). */
typedef struct {
    int32_t H;       /* heads (> 0) */
    int32_t d;       /* head dim, dk = dv = d */
    int32_t conv_k;  /* short-conv kernel size, 1..4 */
    int32_t act;     /* kda_act applied after each conv */
    float l2_eps;    /* epsilon inside the L2 norm: x / sqrt(sum x^2 + eps), >= 0 */
    float scale;     /* output scale */
} kda_geom;

/*
 * kda_prologue: per token of each sequence,
 *   x~ = act(conv(x)) for x in {q, k, v};  q^ = L2(q~), k^ = L2(k~), v^ = v~;
 *   beta = sigmoid(beta_logit);  gate = sigmoid(gate_logit).
 * The conv reads history from conv_cache_in at a sequence start (zeros if
 * NULL) and never crosses sequences.
 *   n_seqs >= 1, total_tokens >= 0, cu_seqlens_dev / cu_seqlens_host: the same
 *     [n_seqs+1] int32 offsets, on device and on host (host copy validated).
 *   in_dtype: dtype of q_raw, k_raw, v_raw, beta_logit, gate_logit and of the
 *     outputs q_out, k_out, v_out, gate_out.
 *   q_raw, k_raw, v_raw [T][H][d]; conv_w [3][H*d][conv_k] fp32;
 *   conv_cache_in NULL or [n_seqs][3][conv_k-1][H*d] fp32;
 *   conv_cache_out NULL (skip) or same shape -- the last conv_k-1 raw inputs
 *     of each sequence (reaching into conv_cache_in for short sequences);
 *     it may alias conv_cache_in;
 *   beta_logit [T][H]; gate_logit NULL or [T][H][d] (then gate_out unused);
 *   q_out, k_out, v_out [T][H][d]; beta_out [T][H] fp32; gate_out [T][H][d].
 */
kda_status kda_prologue(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                        const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                        kda_dtype in_dtype, const void *q_raw, const void *k_raw,
                        const void *v_raw, const float *conv_w, const float *conv_cache_in,
                        float *conv_cache_out, const void *beta_logit, const void *gate_logit,
                        void *q_out, void *k_out, void *v_out, float *beta_out, void *gate_out,
                        void *stream);

/*
 * kda_chunk_forward: chunked prefill, the path the k3 README names for KDA
 * prefill ("What this repository is": the CUDA compute path is FLA's
 * chunk_kda) and whose state it carries is the forum post's "recurrent KDA
 * state" (implementation list), with the fp32 read-modify-write state of
 * the kimi_k3 API docs (Structs: KdaState).
 * (d = 128, bf16, chunk = 64 tokens.)  Inputs are the
 * prologue's outputs plus the per-channel log decay.  Each sequence is cut
 * into 64-token chunks from its own start (the last one may be shorter);
 * within a chunk the recurrence is evaluated in its WY/UT form (cumulative
 * log-decay, unit-lower-triangular inverse, bf16 matrix-core products with
 * fp32 accumulation) and the fp32 state is carried from chunk to chunk.
 * The result equals the token-by-token recurrence up to rounding.
 *
 *   q, k [T][H][128] bf16 (L2-normalised), v [T][H][128] bf16,
 *   log_alpha [T][H][128] bf16, <= 0.  Inside a chunk the decays enter
 *     the matrix-core products as per-token factors: referenced to the chunk
 *     start when every channel's decay over the chunk is at most 64 in log2
 *     units, else to the ends of 16-token sub-chunks, where no factor
 *     exceeds e^{(sum of |log_alpha| over one 16-token sub-chunk)}.  Bound:
 *     that sum stays below 87 per channel (a per-token average above -5.4);
 *     beyond it results overflow to inf/NaN;
 *   beta [T][H] fp32 (post-sigmoid), gate NULL or [T][H][128] bf16 (post-sigmoid);
 *   initial_state NULL (zeros) or [n_seqs][H][128][128] fp32;
 *   final_state NULL (skip) or same shape, may alias initial_state;
 *   out [T][H][128] bf16 = scale * o (.) gate;
 *   chunk: the chunk length, must be 64 (anything else: KDA_ERR_UNSUPPORTED);
 *   workspace: device memory of at least kda_chunk_workspace_bytes(...) bytes,
 *     16-byte aligned; its contents are scratch (only kda_chunk_scan reads
 *     what kda_chunk_prepare wrote there).
 * kda_chunk_workspace_bytes(geom, n_seqs, total_tokens) returns a size that
 * suffices for any split of total_tokens into n_seqs sequences (it counts
 * floor((total_tokens + 63 n_seqs) / 64) chunks, the most such a batch can
 * have), or 0 for an invalid geometry or n_seqs <= 0 or total_tokens < 0.
 * Each (chunk, head) takes 74,240 bytes.
 */
size_t kda_chunk_workspace_bytes(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens);

kda_status kda_chunk_forward(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                             const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                             kda_dtype in_dtype, int32_t chunk, const void *q, const void *k, const void *v,
                             const void *log_alpha, const float *beta, const void *gate,
                             const float *initial_state, float *final_state, void *out,
                             void *workspace, size_t workspace_bytes, void *stream);

/* The two stages of kda_chunk_forward, exported so callers can time or
 * overlap them.  kda_chunk_prepare builds every chunk's WY/UT operands
 * (parallel over chunks and heads) into the workspace; kda_chunk_scan then
 * carries the state through each sequence's chunks in order and writes the
 * output and the final state.  Arguments mean what they mean above; the
 * workspace must be passed unchanged between the two. */
kda_status kda_chunk_prepare(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                             const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                             kda_dtype in_dtype, const void *q, const void *k, const void *v,
                             const void *log_alpha, const float *beta,
                             void *workspace, size_t workspace_bytes, void *stream);

kda_status kda_chunk_scan(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                          const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                          kda_dtype in_dtype, const void *gate, const float *initial_state,
                          float *final_state, void *out, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Fused prefill: the whole path from raw inputs in two stages, with no
 * intermediate q^, k^, v^, beta or gate tensors.  kda_prefill_prepare applies
 * the short conv + activation + L2(q, k) + sigmoid(beta) inside the chunk
 * preparation (reading the incoming conv cache at sequence starts) and then
 * writes the outgoing conv cache; kda_prefill_scan carries the state and
 * applies sigmoid(gate_logit) to the output.  kda_prefill runs both.  The
 * result equals kda_prologue followed by kda_chunk_forward, except that q^,
 * k^, v^ are never rounded to bf16 in between.
 *   geom: d = 128, conv_k in [1, 4]; in_dtype must be KDA_BF16; chunk = 64;
 *   q_raw, k_raw, v_raw [T][H][128] bf16 (pre-conv); conv_w [3][H*128][conv_k]
 *   fp32; conv_cache_in NULL (zeros) or [n_seqs][3][conv_k-1][H*128] fp32;
 *   conv_cache_out NULL (skip) or same shape, may alias conv_cache_in;
 *   log_alpha [T][H][128] bf16 (same contract as kda_chunk_forward);
 *   beta_logit [T][H] bf16; gate_logit NULL (no gate) or [T][H][128] bf16;
 *   initial_state, final_state, out, workspace: as for kda_chunk_forward (the
 *   workspace size is kda_chunk_workspace_bytes()).
 */
kda_status kda_prefill(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                       const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                       int32_t chunk, const void *q_raw, const void *k_raw, const void *v_raw, const float *conv_w,
                       const float *conv_cache_in, float *conv_cache_out, const void *log_alpha,
                       const void *beta_logit, const void *gate_logit, const float *initial_state,
                       float *final_state, void *out, void *workspace, size_t workspace_bytes, void *stream);

kda_status kda_prefill_prepare(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                               const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                               kda_dtype in_dtype, const void *q_raw, const void *k_raw, const void *v_raw,
                               const float *conv_w, const float *conv_cache_in, float *conv_cache_out,
                               const void *log_alpha, const void *beta_logit, void *workspace,
                               size_t workspace_bytes, void *stream);

kda_status kda_prefill_scan(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                            const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, kda_dtype in_dtype,
                            const void *gate_logit, const float *initial_state, float *final_state, void *out,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_prefill_noalloc: kda_prefill for callers that cannot allocate device
 * memory -- code under HIP graph capture, serving loops and harnesses that
 * forbid hipMalloc.  It takes no workspace and calls no allocating routine:
 * the chunk workspace is a fixed array of KDA_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, one per GPU, held until the process ends.  Arguments
 * and results are kda_prefill's (the same kernels: identical bits).
 *   Limit: a batch whose chunk workspace (kda_chunk_workspace_bytes's count
 *   for its exact chunks: 74,240 B per (chunk, head) plus a small table) is
 *   larger than the scratch is rejected with KDA_ERR_WORKSPACE before
 *   anything is launched -- at most 903 (chunk, head) pairs, e.g. one
 *   1,792-token sequence at 32 heads or 14,400 tokens at 4 heads.
 *   Nothing in the scratch needs to start at zero: every byte a call reads
 *   was written earlier in the same call.  All calls on one GPU share its
 *   scratch, which keeps the last call's contents: calls that may overlap on
 *   one GPU (other streams, other threads) race, and the caller must order
 *   them.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)

kda_status kda_prefill_noalloc(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                               const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                               kda_dtype in_dtype, int32_t chunk, const void *q_raw, const void *k_raw,
                               const void *v_raw, const float *conv_w, const float *conv_cache_in,
                               float *conv_cache_out, const void *log_alpha, const void *beta_logit,
                               const void *gate_logit, const float *initial_state, float *final_state,
                               void *out, void *stream);

/*
 * The KDA mixer around the operator: the projections, which the k3 README
 * ("Use this repository as a template") places in the KDA module beside the
 * output gate, around the recurrence primitive.  The output gating itself is the
 * sigmoid gate inside kda_prefill / kda_decode_step.
 *
 * kda_in_projection: one GEMM of hidden states onto every raw input of
 * kda_prefill.
 *   geom: H, d (any d >= 1; the chunk path that consumes the outputs needs 128);
 *   x [T][hidden] bf16; w_in [5 H d + H][hidden] bf16, one row per output
 *     feature, rows in the order q, k, v, gate logit, decay pre-activation
 *     (H d each, head-major) and beta logit (H);
 *   a_log NULL (0) or [H] fp32; dt_bias NULL (0) or [H d] fp32;
 *   outputs bf16, overwritten: q_raw, k_raw, v_raw, gate_logit, log_alpha
 *     [T][H][d], beta_logit [T][H];
 *   log_alpha = -exp(a_log[h]) * softplus(z + dt_bias[h d + c]) for the decay
 *     pre-activation z: a reading (the pages do not say how the decay comes
 *     from the projection); with a_log and dt_bias NULL it is -softplus(z),
 *     which maps any real onto log alpha <= 0.
 *   hidden must be a positive multiple of 8 (KDA_ERR_UNSUPPORTED otherwise);
 *   each operand must stay below 4 GiB (KDA_ERR_SHAPE).  bf16 matrix-core
 *   products with fp32 accumulation; results rounded to bf16.
 *
 * kda_out_projection: out [T][hidden] = y [T][H d] w_out^T, with w_out
 *   [hidden][H d] bf16 (one row per hidden feature); H d a multiple of 8.
 *
 * kda_mixer_prefill: kda_in_projection, kda_prefill (chunk 64, d = 128,
 *   conv cache and state as there) and kda_out_projection in one call, the
 *   intermediates in `workspace` (at least kda_mixer_workspace_bytes(geom,
 *   n_seqs, total_tokens) bytes: the projection outputs, the KDA output and
 *   the chunk workspace).  out [T][hidden] bf16.  Every argument is checked
 *   before the first launch.
 */
kda_status kda_in_projection(const kda_geom *geom, int32_t T, int32_t hidden, const void *x, const void *w_in,
                             const float *a_log, const float *dt_bias, void *q_raw, void *k_raw, void *v_raw,
                             void *gate_logit, void *log_alpha, void *beta_logit, void *stream);

kda_status kda_out_projection(const kda_geom *geom, int32_t T, int32_t hidden, const void *y, const void *w_out,
                              void *out, void *stream);

size_t kda_mixer_workspace_bytes(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens);

kda_status kda_mixer_prefill(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                             const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host, int32_t hidden,
                             const void *x, const void *w_in, const float *a_log, const float *dt_bias,
                             const float *conv_w, const float *conv_cache_in, float *conv_cache_out,
                             const float *initial_state, float *final_state, const void *w_out, void *out,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_decode_step: one token for each of `batch` rows, fused: conv-cache
 * shift and conv, activation, L2(q, k), sigmoid gates, then one step of the
 * recurrence on the row's resident state, read and written once.
 *   slot_idx_dev NULL (row b uses slot b, needs batch <= n_slots) or
 *     [batch] int32 distinct slot numbers in [0, n_slots); a row whose slot
 *     lies outside [0, n_slots) is skipped: no state, cache or output element
 *     of it is read or written (its output row keeps its old contents);
 *   in_dtype: dtype of q_raw, k_raw, v_raw [batch][H][d], log_alpha
 *     [batch][H][d], beta_logit [batch][H], gate_logit NULL or [batch][H][d];
 *   conv_w [3][H*d][conv_k] fp32; conv_cache [n_slots][3][conv_k-1][H*d] fp32
 *     and state [n_slots][H][d][d] fp32 are updated in place;
 *   out [batch][H][d] in out_dtype (fp32 keeps the step's fp32 accuracy).
 * One 256-thread workgroup per (row, head), heads fastest in a 1-D grid:
 * batch <= 65535 * 256 and batch * H <= 2^31 - 1 (else KDA_ERR_SHAPE).
 */
kda_status kda_decode_step(const kda_geom *geom, int32_t batch, const int32_t *slot_idx_dev,
                           int32_t n_slots, kda_dtype in_dtype, const void *q_raw,
                           const void *k_raw, const void *v_raw, const float *conv_w,
                           float *conv_cache, float *state, const void *log_alpha,
                           const void *beta_logit, const void *gate_logit, kda_dtype out_dtype,
                           void *out, void *stream);

/*
 * kda_prologue_backward: gradients of kda_prologue with respect to its
 * inputs, given the gradients that reach its outputs (for instance those
 * kda_chunk_backward returns).  It reverses the prologue's steps: the L2
 * normalisation of q and k with KDA_L2_EPS (kimi_k3 API docs, Constants),
 * the activation and the short causal depthwise conv on q, k and v (the
 * Vulkan-backend forum post's implementation list), and the sigmoids of the
 * beta and gate logits ("KDA output gating", same list).
 *   geom, n_seqs, total_tokens, cu_seqlens_*, in_dtype, q_raw, k_raw, v_raw,
 *     conv_w, conv_cache_in (NULL = zeros), beta_logit, gate_logit (NULL =
 *     none): exactly the forward call's inputs;
 *   dq, dk, dv [T][H][d], dbeta [T][H], dgate [T][H][d] (required when
 *     gate_logit is given): fp32 gradients with respect to q_out, k_out,
 *     v_out, beta_out and gate_out;
 *   outputs, fp32, caller-owned and overwritten: dq_raw, dk_raw, dv_raw
 *     [T][H][d]; dconv_w [3][H*d][conv_k] (summed over every token);
 *     dconv_cache_in NULL (skip) or [n_seqs][3][conv_k-1][H*d] (the gradient
 *     with respect to the incoming cache rows, whether or not a cache was
 *     given); dbeta_logit [T][H]; dgate_logit [T][H][d] (with a gate);
 *   workspace: device buffer of at least kda_prologue_backward_workspace_bytes()
 *     bytes, 16-byte aligned (3 T H d fp32 plus the tap partial sums).
 * The outgoing conv cache copies raw inputs and is taken to receive no
 * gradient.  The result is deterministic (no atomics).  Errors as for
 * kda_prologue, plus KDA_ERR_WORKSPACE; nothing is launched when validation
 * fails.
 */
size_t kda_prologue_backward_workspace_bytes(const kda_geom *geom, int32_t total_tokens);

kda_status kda_prologue_backward(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                                 const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                                 kda_dtype in_dtype, const void *q_raw, const void *k_raw, const void *v_raw,
                                 const float *conv_w, const float *conv_cache_in, const void *beta_logit,
                                 const void *gate_logit, const float *dq, const float *dk, const float *dv,
                                 const float *dbeta, const float *dgate, float *dq_raw, float *dk_raw,
                                 float *dv_raw, float *dconv_w, float *dconv_cache_in, float *dbeta_logit,
                                 float *dgate_logit, void *workspace, size_t workspace_bytes, void *stream);

/*
 * kda_chunk_backward: gradients of kda_chunk_forward with respect to its
 * inputs (reverse-mode differentiation of the recurrence of the Vulkan-backend
 * forum post's "recurrent KDA state", taken through the chunked WY/UT form;
 * the k3 README's functional tiny proxy checks such KDA-layer gradients).
 *   geom: d = 128 (as kda_chunk_forward); in_dtype must be KDA_BF16;
 *   q, k, v, log_alpha, beta, gate, initial_state: exactly the forward call's
 *     inputs (gate NULL when the forward had none; initial_state NULL = zeros);
 *   dy [T][H][128] bf16: gradient of the loss with respect to `out`;
 *   d_final_state NULL (zeros) or [n_seqs][H][128][128] fp32: gradient with
 *     respect to `final_state`;
 *   outputs, fp32, caller-owned and overwritten: dq, dk, dv, dlog_alpha
 *     [T][H][128]; dbeta [T][H]; dgate [T][H][128] (required when gate is
 *     given, ignored otherwise); d_initial_state NULL (skip) or
 *     [n_seqs][H][128][128];
 *   workspace: device buffer of at least kda_chunk_backward_workspace_bytes()
 *     bytes, 16-byte aligned, contents not needed before or after the call
 *     (573,952 B per (chunk, head) plus the chunk table; sized, like
 *     kda_chunk_workspace_bytes, from the totals n_seqs and total_tokens).
 * Runs the forward's chunk quantities again (nothing from a forward call is
 * reused) and is stream-ordered like every other entry point.  Its decays
 * are referenced to each chunk's start (fp32): the sum of |log_alpha| over
 * each 64-token chunk must stay below 80 per channel.  Errors as for
 * kda_chunk_forward; nothing is launched when validation fails.
 */
size_t kda_chunk_backward_workspace_bytes(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens);

kda_status kda_chunk_backward(const kda_geom *geom, int32_t n_seqs, int32_t total_tokens,
                              const int32_t *cu_seqlens_dev, const int32_t *cu_seqlens_host,
                              kda_dtype in_dtype, const void *q, const void *k, const void *v,
                              const void *log_alpha, const float *beta, const void *gate,
                              const float *initial_state, const void *dy, const float *d_final_state,
                              float *dq, float *dk, float *dv, float *dlog_alpha, float *dbeta, float *dgate,
                              float *d_initial_state, void *workspace, size_t workspace_bytes, void *stream);

/*
 * The MLA decode token: the other mixer of the hybrid decoder, one token per
 * sequence (kimi_k3 API docs, Functions: mla_decode_token, whose steps are
 * optional RoPE, K/V append, SDPA and an optional output gate, the
 * projections staying in the MLA mixer; gated_mla_attend, the gated NoPE
 * form without the rotary step, which this is).  Per sequence b and query
 * head h, with kv head h / (H / H_kv) and pos = cache_len[b]:
 *   k_cache[b][kv][pos] = k_new[b][kv], v_cache[b][kv][pos] = v_new[b][kv];
 *   o = softmax over j = 0 .. pos of (scale q[b][h] . k_cache[b][kv][j]),
 *       applied to v_cache[b][kv][j];
 *   out[b][h] = o * sigmoid(gate_logit[b][h])   (no gate: o).
 * The cache holds one k and one v per token and kv head (the docs' MlaKv
 * holds a layer's K/V; the layout is this library's); the new token's
 * position is the count of tokens already cached; the gate is elementwise
 * per (head, value channel).  These are readings of the docs.
 *
 *   geom: H query heads and H_kv kv heads (H a multiple of H_kv), d_qk q/k
 *     channels per head (nope + rope), d_v value channels, both in [1, 256];
 *     scale the softmax scale (1 / sqrt(d_qk) is the usual one);
 *   batch in [0, 65535] sequences, max_len the cache capacity in tokens,
 *     at most 65535 * 256 = 16,776,960;
 *   cache_len_dev [batch] int32, device: tokens already cached per sequence.
 *     The call neither reads past it nor advances it (the caller adds 1 after
 *     the call).  A sequence whose cache_len is outside [0, max_len) is left
 *     alone: nothing is written to its caches and its output is 0;
 *   q [batch][H][d_qk], k_new [batch][H_kv][d_qk], v_new [batch][H_kv][d_v],
 *     gate_logit [batch][H][d_v] or NULL: bf16, device;
 *   k_cache [batch][H_kv][max_len][d_qk], v_cache [batch][H_kv][max_len][d_v]:
 *     bf16, device, caller-owned; the call writes slot pos of each and reads
 *     slots 0 .. pos - 1 (nothing else);
 *   out [batch][H][d_v] bf16, device, overwritten;
 *   workspace: device, 16-byte aligned, at least
 *     kda_mla_decode_workspace_bytes() bytes, contents not needed before or
 *     after the call (split partials: 8 + 4 d_v bytes per (sequence, head,
 *     256 cache slots)).
 * fp32 scores, softmax and accumulation.  Every pointer must be 16-byte
 * aligned (KDA_ERR_ALIGN).  Stream-ordered; calls that share a workspace or
 * a cache must not overlap.  Errors: KDA_ERR_NULL, KDA_ERR_SHAPE,
 * KDA_ERR_UNSUPPORTED (head dims above 256), KDA_ERR_ALIGN,
 * KDA_ERR_WORKSPACE, KDA_ERR_HIP; nothing is launched when validation fails.
 */
typedef struct {
    int32_t H;      /* query heads */
    int32_t H_kv;   /* key/value heads; H % H_kv == 0 */
    int32_t d_qk;   /* q and k channels per head (nope + rope) */
    int32_t d_v;    /* value channels per head */
    float scale;    /* softmax scale */
} kda_mla_geom;

size_t kda_mla_decode_workspace_bytes(const kda_mla_geom *geom, int32_t batch, int32_t max_len);

kda_status kda_mla_decode_step(const kda_mla_geom *geom, int32_t batch, int32_t max_len,
                               const int32_t *cache_len_dev, const void *q, const void *k_new, const void *v_new,
                               const void *gate_logit, void *k_cache, void *v_cache, void *out, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Short name of a status code (static string). */
const char *kda_status_str(kda_status s);
/* Sentence describing the last error returned on the calling thread ("" if none). */
const char *kda_last_error_detail(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
