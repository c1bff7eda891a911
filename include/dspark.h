/*
 * dspark.h -- C ABI of the DSpark draft pass on AMD Instinct MI355X (gfx950).
 *
 * The draft pass (huggingface.co "Kimi-K3-DSpark-NVFP4", original card,
 * "Model Overview"; alphaneural.io "kimi-k3-dspark-gguf", "How it works";
 * graysoft.dev "Lucebox Kimi-K3-DSpark Q8_0 GGUF", "Architecture metadata"):
 * five captured target hidden states of a 7-token block are fused by fc, run
 * through dense non-causal decoder layers whose MLA attention reads the
 * 576-element latent cache with kv_b absorbed, projected through the lm_head,
 * rolled out by the rank-256 Markov head and scored by the confidence head.
 * The acceptance length is the prefix run length of matches against a
 * verifier stream ("Why acceptance is so sensitive"; "Sampling options").
 *
 * Conventions for every call:
 *  - All functions return int32_t: DSPARK_OK (0) or a negative error code.
 *    Arguments are validated before anything is enqueued; on error nothing
 *    is enqueued and dspark_last_error() returns a thread-local message.
 *  - Device pointers are HIP device addresses owned by the caller.  The
 *    library allocates no device memory, never frees caller memory and never
 *    synchronises the stream on the hot path (draft / layer / accept calls
 *    enqueue asynchronously on `stream`, a hipStream_t passed as void*;
 *    NULL means the legacy default stream).
 *  - Element layouts are row-major; "[a][b]" means b is contiguous.
 *  - A model is read-only after creation; calls on distinct streams with
 *    distinct workspaces may run concurrently.  Calls that share a workspace
 *    must be ordered by the caller.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- error codes ---- */
#define DSPARK_OK 0
#define DSPARK_EINVAL (-1)       /* null / misaligned pointer, out-of-range value */
#define DSPARK_EUNSUPPORTED (-2) /* shape or format the kernels do not cover     */
#define DSPARK_EWORKSPACE (-3)   /* buffer smaller than the size query returned  */
#define DSPARK_EHIP (-4)         /* HIP runtime error; message has the HIP text  */
#define DSPARK_ENODEVICE (-5)    /* no usable gfx950 device                      */
#define DSPARK_EPLANONLY (-6)    /* every argument passed validation, but the model
                                    is a plan-only handle (DSPARK_CFG_PLAN_ONLY):
                                    it has no packed weights, nothing was enqueued */

/* ---- storage formats of weights and activations ---- */
#define DSPARK_DT_F32 0
#define DSPARK_DT_BF16 1
/* Q8_0: blocks of 32 consecutive weights along a row, 34 bytes each: an fp16
 * scale d (little-endian) then 32 int8 codes q; weight = d * q (graysoft.dev
 * card, "Conversion result": GGUF MOSTLY_Q8_0).  cols % 32 == 0. */
#define DSPARK_DT_Q8_0 2
/* FP8 E4M3FN codes (OCP: bias 7, no inf, 0x7F/0xFF NaN, max 448) with one fp32
 * scale per output row; weight = scale[row] * e4m3(code) (huggingface.co card,
 * "Limitations": per-channel weight-only FP8). */
#define DSPARK_DT_FP8_E4M3 3
/* MXFP4 (OCP Microscaling): blocks of 32 consecutive weights along a row, 17
 * bytes each: one E8M0 scale code e (X = 2^(e - 127)) then 16 bytes of FP4
 * E2M1 codes, element 2i in the low nibble of byte i and 2i + 1 in the high
 * nibble; weight = X * e2m1(code) (huggingface.co card, "Drift-limited
 * acceptance ceiling" and "Detail": the MXFP4 variant).  cols % 32 == 0 and
 * round_up(cols, 64) % 128 == 0 (the device layout holds four blocks per
 * 1 KiB chunk).  On the device a scale code of 0 decodes as 0 (not 2^-127)
 * and 255 as +inf (not NaN): only the exponent field is formed. */
#define DSPARK_DT_MXFP4 4

/* ---- weight table ids ---- */
#define DSPARK_W_FC 0          /* [hidden][n_captured*hidden] fc ("context_proj")  */
#define DSPARK_W_FC_NORM 1     /* [hidden] f32, RMSNorm gain after fc              */
#define DSPARK_W_FINAL_NORM 2  /* [hidden] f32                                     */
#define DSPARK_W_LM_HEAD 3     /* [vocab][hidden]                                  */
#define DSPARK_W_MARKOV_W1 4   /* [vocab][markov_rank] (BF16 or F32)               */
#define DSPARK_W_MARKOV_W2 5   /* [vocab][markov_rank] (BF16 or F32)               */
#define DSPARK_W_CONF_W 6      /* [hidden + markov_rank] f32                       */
#define DSPARK_W_CONF_B 7      /* [1] f32                                          */
#define DSPARK_W_LAYER_BASE 16
#define DSPARK_W_LAYER_STRIDE 16
/* per-layer tensors: id = DSPARK_LAYER_W(layer, k) */
#define DSPARK_L_IN_NORM 0     /* [hidden] f32                                     */
#define DSPARK_L_Q_A 1         /* [q_lora][hidden]                                  */
#define DSPARK_L_Q_A_NORM 2    /* [q_lora] f32                                      */
#define DSPARK_L_KV_A 3        /* [kv_lora + qk_rope][hidden] (kv_a_proj_with_mqa)  */
#define DSPARK_L_KV_A_NORM 4   /* [kv_lora] f32                                     */
#define DSPARK_L_Q_B 5         /* [n_heads*(qk_nope+qk_rope)][q_lora]               */
#define DSPARK_L_KV_B 6        /* [n_heads*(qk_nope+v_head)][kv_lora]; per head the
                                  first qk_nope rows are W_UK, the next v_head W_UV */
#define DSPARK_L_O 7           /* [hidden][n_heads*v_head]                          */
#define DSPARK_L_POST_NORM 8   /* [hidden] f32                                      */
#define DSPARK_L_GATE 9        /* [inter][hidden]                                   */
#define DSPARK_L_UP 10         /* [inter][hidden]                                   */
#define DSPARK_L_DOWN 11       /* [hidden][inter]                                   */
#define DSPARK_LAYER_W(l, k) (DSPARK_W_LAYER_BASE + (l) * DSPARK_W_LAYER_STRIDE + (k))

/* config flags */
#define DSPARK_CFG_LAYERS_ONLY 1 /* the table holds decoder layers only (no fc,
                                    lm_head, Markov or confidence tensors): only
                                    dspark_layer_forward may be called */
#define DSPARK_CFG_PLAN_ONLY 2   /* dspark_model_create validates the config and
                                    the table (data pointers must be non-NULL but
                                    are never read) and plans the layouts without
                                    a device: packed_buf may be NULL, no HIP call
                                    is made.  The handle answers the size queries;
                                    draft / layer / append / dequant calls on it
                                    run their whole argument validation and then
                                    return DSPARK_EPLANONLY (sizing buffers before
                                    any device work, and host-side tests of the
                                    validation) */

typedef struct dspark_config {
  int32_t hidden, n_layers, n_heads, q_lora, kv_lora, qk_nope, qk_rope, v_head;
  int32_t inter, vocab, markov_rank, block, n_captured;
  int32_t flags;
  float rms_eps;       /* RMSNorm: g * x / sqrt(mean(x^2) + eps)               */
  float rope_theta;    /* RoPE base; consecutive pairs (2k, 2k+1) rotate        */
  float yarn_factor;   /* 1 = plain RoPE; s > 1: YaRN NTK-by-parts, logit x m^2 */
  int32_t yarn_orig_ctx;
  float yarn_beta_fast, yarn_beta_slow;
} dspark_config;

typedef struct dspark_weight {
  int32_t id;          /* DSPARK_W_* or DSPARK_LAYER_W(l, k)                    */
  int32_t dtype;       /* DSPARK_DT_*; norms and the confidence head are F32    */
  const void* data;    /* device; F32 float[rows][cols]; BF16 uint16[rows][cols];
                          Q8_0 uint8[rows][cols/32*34]; FP8 uint8[rows][cols];
                          MXFP4 uint8[rows][cols/32*17]                         */
  const void* scales;  /* device float[rows] for FP8, else NULL                 */
  int64_t rows, cols;  /* vectors: rows = length, cols = 1                      */
} dspark_weight;

typedef struct dspark_model dspark_model; /* opaque, host memory */

/* Bytes of device memory the caller must provide to dspark_model_create for
 * the repacked weights (device layouts: 16-row tiles in MFMA fragment order,
 * Q8_0 / MXFP4 codes and block scales in separate planes).  0 on invalid input (see
 * dspark_last_error). */
size_t dspark_packed_bytes(const dspark_config* cfg, const dspark_weight* w, int32_t n);

/* Validate the config and the weight table, repack every tensor into
 * `packed_buf` (caller-owned device memory of at least packed_bytes, 256-byte
 * aligned) with kernels on `stream`, then synchronise the stream once.  The
 * caller may free the source tensors after this returns.  *out is a host
 * handle owned by the library; free it with dspark_model_destroy. */
int32_t dspark_model_create(const dspark_config* cfg, const dspark_weight* w, int32_t n,
                            void* packed_buf, size_t packed_bytes, void* stream,
                            dspark_model** out);

/* Free the host handle (the packed buffer stays the caller's). */
int32_t dspark_model_destroy(dspark_model* m);

/* Workspace bytes for one draft / layer call over n_seq sequences whose cache
 * lengths sum to total_ctx.  0 on invalid input. */
size_t dspark_workspace_bytes(const dspark_model* m, int32_t n_seq, int64_t total_ctx);

typedef struct dspark_block_in {
  int32_t n_seq;              /* >= 1                                            */
  int32_t act_dtype;          /* captured states: DSPARK_DT_F32 or DSPARK_DT_BF16 */
  int32_t kv_dtype;           /* latent caches: DSPARK_DT_F32 or DSPARK_DT_BF16   */
  int32_t pad_;
  int64_t total_ctx;          /* == kv_offsets[n_seq] (host copy, for planning)   */
  const void* captured;       /* device [n_seq][n_captured][block][hidden]; fc
                                 concatenates the n_captured states per token in
                                 this (capture) order                            */
  const void* const* kv;      /* host array of n_layers device pointers, each
                                 [total_ctx][kv_lora + qk_rope]: per token the
                                 normed c_kv then the roped k_pe, used as stored;
                                 sequence s owns rows kv_offsets[s] .. [s+1]-1   */
  const int32_t* kv_offsets;  /* device int32 [n_seq + 1], non-decreasing, [0]=0 */
  const int32_t* prev_token;  /* device int32 [n_seq]: last verified token, the
                                 Markov predecessor of position 0; -1 (or any
                                 value outside [0, vocab)) = none               */
  const int32_t* forced_prev; /* optional device int32 [n_seq][block]: when set,
                                 position i >= 1 uses forced_prev[s][i-1] as its
                                 Markov predecessor instead of the drafted token
                                 (teacher-forced rollout); NULL = free running   */
  /* Paged latent caches, the layout the draft shares with the target's cache
     (huggingface.co "Kimi-K3-DSpark-NVFP4", original card, "Model Overview":
     one 576-element latent per token, so the draft's pages unify with the
     target's).  page_size == 0: kv[l] is packed as described above.  Else
     kv[l] is a page pool [n_pages][page_size][kv_lora + qk_rope] (bf16 caches
     only), the length of sequence s is still kv_offsets[s+1] - kv_offsets[s],
     and its token j is row j % page_size of page block_table[s][j / page_size]
     in every layer's pool.  Page indices are not range checked: each page a
     sequence's length reaches must exist in every pool.                      */
  int32_t page_size;          /* 0, or a power of two >= 32                     */
  int32_t max_pages;          /* row stride of block_table (>= 1 when paged)    */
  const int32_t* block_table; /* device int32 [n_seq][max_pages] when paged     */
  /* Probabilistic drafting (huggingface.co "Kimi-K3-DSpark-NVFP4", "Sampling
     options": the draft sampled from its own distribution).  sample_u == NULL:
     greedy (argmax).  Else token i is the draw from softmax(l_i / temperature)
     given by the Gumbel-max rule, argmax_v (l_i[v] / temperature
     - ln(-ln sample_u[s][i][v])); the returned logits stay l_i.  Needs bf16
     Markov weights and n_seq <= 16 (EUNSUPPORTED otherwise).               */
  const float* sample_u;      /* device float [n_seq][block][vocab], in (0, 1)  */
  float temperature;          /* > 0 when sample_u is set                       */
  /* Bound of the Markov rollout's wait for the previous position's argmax
     (the rollout is one launch whose workgroups exchange each position's
     argmax through memory): 0 = the library's bound (~4M polls, seconds);
     n > 0: at most n polls per position; < 0: no wait at all, the rollout
     expires at once (host-forced failure path for tests).  On expiry every
     kernel still finishes, every token of the call is -1 and *status = 1. */
  int32_t poll_limit;
} dspark_block_in;

typedef struct dspark_block_out {
  int32_t* tokens;  /* device int32 [n_seq][block]: the draft, greedy or sampled
                       (required); all -1 when the Markov rollout's bounded wait
                       expired (see poll_limit and status): never pass -1 tokens
                       on to acceptance or verification                       */
  float* conf;      /* device float [n_seq][block] confidence (required)         */
  float* logits;    /* optional device float [n_seq][block][vocab]: backbone
                       logits plus the Markov term, the argmax input; NULL = skip */
  float* hidden;    /* optional device float [n_seq][block][hidden]: final-normed
                       hidden state fed to the lm_head; NULL = skip             */
  void* const* stage_events; /* optional host array of 2*DSPARK_N_STAGES
                       hipEvent_t: events[2s] / events[2s+1] are recorded on the
                       stream right before / after stage s (profiling aid);
                       NULL = none                                               */
  int32_t* status;  /* optional device int32 [1]: 0 when the pass completed
                       by the full Markov rollout, 2 when it completed by the
                       candidate rollout (greedy passes without logits or
                       hidden outputs: only the rows that can still be the
                       argmax, by a Cauchy-Schwarz bound on the Markov term,
                       are evaluated; same tokens up to rounding ties), 1 when
                       the full rollout's wait expired (tokens are then -1);
                       NULL = skip.  The library's bound is only reached when
                       the rollout's workgroups cannot all be resident, e.g.
                       kernels of other streams hold CUs for seconds          */
} dspark_block_out;

/* stages of one draft pass, for dspark_block_out.stage_events */
#define DSPARK_STAGE_FC 0      /* input fragments + fc GEMM + fc norm            */
#define DSPARK_STAGE_LAYERS 1  /* all decoder layers and the final norm          */
#define DSPARK_STAGE_LM_HEAD 2 /* the lm_head GEMM (exactly one kernel launch)   */
#define DSPARK_STAGE_MARKOV 3  /* Markov rollout, argmax, confidence              */
#define DSPARK_N_STAGES 4

/* One draft pass for every sequence's block (one pass of the hot path):
 * fc + RMSNorm -> n_layers x (RMSNorm, fused q_a/kv_a, q/kv norms + rope, q_b,
 * absorbed split-K MLA attention over cache rows and the block's own 7 latent
 * rows (no mask), un-absorb, o_proj + residual, RMSNorm, SwiGLU + residual) ->
 * final RMSNorm -> lm_head -> for i = 0..block-1: l_i = z_i + W2 W1[t_{i-1}],
 * t_i = argmax l_i (lowest index on ties), conf_i = sigmoid(w_h . hf_i +
 * w_m . W1[t_{i-1}] + b).  Position of block token i = that sequence's cache
 * length + i.  Asynchronous on `stream`.  `workspace` must hold
 * dspark_workspace_bytes(m, in->n_seq, in->total_ctx) bytes, 256-byte aligned.
 * Alignment: kv caches 16 bytes, captured / outputs / int arrays 4 bytes.
 * Errors: EINVAL (nulls, misaligned pointers, n_seq < 1, total_ctx out of
 * range, dtypes, bad page geometry, temperature <= 0 with sample_u),
 * EUNSUPPORTED (n_seq > 16, sampling without the bf16 rollout, latent sizes
 * without a kernel), EWORKSPACE, EPLANONLY, EHIP. */
int32_t dspark_draft_block(const dspark_model* m, const dspark_block_in* in,
                           dspark_block_out* out, void* workspace, size_t ws_bytes,
                           void* stream);

/* The same draft pass for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): no workspace argument and no allocation of any kind; the
 * pass's scratch lives in a static device array of the library
 * (DSPARK_STATIC_SCRATCH_BYTES, one copy per GPU, held until the process
 * ends).  Same arguments, semantics and results as dspark_draft_block.
 * Calls whose workspace would exceed the array (see dspark_workspace_bytes;
 * e.g. one sequence with more than about 220k cached tokens at the full
 * geometry) fail with DSPARK_EWORKSPACE and enqueue nothing.  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (concurrent streams, or
 * threads) race and must be ordered by the caller.  The array keeps the last
 * call's contents; the pass clears what it needs zeroed itself, with a kernel
 * (no memset node under capture). */
#define DSPARK_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int32_t dspark_draft_block_static(const dspark_model* m, const dspark_block_in* in,
                                  dspark_block_out* out, void* stream);

/* One decoder layer on a given residual stream (the single-layer unit):
 * x_out = x_in + o_proj(MLA(RMSNorm(x_in))) and, when with_mlp != 0, then
 * x_out += SwiGLU(RMSNorm(x_out)).  x_in, x_out: device float
 * [n_seq*block][hidden] (may alias).  kv: device [total_ctx][kv_lora+qk_rope] of
 * kv_dtype; kv_offsets: device [n_seq+1].  Asynchronous on `stream`. */
int32_t dspark_layer_forward(const dspark_model* m, int32_t layer, int32_t with_mlp,
                             int32_t n_seq, const float* x_in, float* x_out,
                             const void* kv, int32_t kv_dtype, const int32_t* kv_offsets,
                             int64_t total_ctx, void* workspace, size_t ws_bytes,
                             void* stream);

/* Cache append: the latent cache rows of newly verified positions.  The
 * draft's latent rows share the target's one-576-element-per-token page format
 * (huggingface.co "Kimi-K3-DSpark-NVFP4", original card, "Model Overview"),
 * and fc consumes the target states captured at a position
 * (graysoft.dev "Lucebox Kimi-K3-DSpark Q8_0 GGUF", "Architecture metadata").
 * Reading taken where the pages stop: the row of layer l at a new position is
 * that layer's kv_a path applied to the position's fc output,
 *   x   = RMSNorm(concat(captured) . W_fc^T; g_fc),
 *   a   = RMSNorm(x; in_norm_l),  kv = a . W_kva_l^T,
 *   row = [RMSNorm(kv[:kv_lora]; g_kva_l) | RoPE(kv[kv_lora:], position)],
 * which for layer 0 is exactly the draft pass's own block key at that
 * position. */
typedef struct dspark_append_in {
  int32_t n_new;               /* rows to append, 1 .. DSPARK_APPEND_MAX        */
  int32_t act_dtype;           /* captured states: DSPARK_DT_F32 or _BF16       */
  int32_t kv_dtype;            /* caches: DSPARK_DT_F32 or DSPARK_DT_BF16       */
  int32_t pad_;
  const void* captured;        /* device [n_new][n_captured][hidden], each row's
                                  states in capture order                      */
  const int32_t* positions;    /* device int32 [n_new]: each row's position in
                                  its sequence (its RoPE angle)                */
  const int64_t* slot_mapping; /* device int64 [n_new]: destination row of each
                                  new row in every layer's cache, viewed as
                                  [rows][kv_lora + qk_rope] (a page pool: page *
                                  page_size + row in page); distinct, and not
                                  range checked                                */
  void* const* kv;             /* host array of n_layers device caches / pools  */
} dspark_append_in;
#define DSPARK_APPEND_MAX 128

/* Bytes of device workspace dspark_cache_append needs for n_new rows
 * (0 and the error text on bad arguments). */
size_t dspark_append_workspace_bytes(const dspark_model* m, int32_t n_new);

/* Computes and writes the rows described at dspark_append_in into every
 * layer's cache; touches no other cache row.  Asynchronous on `stream`;
 * `workspace` (256-byte aligned) is scratch for the call.  The model must
 * hold the whole drafter (not layers_only) and n_captured * hidden inputs.
 * Errors: EINVAL (nulls, n_new out of range, dtypes), EUNSUPPORTED (q_lora
 * not a multiple of 16), EWORKSPACE, EHIP. */
int32_t dspark_cache_append(const dspark_model* m, const dspark_append_in* in, void* workspace,
                            size_t ws_bytes, void* stream);

/* Verification of a sampled draft block (huggingface.co "Kimi-K3-DSpark-
 * NVFP4", "Sampling options": rejection_sample_method verifies the block token
 * by token or "as a unit").  With q_i = softmax(draft_logits[s][i] / T) and
 * p_i = softmax(target_logits[s][i] / T) (i = block: after the whole block):
 *   DSPARK_VERIFY_TOKEN: accept x_i while u[s][i] < min(1, p_i(x_i) / q_i(x_i));
 *     at the first rejection draw the next token from max(p_i - q_i, 0), after
 *     a fully accepted block from p_block;
 *   DSPARK_VERIFY_BLOCK: w_0 = 1, w_k = min(w_{k-1} p_{k-1}(x_{k-1}) /
 *     q_{k-1}(x_{k-1}), 1); length k is accepted when u[s][k-1] < h_k with
 *     h_k = S_k / (S_k + 1 - w_k), S_k the mass of max(w_k p_k - q_k, 0)
 *     (h_block = w_block); the result is the largest accepted k, and the next
 *     token is drawn from max(w_k p_k - q_k, 0) (from p_block when k = block).
 * Draws: the lowest index whose cumulative mass exceeds u[s][block] times the
 * total.  Outputs: out_len[s] in [0, block] accepted draft tokens and
 * out_token[s] the next token.  All pointers are device pointers;
 * asynchronous on `stream`; a draft token outside [0, vocab) is rejected. */
#define DSPARK_VERIFY_TOKEN 0
#define DSPARK_VERIFY_BLOCK 1
typedef struct dspark_verify_in {
  int32_t n_seq, block, vocab, method;  /* 1 <= block <= 63                       */
  float temperature;            /* > 0                                           */
  int32_t pad_;
  const int32_t* draft;         /* [n_seq][block]                                */
  const float* draft_logits;    /* [n_seq][block][vocab]                          */
  const float* target_logits;   /* [n_seq][block + 1][vocab]                      */
  const float* u;               /* [n_seq][block + 1] uniforms in [0, 1)          */
} dspark_verify_in;

/* Workspace bytes dspark_verify needs (0 and the error text on bad sizes):
 * per-chunk normalisers and residual masses and per-row scalars, caller-owned
 * device memory, 256-byte aligned. */
size_t dspark_verify_workspace_bytes(int32_t n_seq, int32_t block);

/* Errors: EINVAL (nulls, sizes, method, temperature), EWORKSPACE, EHIP. */
int32_t dspark_verify(const dspark_verify_in* in, int32_t* out_len, int32_t* out_token, void* workspace,
                      size_t ws_bytes, void* stream);

/* Acceptance length (huggingface.co card, "Why acceptance is so sensitive":
 * a block is accepted up to its first mismatch): out_len[s] = the largest
 * k <= block with draft[s][j] == verifier[s][j] for all j < k.  Device
 * pointers, asynchronous on `stream` (NULL is the device's null stream, as
 * everywhere in this header; the host form is dspark_accept_len_host).
 * Token values are not range-checked.  Errors: EINVAL (nulls, negative
 * sizes), EHIP. */
int32_t dspark_accept_len(const int32_t* draft, const int32_t* verifier, int32_t n_seq,
                          int32_t block, int32_t* out_len, void* stream);

/* Same on host pointers, synchronous, no device needed. */
int32_t dspark_accept_len_host(const int32_t* draft, const int32_t* verifier, int32_t n_seq,
                               int32_t block, int32_t* out_len);

/* Decode one repacked matrix of the model back to float [rows][cols] (device
 * pointer `out`) with the same per-lane decoders the GEMM kernels use.
 * Accepted ids: DSPARK_W_FC, DSPARK_W_LM_HEAD, DSPARK_W_MARKOV_W2 and per layer
 * Q_B, O, DOWN, Q_A (rows of q_a then kv_a, fused on the device) and GATE
 * (rows of gate then up).  Q8_0 gives d*q and BF16 / F32 the stored value,
 * all exact in fp32; FP8 gives s*e4m3(q) rounded to nearest fp32.
 * Asynchronous on `stream`.  Intended for tests. */
int32_t dspark_dequant(const dspark_model* m, int32_t weight_id, float* out, void* stream);

/* Read-bandwidth probe (a measurement aid, no part of the draft pass): reads
 * `bytes` bytes of device memory at `buf` once, with the 16-byte
 * non-temporal loads and the kind of grid the weight-streaming GEMMs use, and
 * writes one 32-bit XOR of the words each workgroup read to out[0 .. 2047]
 * (device memory, 2048 entries, so that no load can be dropped).  Timing it
 * gives the achievable streaming-read rate that the GEMMs' rates are compared
 * with.  buf must be 16-byte aligned and bytes a multiple of 16.
 * Asynchronous on `stream`; DSPARK_EINVAL for a NULL, misaligned or
 * mis-sized argument. */
int32_t dspark_read_probe(const void* buf, size_t bytes, uint32_t* out, void* stream);

/* Thread-local text of the last error ("" if none). */
const char* dspark_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
