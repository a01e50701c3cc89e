/*
 * swiftkv.h -- C ABI of the MI355X (gfx950) SwiftKV prefill library.
 *
 * SwiftKV ("SwiftKV: Fast Prefill-Optimized Inference with Knowledge-
 * Preserving Model Transformation", arXiv 2410.03960) rewires a Llama-style
 * GQA decoder so that prompt tokens run only layers 1..l.  After layer l the
 * KV cache of every later layer j is computed from the one hidden state
 * x_{l+1} (summary page, section 3.4, Eq. 2: KV_j = W_KV^j . x_{l+1}), and
 * only the last prompt token continues through layers l+1..L to produce the
 * first-token logits (section 3.4, "What the first generated token does
 * differently").  AcrossKV (section 3.4, Eq. KV_group) lets each group of g
 * consecutive skipped layers share one KV tensor.  The paper's section 3.5
 * ("Optimized Implementation for Inference", quoted on the
 * AI_PARSE_DOCUMENT page) states the serving form: after layer l the KV of
 * the remaining layers is computed at once and the prompt tokens exit.
 *
 * Everything is asynchronous on the caller's HIP stream except where a
 * function says it is synchronous.  No C++ exception crosses this ABI; every
 * failure returns a negative skv_status and leaves a message readable through
 * skv_last_error() on the calling thread.
 *
 * Conventions
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary CPU memory.  Weight pointers may be either (the
 *     copy direction is inferred from unified addressing).
 *   - Linear weights are row-major [out_features, in_features] (output row n
 *     holds the n-th weight vector), RMSNorm gains are [d_model].
 *   - bf16 tensors are raw IEEE bfloat16 bit patterns (uint16_t).
 *   - Layers are numbered 1..n_layers.
 */
#ifndef SWIFTKV_H_
#define SWIFTKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SKV_OK = 0,
  SKV_ERR_INVALID_ARG = -1, /* argument or shape check failed on the host; nothing was enqueued */
  SKV_ERR_OOM = -2,         /* device allocation failed */
  SKV_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
  SKV_ERR_UNSUPPORTED = -4  /* valid but not implemented for this shape/dtype */
} skv_status;

typedef enum { SKV_BF16 = 0, SKV_FP32 = 1, SKV_FP8_E4M3 = 2 /* cache views only */ } skv_dtype;

/* What the KV cache stores (Appendix B.1 / Table B.1: AcrossKV combined
 * with a per-token FP8 KV cache).
 * SKV_KV_MODEL: K/V in the model dtype.
 * SKV_KV_FP8: OCP FP8 E4M3 codes (bias 7, largest finite value 448) plus
 * one fp32 scale per token position, per KV slot, for K and V separately:
 * scale = max|x| / 448 over the token's K (or V) row across all kv heads,
 * code = E4M3 round-to-nearest-even of x * (1 / scale) clamped to +-448
 * (each step one fp32 operation); the cached value is code * scale.  Every
 * attention (prompt tokens and last tokens alike) reads the cached values.
 * bf16 models only, n_kv_heads * head_dim <= 1024. */
typedef enum { SKV_KV_MODEL = 0, SKV_KV_FP8 = 1 } skv_kv_dtype;

/* Model description.  The transformation is the one of section 3.4:
 * swiftkv_l = number of layers every prompt token runs (0..n_layers;
 * n_layers means no skipping, 0 means every layer's KV comes from the
 * embeddings), acrosskv_g = AcrossKV group size (1 = no merging).
 * Groups are consecutive skipped layers l+1..l+g, l+g+1..l+2g, ...; the
 * first layer of a group is its representative; a short last group is
 * allowed.
 * dtype SKV_BF16: bf16 weights, activations and KV cache, fp32 accumulation,
 * fp32 residual stream, fp32 logits.  SKV_FP32: fp32 throughout.
 * max_tokens / max_batch / max_seqlen size the workspace reserved at create
 * time: a skv_prefill call may carry at most max_tokens prompt tokens in at
 * most max_batch prompts of at most max_seqlen tokens each. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rope_theta; /* RoPE base: pair i of a head rotates by pos * theta^(-2i/head_dim) */
  float rms_eps;    /* RMSNorm epsilon */
  int32_t swiftkv_l;
  int32_t acrosskv_g;
  int32_t dtype; /* skv_dtype */
  int32_t max_tokens, max_batch, max_seqlen;
  int32_t kv_dtype; /* skv_kv_dtype */
} skv_model_config;

typedef struct skv_model skv_model;
typedef struct skv_kv_cache skv_kv_cache;

/* One layer's weights, dtype = the model's dtype.  For a skipped layer
 * (layer > swiftkv_l) wk/wv are read only if the layer is its AcrossKV
 * group's representative and may be NULL otherwise. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *w_gate, *w_up, *w_down;
} skv_layer_weights;

/* Validate cfg and reserve device memory for weights and workspace on the
 * current device.  Synchronous.  Errors: INVALID_ARG (bad dims, l outside
 * 0..n_layers, g < 1, head counts not dividing), UNSUPPORTED (bf16 needs
 * head_dim 128, q heads per kv head a multiple of 4, d_model and ffn_dim
 * multiples of 128, max_batch <= 32), OOM. */
skv_status skv_model_create(const skv_model_config* cfg, skv_model** out);

/* Copy the embedding [vocab, d_model], the final RMSNorm gain [d_model] and
 * the (untied) LM head [vocab, d_model] into the model, values unchanged.
 * Synchronous; the caller's buffers may be reused when it returns. */
skv_status skv_model_load_globals(skv_model* m, const void* embed, const void* final_norm, const void* lm_head);

/* Copy layer `layer`'s weights into the model and repack them on the
 * device: Q/K/V rows concatenated for unskipped layers; gate and up rows
 * interleaved; for an AcrossKV representative j > l, its input-RMSNorm gain
 * folded into its K and V rows (W~ = W_KV diag(gamma_j), the one weight the
 * library changes, as the skipped-layer projection is defined: exact in real
 * arithmetic, RMSNorm(x; gamma) W^T = r (x (W diag gamma)^T) with
 * r = 1/sqrt(mean x^2 + eps); bf16 models round W~ to bf16).  Every other
 * weight keeps its values: bf16 projections take bf16(x * gamma) and scale
 * their products by r (in the GEMM epilogues or the skinny products'
 * finalize pass).  Synchronous. */
skv_status skv_model_load_layer(skv_model* m, int32_t layer, const skv_layer_weights* w);

/* Free everything the model owns.  Accepts NULL. */
void skv_model_destroy(skv_model* m);

/* Paged KV cache for the model: num_kv_slots(m) slots (swiftkv_l unskipped
 * layers + one per AcrossKV group), each holding num_blocks blocks of
 * block_size token positions for every kv head.  block_size must be 16.
 * Zero-filled at creation.  Synchronous. */
skv_status skv_kv_cache_create(const skv_model* m, int32_t num_blocks, int32_t block_size, skv_kv_cache** out);
void skv_kv_cache_destroy(skv_kv_cache* c);
int32_t skv_num_kv_slots(const skv_model* m);

/* Non-owning strided view of one cache tensor, valid until the cache is
 * destroyed.  Element (i0, i1, i2, i3) lives at data + sum_k i_k*stride[k]
 * elements. */
typedef struct {
  void* data;
  int32_t dtype; /* skv_dtype */
  int32_t ndim;
  int64_t shape[4];
  int64_t stride[4];
} skv_tensor_view;

/* K and V of layer `layer` (1-based).  Layers of one AcrossKV group return
 * the same memory.  Layout of both: [num_blocks, n_kv_heads, block_size,
 * head_dim]; dtype = the model's, or SKV_FP8_E4M3 (codes) with an FP8
 * cache.  Token position p of a prompt with block table row bt lives in
 * block bt[p / block_size] at offset p % block_size.  K holds RoPE-rotated
 * keys.  Positions of a prompt's last block beyond its length keep whatever
 * they held (zero after creation); they must stay finite. */
skv_status skv_kv_cache_view(const skv_kv_cache* c, int32_t layer, skv_tensor_view* k, skv_tensor_view* v);

/* Per-token scales of layer `layer`'s K and V in an FP8 cache: fp32
 * [num_blocks, block_size], position p at [bt[p / block_size], p %
 * block_size]; the value of a K element is its code's E4M3 value times the
 * K scale of its position.  INVALID_ARG if the cache is not FP8. */
skv_status skv_kv_cache_scales(const skv_kv_cache* c, int32_t layer, skv_tensor_view* k_scale,
                               skv_tensor_view* v_scale);

/* A batch of independent prompts packed back to back (varlen).
 * cu_seqlens[b]..cu_seqlens[b+1] are prompt b's tokens; every prompt has at
 * least one token.  block_tables is [batch, max_blocks_per_seq] physical
 * block ids; prompt b needs ceil(len_b / block_size) valid entries.  The
 * host copies are used for validation and launch geometry and must hold the
 * same values as the device copies. */
typedef struct {
  int32_t batch;
  int32_t total_tokens;
  int32_t max_seqlen;
  int32_t max_blocks_per_seq;
  const int32_t* cu_seqlens_host;   /* host   [batch + 1] */
  const int32_t* block_tables_host; /* host   [batch * max_blocks_per_seq] */
  const int32_t* token_ids;         /* device [total_tokens], ids in [0, vocab) */
  const int32_t* cu_seqlens;        /* device [batch + 1] */
  const int32_t* block_tables;      /* device [batch * max_blocks_per_seq] */
} skv_batch;

/* SwiftKV prefill (section 3.4 "Inference Implementation"; section 3.5):
 *  1. every prompt token runs layers 1..l (RMSNorm, QKV + RoPE, causal GQA
 *     attention, O + residual, RMSNorm, SwiGLU MLP + residual), its K/V
 *     written to slots 0..l-1;
 *  2. one GEMM of x_{l+1} (RMS-normalised) against the concatenated folded
 *     K/V rows of every AcrossKV group (Eq. 2 / Eq. KV_group) writes, after
 *     RoPE on K, the KV of slots l..l+G-1 for every token, the last included;
 *  3. the last token of each prompt runs layers l+1..L, attending at layer j
 *     to the N positions of its slot;
 *  4. logits[b, :] = RMSNorm(y_b; final gain) W_lm^T in fp32.
 * Writes the cache positions the batch covers and logits (device, fp32,
 * [batch, vocab]).  Asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream); the caller synchronises.  Every layer must have been
 * loaded.  Errors (host-side, nothing enqueued): INVALID_ARG for
 * inconsistent cu_seqlens, an empty prompt, total_tokens > max_tokens,
 * batch < 1 or > max_batch, a prompt longer than max_seqlen, a block table entry
 * outside [0, num_blocks) or too few blocks; HIP on launch failure. */
skv_status skv_prefill(skv_model* m, skv_kv_cache* c, const skv_batch* batch, float* logits, void* stream);

/* A batch of sequences that may already hold cached positions: sequence b
 * has ctx_lens[b] positions in the cache (written by earlier calls with the
 * same block-table entries) and brings the new tokens
 * tokens.cu_seqlens[b]..[b+1], at positions ctx_lens[b] onwards.  Its block
 * table must cover ctx_lens[b] + (new tokens) positions.  tokens.max_seqlen
 * bounds the new tokens of one sequence; ctx_lens[b] + new tokens must not
 * exceed the model's max_seqlen.  Both ctx arrays NULL = no cached
 * positions (the call is then a prefill). */
typedef struct {
  skv_batch tokens;
  const int32_t* ctx_lens_host; /* host   [batch] */
  const int32_t* ctx_lens;      /* device [batch], same values */
  /* host [batch] or NULL (= every entry nonzero): nonzero where the call is
   * to produce sequence b's next-token logits (a decode token, a prompt's
   * final chunk); 0 for a prompt chunk that more chunks follow. */
  const int32_t* need_logits_host;
} skv_step_batch;

/* One forward pass over a mixed batch of prompt chunks and decode tokens
 * (section 3.5 "Optimized Implementation for Inference"; "Inference
 * Implementation in Production Serving Frameworks", chunked prefill):
 *  1. every new token runs layers 1..l, attending to its sequence's cached
 *     positions and to the new tokens up to its own; its K/V go to slots
 *     0..l-1 at its position;
 *  2. the K/V of slots l..l+G-1 (every skipped layer / AcrossKV group) are
 *     computed from x_{l+1} of every new token, as in skv_prefill;
 *  3. the last new token of each sequence runs layers l+1..L, attending at
 *     layer j to all ctx + new positions of its slot;
 *  4. logits[b, :] = RMSNorm(y_b; final gain) W_lm^T, the next-token logits
 *     after that token (a decode token's, a final prompt chunk's first
 *     generated token; a caller ignores the row of an unfinished chunk).
 * When need_logits_host marks no sequence, steps 3 and 4 are skipped: only
 * a prompt's last token runs the layers past l, and a chunk that more
 * chunks follow does not hold it; the call then writes no logits and
 * `logits` may be NULL.  Otherwise every row is computed as above.
 * A decode token is a sequence with one new token.  Splitting a prompt into
 * chunks fed one call after another yields the cache and final logits of
 * skv_prefill over the whole prompt.  Same asynchrony, ownership and errors
 * as skv_prefill, plus INVALID_ARG for a negative ctx_lens entry or only one
 * of the two ctx arrays given. */
skv_status skv_step(skv_model* m, skv_kv_cache* c, const skv_step_batch* batch, float* logits, void* stream);

/* For callers that cannot allocate device memory during a call (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): skv_step over a batch of at most 32 new tokens (decode steps,
 * short chunks) on a bf16 model with a bf16 cache, with every scratch
 * buffer of the call (residual rows, bf16 rows, split-K and attention
 * partials, per-token metadata) taken from a static device array of
 * 64 MiB that the library holds on each device for the life of the
 * process, instead of the model's workspace.  Same arguments, results,
 * asynchrony and ownership as skv_step; it calls no allocator.  The array
 * is shared by every call on a device and keeps the last call's contents:
 * calls that overlap on one device (different streams, or different
 * threads) race on it and must be serialised by the caller.  Errors:
 * skv_step's, plus INVALID_ARG for more than 32 new tokens or a call whose
 * scratch (which grows with rows x q heads x the longest context) exceeds
 * 64 MiB, or no model created on the current device; UNSUPPORTED for an
 * fp32 model or an FP8 cache. */
skv_status skv_step_noalloc(skv_model* m, skv_kv_cache* c, const skv_step_batch* batch, float* logits,
                            void* stream);

/* Closed-form FLOPs of a prefill over prompts of the given lengths (host
 * array), counted the way the summary page's section 3.4 Table 1 ("FLOPs per
 * prefill token", Llama-3.1-70B) breaks a forward pass down: the K/V, Q/O
 * and MLP projections, attention and the vocabulary projection.
 * full = the unmodified model (all layers for every token, LM head for the
 * last token); swiftkv = layers 1..l for every token, one K/V projection
 * per AcrossKV group for every token (Eq. 2 / Eq. KV_group), layers l+1..L
 * for the last token.  Matmuls count 2mnk, attention 4*ctx*head_dim per
 * query per head.  Host only.  INVALID_ARG for a bad config, a negative
 * batch, NULL seqlens with batch > 0 or a NULL output. */
skv_status skv_flops(const skv_model_config* cfg, const int32_t* seqlens, int32_t batch, double* full,
                     double* swiftkv);

/* Kernel classes that skv_profile_* can time.  SKV_K_ATTN_PREFILL is the
 * prompt-token attention of every layer that runs it in plain form;
 * SKV_K_ATTN_PREFILL_SPLIT is layer 1's attention in split-bf16 form (bf16
 * models, bf16 cache), which issues three products per score and per
 * output block, so its rate is kept apart. */
typedef enum {
  SKV_K_GEMM_QKV = 0,
  SKV_K_ATTN_PREFILL = 1,
  SKV_K_GEMM_O = 2,
  SKV_K_GEMM_GATEUP = 3,
  SKV_K_GEMM_DOWN = 4,
  SKV_K_GEMM_KVSKIP = 5,
  SKV_K_RMSNORM = 6,
  SKV_K_LAST_TOKEN = 7,
  SKV_K_ATTN_PREFILL_SPLIT = 8,
  SKV_K_NUM = 9
} skv_kernel_class;

/* Bracket every launch of one kernel class with HIP events on the prefill
 * stream (enable != 0) or stop doing so.  Clears earlier records. */
skv_status skv_profile_enable(skv_model* m, int32_t kernel_class, int32_t enable);

/* Synchronise the recorded events and report, over the launches of the
 * enabled class since skv_profile_enable: total device time (ms), launch
 * count, algorithmic FLOPs and algorithmic HBM bytes of those launches. */
skv_status skv_profile_read(skv_model* m, double* total_ms, int64_t* launches, double* flops, double* bytes);

/* Measurement aid, not part of the method: the dense bf16 MFMA throughput
 * of this GPU.  Runs one workgroup of 4 waves per compute unit, each wave
 * issuing iters x 64 v_mfma_f32_16x16x32_bf16 (the GEMMs' instruction) on
 * 64 independent accumulators from operands held in registers (no memory
 * traffic in the loop), once untimed and once timed with HIP events on `stream`;
 * synchronous (returns when the timed run is done; allocates and frees
 * its own small device buffers).  random_operands != 0 fills the operands
 * with random sign and mantissa bits at the magnitudes of N(0, 0.02)
 * weights, else with one constant (operand toggling sets the chip's power
 * draw and so its clock).  Outputs: tflops (dense, 2 FLOPs per
 * multiply-add), clock_mhz (the shader clock the loop ran at, averaged over
 * workgroups), cus (compute units) and max_clock_mhz (the device's peak
 * engine clock).  INVALID_ARG for iters outside [1, 2^22] or a NULL
 * output; HIP for a failed allocation, copy or launch. */
skv_status skv_mfma_probe(int32_t random_operands, int32_t iters, void* stream, double* tflops, double* clock_mhz,
                          int32_t* cus, double* max_clock_mhz);

/* Message of the last failure on this thread ("" if none). */
const char* skv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SWIFTKV_H_ */
