/*
 * libdllm — one denoising step of block-wise masked-diffusion LLM generation with an
 * approximate KV cache and confidence-aware parallel decoding (Fast-dLLM), for AMD
 * MI355X (gfx950).
 *
 * The method, as described by
 *   [A] the ccyt168.com Fast-dLLM article, section 1.1 "Block-Wise KV Cache" and
 *       section 1.2 "Confidence-Aware Parallel Decoding", and
 *   [B] the techwalker.com explainer "Fast-dLLM: NVIDIA researchers accelerate
 *       diffusion LLMs without training via KV cache and parallel decoding", sections
 *       "Core innovation: a KV cache suited to diffusion models" and "Solving the
 *       quality loss of parallel decoding":
 *   - the generated span is cut into blocks decoded left to right;
 *   - before a block, the KV of every position is computed by a full bidirectional
 *     forward and kept; after the block it is recomputed ([B], steps 1 and 2);
 *   - DualCache keeps the prompt prefix and the masked suffix; prefix mode keeps only
 *     the prefix ([A] 1.1, [B]);
 *   - each step decodes, in parallel, every masked position of the block whose
 *     confidence (the probability the model gives its argmax token) reaches the
 *     threshold; the others wait ([A] 1.2, [B]).
 * Readings where the pages are silent (each used identically by the CPU oracle):
 *   the mask token is never emitted; confidence >= threshold; argmax ties go to the
 *   lowest token id; a sequence with masked block positions but none at the threshold
 *   decodes its single most confident one (lowest position on ties); a refresh decodes
 *   nothing; sequences of a batch move through blocks in lockstep.
 *
 * Model (readings; the pages only name LLaDA and Dream): pre-norm transformer with
 * RMSNorm, rotate-half RoPE, SwiGLU FFN, no biases, untied LM head, grouped-query
 * attention allowed (query head h reads KV head h / (n_heads / n_kv_heads)),
 * bidirectional attention (no mask), LM-head output multiplied by logit_scale.
 *
 * Precision.  DLLM_F32: every tensor fp32.  DLLM_BF16: weights and KV cache bf16;
 * residual stream, logits and confidences fp32; RMSNorm outputs, post-RoPE q/k, v,
 * attention outputs and SwiGLU outputs rounded to bf16 (nearest even); all
 * accumulation fp32.
 *
 * Memory and ownership.  Every pointer in a descriptor is device memory owned by the
 * caller (the per-layer pointer arrays themselves are host arrays).  The library
 * allocates no device memory and keeps no pointer after a call returns.
 *
 * Errors.  Every call returns a dllm_status and never throws.  Arguments are checked
 * on the host before anything is enqueued, so an error leaves tokens, cache and
 * workspace untouched; dllm_last_error() gives a one-line reason (thread-local).
 * DLLM_E_HIP means a HIP call failed after work was enqueued: tokens and cache are
 * then unspecified; restore the tokens of the last block boundary and call
 * dllm_prefill_cache / dllm_refresh_cache again.
 *
 * Streams.  prefill, refresh, block_step and the kernel-level calls only enqueue on
 * `stream`; their outputs are valid once the stream reaches that point.  dllm_generate
 * is synchronous.  One sequence descriptor (tokens + cache + workspace) must not be
 * driven from two streams at once.
 */
#ifndef DLLM_H
#define DLLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* dllm_stream_t; /* a hipStream_t; NULL is the null stream */

typedef enum {
  DLLM_OK = 0,
  DLLM_E_NULL = -1,        /* a required pointer is NULL                               */
  DLLM_E_SHAPE = -2,       /* inconsistent sizes (e.g. gen_len % block_len != 0)        */
  DLLM_E_UNSUPPORTED = -3, /* valid but not implemented (e.g. block_len > 64)           */
  DLLM_E_WORKSPACE = -4,   /* workspace or cache buffer smaller than required           */
  DLLM_E_HIP = -5,         /* a HIP runtime call failed                                 */
  DLLM_E_STATE = -6,       /* block index out of range                                  */
  DLLM_E_ARG = -7          /* bad scalar argument (NaN threshold, bad enum, mask id)    */
} dllm_status;

typedef enum { DLLM_F32 = 0, DLLM_BF16 = 1 } dllm_dtype;
/* DLLM_CACHE_NONE: no approximate cache, the reference the cached modes approximate
 * (every denoising step is a full forward over all S positions of the current tokens;
 * the kv_cache buffer is still needed as the forward's K/V scratch).                 */
typedef enum { DLLM_CACHE_NONE = 0, DLLM_CACHE_PREFIX = 1, DLLM_CACHE_DUAL = 2 } dllm_cache_mode;

/* Model weights.  Shapes are row-major; "T" is float (DLLM_F32) or bf16 (DLLM_BF16).
 * Supported: head_dim divides 128 (and is even); n_heads % n_kv_heads == 0;
 * d_model, d_ffn and n_heads*head_dim multiples of 64; for DLLM_BF16 also head_dim ==
 * 128, d_model, d_ffn, n_heads*head_dim multiples of 256 and vocab a multiple of 8.
 * mask_id in [0, vocab).
 * Token ids in `tokens` must lie in [0, vocab) (others are clamped, never read out of
 * bounds).                                                                           */
typedef struct {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, d_ffn, vocab, mask_id;
  float rope_theta, norm_eps, logit_scale;
  int32_t dtype;                      /* dllm_dtype                                      */
  const void* embed;                  /* T [vocab, d_model]                              */
  const void* final_norm;             /* T [d_model]                                     */
  const void* lm_head;                /* T [vocab, d_model]                              */
  const void* const* attn_norm;       /* n_layers x T [d_model]                          */
  const void* const* w_qkv;           /* n_layers x T [(n_heads+2*n_kv_heads)*head_dim, d_model]:
                                         q rows, then k rows, then v rows               */
  const void* const* w_o;             /* n_layers x T [d_model, n_heads*head_dim]        */
  const void* const* ffn_norm;        /* n_layers x T [d_model]                          */
  const void* const* w_gate_up;       /* n_layers x T [2*d_ffn, d_model]: gate rows first */
  const void* const* w_down;          /* n_layers x T [d_model, d_ffn]                   */
} dllm_model_desc;

/* One batch of sequences being generated.  S = prompt_len + gen_len.
 * tokens: device int32 [batch, S], in/out; the generated span must hold mask_id before
 *   the first call; decoded tokens are written in place.
 * kv_cache: device buffer of dllm_kv_cache_bytes(); layout per layer l (in elements of
 *   T, Sp = S rounded up to a multiple of 64):
 *     K  at l*2*B*Hkv*Sp*D                 : [B][Hkv][Sp][D]  (post-RoPE keys)
 *     Vt at l*2*B*Hkv*Sp*D + B*Hkv*Sp*D    : [B][Hkv][Sp/32][D][32]  (values, transposed
 *        in blocks of 32 positions: value (dim d, position p) of one (sequence, KV head)
 *        at ((p / 32) * D + d) * 32 + p % 32)
 *   positions >= S are never read.
 * workspace: device scratch of dllm_workspace_bytes(); dllm_prefill_cache initialises
 *   it and must run before the first dllm_block_step / dllm_refresh_cache.           */
typedef struct {
  int32_t batch, prompt_len, gen_len, block_len;
  int32_t cache_mode;                 /* dllm_cache_mode                                 */
  float threshold;                    /* confidence threshold, e.g. 0.9                  */
  int32_t* tokens;
  void* kv_cache;
  size_t kv_cache_bytes;
  void* workspace;
  size_t workspace_bytes;
} dllm_seq_desc;

typedef struct {
  int32_t steps;                      /* denoising steps run (each block's first one
                                         fused with its refresh)                         */
  int32_t refreshes;                  /* full forwards run (prefill included)            */
  int32_t tokens;                     /* tokens generated (batch * gen_len)              */
  int32_t blocks;
  double ms_total, ms_refresh, ms_step; /* host wall clock: whole call; from each block's
                                         refresh to its outcome; the block's later steps */
  int32_t* steps_per_block;           /* optional host array [gen_len/block_len], or NULL */
  int32_t speculative_steps;          /* steps queued ahead that found the block already
                                         finished (decode nothing; not in `steps`)       */
  int64_t masked_at_step_start;       /* masked block positions when each step began,
                                         summed over steps and sequences: tokens divided
                                         by it is the mean fraction unmasked per step    */
} dllm_stats;

/* Sizes (host only, no device work).  Return 0 if the descriptors are invalid.       */
size_t dllm_workspace_bytes(const dllm_model_desc* m, const dllm_seq_desc* s);
size_t dllm_kv_cache_bytes(const dllm_model_desc* m, const dllm_seq_desc* s);

/* Prefill = the full forward before block 0 ([B] step 1): initialises the workspace
 * and writes every layer's K/V for all S positions.  Decodes nothing.               */
dllm_status dllm_prefill_cache(const dllm_model_desc* m, const dllm_seq_desc* s,
                               dllm_stream_t stream);

/* Refresh after block `block` is finished ([B] step 2): full bidirectional forward
 * over all S positions of the current tokens; K/V rewritten in place.  The last
 * layer's output projection and FFN are skipped (they do not feed any K/V).
 * block in [0, gen_len/block_len).  Decodes nothing.                                */
dllm_status dllm_refresh_cache(const dllm_model_desc* m, const dllm_seq_desc* s,
                               int32_t block, dllm_stream_t stream);

/* One cached denoising step of block `block` ([A] 1.1 and 1.2; with DLLM_CACHE_NONE the
 * step is the full forward of dllm_refresh_step):
 *   DualCache: the block rows [s0, s1) are recomputed through every layer and attend
 *   to all S cached keys (their own K/V written in place first); prefix mode: rows
 *   [s0, S) are recomputed and only [0, s0) comes from the cache.  Then the final
 *   norm and LM head over the block rows, the vocab-wide confidence/argmax (mask id
 *   excluded), and the threshold unmask, which writes decoded tokens into `tokens`.
 * Outputs (device, may be NULL unless stated):
 *   d_n_unmasked [batch] int32 (required): tokens decoded this step per sequence;
 *   d_remaining  [batch] int32 (required): mask tokens left in the block;
 *   d_logits [batch*block_len, vocab] fp32: the block rows' logits;
 *   d_conf [batch, block_len] fp32 and d_argmax [batch, block_len] int32.           */
dllm_status dllm_block_step(const dllm_model_desc* m, const dllm_seq_desc* s, int32_t block,
                            dllm_stream_t stream, int32_t* d_n_unmasked, int32_t* d_remaining,
                            float* d_logits, float* d_conf, int32_t* d_argmax);

/* A block's refresh fused with its first denoising step.  By [A] property (a) the first
 * step after a refresh equals the full forward, so the full forward over all S
 * positions (K/V of every layer rewritten in place; for block 0 this is the prefill
 * and also initialises the workspace, as dllm_prefill_cache does) is followed only by
 * the last layer over the block rows [s0, s1) against all S fresh keys, the final
 * norm, LM head, confidence and unmask.  Outputs as for dllm_block_step; the result
 * equals dllm_refresh_cache (or dllm_prefill_cache) then dllm_block_step up to
 * floating-point rounding order.                                                     */
dllm_status dllm_refresh_step(const dllm_model_desc* m, const dllm_seq_desc* s, int32_t block,
                              dllm_stream_t stream, int32_t* d_n_unmasked, int32_t* d_remaining,
                              float* d_logits, float* d_conf, int32_t* d_argmax);

/* Whole generation: for every block, dllm_refresh_step (the prefill for block 0), then
 * cached steps until the block has no mask token left (one 4*batch-byte device-to-host
 * read per step); with DLLM_CACHE_NONE every step is a dllm_refresh_step.  The next
 * step is queued before the previous step's read completes whenever that read may not
 * end the block (some sequence had two or more masks left), so the device does not wait
 * for launches; such a step that finds the block finished decodes nothing and is
 * counted in speculative_steps.  Tokens are those of the step-by-step loop.
 * Synchronous.  `out` may be NULL.                                                   */
dllm_status dllm_generate(const dllm_model_desc* m, const dllm_seq_desc* s,
                          dllm_stream_t stream, dllm_stats* out);

/* dllm_generate with each block's cached steps replayed from a HIP graph: the block's
 * first cached step is captured on `stream` (its kernels only; the per-step 4*batch-byte
 * read stays outside) and replayed for the block's later steps.  Same kernels, same
 * results as dllm_generate, bit for bit.  DLLM_E_UNSUPPORTED while a kernel class is
 * being timed (dllm_profile_select): its events cannot be recorded inside a graph.    */
dllm_status dllm_generate_graphs(const dllm_model_desc* m, const dllm_seq_desc* s,
                                 dllm_stream_t stream, dllm_stats* out);

/* Cache staleness: how far the block-wise approximate cache is from the exact K/V of
 * the current tokens.  [A] 1.1 checks that the K/V activations of adjacent steps have a
 * cosine similarity close to 1 and [B] "Core innovation" shows the same similarity;
 * this measures it for the cache a cached step of `block` would read now.  A full
 * forward of the current tokens writes the exact K/V into fresh_cache (caller-owned,
 * dllm_kv_cache_bytes() bytes, the kv_cache layout); then, per layer and for K and V,
 * the cosine similarity of the cached and the fresh D-vector of every (sequence, KV
 * head, position) the step takes from the cache (DualCache: every position outside the
 * block; prefix mode: the positions before it), averaged and minimised.  A vector pair
 * with both norms zero counts 1, with one zero norm 0.
 *   out: device float [n_layers][2][2] = {K mean, K min}, {V mean, V min}.
 *   reuse: host double, may be NULL: the reuse ratio, the fraction of the S positions
 *     whose K/V the step takes from the cache (DualCache (S - block_len) / S; prefix
 *     mode s0 / S); written before the call returns.
 * tokens and kv_cache are not modified; the workspace is (as by any step).  Needs a
 * cache mode other than DLLM_CACHE_NONE and a prior dllm_prefill_cache.             */
dllm_status dllm_cache_staleness(const dllm_model_desc* m, const dllm_seq_desc* s,
                                 int32_t block, void* fresh_cache, size_t fresh_bytes,
                                 float* out, double* reuse, dllm_stream_t stream);

/* ---- kernel-level entries (single stages on caller buffers) ---------------------- */

/* Workspace needed by the two kernel-level calls below: the attention part for
 * (B, Hq, R, S, D) when all are positive (enough for any Hkv dividing Hq: with grouped
 * query heads the attention may split the keys into more, shorter chunks), the
 * confidence part for B sequences of K block positions over a vocabulary of V when K
 * and V are positive; the larger of the two.  Returns 0 if B < 1.                    */
size_t dllm_kernel_workspace_bytes(int32_t B, int32_t Hq, int32_t R, int32_t S, int32_t D,
                                   int32_t K, int32_t V);

/* Non-causal attention of R query rows per (sequence, query head) against S cached
 * keys ([A] 1.1: the block's queries read the cached KV of all positions).
 *   q  T [B][Hq][R][D];  k T [B][Hkv][Sp][D];  vt T [B][Hkv][Sp/32][D][32] (values
 *   transposed in blocks of 32 keys, as in the KV cache; Sp >= S and a multiple of 32;
 *   keys >= S ignored);  o T [B][R][Hq*D]  (row-major, ready for the output projection).
 *   o = softmax(q k^T / sqrt(D)) v over all S keys, fp32 softmax and accumulation.
 * Supported: DLLM_BF16 with D == 128, or DLLM_F32 with D <= 128; Hq % Hkv == 0.     */
dllm_status dllm_kernel_block_attention(const void* q, const void* k, const void* vt, void* o,
                                        int32_t B, int32_t Hq, int32_t Hkv, int32_t R,
                                        int32_t S, int32_t Sp, int32_t D, int32_t dtype,
                                        void* ws, size_t ws_bytes, dllm_stream_t stream);

/* Vocab-wide confidence and threshold unmask for B sequences of K block positions
 * ([A] 1.2).  logits T_l [B*K][V] with T_l = fp32 or bf16 (logits_dtype).  Per row:
 * m = max over v != mask_id, conf = 1 / sum_{v != mask_id} exp(z_v - m), argmax the
 * lowest id reaching m.  Then per sequence: U = {masked i : conf_i >= tau}, or the
 * most confident masked position if U is empty and something is masked;
 * tokens_block[b][i] = argmax for i in U.
 *   tokens_block int32 [B][K] (in/out, row stride ld_tokens);
 *   conf fp32 [B*K], argmax int32 [B*K], n_unmasked int32 [B], remaining int32 [B]
 *   (all required); unmasked_idx int32 [B][K] optional: the positions decoded this
 *   step in increasing order, then -1.  K <= 64.                                     */
dllm_status dllm_kernel_confidence_unmask(const void* logits, int32_t logits_dtype, int32_t B,
                                          int32_t K, int32_t V, int32_t mask_id, float tau,
                                          int32_t* tokens_block, int32_t ld_tokens,
                                          float* conf, int32_t* argmax, int32_t* n_unmasked,
                                          int32_t* remaining, int32_t* unmasked_idx, void* ws,
                                          size_t ws_bytes, dllm_stream_t stream);

/* dllm_kernel_confidence_unmask for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and outputs, with the slice partials in a static device array of the
 * library instead of a workspace (768 KiB per GPU the library runs on, held until the
 * process ends; its address is looked up on the first call on each device).  Allocates
 * nothing and calls no allocating routine.  DLLM_E_UNSUPPORTED when the pass needs more
 * than 65536 slice partials (B * K rows times the slices per row; at most 2048 per
 * sequence, so any B <= 32 fits); DLLM_E_ARG if `stream` belongs to another device than
 * the current one.  Every call on one GPU shares that array: calls that overlap on one
 * GPU (two streams, or two threads) race and must be serialised by the caller.       */
dllm_status dllm_kernel_confidence_unmask_noalloc(const void* logits, int32_t logits_dtype,
                                                  int32_t B, int32_t K, int32_t V,
                                                  int32_t mask_id, float tau,
                                                  int32_t* tokens_block, int32_t ld_tokens,
                                                  float* conf, int32_t* argmax,
                                                  int32_t* n_unmasked, int32_t* remaining,
                                                  int32_t* unmasked_idx, dllm_stream_t stream);

/* y = x W^T for x T [M][K], W T [N][K].  mode 0: y T [M][N]; mode 1: y fp32 [M][N] =
 * scale * x W^T; mode 2: y fp32 [M][N] += x W^T (residual add).  Same kernels as the
 * model path (MFMA for DLLM_BF16: K % 256 == 0, N % 8 == 0; fp32: K % 16 == 0).  ws from
 * dllm_linear_workspace_bytes().                                                     */
size_t dllm_linear_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t dtype);
dllm_status dllm_kernel_linear(const void* x, const void* w, void* y, int32_t M, int32_t N,
                               int32_t K, int32_t dtype, int32_t mode, float scale, void* ws,
                               size_t ws_bytes, dllm_stream_t stream);

/* ---- diagnostics -------------------------------------------------------------------- */

const char* dllm_status_string(dllm_status st);
const char* dllm_last_error(void);

/* Per-kernel-class timing with HIP events on the launching stream.  Select one class
 * (or -1 for none); every later launch of that class (with dllm_profile_select_every:
 * one launch in `every`, counted over all launches of the class, so a stride coprime
 * with the layer count visits every layer) is bracketed by two events (timing-only
 * events without a system-scope fence);
 * dllm_profile_read() synchronises on the recorded events and returns the number of
 * launches and their summed duration, then clears the record.  A GEMM class times the
 * GEMM kernel alone; the split-K reduction that applies a step GEMM's epilogue (QKV,
 * gate/up, LM head) is the class SPLIT_REDUCE.                                          */
typedef enum {
  DLLM_K_NONE = -1,
  DLLM_K_EMBED_NORM = 0, DLLM_K_RMSNORM, DLLM_K_STEP_QKV, DLLM_K_STEP_ATTN, DLLM_K_STEP_O,
  DLLM_K_STEP_GATE_UP, DLLM_K_STEP_DOWN, DLLM_K_LM_HEAD, DLLM_K_CONF_UNMASK,
  DLLM_K_REF_QKV, DLLM_K_REF_ATTN, DLLM_K_REF_O, DLLM_K_REF_GATE_UP, DLLM_K_REF_DOWN,
  DLLM_K_SPLIT_REDUCE,
  DLLM_K_COUNT
} dllm_kernel_class;
dllm_status dllm_profile_select(int32_t kernel_class);
/* As dllm_profile_select, sampling one launch in `every` (every >= 1; 1 = all).          */
dllm_status dllm_profile_select_every(int32_t kernel_class, int32_t every);
dllm_status dllm_profile_read(int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* DLLM_H */
