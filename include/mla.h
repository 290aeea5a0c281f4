/*
 * libmla -- Multi-head Latent Attention (MLA) over a compressed latent KV cache, for AMD
 * MI355X (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * The method (page "DeepSeek-Coder-V2的MLA多头潜在注意力深度解析 512维潜空间压缩KV缓存的完整原理",
 * mtrt.cn/news/26941, sections "MLA 的两个核心部件" and "源码里的压缩全流程"):
 *   - every token's hidden state x is compressed by kv_a_proj_with_mqa into a latent c
 *     (kv_lora_rank values, RMS-normalised by kv_a_layernorm) and a RoPE key k_pe
 *     (qk_rope_head_dim values) that all heads share; only [c | k_pe] is cached;
 *   - queries take the low-rank path q_b_proj(q_a_layernorm(q_a_proj(x))) (or one q_proj),
 *     and split per head into [q_nope | q_pe] with RoPE on q_pe;
 *   - kv_b_proj maps a latent back to per-head [k_nope | v]; attention is softmax over
 *     sigma * (q_nope . k_nope + q_pe . k_pe), weighting v.
 * Decode evaluates the same attention in the weight-absorbed form: q_nope is mapped through
 * the k_nope rows of kv_b_proj into latent space, scored directly against the cached rows,
 * the softmax-weighted sum of latents is taken, and the v rows of kv_b_proj map it to the
 * output.  This equals the explicit form because kv_b_proj is linear.
 *
 * Conventions for every entry point
 *   - All data pointers are device memory owned by the caller, contiguous, row-major, in the
 *     layouts stated below.  The library allocates nothing, keeps no pointer after a call
 *     returns, holds no global state (calls are thread-safe) and never synchronises; the one
 *     exception is mla_decode_noalloc's static per-GPU workspace (see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs
 *     asynchronously; the caller orders later reads after it on that stream.
 *   - Every argument is validated on the host before anything is enqueued.  On an error
 *     status nothing has been enqueued, except MLA_ERR_HIP (a launch failed part way; the
 *     HIP error is read and cleared).  The contents of device arrays (positions, slots,
 *     block tables, lengths) are the caller's contract: kernels skip a cache write whose slot
 *     is negative or beyond the pool, and clamp nothing else.
 *   - Weights use the (out, in) layout of a linear layer, in act_dtype; norm gains are
 *     act_dtype vectors.  Head h's rows of q_b_proj (q_proj) are [q_nope | q_pe]; head h's
 *     rows of kv_b_proj are [k_nope (qk_nope_head_dim) | v (v_head_dim)].
 *   - The cache is a pool of pages of MLA_PAGE_SIZE tokens: data[num_blocks][64][kv_lora_rank
 *     + qk_rope_head_dim] in cache_dtype, row = [latent | k_pe].  An fp8 cache holds e4m3fn
 *     codes with one fp32 scale per token in scale[num_blocks][64]: value = scale * code,
 *     scale = max|row| / 448 (1 for an all-zero row), codes rounded to nearest even and
 *     saturated at +-448.  Token slot s lives at page s / 64, row s % 64.
 *
 * Supported combinations (others return MLA_ERR_UNSUPPORTED):
 *   act MLA_F32  + cache MLA_F32            any dims (even qk_rope_head_dim; dims <= 4096)
 *   act MLA_BF16 + cache MLA_BF16 / FP8     kv_lora_rank 512, qk_rope_head_dim 64,
 *                                           qk_nope_head_dim 128, v_head_dim 128, num_heads
 *                                           a multiple of 16, hidden_size and q_lora_rank
 *                                           multiples of 8
 * Precision of the bf16 path: weights, hidden states and the cache are read as stored;
 * products accumulate in fp32.  Decode carries the normed query latent and q_nope to their
 * projections as bf16 hi + lo pairs (about 16 significant bits), scores the cache with the
 * absorbed query's latent part in bf16 and its RoPE part in fp16 (the rotary key converted
 * exactly; an fp8 cache's latent codes are scored as stored, in fp8 products against the bf16
 * query latent as two e4m3 codes per value, hi + lo / 16 with a power-of-two scale per head, 8
 * significant bits), and weights the latents with bf16 probabilities; each split's softmax
 * state is handed to the merge in fp16
 * under a per-head power-of-two scale (11 significant bits of every entry within 2^-29 of the
 * head's largest); the merged latent enters W_UV as a hi + lo pair and the attention output
 * enters o_proj in bf16.  Prefill rounds the normed query latent, queries, decompressed keys / values
 * and probabilities to fp16 before its MFMAs (q_b_proj enters as an fp16 copy, exact for
 * magnitudes 2^-14 .. 65504; stores to fp16 saturate at +-65504); an fp8 cache enters the
 * decompression as exact code values with the token scale applied in fp32.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_PAGE_SIZE 64

enum mla_dtype { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 };

enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,  /* a null pointer, non-positive size, inconsistent dims */
  MLA_ERR_UNSUPPORTED = 2,  /* a valid configuration with no kernel (see list above)  */
  MLA_ERR_WORKSPACE = 3,    /* workspace null or smaller than the *_workspace_size   */
  MLA_ERR_HIP = 4           /* a HIP launch failed                                    */
};

/* Layer shape.  Field names mirror the model configuration keys the page lists. */
typedef struct mla_config {
  int32_t hidden_size;
  int32_t num_heads;
  int32_t q_lora_rank;       /* 0: no query compression, a single q_proj */
  int32_t kv_lora_rank;
  int32_t qk_nope_head_dim;
  int32_t qk_rope_head_dim;  /* even */
  int32_t v_head_dim;
  int32_t page_size;         /* must be MLA_PAGE_SIZE */
  float rope_theta;          /* RoPE base; pair i of q_pe/k_pe turns by pos * theta^(-2i/d) */
  float rms_eps;             /* RMSNorm: x / sqrt(mean(x^2) + eps) * gain */
  float softmax_scale;       /* 0: 1 / sqrt(qk_nope_head_dim + qk_rope_head_dim) */
  int32_t act_dtype;         /* MLA_F32 or MLA_BF16: weights and hidden states */
  int32_t cache_dtype;       /* MLA_F32, MLA_BF16 or MLA_FP8_E4M3 */
  int32_t out_dtype;         /* MLA_F32 or MLA_BF16 (MLA_BF16 needs act_dtype MLA_BF16): the
                                attention output.  A bf16 output carries its own rounding of up
                                to 2^-8 of each value on top of the computation's error. */
  /* RoPE context extension by frequency interpolation (YaRN), page "MLA 的两个核心部件" /
   * opening section: the 128K context comes from YaRN scaling of the rotary embedding; the page
   * gives no constants, so they are the caller's.  With rope_factor <= 1 (0 included) the
   * rotation is the plain one.  With rope_factor = s > 1, pair i of frequency f_i turns
   * r_i = rope_original_max_position * f_i / (2 pi) times over the original context and uses
   *   f_i                      if r_i >= rope_beta_fast,
   *   f_i / s                  if r_i <= rope_beta_slow,
   *   (1 - g) f_i / s + g f_i  with g = (r_i - rope_beta_slow) / (rope_beta_fast - rope_beta_slow)
   * in between.  rope_mscale (0: 1) multiplies cos and sin of every rotation, of q_pe and k_pe
   * alike; a temperature on all scores goes in softmax_scale. */
  float rope_factor;
  int32_t rope_original_max_position;  /* > 0 when rope_factor > 1 */
  float rope_beta_fast;                /* > rope_beta_slow when rope_factor > 1 */
  float rope_beta_slow;                /* >= 0 */
  float rope_mscale;
  /* mla_prefill decompresses a sequence's cached latents to per-head keys and values in blocks
   * of this many positions (a multiple of 64), one block after another, so its workspace holds
   * one block per sequence however long the context; 0 lets the library choose (blocks that
   * keep the decompressed keys and values of all sequences within 2 GiB, and a single block
   * when the context fits).  Ignored on the fp32 path, which decompresses the whole context. */
  int32_t prefill_key_block;
} mla_config;

/* Weight pointers (device, act_dtype).  With q_lora_rank == 0, q_b_proj is q_proj
 * [num_heads * (nope + rope), hidden] and q_a_proj / q_a_norm are ignored.
 * o_proj is optional: the output projection that takes the attention result back to the model
 * width (page "DeepSeek-Coder-V2的MLA多头潜在注意力深度解析", section "MLA 的两个核心部件": the
 * forward flow ends with the attention result leaving as the layer's output; the pages name no
 * projection, so its form is a reading: a linear layer whose input is the heads' outputs side by
 * side in head order, head h at inputs h * v_head_dim .. h * v_head_dim + v_head_dim - 1).
 * With o_proj NULL, mla_decode and mla_prefill return the per-head outputs [tokens, num_heads,
 * v_head_dim]; with it set they return o_proj applied to them, [tokens, hidden_size]. */
typedef struct mla_weights {
  const void *q_a_proj;   /* [q_lora_rank, hidden]                      */
  const void *q_a_norm;   /* [q_lora_rank]                              */
  const void *q_b_proj;   /* [num_heads * (nope + rope), q_lora_rank]  */
  const void *kv_a_proj;  /* [kv_lora_rank + rope, hidden]  (kv_a_proj_with_mqa) */
  const void *kv_a_norm;  /* [kv_lora_rank]                             */
  const void *kv_b_proj;  /* [num_heads * (nope + v), kv_lora_rank]     */
  const void *o_proj;     /* [hidden, num_heads * v], or NULL           */
} mla_weights;

typedef struct mla_cache {
  void *data;            /* [num_blocks, 64, kv_lora_rank + rope] cache_dtype */
  float *scale;          /* [num_blocks, 64] fp32, fp8 caches only (else ignored) */
  int32_t num_blocks;
} mla_cache;

/* ---------------------------------------------------------------------------------------
 * mla_compress_append: compress tokens and write their rows into the paged cache.
 * Page section "源码里的压缩全流程", steps "KV 压缩" and "写入缓存": a = kv_a_proj x splits
 * into [latent | k_pe]; the latent is RMS-normalised with kv_a_norm; k_pe is rotated by RoPE
 * at the token's position; the row [latent | k_pe] is rounded to cache_dtype and stored.
 *   hidden        [num_tokens, hidden_size] act_dtype
 *   positions     [num_tokens] int32, RoPE position of each token
 *   slot_mapping  [num_tokens] int64, destination slot (page * 64 + row); < 0 skips the token
 *   num_tokens    >= 0 (0 enqueues nothing)
 * Workspace: mla_compress_append_workspace_size(cfg, num_tokens) bytes of device memory.
 */
size_t mla_compress_append_workspace_size(const mla_config *cfg, int32_t num_tokens);
int mla_compress_append(const mla_config *cfg, const mla_weights *w, const void *hidden,
                        const int32_t *positions, const int64_t *slot_mapping,
                        const mla_cache *cache, int32_t num_tokens, void *workspace,
                        size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------
 * mla_decode: one decode step for a batch of sequences, weight-absorbed form.
 * Page "DeepSeek-Coder-V2的MLA多头潜在注意力深度解析", section "MLA 的两个核心部件" (keys and
 * values of every head are decompressed from the one cached latent by kv_b_proj, the shared
 * RoPE key joins every head's key) and its FAQ Q2 (all heads read the same cached row): since
 * kv_b_proj is linear, q_nope is folded through W_UK so each head scores the cached rows
 * directly, and the softmax-weighted latent is mapped through W_UV afterwards.
 * The new token of sequence b is at position context_lens[b] - 1; it is compressed and
 * written to its slot (block_table[b][pos / 64] * 64 + pos % 64) first, then its query
 * attends to all context_lens[b] cached rows of the sequence (itself included).
 *   hidden        [batch, hidden_size] act_dtype, the new tokens
 *   context_lens  [batch] int32 in [1, max_blocks * 64]
 *   block_table   [batch, max_blocks] int32 physical page of each logical page
 *   num_splits    0 = chosen by the library (mla_decode_num_splits), else 1..1024: each
 *                 sequence's pages are cut into num_splits contiguous ranges whose partial
 *                 softmax states are merged by log-sum-exp
 *   out           [batch, num_heads, v_head_dim] out_dtype, or [batch, hidden_size] with
 *                 w->o_proj set
 */
int32_t mla_decode_num_splits(const mla_config *cfg, int32_t batch, int32_t max_blocks);
size_t mla_decode_workspace_size(const mla_config *cfg, int32_t batch, int32_t max_blocks,
                                 int32_t num_splits);
int mla_decode(const mla_config *cfg, const mla_weights *w, const void *hidden,
               const int32_t *context_lens, const int32_t *block_table, int32_t max_blocks,
               const mla_cache *cache, int32_t batch, int32_t num_splits, void *workspace,
               size_t workspace_bytes, void *out, void *stream);

/* mla_decode, and additionally records two caller-created hipEvent_t handles on `stream`:
 * `ev_attn_begin` just before the split-K attention kernel is enqueued and `ev_attn_end` just
 * after it, so hipEventElapsedTime gives that kernel's duration.  Either may be NULL.  For
 * timing and profiling; results are identical to mla_decode. */
int mla_decode_timed(const mla_config *cfg, const mla_weights *w, const void *hidden,
                     const int32_t *context_lens, const int32_t *block_table, int32_t max_blocks,
                     const mla_cache *cache, int32_t batch, int32_t num_splits, void *workspace,
                     size_t workspace_bytes, void *out, void *stream, void *ev_attn_begin,
                     void *ev_attn_end);

/* ---------------------------------------------------------------------------------------
 * mla_decode_noalloc: mla_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments
 * and results as mla_decode without the workspace: the library uses a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES (64 MiB), one copy on each GPU it runs on, held until the process
 * ends; it allocates nothing and calls no allocating routine.  Returns MLA_ERR_WORKSPACE when
 * mla_decode_workspace_size(cfg, batch, max_blocks, num_splits) exceeds the array (e.g. a
 * 236B-shaped batch of 64 x 8192 tokens with 2 splits needs 57.4 MB and fits; 128 sequences
 * do not).  All calls on one GPU share its array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and give undefined
 * results; calls ordered on one stream are safe.  The device address of the array is looked
 * up once per GPU on the first call (MLA_ERR_HIP if that fails).
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
int mla_decode_noalloc(const mla_config *cfg, const mla_weights *w, const void *hidden,
                       const int32_t *context_lens, const int32_t *block_table, int32_t max_blocks,
                       const mla_cache *cache, int32_t batch, int32_t num_splits, void *out,
                       void *stream);

/* ---------------------------------------------------------------------------------------
 * mla_prefill: causal prefill of one chunk per sequence, explicit (decompressing) form.
 * Page section "源码里的压缩全流程" end to end: the chunk's tokens are compressed and
 * appended to the cache, then each chunk token at position p attends to every cached row of
 * its sequence at positions <= p, with k_nope / v decompressed from the cached latents by
 * kv_b_proj and the shared k_pe concatenated to every head's key.
 *   hidden        [total_tokens, hidden_size] act_dtype, chunks packed back to back
 *   cu_seqlens    [num_seqs + 1] int32, chunk s is rows cu_seqlens[s] .. cu_seqlens[s+1]-1
 *   start_pos     [num_seqs] int32, position of chunk s's first token; positions
 *                 0 .. start_pos[s]-1 must already be in the cache
 *   max_q_len     >= every chunk length;  max_ctx >= every start_pos[s] + chunk length,
 *                 and max_ctx <= max_blocks * 64
 *   out           [total_tokens, num_heads, v_head_dim] out_dtype, or [total_tokens,
 *                 hidden_size] with w->o_proj set
 */
size_t mla_prefill_workspace_size(const mla_config *cfg, int32_t num_seqs, int32_t total_tokens,
                                  int32_t max_q_len, int32_t max_ctx);
int mla_prefill(const mla_config *cfg, const mla_weights *w, const void *hidden,
                const int32_t *cu_seqlens, const int32_t *start_pos, const int32_t *block_table,
                int32_t max_blocks, const mla_cache *cache, int32_t num_seqs,
                int32_t total_tokens, int32_t max_q_len, int32_t max_ctx, void *workspace,
                size_t workspace_bytes, void *out, void *stream);

/* ---------------------------------------------------------------------------------------
 * The fp8 cache's number format on the device (page "DeepSeek-V3.2-Exp 中多头潜在注意力的优化",
 * deployment section: the latent is stored in fp8; the format taken is OCP e4m3fn).  These are
 * the conversions mla_compress_append applies to (row value / token scale) and the attention
 * kernels undo, exposed so a caller can fill or read an fp8 cache itself.
 *   mla_fp8_e4m3_encode: codes[i] = nearest e4m3fn value of x[i], ties to even; magnitudes at or
 *                        above 448 saturate to +-448 (0x7E / 0xFE); NaN gives 0x7F / 0xFF.
 *   mla_fp8_e4m3_decode: x[i] = the value of codes[i] (exact in fp32); 0x7F / 0xFF give NaN.
 *   n >= 0 elements (0 enqueues nothing); device pointers; asynchronous on `stream`.
 * Returns MLA_ERR_INVALID_ARG for a null pointer with n > 0 or n < 0.
 */
int mla_fp8_e4m3_encode(const float *x, uint8_t *codes, int64_t n, void *stream);
int mla_fp8_e4m3_decode(const uint8_t *codes, float *x, int64_t n, void *stream);

/* ---------------------------------------------------------------------------------------
 * mla_stream_read: a measurement aid, not part of the method.  Reads `bytes` (a multiple of 16,
 * below 4 TiB) from device memory at `src` (16-byte aligned) once, coalesced, and discards them
 * (`sink`: 4 device bytes the kernel may write).  mode 0: plain loads into registers, a read
 * sweep that leaves the caches holding clean lines of `src` (used to evict a workload's data
 * between timed steps).  mode 1: non-temporal direct loads into LDS, the fastest read pattern
 * measured on this GPU, so the kernel's duration gives the read bandwidth a streaming kernel
 * can reach; the attention's algorithmic bandwidth is quoted against it beside the published
 * peak.  Asynchronous on `stream`.  Returns MLA_ERR_INVALID_ARG for a misaligned or null
 * argument or another mode.
 */
int mla_stream_read(const void *src, size_t bytes, uint32_t *sink, int mode, void *stream);

/* Static text for a status code. */
const char *mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
