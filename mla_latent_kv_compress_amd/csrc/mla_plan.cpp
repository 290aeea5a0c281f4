// Host-side argument validation and workspace planning (no HIP dependency).
#include "mla_plan.h"

#include <cmath>

namespace mla {

namespace {
inline long cdiv(long a, long b) { return (a + b - 1) / b; }
inline long rup(long a, long b) { return cdiv(a, b) * b; }
constexpr long kMaxDim = 1 << 20;
constexpr long kDecodeRound = 256;      // decode work-groups resident at once (one per CU)
constexpr long kRaggedRounds = 2;
constexpr long kRaggedTokens = 4096;    // block tables at least this long may hold ragged lengths
constexpr long kPageTokens = 64;
}  // namespace

size_t dtype_size(int dt) {
  switch (dt) {
    case MLA_F32: return 4;
    case MLA_BF16: return 2;
    case MLA_FP8_E4M3: return 1;
    default: return 0;
  }
}

int check_config(const mla_config* cfg, Dims* d, Path* path) {
  if (!cfg) return MLA_ERR_INVALID_ARG;
  const mla_config& c = *cfg;
  if (c.hidden_size <= 0 || c.num_heads <= 0 || c.q_lora_rank < 0 || c.kv_lora_rank <= 0 ||
      c.qk_nope_head_dim <= 0 || c.qk_rope_head_dim <= 0 || (c.qk_rope_head_dim & 1) ||
      c.v_head_dim <= 0)
    return MLA_ERR_INVALID_ARG;
  if (c.hidden_size > kMaxDim || c.num_heads > 4096 || c.q_lora_rank > kMaxDim ||
      c.kv_lora_rank > kMaxDim || c.qk_nope_head_dim > kMaxDim || c.qk_rope_head_dim > kMaxDim ||
      c.v_head_dim > kMaxDim)
    return MLA_ERR_INVALID_ARG;
  if (c.page_size != MLA_PAGE_SIZE) return MLA_ERR_INVALID_ARG;
  if (!(c.rope_theta > 0.f) || !std::isfinite(c.rope_theta)) return MLA_ERR_INVALID_ARG;
  if (!(c.rms_eps >= 0.f) || !std::isfinite(c.rms_eps)) return MLA_ERR_INVALID_ARG;
  if (!(c.softmax_scale >= 0.f) || !std::isfinite(c.softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (!std::isfinite(c.rope_factor) || !std::isfinite(c.rope_mscale) || c.rope_mscale < 0.f)
    return MLA_ERR_INVALID_ARG;
  if (c.rope_factor > 1.f &&
      (c.rope_original_max_position <= 0 || !std::isfinite(c.rope_beta_fast) || !std::isfinite(c.rope_beta_slow) ||
       !(c.rope_beta_slow >= 0.f) || !(c.rope_beta_fast > c.rope_beta_slow)))
    return MLA_ERR_INVALID_ARG;
  if (c.act_dtype != MLA_F32 && c.act_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (dtype_size(c.cache_dtype) == 0) return MLA_ERR_INVALID_ARG;
  if (c.out_dtype != MLA_F32 && c.out_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (c.prefill_key_block < 0) return MLA_ERR_INVALID_ARG;

  Dims dd;
  dd.D = c.hidden_size; dd.H = c.num_heads; dd.dq = c.q_lora_rank; dd.dc = c.kv_lora_rank;
  dd.dn = c.qk_nope_head_dim; dd.dr = c.qk_rope_head_dim; dd.dv = c.v_head_dim;
  dd.rope.theta = c.rope_theta;
  dd.rope.factor = c.rope_factor > 1.f ? c.rope_factor : 1.f;
  dd.rope.orig = float(c.rope_original_max_position);
  dd.rope.beta_fast = c.rope_beta_fast;
  dd.rope.beta_slow = c.rope_beta_slow;
  dd.rope.mscale = c.rope_mscale > 0.f ? c.rope_mscale : 1.f;
  dd.eps = c.rms_eps;
  dd.cache_dt = c.cache_dtype;
  dd.sigma = c.softmax_scale > 0.f ? c.softmax_scale
                                   : 1.0f / std::sqrt(float(dd.dn + dd.dr));
  Path p = PATH_NONE;
  if (c.act_dtype == MLA_F32 && c.cache_dtype == MLA_F32 && c.out_dtype == MLA_F32) {
    if (dd.dc <= 4096 && dd.dr <= 256 && dd.dn <= 4096 && dd.dv <= 4096) p = PATH_F32;
  } else if (c.act_dtype == MLA_BF16 &&
             (c.cache_dtype == MLA_BF16 || c.cache_dtype == MLA_FP8_E4M3)) {
    if (dd.dc == 512 && dd.dr == 64 && dd.dn == 128 && dd.dv == 128 && dd.H % 16 == 0 &&
        dd.D % 8 == 0 && dd.dq % 8 == 0)
      p = PATH_BF16;
  }
  if (p == PATH_NONE) return MLA_ERR_UNSUPPORTED;
  if (d) *d = dd;
  if (path) *path = p;
  return MLA_OK;
}

SplitK gemm_splitk(long M, long N, long K, int tile_m, int tile_n) {
  long tiles = cdiv(M, tile_m) * cdiv(N, tile_n);
  SplitK s{1, int(rup(K, 32))};
  if (tiles >= 192 || K < 512) return s;
  long want = cdiv(256, tiles);
  long most = K / 256;
  long n = want < most ? want : most;
  if (n <= 1) return s;
  long chunk = rup(cdiv(K, n), 64);
  s.n = int(cdiv(K, chunk));
  s.chunk = int(chunk);
  return s;
}

SplitK pair_splitk(long M, long N0, long N1, long K) {
  if (M > 128 || N0 % 96 != 0 || N1 % 96 != 0 || K % 64 != 0 || K <= 0) return SplitK{0, 0};
  const long tiles = N0 / 96 + N1 / 96;
  long n = 256 / tiles;
  if (n < 1) n = 1;
  const long chunk = rup(cdiv(K, n), 64);
  return SplitK{int(cdiv(K, chunk)), int(chunk)};
}

SplitK tile_splitk(long M, long N, long K) {
  const long tiles = cdiv(M, 256) * cdiv(N, 256);
  const SplitK one{1, int(rup(K, 32))};
  if (M <= 128 || N <= 0 || tiles >= 192 || K % 64 != 0) return one;   // (N 0: no query LoRA)
  for (long n = 256 / tiles; n > 1; --n)
    if (K % (64 * n) == 0 && tiles * n >= 192) return SplitK{int(n), int(K / n)};
  return one;
}

int plan_compress(const Dims& d, Path path, long T, Layout& L, CompressPlan* p, const SplitK* force) {
  (void)path;
  p->split = force ? *force : gemm_splitk(T, d.W(), d.D, 64, 64);
  p->off_acc = L.take(size_t(p->split.n) * T * d.W() * 4);
  return MLA_OK;
}

static void plan_query(const Dims& d, Path path, long T, Layout& L, QueryPlan* q, bool allow_direct,
                       const SplitK* force_a = nullptr) {
  long nq = long(d.H) * d.dqk();
  if (d.dq > 0) {
    q->split_a = force_a ? *force_a : gemm_splitk(T, d.dq, d.D, 64, 64);
    q->off_qa_acc = L.take(size_t(q->split_a.n) * T * d.dq * 4);
    q->off_cq = L.take(size_t(T) * d.dq * 4);
    q->split_b = gemm_splitk(T, nq, d.dq, 64, 64);
  } else {                     // the query projection reads the hidden state: force_a applies to it
    q->split_a = SplitK{1, 32};
    q->off_qa_acc = q->off_cq = 0;
    q->split_b = force_a ? *force_a : gemm_splitk(T, nq, d.D, 64, 64);
  }
  q->direct = allow_direct && path == PATH_BF16 && q->split_b.n == 1;
  q->off_q_acc = q->direct ? 0 : L.take(size_t(q->split_b.n) * T * nq * 4);
}

int decode_heads_per_group(const Dims&, Path path) { return path == PATH_BF16 ? 64 : 1; }

int auto_splits(const Dims& d, Path path, int B, int max_blocks) {
  const int hpg = decode_heads_per_group(d, path);
  long groups = cdiv(d.H, hpg);
  long wgs = long(B) * groups;
  long target = path == PATH_BF16 ? kDecodeRound : 512;
  // A batch that already fills a round of the 64-head kernel with long contexts: the lengths may
  // be ragged, so cut every sequence in kRaggedRounds pieces (taken longest first) and let the
  // short pieces fill in behind the long ones.
  if (hpg == 64 && wgs >= kDecodeRound && long(max_blocks) * kPageTokens >= kRaggedTokens) target = kRaggedRounds * kDecodeRound;
  long s = cdiv(target, wgs);
  long most = max_blocks / 2 > 1 ? max_blocks / 2 : 1;
  if (s > most) s = most;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return int(s);
}

int plan_decode(const Dims& d, Path path, int B, int max_blocks, int splits, DecodePlan* p) {
  Layout L;
  p->splits = splits > 0 ? splits : auto_splits(d, path, B, max_blocks);
  size_t act = path == PATH_F32 ? 4 : 2;
  // The decode front launches the kv_a and q_a projections together (bf16 path with a query
  // LoRA): one K split for both, with the pair's tile shape.
  SplitK pair{0, 0};
  if (path == PATH_BF16 && d.dq > 0) pair = pair_splitk(B, d.dq, d.W(), d.D);
  else if (path == PATH_BF16) pair = pair_splitk(B, long(d.H) * d.dqk(), d.W(), d.D);
  const SplitK* force = pair.n > 0 ? &pair : nullptr;
  plan_compress(d, path, B, L, &p->comp, force);
  plan_query(d, path, B, L, &p->q, false, force);
  p->cq_pair = path == PATH_BF16 && d.dq > 0 && d.dq % 64 == 0;
  p->hidden_pair = path == PATH_BF16 && d.dq == 0 && pair.n > 0;
  p->off_pos = L.take(size_t(B) * 4);
  p->off_slot = L.take(size_t(B) * 8);
  p->off_qnope = L.take(size_t(B) * d.H * d.dn * act);
  p->off_rope = L.take(size_t(B) * d.dr * 4);
  p->off_qhat = L.take(size_t(B) * d.H * d.W() * act);
  p->off_part_o = L.take(size_t(B) * p->splits * d.H * d.dc * (path == PATH_F32 ? 4 : 2));
  p->off_part_ml = L.take(size_t(B) * p->splits * d.H * 2 * 4);
  const int hpg = decode_heads_per_group(d, path);
  // (with many splits per sequence every work-group is short and their order matters little)
  p->ordered = hpg == 64 && B <= kOrderMax && p->splits <= 8 && long(B) * p->splits * cdiv(d.H, hpg) > kDecodeRound;
  p->off_order = L.take(size_t(B) * 4);
  // o_proj: its K-split partials share the merged-state region (dead once W_UV has read it), and
  // the attention output reuses the query region (dead once the attention has run) when it fits
  const long ko = long(d.H) * d.dv;
  p->o_wide = path == PATH_BF16 && B <= 128 && d.D % 160 == 0 && ko % 64 == 0 && d.D / 160 <= 256;
  if (p->o_wide) {
    // one round of 256 work-groups: D / 160 column tiles times the K split
    long n = 256 / (d.D / 160);
    const long most = ko / 256;
    if (n > most) n = most;
    if (n < 1) n = 1;
    const long chunk = rup(cdiv(ko, n), 64);
    p->split_o = SplitK{int(cdiv(ko, chunk)), int(chunk)};
  } else {
    p->split_o = gemm_splitk(B, d.D, ko, 64, 64);
  }
  const size_t otilde_bytes = size_t(B) * d.H * d.dc * 4;
  const size_t oacc_bytes = p->split_o.n > 1 ? size_t(p->split_o.n) * B * d.D * 4 : 0;
  p->off_otilde = L.take(otilde_bytes > oacc_bytes ? otilde_bytes : oacc_bytes);
  p->off_o_acc = p->off_otilde;
  p->off_ml1 = L.take(size_t(B) * d.H * 2 * 4);
  const size_t attn_bytes = size_t(B) * d.H * d.dv * 4;
  const size_t qhat_bytes = size_t(B) * d.H * d.W() * act;
  p->off_attn = attn_bytes <= qhat_bytes ? p->off_qhat : L.take(attn_bytes);
  p->bytes = L.top;
  return MLA_OK;
}

static int prefill_key_block(const Dims& d, Path path, int S, int max_ctx, int key_block) {
  const long whole = rup(max_ctx, 64);
  if (path != PATH_BF16) return int(whole);
  long kb = key_block;
  if (kb <= 0) {
    // the decompressed keys and values of all sequences (fp16) within 2 GiB
    const long per_row = long(S) * d.H * d.dkv() * 2;
    kb = (2L << 30) / per_row / 64 * 64;
    if (kb < 64) kb = 64;
  }
  kb = rup(kb, 64);
  return int(kb < whole ? kb : whole);
}

int plan_prefill(const Dims& d, Path path, int S, int T, int max_q, int max_ctx, int key_block, PrefillPlan* p) {
  (void)max_q;
  Layout L;
  size_t act = path == PATH_F32 ? 4 : 2;
  // kv_a and q_a of a long chunk run on the 256 x 256-tile kernel as fp32 K-split partials
  const bool tiles = path == PATH_BF16 && T >= 1024;
  const SplitK kv_split = tile_splitk(T, d.W(), d.D);
  const SplitK qa_split = d.dq > 0 ? tile_splitk(T, d.dq, d.D) : SplitK{1, 32};
  plan_compress(d, path, T, L, &p->comp, tiles ? &kv_split : nullptr);
  plan_query(d, path, T, L, &p->q, true, tiles && d.dq > 0 ? &qa_split : nullptr);
  p->off_pos = L.take(size_t(T) * 4);
  p->off_slot = L.take(size_t(T) * 8);
  p->off_qs = L.take(size_t(T) * d.H * d.dqk() * act);
  p->kb = prefill_key_block(d, path, S, max_ctx, key_block);
  p->off_lat = L.take(size_t(S) * p->kb * d.W() * act);
  p->off_kpe = L.take(size_t(S) * p->kb * d.dr * 2);
  p->off_kv = L.take(size_t(S) * p->kb * d.H * d.dkv() * act);
  p->off_tscale = L.take(path == PATH_BF16 && d.cache_dt == MLA_FP8_E4M3 ? size_t(S) * p->kb * 4 : 0);
  p->off_state = L.take(p->kb < max_ctx ? size_t(T) * d.H * (d.dv + 2) * 4 : 0);
  p->q16 = path == PATH_BF16 && d.dq > 0 && d.dq % 64 == 0 && p->q.direct;
  p->off_wq16 = L.take(p->q16 ? size_t(d.H) * d.dqk() * d.dq * 2 : 0);
  p->off_attn = L.take(size_t(T) * d.H * d.dv * act);
  p->bytes = L.top;
  return MLA_OK;
}

static bool cache_ok(const mla_config* cfg, const mla_cache* cache) {
  if (!cache || !cache->data || cache->num_blocks <= 0) return false;
  if (cfg->cache_dtype == MLA_FP8_E4M3 && !cache->scale) return false;
  return true;
}

static bool query_weights_ok(const mla_config* cfg, const mla_weights* w) {
  if (!w || !w->q_b_proj || !w->kv_a_proj || !w->kv_a_norm || !w->kv_b_proj) return false;
  if (cfg->q_lora_rank > 0 && (!w->q_a_proj || !w->q_a_norm)) return false;
  return true;
}

int check_compress_args(const mla_config* cfg, const mla_weights* w, const void* hidden,
                        const int32_t* positions, const int64_t* slots, const mla_cache* cache,
                        int32_t T) {
  int st = check_config(cfg, nullptr, nullptr);
  if (st != MLA_OK) return st;
  if (T < 0) return MLA_ERR_INVALID_ARG;
  if (!w || !w->kv_a_proj || !w->kv_a_norm) return MLA_ERR_INVALID_ARG;
  if (!cache_ok(cfg, cache)) return MLA_ERR_INVALID_ARG;
  if (T > 0 && (!hidden || !positions || !slots)) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

int check_decode_args(const mla_config* cfg, const mla_weights* w, const void* hidden,
                      const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks,
                      const mla_cache* cache, int32_t B, int32_t splits, const void* out) {
  int st = check_config(cfg, nullptr, nullptr);
  if (st != MLA_OK) return st;
  if (B <= 0 || max_blocks <= 0 || splits < 0 || splits > 1024) return MLA_ERR_INVALID_ARG;
  if (long(B) * max_blocks > (1L << 30)) return MLA_ERR_INVALID_ARG;
  if (!query_weights_ok(cfg, w) || !cache_ok(cfg, cache)) return MLA_ERR_INVALID_ARG;
  if (!hidden || !context_lens || !block_table || !out) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

int check_prefill_args(const mla_config* cfg, const mla_weights* w, const void* hidden,
                       const int32_t* cu_seqlens, const int32_t* start_pos,
                       const int32_t* block_table, int32_t max_blocks, const mla_cache* cache,
                       int32_t S, int32_t T, int32_t max_q, int32_t max_ctx, const void* out) {
  int st = check_config(cfg, nullptr, nullptr);
  if (st != MLA_OK) return st;
  if (S <= 0 || T <= 0 || max_q <= 0 || max_ctx <= 0 || max_blocks <= 0) return MLA_ERR_INVALID_ARG;
  if (max_q > T || max_q > max_ctx) return MLA_ERR_INVALID_ARG;
  if (long(max_ctx) > long(max_blocks) * MLA_PAGE_SIZE) return MLA_ERR_INVALID_ARG;
  if (long(S) * max_blocks > (1L << 30) || long(S) * max_ctx > (1L << 30)) return MLA_ERR_INVALID_ARG;
  if (!query_weights_ok(cfg, w) || !cache_ok(cfg, cache)) return MLA_ERR_INVALID_ARG;
  if (!hidden || !cu_seqlens || !start_pos || !block_table || !out) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

}  // namespace mla
