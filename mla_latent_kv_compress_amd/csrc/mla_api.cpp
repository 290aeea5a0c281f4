// extern "C" entry points of libmla: validate on the host, then enqueue the kernel pipeline.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla.h"
#include "mla_kernels.h"
#include "mla_plan.h"

using namespace mla;

// Workspace of mla_decode_noalloc: a file-scope device array, one copy on each GPU the library
// runs on, held until the process ends.  Host code never uses its name as an address: the
// device address comes from hipGetSymbolAddress, once per device (scratch_base below).
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_base[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on first use).
int scratch_base(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return MLA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_base[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return MLA_ERR_HIP;
    }
    g_scratch_base[dev] = p;
  }
  *out = g_scratch_base[dev];
  return MLA_OK;
}

constexpr float kLog2eHost = 1.4426950408889634f;

int kdt(int dt) { return dt == MLA_F32 ? K_F32 : dt == MLA_BF16 ? K_BF16 : K_FP8; }

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

int finish() { return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Y = X * W^T (TN) or X * W (NN), fp32 or bf16 inputs per the path; `out` is the bf16 path's
// output storage (K_F32 / K_BF16 / K_F16; the fp32 path always writes fp32).
GemmArgs gemm(Path path, bool nn, int out, int M, int N, int K, SplitK sk, int batch, const void* X,
              long lda, long sx, const void* W, long ldw, long sw, void* Y, long ldc, long sy,
              float alpha = 1.f) {
  GemmArgs g;
  g.kind = path == PATH_F32 ? GEMM_F32 : GEMM_BF16;
  g.nn = nn;
  g.out = path == PATH_F32 ? K_F32 : out;
  g.M = M; g.N = N; g.K = K;
  g.kchunk = sk.chunk; g.nsplit = sk.n; g.batch = batch;
  g.X = X; g.lda = lda; g.sx = sx;
  g.W = W; g.ldw = ldw; g.sw = sw;
  g.Y = Y; g.ldc = ldc; g.sy = sy; g.ssplit = long(M) * ldc;
  g.alpha = alpha;
  return g;
}

SplitK whole(int K) { return SplitK{1, (K + 31) / 32 * 32}; }

// kv_a projection of T tokens into fp32 partials, then the row epilogue into the cache.
void enqueue_compress(const Dims& d, Path path, const mla_config* cfg, const mla_weights* w,
                      const void* hidden, const int32_t* pos, const int64_t* slots,
                      const mla_cache* cache, int T, const CompressPlan& cp, void* ws,
                      hipStream_t s, float* rope_tab = nullptr, const int32_t* ctx = nullptr,
                      const int32_t* bt = nullptr, int max_blocks = 0) {
  float* acc = reinterpret_cast<float*>(at(ws, cp.off_acc));
  launch_gemm(gemm(path, false, K_F32, T, d.W(), d.D, cp.split, 1, hidden, d.D, 0, w->kv_a_proj, d.D, 0,
                   acc, d.W(), 0), s);
  launch_compress_rows(kdt(cfg->act_dtype), kdt(cfg->cache_dtype), T, d.dc, d.dr, cp.split.n, acc,
                       w->kv_a_norm, pos, slots, cache->data, cache->scale,
                       long(cache->num_blocks) * MLA_PAGE_SIZE, d.eps, d.rope, rope_tab, ctx, bt, max_blocks, s);
}

// Query projection of T tokens.  Leaves fp32 partials at q.off_q_acc, or (q.direct) the scaled
// fp16 queries in `direct_out` ([T][H][dqk]).  With wq16 (a workspace region for an fp16 copy of
// q_b_proj) the normed query latent is kept in fp16 and q_b runs on fp16 operands: the latent
// carries 11 significant bits into the product instead of bf16's 8 (the copy is exact for
// weights of magnitude 2^-14 .. 65504).
void enqueue_query(const Dims& d, Path path, const mla_config* cfg, const mla_weights* w,
                   const void* hidden, int T, const QueryPlan& q, void* ws, void* direct_out,
                   float direct_scale, hipStream_t s, void* wq16 = nullptr) {
  const long nq = long(d.H) * d.dqk();
  void* qout = q.direct ? direct_out : at(ws, q.off_q_acc);
  const int out = q.direct ? K_F16 : K_F32;
  const float alpha = q.direct ? direct_scale : 1.f;
  const void* x = hidden;
  const void* wb = w->q_b_proj;
  long ldx = d.D;
  if (d.dq > 0) {
    float* qa = reinterpret_cast<float*>(at(ws, q.off_qa_acc));
    void* cq = at(ws, q.off_cq);
    launch_gemm(gemm(path, false, K_F32, T, d.dq, d.D, q.split_a, 1, hidden, d.D, 0, w->q_a_proj, d.D, 0,
                     qa, d.dq, 0), s);
    launch_rmsnorm_rows(kdt(cfg->act_dtype), T, d.dq, q.split_a.n, qa, w->q_a_norm, cq, d.eps, s, wq16 != nullptr);
    if (wq16) {
      launch_bf16_to_f16(w->q_b_proj, wq16, nq * d.dq, s);
      wb = wq16;
    }
    x = cq;
    ldx = d.dq;
  }
  GemmArgs g = gemm(path, false, out, T, int(nq), int(ldx), q.split_b, 1, x, ldx, 0, wb, ldx, 0, qout, nq, 0, alpha);
  g.f16in = wq16 != nullptr;
  launch_gemm(g, s);
}

// Decode front on the bf16 path with a query LoRA: the kv_a and q_a projections in one launch,
// the compress epilogue and the query-latent RMSNorm in one launch, then q_b.  The normed query
// latent leaves the row kernel as a bf16 hi + lo pair and enters the q_b products as two; with the split epilogue
// (no K split, d_n 128, d_r 64) q_nope leaves scaled in fp32 for the absorb, q_pe in fp32.  Same
// computation as enqueue_compress + enqueue_query up to rounding; false (nothing enqueued) if the
// grouped launch does not apply.
bool enqueue_decode_front(const Dims& d, Path path, const mla_config* cfg, const mla_weights* w,
                          const void* hidden, const mla_cache* cache, int B, const DecodePlan& p, void* ws,
                          float* rope, const int32_t* ctx, const int32_t* bt, int max_blocks, float qscale,
                          const float** qn32, const float** qpe32, hipStream_t s) {
  *qn32 = *qpe32 = nullptr;
  const QueryPlan& q = p.q;
  if (p.hidden_pair && !q.direct) {
    // No query LoRA: the query projection (q_b_proj holds it) and kv_a in one launch, then the
    // compress epilogue; where the absorb takes fp32 queries (d_n 128, d_r 64, d_c 512) the same
    // launch sums the query partials into the split epilogue's layout, in the attention
    // partials' region (dead until the attention, which runs after the absorb; B H (d_c 2 B) >=
    // B H 192 4 B for any split count)
    float* qn = nullptr;
    float* qp = nullptr;
    if (d.dn == 128 && d.dr == 64 && d.dc == 512) {
      qn = reinterpret_cast<float*>(at(ws, p.off_part_o));
      qp = qn + size_t(B) * d.H * d.dn;
    }
    const long nq = long(d.H) * d.dqk();
    const GemmArgs g_q = gemm(path, false, K_F32, B, int(nq), d.D, q.split_b, 1, hidden, d.D, 0, w->q_b_proj, d.D, 0,
                              at(ws, q.off_q_acc), nq, 0);
    float* acc_kv = reinterpret_cast<float*>(at(ws, p.comp.off_acc));
    const GemmArgs g_kv = gemm(path, false, K_F32, B, d.W(), d.D, p.comp.split, 1, hidden, d.D, 0, w->kv_a_proj,
                               d.D, 0, acc_kv, d.W(), 0);
    if (!launch_gemm_pair(g_q, g_kv, s)) return false;
    launch_compress_rows(kdt(cfg->act_dtype), kdt(cfg->cache_dtype), B, d.dc, d.dr, p.comp.split.n, acc_kv,
                         w->kv_a_norm, nullptr, nullptr, cache->data, cache->scale,
                         long(cache->num_blocks) * MLA_PAGE_SIZE, d.eps, d.rope, rope, ctx, bt, max_blocks, s,
                         q.split_b.n, qn ? reinterpret_cast<const float*>(at(ws, q.off_q_acc)) : nullptr, d.H, qscale,
                         qn, qp);
    *qn32 = qn;
    *qpe32 = qp;
    return true;
  }
  if (path != PATH_BF16 || d.dq <= 0 || q.direct || !p.cq_pair) return false;
  float* acc_kv = reinterpret_cast<float*>(at(ws, p.comp.off_acc));
  float* acc_q = reinterpret_cast<float*>(at(ws, q.off_qa_acc));
  void* cq = at(ws, q.off_cq);                        // bf16 hi + lo pair [B][2 dq]
  const long nq = long(d.H) * d.dqk();
  GemmArgs g_b = gemm(path, false, K_F32, B, int(nq), d.dq, q.split_b, 1, cq, 2L * d.dq, 0, w->q_b_proj, d.dq, 0,
                      at(ws, q.off_q_acc), nq, 0);
  g_b.xpair = true;
  if (!launch_gemm_skinny_ok(g_b)) return false;
  const GemmArgs g_q = gemm(path, false, K_F32, B, d.dq, d.D, q.split_a, 1, hidden, d.D, 0, w->q_a_proj, d.D, 0,
                            acc_q, d.dq, 0);
  const GemmArgs g_kv = gemm(path, false, K_F32, B, d.W(), d.D, p.comp.split, 1, hidden, d.D, 0, w->kv_a_proj,
                             d.D, 0, acc_kv, d.W(), 0);
  if (!launch_gemm_pair(g_q, g_kv, s)) return false;
  const long num_slots = long(cache->num_blocks) * MLA_PAGE_SIZE;
  if (!launch_decode_rows(kdt(cfg->act_dtype), kdt(cfg->cache_dtype), B, d.dc, d.dr, p.comp.split.n, acc_kv,
                          w->kv_a_norm, cache->data, cache->scale, num_slots, d.eps, d.rope, rope, ctx, bt,
                          max_blocks, d.dq, q.split_a.n, acc_q, w->q_a_norm, cq, s))
    return false;                                 // (cannot happen: bf16 activations, bf16 / fp8 cache, q_lora_rank % 64 == 0)
  // q_b with the split epilogue (q_nope as fp32 scale q, q_pe fp32, in the q_acc region) when
  // it applies.
  if (q.split_b.n == 1 && d.dn == 128 && d.dr == 64) {
    char* qn = at(ws, q.off_q_acc);
    float* qpe = reinterpret_cast<float*>(qn + size_t(B) * d.H * d.dn * 4);
    GemmArgs g = g_b;
    g.alpha = qscale;
    if (launch_q_split_gemm(g, qpe, s)) {
      *qn32 = reinterpret_cast<const float*>(qn);
      *qpe32 = qpe;
      return true;
    }
  }
  launch_gemm(g_b, s);
  return true;
}

}  // namespace

extern "C" {

int mla_fp8_e4m3_encode(const float* x, uint8_t* codes, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!x || !codes))) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  (void)hipGetLastError();
  launch_fp8_codec(true, x, codes, long(n), static_cast<hipStream_t>(stream));
  return finish();
}

int mla_fp8_e4m3_decode(const uint8_t* codes, float* x, int64_t n, void* stream) {
  if (n < 0 || (n > 0 && (!x || !codes))) return MLA_ERR_INVALID_ARG;
  if (n == 0) return MLA_OK;
  (void)hipGetLastError();
  launch_fp8_codec(false, codes, x, long(n), static_cast<hipStream_t>(stream));
  return finish();
}

int mla_stream_read(const void* src, size_t bytes, uint32_t* sink, int mode, void* stream) {
  if (bytes % 16 != 0 || (bytes > 0 && (!src || !sink)) || (reinterpret_cast<uintptr_t>(src) & 15) != 0 ||
      (mode != 0 && mode != 1) || bytes >= (size_t(1) << 42))
    return MLA_ERR_INVALID_ARG;
  if (bytes == 0) return MLA_OK;
  (void)hipGetLastError();
  launch_stream_read(src, long(bytes / 16), sink, mode, static_cast<hipStream_t>(stream));
  return finish();
}

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

size_t mla_compress_append_workspace_size(const mla_config* cfg, int32_t num_tokens) {
  Dims d;
  Path path;
  if (check_config(cfg, &d, &path) != MLA_OK || num_tokens < 0) return 0;
  Layout L;
  CompressPlan cp;
  plan_compress(d, path, num_tokens, L, &cp);
  return L.top;
}

int mla_compress_append(const mla_config* cfg, const mla_weights* w, const void* hidden,
                        const int32_t* positions, const int64_t* slot_mapping, const mla_cache* cache,
                        int32_t num_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_compress_args(cfg, w, hidden, positions, slot_mapping, cache, num_tokens);
  if (st != MLA_OK) return st;
  Dims d;
  Path path;
  check_config(cfg, &d, &path);
  if (num_tokens == 0) return MLA_OK;
  Layout L;
  CompressPlan cp;
  plan_compress(d, path, num_tokens, L, &cp);
  if (!workspace || workspace_bytes < L.top) return MLA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  enqueue_compress(d, path, cfg, w, hidden, positions, slot_mapping, cache, num_tokens, cp, workspace, s);
  return finish();
}

int32_t mla_decode_num_splits(const mla_config* cfg, int32_t batch, int32_t max_blocks) {
  Dims d;
  Path path;
  if (check_config(cfg, &d, &path) != MLA_OK || batch <= 0 || max_blocks <= 0) return 0;
  return auto_splits(d, path, batch, max_blocks);
}

size_t mla_decode_workspace_size(const mla_config* cfg, int32_t batch, int32_t max_blocks,
                                 int32_t num_splits) {
  Dims d;
  Path path;
  if (check_config(cfg, &d, &path) != MLA_OK || batch <= 0 || max_blocks <= 0 || num_splits < 0 ||
      num_splits > 1024)
    return 0;
  DecodePlan p;
  plan_decode(d, path, batch, max_blocks, num_splits, &p);
  return p.bytes;
}

int mla_decode_timed(const mla_config* cfg, const mla_weights* w, const void* hidden,
                     const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks,
                     const mla_cache* cache, int32_t batch, int32_t num_splits, void* workspace,
                     size_t workspace_bytes, void* out, void* stream, void* ev_attn_begin,
                     void* ev_attn_end) {
  int st = check_decode_args(cfg, w, hidden, context_lens, block_table, max_blocks, cache, batch,
                             num_splits, out);
  if (st != MLA_OK) return st;
  Dims d;
  Path path;
  check_config(cfg, &d, &path);
  DecodePlan p;
  plan_decode(d, path, batch, max_blocks, num_splits, &p);
  if (!workspace || workspace_bytes < p.bytes) return MLA_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int act = kdt(cfg->act_dtype);
  const size_t asz = dtype_size(cfg->act_dtype);
  const int B = batch;
  int32_t* pos = reinterpret_cast<int32_t*>(at(workspace, p.off_pos));
  int64_t* slot = reinterpret_cast<int64_t*>(at(workspace, p.off_slot));

  float* rope = reinterpret_cast<float*>(at(workspace, p.off_rope));
  // Scaled queries: sigma * log2(e) folded in, so the kernels use exp2.
  const float qscale = d.sigma * kLog2eHost;
  // fp32 queries in the split epilogue's layout (q_nope scaled, q_pe), when the front leaves them
  const float* qn32 = nullptr;
  const float* qpe32 = nullptr;
  const bool front = enqueue_decode_front(d, path, cfg, w, hidden, cache, B, p, workspace, rope, context_lens,
                                          block_table, max_blocks, qscale, &qn32, &qpe32, s);
  const bool qfp32 = qn32 != nullptr;
  if (front) {
    // compress / append and the query projection enqueued by the grouped front
  } else if (path == PATH_BF16) {
    // the row epilogue takes each token's position and slot from its context length itself
    enqueue_compress(d, path, cfg, w, hidden, nullptr, nullptr, cache, B, p.comp, workspace, s, rope, context_lens,
                     block_table, max_blocks);
  } else {
    launch_decode_prep(B, context_lens, block_table, max_blocks, pos, slot, s);
    enqueue_compress(d, path, cfg, w, hidden, pos, slot, cache, B, p.comp, workspace, s, rope);
  }
  if (!front) enqueue_query(d, path, cfg, w, hidden, B, p.q, workspace, nullptr, 0.f, s);

  void* qnope = at(workspace, p.off_qnope);
  void* qhat = at(workspace, p.off_qhat);
  const float* qacc = reinterpret_cast<const float*>(at(workspace, p.q.off_q_acc));
  // Absorb: qhat[b][h][0:dc] = q_nope[b][h] . W_UK^h  (W_UK^h = kv_b_proj rows of head h's k_nope),
  // qhat[b][h][dc:] = RoPE(q_pe[b][h]); one kernel on the bf16 path.
  if (!qfp32 && path == PATH_BF16 && d.dn == 128 && d.dr == 64 && d.dc == 512) {
    // The query arrives as K-split partials: sum them once into the split epilogue's layout, in
    // the attention partials' region (dead until the attention, which runs after the absorb;
    // B H (dc 2 B) >= B H 192 4 B for any split count)
    float* qn = reinterpret_cast<float*>(at(workspace, p.off_part_o));
    float* qp = qn + size_t(B) * d.H * d.dn;
    launch_q_split_sum(B, d.H, p.q.split_b.n, qacc, qscale, qn, qp, s);
    qn32 = qn;
    qpe32 = qp;
  }
  if (!(path == PATH_BF16 && launch_absorb_rope(B, d.H, d.dn, d.dr, d.dc, d.dv, p.q.split_b.n, qacc, rope, qscale,
                                                w->kv_b_proj, qhat, s, qn32, qpe32))) {
    if (qfp32) return MLA_ERR_UNSUPPORTED;        // (cannot happen: both need dn 128, dr 64, dc 512)
    if (path == PATH_BF16) launch_decode_prep(B, context_lens, block_table, max_blocks, pos, slot, s);
    launch_q_pack(act, act, true, B, d.H, d.dn, d.dr, d.dc, p.q.split_b.n, qacc, pos, qscale, d.rope, qnope, qhat,
                  nullptr, s);
    launch_gemm(gemm(path, true, act, B, d.dc, d.dn, whole(d.dn), d.H, qnope, long(d.H) * d.dn, d.dn,
                     w->kv_b_proj, d.dc, long(d.dkv()) * d.dc, qhat, long(d.H) * d.W(), d.W()), s);
  }

  DecodeAttnArgs a;
  a.B = B; a.H = d.H; a.dc = d.dc; a.dr = d.dr; a.splits = p.splits;
  a.qhat = qhat;
  a.cache = cache->data; a.cache_scale = cache->scale;
  a.block_table = block_table; a.max_blocks = max_blocks; a.ctx = context_lens;
  a.part_o = at(workspace, p.off_part_o);
  a.part_ml = reinterpret_cast<float*>(at(workspace, p.off_part_ml));
  a.order = p.ordered ? reinterpret_cast<int32_t*>(at(workspace, p.off_order)) : nullptr;
  if (ev_attn_begin) (void)hipEventRecord(static_cast<hipEvent_t>(ev_attn_begin), s);
  if (!launch_decode_attn(act, kdt(cfg->cache_dtype), a, s)) return MLA_ERR_UNSUPPORTED;
  if (ev_attn_end) (void)hipEventRecord(static_cast<hipEvent_t>(ev_attn_end), s);

  float* otilde = reinterpret_cast<float*>(at(workspace, p.off_otilde));
  // With o_proj the attention output goes to the workspace first, in the activation dtype (bf16:
  // its rounding moves the projected output by about 2^-9 of its rms, and the weight stream, not
  // the activation, is what the product should spend its loads on).
  const int out_type = kdt(cfg->out_dtype);
  const long nv = long(d.H) * d.dv;
  GemmArgs go;
  int attn_type = out_type;
  void* attn = out;
  if (w->o_proj) {
    attn = at(workspace, p.off_attn);
    attn_type = act;
    const bool direct = p.split_o.n == 1;
    go = gemm(path, false, direct ? out_type : K_F32, B, d.D, int(nv), p.split_o, 1, attn, nv, 0, w->o_proj, nv, 0,
              direct ? out : at(workspace, p.off_o_acc), d.D, 0);
    if (p.o_wide) go.bn = 160;
  }
  // attn[b][h] = W_UV^h otilde[b][h]  (W_UV^h = kv_b_proj rows of head h's v).  The bf16 path
  // merges the split partials inside the projection kernel (its shape checks admit only the
  // d_c 512, d_v 128 it requires).
  if (path == PATH_BF16) {
    if (!launch_decode_merge_uv(attn_type, B, d.H, d.dc, d.dn, d.dv, p.splits,
                                static_cast<const uint16_t*>(a.part_o), a.part_ml, w->kv_b_proj, attn, s, otilde,
                                reinterpret_cast<float*>(at(workspace, p.off_ml1))))
      return MLA_ERR_UNSUPPORTED;
  } else {
    launch_decode_merge(B, d.H, d.dc, p.splits, static_cast<const float*>(a.part_o), a.part_ml, otilde, s);
    const char* w_uv = static_cast<const char*>(w->kv_b_proj) + size_t(d.dn) * d.dc * asz;
    launch_gemm(gemm(path, false, attn_type, B, d.dv, d.dc, whole(d.dc), d.H, otilde, long(d.H) * d.dc, d.dc,
                     w_uv, d.dc, long(d.dkv()) * d.dc, attn, nv, d.dv), s);
  }
  if (w->o_proj) {
    // out[b] = o_proj [attn[b][0] | ... | attn[b][H-1]]: K-split partials summed by a second kernel
    launch_gemm(go, s);
    if (p.split_o.n > 1)
      launch_sum_splits(out_type, long(B) * d.D, p.split_o.n, static_cast<const float*>(go.Y), out, s);
  }
  return finish();
}

int mla_decode(const mla_config* cfg, const mla_weights* w, const void* hidden,
               const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks,
               const mla_cache* cache, int32_t batch, int32_t num_splits, void* workspace,
               size_t workspace_bytes, void* out, void* stream) {
  return mla_decode_timed(cfg, w, hidden, context_lens, block_table, max_blocks, cache, batch, num_splits,
                          workspace, workspace_bytes, out, stream, nullptr, nullptr);
}

int mla_decode_noalloc(const mla_config* cfg, const mla_weights* w, const void* hidden,
                       const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks,
                       const mla_cache* cache, int32_t batch, int32_t num_splits, void* out, void* stream) {
  int st = check_decode_args(cfg, w, hidden, context_lens, block_table, max_blocks, cache, batch,
                             num_splits, out);
  if (st != MLA_OK) return st;
  Dims d;
  Path path;
  check_config(cfg, &d, &path);
  DecodePlan p;
  plan_decode(d, path, batch, max_blocks, num_splits, &p);
  if (p.bytes > size_t(MLA_NOALLOC_SCRATCH_BYTES)) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_base(&ws);
  if (st != MLA_OK) return st;
  // Every region of the plan is written before it is read within the call (split partials,
  // states, queries), so nothing needs clearing between calls.
  return mla_decode(cfg, w, hidden, context_lens, block_table, max_blocks, cache, batch, num_splits, ws,
                    size_t(MLA_NOALLOC_SCRATCH_BYTES), out, stream);
}

size_t mla_prefill_workspace_size(const mla_config* cfg, int32_t num_seqs, int32_t total_tokens,
                                  int32_t max_q_len, int32_t max_ctx) {
  Dims d;
  Path path;
  if (check_config(cfg, &d, &path) != MLA_OK || num_seqs <= 0 || total_tokens <= 0 || max_q_len <= 0 ||
      max_ctx <= 0)
    return 0;
  PrefillPlan p;
  plan_prefill(d, path, num_seqs, total_tokens, max_q_len, max_ctx, cfg->prefill_key_block, &p);
  return p.bytes;
}

int mla_prefill(const mla_config* cfg, const mla_weights* w, const void* hidden,
                const int32_t* cu_seqlens, const int32_t* start_pos, const int32_t* block_table,
                int32_t max_blocks, const mla_cache* cache, int32_t num_seqs, int32_t total_tokens,
                int32_t max_q_len, int32_t max_ctx, void* workspace, size_t workspace_bytes, void* out,
                void* stream) {
  int st = check_prefill_args(cfg, w, hidden, cu_seqlens, start_pos, block_table, max_blocks, cache,
                              num_seqs, total_tokens, max_q_len, max_ctx, out);
  if (st != MLA_OK) return st;
  Dims d;
  Path path;
  check_config(cfg, &d, &path);
  PrefillPlan p;
  plan_prefill(d, path, num_seqs, total_tokens, max_q_len, max_ctx, cfg->prefill_key_block, &p);
  if (!workspace || workspace_bytes < p.bytes) return MLA_ERR_WORKSPACE;
  if (path == PATH_BF16 && cfg->cache_dtype == MLA_FP8_E4M3) {
    // the fp8 decompression applies the token scales in the large-tile kernel's epilogue
    GemmArgs probe = gemm(path, false, K_F16, p.kb, int(long(d.H) * d.dkv()), d.dc, whole(d.dc), num_seqs,
                          at(workspace, p.off_lat), d.W(), long(p.kb) * d.W(), w->kv_b_proj, d.dc, 0,
                          at(workspace, p.off_kv), long(d.H) * d.dkv(), long(p.kb) * d.H * d.dkv());
    probe.row_scale = reinterpret_cast<const float*>(at(workspace, p.off_tscale));
    if (!launch_gemm_tile_ok(probe)) return MLA_ERR_UNSUPPORTED;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int act = kdt(cfg->act_dtype);
  const int T = total_tokens, S = num_seqs;
  int32_t* pos = reinterpret_cast<int32_t*>(at(workspace, p.off_pos));
  int64_t* slot = reinterpret_cast<int64_t*>(at(workspace, p.off_slot));

  launch_prefill_prep(S, max_q_len, cu_seqlens, start_pos, block_table, max_blocks, pos, slot, s);
  enqueue_compress(d, path, cfg, w, hidden, pos, slot, cache, T, p.comp, workspace, s);
  // Queries scaled by sigma * log2(e), RoPE'd: fp16 on the bf16 path, fp32 on the fp32 path.
  void* qs = at(workspace, p.off_qs);
  const float qscale = d.sigma * kLog2eHost;
  const int qs_type = path == PATH_F32 ? K_F32 : K_F16;
  void* wq16 = nullptr;
  if (p.q16) {
    GemmArgs probe = gemm(path, false, K_F16, T, int(long(d.H) * d.dqk()), d.dq, p.q.split_b, 1, at(workspace, p.q.off_cq),
                          d.dq, 0, at(workspace, p.off_wq16), d.dq, 0, qs, long(d.H) * d.dqk(), 0);
    probe.f16in = true;
    if (launch_gemm_tile_ok(probe)) wq16 = at(workspace, p.off_wq16);
  }
  enqueue_query(d, path, cfg, w, hidden, T, p.q, workspace, qs, qscale, s, wq16);
  if (p.q.direct)
    launch_q_rope_f16(T, d.H, d.dn, d.dr, pos, d.rope, qs, s);
  else
    launch_q_pack(act, qs_type, false, T, d.H, d.dn, d.dr, d.dc, p.q.split_b.n,
                  reinterpret_cast<const float*>(at(workspace, p.q.off_q_acc)), pos, qscale, d.rope, nullptr,
                  nullptr, qs, s);
  void* lat = at(workspace, p.off_lat);
  void* kpe = path == PATH_BF16 ? at(workspace, p.off_kpe) : nullptr;
  const bool fp8 = path == PATH_BF16 && cfg->cache_dtype == MLA_FP8_E4M3;
  float* tscale = fp8 ? reinterpret_cast<float*>(at(workspace, p.off_tscale)) : nullptr;
  void* kv = at(workspace, p.off_kv);
  const long nkv = long(d.H) * d.dkv();
  const int kb = p.kb;
  PrefillAttnArgs a;
  a.S = S; a.H = d.H; a.dn = d.dn; a.dr = d.dr; a.dv = d.dv; a.dc = d.dc;
  a.max_q = max_q_len; a.max_ctx = max_ctx; a.out_type = kdt(cfg->out_dtype);
  a.cu = cu_seqlens; a.start = start_pos;
  a.qs = qs; a.kv = kv; a.lat = lat; a.kpe = kpe; a.out = out;
  a.kb = kb;
  if (w->o_proj) {
    // attention output in act dtype to the workspace, then out = o_proj [heads side by side]
    a.out = at(workspace, p.off_attn);
    a.out_type = act;
  }
  float* state = kb < max_ctx ? reinterpret_cast<float*>(at(workspace, p.off_state)) : nullptr;
  // Key blocks of kb positions, one after another: gather the block's cached rows, decompress
  // them (kv[s][t] = kv_b_proj . latent -> per head [k_nope | v]; fp8 cache: kv_b_proj . codes,
  // times the token's scale in fp32), then attend to them, the running softmax state carried in
  // `state` from block to block and normalised into the output after the last.
  for (int k0 = 0; k0 < max_ctx; k0 += kb) {
    const int rows = max_ctx - k0 < kb ? max_ctx - k0 : kb;
    launch_gather_rows(act, kdt(cfg->cache_dtype), S, k0, rows, kb, d.W(), d.dc, cu_seqlens, start_pos, block_table,
                       max_blocks, cache->data, cache->scale, lat, kpe, tscale, s);
    GemmArgs gkv = gemm(path, false, K_F16, rows, int(nkv), d.dc, whole(d.dc), S, lat, d.W(), long(kb) * d.W(),
                        w->kv_b_proj, d.dc, 0, kv, nkv, long(kb) * nkv);
    if (fp8) {
      gkv.row_scale = tscale;
      gkv.srs = kb;
    }
    launch_gemm(gkv, s);
    a.k0 = k0;
    a.state_in = k0 > 0 ? state : nullptr;
    a.state_out = k0 + kb < max_ctx ? state : nullptr;
    if (!launch_prefill_attn(act, a, s)) return MLA_ERR_UNSUPPORTED;
  }
  if (w->o_proj) {
    const long nv = long(d.H) * d.dv;
    launch_gemm(gemm(path, false, kdt(cfg->out_dtype), T, d.D, int(nv), whole(int(nv)), 1, a.out, nv, 0, w->o_proj,
                     nv, 0, out, d.D, 0), s);
  }
  return finish();
}

}  // extern "C"
