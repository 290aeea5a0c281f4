// Host-side argument validation and workspace planning for libmla.  No HIP dependency: this
// translation unit also builds with a plain host compiler for sanitizer tests on the CPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "mla.h"
#include "mla_rope.h"

namespace mla {

enum Path { PATH_NONE = 0, PATH_F32 = 1, PATH_BF16 = 2 };

struct Dims {
  int D, H, dq, dc, dn, dr, dv;
  int cache_dt;                          // mla_dtype of the cache
  int W() const { return dc + dr; }      // cached row width
  int dqk() const { return dn + dr; }    // per-head query width
  int dkv() const { return dn + dv; }    // per-head kv_b_proj rows
  RopeParams rope;
  float eps, sigma;
};

// Element size in bytes of an mla_dtype (0 for an unknown code).
size_t dtype_size(int dt);

// Validates the configuration; fills dims and the kernel path.  Returns a status.
int check_config(const mla_config* cfg, Dims* d, Path* path);

// A bump allocator over one workspace: every region 256-byte aligned.
struct Layout {
  size_t top = 0;
  size_t take(size_t bytes) {
    size_t off = top;
    top += (bytes + 255) & ~size_t(255);
    return off;
  }
};

// Split-K of a GEMM's K range so that an M x N output grid covers the GPU: `n` slices of
// `chunk` (a multiple of 32) K values each; the last slice may be shorter.
struct SplitK {
  int n;
  int chunk;
};
SplitK gemm_splitk(long M, long N, long K, int tile_m, int tile_n);
// One K split shared by two skinny GEMMs (M <= 64 rows, N0 and N1 columns, K deep) launched
// together with 96-column tiles, sized so that the pair fills 256 CUs in one round; n = 0 when
// that launch does not apply (N0 or N1 not a multiple of 96, M > 64, K not a multiple of 64).
SplitK pair_splitk(long M, long N0, long N1, long K);
// K split of a prefill-sized fp32-output GEMM (M > 128 rows) for the 256 x 256-tile kernel:
// equal slices of whole 64-steps, as many as keep the work-groups within one round of 256 while
// filling at least 192 of them; n = 1 when the tiles alone reach 192 or no such split exists.
SplitK tile_splitk(long M, long N, long K);

struct CompressPlan {
  SplitK split;
  size_t off_acc;        // fp32 [split.n][T][W]
};
int plan_compress(const Dims& d, Path path, long T, Layout& L, CompressPlan* p, const SplitK* force = nullptr);

struct QueryPlan {            // q path for T tokens, shared by decode and prefill
  SplitK split_a, split_b;
  bool direct;                // prefill, bf16 path, no K split: the q projection writes the
                              // scaled fp16 queries straight into their final buffer
  size_t off_qa_acc;          // fp32 [split_a.n][T][dq]          (dq > 0)
  size_t off_cq;              // [T][dq] normed query latent       (dq > 0): act dtype, or a bf16
                              // hi + lo pair [T][2 dq] (decode, bf16 path) -- 4 bytes per value
  size_t off_q_acc;           // fp32 [split_b.n][T][H*dqk]        (!direct)
};

// Heads one decode work-group serves: 64 on the bf16 path (bf16 or fp8 cache; the last group is
// padded when H is not a multiple; the head groups of a sequence split stream its rows together),
// 1 on the fp32 path.
int decode_heads_per_group(const Dims& d, Path path);

// Longest batch for which the 64-head decode kernel takes the sequences longest first.
constexpr int kOrderMax = 2048;

struct DecodePlan {
  int splits;
  bool cq_pair;                // the grouped decode front applies: the query latent as a bf16 hi + lo
                              // pair, taken by the q_b projection as two products (bf16 path, dq > 0,
                              // dq % 64 == 0)
  bool hidden_pair;           // no query LoRA (bf16 path, B <= 128): the direct query projection
                              // and kv_a, both reading the hidden state, run in one launch with
                              // one K split
  bool ordered;               // rank the sequences by length before the attention (more than one
                              // round of work-groups on the 64-head kernel, at most 8 splits)
  size_t off_order;           // int32 [B]
  CompressPlan comp;
  QueryPlan q;
  size_t off_pos;             // int32 [B]
  size_t off_slot;            // int64 [B]
  size_t off_qnope;           // act  [B][H][dn]   scaled q_nope
  size_t off_rope;            // fp32 [B][dr]      RoPE angles of the decode tokens (cos | sin)
  size_t off_qhat;            // act  [B][H][W]    absorbed, scaled query
  size_t off_part_o;          // [B][splits][H][dc]: fp32 on the fp32 path, else fp16
  size_t off_part_ml;         // fp32 [B][splits][H][2]
  size_t off_otilde;          // fp32 [B][H][dc]: the merged state (many splits on the bf16 path)
  size_t off_ml1;             // fp32 [B][H][2]: merged state (0, 1) when the splits are merged first
  // Output projection (taken only when the weights carry o_proj; the regions are always planned,
  // inside regions that are dead by then):
  SplitK split_o;             // K split of the o_proj product (M = B, N = D, K = H * dv)
  bool o_wide;                // o_proj on the skinny kernel's 160-column tiles (bf16 path,
                              // B <= 128, D % 160 == 0), its split sized for them
  size_t off_attn;            // [B][H][dv] attention output (bf16 on the bf16 path, fp32 on the
                              // fp32 path): inside the qhat region when it fits
  size_t off_o_acc;           // fp32 [split_o.n][B][D] o_proj partials (split_o.n > 1): the
                              // otilde region, sized for both
  size_t bytes;
};
int auto_splits(const Dims& d, Path path, int B, int max_blocks);
int plan_decode(const Dims& d, Path path, int B, int max_blocks, int splits, DecodePlan* p);

struct PrefillPlan {
  CompressPlan comp;
  QueryPlan q;
  size_t off_pos;             // int32 [T]
  size_t off_slot;            // int64 [T]
  size_t off_qs;              // [T][H][dqk] scaled, RoPE'd queries (fp32; fp16 on the bf16 path)
  size_t off_lat;             // act  [S][kb][W] gathered (dequantised) cache rows of one key block
  size_t off_kpe;             // fp16 [S][kb][dr] their k_pe part (bf16 path)
  size_t off_kv;              // [S][kb][H*dkv] decompressed k_nope | v (fp32; fp16 on the bf16 path)
  size_t off_tscale;          // fp32 [S][kb] token scales of an fp8 cache (bf16 path)
  size_t off_wq16;            // fp16 copy of q_b_proj (bf16 path with a query LoRA, q16)
  bool q16;                   // bf16 path, dq > 0, dq % 64 == 0: the normed query latent and
                              // q_b_proj enter the q_b projection in fp16
  size_t off_attn;            // act [T][H][dv] attention output before o_proj (weights with o_proj)
  int kb;                     // key block: positions decompressed at a time (lat, kpe, kv and
                              // tscale hold kb rows per sequence); >= max_ctx: one block
  size_t off_state;           // fp32 [T][H][dv + 2] running softmax state between key blocks
  size_t bytes;
};
// key_block: mla_config.prefill_key_block (0: the library's choice).
int plan_prefill(const Dims& d, Path path, int S, int T, int max_q, int max_ctx, int key_block, PrefillPlan* p);

// Per-call argument checks (pointers, sizes); return a status.
int check_compress_args(const mla_config* cfg, const mla_weights* w, const void* hidden,
                        const int32_t* positions, const int64_t* slots, const mla_cache* cache,
                        int32_t T);
int check_decode_args(const mla_config* cfg, const mla_weights* w, const void* hidden,
                      const int32_t* context_lens, const int32_t* block_table, int32_t max_blocks,
                      const mla_cache* cache, int32_t B, int32_t splits, const void* out);
int check_prefill_args(const mla_config* cfg, const mla_weights* w, const void* hidden,
                       const int32_t* cu_seqlens, const int32_t* start_pos,
                       const int32_t* block_table, int32_t max_blocks, const mla_cache* cache,
                       int32_t S, int32_t T, int32_t max_q, int32_t max_ctx, const void* out);

}  // namespace mla
