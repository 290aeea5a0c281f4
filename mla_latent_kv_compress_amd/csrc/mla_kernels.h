// Internal launcher interface between the C ABI (mla_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_rope.h"

namespace mla {

enum GemmKind { GEMM_F32 = 0, GEMM_BF16 = 1 };

struct GemmArgs {
  int kind;                  // GEMM_F32 (fp32 in/out) or GEMM_BF16 (bf16 in, fp32 accumulate)
  bool nn;                   // W is [K][N] (else [N][K])
  int out;                   // bf16 path output: K_F32, K_BF16 or K_F16
  int M, N, K;
  int kchunk, nsplit;        // K split into nsplit slices of kchunk (multiple of 32)
  int batch;
  const void* X; long lda, sx;
  const void* W; long ldw, sw;
  void* Y; long ldc, sy, ssplit;
  float alpha;
  bool xpair = false;        // X is a bf16 hi + lo pair, row m holding hi in columns [0, K) and
                             // lo in [K, 2K) (lda counts bf16 values), that enters the products as
                             // two (skinny kernel only: launch_gemm_skinny_ok must hold)
  bool f16in = false;        // X and W are fp16 (large-tile kernel only)
  const float* row_scale = nullptr;  // large-tile kernel: output row m of batch z times
  long srs = 0;                      // row_scale[z * srs + m]
  int bn = 0;                // skinny kernel column tile: 0 chooses 64 or 96; 160 (N % 160 == 0)
                             // for wide outputs whose K split was planned with it
};
void launch_gemm(const GemmArgs& g, hipStream_t st);
// 256 x 256-tile GEMM (k_gemm_tile.hip) for large TN products: bf16 or fp16 outputs without a K
// split (the prefill's q_b projection and kv_b decompression), or fp32 outputs, also as K-split
// partials of equal slices for more than 128 rows (the prefill's kv_a and q_a); bf16 or fp16
// operands, optional per-row output scale; false if the problem does not fit.
bool launch_gemm_tile(const GemmArgs& g, hipStream_t st);
// Whether the large-tile kernel takes the problem's shape (always so for fp16 operands or a row
// scale, which only it implements).
bool launch_gemm_tile_ok(const GemmArgs& g);
// Whether the skinny (decode-batch) kernel takes this problem; required for xpair.
bool launch_gemm_skinny_ok(const GemmArgs& g);
// Two independent fp32-output skinny GEMMs in one launch; false (nothing launched) when either
// does not meet the skinny kernel's conditions.
bool launch_gemm_pair(const GemmArgs& a, const GemmArgs& b, hipStream_t st);

// Dtype codes for cache, activations and intermediate buffers inside the kernels.
enum { K_F32 = 0, K_BF16 = 1, K_FP8 = 2, K_F16 = 3 };

// Cache rows from fp32 kv_a partials: RMSNorm on the latent, RoPE on k_pe, cast, scatter.
void launch_compress_rows(int act, int cache, int T, int dc, int dr, int nsplit, const float* acc,
                          const void* gamma, const int32_t* pos, const int64_t* slots,
                          void* cache_data, float* cache_scale, long num_slots, float eps,
                          const RopeParams& rp, float* rope_tab, const int32_t* ctx, const int32_t* bt, int max_blocks,
                          hipStream_t st, int qsplit_n = 1, const float* q_acc = nullptr, int H = 0,
                          float alpha = 1.f, float* q_nope32 = nullptr, float* q_pe32 = nullptr);
// (With q_acc, the same launch also does launch_q_split_sum's work for T tokens of H heads.)
// Decode queries on the bf16 path, from the fp32 query projection q ([nsplit][B][H][dn + dr]):
// qhat[b][h] = [ W_UK^h^T (scale q_nope) (bf16, dc values) | scale RoPE(q_pe) (fp16, dr values) ],
// q_nope entering the products as a bf16 hi + lo pair; the angles of each token come from
// rope_tab ([B][dr]: cos | sin).  With q_nope32 / q_pe32 the query comes from the split epilogue
// instead (q_nope32 already scaled).  False if the shape does not apply (dn 128, dc 512).
bool launch_absorb_rope(int B, int H, int dn, int dr, int dc, int dv, int nsplit, const float* q_acc,
                        const float* rope_tab, float scale, const void* kv_b, void* qhat, hipStream_t st,
                        const float* q_nope32 = nullptr, const float* q_pe32 = nullptr);
// Decode q_b projection (no K split, N = H x 192) whose epilogue stores q_nope as fp32 alpha q
// to g.Y [M][H][128] and q_pe as fp32 q to q_pe [M][H][64] (the absorb kernel's split input);
// false (nothing launched) if the skinny kernel does not apply.
bool launch_q_split_gemm(const GemmArgs& g, float* q_pe, hipStream_t st);

// out[t][:] = RMSNorm(sum_s acc[s][t][:]) * gamma, in act dtype (or fp16, saturating, with
// out_f16 on the bf16 path).
void launch_rmsnorm_rows(int act, int T, int n, int nsplit, const float* acc, const void* gamma,
                         void* out, float eps, hipStream_t st, bool out_f16 = false);
// dst = fp16 copy of n bf16 values (n a multiple of 8, 16-byte aligned), saturating at +-65504.
void launch_bf16_to_f16(const void* src, void* dst, long n, hipStream_t st);
// Decode, bf16 activations: the compress epilogue (positions from the context lengths, RoPE
// table written) and the query-latent RMSNorm (cq: bf16 hi + lo pair [T][2 nq]) in one launch
// of 2T blocks; false if unsupported.
bool launch_decode_rows(int act, int cache, int T, int dc, int dr, int nsplit_kv, const float* acc_kv,
                        const void* gamma_kv, void* cache_data, float* cache_scale, long num_slots, float eps,
                        const RopeParams& rp, float* rope_tab, const int32_t* ctx, const int32_t* bt, int max_blocks,
                        int nq, int nsplit_q, const float* acc_q, const void* gamma_q, void* cq, hipStream_t st);

// Query packing from fp32 partials q_acc [nsplit][T][H*(dn+dr)]: sum, scale by `scale`,
// RoPE on q_pe.
//   absorbed: q_nope -> qnope[t][h][dn]; rotated q_pe -> qhat[t][h][dc + i]  (act dtype)
//   explicit: [q_nope | rotated q_pe] -> qs[t][h][dn + dr]                   (qs_type)
void launch_q_pack(int act, int qs_type, bool absorbed, int T, int H, int dn, int dr, int dc,
                   int nsplit, const float* q_acc, const int32_t* pos, float scale, const RopeParams& rp,
                   void* qnope, void* qhat, void* qs, hipStream_t st);
// RoPE in place on the q_pe part of fp16 queries qs[t][h][dn + dr] (already scaled).
void launch_q_rope_f16(int T, int H, int dn, int dr, const int32_t* pos, const RopeParams& rp, void* qs,
                       hipStream_t st);

void launch_decode_prep(int B, const int32_t* ctx, const int32_t* bt, int max_blocks,
                        int32_t* pos, int64_t* slot, hipStream_t st);
void launch_prefill_prep(int S, int max_q, const int32_t* cu, const int32_t* start,
                         const int32_t* bt, int max_blocks, int32_t* pos, int64_t* slot,
                         hipStream_t st);

// Split-K decode attention over the latent cache (weight-absorbed form).
//   qhat [B][H][dc+dr] (pre-scaled by sigma*log2 e), partials o [B][S][H][dc], ml [B][S][H][2]
struct DecodeAttnArgs {
  int B, H, dc, dr, splits;
  const void* qhat;
  const void* cache; const float* cache_scale;
  const int32_t* block_table; int max_blocks;
  const int32_t* ctx;
  void* part_o;              // [B][splits][H][dc]: fp32 on the fp32 path, fp16 (scaled state) on the bf16 path
  float* part_ml;
  int32_t* order = nullptr;   // [B] scratch: sequences by length, longest first (64-head kernel)
};
// False (nothing launched) when no kernel takes the shape.
bool launch_decode_attn(int act, int cache, const DecodeAttnArgs& a, hipStream_t st);
// 64-head work-groups over a bf16 or fp8 cache (k_decode.hip); false if the shape does not apply.
// With a.order set, a first kernel ranks the sequences by context length (a.B <= kOrderMax) and
// the work-groups take them longest first.
bool launch_decode_attn_v2(int cache_type, const DecodeAttnArgs& a, hipStream_t st);

// Merge of the split partials fused with the W_UV projection (bf16 path, dc = 512, dv = 128):
// out[b][h] = W_UV^h Otilde[b][h], out fp32 or bf16 per out_type; false if the shape does not apply.
// With more than 4 splits (dc 512) and the two fp32 scratch buffers otilde [B][H][dc] and
// ml1 [B][H][2], the splits are merged by a first kernel and the projection reads the result.
// The bf16 path's partials O_j are fp16 (the attention scales each (split, head) state by a power of two).
bool launch_decode_merge_uv(int out_type, int B, int H, int dc, int dn, int dv, int splits, const uint16_t* part_o,
                            const float* part_ml, const void* kv_b, void* out, hipStream_t st,
                            float* otilde = nullptr, float* ml1 = nullptr);
void launch_merge_splits(int B, int H, int dc, int splits, const uint16_t* part_o, const float* part_ml,
                         float* otilde, float* ml1, hipStream_t st);
// The fp32 path's merge: otilde [B][H][dc] fp32.
void launch_decode_merge(int B, int H, int dc, int splits, const float* part_o, const float* part_ml,
                         float* otilde, hipStream_t st);

// Prefill: gather the cached rows of positions [k0, k0 + rows) of each sequence (zeros past its
// context) into lat [S][kb][W], row t for position k0 + t (an fp8 cache's codes as their exact
// values, the token scales into tscale [S][kb]); with kpe16 also their k_pe part (columns
// [dc, W), dequantised) in fp16 into kpe16 [S][kb][W - dc].
void launch_gather_rows(int act, int cache, int S, int k0, int rows, int kb, int W, int dc, const int32_t* cu,
                        const int32_t* start, const int32_t* bt, int max_blocks,
                        const void* cache_data, const float* cache_scale, void* lat, void* kpe16,
                        float* tscale, hipStream_t st);

// Causal attention of packed chunk queries against decompressed keys / values.
// Keys and values of positions [k0, k0 + kb) (one key block; row t is position k0 + t).
// state_in (null for the first block) holds the running softmax state the previous block left,
// state_out (null for the last block) receives it instead of the output: fp32 [T][H][dv + 2],
// per (query, head) the unnormalised output, then the running max and the row sum (bf16 path;
// the fp32 path takes the whole context as one block).
struct PrefillAttnArgs {
  int S, H, dn, dr, dv, dc, max_q, max_ctx, out_type;
  const int32_t* cu; const int32_t* start;
  const void* qs;            // [T][H][dn+dr], pre-scaled by sigma*log2 e (fp16 on the bf16 path)
  const void* kv;            // [S][kb][H][dn+dv]  (fp16 on the bf16 path)
  const void* lat;           // [S][kb][dc+dr] act dtype (k_pe at column dc)
  const void* kpe;           // [S][kb][dr] fp16 copy of k_pe (bf16 path)
  void* out;                 // [T][H][dv] out_type
  int k0 = 0, kb = 0;
  const float* state_in = nullptr;
  float* state_out = nullptr;
};
// False (nothing launched) when no kernel takes the shape.
bool launch_prefill_attn(int act, const PrefillAttnArgs& a, hipStream_t st);
// Flash-style causal prefill attention (k_prefill.hip), bf16 path with nope 128, rope 64, v 128,
// d_c 512; false if the shape does not apply.
bool launch_prefill_attn_fa(const PrefillAttnArgs& a, hipStream_t st);

// Elementwise e4m3fn codec of the fp8 cache: encode fp32 -> codes, or decode codes -> fp32.
void launch_fp8_codec(bool encode, const void* in, void* out, long n, hipStream_t st);
// Decode query (nope 128, rope 64): the projection's partials acc [nsplit][T][H][192] summed into
// q_nope32 [T][H][128] = alpha q_nope and q_pe32 [T][H][64] (fp32; the absorb's split input).
void launch_q_split_sum(int T, int H, int nsplit, const float* acc, float alpha, float* q_nope32, float* q_pe32,
                        hipStream_t st);
// out[i] = sum over the nsplit slices of acc ([nsplit][n] fp32), stored fp32 or bf16 per out_type.
void launch_sum_splits(int out_type, long n, int nsplit, const float* acc, void* out, hipStream_t st);
// Reads n16 16-byte words and discards them: mode 0 with plain loads into registers (a read
// sweep that leaves clean lines in the caches), mode 1 with non-temporal direct loads into LDS
// (the fastest read pattern measured: the reference for the achievable read bandwidth).
void launch_stream_read(const void* p, long n16, uint32_t* sink, int mode, hipStream_t st);

}  // namespace mla
