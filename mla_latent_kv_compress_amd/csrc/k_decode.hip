// Split-K decode attention over a bf16 or fp8 latent cache, 64 heads per work-group
// (weight-absorbed).  A layer of 32 heads or fewer runs an instance that skips the group's empty
// head tiles.
//
// One work-group of 8 waves per (sequence, split, group of 64 heads), two waves per SIMD with
// separate roles:
//   score waves 0-3   wave w owns token tile w & 1 (16 tokens of each stage) and head half
//                     w >> 1 (32 heads): S[token][head] = R . Qhat^T with
//                     v_mfma_f32_16x16x32_bf16 over the latent and v_mfma_f32_16x16x32_f16 over
//                     the RoPE part (the query's RoPE part is fp16, the key's converted exactly)
//                     (2 head tiles, 18 K steps over two accumulators per tile), the query slice
//                     (144 registers) held for the whole split;
//                     softmax per head in base 2 (log2 e is folded into Qhat); P to LDS.
//   value waves 4-7   wave 4+w owns latent columns [128w, 128w+128) for the 64 heads:
//                     O^T[c][head] += R^T . P^T with v_mfma_f32_32x32x16_bf16 (4 column tiles x
//                     2 head tiles, 2 K steps of 16 tokens), R^T read with transposing LDS reads;
//                     they also issue the direct global->LDS loads of the cache rows.
// The split's rows stream through LDS in stages of 32 tokens (bf16: 36 KiB, a ring of 4, three
// stages ahead; fp8: 18 KiB plus the scales, a ring of 8, seven ahead).  Step i runs the value
// product of stage i next to the score product of stage i + 1 (on different waves of each SIMD),
// with one work-group barrier per step.  The cached latent is also the value, so one LDS stage
// feeds both products.  The work-groups of the head groups of one (sequence, split) are dealt to
// the same XCD next to each other, so they stream the same rows together and the second read of
// every row is an L2 hit: the cache leaves HBM once per split.
//
// LDS: a stage holds rows of 72 16-byte chunks, unpadded (each direct load instruction fills a
// contiguous KiB), with chunk c of row r stored at c ^ rsw(r), rsw(r) < 8 (the XOR stays inside
// an aligned group of 8 chunks, so a load instruction still covers one contiguous KiB of the
// page).  Measured on gfx950, this choice lets the score operand reads (16 rows x 4 chunks per
// instruction) run at the full 128-bit LDS rate, about twice the rate of the unswizzled rows or
// of some other XOR patterns; the transposing reads run at their own (lower) rate whatever the
// pattern.  P is stored [head][token] (64 bytes per head) with the chunk index XORed by
// (head >> 2) & 3.
//
// Reference max: each head accumulates p = 2^(s - m) against a reference m fixed after the
// first stage (that stage's max), so the accumulators are never rescaled inside the loop.  Later
// scores may exceed m; p <= 2^kSlack stays far inside bf16 and fp32 range.  If some head's stage
// max exceeds m + kSlack, the work-group drops what it accumulated, makes a scores-only pass over
// the split to find every head's exact max, and accumulates again with that reference (exact,
// and it costs two extra passes only on such splits).  The partial state (m, l, O) is consistent
// for the log-sum-exp merge whatever m is.  Rows of a stage beyond the context re-read the last
// valid row (finite data) and get p = 0.
//
// The split's state leaves as (m - k, 2^k l, 2^k O) with O in fp16, k chosen per head so that
// the largest |O| entry lies in [2^14, 2^15) (the value waves exchange their per-head maxima and
// the score waves their row sums through LDS): the same state, half the bytes of fp32, and 11
// significant bits where bf16 would keep 8.
//
// fp8 cache (e4m3 codes plus one fp32 scale per token): the same kernel with 576-byte rows, so a
// 32-token stage is 18 KiB of codes plus the stage's 32 scales, and the ring holds 8 stages.  The
// token scale s_t is applied outside the products: score = s_t (code . Qhat), and the value
// product takes p s_t as its weight (l still sums p).  Scores over the latent use the codes as
// they are, in v_mfma_scale_f32_16x16x128_f8f6f4 (K 128 per product, A: two 128-bit reads per
// lane, block scale 1) against the query slice as two e4m3 codes per value, hi and lo, with
// per-head power-of-two block scales 2^e and 2^(e - 4): hi + lo / 16 keeps the 8 significant
// bits of the bf16 query, and an fp8 product does twice the bf16 work per cycle, so the pair
// costs the bf16 product's matrix time while the conversion of every key code disappears.  The
// RoPE part's codes are converted exactly to fp16 for fp16 products, and the value operand (one
// ds_read_b64_tr_b8: lane i of each 16-lane group gets column c0 + i over the 8 rows addressed
// by lanes 2j, 2j + 1) exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1).  Stored chunk of
// row r, logical chunk c: c ^ ((r >> 2) & 3).
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_lds.h"
#include "mla_plan.h"

namespace mla {

namespace {

constexpr int kDC = 512, kDR = 64, kDW = kDC + kDR;
constexpr int kStage = 32;                            // tokens per pipeline stage
constexpr int kThreads = 512;                         // 4 score waves + 4 value waves

// Per cache type: row bytes, stage codes, ring slot size and depth, direct loads per value-wave
// thread per stage.
template <bool FP8> struct Geo;
template <> struct Geo<false> {
  static constexpr int kRowBytes = kDW * 2;           // 1152
  static constexpr int kCodeBytes = kStage * kRowBytes;   // 36864
  static constexpr int kSlot = kCodeBytes;
  static constexpr int kRing = 4;
  static constexpr int kLoads = kCodeBytes / 16 / 256;    // 9 dwordx4 loads
};
template <> struct Geo<true> {
  static constexpr int kRowBytes = kDW;               // 576
  static constexpr int kCodeBytes = kStage * kRowBytes;   // 18432: 18 dwordx4 loads per stage
  static constexpr int kScaleOff = kCodeBytes;        // two copies of the stage's scales (256 B each)
  static constexpr int kSlot = kCodeBytes + 512;
  static constexpr int kRing = 8;
  // Waves 0, 1: code loads 4k + w, k < 5; waves 2, 3: code loads 4k + w, k < 4, and one dword
  // load of the stage's scales.
  static constexpr int kLoads = 5;
};
constexpr int kKS = kDW / 32;                         // 18 score K steps
constexpr int kHeads = 64;                            // heads per work-group
constexpr int kPBytes = kHeads * kStage * 2;          // 4096
constexpr float kSlack = 64.0f;
constexpr int kChecked = 0, kFixed = 2;                   // pass kinds
constexpr int kScoreRing = 5;                         // score operand fragments in flight + 1

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int rsw(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }
__device__ __forceinline__ int psw(int h) { return (h >> 2) & 3; }

__device__ __forceinline__ s16x4_t tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ bf16x8_t join(s16x4_t lo, s16x4_t hi) {
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = {(__bf16)a, (__bf16)b};                 // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  f16x2_t v = {(_Float16)a, (_Float16)b};             // round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// Exponent k of the power-of-two scale a split's state (m, l, O) leaves with: (m - k, 2^k l,
// 2^k O) stands for the same 2^m (l, O).  The largest |O| entry a lands in [2^14, 2^15), where
// fp16 holds it and every entry down to 2^-29 a with 11 significant bits, unless 2^k l would
// pass 2^100 (a state whose largest entry is below 2^-85 l, i.e. latent values that small).
__device__ __forceinline__ int part_scale(float a, float l) {
  if (!(a > 0.f) || a == INFINITY) return 0;        // an empty split (a = 0) keeps its state
  int ea, el;
  frexpf(a, &ea);                                    // a < 2^ea
  frexpf(l, &el);
  return min(15 - ea, 100 - el);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one per 16-lane row) with the gfx950
// row-swap instructions (VALU, no LDS round trip): permlane16_swap(x, x) returns rows (0,0,2,2)
// and (1,1,3,3) of x, permlane32_swap(x, x) returns rows (0,1,0,1) and (2,3,2,3).
__device__ __forceinline__ float max_across_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

using lds::dma16;
__device__ __forceinline__ void dma16nt(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}
using lds::dma4;
using lds::wait_vm;
__device__ __forceinline__ void lds_barrier() { lds::barrier(); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return lds::addr(p); }

// Offset, within a stage, of the 16 bytes that lane `lane` of direct-load instruction k of wave
// `wave` fetches: instruction k of wave w fills LDS bytes [(4k + w) KiB, +1 KiB) of the stage;
// lane i supplies stored chunk (4k + w) * 64 + i.  bf16 rows (72 chunks): row r = chunk / 72,
// logical chunk (chunk % 72) ^ rsw(r).  fp8 rows (36 chunks): row r = chunk / 36, logical chunk
// (chunk % 36) ^ ((r >> 2) & 3).  Rows at or beyond `valid` re-read row valid - 1.
template <bool FP8>
__device__ __forceinline__ uint32_t stage_offset(int k, int wave, int lane, int valid) {
  constexpr int kChunks = Geo<FP8>::kRowBytes / 16;
  const int idx = (4 * k + wave) * 64 + lane;
  const int r = idx / kChunks, cp = idx - r * kChunks;
  const int c = FP8 ? (cp ^ ((r >> 2) & 3)) : (cp ^ rsw(r));
  const int rs = r < valid ? r : valid - 1;
  return uint32_t(rs * Geo<FP8>::kRowBytes + c * 16);
}

// Wait until at most A * L of this wave's direct loads are outstanding, A the largest of
// A_MAX, ..., 1 not above `ahead` (0 if none).
template <int A, int L>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (A == 0) {
    wait_vm<0>();
  } else {
    if (ahead >= A) wait_vm<A * L>();
    else wait_ahead<A - 1, L>(ahead);
  }
}

typedef int v2i_t __attribute__((ext_vector_type(2)));

// Eight bf16 values to fp16, exactly for magnitudes in [2^-14, 65504] (the RoPE key's range;
// smaller ones lose at most 2^-24, larger ones saturate).
__device__ __forceinline__ f16x8_t bf16x8_to_f16(bf16x8_t v) {
  const uint4 u = __builtin_bit_cast(uint4, v);
  auto cv = [](uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                   __uint_as_float(w & 0xFFFF0000u)));
  };
  return __builtin_bit_cast(f16x8_t, make_uint4(cv(u.x), cv(u.y), cv(u.z), cv(u.w)));
}

// Eight e4m3 codes (two words, code j in byte j) to eight fp16 values, exactly.
__device__ __forceinline__ f16x8_t fp8x8_to_f16(uint32_t w0, uint32_t w1) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(w0), 1.0f, false);
  const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(w0), 1.0f, true);
  const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(w1), 1.0f, false);
  const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(int(w1), 1.0f, true);
  return f16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight e4m3 codes (two words, code j in byte j) to eight bf16 values, exactly.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w0), 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w0), 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w1), 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w1), 1.0f, true);
  return bf16x8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

typedef int v8i_t __attribute__((ext_vector_type(8)));

// Four query values x (already divided by their head's power-of-two scale, |x| < 256) as e4m3
// codes in two words: hi = e4m3(x) and lo = e4m3(16 (x - hi)), both rounded to nearest even
// (code j in byte j).  hi + lo / 16 carries 8 significant bits, the precision of the bf16 query.
__device__ __forceinline__ void e4m3_pair4(float x0, float x1, float x2, float x3, int& hi, int& lo) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  s16x2_t h = {0, 0}, l = {0, 0};
  h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x0, x1, 1.0f, false);
  h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, x2, x3, 1.0f, true);
  hi = __builtin_bit_cast(int, h);
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, 1.0f, true);
  l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, 16.f * (x0 - a[0]), 16.f * (x1 - a[1]), 1.0f, false);
  l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, 16.f * (x2 - b[0]), 16.f * (x3 - b[1]), 1.0f, true);
  lo = __builtin_bit_cast(int, l);
}

}  // namespace

template <bool FP8, int HT>
__global__ __launch_bounds__(kThreads, 1) void decode_attn_latent_kernel(
    int H, int splits, int max_blocks, int by_seq, int nunits, const uint16_t* __restrict__ qhat,
    const void* __restrict__ cache, const float* __restrict__ cache_scale, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ ctx_lens, const int32_t* __restrict__ order, uint16_t* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using Gm = Geo<FP8>;
  constexpr int kRowBytes = Gm::kRowBytes, kSlot = Gm::kSlot, kRing = Gm::kRing, kLoads = Gm::kLoads;
  constexpr int kPageBytes = kPage * kRowBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kRing * kSlot + 2 * kPBytes];
  char* const ring = smem;
  char* const pbase = smem + kRing * kSlot;                // P of stage j in pbase + (j & 1) * kPBytes
  auto slot = [&](int j) { return ring + (j & (kRing - 1)) * kSlot; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool scorer = wid < 4;                             // else a value wave
  const int wave = wid & 3;                                // index within the role
  const int g = lane >> 4, li = lane & 15;
  // Work-group -> (sequence slot, split, head group).  Work-groups are dealt to the 8 XCDs
  // round-robin; the head groups of one (sequence, split) land on the same XCD in consecutive
  // rounds (by_seq: eight sequences' splits per round, B % 8 == 0; else eight (sequence, split)
  // units per round, their count nunits padded to a multiple of 8 by work-groups that leave at
  // once).  Slots go to sequences in `order` (longest first) when it is given, so
  // the long sequences' work-groups are dispatched first and the short ones fill in behind them.
  const int G = (H + kHeads - 1) / kHeads;                  // the last group may be partial
  int b, sp, hg;
  {
    const int unit = blockIdx.x;
    const int k = unit >> 3;
    const int k2 = k / G;
    hg = k - k2 * G;
    if (by_seq) {
      b = (k2 / splits) * 8 + (unit & 7);
      sp = k2 - (k2 / splits) * splits;
    } else {
      const int u = k2 * 8 + (unit & 7);
      if (u >= nunits) return;                             // padding (uniform over the work-group)
      b = u / splits;
      sp = u - b * splits;
    }
    if (order) b = order[b];
  }
  const int hbase = hg * kHeads;
  const int ctx = ctx_lens[b];
  const int nst = (ctx + kStage - 1) / kStage;
  const int per = (nst + splits - 1) / splits;
  const int s0 = sp * per;
  const int n = max(0, min(nst, s0 + per) - s0);
  const char* cbase = reinterpret_cast<const char*>(cache);
  const int32_t* btab = bt + long(b) * max_blocks;
  auto stage_valid = [&](int j) { return j < n ? min(kStage, ctx - kStage * (s0 + j)) : 0; };

  // ---- value-wave state: direct loads, transposing reads, accumulators
  uint32_t full_off[kLoads];             // offsets of a stage whose rows are all cached
  if (!scorer) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) full_off[k] = stage_offset<FP8>(k, wave, lane, kStage);
  }
  // Loads of stage j (of this split) into ring slot j % kRing.  fp8: the last load of waves 2
  // and 3 fetches the stage's scales (lane i: token i % 32) into their own copy.
  auto issue = [&](int j) {
    if (j >= n) return;
    char* dst = slot(j);
    const long page = btab[(s0 + j) >> 1];
    const int half = (s0 + j) & 1;
    const char* src = cbase + page * kPageBytes + half * Gm::kCodeBytes;
    const int valid = stage_valid(j);
    constexpr int kCode = FP8 ? kLoads - 1 : kLoads;      // code loads every wave issues
    if (valid == kStage) {
#pragma unroll
      for (int k = 0; k < kCode; ++k) dma16nt(src, full_off[k], lds_addr(dst + (4 * k + wave) * 1024));
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int k = 0; k < kCode; ++k)
        dma16nt(src, stage_offset<FP8>(k, wave, ln, valid), lds_addr(dst + (4 * k + wave) * 1024));
    }
    if constexpr (FP8) {
      if (wave < 2) {
        dma16nt(src, valid == kStage ? full_off[kLoads - 1] : stage_offset<FP8>(kLoads - 1, wave, lane, valid),
              lds_addr(dst + (4 * (kLoads - 1) + wave) * 1024));
      } else {
        const char* ssrc = reinterpret_cast<const char*>(cache_scale) + (page * kPage + kStage * half) * 4;
        const int t = min(lane & (kStage - 1), valid - 1);
        dma4(ssrc, uint32_t(4 * t), lds_addr(dst + Gm::kScaleOff + 256 * (wave - 2)));
      }
    }
  };
  // Wait until stage j is in LDS, stages up to `last` having been issued (in order).
  auto wait_stage = [&](int j, int last) { wait_ahead<kRing - 2, kLoads>(min(n - 1, last) - j); };

  // ---- shared LDS addressing
  // Score operand offsets.  A score wave owns token tile mt_w (tokens [16 mt_w, 16 mt_w + 16) of
  // every stage) and head half hh (heads [32 hh, 32 hh + 32) of the group).
  // bf16: row 16 mt + li, logical chunk 4 ks + g, stored at (4 ks + g) ^ rsw(li) = 4 (ks ^ y) + x
  // (rsw(16 mt_w + li) = rsw(li)).
  // fp8: read m (m < 9) is 16 bytes per lane: row 16 mt + li, logical chunk 4m + g, stored at
  // 4m + (g ^ ((li >> 2) & 3)), i.e. columns 64m + 16g .. +15; reads 2 kb and 2 kb + 1 form the
  // A operand of latent block kb, read 8 the two fp16 K steps of the RoPE part (byte 8e + j:
  // column 512 + 16g + 8e + j).  The query is loaded to match.
  const int mt_w = wave & 1, hh = wave >> 1;
  // Live 16-head tiles of the group: HT of 4.  A narrow layer (H <= 32) fills only head half 0:
  // the score waves of head half 1 skip their products and operand reads, and so do the value
  // waves for their second 32-head tile (its P rows are never read).
  static_assert(HT == 1 || HT == 2 || HT == 4, "live head tiles");
  constexpr int kSNT = HT >= 2 ? 2 : 1;                    // score head tiles of a live score wave
  constexpr int kVNT = HT == 4 ? 2 : 1;                    // value head tiles
  const bool s_live = 32 * hh < 16 * HT;
  const int sx = g ^ (rsw(li) & 3), sy = rsw(li) >> 2;
  const int s_row = (16 * mt_w + li) * kRowBytes + 16 * (FP8 ? (g ^ ((li >> 2) & 3)) : sx);
  const int s_even = s_row + 64 * sy;                      // ks even: + 64 ks
  const int s_odd = s_row - 64 * sy;                       // ks odd:  + 64 ks
  auto score_a = [&](const char* st, int ks) {
    return *reinterpret_cast<const bf16x8_t*>(st + ((ks & 1) ? s_odd : s_even) + 64 * ks);
  };
  auto score_raw = [&](const char* st, int m) { return *reinterpret_cast<const uint4*>(st + s_row + 64 * m); };
  // Transposing reads for the value product.
  // bf16: lane reads row 8 (lane >> 5) + 4 rd + (li >> 2) (+16 per K step), element column
  // 128 w + 32 ct + 16 ((lane >> 4) & 1) + 4 (li & 3).
  // fp8: lane reads row 8 (lane >> 5) + (li >> 1) (+16 per K step), byte column
  // 128 w + 32 ct + 16 ((lane >> 4) & 1) + 8 (li & 1); the row's chunk XOR (r >> 2) & 3 is
  // (2 (lane >> 5) + (li >> 3)), so column tiles ct = 2u + e sit at t_even / t_odd + 64 u.
  int t_even[2], t_odd[2];
  if constexpr (FP8) {
    const int f1 = lane >> 5, f0 = li >> 3, e = (lane >> 4) & 1;
    const int rr = 8 * f1 + (li >> 1);
    const int base = rr * kRowBytes + 16 * (8 * wave + (e ^ f0)) + 8 * (li & 1);
    t_even[0] = base + 32 * f1;
    t_odd[0] = base + 32 * (1 - f1);
    t_even[1] = t_odd[1] = 0;
  } else {
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int rr = 8 * (lane >> 5) + 4 * rd + (li >> 2);
      const int gs = rsw(rr);
      const int x = 2 * ((lane >> 4) & 1) + ((li & 3) >> 1);
      const int base = rr * kRowBytes + 256 * wave + 16 * (x ^ (gs & 3)) + 8 * (li & 1);
      t_even[rd] = base + 64 * (gs >> 2);
      t_odd[rd] = base - 64 * (gs >> 2);
    }
  }
  auto val_a = [&](const char* st, int ks, int ct) {
    const int add = 64 * ct + ks * 16 * kRowBytes;
    const char* p0 = st + ((ct & 1) ? t_odd[0] : t_even[0]) + add;
    const char* p1 = st + ((ct & 1) ? t_odd[1] : t_even[1]) + add;
    return join(tr_read(p0), tr_read(p1));
  };
  auto val_raw = [&](const char* st, int ks, int ct) {
    const char* p = st + ((ct & 1) ? t_odd[0] : t_even[0]) + 64 * (ct >> 1) + ks * 16 * kRowBytes;
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i_t __attribute__((address_space(3)))*)(p));
  };
  const int ph = lane & 31;
  // P operand: Pbuf[head 32 nt + ph][tokens 16 ks + 8 (lane >> 5) .. +7].
  auto p_frag = [&](const char* pb, int ks, int nt) {
    const int h = 32 * nt + ph;
    const int c = 2 * ks + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(pb + h * 64 + 16 * (c ^ psw(h)));
  };

  // ---- score-wave state
  // Query fragments (B operand of the score product): Qhat[head 32 hh + 16 nt + li][32 ks + 8 g .. +7].
  // Heads past H (a partial last group, e.g. 16 heads in a group of 64) get a zero query: their
  // scores are 0, their sums finite, and nothing of theirs is stored.
  // fp8 cache: the latent part enters scaled fp8 products of K 128 (block kb: latent columns
  // [128 kb, 128 kb + 128)) whose A operand is two of the 16-byte score reads above, so lane
  // (li, g) holds columns 128 kb + 16 g .. +15 and 128 kb + 64 + 16 g .. +15 of its head, as e4m3
  // codes hi (qc[..][0], block scale 2^e) and lo (qc[..][1], 2^(e - 4)), e the head's exponent
  // (its largest |value| below 2^(e + 8)); the RoPE part stays fp16 (qr: columns
  // 512 + 16 g + 8 i .. +7).
  bf16x8_t qf[2][FP8 ? 1 : kKS];
  v8i_t qc[2][FP8 ? 4 : 1][2];
  f16x8_t qr[2][2];
  int qsh[2], qsl[2];                                      // hi / lo E8M0 scale bytes per head tile
  if (scorer) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int head = hbase + 32 * hh + 16 * nt + li;
      const uint16_t* q = qhat + (long(b) * H + min(head, H - 1)) * kDW;
      if constexpr (FP8) {
        bf16x8_t v[4][4];                                  // [kb][columns +0, +8, +64, +72]
        float amax = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) {
            const int col = 128 * kb + 64 * (pt >> 1) + 16 * g + 8 * (pt & 1);
            v[kb][pt] = head < H ? *reinterpret_cast<const bf16x8_t*>(q + col) : bf16x8_t{};
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(float(v[kb][pt][j])));
          }
        amax = max_across_rows(amax);                      // over the head's four lanes
        int ea = 0;
        frexpf(amax, &ea);                                 // amax < 2^ea
        const int e = amax > 0.f ? max(ea - 8, -119) : 0;
        const float inv = __uint_as_float(uint32_t(127 - e) << 23);   // 2^-e
        qsh[nt] = 127 + e;
        qsl[nt] = 123 + e;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int pt = 0; pt < 4; ++pt)
#pragma unroll
            for (int w = 0; w < 2; ++w) {
              int hi, lo;
              e4m3_pair4(inv * float(v[kb][pt][4 * w]), inv * float(v[kb][pt][4 * w + 1]),
                         inv * float(v[kb][pt][4 * w + 2]), inv * float(v[kb][pt][4 * w + 3]), hi, lo);
              qc[nt][kb][0][2 * pt + w] = hi;
              qc[nt][kb][1][2 * pt + w] = lo;
            }
#pragma unroll
        for (int i = 0; i < 2; ++i)
          qr[nt][i] = head < H ? *reinterpret_cast<const f16x8_t*>(q + kDC + 16 * g + 8 * i) : f16x8_t{};
      } else {
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks)
          qf[nt][ks] = head < H ? *reinterpret_cast<const bf16x8_t*>(q + 32 * ks + 8 * g) : bf16x8_t{};
      }
    }
  }
  float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  f32x4_t s[2][2];                      // [head tile][K-step parity]
  f32x16_t o[4][2];
  // The two score waves of a head half (wave and wave ^ 1) exchange their per-head maxima and
  // row sums through LDS: xm / lx[head][token tile], in the second P buffer (idle then).
  float* const xm = reinterpret_cast<float*>(pbase + kPBytes);
  float* const lx = reinterpret_cast<float*>(pbase + kPBytes + 2 * kHeads * 4);
  auto hrow = [&](int nt) { return 32 * hh + 16 * nt + li; };
  // At the end of the split: xa[value wave][head] = largest |O| entry over the wave's columns,
  // xl[head] = the head's row sum (in the ring, idle by then).
  float* const xa = reinterpret_cast<float*>(ring);
  float* const xl = reinterpret_cast<float*>(ring + 4 * kHeads * 4);
  // fp8: scales of the lane's four tokens 16 mt_w + 4 g + j of the current stage (read by scores).
  f32x4_t tsc = f32x4_t{1.f, 1.f, 1.f, 1.f};

  // Scores of the stage's tile (C layout: lane holds tokens 16 mt_w + 4 g + j, j < 4, of head
  // hrow(nt)), scaled by the token scales (fp8), masked beyond the `valid` cached tokens, and
  // each head's max over the tile.
  auto mask = [&](int valid, f32x4_t (&v)[2]) {
    const int lim = valid - 16 * mt_w - 4 * g;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float x = s[nt][0][j] + s[nt][1][j];
        if constexpr (FP8) x *= tsc[j];
        v[nt][j] = j < lim ? x : -INFINITY;
      }
  };
  auto tile = [&](int valid, f32x4_t (&v)[2], float (&mx)[2]) {
    mask(valid, v);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      mx[nt] = max_across_rows(fmaxf(fmaxf(v[nt][0], v[nt][1]), fmaxf(v[nt][2], v[nt][3])));
  };
  // Whether some score of the tile exceeds its head's reference by more than kSlack.
  auto beyond = [&](const f32x4_t (&v)[2]) {
    bool r = false;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) r |= v[nt][j] > m_ref[nt] + kSlack;
    return r;
  };
  // p = 2^(s - m) against the reference (an empty split keeps m = -inf and uses 0: its masked
  // scores still give p = 0), packed to bf16 for the value product (fp8: p s_t); l accumulates
  // the fp32 p.
  auto weigh = [&](const f32x4_t (&v)[2], uint2 (&pk)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float m_use = m_ref[nt] == -INFINITY ? 0.f : m_ref[nt];
      float p[4], psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = __builtin_amdgcn_exp2f(v[nt][j] - m_use);   // 0 for masked tokens
        psum += p[j];
      }
      l_run[nt] += psum;
      if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] *= tsc[j];
      }
      pk[nt] = make_uint2(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]));
    }
  };
  auto store_p = [&](char* pb, const uint2 (&pk)[2]) {
    const int c = 2 * mt_w + (g >> 1);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int h = hrow(nt);
      *reinterpret_cast<uint2*>(pb + h * 64 + 16 * (c ^ psw(h)) + 8 * (g & 1)) = pk[nt];
    }
  };
  // Score tile of one stage: each K-tile fragment feeds both head tiles; K steps alternate
  // between two accumulators per head tile (four independent MFMA chains); fragments are read
  // kScoreRing - 1 K steps ahead of use (fp8: 16-byte reads two K-step pairs ahead).
  auto scores = [&](const char* st) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int q = 0; q < 2; ++q) s[nt][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (!s_live) return;                                  // head half past H: scores stay 0
    if constexpr (FP8) {
      tsc = *reinterpret_cast<const f32x4_t*>(st + Gm::kScaleOff + 4 * (16 * mt_w + 4 * g));
      // Reads m = 0 .. 7 pair up into the A operands of the four latent blocks (read 2 kb, then
      // 2 kb + 1); read 8 is the RoPE part.  Reads run two ahead of use.
      constexpr int kR = 4, kL = 2, kM = kKS / 2;
      uint4 raw[kR];
#pragma unroll
      for (int j = 0; j < kL; ++j) raw[j] = score_raw(st, j);
#pragma unroll
      for (int m = 0; m < kM; ++m) {
        const int mn = m + kL;
        if (mn < kM) raw[mn % kR] = score_raw(st, mn);
        if (m < kM - 1) {                                 // latent: scaled fp8 products, hi and lo
          if (m & 1) {
            const uint4 r0 = raw[(m - 1) % kR], r1 = raw[m % kR];
            const v8i_t a = {int(r0.x), int(r0.y), int(r0.z), int(r0.w), int(r1.x), int(r1.y), int(r1.z), int(r1.w)};
            const int kb = m >> 1;
#pragma unroll
            for (int nt = 0; nt < kSNT; ++nt)
              s[nt][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qc[nt][kb][0], s[nt][0], 0, 0, 0, 127, 0, qsh[nt]);
#pragma unroll
            for (int nt = 0; nt < kSNT; ++nt)
              s[nt][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, qc[nt][kb][1], s[nt][1], 0, 0, 0, 127, 0, qsl[nt]);
          }
        } else {                                          // RoPE part: fp16 products
          const uint4 r = raw[m % kR];
          const f16x8_t a0 = fp8x8_to_f16(r.x, r.y), a1 = fp8x8_to_f16(r.z, r.w);
#pragma unroll
          for (int nt = 0; nt < kSNT; ++nt)
            s[nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qr[nt][0], s[nt][0], 0, 0, 0);
#pragma unroll
          for (int nt = 0; nt < kSNT; ++nt)
            s[nt][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qr[nt][1], s[nt][1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      return;
    }
    bf16x8_t a[kScoreRing];
#pragma unroll
    for (int j = 0; j < kScoreRing - 1; ++j) a[j] = score_a(st, j);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      const int kn = ks + kScoreRing - 1;
      if (kn < kKS) a[kn % kScoreRing] = score_a(st, kn);
      if (ks < kDC / 32) {                       // latent: bf16 products
#pragma unroll
        for (int nt = 0; nt < kSNT; ++nt)
          s[nt][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks % kScoreRing], qf[nt][ks], s[nt][ks & 1], 0, 0, 0);
      } else {                                   // RoPE part: the key converted to fp16, fp16 products
        const f16x8_t ah = bf16x8_to_f16(a[ks % kScoreRing]);
#pragma unroll
        for (int nt = 0; nt < kSNT; ++nt)
          s[nt][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(f16x8_t, qf[nt][ks]), s[nt][ks & 1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);        // keep the source order: reads stay ahead of use
    }
  };
  // Value product of one stage (value waves).
  auto values = [&](const char* st, const char* pb) {
    bf16x8_t pf[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < kVNT; ++nt) pf[ks][nt] = p_frag(pb, ks, nt);
    if constexpr (FP8) {                                 // codes read four steps ahead, converted one ahead
      v2i_t raw[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) raw[u] = val_raw(st, u >> 2, u & 3);
      bf16x8_t av[2];
      av[0] = fp8x8_to_bf16(uint32_t(raw[0][0]), uint32_t(raw[0][1]));
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u + 4 < 8) raw[u + 4] = val_raw(st, (u + 4) >> 2, (u + 4) & 3);
        if (u + 1 < 8) av[(u + 1) & 1] = fp8x8_to_bf16(uint32_t(raw[u + 1][0]), uint32_t(raw[u + 1][1]));
        const int ks = u >> 2, ct = u & 3;
#pragma unroll
        for (int nt = 0; nt < kVNT; ++nt)
          o[ct][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u & 1], pf[ks][nt], o[ct][nt], 0, 0, 0);
      }
      return;
    }
    bf16x8_t av[2];
    av[0] = val_a(st, 0, 0);
#pragma unroll
    for (int u = 0; u < 8; ++u) {                        // (K step u >> 2, column tile u & 3)
      if (u + 1 < 8) av[(u + 1) & 1] = val_a(st, (u + 1) >> 2, (u + 1) & 3);
      const int ks = u >> 2, ct = u & 3;
#pragma unroll
      for (int nt = 0; nt < kVNT; ++nt)
        o[ct][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[u & 1], pf[ks][nt], o[ct][nt], 0, 0, 0);
    }
  };

  // The two roles run separate code (so their registers overlap) with the same sequence of
  // work-group barriers.  Pass structure: an accumulating pass against the first stage's max;
  // if any score outgrew its reference by kSlack, a scores-only pass for the exact maxima and an
  // accumulating pass against them.  Stage j's P lives in P buffer j % 2; stage j in ring slot
  // j % kRing.
  int* flags = reinterpret_cast<int*>(pbase);
  // Every wave calls this at the end of a pass; score waves also add their partner's row sums.
  auto restart_needed = [&](bool over, float (&lsum)[2]) {
    if (scorer) {
      const bool any_over = __any(over);
      if (lane == 0) flags[wave] = any_over ? 1 : 0;
      if (g == 0) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) lx[2 * hrow(nt) + mt_w] = lsum[nt];
      }
    }
    lds_barrier();
    const int4 f = *reinterpret_cast<const int4*>(flags);
    if (scorer) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) lsum[nt] += lx[2 * hrow(nt) + (mt_w ^ 1)];
    }
    lds_barrier();
    return (f.x | f.y | f.z | f.w) != 0;
  };
  if (scorer) {
    // The score waves carry each stage's serial chain (operand reads, products, softmax, P), the
    // value waves' products fill the matrix core around it: give the score waves issue priority.
    __builtin_amdgcn_s_setprio(1);
    // One accumulating pass.  At stage 0 the two waves of a head half agree on the reference:
    // the stage's max (checked pass) or the maxima the scores-only pass found (fixed pass).
    auto accumulate = [&](auto mode) {
      constexpr int kMode = decltype(mode)::value;
      bool over = false;
      l_run[0] = l_run[1] = 0.f;
      lds_barrier();                            // stage 0 loaded
      {
        f32x4_t v[2];
        float mx[2], mine[2];
        uint2 pk[2];
        scores(ring);
        tile(stage_valid(0), v, mx);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          mine[nt] = kMode == kChecked ? mx[nt] : m_ref[nt];
          if (g == 0) xm[2 * hrow(nt) + mt_w] = mine[nt];
        }
        lds_barrier();                          // maxima exchanged
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) m_ref[nt] = fmaxf(mine[nt], xm[2 * hrow(nt) + (mt_w ^ 1)]);
        weigh(v, pk);
        store_p(pbase, pk);
      }
      lds_barrier();                            // P(0) published, stage 1 loaded
      for (int i = 0; i < n; ++i) {
        if (i + 1 < n) {
          f32x4_t v[2];
          uint2 pk[2];
          scores(slot(i + 1));
          mask(stage_valid(i + 1), v);
          if (kMode == kChecked) over |= beyond(v);
          weigh(v, pk);
          store_p(pbase + ((i + 1) & 1) * kPBytes, pk);
        }
        lds_barrier();
      }
      return over;
    };
    float lsum[2];
    auto totals = [&]() {
      lsum[0] = sum_across_rows(l_run[0]);
      lsum[1] = sum_across_rows(l_run[1]);
    };
    const bool over = accumulate(std::integral_constant<int, kChecked>());
    totals();
    if (restart_needed(over, lsum)) {
      m_ref[0] = m_ref[1] = -INFINITY;
      lds_barrier();                            // stage 0 loaded
      for (int i = 0; i < n; ++i) {
        f32x4_t v[2];
        float mx[2];
        scores(slot(i));
        tile(stage_valid(i), v, mx);
        m_ref[0] = fmaxf(m_ref[0], mx[0]);
        m_ref[1] = fmaxf(m_ref[1], mx[1]);
        lds_barrier();
      }
      accumulate(std::integral_constant<int, kFixed>());
      totals();
      restart_needed(false, lsum);
    }
    // Row sums to the value waves, their per-head maxima |O| back (the ring is idle now).
    if (mt_w == 0 && g == 0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) xl[hrow(nt)] = lsum[nt];
    }
    lds_barrier();
    if (mt_w == 0 && g == 0) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int h = hrow(nt);
        if (hbase + h >= H) continue;
        const float a = fmaxf(fmaxf(xa[h], xa[kHeads + h]), fmaxf(xa[2 * kHeads + h], xa[3 * kHeads + h]));
        const int k = part_scale(a, lsum[nt]);
        const long row = (long(b) * splits + sp) * H + hbase + h;
        part_ml[row * 2] = m_ref[nt] - float(k);
        part_ml[row * 2 + 1] = lsum[nt] * ldexpf(1.f, k);
      }
    }
  } else {
    auto accumulate = [&]() {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[ct][nt][e] = 0.f;
      for (int j = 0; j < kRing - 1; ++j) issue(j);
      wait_stage(0, kRing - 2);
      lds_barrier();                            // stage 0 loaded
      lds_barrier();                            // (score waves exchange maxima)
      wait_stage(1, kRing - 2);
      lds_barrier();
      for (int i = 0; i < n; ++i) {
        issue(i + kRing - 1);                   // into the slot of stage i - 1, free since the last barrier
        values(slot(i), pbase + (i & 1) * kPBytes);
        wait_stage(i + 2, i + kRing - 1);
        lds_barrier();
      }
      return false;
    };
    float unused[2] = {0.f, 0.f};
    if (restart_needed(accumulate(), unused)) {
      for (int j = 0; j < kRing - 1; ++j) issue(j);
      wait_stage(0, kRing - 2);
      lds_barrier();
      for (int i = 0; i < n; ++i) {
        issue(i + kRing - 1);
        wait_stage(i + 1, i + kRing - 1);
        lds_barrier();
      }
      restart_needed(accumulate(), unused);
    }
    // Each head's largest |O| over this wave's 128 columns (the lane and lane ^ 32 hold them).
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float a = 0.f;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e) a = fmaxf(a, fabsf(o[ct][nt][e]));
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
      a = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      if (lane < 32) xa[wave * kHeads + 32 * nt + ph] = a;
    }
    lds_barrier();
    const long row0 = (long(b) * splits + sp) * H + hbase;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int h = 32 * nt + ph;
      if (hbase + h >= H) continue;
      const float a = fmaxf(fmaxf(xa[h], xa[kHeads + h]), fmaxf(xa[2 * kHeads + h], xa[3 * kHeads + h]));
      const float sc = ldexpf(1.f, part_scale(a, xl[h]));
      uint16_t* dst = part_o + (row0 + h) * kDC + 128 * wave + 4 * (lane >> 5);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q)             // 2^k O in fp16 (the merge reads half the bytes)
          *reinterpret_cast<uint2*>(dst + 32 * ct + 8 * q) =
              make_uint2(pack_h2(sc * o[ct][nt][4 * q], sc * o[ct][nt][4 * q + 1]),
                         pack_h2(sc * o[ct][nt][4 * q + 2], sc * o[ct][nt][4 * q + 3]));
    }
  }
}

// Sequences ranked by context length, longest first, ties by index: order[rank] = sequence.
__global__ __launch_bounds__(1024) void seq_order_kernel(int B, const int32_t* __restrict__ ctx,
                                                         int32_t* __restrict__ order) {
  __shared__ int32_t len[kOrderMax];
  for (int i = threadIdx.x; i < B; i += 1024) len[i] = ctx[i];
  __syncthreads();
  for (int t = threadIdx.x; t < B; t += 1024) {
    const int c = len[t];
    int r = 0;
    for (int u = 0; u < B; ++u) {
      const int cu = len[u];
      r += (cu > c || (cu == c && u < t)) ? 1 : 0;
    }
    order[r] = t;
  }
}

bool launch_decode_attn_v2(int cache_type, const DecodeAttnArgs& a, hipStream_t st) {
  if (a.H % 16 != 0 || a.dc != kDC || a.dr != kDR) return false;
  if (cache_type != K_BF16 && cache_type != K_FP8) return false;
  const int by_seq = a.B % 8 == 0 ? 1 : 0;
  const long nunits = long(a.B) * a.splits;
  const long G = (a.H + kHeads - 1) / kHeads;
  const long grid = by_seq ? nunits * G : (nunits + 7) / 8 * 8 * G;
  const int32_t* order = nullptr;
  if (a.order && a.B <= kOrderMax) {
    hipLaunchKernelGGL(seq_order_kernel, dim3(1), dim3(1024), 0, st, a.B, a.ctx, a.order);
    order = a.order;
  }
  // A layer of at most 32 heads fills one group partly: its instance skips the empty head tiles.
  auto pick = [&](auto fp8) {
    constexpr bool F = decltype(fp8)::value;
    return a.H <= 16 ? decode_attn_latent_kernel<F, 1>
         : a.H <= 32 ? decode_attn_latent_kernel<F, 2>
                     : decode_attn_latent_kernel<F, 4>;
  };
  const auto kern = cache_type == K_FP8 ? pick(std::true_type()) : pick(std::false_type());
  hipLaunchKernelGGL(kern, dim3(unsigned(grid)), dim3(kThreads), 0, st, a.H, a.splits, a.max_blocks, by_seq,
                     int(nunits), static_cast<const uint16_t*>(a.qhat), a.cache, a.cache_scale, a.block_table, a.ctx, order,
                     static_cast<uint16_t*>(a.part_o), a.part_ml);
  return true;
}

}  // namespace mla
