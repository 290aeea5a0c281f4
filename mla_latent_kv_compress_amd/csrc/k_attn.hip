// Attention kernels: weight-absorbed split-K decode over the latent cache, and causal
// prefill over decompressed keys / values.
//
// MFMA layout used throughout (v_mfma_f32_16x16x32_bf16, wave64):
//   A [16 x 32]: lane l holds A[l%16][8(l/16) .. 8(l/16)+7]
//   B [32 x 16]: lane l holds B[8(l/16) .. +7][l%16]
//   C [16 x 16]: lane l holds C[4(l/16) .. +3][l%16]
// Scores are computed transposed, S^T[token][head] = R[token] . Q[head], so each lane owns one
// head (column l%16) and four tokens per 16-token sub-tile.  Taking two sub-tiles as the 32
// K values of the next MFMA (lane order k = 8g + j -> token 4g + j, then 16 + 4g + j - 4),
// the probabilities are already the B operand of O^T[c][head] += R^T[c][token] P^T[token][head],
// and the online-softmax rescale of O^T is a per-lane scalar.  R^T comes from the row-major
// LDS tile through ds_read_b64_tr_b16, which hands lane i of each 16-lane group one column of
// four consecutive rows.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ s16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4_t __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ bf16x8_t join_tr(s16x4_t lo, s16x4_t hi) {
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// bf16 pair (RNE) packed into a 32-bit word: low half = a.
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
}

// Four e4m3 codes (one 32-bit word) to four bf16 values (exact).
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, false);
  bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// ==================================================================== decode, bf16 MFMA
constexpr int kDC = 512, kDR = 64, kDW = kDC + kDR;   // latent, RoPE key, cached row width
constexpr int kLRow = kDW + 8;                        // LDS row stride (elements): 1168 bytes
constexpr int kKC = kDW / 32;                         // 18 K-chunks of the score MFMA
constexpr int kCT = kDC / 16;                         // 32 column tiles of the latent

// One work-group per (sequence, split, head group): NW waves of HT x 16 heads share each
// 64-token page tile in LDS.  The 1-D grid places the G head groups of one (sequence, split)
// eight work-groups apart, i.e. on the same XCD (work-groups go round-robin over the 8 XCDs)
// and dispatched together, so the second read of a page is served by that XCD's L2.
template <int NW, int HT, bool FP8>
__global__ __launch_bounds__(NW * 64) void decode_attn_mfma_kernel(
    int H, int G, int B, int splits, int max_blocks, const uint16_t* __restrict__ qhat,
    const void* __restrict__ cache, const float* __restrict__ cache_scale,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ ctx_lens,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kPage * kLRow];
  __shared__ float tscale[kPage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int L = blockIdx.x;
  const int unit = (L / (8 * G)) * 8 + (L & 7);     // (sequence, split) index
  const int hg = (L >> 3) % G;
  if (unit >= B * splits) return;
  const int b = unit / splits, sp = unit % splits;
  const int h0 = (hg * NW + wave) * HT * 16;
  const int ctx = ctx_lens[b];
  const int npages = (ctx + kPage - 1) / kPage;
  const int pps = (npages + splits - 1) / splits;
  const int p0 = sp * pps, p1 = min(npages, p0 + pps);

  bf16x8_t qf[HT][kKC];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* qrow = qhat + (long(b) * H + h0 + 16 * ht + li) * kDW + 8 * g;
#pragma unroll
    for (int kc = 0; kc < kKC; ++kc) qf[ht][kc] = *reinterpret_cast<const bf16x8_t*>(qrow + 32 * kc);
  }
  f32x4_t o[HT][kCT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < kCT; ++i) o[ht][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[HT], l_run[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
  }

  for (int p = p0; p < p1; ++p) {
    const long phys = bt[long(b) * max_blocks + p];
    const int valid = min(kPage, ctx - p * kPage);
    __syncthreads();
    if (!FP8) {
      const uint16_t* src = static_cast<const uint16_t*>(cache) + phys * kPage * kDW;
      for (int c = tid; c < kPage * (kDW / 8); c += NW * 64) {
        int r = c / (kDW / 8), col = (c % (kDW / 8)) * 8;
        uint4 v = r < valid ? *reinterpret_cast<const uint4*>(src + r * kDW + col) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&tile[r * kLRow + col]) = v;
      }
    } else {
      const uint8_t* src = static_cast<const uint8_t*>(cache) + phys * kPage * kDW;
      for (int c = tid; c < kPage * (kDW / 16); c += NW * 64) {
        int r = c / (kDW / 16), col = (c % (kDW / 16)) * 16;
        uint4 v = r < valid ? *reinterpret_cast<const uint4*>(src + r * kDW + col) : make_uint4(0, 0, 0, 0);
        uint2 a0 = fp8x4_to_bf16x4(v.x), a1 = fp8x4_to_bf16x4(v.y);
        uint2 a2 = fp8x4_to_bf16x4(v.z), a3 = fp8x4_to_bf16x4(v.w);
        *reinterpret_cast<uint4*>(&tile[r * kLRow + col]) = make_uint4(a0.x, a0.y, a1.x, a1.y);
        *reinterpret_cast<uint4*>(&tile[r * kLRow + col + 8]) = make_uint4(a2.x, a2.y, a3.x, a3.y);
      }
      if (tid < kPage) tscale[tid] = tid < valid ? cache_scale[phys * kPage + tid] : 0.f;
    }
    __syncthreads();

    // S^T sub-tiles: s[ht][st][r] = score of token 16 st + 4 g + r for head h0 + 16 ht + li.
    f32x4_t s[HT][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) s[ht][st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* arow = &tile[(16 * st + li) * kLRow + 8 * g];
#pragma unroll
      for (int kc = 0; kc < kKC; ++kc) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(arow + 32 * kc);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          s[ht][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ht][kc], s[ht][st], 0, 0, 0);
      }
    }
    bf16x8_t pf[HT][2];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * st + 4 * g + r;
          float v = s[ht][st][r];
          if (FP8) v *= tscale[t];
          v = t < valid ? v : -INFINITY;
          s[ht][st][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[ht], mx);
      const float alpha = exp2f(m_run[ht] - m_new);
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float pv = exp2f(s[ht][st][r] - m_new);
          psum += pv;
          if (FP8) pv *= tscale[16 * st + 4 * g + r];
          s[ht][st][r] = pv;
        }
      l_run[ht] = l_run[ht] * alpha + psum;
      m_run[ht] = m_new;
#pragma unroll
      for (int i = 0; i < kCT; ++i) o[ht][i] *= alpha;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint4 w = make_uint4(pack_bf2(s[ht][2 * q][0], s[ht][2 * q][1]), pack_bf2(s[ht][2 * q][2], s[ht][2 * q][3]),
                             pack_bf2(s[ht][2 * q + 1][0], s[ht][2 * q + 1][1]),
                             pack_bf2(s[ht][2 * q + 1][2], s[ht][2 * q + 1][3]));
        pf[ht][q] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    // O^T[c][h] += R^T[c][t] P^T[t][h]; lane (g, li) addresses row 4g + li/4 (+16), column 4(li%4).
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint16_t* base = &tile[(32 * q + 4 * g + (li >> 2)) * kLRow + 4 * (li & 3)];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        const bf16x8_t a = join_tr(lds_read_tr(base + 16 * ct), lds_read_tr(base + 16 * kLRow + 16 * ct));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          o[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[ht][q], o[ht][ct], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    float l = l_run[ht];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const long row = (long(b) * splits + sp) * H + h0 + 16 * ht + li;
    if (g == 0) {
      part_ml[row * 2] = m_run[ht];
      part_ml[row * 2 + 1] = l;
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
      *reinterpret_cast<f32x4_t*>(part_o + row * kDC + 16 * ct + 4 * g) = o[ht][ct];
  }
}

// ==================================================================== decode, fp32 SIMT
// Generic dims.  Grid (H, splits, B); 256 threads: one token per thread for the scores, one
// latent column per thread for the weighted sum.
__global__ __launch_bounds__(256) void decode_attn_simt_kernel(
    int H, int dc, int dr, int splits, int max_blocks, const float* __restrict__ qhat,
    const float* __restrict__ cache, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ part_o, float* __restrict__ part_ml) {
  extern __shared__ long shl[];                     // slot [256] | p [256] | q [W]
  __shared__ float red[16];
  const int W = dc + dr;
  long* sbuf = shl;
  float* pbuf = reinterpret_cast<float*>(shl + 256);
  float* q = pbuf + 256;
  const int h = blockIdx.x, sp = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int ctx = ctx_lens[b];
  const int npages = (ctx + kPage - 1) / kPage;
  const int pps = (npages + splits - 1) / splits;
  const int t0 = sp * pps * kPage, t1 = min(ctx, (sp + 1) * pps * kPage);
  for (int i = tid; i < W; i += 256) q[i] = qhat[(long(b) * H + h) * W + i];
  constexpr int KO = 16;                            // dc <= 4096
  float o[KO];
#pragma unroll
  for (int k = 0; k < KO; ++k) o[k] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();
  for (int tb = t0; tb < t1; tb += 256) {
    const int t = tb + tid;
    float sc = -INFINITY;
    long slot = 0;
    if (t < t1) {
      slot = long(bt[long(b) * max_blocks + t / kPage]) * kPage + t % kPage;
      const float* rw = cache + slot * W;
      float acc = 0.f;
      for (int k = 0; k < W; ++k) acc = fmaf(q[k], rw[k], acc);
      sc = acc;
    }
    const float mx = block_max(sc, red);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    const float pv = t < t1 ? exp2f(sc - m_new) : 0.f;
    const float ps = block_sum(pv, red);
    pbuf[tid] = pv;
    sbuf[tid] = slot;
    __syncthreads();
    l_run = l_run * alpha + ps;
    m_run = m_new;
    const int n = min(256, t1 - tb);
#pragma unroll
    for (int k = 0; k < KO; ++k) {
      const int c = tid + 256 * k;
      if (c < dc) {
        float acc = o[k] * alpha;
        for (int j = 0; j < n; ++j) acc = fmaf(pbuf[j], cache[sbuf[j] * W + c], acc);
        o[k] = acc;
      }
    }
    __syncthreads();
  }
  const long row = (long(b) * splits + sp) * H + h;
  if (tid == 0) {
    part_ml[row * 2] = m_run;
    part_ml[row * 2 + 1] = l_run;
  }
#pragma unroll
  for (int k = 0; k < KO; ++k) {
    const int c = tid + 256 * k;
    if (c < dc) part_o[row * dc + c] = o[k];
  }
}

void launch_decode_attn(int act, int cache, const DecodeAttnArgs& a, hipStream_t st) {
  if (act == K_F32) {
    size_t sh = size_t(a.dc + a.dr + 256) * sizeof(float) + 256 * sizeof(long);
    hipLaunchKernelGGL(decode_attn_simt_kernel, dim3(a.H, a.splits, a.B), dim3(256), sh, st, a.H, a.dc,
                       a.dr, a.splits, a.max_blocks, static_cast<const float*>(a.qhat),
                       static_cast<const float*>(a.cache), a.block_table, a.ctx, a.part_o, a.part_ml);
    return;
  }
  if (a.heads_per_group == 64 && launch_decode_attn_v2(cache, a, st)) return;
  // heads_per_group = NW * 16: 64 -> 4 waves, 32 -> 2 waves, 16 -> 1 wave.
  const int G = a.H / a.heads_per_group;
  const long units = (long(a.B) * a.splits + 7) / 8 * 8;
  dim3 grid(unsigned(units * G));
#define MLA_DA(NW, HT, F8)                                                                                  \
  hipLaunchKernelGGL((decode_attn_mfma_kernel<NW, HT, F8>), grid, dim3(NW * 64), 0, st, a.H, G, a.B,        \
                     a.splits, a.max_blocks, static_cast<const uint16_t*>(a.qhat), a.cache, a.cache_scale,  \
                     a.block_table, a.ctx, a.part_o, a.part_ml)
#define MLA_DA_NW(F8)                              \
  switch (a.heads_per_group) {                     \
    case 64: MLA_DA(4, 1, F8); break;              \
    case 32: MLA_DA(2, 1, F8); break;              \
    default: MLA_DA(1, 1, F8); break;              \
  }
  if (cache == K_FP8) {
    MLA_DA_NW(true)
  } else {
    MLA_DA_NW(false)
  }
#undef MLA_DA_NW
#undef MLA_DA
}

// ==================================================================== prefill, fp16 MFMA
// Head dims fixed at nope 128, rope 64, v 128.  Grid (query tiles of 64, H, S); 4 waves of 16
// queries.  Keys t of sequence s: [k_nope from kv | k_pe from lat], values from kv.  Queries,
// keys, values and probabilities are fp16 (v_mfma_f32_16x16x32_f16); k_pe arrives as bf16
// cache values and is converted while it is staged in LDS.
constexpr int kPN = 128, kPR = 64, kPV = 128, kPQK = kPN + kPR;
constexpr int kKRow = kPQK + 8, kVRow = kPV + 8;

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return uint32_t(f2h(a)) | (uint32_t(f2h(b)) << 16);
}

template <int OUT>
__global__ __launch_bounds__(256) void prefill_attn_mfma_kernel(
    int H, int max_ctx, const int32_t* __restrict__ cu, const int32_t* __restrict__ start,
    const uint16_t* __restrict__ qs, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ lat,
    typename StoreT<OUT>::type* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kPage * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kPage * kVRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int qt = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int q_begin = cu[s], len = cu[s + 1] - q_begin, st0 = start[s];
  if (qt * 64 >= len) return;                       // whole work-group leaves together
  const int ctx = st0 + len;
  const int qi = qt * 64 + wave * 16 + li;          // this lane's query (column of S^T)
  const int qpos = st0 + min(qi, len - 1);
  const int kv_w = H * (kPN + kPV);
  const int lat_w = kDW;

  f16x8_t qf[kPQK / 32];
  {
    const uint16_t* qrow = qs + (long(q_begin + min(qi, len - 1)) * H + h) * kPQK + 8 * g;
#pragma unroll
    for (int kc = 0; kc < kPQK / 32; ++kc) qf[kc] = *reinterpret_cast<const f16x8_t*>(qrow + 32 * kc);
  }
  f32x4_t o[kPV / 16];
#pragma unroll
  for (int i = 0; i < kPV / 16; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const int key_end = min(ctx, st0 + min(len, qt * 64 + 64));
  const long kv_base = long(s) * max_ctx;

  for (int t0 = 0; t0 < key_end; t0 += kPage) {
    __syncthreads();
    // K rows: 16 chunks of k_nope + 8 chunks of k_pe; V rows: 16 chunks.
    for (int c = tid; c < kPage * 40; c += 256) {
      const int r = c / 40, j = c % 40, t = t0 + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < 16) {
        if (t < ctx) v = *reinterpret_cast<const uint4*>(kv + (kv_base + t) * kv_w + h * (kPN + kPV) + 8 * j);
        *reinterpret_cast<uint4*>(&ks[r * kKRow + 8 * j]) = v;
      } else if (j < 24) {
        if (t < ctx) {
          uint4 b = *reinterpret_cast<const uint4*>(lat + (kv_base + t) * lat_w + kDC + 8 * (j - 16));
          const uint16_t* e = reinterpret_cast<const uint16_t*>(&b);
          v = make_uint4(pack_h2(bf2f(e[0]), bf2f(e[1])), pack_h2(bf2f(e[2]), bf2f(e[3])),
                         pack_h2(bf2f(e[4]), bf2f(e[5])), pack_h2(bf2f(e[6]), bf2f(e[7])));
        }
        *reinterpret_cast<uint4*>(&ks[r * kKRow + kPN + 8 * (j - 16)]) = v;
      } else {
        if (t < ctx) v = *reinterpret_cast<const uint4*>(kv + (kv_base + t) * kv_w + h * (kPN + kPV) + kPN + 8 * (j - 24));
        *reinterpret_cast<uint4*>(&vs[r * kVRow + 8 * (j - 24)]) = v;
      }
    }
    __syncthreads();
    f32x4_t sc[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      sc[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* arow = &ks[(16 * st + li) * kKRow + 8 * g];
#pragma unroll
      for (int kc = 0; kc < kPQK / 32; ++kc)
        sc[st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            *reinterpret_cast<const f16x8_t*>(arow + 32 * kc), qf[kc], sc[st], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * st + 4 * g + r;
        float v = (t <= qpos && t < ctx) ? sc[st][r] : -INFINITY;
        sc[st][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    // Tile 0 holds key 0 <= every query's position, so m_new is finite from the first tile on;
    // a later tile entirely in a query's future leaves its state unchanged (alpha 1, p 0).
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float pv = m_new == -INFINITY ? 0.f : exp2f(sc[st][r] - m_new);
        psum += pv;
        sc[st][r] = pv;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < kPV / 16; ++i) o[i] *= alpha;
    f16x8_t pf[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 w = make_uint4(pack_h2(sc[2 * q][0], sc[2 * q][1]), pack_h2(sc[2 * q][2], sc[2 * q][3]),
                           pack_h2(sc[2 * q + 1][0], sc[2 * q + 1][1]), pack_h2(sc[2 * q + 1][2], sc[2 * q + 1][3]));
      pf[q] = __builtin_bit_cast(f16x8_t, w);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint16_t* base = &vs[(32 * q + 4 * g + (li >> 2)) * kVRow + 4 * (li & 3)];
#pragma unroll
      for (int vt = 0; vt < kPV / 16; ++vt) {
        const f16x8_t a = __builtin_bit_cast(f16x8_t, join_tr(lds_read_tr(base + 16 * vt),
                                                              lds_read_tr(base + 16 * kVRow + 16 * vt)));
        o[vt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf[q], o[vt], 0, 0, 0);
      }
    }
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (qi < len) {
    const float inv = 1.0f / l_run;
    const long row = (long(q_begin + qi) * H + h) * kPV + 4 * g;
#pragma unroll
    for (int vt = 0; vt < kPV / 16; ++vt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sts_<OUT>(out, row + 16 * vt + r, o[vt][r] * inv);
  }
}

// ==================================================================== prefill, fp32 SIMT
// Generic dims.  Grid (max_q, H, S); one query per block, 256 threads over keys.
__global__ __launch_bounds__(256) void prefill_attn_simt_kernel(
    int H, int dn, int dr, int dv, int dc, int max_ctx, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ start, const float* __restrict__ qs, const float* __restrict__ kv,
    const float* __restrict__ lat, float* __restrict__ out) {
  extern __shared__ float sh[];                     // q [dn+dr] | p [256]
  __shared__ float red[16];
  const int i = blockIdx.x, h = blockIdx.y, s = blockIdx.z, tid = threadIdx.x;
  const int q_begin = cu[s], len = cu[s + 1] - q_begin;
  if (i >= len) return;
  const int dqk = dn + dr, dkv = dn + dv, W = dc + dr;
  const int qpos = start[s] + i;
  float* q = sh;
  float* pbuf = sh + dqk;
  for (int k = tid; k < dqk; k += 256) q[k] = qs[(long(q_begin + i) * H + h) * dqk + k];
  __syncthreads();
  const long kvb = long(s) * max_ctx;
  constexpr int KO = 16;                            // dv <= 4096
  float o[KO];
#pragma unroll
  for (int k = 0; k < KO; ++k) o[k] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int tb = 0; tb <= qpos; tb += 256) {
    const int t = tb + tid;
    float sc = -INFINITY;
    if (t <= qpos) {
      const float* kr = kv + ((kvb + t) * H + h) * dkv;
      const float* pr = lat + (kvb + t) * W + dc;
      float acc = 0.f;
      for (int k = 0; k < dn; ++k) acc = fmaf(q[k], kr[k], acc);
      for (int k = 0; k < dr; ++k) acc = fmaf(q[dn + k], pr[k], acc);
      sc = acc;
    }
    const float mx = block_max(sc, red);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    const float pv = t <= qpos ? exp2f(sc - m_new) : 0.f;
    const float ps = block_sum(pv, red);
    pbuf[tid] = pv;
    __syncthreads();
    l_run = l_run * alpha + ps;
    m_run = m_new;
    const int n = min(256, qpos + 1 - tb);
#pragma unroll
    for (int k = 0; k < KO; ++k) {
      const int c = tid + 256 * k;
      if (c < dv) {
        float acc = o[k] * alpha;
        for (int j = 0; j < n; ++j) acc = fmaf(pbuf[j], kv[((kvb + tb + j) * H + h) * dkv + dn + c], acc);
        o[k] = acc;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < KO; ++k) {
    const int c = tid + 256 * k;
    if (c < dv) out[(long(q_begin + i) * H + h) * dv + c] = o[k] / l_run;
  }
}

void launch_prefill_attn(int act, const PrefillAttnArgs& a, hipStream_t st) {
  if (act == K_F32) {
    size_t sh = size_t(a.dn + a.dr + 256) * sizeof(float);
    hipLaunchKernelGGL(prefill_attn_simt_kernel, dim3(a.max_q, a.H, a.S), dim3(256), sh, st, a.H, a.dn,
                       a.dr, a.dv, a.dc, a.max_ctx, a.cu, a.start, static_cast<const float*>(a.qs),
                       static_cast<const float*>(a.kv), static_cast<const float*>(a.lat),
                       static_cast<float*>(a.out));
    return;
  }
  if (launch_prefill_attn_fa(a, st)) return;
  dim3 grid((a.max_q + 63) / 64, a.H, a.S);
  if (a.out_type == K_BF16)
    hipLaunchKernelGGL(prefill_attn_mfma_kernel<S_BF16>, grid, dim3(256), 0, st, a.H, a.max_ctx, a.cu, a.start,
                       static_cast<const uint16_t*>(a.qs), static_cast<const uint16_t*>(a.kv),
                       static_cast<const uint16_t*>(a.lat), static_cast<uint16_t*>(a.out));
  else
    hipLaunchKernelGGL(prefill_attn_mfma_kernel<S_F32>, grid, dim3(256), 0, st, a.H, a.max_ctx, a.cu, a.start,
                       static_cast<const uint16_t*>(a.qs), static_cast<const uint16_t*>(a.kv),
                       static_cast<const uint16_t*>(a.lat), static_cast<float*>(a.out));
}

}  // namespace mla
