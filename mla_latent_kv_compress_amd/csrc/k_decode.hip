// Split-K decode attention over a bf16 latent cache, 128-head work-groups (weight-absorbed).
//
// One work-group per (sequence, split): 4 waves x 32 heads.  A work-group walks its split's
// 64-token pages; each page (64 rows x 576 bf16 = 72 KiB) is brought into LDS once by direct
// global->LDS loads (no staging registers), double-buffered so page p+1 streams in while page p
// is computed.  Per page and wave:
//   S^T[token][head] = R . Qhat^T     18 K-chunks x 4 token sub-tiles x 2 head tiles of
//                                     v_mfma_f32_16x16x32_bf16, R read with ds_read_b128
//   online softmax per head           base-2 (log2 e folded into Qhat), lazy rescale
//   O^T[c][head] += R^T . P^T         32 latent tiles x 2 token chunks x 2 head tiles,
//                                     R^T read with ds_read_b64_tr_b16
// The cached latent is also the value, so one LDS tile serves both products.
//
// LDS layout: rows of 72 16-byte chunks, unpadded (the direct loads fill 1 KiB runs), with the
// chunk index of row r XORed by swz(r) < 8.  This keeps a 16-row column of chunks (the score
// MFMA's A operand) and an 8-row x 32-byte block (the transpose read of 32 lanes) on distinct
// banks.
//
// Lazy rescale: each head keeps a reference max m and accumulates p = 2^(s - m).  m moves only
// when a page's max exceeds it by more than kSlack (then l and O are rescaled, exactly); p stays
// <= 2^kSlack, far inside bf16 and fp32 range.  The partial state (m, l, O) is consistent for the
// log-sum-exp merge whatever m is.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

namespace {

constexpr int kDC = 512, kDR = 64, kDW = kDC + kDR;
constexpr int kRowBytes = kDW * 2;                    // 1152
constexpr int kTileBytes = kPage * kRowBytes;         // 73728
constexpr int kChunks = kTileBytes / 16;              // 4608 16-byte chunks per page
constexpr int kKC = kDW / 32;                         // 18
constexpr int kCT = kDC / 16;                         // 32
constexpr float kSlack = 8.0f;

__device__ __forceinline__ int swz(int r) {
  r &= 15;
  return 2 * ((r >> 1) & 3) + ((r >> 3) & 1);
}

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ s16x4_t tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ bf16x8_t join(s16x4_t lo, s16x4_t hi) {
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  return uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
}

// Enqueue the direct loads of one page into `tile`: instruction k of wave w fills bytes
// [(w * per + k) * 1024, +1024) of the tile; lane i supplies physical chunk (w*per + k)*64 + i.
// Rows at or beyond `valid` re-read row valid-1 (finite data; their scores are masked).
// The lane id arrives opaque so the per-load offsets are recomputed here (a few integer ops)
// instead of being hoisted out of the page loop into registers.
template <int NW>
__device__ __forceinline__ void load_page(char* tile, const char* page, int valid, int wave, int lane) {
  constexpr int per = kChunks / 64 / NW;
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int k = 0; k < per; ++k) {
    const int pidx = (wave * per + k) * 64 + lane;
    const int r = pidx / 72, cp = pidx - r * 72;
    const int c = cp ^ swz(r);
    const int rs = r < valid ? r : valid - 1;
    const uint32_t off = uint32_t(rs * kRowBytes + c * 16);
    __builtin_amdgcn_global_load_lds(page + off, (lds_void*)(tile + (wave * per + k) * 1024), 16, 0, 0);
  }
}

}  // namespace

template <int NW, int HT>
__global__ __launch_bounds__(NW * 64, 1) void decode_attn_v2_kernel(
    int H, int B, int splits, int max_blocks, const uint16_t* __restrict__ qhat,
    const uint16_t* __restrict__ cache, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(1024))) char tile0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) char tile1[kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: keeps LDS offsets scalar
  const int g = lane >> 4, li = lane & 15;
  const int unit = blockIdx.x;                      // (sequence, split)
  const int b = unit / splits, sp = unit - b * splits;
  const int G = H / (NW * HT * 16);
  const int hg = blockIdx.y;
  const int h0 = (hg * NW + wave) * HT * 16;
  (void)G;
  const int ctx = ctx_lens[b];
  const int npages = (ctx + kPage - 1) / kPage;
  const int pps = (npages + splits - 1) / splits;
  const int p0 = sp * pps, p1 = min(npages, p0 + pps);
  const char* cbase = reinterpret_cast<const char*>(cache);
  const int32_t* btab = bt + long(b) * max_blocks;

  // Query fragments (B operand): lane holds Qhat[h0 + 16 ht + li][32 kc + 8 g .. +7].
  bf16x8_t qf[HT][kKC];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* q = qhat + (long(b) * H + h0 + 16 * ht + li) * kDW + 8 * g;
#pragma unroll
    for (int kc = 0; kc < kKC; ++kc) qf[ht][kc] = *reinterpret_cast<const bf16x8_t*>(q + 32 * kc);
  }
  f32x4_t o[HT][kCT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < kCT; ++i) o[ht][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_ref[HT], l_run[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m_ref[ht] = -INFINITY;
    l_run[ht] = 0.f;
  }

  // Per-lane LDS byte offsets (see the layout note above).
  // Score reads: row 16 st + li, logical chunk 4 kc + g -> ((4kc + g) ^ sw) = 4 (kc ^ xb) + xl.
  const int xs = g ^ swz(li);
  const int xl = xs & 3, xb = xs >> 2;
  const int s_even = li * kRowBytes + xl * 16 + xb * 64;     // kc even: + 64 kc
  const int s_odd = li * kRowBytes + xl * 16 - xb * 64;      // kc odd:  + 64 kc
  // Transpose reads: row 4 g + li/4 (+16, +32 q), element column 16 ct + 4 (li % 4):
  // chunk 2 ct + hh (hh = (li % 4) / 2), byte 8 (li % 2); (2ct + hh) ^ sw = 2 (ct ^ z) + (y & 1).
  const int tr_row = 4 * g + (li >> 2);
  const int y = ((li & 3) >> 1) ^ swz(tr_row);
  const int z = y >> 1;
  int t_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) t_base[j] = tr_row * kRowBytes + 32 * (j ^ z) + 16 * (y & 1) + 8 * (li & 1);

  auto compute = [&](const char* tile, int valid) {
    f32x4_t s[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
      for (int st = 0; st < 4; ++st) s[ht][st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < kKC; ++kc) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int off = ((kc & 1) ? s_odd : s_even) + 64 * kc + 16 * st * kRowBytes;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(tile + off);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          s[ht][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ht][kc], s[ht][st], 0, 0, 0);
      }
    }
    bf16x8_t pf[HT][2];
    // token 16 st + 4 g + r is cached iff 16 st + r < valid - 4 g (one per-lane limit)
    const int lim = valid - 4 * g;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = (16 * st + r) < lim ? s[ht][st][r] : -INFINITY;
          s[ht][st][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool move = mx > m_ref[ht] + kSlack;
      if (__any(move)) {
        const float m_new = move ? mx : m_ref[ht];
        const float alpha = exp2f(m_ref[ht] - m_new);          // 0 when m_ref = -inf
        l_run[ht] *= alpha;
#pragma unroll
        for (int i = 0; i < kCT; ++i) o[ht][i] *= alpha;
        m_ref[ht] = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = exp2f(s[ht][st][r] - m_ref[ht]);
          psum += pv;
          s[ht][st][r] = pv;
        }
      l_run[ht] += psum;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint4 w = make_uint4(pack_bf2(s[ht][2 * q][0], s[ht][2 * q][1]), pack_bf2(s[ht][2 * q][2], s[ht][2 * q][3]),
                                   pack_bf2(s[ht][2 * q + 1][0], s[ht][2 * q + 1][1]),
                                   pack_bf2(s[ht][2 * q + 1][2], s[ht][2 * q + 1][3]));
        pf[ht][q] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        const char* p = tile + t_base[ct & 3] + 32 * (ct & ~3) + 32 * q * kRowBytes;
        const bf16x8_t a = join(tr_read(p), tr_read(p + 16 * kRowBytes));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          o[ht][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[ht][q], o[ht][ct], 0, 0, 0);
      }
    }
  };

  auto page_ptr = [&](int p) { return cbase + long(btab[p]) * kTileBytes; };
  auto valid_of = [&](int p) { return min(kPage, ctx - p * kPage); };

  if (p0 < p1) load_page<NW>(tile0, page_ptr(p0), valid_of(p0), wave, lane);
  for (int p = p0; p < p1; p += 2) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (p + 1 < p1) load_page<NW>(tile1, page_ptr(p + 1), valid_of(p + 1), wave, lane);
    compute(tile0, valid_of(p));
    if (p + 1 < p1) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (p + 2 < p1) load_page<NW>(tile0, page_ptr(p + 2), valid_of(p + 2), wave, lane);
      compute(tile1, valid_of(p + 1));
    }
  }

#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    float l = l_run[ht];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const long row = (long(b) * splits + sp) * H + h0 + 16 * ht + li;
    if (g == 0) {
      part_ml[row * 2] = m_ref[ht];
      part_ml[row * 2 + 1] = l;
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct)
      *reinterpret_cast<f32x4_t*>(part_o + row * kDC + 16 * ct + 4 * g) = o[ht][ct];
  }
}

bool launch_decode_attn_v2(const DecodeAttnArgs& a, hipStream_t st) {
  if (a.H % 128 != 0 || a.dc != kDC || a.dr != kDR) return false;
  dim3 grid(unsigned(long(a.B) * a.splits), a.H / 128);     // 8 waves x 16 heads
  hipLaunchKernelGGL((decode_attn_v2_kernel<8, 1>), grid, dim3(512), 0, st, a.H, a.B, a.splits, a.max_blocks,
                     static_cast<const uint16_t*>(a.qhat), static_cast<const uint16_t*>(a.cache), a.block_table,
                     a.ctx, a.part_o, a.part_ml);
  return true;
}

}  // namespace mla
