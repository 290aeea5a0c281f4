// GEMMs of the MLA projections.
//   Y[z] = alpha * X[z] (M x K, row-major, lda) * op(W[z])
//   TN: W is [N][K] (linear-layer layout, K contiguous)    NN: W is [K][N] (N contiguous)
// z indexes (batch, K-split): slice `sp` of the K range writes its own partial output at
// Y + sp * ssplit, which the consumer sums in a fixed order (deterministic, no atomics).
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

// ------------------------------------------------------------------ bf16 MFMA GEMM
// 256 threads = 4 waves in a 2 x 2 arrangement; each wave owns a (BM/2) x (BN/2) block of
// 16 x 16 MFMA tiles (v_mfma_f32_16x16x32_bf16, fp32 accumulate).  Tiles of A and B are
// staged through LDS with K contiguous per row, so every MFMA operand is one 16-byte LDS
// read.  The next K step is prefetched into registers while the current one computes.
template <int BM, int BN, int BK, bool NN, int OUT>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(
    int M, int N, int K, int kchunk, const uint16_t* __restrict__ X, long lda, long sx,
    const uint16_t* __restrict__ W, long ldw, long sw, typename StoreT<OUT>::type* __restrict__ Y,
    long ldc, long sy, long ssplit, float alpha, int nsplit) {
  constexpr int LDK = BK + 8;                       // padded row: 16-lane reads hit distinct banks
  constexpr int TM = BM / 32, TN = BN / 32;         // MFMA tiles per wave
  constexpr int A_CH = BM * BK / 8 / 256;           // 16-byte chunks per thread
  constexpr int B_CH = BN * BK / 8 / 256;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small for 256 threads");
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int b = blockIdx.z / nsplit, sp = blockIdx.z % nsplit;
  X += b * sx;
  W += b * sw;
  Y += b * sy + sp * ssplit;
  const int k0 = sp * kchunk;
  const int k1 = min(K, k0 + kchunk);
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  uint4 ra[A_CH], rb[B_CH];
  auto load = [&](int k) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + i * 256, row = c / (BK / 8), kq = (c % (BK / 8)) * 8;
      int gm = m0 + row, gk = k + kq;
      ra[i] = (gm < M && gk < k1) ? *reinterpret_cast<const uint4*>(X + gm * lda + gk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + i * 256;
      if (!NN) {
        int row = c / (BK / 8), kq = (c % (BK / 8)) * 8;
        int gn = n0 + row, gk = k + kq;
        rb[i] = (gn < N && gk < k1) ? *reinterpret_cast<const uint4*>(W + gn * ldw + gk) : make_uint4(0, 0, 0, 0);
      } else {
        int krow = c / (BN / 8), nq = (c % (BN / 8)) * 8;
        int gk = k + krow, gn = n0 + nq;
        rb[i] = (gn < N && gk < k1) ? *reinterpret_cast<const uint4*>(W + long(gk) * ldw + gn) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      int c = tid + i * 256, row = c / (BK / 8), kq = (c % (BK / 8)) * 8;
      *reinterpret_cast<uint4*>(&As[row * LDK + kq]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      int c = tid + i * 256;
      if (!NN) {
        int row = c / (BK / 8), kq = (c % (BK / 8)) * 8;
        *reinterpret_cast<uint4*>(&Bs[row * LDK + kq]) = rb[i];
      } else {                                      // transpose into [n][k]
        int krow = c / (BN / 8), nq = (c % (BN / 8)) * 8;
        const uint16_t* v = reinterpret_cast<const uint16_t*>(&rb[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) Bs[(nq + j) * LDK + krow] = v[j];
      }
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (k0 < k1) load(k0);
  for (int k = k0; k < k1; k += BK) {
    __syncthreads();
    store();
    __syncthreads();
    if (k + BK < k1) load(k + BK);
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * (BM / 2) + i * 16 + (lane & 15)) * LDK + kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[(wn * (BN / 2) + j * 16 + (lane & 15)) * LDK + kk + 8 * (lane >> 4)]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // C layout: lane holds C[4*(lane/16) + r][lane%16] of each 16 x 16 tile.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int gn = n0 + wn * (BN / 2) + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int gm = m0 + wm * (BM / 2) + i * 16 + 4 * (lane >> 4) + r;
        if (gm < M && gn < N) sts_<OUT>(Y, long(gm) * ldc + gn, alpha * acc[i][j][r]);
      }
    }
}

// ------------------------------------------------------------------ fp32 SIMT GEMM
// 16 x 16 threads, each computing a 4 x 4 block of a 64 x 64 output tile; K in steps of 16.
template <bool NN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    int M, int N, int K, int kchunk, const float* __restrict__ X, long lda, long sx,
    const float* __restrict__ W, long ldw, long sw, float* __restrict__ Y, long ldc, long sy,
    long ssplit, float alpha, int nsplit) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int b = blockIdx.z / nsplit, sp = blockIdx.z % nsplit;
  X += b * sx;
  W += b * sw;
  Y += b * sy + sp * ssplit;
  const int k0 = sp * kchunk, k1 = min(K, k0 + kchunk);
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k = k0; k < k1; k += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      int kk = e & 15, mm = e >> 4;
      int gm = m0 + mm, gk = k + kk;
      As[kk][mm] = (gm < M && gk < k1) ? X[long(gm) * lda + gk] : 0.f;
      int gn = n0 + mm;
      float wv = 0.f;
      if (gn < N && gk < k1) wv = NN ? W[long(gk) * ldw + gn] : W[long(gn) * ldw + gk];
      Bs[kk][mm] = wv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int gm = m0 + ty * 4 + i, gn = n0 + tx * 4 + j;
      if (gm < M && gn < N) Y[long(gm) * ldc + gn] = alpha * acc[i][j];
    }
}

// ------------------------------------------------------------------ skinny bf16 GEMM (M <= 128)
// Y = alpha X W^T for M <= 128 rows (a decode batch): the weight stream is the whole cost, so
// each work-group owns 64 or 96 output columns and streams its [columns x K-chunk] slice of W
// (and the matching slice of X, an L2 hit) through a ring of LDS stages with direct
// global->LDS loads, several stages ahead of the MFMAs.  A stage is 64 k of X (MR = 64 or 128
// rows) and of W.  bf16 rows are 128 bytes with 16-byte chunk c of row r stored at
// c ^ ((r >> 1) & 7), so the 16 rows of an MFMA operand read fall on distinct banks.  With XF
// the activation X is a bf16 pair hi = bf16(x), lo = bf16(x - hi) laid side by side (row m: hi
// in columns [0, K), lo in [K, 2K)); a stage holds each row's 64-wide hi and lo slices as one
// 256-byte row (16 chunks: hi 0..7, lo 8..15; chunk c of row r at c ^ (r & 15)), and both enter
// the matrix core, two products per fragment, so the activation is carried to about 2^-16 of
// its value instead of bf16's 2^-9 (the pair is formed once, by the producer of X, not by every
// work-group that reads it).  Rows past M (or N)
// re-read the last valid row; their outputs are not stored.  Requires K and the K chunk to be
// multiples of 64.
namespace {
template <int BN, int MR, bool XF = false> constexpr int sk_stage_bytes() { return MR * (XF ? 256 : 128) + BN * 128; }
// Ring depth: 4 stages (16 to 40 KiB each), three stages of loads in flight; 3 when four stages
// would not fit the 160 KiB of LDS (the 128-row fp32 activation tile).  (Measured: a 7-stage
// ring for the one-per-CU 96-column tiles made the 236B-shaped q_b and kv_a + q_a projections
// slower, not faster.)
template <int BN, int MR = 64, bool XF = false> constexpr int sk_stages() {
  return 4 * sk_stage_bytes<BN, MR, XF>() <= 160 * 1024 ? 4 : 3;
}

__device__ __forceinline__ void sk_dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void sk_dma16nt(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t sk_lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}
template <int n>
__device__ __forceinline__ void sk_wait_vm() {
  __builtin_amdgcn_s_waitcnt(((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF));
}
__device__ __forceinline__ void sk_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace

// One skinny problem: Y[z / nsplit] (+ split z % nsplit) = alpha X W^T over the split's K chunk.
struct SkinnyProb {
  int M, N, K, kchunk, nsplit;
  const void* X;             // bf16, or a bf16 hi + lo pair (XF: row m = [hi (K) | lo (K)])
  long lda, sx;
  const uint16_t* W;
  long ldw, sw;
  void* Y;
  long ldc, sy, ssplit;
  float alpha;
  float* Y2;                 // (query-split output only) fp32 q_pe
};

// Output mode of the decode query projection (q_b, N = H x 192): columns 0..127 of each head
// (q_nope) are stored as fp32 alpha q to Y [M][H][128], which the absorb kernel feeds to the
// matrix core as a bf16 hi + lo pair, and columns 128..191 (q_pe) as fp32 q to Y2 [M][H][64],
// which the absorb kernel rotates.
constexpr int kOutQSplit = 7;

// Output tile (MR rows x BN columns from column tile nx) of batch-and-split index z.  BN is 64,
// 96 or 160, MR 64 or 128: a stage holds the X tile (MR rows x 64 k) and the W tile (BN rows x 64 k);
// whole KiBs of it are filled by one direct-load instruction each (8 bf16 rows of 128 bytes, or
// 4 fp32 rows of 256 bytes), dealt round-robin to the four waves; wave (wm, wn) computes rows
// MR / 2 wm .. + MR / 2 and columns BN / 2 wn .. + BN / 2.
template <int OUT, int BN, int MR, bool XF = false>
__device__ __forceinline__ void skinny_tile(const SkinnyProb& p, int nx, int z, int rank, char* ring) {
  constexpr int kStageB = sk_stage_bytes<BN, MR, XF>();
  constexpr int S = sk_stages<BN, MR, XF>();
  constexpr int XK = MR * (XF ? 256 : 128) / 1024;       // KiBs of the stage that hold X
  constexpr int NQ = (XK + BN / 8) / 4;                  // load instructions per wave per stage
  constexpr int NC = BN / 32;                            // 16-column tiles per wave
  constexpr int MT = MR / 32;                            // 16-row tiles per wave
  static_assert((XK + BN / 8) % 4 == 0, "whole instructions per wave");
  const int M = p.M, N = p.N, K = p.K, kchunk = p.kchunk, nsplit = p.nsplit;
  const long lda = p.lda, ldw = p.ldw, ldc = p.ldc;
  const float alpha = p.alpha;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int b = z / nsplit, sp = z % nsplit;
  const char* X = reinterpret_cast<const char*>(p.X) + b * p.sx * 2;
  const uint16_t* W = p.W + b * p.sw;
  typename StoreT<OUT>::type* Y = static_cast<typename StoreT<OUT>::type*>(p.Y) + b * p.sy + sp * p.ssplit;
  const int k0 = sp * kchunk;
  const int nk = (min(K, k0 + kchunk) - k0) / 64;      // 64-wide K steps of this split
  const int n0 = nx * BN;

  // Instruction q = wave + 4 j fills KiB q of the stage: q < XK are X rows (bf16: 8q .. +7, lane
  // i -> row + (i >> 3), stored chunk i & 7; fp32: 4q .. +3, lane i -> row + (i >> 4), stored
  // chunk i & 15), the rest W rows 8 (q - XK) .. +7 (lane i -> row + (i >> 3), stored chunk i & 7).
  uint32_t off[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    const int q = wave + 4 * j;
    if (q < XK) {
      if constexpr (XF) {
        const int r = 4 * q + (lane >> 4);
        const int c = (lane & 15) ^ (r & 15);           // hi chunks 0..7, lo chunks 8..15
        off[j] = uint32_t((long(min(r, M - 1)) * lda + (c < 8 ? 8 * c : K + 8 * (c - 8))) * 2);
      } else {
        const int r = 8 * q + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        off[j] = uint32_t((long(min(r, M - 1)) * lda + 8 * c) * 2);
      }
    } else {
      const int r = 8 * (q - XK) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      off[j] = uint32_t((long(min(n0 + r, N - 1)) * ldw + 8 * c) * 2);
    }
  }
  // The work-groups of one XCD that share a K chunk read the same X rows; each starts its K loop
  // at its own step (rot, from its rank among the XCD's work-groups: work-groups are dealt to
  // the 8 XCDs round-robin) so that they do not request the same L2 lines at the same time.
  const int rot = rank % max(nk, 1);
  auto issue = [&](int jj) {
    if (jj >= nk) return;
    char* st = ring + (jj % S) * kStageB;
    const int js = jj + rot < nk ? jj + rot : jj + rot - nk;
    const long kb = long(k0 + 64 * js);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = wave + 4 * j;                       // uniform: q < XK selects X
      if (q < XK) sk_dma16(X + kb * 2, off[j], sk_lds_addr(st + q * 1024));
      else sk_dma16nt(reinterpret_cast<const char*>(W) + kb * 2, off[j], sk_lds_addr(st + q * 1024));
    }
  };
  auto wait_for = [&](int jj) {                         // stage jj landed (this wave's part)
    const int ahead = min(nk - 1, jj + S - 2) - jj;     // later stages already issued
    static_assert(S <= 7 && (S - 2) * NQ < 64, "wait counts");
    switch (ahead) {
      case 5: sk_wait_vm<(S >= 7 ? 5 : 0) * NQ>(); break;
      case 4: sk_wait_vm<(S >= 6 ? 4 : 0) * NQ>(); break;
      case 3: sk_wait_vm<(S >= 5 ? 3 : 0) * NQ>(); break;
      case 2: sk_wait_vm<(S >= 4 ? 2 : 0) * NQ>(); break;
      case 1: sk_wait_vm<NQ>(); break;
      default: sk_wait_vm<0>(); break;
    }
  };

  f32x4_t acc[MT][NC];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // operand rows and their chunk XOR
  int arow[MT], brow[NC];
#pragma unroll
  for (int i = 0; i < MT; ++i) arow[i] = (MR / 2) * wm + 16 * i + (lane & 15);
#pragma unroll
  for (int i = 0; i < NC; ++i) brow[i] = (BN / 2) * wn + 16 * i + (lane & 15);
  const int g = lane >> 4;

#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(j);
  for (int i = 0; i < nk; ++i) {
    wait_for(i);
    sk_barrier();                                       // stage i visible; stage i - 1 consumed
    issue(i + S - 1);
    const char* st = ring + (i % S) * kStageB;
    constexpr int kXB = XF ? 256 : 128;                 // X row bytes
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t af[MT], bf[NC];
      [[maybe_unused]] bf16x8_t al[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        if constexpr (XF) {                             // hi: stored chunk 4 kk + g, lo: 8 + 4 kk + g
          const char* row = st + arow[t] * kXB;
          const int sw = arow[t] & 15;
          af[t] = *reinterpret_cast<const bf16x8_t*>(row + 16 * ((4 * kk + g) ^ sw));
          al[t] = *reinterpret_cast<const bf16x8_t*>(row + 16 * ((8 + 4 * kk + g) ^ sw));
        } else {
          af[t] = *reinterpret_cast<const bf16x8_t*>(st + arow[t] * 128 + 16 * ((4 * kk + g) ^ ((arow[t] >> 1) & 7)));
        }
      }
#pragma unroll
      for (int t = 0; t < NC; ++t)
        bf[t] = *reinterpret_cast<const bf16x8_t*>(st + MR * kXB + brow[t] * 128 +
                                                   16 * ((4 * kk + g) ^ ((brow[t] >> 1) & 7)));
#pragma unroll
      for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bf[c], acc[a][c], 0, 0, 0);
          if constexpr (XF) acc[a][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[a], bf[c], acc[a][c], 0, 0, 0);
        }
    }
  }
  // C layout: lane holds C[4 (lane / 16) + r][lane % 16] of each 16 x 16 tile.
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int gn = n0 + (BN / 2) * wn + 16 * c + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gm = (MR / 2) * wm + 16 * a + 4 * (lane >> 4) + r;
        if (gm < M && gn < N) {
          if constexpr (OUT == kOutQSplit) {
            const int hh = gn / 192, cc = gn - 192 * hh, HH = N / 192;
            if (cc < 128)
              reinterpret_cast<float*>(p.Y)[(long(gm) * HH + hh) * 128 + cc] = alpha * acc[a][c][r];
            else
              p.Y2[(long(gm) * HH + hh) * 64 + cc - 128] = acc[a][c][r];
          } else {
            sts_<OUT>(Y, long(gm) * ldc + gn, alpha * acc[a][c][r]);
          }
        }
      }
    }
}

template <int OUT, int BN, int MR, bool XF = false>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(SkinnyProb p) {
  __shared__ __attribute__((aligned(1024))) char ring[sk_stages<BN, MR, XF>() * sk_stage_bytes<BN, MR, XF>()];
  skinny_tile<OUT, BN, MR, XF>(p, blockIdx.x, blockIdx.z, int((blockIdx.x + gridDim.x * blockIdx.z) >> 3), ring);
}

// Two independent skinny problems in one launch: work-groups [0, tiles0) take p0's tiles,
// the rest p1's (one launch instead of two dependent-free ones back to back).
template <int OUT, int BN, int MR>
__global__ __launch_bounds__(256) void gemm_skinny_pair_kernel(SkinnyProb p0, SkinnyProb p1, int tiles0) {
  __shared__ __attribute__((aligned(1024))) char ring[sk_stages<BN, MR>() * sk_stage_bytes<BN, MR>()];
  const int id = blockIdx.x;
  if (id < tiles0) {
    const int nx = (p0.N + BN - 1) / BN;
    skinny_tile<OUT, BN, MR>(p0, id % nx, id / nx, id >> 3, ring);
  } else {
    const int nx = (p1.N + BN - 1) / BN;
    skinny_tile<OUT, BN, MR>(p1, (id - tiles0) % nx, (id - tiles0) / nx, id >> 3, ring);
  }
}


// ------------------------------------------------------------------ merge + W_UV (decode)
// out[b][h][n] = sum_c W_UV^h[n][c] * Otilde[b][h][c] for the heads' 32-row blocks, where Otilde
// is the log-sum-exp merge of the attention's split partials, formed on the fly:
//   m = max_j m_j,  w_j = 2^(m_j - m) / sum_j' 2^(m_j' - m) l_j',  Otilde = sum_j w_j O_j
// (scores are in base 2).  The partials O_j are fp16 as the attention writes them, or one fp32
// state when the splits were merged beforehand.  Otilde is summed in fp32 and enters the bf16
// MFMA as a hi + lo pair (hi = bf16(v), lo = bf16(v - hi)), so the product sees it to ~2^-16
// relative.  W_UV^h is rows [h (dn + dv) + dn, +dv) of kv_b_proj ([n][c], c contiguous).
// The split count SPL and the latent width DC are fixed at compile time, so that the K loop
// unrolls into straight-line code with its loads AH steps ahead of use (the weights of
// every split are likewise fetched at once).  Rows past B read row 0 of the partials with merge
// weight 0 (the partials are finite), so no branch guards the loads.

// Eight consecutive partials of one split, held as loaded and widened to fp32 at use.
template <typename P> struct Part8;
template <> struct Part8<float> {
  float4 x0, x1;
  __device__ __forceinline__ void load(const float* p) {
    x0 = *reinterpret_cast<const float4*>(p);
    x1 = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
    v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
  }
};
template <> struct Part8<uint16_t> {
  uint4 u;
  __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float* v) const {
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    const f16x8_t x = __builtin_bit_cast(f16x8_t, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = float(x[i]);
  }
};

// NKH: the latent range is cut into NKH parts, one wave per part covering both 16-row tiles
// (RT), so W_UV is requested once per work-group rather than once per row tile (the request
// stream, not the bytes, bounds this kernel).  AH: K steps prefetched.  The d_v = 128 output
// columns are cut into 128 / (16 NT) blocks, one per blockIdx.z.
template <int NT, int OUT, int SPL, int DC, int NKH, typename P, int AH>
__global__ __launch_bounds__(64 * NKH) void merge_uv_fixed_kernel(
    int B, int H, int dn, const P* __restrict__ part_o, const float* __restrict__ part_ml,
    const uint16_t* __restrict__ kv_b, typename StoreT<OUT>::type* __restrict__ out) {
  constexpr int dv = 128, half = DC / NKH, nk = half / 32, RT = 2;
  const int vb = blockIdx.z * 16 * NT;               // this work-group's output columns [vb, vb + 16 NT)
  static_assert(nk >= AH, "prefetch depth within the K loop");
  __shared__ f32x4_t red[2][NKH - 1][NT][64];       // other parts' sums, [row tile][part][tile][lane]
  __shared__ float wts[32][SPL];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = 0;                                 // first row tile of this wave
  const int kh = wave;                              // latent part
  const int h = blockIdx.x, b0 = blockIdx.y * 32;
  // Order of the requests: the merge statistics (every thread fetches its row's, tid & 31, so no
  // branch splits the loads), then the first AH steps of partials and weights, and only then the
  // wait for the statistics: the main stream is already in flight across the barrier.
  float mj[SPL], lj[SPL];
  {
    const int bm = min(b0 + (tid & 31), B - 1);       // (tid & 31: every thread, rows alike)
    const float* ml = part_ml + (long(bm) * SPL * H + h) * 2;
    const long step = long(H) * 2;
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      mj[j] = ml[j * step];
      lj[j] = ml[j * step + 1];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const int kq = 8 * (lane >> 4);
  const int kbeg = kh * half;
  const P* po[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int b = b0 + 16 * (rg + t) + (lane & 15);
    po[t] = part_o + (long(b < B ? b : 0) * SPL * H + h) * DC + kbeg + kq;
  }
  const long pstride = long(H) * DC;
  const uint16_t* wuv = kv_b + (long(h) * (dn + dv) + dn + vb + (lane & 15)) * DC + kbeg + kq;
  bf16x8_t wf[AH][NT];
  Part8<P> xo[AH][RT][SPL];
#pragma unroll
  for (int k = 0; k < AH; ++k) {
#pragma unroll
    for (int c = 0; c < NT; ++c) wf[k][c] = *reinterpret_cast<const bf16x8_t*>(wuv + long(16 * c) * DC + 32 * k);
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int j = 0; j < SPL; ++j) xo[k][t][j].load(po[t] + j * pstride + 32 * k);
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    // (every thread computes its row's weights and stores them, the copies of a row alike: a
    // store guarded by tid < 32 would let the compiler sink the statistics loads behind the
    // stream)
    const int b = b0 + (tid & 31);
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < SPL; ++j) m = fmaxf(m, mj[j]);
    float l = 0.f, e[SPL];
#pragma unroll
    for (int j = 0; j < SPL; ++j) {
      e[j] = mj[j] == -INFINITY ? 0.f : exp2f(mj[j] - m);
      l += e[j] * lj[j];
    }
    const float inv = (b < B && l > 0.f) ? 1.0f / l : 0.f;
#pragma unroll
    for (int j = 0; j < SPL; ++j) wts[tid & 31][j] = e[j] * inv;
  }
  __syncthreads();

  float wr[RT][SPL];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int j = 0; j < SPL; ++j) wr[t][j] = wts[16 * (rg + t) + (lane & 15)][j];
  f32x4_t acc[RT][NT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c) acc[t][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // (scheduling barriers keep the source order: the compiler would otherwise move each load
  // next to its use and shorten the prefetch distance to nothing)
#pragma unroll
  for (int k = 0; k < nk; ++k) {
    __builtin_amdgcn_sched_barrier(0);
    const int sl = k % AH;
    typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
    bf16x8v hi[RT], lo[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        const float wj = wr[t][j];
        float x[8];
        xo[sl][t][j].get(x);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += wj * x[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[t][e] = (__bf16)v[e];                     // round to nearest even
        lo[t][e] = (__bf16)(v[e] - (float)hi[t][e]);
      }
    }
    bf16x8_t w[NT];
#pragma unroll
    for (int c = 0; c < NT; ++c) w[c] = wf[sl][c];
    if (k + AH < nk) {                               // refill the slot AH steps ahead
      const int kn = 32 * (k + AH);
#pragma unroll
      for (int c = 0; c < NT; ++c) wf[sl][c] = *reinterpret_cast<const bf16x8_t*>(wuv + long(16 * c) * DC + kn);
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int j = 0; j < SPL; ++j) xo[sl][t][j].load(po[t] + j * pstride + kn);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NT; ++c) {
        acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi[t], w[c], acc[t][c], 0, 0, 0);
        acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo[t], w[c], acc[t][c], 0, 0, 0);
      }
  }
  if (kh > 0) {
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int c = 0; c < NT; ++c) red[rg + t][kh - 1][c][lane] = acc[t][c];
  }
  __syncthreads();
  if (kh > 0) return;
  // C layout: lane holds C[4 (lane / 16) + i][lane % 16] of each 16 x 16 tile.  The parts are
  // added in order.
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      f32x4_t o = acc[t][c];
#pragma unroll
      for (int q = 0; q < NKH - 1; ++q) o += red[rg + t][q][c][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bo = b0 + 16 * (rg + t) + 4 * (lane >> 4) + i;
        if (bo < B) sts_<OUT>(out, (long(bo) * H + h) * dv + vb + 16 * c + (lane & 15), o[i]);
      }
    }
}

template <int OUT, int SPL, typename P>
static void launch_merge_uv_fixed(int B, int H, int dn, const P* part_o, const float* part_ml,
                                  const void* kv_b, void* out, hipStream_t st) {
  constexpr int kParts = 4;
  const unsigned rows = unsigned((B + 31) / 32);
  // Few (head, 32-row) blocks (the Lite shape's 16 heads, a handful of long sequences): cut the
  // output columns over 2 or 4 work-groups, each streaming that share of W_UV^h.  (One wave per
  // latent quarter over both row tiles measured faster than two waves per quarter, one per row
  // tile, in all three forms: 17.0 -> 13.9, 9.6 -> 8.4 and 5.6 -> 5.3 us at the 236B, 128K and
  // Lite decode workloads.)
  const long blocks = long(H) * rows;
#define MLA_MUF(NT, Z, AH)                                                                           \
  hipLaunchKernelGGL((merge_uv_fixed_kernel<NT, OUT, SPL, 512, kParts, P, AH>), dim3(H, rows, Z),         \
                     dim3(64 * kParts), 0, st, B, H, dn, part_o, part_ml,                                 \
                     static_cast<const uint16_t*>(kv_b), static_cast<typename StoreT<OUT>::type*>(out))
  if (blocks <= 64) MLA_MUF(2, 4, 2);
  else if (blocks <= 128) MLA_MUF(4, 2, 2);
  else MLA_MUF(8, 1, 2);
#undef MLA_MUF
}

bool launch_decode_merge_uv(int out_type, int B, int H, int dc, int dn, int dv, int splits, const uint16_t* part_o,
                            const float* part_ml, const void* kv_b, void* out, hipStream_t st, float* otilde,
                            float* ml1) {
  if (dv != 128 || dc != 512 || splits < 1) return false;
#define MLA_MU(SPL, PO, ML)                                                                             \
  (out_type == K_BF16 ? launch_merge_uv_fixed<S_BF16, SPL>(B, H, dn, PO, ML, kv_b, out, st)             \
                      : launch_merge_uv_fixed<S_F32, SPL>(B, H, dn, PO, ML, kv_b, out, st))
  if (splits > 4) {
    if (!otilde || !ml1) return false;
    // Many splits: merge them first (every partial read once, one work-group per (b, h)), then
    // project the single merged fp32 state.
    launch_merge_splits(B, H, dc, splits, part_o, part_ml, otilde, ml1, st);
    MLA_MU(1, static_cast<const float*>(otilde), static_cast<const float*>(ml1));
    return true;
  }
  switch (splits) {
    case 1: MLA_MU(1, part_o, part_ml); break;
    case 2: MLA_MU(2, part_o, part_ml); break;
    case 3: MLA_MU(3, part_o, part_ml); break;
    default: MLA_MU(4, part_o, part_ml); break;
  }
#undef MLA_MU
  return true;
}

// ------------------------------------------------------------------ absorb + query RoPE (decode)
// qhat[b][h] = [ W_UK^h^T q_nope[b][h] (bf16, d_c values) | RoPE(q_pe[b][h]) (fp16, d_r values) ]
// with the softmax scale (times log2 e) folded in.  W_UK^h is rows [h (dn + dv), +dn) of
// kv_b_proj ([d][c], c contiguous).  Grid (d_c / KC + 1, H, ceil(B / 64)): blocks x < d_c / KC
// take latent columns [KC x, KC x + KC) of head h for 64 decode rows, the last x rotates q_pe.
// A latent block stages its [128 d x KC c] slice of W_UK^h in LDS (rows of 2 KC bytes, 32-byte
// segment s of row d at s ^ (d mod KC / 16), so the transposing reads of 16 rows spread over the
// banks) and forms the transposed product C[c][b] = sum_d W_UK[d][c] q[b][d]: W enters as the A
// operand through ds_read_b64_tr_b16 (8 consecutive d per lane), the query as the B operand.
// Wave w owns decode rows b0 + 16 w .. + 15 (it loads only its own queries) and every column
// tile of the block; the C layout leaves four consecutive columns of one row in a lane, stored
// as one 8-byte write.  The query q_nope (fp32) enters the products as a bf16 pair hi + lo (two
// MFMAs per fragment), so the latent query carries no bf16 rounding of its input; only the
// result is rounded (to bf16).  The RoPE part is kept in fp16 (11 significant bits): with the
// rotary key it scores in an fp16 product, where it would lose three bits in bf16.
// QS: q_nope arrives as fp32 alpha q [B][H][DN] and q_pe as fp32 q [B][H][dr] (the projection's
// split epilogue); otherwise q is the sum of nsplit fp32 partials of the projection.
template <int DN, int KC, bool QS>
__global__ __launch_bounds__(256) void absorb_rope_kernel(
    int B, int H, int dr, int dc, int dv, int nsplit, const float* __restrict__ q_acc,
    const float* __restrict__ q_nope32, const float* __restrict__ q_pe32,
    const float* __restrict__ rope_tab, float scale, const uint16_t* __restrict__ kv_b,
    uint16_t* __restrict__ qhat) {
  constexpr int kKs = DN / 32;                        // K steps
  constexpr int kMt = KC / 16;                        // 16-column tiles
  constexpr int kSeg = KC / 16;                       // 32-byte segments per staged row
  __shared__ __attribute__((aligned(16))) char wt[DN * KC * 2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, b0 = blockIdx.z * 64;
  const int dqk = DN + dr, W = dc + dr;
  const long nq = long(H) * dqk, sstride = long(B) * nq;
  const float* qh = q_acc + long(h) * dqk;            // (!QS) partial 0 of head h, row 0
  auto qsum = [&](int b, int i) {
    float v = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) v += qh[sp * sstride + long(b) * nq + i];
    return v;
  };
  if (blockIdx.x == gridDim.x - 1) {                  // RoPE block: fp16 (scale RoPE(q_pe))
    const int half = dr / 2;
    for (int e = tid; e < 64 * half; e += 256) {
      const int b = b0 + e / half, pi = e % half;
      if (b >= B) continue;
      const float c = rope_tab[long(b) * dr + pi], sn = rope_tab[long(b) * dr + half + pi];
      float ev, ov;
      if constexpr (QS) {
        const float* qp = q_pe32 + (long(b) * H + h) * dr + 2 * pi;
        ev = qp[0];
        ov = qp[1];
      } else {
        ev = qsum(b, DN + 2 * pi);
        ov = qsum(b, DN + 2 * pi + 1);
      }
      const uint32_t pr = uint32_t(f2h(scale * (ev * c - ov * sn))) | (uint32_t(f2h(scale * (ev * sn + ov * c))) << 16);
      *reinterpret_cast<uint32_t*>(qhat + (long(b) * H + h) * W + dc + 2 * pi) = pr;
    }
    return;
  }
  const int c0 = blockIdx.x * KC;
  const int li = lane & 15, g = lane >> 4;
  const int rb = b0 + 16 * wave;                      // the wave's first decode row (a wave past
                                                      // B still stages its share of the weight)
  // The wave's queries (B operand): lane (li, g) holds q_nope[rb + li][32 ks + 8 g .. + 7],
  // scaled; rows past B re-read row B - 1 and are not stored.  Requested before the weight, so
  // the two loads overlap.
  float v[kKs][8];
  {
    const int bl = min(rb + li, B - 1);
    if constexpr (QS) {
      const float* src = q_nope32 + (long(bl) * H + h) * DN + 8 * g;
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        const float4 x0 = *reinterpret_cast<const float4*>(src + 32 * ks);
        const float4 x1 = *reinterpret_cast<const float4*>(src + 32 * ks + 4);
        v[ks][0] = x0.x; v[ks][1] = x0.y; v[ks][2] = x0.z; v[ks][3] = x0.w;
        v[ks][4] = x1.x; v[ks][5] = x1.y; v[ks][6] = x1.z; v[ks][7] = x1.w;
      }
    } else {
      // fp32 partials, added in split order, then scaled
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[ks][j] = 0.f;
      const float* src = qh + long(bl) * nq + 8 * g;
      for (int sp = 0; sp < nsplit; ++sp) {
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks) {
          const float4 x0 = *reinterpret_cast<const float4*>(src + sp * sstride + 32 * ks);
          const float4 x1 = *reinterpret_cast<const float4*>(src + sp * sstride + 32 * ks + 4);
          v[ks][0] += x0.x; v[ks][1] += x0.y; v[ks][2] += x0.z; v[ks][3] += x0.w;
          v[ks][4] += x1.x; v[ks][5] += x1.y; v[ks][6] += x1.z; v[ks][7] += x1.w;
        }
      }
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[ks][j] *= scale;
    }
  }
  {
    // W_UK^h[d][c0 .. c0 + KC): 16-byte chunk ch of row d (columns 8 ch .. + 7) at segment
    // (ch >> 1) ^ (d mod kSeg), half ch & 1
    const uint16_t* wsrc = kv_b + long(h) * (DN + dv) * dc + c0;
    constexpr int kRowCh = KC / 8, kChunks = DN * kRowCh;
    static_assert(kChunks % 256 == 0, "whole chunks per thread");
    uint4 w[kChunks / 256];
#pragma unroll
    for (int j = 0; j < kChunks / 256; ++j) {
      const int i = tid + 256 * j, d = i / kRowCh, ch = i % kRowCh;
      w[j] = *reinterpret_cast<const uint4*>(wsrc + long(d) * dc + 8 * ch);
    }
#pragma unroll
    for (int j = 0; j < kChunks / 256; ++j) {
      const int i = tid + 256 * j, d = i / kRowCh, ch = i % kRowCh;
      *reinterpret_cast<uint4*>(wt + d * (2 * KC) + 32 * ((ch >> 1) ^ (d % kSeg)) + 16 * (ch & 1)) = w[j];
    }
  }
  __syncthreads();
  if (rb >= B) return;                                // uniform over the wave
  typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
  typedef short s16x4v __attribute__((ext_vector_type(4)));
  typedef short s16x8v __attribute__((ext_vector_type(8)));
  f32x4_t acc[kMt];
#pragma unroll
  for (int mt = 0; mt < kMt; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks) {
    bf16x8v hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hi[j] = (__bf16)v[ks][j];                       // round to nearest even
      lo[j] = (__bf16)(v[ks][j] - (float)hi[j]);
    }
    const bf16x8_t qh8 = __builtin_bit_cast(bf16x8_t, hi), ql8 = __builtin_bit_cast(bf16x8_t, lo);
    // A fragments of this K step: W_UK[32 ks + 8 g + j][c0 + 16 mt + li], transposing reads of
    // rows d0 .. d0 + 3 (and + 4 .. + 7), lane (li & 3) taking columns 4 (li & 3) .. + 3 of the
    // tile's segment
    bf16x8_t aw[kMt];
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt) {
      const int d0 = 32 * ks + 8 * g + (li >> 2);
      const char* p0 = wt + d0 * (2 * KC) + 32 * (mt ^ (d0 % kSeg)) + 8 * (li & 3);
      const char* p1 = wt + (d0 + 4) * (2 * KC) + 32 * (mt ^ ((d0 + 4) % kSeg)) + 8 * (li & 3);
      const s16x4v a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4v __attribute__((address_space(3)))*)(p0));
      const s16x4v a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4v __attribute__((address_space(3)))*)(p1));
      const s16x8v av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      aw[mt] = __builtin_bit_cast(bf16x8_t, av);
    }
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt) {
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[mt], qh8, acc[mt], 0, 0, 0);
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[mt], ql8, acc[mt], 0, 0, 0);
    }
  }
  // C layout: lane holds C[c = 16 mt + 4 g + r][b = rb + li], r = 0..3: four consecutive latent
  // columns of one row, one 8-byte store
  const int bo = rb + li;
  if (bo < B) {
    uint16_t* dst = qhat + (long(bo) * H + h) * W + c0 + 4 * g;
#pragma unroll
    for (int mt = 0; mt < kMt; ++mt)
      *reinterpret_cast<uint2*>(dst + 16 * mt) =
          make_uint2(uint32_t(f2bf(acc[mt][0])) | (uint32_t(f2bf(acc[mt][1])) << 16),
                     uint32_t(f2bf(acc[mt][2])) | (uint32_t(f2bf(acc[mt][3])) << 16));
  }
}

bool launch_absorb_rope(int B, int H, int dn, int dr, int dc, int dv, int nsplit, const float* q_acc,
                        const float* rope_tab, float scale, const void* kv_b, void* qhat, hipStream_t st,
                        const float* q_nope32, const float* q_pe32) {
  if (dn != 128 || dc != 512 || dr % 2 != 0 || B <= 0) return false;
  // 128-column blocks; 64-column ones when there are few heads, so that the blocks still spread
  // over the CUs
  const bool narrow = H < 64;
  const dim3 grid(dc / (narrow ? 64 : 128) + 1, H, (B + 63) / 64);
  const bool qs = q_nope32 && q_pe32;
#define MLA_AB(KC, QS)                                                                                   \
  hipLaunchKernelGGL((absorb_rope_kernel<128, KC, QS>), grid, dim3(256), 0, st, B, H, dr, dc, dv, nsplit, \
                     QS ? nullptr : q_acc, q_nope32, q_pe32, rope_tab, scale, static_cast<const uint16_t*>(kv_b), \
                     static_cast<uint16_t*>(qhat))
  if (narrow) {
    if (qs) MLA_AB(64, true);
    else MLA_AB(64, false);
  } else {
    if (qs) MLA_AB(128, true);
    else MLA_AB(128, false);
  }
#undef MLA_AB
  return true;
}


// ------------------------------------------------------------------ launcher
template <int BM, int BN, int BK, bool NN, int OUT>
static void launch_bf16(const GemmArgs& g, hipStream_t st) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch * g.nsplit);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NN, OUT>), grid, dim3(256), 0, st, g.M, g.N, g.K,
                     g.kchunk, static_cast<const uint16_t*>(g.X), g.lda, g.sx,
                     static_cast<const uint16_t*>(g.W), g.ldw, g.sw,
                     static_cast<typename StoreT<OUT>::type*>(g.Y), g.ldc, g.sy, g.ssplit, g.alpha, g.nsplit);
}

// The skinny kernel's conditions: TN, M <= 128, K and the chunk in 64-steps, 16-byte rows, and
// per-operand offsets that fit the 32-bit load offsets.
static bool skinny_ok(const GemmArgs& g) {
  return g.kind == GEMM_BF16 && !g.nn && g.M <= 128 && g.K % 64 == 0 && g.kchunk % 64 == 0 &&
         g.lda % 8 == 0 && g.ldw % 8 == 0 && (!g.xpair || g.lda >= 2L * g.K) &&
         long(g.M) * g.lda * 2 < (1L << 32) && long(g.N) * g.ldw * 2 < (1L << 32);
}

bool launch_gemm_skinny_ok(const GemmArgs& g) { return skinny_ok(g); }

static SkinnyProb skinny_prob(const GemmArgs& g) {
  SkinnyProb p;
  p.M = g.M; p.N = g.N; p.K = g.K; p.kchunk = g.kchunk; p.nsplit = g.nsplit;
  p.X = g.X; p.lda = g.lda; p.sx = g.sx;
  p.W = static_cast<const uint16_t*>(g.W); p.ldw = g.ldw; p.sw = g.sw;
  p.Y = g.Y; p.ldc = g.ldc; p.sy = g.sy; p.ssplit = g.ssplit;
  p.alpha = g.alpha;
  p.Y2 = nullptr;
  return p;
}

// A skinny launch: 96-column tiles when they fill the CUs in whole rounds and 64-column tiles do
// not (fewer, better balanced work-groups, each re-reading X for more columns).
template <int OUT, bool XF>
static void launch_skinny(const GemmArgs& g, const SkinnyProb& p, hipStream_t st) {
  const long z = long(g.batch) * g.nsplit;
#define MLA_SK(BN, MR, NX) \
  hipLaunchKernelGGL((gemm_skinny_kernel<OUT, BN, MR, XF>), dim3(NX, 1, unsigned(z)), dim3(256), 0, st, p)
  if (g.bn == 160 && g.N % 160 == 0) {
    if (g.M <= 64) MLA_SK(160, 64, g.N / 160);
    else MLA_SK(160, 128, g.N / 160);
    return;
  }
  if (g.N % 96 == 0 && (g.N / 96) * z % 256 == 0 && ((g.N + 63) / 64) * z % 256 != 0) {
    if (g.M <= 64) MLA_SK(96, 64, g.N / 96);
    else MLA_SK(96, 128, g.N / 96);
    return;
  }
  if (g.M <= 64) MLA_SK(64, 64, (g.N + 63) / 64);
  else MLA_SK(64, 128, (g.N + 63) / 64);
#undef MLA_SK
}

template <bool NN, int OUT>
static void launch_bf16_shape(const GemmArgs& g, hipStream_t st) {
  long tiles_big = long((g.M + 127) / 128) * ((g.N + 127) / 128) * g.batch * g.nsplit;
  if (!NN && skinny_ok(g)) {
    if (g.xpair) launch_skinny<OUT, true>(g, skinny_prob(g), st);
    else launch_skinny<OUT, false>(g, skinny_prob(g), st);
    return;
  }
  if (g.xpair) return;                              // (callers check skinny_ok first)
  if (g.M <= 64)
    launch_bf16<64, 128, 64, NN, OUT>(g, st);
  else if (tiles_big >= 256)
    launch_bf16<128, 128, 32, NN, OUT>(g, st);
  else
    launch_bf16<64, 64, 64, NN, OUT>(g, st);
}

template <bool NN>
static void launch_bf16_out(const GemmArgs& g, hipStream_t st) {
  if (g.out == K_BF16) launch_bf16_shape<NN, S_BF16>(g, st);
  else if (g.out == K_F16) launch_bf16_shape<NN, S_F16>(g, st);
  else launch_bf16_shape<NN, S_F32>(g, st);
}

bool launch_q_split_gemm(const GemmArgs& g, float* q_pe, hipStream_t st) {
  if (!skinny_ok(g) || g.nsplit != 1 || g.batch != 1 || g.N % 192 != 0) return false;
  SkinnyProb p = skinny_prob(g);
  p.Y2 = q_pe;
  const GemmArgs one = g;
  if (g.xpair) launch_skinny<kOutQSplit, true>(one, p, st);
  else launch_skinny<kOutQSplit, false>(one, p, st);
  return true;
}

bool launch_gemm_pair(const GemmArgs& a, const GemmArgs& b, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0 || b.M <= 0 || b.N <= 0 || b.batch <= 0) return false;
  if (!skinny_ok(a) || !skinny_ok(b) || a.out != K_F32 || b.out != K_F32) return false;
  // 96-column tiles when both widths allow them (the split planned for the pair assumes so)
  const int bn = (a.N % 96 == 0 && b.N % 96 == 0) ? 96 : 64;
  const long t0 = long((a.N + bn - 1) / bn) * a.batch * a.nsplit;
  const long t1 = long((b.N + bn - 1) / bn) * b.batch * b.nsplit;
  if (t0 + t1 > (1L << 31) - 1) return false;
#define MLA_SKP(BN, MR)                                                                                  \
  hipLaunchKernelGGL((gemm_skinny_pair_kernel<S_F32, BN, MR>), dim3(unsigned(t0 + t1)), dim3(256), 0, st, \
                     skinny_prob(a), skinny_prob(b), int(t0))
  const bool m64 = a.M <= 64 && b.M <= 64;
  if (bn == 96) {
    if (m64) MLA_SKP(96, 64);
    else MLA_SKP(96, 128);
  } else {
    if (m64) MLA_SKP(64, 64);
    else MLA_SKP(64, 128);
  }
#undef MLA_SKP
  return true;
}

void launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return;
  if (g.kind == GEMM_F32) {
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batch * g.nsplit);
    if (g.nn)
      hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, st, g.M, g.N, g.K, g.kchunk,
                         static_cast<const float*>(g.X), g.lda, g.sx, static_cast<const float*>(g.W),
                         g.ldw, g.sw, static_cast<float*>(g.Y), g.ldc, g.sy, g.ssplit, g.alpha, g.nsplit);
    else
      hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, st, g.M, g.N, g.K, g.kchunk,
                         static_cast<const float*>(g.X), g.lda, g.sx, static_cast<const float*>(g.W),
                         g.ldw, g.sw, static_cast<float*>(g.Y), g.ldc, g.sy, g.ssplit, g.alpha, g.nsplit);
    return;
  }
  if (launch_gemm_tile(g, st)) return;
  if (g.f16in || g.row_scale) return;               // (callers check launch_gemm_tile_ok first)
  if (g.nn) launch_bf16_out<true>(g, st);
  else launch_bf16_out<false>(g, st);
}

}  // namespace mla
