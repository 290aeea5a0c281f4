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
    int M, int N, int K, int kchunk, int kwrap, const uint16_t* __restrict__ X, long lda, long sx,
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
        int wk = kwrap ? gk % kwrap : gk;
        rb[i] = (gn < N && gk < k1) ? *reinterpret_cast<const uint4*>(W + gn * ldw + wk) : make_uint4(0, 0, 0, 0);
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

// ------------------------------------------------------------------ launcher
template <int BM, int BN, int BK, bool NN, int OUT>
static void launch_bf16(const GemmArgs& g, hipStream_t st) {
  dim3 grid((g.N + BN - 1) / BN, (g.M + BM - 1) / BM, g.batch * g.nsplit);
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NN, OUT>), grid, dim3(256), 0, st, g.M, g.N, g.K,
                     g.kchunk, g.kwrap, static_cast<const uint16_t*>(g.X), g.lda, g.sx,
                     static_cast<const uint16_t*>(g.W), g.ldw, g.sw,
                     static_cast<typename StoreT<OUT>::type*>(g.Y), g.ldc, g.sy, g.ssplit, g.alpha, g.nsplit);
}

template <bool NN, int OUT>
static void launch_bf16_shape(const GemmArgs& g, hipStream_t st) {
  long tiles_big = long((g.M + 127) / 128) * ((g.N + 127) / 128) * g.batch * g.nsplit;
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
  if (g.nn) launch_bf16_out<true>(g, st);
  else launch_bf16_out<false>(g, st);
}

}  // namespace mla
