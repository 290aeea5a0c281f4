// Large-tile bf16 GEMM for the prefill projections (q_b and the kv_b decompression), TN with a
// 2-byte output:  Y[z] = alpha * X[z] (M x K, row-major) * W[z]^T  (W [N][K], K contiguous).
//
// One work-group of 8 waves per 256 x 256 output tile; wave w computes rows
// [128 (w >> 2), +128) x columns [64 (w & 3), +64) as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16
// (128 fp32 accumulators).  X and W tiles (256 rows x 64 K each, 32 KiB) stream through LDS
// with direct global->LDS loads, double-buffered (128 KiB); 16-byte chunk c of tile row r is
// stored at c ^ ((r >> 1) & 7), so the operand reads (16 rows x one chunk per 16 lanes) hit
// distinct banks.  The result goes through the same LDS (chunk XOR (row & 7)) and leaves as
// whole 16-byte row segments.  Rows of X or W past M or N re-read the last row; their results
// are not stored.
#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_lds.h"

namespace mla {

namespace {

constexpr int kTM = 256, kTN = 256, kTK = 64;
constexpr int kTileA = kTM * kTK * 2;            // 32 KiB
constexpr int kStageBytes = 2 * kTileA;          // X tile | W tile
constexpr int kLoadsPerOperand = 4;              // per wave and stage: 32 one-KiB loads / 8 waves

typedef float f32x16_t __attribute__((ext_vector_type(16)));

}  // namespace

template <int OUT>
__global__ __launch_bounds__(512, 1) void gemm_tile_kernel(
    int M, int N, int K, int tiles_m, const uint16_t* __restrict__ X, long lda, long sx,
    const uint16_t* __restrict__ W, long ldw, long sw, uint16_t* __restrict__ Y, long ldc, long sy,
    float alpha) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * kTM, n0 = tn * kTN;
  const long z = blockIdx.y;
  const char* xb = reinterpret_cast<const char*>(X + z * sx + long(m0) * lda);
  const char* wb = reinterpret_cast<const char*>(W + z * sw + long(n0) * ldw);
  Y += z * sy;
  const int nks = K / kTK;

  // Load q of wave w (q < 4) fills KiB w + 8 q of a tile: rows 8 (w + 8 q) + (lane >> 3), stored
  // chunk lane & 7, logical chunk (lane & 7) ^ ((row >> 1) & 7).
  uint32_t off_x[kLoadsPerOperand], off_w[kLoadsPerOperand];
#pragma unroll
  for (int q = 0; q < kLoadsPerOperand; ++q) {
    const int row = 8 * (wave + 8 * q) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    off_x[q] = uint32_t(min(row, M - 1 - m0)) * uint32_t(lda * 2) + 16u * c;
    off_w[q] = uint32_t(min(row, N - 1 - n0)) * uint32_t(ldw * 2) + 16u * c;
  }
  auto issue = [&](int ks) {
    if (ks >= nks) return;
    char* dst = smem + (ks & 1) * kStageBytes;
    const char* xa = xb + ks * (kTK * 2);
    const char* wa = wb + ks * (kTK * 2);
#pragma unroll
    for (int q = 0; q < kLoadsPerOperand; ++q) lds::dma16(xa, off_x[q], lds::addr(dst + (wave + 8 * q) * 1024));
#pragma unroll
    for (int q = 0; q < kLoadsPerOperand; ++q)
      lds::dma16(wa, off_w[q], lds::addr(dst + kTileA + (wave + 8 * q) * 1024));
  };

  const int wm = wave >> 2, wn = wave & 3;
  const int xr = (lane & 31) * 128, sw_x = ((lane & 31) >> 1) & 7, e = lane >> 5;
  auto opnd = [&](const char* t, int row0, int st) {     // rows row0 + (lane & 31), K 16 st + 8 e
    return *reinterpret_cast<const bf16x8_t*>(t + row0 * 128 + xr + 16 * ((2 * st + e) ^ sw_x));
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[i][j][k] = 0.f;

  issue(0);
  for (int ks = 0; ks < nks; ++ks) {
    issue(ks + 1);
    if (ks + 1 < nks) lds::wait_vm<2 * kLoadsPerOperand>();
    else lds::wait_vm<0>();
    lds::barrier();                                  // stage ks in LDS for every wave
    const char* ta = smem + (ks & 1) * kStageBytes;
    const char* tb = ta + kTileA;
#pragma unroll
    for (int st = 0; st < kTK / 16; ++st) {
      bf16x8_t a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = opnd(ta, 128 * wm + 32 * i, st);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = opnd(tb, 64 * wn + 32 * j, st);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    lds::barrier();                                  // stage ks's buffer free for stage ks + 2
  }

  // Result tile through LDS: [256][256] 2-byte values, 16-byte chunk c of row r at c ^ (r & 7).
  // C layout: lane holds C[8 (k >> 2) + 4 e + (k & 3)][lane & 31] of each 32 x 32 tile.
  uint16_t* ct = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = 64 * wn + 32 * j + (lane & 31);
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int m = 128 * wm + 32 * i + 8 * (k >> 2) + 4 * e + (k & 3);
        const float v = alpha * acc[i][j][k];
        ct[m * kTN + 8 * ((n >> 3) ^ (m & 7)) + (n & 7)] = OUT == S_BF16 ? f2bf(v) : f2h(v);
      }
    }
  lds::barrier();
#pragma unroll 4
  for (int it = 0; it < kTM * kTN / 8 / 512; ++it) {
    const int idx = tid + 512 * it;
    const int r = idx >> 5, c = idx & 31;
    const int gm = m0 + r, gn = n0 + 8 * c;
    const uint4 v = *reinterpret_cast<const uint4*>(ct + r * kTN + 8 * (c ^ (r & 7)));
    if (gm < M && gn < N) *reinterpret_cast<uint4*>(Y + long(gm) * ldc + gn) = v;
  }
}

bool launch_gemm_tile(const GemmArgs& g, hipStream_t st) {
  if (g.kind != GEMM_BF16 || g.nn || g.nsplit != 1) return false;
  if (g.out != K_BF16 && g.out != K_F16) return false;
  if (g.K % kTK != 0 || g.N % 8 != 0 || g.lda % 8 != 0 || g.ldw % 8 != 0 || g.ldc % 8 != 0) return false;
  if (g.sx % 8 != 0 || g.sw % 8 != 0 || g.sy % 8 != 0) return false;
  if ((reinterpret_cast<uintptr_t>(g.X) | reinterpret_cast<uintptr_t>(g.W) | reinterpret_cast<uintptr_t>(g.Y)) & 15)
    return false;
  // 32-bit load offsets: 255 rows of X or W
  if (long(kTM) * g.lda * 2 >= (1L << 31) || long(kTN) * g.ldw * 2 >= (1L << 31)) return false;
  const long tiles_m = (g.M + kTM - 1) / kTM, tiles_n = (g.N + kTN - 1) / kTN;
  if (tiles_m * tiles_n * g.batch < 256 || g.batch > 65535 || tiles_m * tiles_n > (1L << 30)) return false;
  const dim3 grid(unsigned(tiles_m * tiles_n), unsigned(g.batch));
  if (g.out == K_BF16)
    hipLaunchKernelGGL(gemm_tile_kernel<S_BF16>, grid, dim3(512), 0, st, g.M, g.N, g.K, int(tiles_m),
                       static_cast<const uint16_t*>(g.X), g.lda, g.sx, static_cast<const uint16_t*>(g.W), g.ldw,
                       g.sw, static_cast<uint16_t*>(g.Y), g.ldc, g.sy, g.alpha);
  else
    hipLaunchKernelGGL(gemm_tile_kernel<S_F16>, grid, dim3(512), 0, st, g.M, g.N, g.K, int(tiles_m),
                       static_cast<const uint16_t*>(g.X), g.lda, g.sx, static_cast<const uint16_t*>(g.W), g.ldw,
                       g.sw, static_cast<uint16_t*>(g.Y), g.ldc, g.sy, g.alpha);
  return true;
}

}  // namespace mla
