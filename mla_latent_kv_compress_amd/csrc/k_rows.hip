// Row-wise kernels of the MLA path: cache-row epilogue of the KV compression, the query
// RMSNorm and packing, index preparation, the split-K merge and the prefill gather.
#include <algorithm>
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_lds.h"

namespace mla {

// Sum of the K-split partials acc[s * stride + i], s = 0 .. n-1, in split order.  Eight loads are
// issued before the adds so the chain is not one memory latency per split.
__device__ __forceinline__ float split_sum(const float* __restrict__ acc, int n, long stride, long i) {
  float v = 0.f;
  int s = 0;
  for (; s + 8 <= n; s += 8) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = acc[(s + j) * stride + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += x[j];
  }
  for (; s < n; ++s) v += acc[s * stride + i];
  return v;
}

// Same for four consecutive values i .. i+3 (i and stride multiples of 4, acc 16-byte aligned).
// The loads of up to 8 splits are in flight together, so a row costs one or two memory
// latencies rather than one per few splits; the adds stay in split order.
__device__ __forceinline__ float4 split_sum4(const float* __restrict__ acc, int n, long stride, long i) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < n; s += 8) {
    float4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      x[j] = s + j < n ? *reinterpret_cast<const float4*>(acc + (s + j) * stride + i) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s + j < n) {
        v.x += x[j].x; v.y += x[j].y; v.z += x[j].z; v.w += x[j].w;
      }
    }
  }
  return v;
}

// ------------------------------------------------------------------ query partial sum (decode)
struct QSumArgs {
  long n4 = 0;                 // (T H 192) / 4; 0: nothing to do
  int nsplit = 1;
  const float* acc = nullptr;
  long stride = 0;             // T H 192
  float alpha = 1.f;
  float* q_nope32 = nullptr;
  float* q_pe32 = nullptr;
};
__device__ __forceinline__ void q_split_sum_part(const QSumArgs& q, long part, long parts) {
  for (long i4 = part * 256 + threadIdx.x; i4 < q.n4; i4 += parts * 256) {
    const long i = 4 * i4;                                    // element of [T][H][192]
    const float4 v = split_sum4(q.acc, q.nsplit, q.stride, i);
    const long th = i / 192;
    const int c = int(i - th * 192);                          // a multiple of 4: never straddles 128
    if (c < 128)
      *reinterpret_cast<float4*>(q.q_nope32 + th * 128 + c) =
          make_float4(q.alpha * v.x, q.alpha * v.y, q.alpha * v.z, q.alpha * v.w);
    else
      *reinterpret_cast<float4*>(q.q_pe32 + th * 64 + c - 128) = v;
  }
}

// ------------------------------------------------------------------ compress epilogue
// One block per token.  a = sum of the kv_a partials = [latent (dc) | k_pe (dr)].
// latent <- latent / sqrt(mean(latent^2) + eps) * gamma;  k_pe <- RoPE(k_pe, pos);
// the row is rounded to the cache format and written to its slot (skipped if out of range).
template <typename ActT, int CACHE>
__device__ __forceinline__ void compress_row(
    int t, int dc, int dr, int T, int nsplit, const float* __restrict__ acc, const ActT* __restrict__ gamma,
    const int32_t* __restrict__ pos, const int64_t* __restrict__ slots, void* __restrict__ cache,
    float* __restrict__ cache_scale, long num_slots, float eps, RopeParams rp, float* __restrict__ rope_tab,
    const int32_t* __restrict__ ctx, const int32_t* __restrict__ bt, int max_blocks, float* row, float* red) {
  const int W = dc + dr;
  // Decode (ctx given): the token is the last of a context of ctx[t] rows, at position ctx[t] - 1.
  int p;
  long slot;
  if (ctx) {
    p = ctx[t] - 1;
    const int page = p >= 0 ? p / kPage : -1;
    slot = (page >= 0 && page < max_blocks) ? long(bt[long(t) * max_blocks + page]) * kPage + p % kPage : -1;
    if (p < 0) p = 0;
  } else {
    p = pos[t];
    slot = slots[t];
  }
  // The token's RoPE angles, pair ri on the block's last dr / 2 threads (which the split sums
  // below leave idle when the row is narrow, so the fp64 work overlaps their loads); also written
  // to rope_tab for the query's RoPE.  dr <= 256 (validated), so dr / 2 <= blockDim.x.
  const int ri = int(threadIdx.x) - (int(blockDim.x) - dr / 2);
  float rc = 1.f, rsn = 0.f;
  if (ri >= 0) {
    rope_cs(p, ri, dr, rp, &rc, &rsn);
    if (rope_tab) {
      rope_tab[long(t) * dr + ri] = rc;
      rope_tab[long(t) * dr + dr / 2 + ri] = rsn;
    }
  }
  if (slot < 0 || slot >= num_slots) return;        // uniform over the block
  if (W % 4 == 0) {
    for (int i = 4 * threadIdx.x; i < W; i += 4 * blockDim.x)
      *reinterpret_cast<float4*>(&row[i]) = split_sum4(acc, nsplit, long(T) * W, long(t) * W + i);
  } else {
    for (int i = threadIdx.x; i < W; i += blockDim.x) row[i] = split_sum(acc, nsplit, long(T) * W, long(t) * W + i);
  }
  __syncthreads();
  float ss = 0.f;
  for (int i = threadIdx.x; i < dc; i += blockDim.x) ss += row[i] * row[i];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / float(dc) + eps);
  for (int i = threadIdx.x; i < dc; i += blockDim.x) row[i] = row[i] * r * ldf<ActT>(gamma, i);
  if (ri >= 0) {
    const float e = row[dc + 2 * ri], o = row[dc + 2 * ri + 1];
    row[dc + 2 * ri] = e * rc - o * rsn;
    row[dc + 2 * ri + 1] = e * rsn + o * rc;
  }
  __syncthreads();
  if (CACHE == K_F32) {
    float* dst = static_cast<float*>(cache) + slot * W;
    for (int i = threadIdx.x; i < W; i += blockDim.x) dst[i] = row[i];
  } else if (CACHE == K_BF16) {
    uint16_t* dst = static_cast<uint16_t*>(cache) + slot * W;
    for (int i = threadIdx.x; i < W; i += blockDim.x) dst[i] = f2bf(row[i]);
  } else {
    float am = 0.f;
    for (int i = threadIdx.x; i < W; i += blockDim.x) am = fmaxf(am, fabsf(row[i]));
    am = block_max(am, red);
    const float sc = am > 0.f ? __fdiv_rn(am, 448.0f) : 1.0f;
    uint8_t* dst = static_cast<uint8_t*>(cache) + slot * W;
    for (int i = threadIdx.x; i < W; i += blockDim.x) dst[i] = uint8_t(f_to_e4m3(__fdiv_rn(row[i], sc)));
    if (threadIdx.x == 0) cache_scale[slot] = sc;
  }
}

template <typename ActT, int CACHE>
__global__ __launch_bounds__(256) void compress_rows_kernel(
    int dc, int dr, int T, int nsplit, const float* __restrict__ acc, const ActT* __restrict__ gamma,
    const int32_t* __restrict__ pos, const int64_t* __restrict__ slots, void* __restrict__ cache,
    float* __restrict__ cache_scale, long num_slots, float eps, RopeParams rp, float* __restrict__ rope_tab,
    const int32_t* __restrict__ ctx, const int32_t* __restrict__ bt, int max_blocks, QSumArgs qs) {
  extern __shared__ float row[];                    // [dc + dr]
  __shared__ float red[16];
  if (int(blockIdx.x) >= T) {                       // the query partial sum, in the same launch
    q_split_sum_part(qs, blockIdx.x - T, gridDim.x - T);
    return;
  }
  compress_row<ActT, CACHE>(blockIdx.x, dc, dr, T, nsplit, acc, gamma, pos, slots, cache, cache_scale, num_slots,
                            eps, rp, rope_tab, ctx, bt, max_blocks, row, red);
}

void launch_compress_rows(int act, int cache, int T, int dc, int dr, int nsplit, const float* acc,
                          const void* gamma, const int32_t* pos, const int64_t* slots,
                          void* cache_data, float* cache_scale, long num_slots, float eps,
                          const RopeParams& rp, float* rope_tab, const int32_t* ctx, const int32_t* bt, int max_blocks,
                          hipStream_t st, int qsplit_n, const float* q_acc, int H, float alpha, float* q_nope32,
                          float* q_pe32) {
  if (T <= 0) return;
  size_t sh = size_t(dc + dr) * sizeof(float);
  QSumArgs qs;
  long qblocks = 0;
  if (q_acc) {
    qs.n4 = long(T) * H * 192 / 4;
    qs.nsplit = qsplit_n;
    qs.acc = q_acc;
    qs.stride = long(T) * H * 192;
    qs.alpha = alpha;
    qs.q_nope32 = q_nope32;
    qs.q_pe32 = q_pe32;
    qblocks = std::min<long>((qs.n4 + 255) / 256, 1024);
  }
#define MLA_CR(A, C)                                                                          \
  hipLaunchKernelGGL((compress_rows_kernel<A, C>), dim3(unsigned(T + qblocks)), dim3(256), sh, st, dc, dr, T, nsplit, \
                     acc, static_cast<const A*>(gamma), pos, slots, cache_data, cache_scale,      \
                     num_slots, eps, rp, rope_tab, ctx, bt, max_blocks, qs)
  if (act == K_F32) {
    MLA_CR(float, K_F32);
  } else if (cache == K_BF16) {
    MLA_CR(uint16_t, K_BF16);
  } else {
    MLA_CR(uint16_t, K_FP8);
  }
#undef MLA_CR
}

// ------------------------------------------------------------------ RMSNorm of query latents
template <typename ActT, typename OutT = ActT>
__device__ __forceinline__ void rmsnorm_row(int t, int T, int n, int nsplit, const float* __restrict__ acc,
                                            const ActT* __restrict__ gamma, OutT* __restrict__ out, float eps,
                                            float* row, float* red) {
  float ss = 0.f;
  if (n % 4 == 0) {
    for (int i = 4 * threadIdx.x; i < n; i += 4 * blockDim.x) {
      const float4 v = split_sum4(acc, nsplit, long(T) * n, long(t) * n + i);
      *reinterpret_cast<float4*>(&row[i]) = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
  } else {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const float v = split_sum(acc, nsplit, long(T) * n, long(t) * n + i);
      row[i] = v;
      ss += v * v;
    }
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / float(n) + eps);
  for (int i = threadIdx.x; i < n; i += blockDim.x)
    stf<OutT>(out, long(t) * n + i, row[i] * r * ldf<ActT>(gamma, i));
}

// The same normalised row stored as a bf16 pair: hi = bf16(y) in out[t][0, n), lo = bf16(y - hi)
// in out[t][n, 2n) (round to nearest even both), so a bf16 product of hi and of lo carries y to
// about 2^-16 of its value.
template <typename ActT>
__device__ __forceinline__ void rmsnorm_row_pair(int t, int T, int n, int nsplit, const float* __restrict__ acc,
                                                 const ActT* __restrict__ gamma, uint16_t* __restrict__ out,
                                                 float eps, float* row, float* red) {
  // Four values per thread and step (n % 4 == 0), the loads of every split in flight together.
  const int n4 = n >> 2;
  float ss = 0.f;
  for (int i4 = threadIdx.x; i4 < n4; i4 += blockDim.x) {
    const float4 v = split_sum4(acc, nsplit, long(T) * n, long(t) * n + 4 * i4);
    *reinterpret_cast<float4*>(&row[4 * i4]) = v;
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / float(n) + eps);
  uint16_t* hi_row = out + long(t) * 2 * n;
  for (int i4 = threadIdx.x; i4 < n4; i4 += blockDim.x) {
    const float4 v = *reinterpret_cast<const float4*>(&row[4 * i4]);
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float y0 = x[2 * j] * r * ldf<ActT>(gamma, 4 * i4 + 2 * j);
      const float y1 = x[2 * j + 1] * r * ldf<ActT>(gamma, 4 * i4 + 2 * j + 1);
      const uint16_t h0 = f2bf(y0), h1 = f2bf(y1);
      hw[j] = uint32_t(h0) | (uint32_t(h1) << 16);
      lw[j] = uint32_t(f2bf(y0 - bf2f(h0))) | (uint32_t(f2bf(y1 - bf2f(h1))) << 16);
    }
    *reinterpret_cast<uint2*>(hi_row + 4 * i4) = make_uint2(hw[0], hw[1]);
    *reinterpret_cast<uint2*>(hi_row + n + 4 * i4) = make_uint2(lw[0], lw[1]);
  }
}

template <typename ActT, typename OutT>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(int T, int n, int nsplit,
                                                           const float* __restrict__ acc,
                                                           const ActT* __restrict__ gamma,
                                                           OutT* __restrict__ out, float eps) {
  extern __shared__ float row[];
  __shared__ float red[16];
  rmsnorm_row<ActT, OutT>(blockIdx.x, T, n, nsplit, acc, gamma, out, eps, row, red);
}

// Decode: the compress epilogue of the T new tokens (blocks [0, T)) and the RMSNorm of their
// query latents (blocks [T, 2T), written as a bf16 hi + lo pair [T][2 nq], which the query
// projection takes as two products) in one launch; the two read disjoint partials.
template <typename ActT, int CACHE>
__global__ __launch_bounds__(256) void decode_rows_kernel(
    int dc, int dr, int T, int nsplit_kv, const float* __restrict__ acc_kv, const ActT* __restrict__ gamma_kv,
    void* __restrict__ cache, float* __restrict__ cache_scale, long num_slots, float eps, RopeParams rp,
    float* __restrict__ rope_tab, const int32_t* __restrict__ ctx, const int32_t* __restrict__ bt, int max_blocks,
    int nq, int nsplit_q, const float* __restrict__ acc_q, const ActT* __restrict__ gamma_q, uint16_t* __restrict__ cq) {
  extern __shared__ float row[];                    // [max(dc + dr, nq)]
  __shared__ float red[16];
  const int t = blockIdx.x;
  if (t < T)
    compress_row<ActT, CACHE>(t, dc, dr, T, nsplit_kv, acc_kv, gamma_kv, nullptr, nullptr, cache, cache_scale,
                              num_slots, eps, rp, rope_tab, ctx, bt, max_blocks, row, red);
  else
    rmsnorm_row_pair<ActT>(t - T, T, nq, nsplit_q, acc_q, gamma_q, cq, eps, row, red);
}

bool launch_decode_rows(int act, int cache, int T, int dc, int dr, int nsplit_kv, const float* acc_kv,
                        const void* gamma_kv, void* cache_data, float* cache_scale, long num_slots, float eps,
                        const RopeParams& rp, float* rope_tab, const int32_t* ctx, const int32_t* bt, int max_blocks,
                        int nq, int nsplit_q, const float* acc_q, const void* gamma_q, void* cq, hipStream_t st) {
  if (T <= 0 || act != K_BF16 || (cache != K_BF16 && cache != K_FP8) || !ctx || !rope_tab || nq % 4 != 0)
    return false;
  const size_t sh = size_t(max(dc + dr, nq)) * sizeof(float);
#define MLA_DR(C)                                                                                     \
  hipLaunchKernelGGL((decode_rows_kernel<uint16_t, C>), dim3(2 * T), dim3(256), sh, st, dc, dr, T, nsplit_kv, \
                     acc_kv, static_cast<const uint16_t*>(gamma_kv), cache_data, cache_scale, num_slots, eps, \
                     rp, rope_tab, ctx, bt, max_blocks, nq, nsplit_q, acc_q,                        \
                     static_cast<const uint16_t*>(gamma_q), static_cast<uint16_t*>(cq))
  if (cache == K_BF16)
    MLA_DR(K_BF16);
  else
    MLA_DR(K_FP8);
#undef MLA_DR
  return true;
}

void launch_rmsnorm_rows(int act, int T, int n, int nsplit, const float* acc, const void* gamma,
                         void* out, float eps, hipStream_t st, bool out_f16) {
  if (T <= 0) return;
  size_t sh = size_t(n) * sizeof(float);
  if (act == K_F32)
    hipLaunchKernelGGL((rmsnorm_rows_kernel<float, float>), dim3(T), dim3(256), sh, st, T, n, nsplit, acc,
                       static_cast<const float*>(gamma), static_cast<float*>(out), eps);
  else if (out_f16)
    hipLaunchKernelGGL((rmsnorm_rows_kernel<uint16_t, F16Out>), dim3(T), dim3(256), sh, st, T, n, nsplit, acc,
                       static_cast<const uint16_t*>(gamma), static_cast<F16Out*>(out), eps);
  else
    hipLaunchKernelGGL((rmsnorm_rows_kernel<uint16_t, uint16_t>), dim3(T), dim3(256), sh, st, T, n, nsplit, acc,
                       static_cast<const uint16_t*>(gamma), static_cast<uint16_t*>(out), eps);
}

// bf16 -> fp16 copy (saturating at +-65504; exact for magnitudes in [2^-14, 65504]).
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                          long n8) {
  for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n8; i += long(gridDim.x) * 256) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = uint32_t(f2h_sat(__uint_as_float(w[j] << 16))) | (uint32_t(f2h_sat(__uint_as_float(w[j] & 0xFFFF0000u))) << 16);
    reinterpret_cast<uint4*>(dst)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

void launch_bf16_to_f16(const void* src, void* dst, long n, hipStream_t st) {
  if (n <= 0) return;
  const long n8 = n / 8;
  const long blocks = std::min<long>((n8 + 255) / 256, 8192);
  hipLaunchKernelGGL(bf16_to_f16_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<const uint16_t*>(src),
                     static_cast<uint16_t*>(dst), n8);
}

// ------------------------------------------------------------------ query packing
// Block per (token, group of kQH heads): the RoPE angles of the token's position are formed
// once per block (fp64 phase) in shared memory; threads then loop over the group's values.
// ACT is the absorbed outputs' storage, QS the explicit output's.
constexpr int kQH = 4;

template <int ACT, int QS>
__global__ __launch_bounds__(256) void q_pack_kernel(bool absorbed, int T, int H, int dn, int dr, int dc,
                                                     int nsplit, const float* __restrict__ q_acc,
                                                     const int32_t* __restrict__ pos, float scale, RopeParams rp,
                                                     typename StoreT<ACT>::type* __restrict__ qnope,
                                                     typename StoreT<ACT>::type* __restrict__ qhat,
                                                     typename StoreT<QS>::type* __restrict__ qs) {
  extern __shared__ float cs[];                      // [dr/2] cos | [dr/2] sin
  const int t = blockIdx.x, h_lo = blockIdx.y * kQH;
  const int dqk = dn + dr, half = dr / 2;
  const long nq = long(H) * dqk;
  const int per_head = dn + half;
  const int nh = min(kQH, H - h_lo);
  for (int i = threadIdx.x; i < half; i += blockDim.x) rope_cs(pos[t], i, dr, rp, &cs[i], &cs[half + i]);
  __syncthreads();
  auto q_at = [&](long j) -> float { return split_sum(q_acc, nsplit, long(T) * nq, long(t) * nq + j); };
  for (int e = threadIdx.x; e < nh * per_head; e += blockDim.x) {
    const int h = h_lo + e / per_head, i = e % per_head;
    const long base = long(h) * dqk;
    if (i < dn) {
      float v = scale * q_at(base + i);
      if (absorbed) sts_<ACT>(qnope, (long(t) * H + h) * dn + i, v);
      else sts_<QS>(qs, (long(t) * H + h) * dqk + i, v);
    } else {
      const int pi = i - dn;
      const float c = cs[pi], sn = cs[half + pi];
      float ev = q_at(base + dn + 2 * pi), ov = q_at(base + dn + 2 * pi + 1);
      float re = scale * (ev * c - ov * sn), ro = scale * (ev * sn + ov * c);
      if (absorbed) {
        long o = (long(t) * H + h) * (dc + dr) + dc + 2 * pi;
        sts_<ACT>(qhat, o, re);
        sts_<ACT>(qhat, o + 1, ro);
      } else {
        long o = (long(t) * H + h) * dqk + dn + 2 * pi;
        sts_<QS>(qs, o, re);
        sts_<QS>(qs, o + 1, ro);
      }
    }
  }
}

void launch_q_pack(int act, int qs_type, bool absorbed, int T, int H, int dn, int dr, int dc, int nsplit,
                   const float* q_acc, const int32_t* pos, float scale, const RopeParams& rp, void* qnope, void* qhat,
                   void* qs, hipStream_t st) {
  if (T <= 0) return;
  dim3 grid(T, (H + kQH - 1) / kQH);
  size_t sh = size_t(dr) * sizeof(float);
  if (act == K_F32)
    hipLaunchKernelGGL((q_pack_kernel<S_F32, S_F32>), grid, dim3(256), sh, st, absorbed, T, H, dn, dr, dc,
                       nsplit, q_acc, pos, scale, rp, static_cast<float*>(qnope), static_cast<float*>(qhat),
                       static_cast<float*>(qs));
  else if (qs_type == K_F16)
    hipLaunchKernelGGL((q_pack_kernel<S_BF16, S_F16>), grid, dim3(256), sh, st, absorbed, T, H, dn, dr, dc,
                       nsplit, q_acc, pos, scale, rp, static_cast<uint16_t*>(qnope),
                       static_cast<uint16_t*>(qhat), static_cast<uint16_t*>(qs));
  else
    hipLaunchKernelGGL((q_pack_kernel<S_BF16, S_BF16>), grid, dim3(256), sh, st, absorbed, T, H, dn, dr, dc,
                       nsplit, q_acc, pos, scale, rp, static_cast<uint16_t*>(qnope),
                       static_cast<uint16_t*>(qhat), static_cast<uint16_t*>(qs));
}

// In-place RoPE of the q_pe part of fp16 queries (the projection already wrote them scaled).
// Block per token; the token's angles are formed once in shared memory.
__global__ __launch_bounds__(256) void q_rope_f16_kernel(int H, int dn, int dr, const int32_t* __restrict__ pos,
                                                         RopeParams rp, uint16_t* __restrict__ qs) {
  extern __shared__ float cs[];
  const int t = blockIdx.x, half = dr / 2, dqk = dn + dr;
  for (int i = threadIdx.x; i < half; i += blockDim.x) rope_cs(pos[t], i, dr, rp, &cs[i], &cs[half + i]);
  __syncthreads();
  if ((dn | dr) % 8 == 0) {                        // 16-byte pieces: four pairs per thread
    const int pieces = dr / 8;
    for (int e = threadIdx.x; e < H * pieces; e += blockDim.x) {
      const int h = e / pieces, pc = e % pieces;
      uint4* q = reinterpret_cast<uint4*>(qs + (long(t) * H + h) * dqk + dn + 8 * pc);
      uint4 v = *q;
      uint16_t* x = reinterpret_cast<uint16_t*>(&v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pi = 4 * pc + j;
        const float c = cs[pi], s = cs[half + pi];
        const float ev = h2f(x[2 * j]), ov = h2f(x[2 * j + 1]);
        x[2 * j] = f2h(ev * c - ov * s);
        x[2 * j + 1] = f2h(ev * s + ov * c);
      }
      *q = v;
    }
    return;
  }
  for (int e = threadIdx.x; e < H * half; e += blockDim.x) {
    const int h = e / half, pi = e % half;
    const float c = cs[pi], s = cs[half + pi];
    uint16_t* q = qs + (long(t) * H + h) * dqk + dn + 2 * pi;
    float ev = h2f(q[0]), ov = h2f(q[1]);
    q[0] = f2h(ev * c - ov * s);
    q[1] = f2h(ev * s + ov * c);
  }
}

void launch_q_rope_f16(int T, int H, int dn, int dr, const int32_t* pos, const RopeParams& rp, void* qs,
                       hipStream_t st) {
  if (T <= 0) return;
  hipLaunchKernelGGL(q_rope_f16_kernel, dim3(T), dim3(256), size_t(dr) * sizeof(float), st, H, dn, dr, pos, rp,
                     static_cast<uint16_t*>(qs));
}

// ------------------------------------------------------------------ positions and slots
__global__ void decode_prep_kernel(int B, const int32_t* __restrict__ ctx, const int32_t* __restrict__ bt,
                                   int max_blocks, int32_t* __restrict__ pos, int64_t* __restrict__ slot) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int p = ctx[b] - 1;
  int page = p >= 0 ? p / kPage : -1;
  pos[b] = p > 0 ? p : 0;
  slot[b] = (page >= 0 && page < max_blocks) ? int64_t(bt[long(b) * max_blocks + page]) * kPage + p % kPage : -1;
}

void launch_decode_prep(int B, const int32_t* ctx, const int32_t* bt, int max_blocks, int32_t* pos,
                        int64_t* slot, hipStream_t st) {
  hipLaunchKernelGGL(decode_prep_kernel, dim3((B + 255) / 256), dim3(256), 0, st, B, ctx, bt, max_blocks,
                     pos, slot);
}

__global__ void prefill_prep_kernel(const int32_t* __restrict__ cu, const int32_t* __restrict__ start,
                                    const int32_t* __restrict__ bt, int max_blocks,
                                    int32_t* __restrict__ pos, int64_t* __restrict__ slot) {
  const int s = blockIdx.y, i = blockIdx.x * blockDim.x + threadIdx.x;
  const int t = cu[s] + i;
  if (t >= cu[s + 1]) return;
  const int p = start[s] + i;
  const int page = p / kPage;
  pos[t] = p;
  slot[t] = (p >= 0 && page < max_blocks) ? int64_t(bt[long(s) * max_blocks + page]) * kPage + p % kPage : -1;
}

void launch_prefill_prep(int S, int max_q, const int32_t* cu, const int32_t* start, const int32_t* bt,
                         int max_blocks, int32_t* pos, int64_t* slot, hipStream_t st) {
  hipLaunchKernelGGL(prefill_prep_kernel, dim3((max_q + 255) / 256, S), dim3(256), 0, st, cu, start, bt,
                     max_blocks, pos, slot);
}

// ------------------------------------------------------------------ split-K merge
// For each (b, h): m = max_j m_j, w_j = 2^(m_j - m), otilde = sum_j w_j o_j / sum_j w_j l_j.
// Partial states use base-2 exponents (scores carry a log2 e factor).  Empty splits have
// m_j = -inf and l_j = 0 and weigh nothing.
// (The fp32 path's merge, fp32 throughout.)
__global__ __launch_bounds__(256) void decode_merge_kernel(int H, int dc, int splits,
                                                           const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           float* __restrict__ otilde) {
  extern __shared__ float wts[];                    // [splits] normalised split weights
  __shared__ float red[16];
  const int h = blockIdx.x, b = blockIdx.y;
  float m = -INFINITY;
  for (int s = threadIdx.x; s < splits; s += blockDim.x) m = fmaxf(m, part_ml[((long(b) * splits + s) * H + h) * 2]);
  m = block_max(m, red);
  float l = 0.f;
  for (int s = threadIdx.x; s < splits; s += blockDim.x) {
    const float* ml = part_ml + ((long(b) * splits + s) * H + h) * 2;
    const float w = ml[0] == -INFINITY ? 0.f : exp2f(ml[0] - m);
    wts[s] = w;
    l += w * ml[1];
  }
  l = block_sum(l, red);                            // also orders the wts writes before the reads
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const long stride = long(H) * dc;                 // between consecutive splits of one (b, h)
  const float* po = part_o + (long(b) * splits * H + h) * dc;
  for (int c = threadIdx.x; c < dc; c += blockDim.x) {
    float v = 0.f;
    int s = 0;
    for (; s + 4 <= splits; s += 4) {
      float x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = po[(s + j) * stride + c];
#pragma unroll
      for (int j = 0; j < 4; ++j) v += wts[s + j] * x[j];
    }
    for (; s < splits; ++s) v += wts[s] * po[s * stride + c];
    otilde[(long(b) * H + h) * dc + c] = v * inv;
  }
}

// The same merge for many splits ahead of the fused merge + W_UV kernel, fp32 out: otilde[b][h]
// (dc % 4 == 0) and ml1[b][h] = (0, 1), the state of one already-normalised split.  A work-group
// of 128 threads per (b, h) reads four columns per thread and eight splits per step, so the
// partials of every split are in flight together.
__global__ __launch_bounds__(128) void merge_splits_kernel(int H, int dc, int splits, const uint16_t* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           float* __restrict__ otilde, float* __restrict__ ml1) {
  extern __shared__ float wts[];                    // [splits] normalised split weights
  __shared__ float red[16];
  const int h = blockIdx.x, b = blockIdx.y;
  float m = -INFINITY;
  for (int s = threadIdx.x; s < splits; s += blockDim.x) m = fmaxf(m, part_ml[((long(b) * splits + s) * H + h) * 2]);
  m = block_max(m, red);
  float l = 0.f;
  for (int s = threadIdx.x; s < splits; s += blockDim.x) {
    const float* ml = part_ml + ((long(b) * splits + s) * H + h) * 2;
    const float w = ml[0] == -INFINITY ? 0.f : exp2f(ml[0] - m);
    wts[s] = w;
    l += w * ml[1];
  }
  l = block_sum(l, red);                            // also orders the wts writes before the reads
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const long stride = long(H) * dc;                 // between consecutive splits of one (b, h)
  const uint16_t* po = part_o + (long(b) * splits * H + h) * dc;
  auto load4 = [&](long i) {                        // four fp16 partials as floats
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    const f16x4_t u = *reinterpret_cast<const f16x4_t*>(po + i);
    return make_float4(float(u[0]), float(u[1]), float(u[2]), float(u[3]));
  };
  for (int c = 4 * threadIdx.x; c < dc; c += 4 * blockDim.x) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = 0;
    for (; s + 8 <= splits; s += 8) {
      float4 x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = load4((s + j) * stride + c);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float w = wts[s + j];
        v.x += w * x[j].x; v.y += w * x[j].y; v.z += w * x[j].z; v.w += w * x[j].w;
      }
    }
    for (; s < splits; ++s) {
      const float4 x = load4(s * stride + c);
      const float w = wts[s];
      v.x += w * x.x; v.y += w * x.y; v.z += w * x.z; v.w += w * x.w;
    }
    *reinterpret_cast<float4*>(otilde + (long(b) * H + h) * dc + c) =
        make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
  }
  if (threadIdx.x == 0) {
    ml1[(long(b) * H + h) * 2] = 0.f;
    ml1[(long(b) * H + h) * 2 + 1] = 1.f;
  }
}

void launch_merge_splits(int B, int H, int dc, int splits, const uint16_t* part_o, const float* part_ml,
                         float* otilde, float* ml1, hipStream_t st) {
  hipLaunchKernelGGL(merge_splits_kernel, dim3(H, B), dim3(128), size_t(splits) * 4, st, H, dc, splits, part_o,
                     part_ml, otilde, ml1);
}

void launch_decode_merge(int B, int H, int dc, int splits, const float* part_o, const float* part_ml,
                         float* otilde, hipStream_t st) {
  hipLaunchKernelGGL(decode_merge_kernel, dim3(H, B), dim3(256), size_t(splits) * 4, st, H, dc, splits, part_o,
                     part_ml, otilde);
}

// ------------------------------------------------------------------ prefill gather
// lat[s][r][:] = cache row of position k0 + r of sequence s (one key block of kb rows per
// sequence), zero past the sequence's context.  bf16 / fp32 caches: the stored values.  fp8
// cache: the codes' values (exact in bf16), with the token's scale in tscale[s][r] (1 past the
// context), which the decompression applies in fp32.  kpe16 (bf16 path) gets the k_pe part
// (columns [dc, W)) as fp16: the stored value, or scale * code rounded once.
template <typename ActT, int CACHE>
__global__ __launch_bounds__(256) void gather_rows_kernel(int k0, int kb, int W, int dc, const int32_t* __restrict__ cu,
                                                          const int32_t* __restrict__ start,
                                                          const int32_t* __restrict__ bt, int max_blocks,
                                                          const void* __restrict__ cache,
                                                          const float* __restrict__ cache_scale,
                                                          ActT* __restrict__ lat, uint16_t* __restrict__ kpe16,
                                                          float* __restrict__ tscale) {
  const int s = blockIdx.y, t = k0 + blockIdx.x;     // position t, row blockIdx.x of the block
  const int ctx = start[s] + (cu[s + 1] - cu[s]);
  const long row = long(s) * kb + blockIdx.x;
  ActT* dst = lat + row * W;
  uint16_t* pe = kpe16 ? kpe16 + row * (W - dc) : nullptr;          // pe[i - dc], i in [dc, W)
  if (t >= ctx) {
    for (int i = threadIdx.x; i < W; i += blockDim.x) {
      stf<ActT>(dst, i, 0.f);
      if (pe && i >= dc) pe[i - dc] = f2h(0.f);
    }
    if (CACHE == K_FP8 && threadIdx.x == 0) tscale[row] = 1.f;
    return;
  }
  const long slot = long(bt[long(s) * max_blocks + t / kPage]) * kPage + t % kPage;
  const float sc = CACHE == K_FP8 ? cache_scale[slot] : 1.f;
  if (CACHE == K_FP8 && threadIdx.x == 0) tscale[row] = sc;
  for (int i = threadIdx.x; i < W; i += blockDim.x) {
    float v;
    if (CACHE == K_F32) v = static_cast<const float*>(cache)[slot * W + i];
    else if (CACHE == K_BF16) v = bf2f(static_cast<const uint16_t*>(cache)[slot * W + i]);
    else v = e4m3_to_f(static_cast<const uint8_t*>(cache)[slot * W + i]);
    stf<ActT>(dst, i, v);
    if (pe && i >= dc) pe[i - dc] = f2h_sat(sc * v);
  }
}

void launch_gather_rows(int act, int cache, int S, int k0, int rows, int kb, int W, int dc, const int32_t* cu,
                        const int32_t* start, const int32_t* bt, int max_blocks, const void* cache_data,
                        const float* cache_scale, void* lat, void* kpe16, float* tscale, hipStream_t st) {
  dim3 grid(rows, S);
#define MLA_GR(A, C)                                                                                   \
  hipLaunchKernelGGL((gather_rows_kernel<A, C>), grid, dim3(256), 0, st, k0, kb, W, dc, cu, start, bt, \
                     max_blocks, cache_data, cache_scale, static_cast<A*>(lat), static_cast<uint16_t*>(kpe16), tscale)
  if (act == K_F32) {
    MLA_GR(float, K_F32);
  } else if (cache == K_BF16) {
    MLA_GR(uint16_t, K_BF16);
  } else {
    MLA_GR(uint16_t, K_FP8);
  }
#undef MLA_GR
}

// ------------------------------------------------------------------ fp8 codec
__global__ __launch_bounds__(256) void fp8_encode_kernel(const float* __restrict__ x, uint8_t* __restrict__ codes,
                                                         long n) {
  for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n; i += long(gridDim.x) * 256)
    codes[i] = uint8_t(f_to_e4m3(x[i]));
}
__global__ __launch_bounds__(256) void fp8_decode_kernel(const uint8_t* __restrict__ codes, float* __restrict__ x,
                                                         long n) {
  for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n; i += long(gridDim.x) * 256)
    x[i] = e4m3_to_f(codes[i]);
}

// ------------------------------------------------------------------ K-split sum
// out[i] = sum over s of acc[s * n + i], i < n, stored as OutT.
template <typename OutT>
__global__ __launch_bounds__(256) void sum_splits_kernel(long n, int nsplit, const float* __restrict__ acc,
                                                         OutT* __restrict__ out) {
  for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n; i += long(gridDim.x) * 256) {
    float t = acc[i];
    for (int s = 1; s < nsplit; ++s) t += acc[long(s) * n + i];
    stf<OutT>(out, i, t);
  }
}

// The same sum, four values per thread, with every split's loads requested before the first add
// (a loop over a run-time split count would wait for each load in turn); splits added in order.
template <typename OutT, int MAXS>
__global__ __launch_bounds__(256) void sum_splits4_kernel(long n4, int nsplit, const float4* __restrict__ acc,
                                                          OutT* __restrict__ out) {
  for (long i = long(blockIdx.x) * 256 + threadIdx.x; i < n4; i += long(gridDim.x) * 256) {
    float4 v[MAXS];
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
      if (s < nsplit) v[s] = acc[long(s) * n4 + i];
    float4 t = v[0];
#pragma unroll
    for (int s = 1; s < MAXS; ++s)
      if (s < nsplit) {
        t.x += v[s].x;
        t.y += v[s].y;
        t.z += v[s].z;
        t.w += v[s].w;
      }
    if constexpr (std::is_same<OutT, float>::value) {
      reinterpret_cast<float4*>(out)[i] = t;
    } else {
      reinterpret_cast<uint2*>(out)[i] = make_uint2(uint32_t(f2bf(t.x)) | (uint32_t(f2bf(t.y)) << 16),
                                                    uint32_t(f2bf(t.z)) | (uint32_t(f2bf(t.w)) << 16));
    }
  }
}

void launch_sum_splits(int out_type, long n, int nsplit, const float* acc, void* out, hipStream_t st) {
  if (n <= 0) return;
  const uintptr_t oal = out_type == K_BF16 ? 7 : 15;   // one 8- or 16-byte store per thread
  if (n % 4 == 0 && nsplit >= 1 && nsplit <= 16 && (reinterpret_cast<uintptr_t>(acc) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(out) & oal) == 0) {
    const long n4 = n / 4;
    const long blocks = std::min<long>((n4 + 255) / 256, 2048);
    const float4* a4 = reinterpret_cast<const float4*>(acc);
#define MLA_SS4(MAXS)                                                                                 \
    if (out_type == K_BF16)                                                                           \
      hipLaunchKernelGGL((sum_splits4_kernel<uint16_t, MAXS>), dim3(unsigned(blocks)), dim3(256), 0, st, n4,     \
                         nsplit, a4, static_cast<uint16_t*>(out));                                    \
    else                                                                                              \
      hipLaunchKernelGGL((sum_splits4_kernel<float, MAXS>), dim3(unsigned(blocks)), dim3(256), 0, st, n4, nsplit, \
                         a4, static_cast<float*>(out))
    if (nsplit <= 4) { MLA_SS4(4); }
    else if (nsplit <= 8) { MLA_SS4(8); }
    else { MLA_SS4(16); }
#undef MLA_SS4
    return;
  }
  const long blocks = std::min<long>((n + 255) / 256, 2048);
  if (out_type == K_BF16)
    hipLaunchKernelGGL(sum_splits_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(256), 0, st, n, nsplit, acc,
                       static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(sum_splits_kernel<float>, dim3(unsigned(blocks)), dim3(256), 0, st, n, nsplit, acc,
                       static_cast<float*>(out));
}

// The query projection's K-split partials acc [nsplit][T][H][192] summed once (split order) into
// the layout of the projection's split epilogue: q_nope32 [T][H][128] = alpha q_nope and
// q_pe32 [T][H][64] = q_pe (fp32), so the absorb reads each query once.  Four values per thread;
// `part` of `parts` work-groups take a grid-stride share.
__global__ __launch_bounds__(256) void q_split_sum_kernel(QSumArgs q) {
  q_split_sum_part(q, blockIdx.x, gridDim.x);
}

void launch_q_split_sum(int T, int H, int nsplit, const float* acc, float alpha, float* q_nope32, float* q_pe32,
                        hipStream_t st) {
  QSumArgs q;
  q.n4 = long(T) * H * 192 / 4;
  if (q.n4 <= 0) return;
  q.nsplit = nsplit;
  q.acc = acc;
  q.stride = long(T) * H * 192;
  q.alpha = alpha;
  q.q_nope32 = q_nope32;
  q.q_pe32 = q_pe32;
  const long blocks = std::min<long>((q.n4 + 255) / 256, 1024);
  hipLaunchKernelGGL(q_split_sum_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, q);
}

// ------------------------------------------------------------------ stream-read reference
// Reads n16 16-byte words once (grid-stride, four loads in flight per lane) and keeps only an
// XOR of them, so the kernel's time is that of reading the bytes from memory.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ p, long n16, uint32_t* sink) {
  uint32_t acc = 0;
  const long stride = long(gridDim.x) * 256;
  long i = long(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^ (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) acc ^= p[i].x ^ p[i].y ^ p[i].z ^ p[i].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;           // keeps the loads; almost never stores
}

// The same read through direct global->LDS loads with the non-temporal hint, the fastest read
// pattern measured on gfx950: every wave streams its own contiguous part of the buffer in steps
// of 4 KiB (4 loads of 1 KiB) through its own ring of 8 steps in LDS, six steps in flight, and
// folds each step back out of LDS (its lanes read what their own loads wrote, so no barrier) into
// the same XOR as above; words past the end are fetched from the part's first word and not
// folded in.
constexpr int kSrRing = 8, kSrStep = 4096;
__global__ __launch_bounds__(256) void stream_read_lds_kernel(const char* __restrict__ p, long n16, long per16,
                                                              uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) char ring[4 * kSrRing * kSrStep];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const long w0 = (long(blockIdx.x) * 4 + wave) * per16;       // this wave's first 16-byte word
  if (w0 >= n16) return;                                        // (uniform over the wave)
  const long w1 = min(n16, w0 + per16);
  const int steps = int((w1 - w0 + 255) / 256);
  const char* base = p + w0 * 16;
  char* mine = ring + wave * kSrRing * kSrStep;
  uint32_t acc = 0;
  auto fold = [&](int s) {                                      // step s has landed in its slot
    const char* slot = mine + (s % kSrRing) * kSrStep;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long w = w0 + long(s) * 256 + 64 * k + lane;
      const uint4 v = *reinterpret_cast<const uint4*>(slot + k * 1024 + 16 * lane);
      if (w < w1) acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  };
  for (int s = 0; s < steps; ++s) {
    char* slot = mine + (s % kSrRing) * kSrStep;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long w = long(s) * 256 + 64 * k + lane;             // relative to w0
      const uint32_t off = uint32_t(w0 + w < w1 ? w * 16 : 0);
      const uint32_t l = lds::addr(slot + k * 1024);
      asm volatile("global_load_lds_dwordx4 %0, %1 nt" : : "v"(off), "s"(base), "{m0}"(l) : "memory");
    }
    if (s >= kSrRing - 2) {
      lds::wait_vm<4 * (kSrRing - 2)>();
      fold(s - (kSrRing - 2));
    }
  }
  lds::wait_vm<0>();
  for (int s = max(0, steps - (kSrRing - 2)); s < steps; ++s) fold(s);
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

void launch_stream_read(const void* p, long n16, uint32_t* sink, int mode, hipStream_t st) {
  if (n16 <= 0) return;
  if (mode == 0) {
    hipLaunchKernelGGL(stream_read_kernel, dim3(1024), dim3(256), 0, st, static_cast<const uint4*>(p), n16, sink);
    return;
  }
  // 256 work-groups of 4 waves, each wave a part of whole 4 KiB steps
  const long per16 = ((n16 + 1023) / 1024 + 255) & ~255L;
  hipLaunchKernelGGL(stream_read_lds_kernel, dim3(256), dim3(256), 0, st, static_cast<const char*>(p), n16, per16, sink);
}

void launch_fp8_codec(bool encode, const void* in, void* out, long n, hipStream_t st) {
  if (n <= 0) return;
  const long blocks = std::min<long>((n + 255) / 256, 4096);
  if (encode)
    hipLaunchKernelGGL(fp8_encode_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<const float*>(in),
                       static_cast<uint8_t*>(out), n);
  else
    hipLaunchKernelGGL(fp8_decode_kernel, dim3(unsigned(blocks)), dim3(256), 0, st, static_cast<const uint8_t*>(in),
                       static_cast<float*>(out), n);
}

}  // namespace mla
