// Attention dispatch, and the fp32 attention kernels of the generic-shape path (tiny
// configurations): weight-absorbed split-K decode over the latent cache and causal prefill over
// decompressed keys / values, one work-group per (head, split, sequence) or (query, head,
// sequence), SIMT fp32.  The bf16 path's kernels are in k_decode.hip and k_prefill.hip.
#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

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

bool launch_decode_attn(int act, int cache, const DecodeAttnArgs& a, hipStream_t st) {
  if (act == K_F32) {
    size_t sh = size_t(a.dc + a.dr + 256) * sizeof(float) + 256 * sizeof(long);
    hipLaunchKernelGGL(decode_attn_simt_kernel, dim3(a.H, a.splits, a.B), dim3(256), sh, st, a.H, a.dc,
                       a.dr, a.splits, a.max_blocks, static_cast<const float*>(a.qhat),
                       static_cast<const float*>(a.cache), a.block_table, a.ctx, static_cast<float*>(a.part_o),
                       a.part_ml);
    return true;
  }
  return launch_decode_attn_v2(cache, a, st);    // every bf16-path shape (d_c 512, d_r 64, H % 16 == 0)
}

// ==================================================================== prefill, fp32 SIMT
// Generic dims.  Grid (max_q, H, S); one query per block, 256 threads over keys; kv and lat hold
// kb >= max_ctx rows per sequence.
__global__ __launch_bounds__(256) void prefill_attn_simt_kernel(
    int H, int dn, int dr, int dv, int dc, int kb, const int32_t* __restrict__ cu,
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
  const long kvb = long(s) * kb;                    // kv / lat rows of sequence s
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

bool launch_prefill_attn(int act, const PrefillAttnArgs& a, hipStream_t st) {
  if (act == K_F32) {
    // the whole context as one block (kb rows per sequence)
    if (a.k0 != 0 || a.state_in || a.state_out || a.kb < a.max_ctx) return false;
    size_t sh = size_t(a.dn + a.dr + 256) * sizeof(float);
    hipLaunchKernelGGL(prefill_attn_simt_kernel, dim3(a.max_q, a.H, a.S), dim3(256), sh, st, a.H, a.dn,
                       a.dr, a.dv, a.dc, a.kb, a.cu, a.start, static_cast<const float*>(a.qs),
                       static_cast<const float*>(a.kv), static_cast<const float*>(a.lat),
                       static_cast<float*>(a.out));
    return true;
  }
  return launch_prefill_attn_fa(a, st);          // every bf16-path shape (nope 128, rope 64, v 128)
}

}  // namespace mla
