// Causal prefill attention over decompressed keys and values (the explicit flow), bf16 path,
// head dims nope 128, rope 64, v 128.
//
// One work-group of 4 waves per (query tile of 128, head, sequence); wave w owns queries
// [32w, 32w + 32) of the tile.  Keys and values stream through LDS in tiles of 64 keys (k_nope
// 16 KiB | k_pe 8 KiB | v 16 KiB), double-buffered with direct global->LDS loads, so two
// work-groups (80 KiB each) share a CU.  Per tile and wave:
//   S^T[key][query] = K . Q^T with v_mfma_f32_32x32x16_f16 (k_nope from the decompression, k_pe
//   from an fp16 copy the gather writes, the query in registers: 12 K steps per 32-key sub-tile);
//   online softmax per query in base 2 (queries are pre-scaled by sigma * log2 e), with the
//   running max moved only when a tile's max passes it by more than kLazy (p <= 2^kLazy, far
//   inside fp16), so the output accumulators are rescaled only then;
//   O^T[v][query] += V^T . P^T with v_mfma_f32_32x32x16_f16, P taken straight from the score
//   accumulators: in the 32x32 C layout a lane holds keys {0-3, 8-11, 16-19, 24-27} (+4 for
//   lanes 32-63) of one query, which is the B operand of the value product when its K order
//   lists keys that way; the transposing LDS reads of V^T (ds_read_b64_tr_b16, four key rows per
//   read) fetch the same key order.
// LDS rows are swizzled per 16-byte chunk: k_nope chunk c of key r at c ^ (r & 15) (256-byte
// rows), k_pe at c ^ ((r >> 1) & 7) (128-byte rows), v at c ^ (2 (r & 7)); the direct loads place
// every chunk where the operand reads expect it (a load instruction fills one contiguous KiB).
// The query tiles of one (head, sequence) run back to back on one XCD, heaviest (latest in the
// chunk, most keys) first, so their key and value reads are shared through that XCD's L2.
// Long contexts are decompressed in key blocks (positions [k0, k0 + kb)); one launch per block
// continues the online softmax from the state the previous block saved (the unnormalised output,
// the running max and the row sum per query and head), and the last one normalises.
#include "mla_device.h"
#include "mla_kernels.h"
#include "mla_lds.h"

namespace mla {

namespace {

constexpr int kQT = 128;                       // queries per work-group
constexpr int kKT = 64;                        // keys per tile
constexpr int kNopeOff = 0, kPeOff = 16384, kVOff = 24576, kTileBytes = 40960;
constexpr int kLoadsPerWave = 10;              // 40 one-KiB loads per tile over 4 waves
constexpr float kLazy = 8.0f;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

using lds::barrier;
using lds::dma16;
using lds::wait_vm;
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return lds::addr(p); }

__device__ __forceinline__ s16x4_t tr_read(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_t __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ f16x8_t join_f16(s16x4_t lo, s16x4_t hi) {
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(f16x8_t, v);
}

// Load k of wave w: instruction i = w + 4k of the tile.  Returns the byte offset, relative to
// the tile's base (kv for k_nope and v, the fp16 k_pe copy for k_pe), of the 16 bytes lane `lane`
// fetches, rows at or beyond `valid` re-reading row valid - 1; `row_bytes` is H * 512 (one key's
// k_nope | v of all heads).
__device__ __forceinline__ uint32_t load_offset(int k, int wave, int lane, int valid, uint32_t row_bytes) {
  const int i = wave + 4 * k;
  int row, c;
  uint32_t extra = 0, stride = row_bytes;
  if (i < 16) {                                // k_nope: 4 rows of 256 B per KiB
    row = 4 * i + (lane >> 4);
    c = (lane & 15) ^ (row & 15);
  } else if (i < 24) {                         // k_pe: 8 rows of 128 B per KiB
    row = 8 * (i - 16) + (lane >> 3);
    c = (lane & 7) ^ ((row >> 1) & 7);
    stride = 128;
  } else {                                     // v: 4 rows of 256 B per KiB
    row = 4 * (i - 24) + (lane >> 4);
    c = (lane & 15) ^ (2 * (row & 7));
    extra = 256;
  }
  const int rs = row < valid ? row : valid - 1;
  return uint32_t(rs) * stride + extra + 16u * uint32_t(c);
}

__device__ __forceinline__ int load_lds_offset(int k, int wave) {
  const int i = wave + 4 * k;
  return i < 16 ? i * 1024 : (i < 24 ? kPeOff + (i - 16) * 1024 : kVOff + (i - 24) * 1024);
}

}  // namespace

template <int OUT>
__global__ __launch_bounds__(256, 2) void prefill_attn_fa_kernel(
    int H, int S, int nqt, int k0, int kb, const int32_t* __restrict__ cu, const int32_t* __restrict__ start,
    const uint16_t* __restrict__ qs, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ kpe,
    typename StoreT<OUT>::type* __restrict__ out, const float* __restrict__ state_in, float* __restrict__ state_out) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work-groups are dealt to the 8 XCDs round-robin: (head, sequence) pair P runs on XCD P % 8,
  // its nqt query tiles one after another there (heaviest first), so they stream the same keys
  // and values at about the same time and all but the first read of each tile hit that XCD's L2.
  // The pair count is padded to a multiple of 8 by work-groups that leave at once.
  const int L = blockIdx.x;
  const int t = L >> 3, g = t / nqt, j = t - g * nqt;
  const int P = 8 * g + (L & 7);
  if (P >= H * S) return;
  const int qt = nqt - 1 - j;
  const int h = P % H, s = P / H;
  const int q_begin = cu[s], len = cu[s + 1] - q_begin, st0 = start[s];
  if (qt * kQT >= len) return;                     // the whole work-group leaves together
  const int ctx = st0 + len;
  const int key_end = st0 + min(len, (qt + 1) * kQT);   // keys the tile's last query sees
  // This key block: positions [k0, k0 + kb), row t of the buffers holding position k0 + t.
  const int blk_end = min(key_end, k0 + kb);
  const int nt = blk_end > k0 ? (blk_end - k0 + kKT - 1) / kKT : 0;
  const int ctx_rows = min(ctx, k0 + kb) - k0;           // rows of the block inside the context
  const int ql = lane & 31, e = lane >> 5;
  const int qi = qt * kQT + 32 * wave + ql;        // this lane's query (column of S^T)
  const int qpos = st0 + min(qi, len - 1);
  const int wave_qmin = st0 + qt * kQT + 32 * wave;
  const uint32_t row_bytes = uint32_t(H) * 512u;
  const char* kvc = reinterpret_cast<const char*>(kv) + (long(s) * kb * H + h) * 512;
  const char* kpec = reinterpret_cast<const char*>(kpe) + long(s) * kb * 128;

  // Query fragments (B operand): Q[query ql][16 st + 8 e .. +7].
  f16x8_t qn[8], qr[4];
  {
    const _Float16* qp =
        reinterpret_cast<const _Float16*>(qs) + (long(q_begin + min(qi, len - 1)) * H + h) * 192 + 8 * e;
#pragma unroll
    for (int st = 0; st < 8; ++st) qn[st] = *reinterpret_cast<const f16x8_t*>(qp + 16 * st);
#pragma unroll
    for (int st = 0; st < 4; ++st) qr[st] = *reinterpret_cast<const f16x8_t*>(qp + 128 + 16 * st);
  }

  uint32_t full_off[kLoadsPerWave];
#pragma unroll
  for (int k = 0; k < kLoadsPerWave; ++k) full_off[k] = load_offset(k, wave, lane, kKT, row_bytes);
  auto issue = [&](int j) {
    if (j >= nt) return;
    char* dst = smem + (j & 1) * kTileBytes;
    const char* kvb = kvc + long(kKT * j) * row_bytes;
    const char* lb = kpec + long(kKT * j) * 128;
    const int valid = min(kKT, ctx_rows - kKT * j);
    if (valid == kKT) {
#pragma unroll
      for (int k = 0; k < kLoadsPerWave; ++k)
        dma16((k == 4 || k == 5) ? lb : kvb, full_off[k], lds_addr(dst + load_lds_offset(k, wave)));
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int k = 0; k < kLoadsPerWave; ++k)
        dma16((k == 4 || k == 5) ? lb : kvb, load_offset(k, wave, ln, valid, row_bytes),
              lds_addr(dst + load_lds_offset(k, wave)));
    }
  };

  // Operand offsets within a tile.
  const int n_row = ql * 256, n_x = lane & 15;                  // k_nope: row ql (+32 u)
  const int p_row = kPeOff + ql * 128, p_x = (ql >> 1) & 7;      // k_pe
  auto nope_a = [&](const char* t, int u, int st) {
    return *reinterpret_cast<const f16x8_t*>(t + n_row + 8192 * u + 16 * ((2 * st + e) ^ n_x));
  };
  auto pe_a = [&](const char* t, int u, int st) {
    return *reinterpret_cast<const f16x8_t*>(t + p_row + 4096 * u + 16 * ((2 * st + e) ^ p_x));
  };
  // V^T reads: lane i of each 16-lane group supplies key row T + (i >> 2), v column
  // c0 + 4 (i & 3), c0 = 32 vt + 16 ((lane >> 4) & 1); T = 16 q + 4 e (and + 8 for the second read).
  int v_off[4];
  {
    const int i = lane & 15;
    const int r0 = 4 * e + (i >> 2);
    const int gv = 2 * (r0 & 7);
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) {
      const int chunk = 4 * vt + 2 * ((lane >> 4) & 1) + ((i & 3) >> 1);
      v_off[vt] = kVOff + r0 * 256 + 16 * (chunk ^ gv) + 8 * (i & 1);
    }
  }

  f32x16_t o[4];
#pragma unroll
  for (int vt = 0; vt < 4; ++vt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[vt][j] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // The state an earlier key block left (the unnormalised output, the running max and the row
  // sum; the sum goes to the lane of the pair that holds key half 0).
  if (state_in && qi < len) {
    const float* sp = state_in + (long(q_begin + qi) * H + h) * 130;
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int k = 0; k < 16; ++k) o[vt][k] = sp[32 * vt + 8 * (k >> 2) + 4 * e + (k & 3)];
    m_run = sp[128];
    l_run = e == 0 ? sp[129] : 0.f;
  }

  issue(0);
  for (int j = 0; j < nt; ++j) {
    issue(j + 1);
    if (j + 1 < nt) wait_vm<kLoadsPerWave>();
    else wait_vm<0>();
    barrier();                                 // tile j in LDS for every wave
    const char* t = smem + (j & 1) * kTileBytes;
    const int t0 = k0 + kKT * j;                 // position of the tile's first key

    f32x16_t sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int k = 0; k < 16; ++k) sc[u][k] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) sc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(nope_a(t, u, st), qn[st], sc[u], 0, 0, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) sc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pe_a(t, u, st), qr[st], sc[u], 0, 0, 0);

    // Causal mask (only where some key of the tile passes some query of the wave) and the
    // tile max per query (the lane and its partner lane ^ 32 hold the query's 64 keys).
    if (t0 + kKT - 1 > wave_qmin) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int kp = t0 + 32 * u + 8 * (k >> 2) + 4 * e + (k & 3);
          if (kp > qpos) sc[u][k] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int k = 0; k < 16; ++k) mt = fmaxf(mt, sc[u][k]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    if (__any(mt > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) o[vt] *= alpha;
      m_run = m_new;
    }
    // p = 2^(s - m) with the bare v_exp_f32 (arguments at most kLazy; a query with every key
    // masked so far keeps m = -inf and takes 2^(-inf - 0) = 0 for each key)
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    f16x8_t pf[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f16x8_t v;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float p = __builtin_amdgcn_exp2f(sc[u][8 * hf + k] - m_use);
          l_run += p;
          v[k] = (_Float16)p;
        }
        pf[u][hf] = v;
      }
#pragma unroll
    for (int q = 0; q < 4; ++q) {                  // K step q: keys 16 q + {0-3, 8-11} (+4 e)
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) {
        const char* p0 = t + v_off[vt] + 16 * 256 * q;
        const f16x8_t a = join_f16(tr_read(p0), tr_read(p0 + 8 * 256));
        o[vt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[q >> 1][q & 1], o[vt], 0, 0, 0);
      }
    }
    barrier();                                 // tile j's buffer free for tile j + 2
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qi < len && state_out) {                   // more key blocks follow: pass the state on
    float* sp = state_out + (long(q_begin + qi) * H + h) * 130;
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int k = 0; k < 16; ++k) sp[32 * vt + 8 * (k >> 2) + 4 * e + (k & 3)] = o[vt][k];
    if (e == 0) {
      sp[128] = m_run;
      sp[129] = l_tot;
    }
  } else if (qi < len) {
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const long row = (long(q_begin + qi) * H + h) * 128;
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int k = 0; k < 16; ++k)
        sts_<OUT>(out, row + 32 * vt + 8 * (k >> 2) + 4 * e + (k & 3), o[vt][k] * inv);
  }
}

bool launch_prefill_attn_fa(const PrefillAttnArgs& a, hipStream_t st) {
  if (a.dn != 128 || a.dr != 64 || a.dv != 128 || a.dc != 512) return false;
  const int nqt = (a.max_q + kQT - 1) / kQT;
  const dim3 grid(unsigned(8L * nqt * ((long(a.H) * a.S + 7) / 8)));
  if (a.kb <= 0 || a.kb % kKT != 0) return false;
  if (a.out_type == K_BF16)
    hipLaunchKernelGGL(prefill_attn_fa_kernel<S_BF16>, grid, dim3(256), 0, st, a.H, a.S, nqt, a.k0, a.kb, a.cu,
                       a.start, static_cast<const uint16_t*>(a.qs), static_cast<const uint16_t*>(a.kv),
                       static_cast<const uint16_t*>(a.kpe), static_cast<uint16_t*>(a.out), a.state_in, a.state_out);
  else
    hipLaunchKernelGGL(prefill_attn_fa_kernel<S_F32>, grid, dim3(256), 0, st, a.H, a.S, nqt, a.k0, a.kb, a.cu,
                       a.start, static_cast<const uint16_t*>(a.qs), static_cast<const uint16_t*>(a.kv),
                       static_cast<const uint16_t*>(a.kpe), static_cast<float*>(a.out), a.state_in, a.state_out);
  return true;
}

}  // namespace mla
