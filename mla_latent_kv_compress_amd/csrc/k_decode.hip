// Split-K decode attention over a bf16 latent cache, 128 heads per work-group (weight-absorbed).
//
// One work-group of 4 waves (one per SIMD) per (sequence, split, 128 heads).  The split's
// cached rows stream through LDS in stages of 32 tokens (32 rows x 576 bf16 = 36 KiB), fetched
// with direct global->LDS loads into a ring of 4 stages, three stages ahead of the one being
// computed.  Per stage:
//   scores    wave w owns heads [32w, 32w+32): S[token][head] = R . Qhat^T with
//             v_mfma_f32_16x16x32_bf16 (2 token tiles x 2 head tiles, 18 K steps), the query
//             slice held in registers for the whole split; online softmax per head in base 2
//             (log2 e is folded into Qhat) with a lazy reference max; P goes to LDS as bf16.
//   values    wave w owns latent columns [128w, 128w+128) for all 128 heads:
//             O^T[c][head] += R^T . P^T with v_mfma_f32_32x32x16_bf16 (4 column tiles x 4 head
//             tiles, 2 K steps of 16 tokens), R^T read with the transposing ds_read_b64_tr_b16.
// The cached latent is also the value, so one LDS stage feeds both products and each cache row
// leaves HBM once per split.  Splitting the value product by columns means every wave reads
// only its quarter of the stage for it (instead of all of it), and the score product's operand
// is shared by 32 heads per read.
//
// LDS: a stage holds rows of 72 16-byte chunks, unpadded (each direct load instruction fills a
// contiguous KiB), with chunk c of row r stored at c ^ rsw(r), rsw(r) < 8 (the XOR stays inside
// an aligned group of 8 chunks, so a load instruction still covers one contiguous KiB of the
// page).  Measured on gfx950, this choice lets the score operand reads (16 rows x 4 chunks per
// instruction) run at the full 128-bit LDS rate, about twice the rate of the unswizzled rows or
// of some other XOR patterns; the transposing reads run at their own (lower) rate whatever the
// pattern.  P is stored [head][token] (64 bytes per head) with the chunk index XORed by
// (head >> 2) & 3, so 16 consecutive heads of one chunk column (the B operand of 16 lanes) are
// conflict-free.  A 128-float buffer carries each head's rescale factor from the wave that owns
// its scores to the waves that own its value columns.
//
// Reference max: each head accumulates p = 2^(s - m) against a reference m fixed after the
// first stage (that stage's max), so the accumulators are never rescaled inside the loop.  Later
// scores may exceed m; p <= 2^kSlack stays far inside bf16 and fp32 range.  If some head's stage
// max exceeds m + kSlack, the work-group drops what it accumulated, makes a scores-only pass over
// the split to find every head's exact max, and accumulates again with that reference (exact,
// and it costs two extra passes only on such splits).  The partial state (m, l, O) is consistent
// for the log-sum-exp merge whatever m is.  Rows of a stage beyond the context re-read the last
// valid row (finite data) and get p = 0.
#include <type_traits>

#include "mla_device.h"
#include "mla_kernels.h"

namespace mla {

namespace {

constexpr int kDC = 512, kDR = 64, kDW = kDC + kDR;
constexpr int kRowBytes = kDW * 2;                    // 1152
constexpr int kPageBytes = kPage * kRowBytes;         // 73728
constexpr int kStage = 32;                            // tokens per pipeline stage
constexpr int kStageBytes = kStage * kRowBytes;       // 36864
constexpr int kRing = 4;
constexpr int kThreads = 256;
constexpr int kLoads = kStageBytes / 16 / kThreads;   // 9 direct loads per thread per stage
constexpr int kKS = kDW / 32;                         // 18 score K steps
constexpr int kHeads = 128;                           // heads per work-group
constexpr int kPBytes = kHeads * kStage * 2;          // 8192
constexpr float kSlack = 64.0f;
constexpr int kChecked = 0, kMaxOnly = 1, kFixed = 2;     // pass kinds

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

// Wait until at most `n` vector-memory operations of this wave are outstanding (n a constant).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF));
}

// Work-group barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding global loads (the ring's prefetches stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One direct global->LDS load: lane i's 16 bytes at base + off land at LDS byte lds + 16 i.
// Written as inline assembly so that the compiler does not track it: its own tracking of such
// loads makes every later LDS read wait for all of them (vmcnt(0)), which would serialise the
// prefetch ring.  Completion is awaited explicitly (wait_vm) before the barrier that publishes a
// stage.  The instruction has no register results; its address operands are read at issue.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(off), "s"(base), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Enqueue the direct loads of one stage: instruction k of wave w fills LDS bytes
// [(4k + w) KiB, +1 KiB) of the stage; lane i supplies stored chunk (4k + w) * 64 + i, i.e. row
// r = chunk / 72, logical chunk (chunk % 72) ^ rsw(r).  Rows at or beyond `valid` re-read row
// valid - 1.  The lane id arrives opaque so the offsets are recomputed per stage (a few integer
// ops) instead of being hoisted into registers for the whole loop.
__device__ __forceinline__ void load_stage(char* dst, const char* src, int valid, int wave, int lane) {
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int k = 0; k < kLoads; ++k) {
    const int idx = (4 * k + wave) * 64 + lane;
    const int r = idx / 72, cp = idx - r * 72;
    const int c = cp ^ rsw(r);
    const int rs = r < valid ? r : valid - 1;
    const uint32_t off = uint32_t(rs * kRowBytes + c * 16);
    dma16(src, off, lds_addr(dst + (4 * k + wave) * 1024));
  }
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void decode_attn_latent_kernel(
    int H, int splits, int max_blocks, int xcd_map, const uint16_t* __restrict__ qhat,
    const uint16_t* __restrict__ cache, const int32_t* __restrict__ bt, const int32_t* __restrict__ ctx_lens,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(1024))) char smem[kRing * kStageBytes + 2 * kPBytes];   // 160 KiB
  char* const ring = smem;
  char* const pbase = smem + kRing * kStageBytes;          // P of stage j in pbase + (j & 1) * kPBytes

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  // Work-group -> (sequence, split).  With xcd_map the splits of one sequence share an XCD
  // (work-groups are dealt to the 8 XCDs round-robin), so its query rows are fetched once per L2.
  int b, sp;
  {
    const int unit = blockIdx.x;
    if (xcd_map) {
      const int k = unit >> 3;
      b = (k / splits) * 8 + (unit & 7);
      sp = k - (k / splits) * splits;
    } else {
      b = unit / splits;
      sp = unit - b * splits;
    }
  }
  const int hbase = blockIdx.y * kHeads;
  const int ctx = ctx_lens[b];
  const int nst = (ctx + kStage - 1) / kStage;
  const int per = (nst + splits - 1) / splits;
  const int s0 = sp * per;
  const int n = max(0, min(nst, s0 + per) - s0);
  const char* cbase = reinterpret_cast<const char*>(cache);
  const int32_t* btab = bt + long(b) * max_blocks;
  auto stage_valid = [&](int j) { return j < n ? min(kStage, ctx - kStage * (s0 + j)) : 0; };
  auto issue = [&](int j) {              // loads of stage j (of this split) into ring slot j % 4
    if (j < n)
      load_stage(ring + (j & 3) * kStageBytes,
                 cbase + long(btab[(s0 + j) >> 1]) * kPageBytes + ((s0 + j) & 1) * kStageBytes, stage_valid(j),
                 wave, lane);
  };
  // Wait until stage j is in LDS, stages up to `last` having been issued (in order).
  auto wait_stage = [&](int j, int last) {
    const int ahead = min(n - 1, last) - j;
    if (ahead >= 2) wait_vm<2 * kLoads>();
    else if (ahead == 1) wait_vm<kLoads>();
    else wait_vm<0>();
  };

  // Query fragments (B operand of the score product): Qhat[head 32w + 16nt + li][32ks + 8g .. +7].
  bf16x8_t qf[2][kKS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const uint16_t* q = qhat + (long(b) * H + hbase + 32 * wave + 16 * nt + li) * kDW + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[nt][ks] = *reinterpret_cast<const bf16x8_t*>(q + 32 * ks);
  }

  // Score operand offsets: row 16 mt + li, logical chunk 4 ks + g, stored at
  // (4 ks + g) ^ rsw(li) = 4 (ks ^ y) + x.
  const int sx = g ^ (rsw(li) & 3), sy = rsw(li) >> 2;
  const int s_even = li * kRowBytes + 16 * sx + 64 * sy;   // ks even: + 64 ks
  const int s_odd = li * kRowBytes + 16 * sx - 64 * sy;    // ks odd:  + 64 ks
  auto score_a = [&](const char* st, int ks, int mt) {
    const int off = ((ks & 1) ? s_odd : s_even) + 64 * ks + mt * 16 * kRowBytes;
    return *reinterpret_cast<const bf16x8_t*>(st + off);
  };
  // Transposing reads for the value product: lane reads row 8 (lane >> 5) + 4 rd + (li >> 2)
  // (+16 per K step), element column 128 w + 32 ct + 16 ((lane >> 4) & 1) + 4 (li & 3).
  int t_even[2], t_odd[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int rr = 8 * (lane >> 5) + 4 * rd + (li >> 2);
    const int gs = rsw(rr);
    const int x = 2 * ((lane >> 4) & 1) + ((li & 3) >> 1);
    const int base = rr * kRowBytes + 256 * wave + 16 * (x ^ (gs & 3)) + 8 * (li & 1);
    t_even[rd] = base + 64 * (gs >> 2);
    t_odd[rd] = base - 64 * (gs >> 2);
  }
  auto val_a = [&](const char* st, int ks, int ct) {
    const int add = 64 * ct + ks * 16 * kRowBytes;
    const char* p0 = st + ((ct & 1) ? t_odd[0] : t_even[0]) + add;
    const char* p1 = st + ((ct & 1) ? t_odd[1] : t_even[1]) + add;
    return join(tr_read(p0), tr_read(p1));
  };
  const int ph = lane & 31;
  // P operand: Pbuf[head 32 nt + ph][tokens 16 ks + 8 (lane >> 5) .. +7].
  auto p_frag = [&](const char* pb, int ks, int nt) {
    const int h = 32 * nt + ph;
    const int c = 2 * ks + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(pb + h * 64 + 16 * (c ^ psw(h)));
  };

  f32x16_t o[4][4];
  float m_ref[2] = {-INFINITY, -INFINITY}, l_run[2];
  f32x4_t s[2][2];

  // Online softmax of the score tile s against the reference; `valid` tokens of the stage are
  // cached.  kChecked: the first stage sets the reference; flags scores beyond it + kSlack.
  auto softmax = [&](auto mode, int valid, uint2 (&pk)[2][2], bool& over) {
    constexpr int kMode = decltype(mode)::value;
    const int lim = valid - 4 * g;      // token 16 mt + 4 g + j is cached iff 16 mt + j < lim
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = (16 * mt + j) < lim ? s[mt][nt][j] : -INFINITY;
          s[mt][nt][j] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (kMode == kMaxOnly) {
        m_ref[nt] = fmaxf(m_ref[nt], mx);
        continue;
      }
      if (kMode == kChecked) {
        if (m_ref[nt] == -INFINITY) m_ref[nt] = mx;      // first stage of the split
        over |= mx > m_ref[nt] + kSlack;
      }
      // (an empty split keeps m = -inf; its masked scores then still give p = 0)
      const float m_use = m_ref[nt] == -INFINITY ? 0.f : m_ref[nt];
      float psum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] = __builtin_amdgcn_exp2f(s[mt][nt][j] - m_use);       // 0 for masked tokens
          psum += p[j];
        }
        pk[mt][nt] = make_uint2(pack_bf2(p[0], p[1]), pack_bf2(p[2], p[3]));
      }
      l_run[nt] += psum;
    }
  };
  auto store_p = [&](char* pb, const uint2 (&pk)[2][2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int h = 32 * wave + 16 * nt + li;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int c = 2 * mt + (g >> 1);
        *reinterpret_cast<uint2*>(pb + h * 64 + 16 * (c ^ psw(h)) + 8 * (g & 1)) = pk[mt][nt];
      }
    }
  };
  auto zero_s = [&]() {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) s[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  };
  // Score tile of one stage, with `extra(ks)` issued after each K step's MFMAs (the value
  // product of the previous stage rides along so the MFMA pipe stays busy).
  auto scores = [&](const char* st, auto extra) {
    zero_s();
    bf16x8_t a[2][2];
    a[0][0] = score_a(st, 0, 0);
    a[0][1] = score_a(st, 0, 1);
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) {
      if (ks + 1 < kKS) {
        a[(ks + 1) & 1][0] = score_a(st, ks + 1, 0);
        a[(ks + 1) & 1][1] = score_a(st, ks + 1, 1);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks & 1][mt], qf[nt][ks], s[mt][nt], 0, 0, 0);
      extra(ks);
    }
  };

  // Scores-only pass over the split: each head's exact max.
  auto max_pass = [&]() {
    issue(0);
    issue(1);
    issue(2);
    wait_stage(0, 2);
    lds_barrier();
    for (int i = 0; i < n; ++i) {
      scores(ring + (i & 3) * kStageBytes, [](int) {});
      uint2 pk[2][2];
      bool over = false;
      softmax(std::integral_constant<int, kMaxOnly>(), stage_valid(i), pk, over);
      lds_barrier();                    // every wave is done with stage i's slot
      issue(i + 3);
      wait_stage(i + 1, i + 3);
      lds_barrier();
    }
  };

  // Accumulating pass, software-pipelined: step i computes the value product of stage i
  // interleaved with the score product of stage i + 1, then the softmax of stage i + 1, with
  // one barrier per step.  Stage j's P lives in P buffer j % 2; stage j in ring slot j % 4.
  // Returns true (work-group uniform) if a kChecked pass gave up.
  auto accumulate = [&](auto mode) -> bool {
    constexpr int kMode = decltype(mode)::value;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[ct][nt][e] = 0.f;
    l_run[0] = l_run[1] = 0.f;
    bool over = false;
    issue(0);
    issue(1);
    issue(2);
    wait_stage(0, 2);
    lds_barrier();
    {
      uint2 pk[2][2];
      scores(ring, [](int) {});
      softmax(mode, stage_valid(0), pk, over);
      store_p(pbase, pk);
    }
    wait_stage(1, 2);
    lds_barrier();
    for (int i = 0; i < n; ++i) {
      issue(i + 3);                     // into the slot of stage i - 1, free since the last barrier
      const char* st_v = ring + (i & 3) * kStageBytes;
      const char* pb_v = pbase + (i & 1) * kPBytes;
      // value product of stage i: unit u = (K step u >> 4, column tile (u >> 2) & 3, head tile u & 3)
      bf16x8_t pb[4], av[2];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) pb[nt] = p_frag(pb_v, 0, nt);
      av[0] = val_a(st_v, 0, 0);
      auto pv_unit = [&](int u) {
        const int ks = u >> 4, ct = (u >> 2) & 3, nt = u & 3;
        if (nt == 0 && u + 4 < 32) av[((u >> 2) + 1) & 1] = val_a(st_v, (u + 4) >> 4, ((u + 4) >> 2) & 3);
        o[ct][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[(u >> 2) & 1], pb[nt], o[ct][nt], 0, 0, 0);
        if (ks == 0 && ct == 3) pb[nt] = p_frag(pb_v, 1, nt);     // last use of K step 0's fragment
      };
      // score product of stage i + 1 (a stage past the split's end scores with every token masked)
      scores(ring + ((i + 1) & 3) * kStageBytes, [&](int ks) {
        if (ks < 12) {
          pv_unit(2 * ks);
          pv_unit(2 * ks + 1);
        }
      });
      uint2 pk[2][2];
      softmax(mode, stage_valid(i + 1), pk, over);
#pragma unroll
      for (int u = 24; u < 32; ++u) pv_unit(u);
      store_p(pbase + ((i + 1) & 1) * kPBytes, pk);
      wait_stage(i + 2, i + 3);
      lds_barrier();
    }
    if (kMode != kChecked) return false;
    // gave up if any wave saw a score beyond its head's reference + kSlack
    int* flags = reinterpret_cast<int*>(pbase);
    const bool any_over = __any(over);
    if (lane == 0) flags[wave] = any_over ? 1 : 0;
    lds_barrier();
    const int4 f = *reinterpret_cast<const int4*>(flags);
    lds_barrier();
    return (f.x | f.y | f.z | f.w) != 0;
  };

  if (accumulate(std::integral_constant<int, kChecked>())) {
    max_pass();
    accumulate(std::integral_constant<int, kFixed>());
  }

  // ---- partial state of this split
  const long row0 = (long(b) * splits + sp) * H + hbase;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g == 0) {
      const long row = row0 + 32 * wave + 16 * nt + li;
      part_ml[row * 2] = m_ref[nt];
      part_ml[row * 2 + 1] = l;
    }
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float* dst = part_o + (row0 + 32 * nt + ph) * kDC + 128 * wave + 4 * (lane >> 5);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t*>(dst + 32 * ct + 8 * q) =
            f32x4_t{o[ct][nt][4 * q], o[ct][nt][4 * q + 1], o[ct][nt][4 * q + 2], o[ct][nt][4 * q + 3]};
  }
}

bool launch_decode_attn_v2(const DecodeAttnArgs& a, hipStream_t st) {
  if (a.H % kHeads != 0 || a.dc != kDC || a.dr != kDR) return false;
  const long units = long(a.B) * a.splits;
  const int xcd_map = (a.B % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(decode_attn_latent_kernel, dim3(unsigned(units), a.H / kHeads), dim3(kThreads), 0, st, a.H,
                     a.splits, a.max_blocks, xcd_map, static_cast<const uint16_t*>(a.qhat),
                     static_cast<const uint16_t*>(a.cache), a.block_table, a.ctx, a.part_o, a.part_ml);
  return true;
}

}  // namespace mla
