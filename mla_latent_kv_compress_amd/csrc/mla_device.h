// Device helpers shared by the libmla kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_rope.h"

namespace mla {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPage = 64;
constexpr float kLog2e = 1.4426950408889634f;

// bf16 storage is uint16_t bit patterns.  Rounding is to nearest, ties to even (finite input).
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// OCP e4m3fn ("fn": no infinities; 0x7F/0xFF are NaN; largest finite 448).
__device__ __forceinline__ float e4m3_to_f(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  if ((c & 0x7Fu) == 0x7Fu) return __uint_as_float(0x7FC00000u);
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
  return (c & 0x80u) ? -v : v;
}
// Nearest e4m3fn code of v (ties to even), saturating at +-448; NaN gives the NaN code.
__device__ __forceinline__ uint32_t f_to_e4m3(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fabsf(v);
  uint32_t code;
  if (a != a) {
    code = 0x7Fu;
  } else if (!(a < 448.0f)) {
    code = 0x7Eu;                                   // 448
  } else if (a < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
    code = uint32_t(rintf(a * 512.0f));             // 8 carries into the smallest normal
  } else {
    int e = int((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6 .. 8
    float frac = __uint_as_float((__float_as_uint(a) & 0x007FFFFFu) | 0x3F800000u);  // [1, 2)
    uint32_t m = uint32_t(rintf((frac - 1.0f) * 8.0f));
    if (m == 8u) { m = 0u; ++e; }
    code = (uint32_t(e + 7) << 3) | m;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

// fp16 storage is uint16_t bit patterns as well (IEEE binary16, round to nearest even).
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }
// The same, saturating at +-65504 instead of overflowing to infinity.
__device__ __forceinline__ uint16_t f2h_sat(float f) { return f2h(fminf(fmaxf(f, -65504.0f), 65504.0f)); }

// Storage codes: fp32, bf16, fp16 (the fp8 cache has its own path).
enum { S_F32 = 0, S_BF16 = 1, S_F16 = 3 };
template <int S> struct StoreT { typedef uint16_t type; };
template <> struct StoreT<S_F32> { typedef float type; };
template <int S> __device__ __forceinline__ float lds_(const typename StoreT<S>::type* p, long i);
template <> __device__ __forceinline__ float lds_<S_F32>(const float* p, long i) { return p[i]; }
template <> __device__ __forceinline__ float lds_<S_BF16>(const uint16_t* p, long i) { return bf2f(p[i]); }
template <> __device__ __forceinline__ float lds_<S_F16>(const uint16_t* p, long i) { return h2f(p[i]); }
template <int S> __device__ __forceinline__ void sts_(typename StoreT<S>::type* p, long i, float v);
template <> __device__ __forceinline__ void sts_<S_F32>(float* p, long i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void sts_<S_BF16>(uint16_t* p, long i, float v) { p[i] = f2bf(v); }
template <> __device__ __forceinline__ void sts_<S_F16>(uint16_t* p, long i, float v) { p[i] = f2h(v); }

// fp16 storage in the typed helpers below (a distinct type from bf16's uint16_t).
struct F16Out { uint16_t bits; };

template <typename T> __device__ __forceinline__ float ldf(const T* p, long i);
template <> __device__ __forceinline__ float ldf<float>(const float* p, long i) { return p[i]; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, long i) { return bf2f(p[i]); }
template <typename T> __device__ __forceinline__ void stf(T* p, long i, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, long i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void stf<uint16_t>(uint16_t* p, long i, float v) { p[i] = f2bf(v); }
template <> __device__ __forceinline__ void stf<F16Out>(F16Out* p, long i, float v) { p[i].bits = f2h_sat(v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Block-wide reductions for blockDim.x a multiple of 64 (<= 1024); `red` holds >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
  for (int i = 0; i < nw; ++i) s = fmaxf(s, red[i]);
  return s;
}

// RoPE of pair i (of a d_r-wide vector) at position pos: cos and sin of its angle, formed in
// double precision, times mscale.  Frequencies as described with RopeParams (YaRN when
// factor > 1, after the YaRN paper's interpolation by parts).
__device__ __forceinline__ void rope_cs(int pos, int i, int dr, const RopeParams& rp, float* c, float* s) {
  double freq = pow(double(rp.theta), -2.0 * double(i) / double(dr));
  if (rp.factor > 1.f) {
    const double turns = double(rp.orig) * freq / (2.0 * 3.14159265358979323846);
    double g = (turns - double(rp.beta_slow)) / (double(rp.beta_fast) - double(rp.beta_slow));
    g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
    freq = (1.0 - g) * freq / double(rp.factor) + g * freq;
  }
  const double ang = double(pos) * freq;
  *c = float(cos(ang) * double(rp.mscale));
  *s = float(sin(ang) * double(rp.mscale));
}

}  // namespace mla
