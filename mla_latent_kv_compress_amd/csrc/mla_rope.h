// RoPE parameters shared by the host planner and the kernels (plain struct, no HIP).
#pragma once

namespace mla {

// Pair i of a d_r-wide vector turns by pos * f_i, f_i = theta^(-2i/d_r).  With factor > 1 the
// frequencies are interpolated by parts (YaRN): a pair making r_i = orig * f_i / (2 pi) turns over
// the original context keeps f_i when r_i >= beta_fast, becomes f_i / factor when
// r_i <= beta_slow, and in between mixes the two linearly in r_i.  cos and sin are multiplied by
// mscale (both q_pe and k_pe, so their product by mscale^2).
struct RopeParams {
  float theta;
  float factor;       // <= 1: no interpolation
  float orig;         // original context length of the base frequencies
  float beta_fast, beta_slow;
  float mscale;
};

}  // namespace mla
