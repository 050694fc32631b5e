// frontend.cuh -- the per-channel and per-head arithmetic of the GDN layer's
// front-end, shared by the prefill front-end (frontend.hip) and the
// decode-side conv step (conv.hip) so that both give bitwise the same value
// for a token with the same conv window.
//
// Conv width 4: tap j multiplies x[t - 3 + j]; SiLU; q and k to unit L2 norm
// per (token, head) as y / sqrt(sum y^2 + eps); g = -softplus(a_raw),
// beta = sigmoid(b_raw).
#pragma once

#include <math.h>

#include "device.h"

namespace gdn {

// SiLU with the hardware exp and reciprocal: x * 1 / (1 + e^-x)
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// one DPP permutation of a float, every lane reading the lane CTRL selects
template <int CTRL>
__device__ __forceinline__ float dpp_perm(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the N lanes of a head (N a power of two, at most 32), left in all
// of them: the pairs of an xor butterfly, formed by DPP inside each 16-lane
// row (quad permutes, then the half-row and row mirrors), a shuffle across rows.
template <int N>
__device__ __forceinline__ float head_sum(float x) {
  if constexpr (N >= 2) x += dpp_perm<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (N >= 4) x += dpp_perm<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp_perm<0x141>(x);  // row_half_mirror: the other quad
  if constexpr (N >= 16) x += dpp_perm<0x140>(x); // row_mirror: the other half row
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Scales the CH channels this lane holds so that the head (PPH neighbouring
// lanes) has unit L2 norm: y / sqrt(sum y^2 + eps), with the hardware 1/sqrt.
template <int PPH, int CH>
__device__ __forceinline__ void l2_scale(float (&y)[CH], float eps) {
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) ss = fmaf(y[c], y[c], ss);
  const float inv = __builtin_amdgcn_rsqf(head_sum<PPH>(ss) + eps);
#pragma unroll
  for (int c = 0; c < CH; ++c) y[c] *= inv;
}

// the conv of one channel over its window (x3 = token t-3 ... x0 = token t,
// w = taps 0..3) followed by SiLU; the accumulation order is fixed
__device__ __forceinline__ float conv4_silu(const float4 &w, float x3, float x2, float x1,
                                            float x0) {
  return silu_fast(fmaf(w.x, x3, fmaf(w.y, x2, fmaf(w.z, x1, w.w * x0))));
}

// g = -softplus(a) computed as -(max(a,0) + log1p(exp(-|a|)))
__device__ __forceinline__ float gate_g(float a) { return -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a)))); }

// beta = sigmoid(b)
__device__ __forceinline__ float gate_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

}  // namespace gdn
