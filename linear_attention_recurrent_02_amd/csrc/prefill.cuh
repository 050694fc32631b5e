// prefill.cuh -- chunked prefill of the Gated DeltaNet recurrence on MFMA.
//
// One workgroup (4 waves) walks one (sequence, state head) chain chunk by
// chunk (C = 64 tokens), carrying the FP32 state M (d_k x d_v) in MFMA
// accumulator registers.  Per chunk, with G = cumsum(log a), gamma = exp(G),
// and everything below derived from the token recurrence written in the
// residual form of the Kimi Linear section of "Seven Architectures Replacing
// KV Cache With Bounded Mutable State" (scalar decay, which the Gated
// DeltaNet-2 section says is Gated DeltaNet):
//
//   S = K K^T,  P = Q K^T                                    (intra-chunk)
//   A[r,s] = beta_r exp(G_r - G_s) S[r,s]  (s < r),  T = (I + A)^-1
//   R = diag(beta) (V - diag(gamma) K M)                      (needs M)
//   U = T R                        (= the per-token residual writes u_r)
//   O = diag(gamma) Q M + (L o P) U,  L[r,s] = exp(G_r - G_s) (s <= r)
//   M <- gamma_last M + (diag(exp(G_last - G)) K)^T U
//
// linear / gated have no erase: A = 0, T = I, R = V.  linear / delta have no
// decay: G = 0.  Rows past the end of a ragged tail chunk are zero (k, q, v,
// beta = 0, g = 0), so they add nothing and gamma_last is the last real
// token's.
//
// Every matrix product runs on MFMA with operands read from LDS as fragments
// of 8 K-consecutive elements (K-contiguous layouts: the right-hand operand
// of each product is stored transposed).  With BF16 activations (F32 =
// false) the operands are BF16 and each product is one
// v_mfma_f32_16x16x32_bf16 per 32-wide K slab, FP32 accumulate -- measured at
// ~6e-3 scaled error over 8192 tokens against the FP64 oracle, inside the 2e-2
// bar.  With FP32 activations (F32 = true) the operands stay FP32 and each
// slab is eight v_mfma_f32_16x16x4f32, for the 1e-4 bar.  The state M is FP32
// in accumulator registers in both.  T is formed in FP32 on the vector ALUs by
// blocked forward substitution (16 x 16 diagonal blocks, then three levels of
// off-diagonal blocks).
#pragma once

#include <math.h>

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct PrefillParams {
  int32_t n_seq, H_qk, H_v, group;
  int64_t n_slots;
  float scale;
  int32_t rule;
  const int32_t *cu;
  const void *q, *k, *v;  // [N, H_qk, d_k], [N, H_qk, d_k], [N, H_v, d_v] (act dtype)
  const float *g, *beta;  // [N, H_v]
  void *pool;
  const int32_t *read_slot, *write_slot;
  void *o;
  uint32_t *status;
};

// LDS layout of the chain kernel (byte offsets).  OT is the operand storage
// type: raw BF16 bits, or float on the FP32 path.  Rows are padded by 16
// bytes so the 16 lanes of a fragment read hit different banks.
template <int DK, int DV, bool F32>
struct PrefillLayout {
  using OT = std::conditional_t<F32, float, uint16_t>;
  static constexpr int C = 64;
  static constexpr int DKP = DK < 32 ? 32 : DK;  // MFMA K-steps are 32 wide
  static constexpr int PADE = 16 / (int)sizeof(OT);
  static constexpr int LDK = DKP + PADE;  // Kh, Qh (token rows), Mt (column rows)
  static constexpr int LDC = C + PADE;    // Kt, Sq, Rt (rows of 64 tokens)
  static constexpr int LDF = C + 4;       // Af, Tf (float)
  static constexpr size_t KH = 0;
  static constexpr size_t QH = KH + (size_t)C * LDK * sizeof(OT);
  static constexpr size_t KT = QH + (size_t)C * LDK * sizeof(OT);
  static constexpr size_t MT = KT + (size_t)DK * LDC * sizeof(OT);
  static constexpr size_t SQ = MT + (size_t)DV * LDK * sizeof(OT);
  static constexpr int LDV = DV + PADE;   // Vh / Oh rows (64 tokens x d_v)
  static constexpr size_t VH = SQ + (size_t)C * LDC * sizeof(OT);  // V, then O, row-major
  static constexpr size_t RT = VH + (size_t)C * LDV * sizeof(OT);
  static constexpr size_t RT_BYTES = (size_t)DV * LDC * sizeof(OT);
  static constexpr size_t AF_BYTES = (size_t)C * LDF * 4;
  // Af (only live while T is formed) shares its bytes with Rt/Ut
  static constexpr size_t TF = RT + (RT_BYTES > AF_BYTES ? RT_BYTES : AF_BYTES);
  static constexpr size_t GATES = TF + (size_t)C * LDF * 4;  // G, gamma, beta, eGn
  static constexpr size_t XS = GATES + 4 * C * 4;            // 4 x 16 x 17 floats
  static constexpr size_t BYTES = XS + 4 * 16 * 17 * 4;
};

// ---- MFMA fragments -------------------------------------------------------
//
// A fragment is 8 consecutive K-elements of one row: lane l of a wave holds
// row r0 + l%16, columns k0 + 8*(l/16) .. +8 of a row-major LDS matrix
// (leading dimension ld).  That is the operand layout of
// v_mfma_f32_16x16x32_bf16 for A (rows = M) and for B stored transposed
// (rows = N).  The FP32 path feeds the same 8 elements, one per instruction,
// to eight v_mfma_f32_16x16x4f32: instruction i sums k = k0 + 8g + i over the
// four lane groups g, so the eight together cover the same 32-wide K slab.

template <bool F32> struct Frag;
template <> struct Frag<false> { bf16x8_t v; };
template <> struct Frag<true> { float v[8]; };

__device__ __forceinline__ const void *frag_addr(const void *base, int esize, int ld, int r0,
                                                 int k0) {
  const int l = threadIdx.x & 63;
  return static_cast<const char *>(base) + ((r0 + (l & 15)) * ld + k0 + 8 * (l >> 4)) * esize;
}

template <bool F32>
__device__ __forceinline__ Frag<F32> load_frag(const uint16_t *base, int ld, int r0, int k0) {
  static_assert(!F32, "FP32 fragments come from float buffers");
  Frag<false> f;
  f.v = __builtin_bit_cast(bf16x8_t, *static_cast<const uint4 *>(frag_addr(base, 2, ld, r0, k0)));
  return f;
}
template <bool F32>
__device__ __forceinline__ Frag<F32> load_frag(const float *base, int ld, int r0, int k0) {
  const float4 *src = static_cast<const float4 *>(frag_addr(base, 4, ld, r0, k0));
  const float4 x0 = src[0], x1 = src[1];
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  Frag<F32> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (F32) f.v[j] = x[j];
    else f.v[j] = (__bf16)x[j];  // round to nearest even
  }
  return f;
}

template <bool F32>
__device__ __forceinline__ f32x4_t mma(f32x4_t c, const Frag<F32> &a, const Frag<F32> &b) {
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], c, 0, 0, 0);
  } else {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
  }
  return c;
}

// Split of an NX x NY grid of 16 x 16 tiles over the 4 waves: by columns when
// there are at least 4 column blocks (each wave then shares its column
// fragments across all rows), else by rows, else one tile per wave.
template <int NX, int NY>
struct TileSplit {
  static constexpr int BY_Y = NY >= 4, BY_X = !BY_Y && NX >= 4;
  static constexpr int PER = BY_Y ? NX * (NY / 4) : (BY_X ? (NX / 4) * NY : 1);
  static constexpr int XN = BY_Y ? NX : (BY_X ? NX / 4 : 1);  // rows per wave
  static constexpr int YN = BY_Y ? NY / 4 : (BY_X ? NY : 1);  // columns per wave
  // tile j of wave w -> (x, y); valid() false for waves without a tile
  __device__ static __forceinline__ int x(int w, int j) {
    return BY_Y ? j / YN : (BY_X ? w * XN + j / YN : w / NY);
  }
  __device__ static __forceinline__ int y(int w, int j) {
    return BY_Y ? w * YN + j % YN : (BY_X ? j % YN : w % NY);
  }
  __device__ static __forceinline__ bool valid(int w) { return BY_Y || BY_X || w < NX * NY; }
};

// 2^x on the hardware transcendental unit (v_exp_f32)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// store a float into an operand buffer
__device__ __forceinline__ void put(uint16_t *p, float x) { *p = f32_to_bf16(x); }
__device__ __forceinline__ void put(float *p, float x) { *p = x; }
__device__ __forceinline__ float get(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float get(const float *p) { return *p; }

}  // namespace gdn
