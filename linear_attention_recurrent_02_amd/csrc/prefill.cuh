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
//   A[r,s] = beta_r exp(G_r - G_s) S[r,s]  (s < r)
//   R = diag(beta) (V - diag(gamma) K M)                      (needs M)
//   U = (I + A)^-1 R               (= the per-token residual writes u_r)
//   O = diag(gamma) Q M + (L o P) U,  L[r,s] = exp(G_r - G_s) (s <= r)
//   M <- gamma_last M + (diag(exp(G_last - G)) K)^T U
//
// linear / gated have no erase: A = 0, T = I, R = V.  linear / delta have no
// decay: G = 0.  Rows past the end of a ragged tail chunk repeat the last
// token's k, q, v but carry beta = 0 (R = beta V under the plain rules) and
// g = 0: their rows of A, R and U vanish, so they add nothing, and gamma_last
// is the last real token's.
//
// Every product runs on MFMA with FP32 accumulation.  The recurrence is
// independent per state column (a column of M only ever meets the same column
// of V, R, U and O), so each wave owns a slice of d_v columns and keeps its
// columns of M, of K M and Q M, of R, U and O in its own accumulator
// registers: the M-dependent half of a chunk needs no LDS round trip and no
// barrier.  An accumulator tile serves directly as the right-hand operand of
// the next product through a permuted K order (see bfrag); the left-hand
// operands (Q, K, K^T, A, T_ii, L o P) are chunk-local and read from LDS.  With BF16 activations (F32 = false) operands are BF16, one
// v_mfma_f32_16x16x32_bf16 per 32-wide K slab -- measured at ~6e-3 scaled
// error over 8192 tokens against the FP64 oracle, inside the 2e-2 bar.  With
// FP32 activations (F32 = true) they stay FP32, eight v_mfma_f32_16x16x4f32
// per slab, for the 1e-4 bar.  U = (I + A)^-1 R is solved by block forward
// substitution over the four 16-row blocks, each wave on its own columns:
// U_i = T_ii (R_i - sum_{j<i} A_ij U_j), with T_ii = (I + A_ii)^-1 formed in
// FP32 on the vector ALUs (every wave forms all four, so no wave waits on
// another) and the 16-wide products on MFMA.
#pragma once

#include <math.h>

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace gdn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // 16 raw bytes

struct PrefillParams {
  int32_t n_seq, H_qk, H_v, group;
  int64_t n_tokens, n_slots;
  float scale;
  int32_t rule;
  const int32_t *cu;
  const void *q, *k, *v;  // [N, H_qk, d_k], [N, H_qk, d_k], [N, H_v, d_v] (act dtype)
  const float *g, *beta;  // [N, H_v]
  void *pool;
  const int32_t *read_slot, *write_slot;
  void *o;
  uint32_t *status;
  // intermediate checkpoints: after every ckpt_chunks chunks (0 = none), the
  // state goes to ckpt_slot[seq * ckpt_per_seq + j]
  int32_t ckpt_chunks, ckpt_per_seq;
  const int32_t *ckpt_slot;
  int32_t channel_decay;  // g is [N, H_v, d_k]: one log-decay per key channel
};

// LDS layout of the chain kernel (byte offsets).  IT is the storage type of
// the staged inputs (K, Q, V rows: the activation dtype, BF16 bits or float);
// OT that of the chunk-local operand L o P: BF16 bits, or float on the FP32
// path (F32), which also keeps A and T_ii in float.  Rows are padded by 16
// bytes so the 16 lanes of a fragment read hit different banks.  The chunk's
// inputs (K, Q, V rows and the gates) live in one of two alternating sets:
// while a chunk computes from one set, the next chunk's inputs are written
// into the other.
template <int DK, int DV, bool F32, bool AB = !F32>
struct PrefillLayout {
  using IT = std::conditional_t<AB, uint16_t, float>;
  using OT = std::conditional_t<F32, float, uint16_t>;
  static_assert(F32 || AB, "FP32 activations take FP32 operands");
  static constexpr int C = 64;
  static constexpr int DKP = DK < 32 ? 32 : DK;  // MFMA K-steps are 32 wide
  static constexpr int PADI = 16 / (int)sizeof(IT), PADO = 16 / (int)sizeof(OT);
  static constexpr int LDK = DKP + PADI;  // Kh, Qh (token rows)
  static constexpr int LDC = C + PADO;    // Sq (rows of 64 tokens)
  static constexpr int LDF = C + 4;       // Af, Tf (float)
  static constexpr int LDV = DV + PADI;   // Vh rows (64 tokens x d_v)
  // one input set
  static constexpr size_t KH = 0;
  static constexpr size_t QH = KH + (size_t)C * LDK * sizeof(IT);
  static constexpr size_t VH = QH + (size_t)C * LDK * sizeof(IT);
  // G, gamma, beta, exp(G_last - G), scale * gamma, e * gamma (e = 1 for the
  // delta rules, else 0)
  static constexpr size_t GATES = VH + (size_t)C * LDV * sizeof(IT);
  static constexpr size_t SET = GATES + 6 * C * 4;  // bytes per set
  // shared by both sets
  static constexpr size_t SQ = 2 * SET;
  static constexpr size_t AF = SQ + (size_t)C * LDC * sizeof(OT);
  static constexpr int LDT = 20;  // T_ii rows (float); 16-byte aligned rows
  static constexpr size_t TF = AF + (size_t)C * LDF * 4;  // the four T_ii, stacked
  static constexpr size_t BYTES = TF + (size_t)C * LDT * 4;
  // BF16 copies for the substitution's operands (-A below the diagonal, T_ii),
  // where no FP32 reader needs them: in the AF and TF regions
  static constexpr int LDAB = C + 8, LDTB = 16 + 8;
  static_assert((size_t)C * LDAB * 2 <= (size_t)C * LDF * 4 && LDTB * 2 <= LDT * 4, "BF16 copies fit");
  static_assert(SET % 16 == 0, "16-byte aligned sets");
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

// Eight BF16 values (16 raw bytes) as an operand fragment: as loaded for BF16
// operands, widened exactly for FP32 ones.
template <bool F32>
__device__ __forceinline__ Frag<F32> frag_of_bf16(const uint4 &u) {
  Frag<F32> f;
  if constexpr (F32) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f.v[2 * j] = bf16_lo(w[j]);
      f.v[2 * j + 1] = bf16_hi(w[j]);
    }
  } else {
    f.v = __builtin_bit_cast(bf16x8_t, u);
  }
  return f;
}

template <bool F32>
__device__ __forceinline__ Frag<F32> load_frag(const uint16_t *base, int ld, int r0, int k0) {
  return frag_of_bf16<F32>(*static_cast<const uint4 *>(frag_addr(base, 2, ld, r0, k0)));
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

// ---- accumulator tiles as right-hand operands ------------------------------
//
// An FP32 accumulator tile of a 16 x 16 product holds, in lane l = 16 g + n,
// rows 4g .. 4g+3 of column n.  Two stacked tiles (rows 0-15 = lo, 16-31 =
// hi) give lane (g, n) the eight values B[k][n] for k in {4g..4g+3} and
// {16+4g..16+4g+3}.  Feeding those as the lane's eight K-elements of a
// 32-wide slab, with the left-hand operand's elements taken at the same k
// (load_afrag), sums over all 32 k exactly once: the K order inside a slab is
// permuted, the product is not.  So the output of one product becomes the
// right-hand operand of the next without leaving the wave's registers.

template <bool F32>
__device__ __forceinline__ Frag<F32> bfrag(const f32x4_t &lo, const f32x4_t &hi) {
  Frag<F32> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (F32) {
      f.v[i] = lo[i];
      f.v[4 + i] = hi[i];
    } else {
      f.v[i] = (__bf16)lo[i];  // round to nearest even
      f.v[4 + i] = (__bf16)hi[i];
    }
  }
  return f;
}

// Left-hand fragment matching bfrag's K order: lane (g, m) holds row r0 + m
// at columns k0 + 4g + {0..3} and k0 + 16 + 4g + {0..3}.
template <bool F32>
__device__ __forceinline__ Frag<F32> load_afrag(const uint16_t *base, int ld, int r0, int k0) {
  const int l = threadIdx.x & 63;
  const uint16_t *row = base + (r0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
  uint4 u;
  const uint2 a = *reinterpret_cast<const uint2 *>(row);
  const uint2 b = *reinterpret_cast<const uint2 *>(row + 16);
  u.x = a.x; u.y = a.y; u.z = b.x; u.w = b.y;
  return frag_of_bf16<F32>(u);
}
template <bool F32>
__device__ __forceinline__ Frag<F32> load_afrag(const float *base, int ld, int r0, int k0) {
  const int l = threadIdx.x & 63;
  const float *row = base + (r0 + (l & 15)) * ld + k0 + 4 * (l >> 4);
  const float4 x0 = *reinterpret_cast<const float4 *>(row);
  const float4 x1 = *reinterpret_cast<const float4 *>(row + 16);
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  Frag<F32> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (F32) f.v[j] = x[j];
    else f.v[j] = (__bf16)x[j];  // round to nearest even
  }
  return f;
}

// The same fragment of a transposed operand: lane (g, m) holds column r0 + m
// of a row-major matrix at rows k0 + 4g + {0..3} and k0 + 16 + 4g + {0..3},
// i.e. A[m][k] = base[k][r0 + m].  BF16: two ds_read_b64_tr_b16 per fragment.
// That gfx950 load transposes inside each 16-lane group: result lane i,
// element j is element i % 4 of the 8 bytes addressed by lane 4j + i / 4
// (checked on the hardware with index-valued LDS).  So lane (g, s) points at
// row k0 + 4g + s / 4, columns r0 + 4 (s % 4) .. +3 -- 8 contiguous bytes.
template <bool F32>
__device__ __forceinline__ Frag<F32> load_afrag_t(const uint16_t *base, int ld, int r0, int k0) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
  const uint16_t *a = base + (k0 + 4 * g + (s >> 2)) * ld + r0 + 4 * (s & 3);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(a + 16 * ld));
  const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
  return frag_of_bf16<F32>(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
}
// Four consecutive rows of one column, in the accumulator layout: lane (g, n)
// gets base[(r0 + 4g + e) * ld + c0 + n], e = 0..3 -- one transposing load
// (lane (g, s) points at row r0 + 4g + s / 4, columns c0 + 4 (s % 4) .. +3).
__device__ __forceinline__ void load_col4(const uint16_t *base, int ld, int r0, int c0, float *x) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(base + (r0 + 4 * g + (s >> 2)) * ld + c0 + 4 * (s & 3)));
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = bf16_to_f32((uint16_t)v[e]);
}
__device__ __forceinline__ void load_col4(const float *base, int ld, int r0, int c0, float *x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = base[(r0 + 4 * (l >> 4) + e) * ld + c0 + (l & 15)];
}

template <bool F32>
__device__ __forceinline__ Frag<F32> load_afrag_t(const float *base, int ld, int r0, int k0) {
  const int l = threadIdx.x & 63;
  const float *c = base + (k0 + 4 * (l >> 4)) * ld + r0 + (l & 15);
  Frag<F32> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (F32) {
      f.v[j] = c[j * ld];
      f.v[4 + j] = c[(16 + j) * ld];
    } else {
      f.v[j] = (__bf16)c[j * ld];
      f.v[4 + j] = (__bf16)c[(16 + j) * ld];
    }
  }
  return f;
}

// ---- 16-wide K products -----------------------------------------------------
//
// One accumulator tile is exactly the right-hand operand of a K = 16 product
// (v_mfma_f32_16x16x16_bf16: lane (g, n) holds B[4g + j][n]; FP32: four
// v_mfma_f32_16x16x4f32, instruction j taking k = 4g + j); the left-hand
// operand's lane (g, m) holds row m at columns 4g .. 4g+3.

template <bool F32> struct Frag16;
template <> struct Frag16<false> { s16x4_t v; };
template <> struct Frag16<true> { float v[4]; };

template <bool F32>
__device__ __forceinline__ Frag16<F32> bfrag16(const f32x4_t &x) {
  Frag16<F32> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (F32) f.v[j] = x[j];
    else f.v[j] = __builtin_bit_cast(short, (__bf16)x[j]);  // round to nearest even
  }
  return f;
}

// rows r0 .. r0+15, columns k0 .. k0+15 of a row-major float matrix, times sgn
template <bool F32>
__device__ __forceinline__ Frag16<F32> load_afrag16(const float *base, int ld, int r0, int k0,
                                                    float sgn) {
  const int l = threadIdx.x & 63;
  const float4 x = *reinterpret_cast<const float4 *>(base + (r0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  const float y[4] = {sgn * x.x, sgn * x.y, sgn * x.z, sgn * x.w};
  Frag16<F32> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (F32) f.v[j] = y[j];
    else f.v[j] = __builtin_bit_cast(short, (__bf16)y[j]);
  }
  return f;
}

// the same 16 x 16 fragment of a row-major BF16 matrix (stored ready to use:
// no conversion, no sign)
__device__ __forceinline__ Frag16<false> load_afrag16(const uint16_t *base, int ld, int r0, int k0) {
  const int l = threadIdx.x & 63;
  Frag16<false> f;
  f.v = *reinterpret_cast<const s16x4_t *>(base + (r0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  return f;
}
template <bool F32>
__device__ __forceinline__ f32x4_t mma16(f32x4_t c, const Frag16<F32> &a, const Frag16<F32> &b) {
  if constexpr (F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  } else {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, c, 0, 0, 0);
  }
  return c;
}

// 2^x on the hardware transcendental unit (v_exp_f32)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// one DPP move of a float: lanes of the rows in ROWS read the lane CTRL
// selects; every other lane reads 0
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave, without LDS: shifts by
// 1, 2, 4, 8 inside each 16-lane row, then lane 15's total is broadcast into
// rows 1 and 3 and lane 31's into rows 2 and 3.
__device__ __forceinline__ float wave_inclusive_sum(float x) {
  x += dpp_move<0x111, 0xf>(x);  // row_shr:1
  x += dpp_move<0x112, 0xf>(x);  // row_shr:2
  x += dpp_move<0x114, 0xf>(x);  // row_shr:4
  x += dpp_move<0x118, 0xf>(x);  // row_shr:8
  x += dpp_move<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_move<0x143, 0xc>(x);  // row_bcast:31
  return x;
}

// store a float into an operand buffer
// BF16 rows of a K, Q or V tile in LDS (W values each), in one of three
// layouts.  The chains read these tiles in three shapes: 8-byte row reads
// (16 rows x 2 groups of 8 bytes per 32 lanes: Q M, K M), transposing 8-byte
// reads (8 rows x 4 groups per 32 lanes: V, and K^T for the update of M) and
// 16-byte row reads (S and P).
//  - kRowsPadded: rows padded by 16 bytes.
//  - kRowsXor (128-value rows): unpadded, 8-byte group j of row r at group
//    j ^ sw(r), sw(r) = 4 (r mod 8) + 2 ((r / 8) mod 2).  sw's bits 1-4 are a
//    bijection of r mod 16 and its bits 2-4 one of r mod 8, so both 8-byte
//    shapes meet 64 distinct banks; sw is even, so a 16-byte piece stays
//    whole.  The permutation reaches the bits that slab offsets change, so
//    each read computes its own address.
//  - kRowsSwap (128-value rows): padded by 32 bytes (a row starts 8 banks
//    after the one before it, so eight rows cover the 64 banks) and, on
//    every other block of 8 rows, the 16-byte pieces swapped in pairs (group
//    j at j ^ 2), giving rows r and r + 8 the other half of their 8-bank
//    window: both 8-byte shapes again meet 64 distinct banks.  The swap
//    flips one bit that no slab or half-row offset touches, so a lane's reads
//    are one base plus constant offsets.
// Measured on gfx950 (one CU, 8 waves), LDS clocks per 512 bytes read, padded
// / xor / swap: row 8.5 / 3.4 / 3.3, transposing 4.5 / 3.3 / 3.35, 16-byte
// 9.1 / 8.4 / 8.5 per 1 KB.  In the chains, the pipelined one ran faster
// with kRowsXor (0.770 against 0.786 ms for the varlen prefill), the
// channel-wise one with kRowsSwap (1.483 against 1.525 ms padded; with
// kRowsXor its per-read addresses spilled 248 bytes per lane).
constexpr int kRowsPadded = 0, kRowsXor = 1, kRowsSwap = 2;
template <int W, int KIND>
struct LdsRows {
  static_assert(KIND == kRowsPadded || W == 128, "the permuted layouts are of 128-value rows");
  static constexpr int LD = KIND == kRowsSwap ? W + 16 : KIND == kRowsXor ? W : W + 8;  // elements
  // element offset of (r, c), c a multiple of 4
  __device__ static __forceinline__ int at(int r, int c) {
    if constexpr (KIND == kRowsXor) return r * LD + (((c >> 2) ^ (4 * (r & 7) + 2 * ((r >> 3) & 1))) << 2) + (c & 3);
    else if constexpr (KIND == kRowsSwap) return r * LD + (c ^ (8 * ((r >> 3) & 1)));
    else return r * LD + c;
  }
  // (r0 + r, k0 + c) with r0 and k0 multiples of 16 and r < 16, c < 16
  __device__ static __forceinline__ int at(int r0, int k0, int r, int c) {
    if constexpr (KIND == kRowsXor) return at(r0 + r, k0 + c);
    else return r0 * LD + k0 + at(r, c);  // only the lane's part is permuted
  }
};

// BF16 operand fragments from LdsRows rows (R), in the layouts of load_frag,
// load_afrag, load_afrag_t and load_col4.
template <class R>
__device__ __forceinline__ Frag<false> rows_frag(const uint16_t *base, int r0, int k0) {
  const int l = threadIdx.x & 63;
  return frag_of_bf16<false>(*reinterpret_cast<const uint4 *>(base + R::at(r0, k0, l & 15, 8 * (l >> 4))));
}
template <class R>
__device__ __forceinline__ Frag<false> rows_afrag(const uint16_t *base, int r0, int k0) {
  const int l = threadIdx.x & 63;
  const uint2 a = *reinterpret_cast<const uint2 *>(base + R::at(r0, k0, l & 15, 4 * (l >> 4)));
  const uint2 b = *reinterpret_cast<const uint2 *>(base + R::at(r0, k0 + 16, l & 15, 4 * (l >> 4)));
  return frag_of_bf16<false>(make_uint4(a.x, a.y, b.x, b.y));
}
template <class R>
__device__ __forceinline__ Frag<false> rows_afrag_t(const uint16_t *base, int r0, int k0) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
  const uint16_t *const p = base + R::at(k0, r0, 4 * g + (s >> 2), 4 * (s & 3));
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + 16 * R::LD));
  const uint2 ulo = __builtin_bit_cast(uint2, lo), uhi = __builtin_bit_cast(uint2, hi);
  return frag_of_bf16<false>(make_uint4(ulo.x, ulo.y, uhi.x, uhi.y));
}
template <class R>
__device__ __forceinline__ void rows_col4(const uint16_t *base, int r0, int c0, float *x) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const int l = threadIdx.x & 63, g = l >> 4, s = l & 15;
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(base + R::at(r0, c0, 4 * g + (s >> 2), 4 * (s & 3))));
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = bf16_to_f32((uint16_t)v[e]);
}

__device__ __forceinline__ void put(uint16_t *p, float x) { *p = f32_to_bf16(x); }
__device__ __forceinline__ void put(float *p, float x) { *p = x; }
__device__ __forceinline__ float get(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float get(const float *p) { return *p; }

}  // namespace gdn
