// prefill_cw.cuh -- one (sequence, state head) chain of the chunked prefill
// with one decay per key channel (Kimi Delta Attention: "Seven Architectures
// Replacing KV Cache With Bounded Mutable State", Kimi Linear section, whose
// chunkwise form the Gated DeltaNet-2 section describes as absorbing a
// cumulative channel-wise decay into the WY products).
//
// Per chunk of C = 64 tokens, with G[r, i] the cumulative log-decay of key
// channel i over the chunk's first r + 1 tokens, the scalar chain's
// gamma-weighted rows become per-channel scalings:
//
//   K_g = K o e^G,  Q_g = Q o e^G,  K_e = K o e^(G_last - G)
//   A[r, s] = beta_r sum_i k_ri k_si e^(G_ri - G_si)      (s < r)
//   P[r, s] =        sum_i q_ri k_si e^(G_ri - G_si)      (s <= r)
//   R = beta (V - K_g M)  (delta rules; V otherwise),  U = (I + A)^-1 R
//   O = scale (Q_g M + P U),   M <- Diag(e^(G_last)) M + K_e^T U
//
// A and P are formed per 16 x 16 tile, each one MFMA product of K / Q
// fragments scaled on the fly through a reference token m:
// e^(G_r - G_s) = e^(G_r - G_m) e^(G_m - G_s).  Below the diagonal, tile
// (I, J) takes m = the last token of column tile J: both factors are <= 1
// for r > m >= s, so nothing overflows and no O(1) weight is lost.  A
// diagonal tile takes m = its first token: the row factors are <= 1 and the
// column factors at most 2^span, span being the tile's largest cumulative
// log2-decay over a channel; while span <= kCwDiagSpan the products stay far
// inside FP32 / BF16 range (the entries above the diagonal, at most 2^span,
// are discarded).  A diagonal tile with a larger span (a channel that
// forgets nearly everything within 16 tokens) takes its weights entry by
// entry on the vector ALUs instead, each e^(G_r - G_s) <= 1.  Everything else
// -- the block substitution for U, the read-out, the state update, state in
// and out, checkpoints -- follows the plain chain (prefill_chain.cuh), with
// the chunk's inputs in one LDS set (the per-channel decays take the room of
// the second).  The chain runs NW = 4 or 8 waves: with 8, two waves share
// each SIMD, so one's LDS and exp latencies hide behind the other's work;
// waves 0-3 form the diagonal tiles and waves 4-7 the six below, and each
// wave owns d_v / 8 state columns.
#pragma once

#include <algorithm>

#include "prefill_chain.cuh"

namespace gdn {

// LDS layout (byte offsets).  IT: the staged K, Q, V rows (activation dtype);
// OT: the scaled operands K_g, Q_g, K_e, L o P, -A and T_ii (BF16, or float
// on the FP32 path).  With IT == OT the scaled K and Q overwrite the raw ones
// once the chunk-local products are formed.
template <int DK, int DV, bool F32, bool AB>
struct CwLayout {
  using IT = std::conditional_t<AB, uint16_t, float>;
  using OT = std::conditional_t<F32, float, uint16_t>;
  static_assert(F32 || AB, "FP32 activations take FP32 operands");
  static constexpr bool ALIAS = sizeof(IT) == sizeof(OT);
  static constexpr int C = 64;
  static constexpr int DKP = DK < 32 ? 32 : DK;  // MFMA K-steps are 32 wide
  static constexpr int PADI = 16 / (int)sizeof(IT), PADO = 16 / (int)sizeof(OT);
  // BF16 rows of 128 values (K, Q, K_g, Q_g, K_e at d_k = 128, V at d_v =
  // 128) in the layout of LdsRows; other rows padded by 16 bytes
  static constexpr bool SWK = !F32 && DKP == 128;
  static constexpr bool SWV = !F32 && DV == 128;
  using RS = LdsRows<128, kRowsSwap>;
  static constexpr int LDK = SWK ? RS::LD : DKP + PADI;   // K, Q rows (IT)
  static constexpr int LDKO = SWK ? RS::LD : DKP + PADO;  // K_g, Q_g, K_e rows (OT)
  static constexpr int LDV = SWV ? RS::LD : DV + PADI;    // V rows (IT)
  // element offsets of (r, c) in those rows, c a multiple of 4
  __device__ static __forceinline__ int ak(int r, int c) {
    if constexpr (SWK) return RS::at(r, c); else return r * LDK + c;
  }
  __device__ static __forceinline__ int ako(int r, int c) {
    if constexpr (SWK) return RS::at(r, c); else return r * LDKO + c;
  }
  // (r0 + r, k0 + c) of K and Q rows, r0 and k0 multiples of 16
  __device__ static __forceinline__ int ak(int r0, int k0, int r, int c) {
    if constexpr (SWK) return RS::at(r0, k0, r, c); else return (r0 + r) * LDK + k0 + c;
  }
  __device__ static __forceinline__ int av(int r, int c) {
    if constexpr (SWV) return RS::at(r, c); else return r * LDV + c;
  }
  static constexpr int LDG = DKP + 4;      // G rows (float)
  static constexpr int LDC = C + PADO;     // L o P rows (OT)
  static constexpr int LDAB = C + PADO;    // -A rows (OT)
  static constexpr int LDT = 16 + PADO;    // T_ii rows (OT)
  static constexpr int LDD = 20;           // diagonal blocks of A in float, transposed
  static constexpr size_t KH = 0;
  static constexpr size_t QH = KH + (size_t)C * LDK * sizeof(IT);
  static constexpr size_t VH = QH + (size_t)C * LDK * sizeof(IT);
  static constexpr size_t KG = ALIAS ? KH : VH + (size_t)C * LDV * sizeof(IT);
  static constexpr size_t QG = ALIAS ? QH : KG + (size_t)C * LDKO * sizeof(OT);
  static constexpr size_t KE = ALIAS ? VH + (size_t)C * LDV * sizeof(IT) : QG + (size_t)C * LDKO * sizeof(OT);
  static constexpr size_t GC = KE + (size_t)C * LDKO * sizeof(OT);
  static constexpr size_t BETA = GC + (size_t)C * LDG * 4;
  static constexpr size_t TOT = BETA + C * 4;  // 512 floats: the scan's partial sums
  static constexpr size_t SQ = TOT + 512 * 4;
  static constexpr size_t AB_ = SQ + (size_t)C * LDC * sizeof(OT);
  static constexpr size_t TB = AB_ + (size_t)C * LDAB * sizeof(OT);
  static constexpr size_t AD = TB + (size_t)C * LDT * sizeof(OT);
  static constexpr size_t BYTES = AD + (size_t)C * LDD * 4;
  static_assert(KH % 16 == 0 && QH % 16 == 0 && VH % 16 == 0 && KG % 16 == 0 && QG % 16 == 0 &&
                    KE % 16 == 0 && GC % 16 == 0 && SQ % 16 == 0 && AB_ % 16 == 0 &&
                    TB % 16 == 0 && AD % 16 == 0,
                "16-byte aligned regions");
};

// Eight consecutive K-elements of row `row` (an MFMA fragment's piece) from a
// staged row, each times its factor, as an operand fragment (RNE to BF16
// unless F32).
template <bool F32, typename T>
__device__ __forceinline__ Frag<F32> scaled_frag(const T *row, const float *fac) {
  float x[8];
  if constexpr (sizeof(T) == 2) {
    const uint4 u = *reinterpret_cast<const uint4 *>(row);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16_lo(w[j]);
      x[2 * j + 1] = bf16_hi(w[j]);
    }
  } else {
    const float4 a = reinterpret_cast<const float4 *>(row)[0];
    const float4 b = reinterpret_cast<const float4 *>(row)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  Frag<F32> f;
  if constexpr (F32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) f.v[j] = x[j] * fac[j];
  } else {
    // pairs through the hardware RNE conversion, then the raw bits
    const uint4 u = make_uint4(pack_bf16x2(x[0] * fac[0], x[1] * fac[1]),
                               pack_bf16x2(x[2] * fac[2], x[3] * fac[3]),
                               pack_bf16x2(x[4] * fac[4], x[5] * fac[5]),
                               pack_bf16x2(x[6] * fac[6], x[7] * fac[7]));
    f.v = __builtin_bit_cast(bf16x8_t, u);
  }
  return f;
}

__device__ __forceinline__ void load8f(const float *p, float *x) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t *p, float *x) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_lo(w[j]);
    x[2 * j + 1] = bf16_hi(w[j]);
  }
}
__device__ __forceinline__ void load8(const float *p, float *x) { load8f(p, x); }

// Eight (sixteen) consecutive values of an operand row: BF16 pairs through the
// hardware RNE conversion stored as whole words, or floats as they are.
__device__ __forceinline__ void put_row8(uint16_t *p, const float *x) {
  *reinterpret_cast<uint4 *>(p) = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                             pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
}
__device__ __forceinline__ void put_row8(float *p, const float *x) {
  reinterpret_cast<float4 *>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4 *>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}
template <typename T>
__device__ __forceinline__ void put_row16(T *p, const float *x) {
  put_row8(p, x);
  put_row8(p + 8, x + 8);
}

// The chunk-local tiles that wave w forms: (I, J) pairs, a diagonal tile
// (I = J) first.  Four waves: wave w its diagonal tile (w, w) and two (waves
// 0, 1) or one (waves 2, 3) below the diagonal.  Eight waves: waves 0-3 the
// diagonal tiles, waves 4-7 the six below.
struct CwTiles {
  int n;
  int ij[3][2];
};
constexpr CwTiles kCwTiles4[4] = {{3, {{0, 0}, {1, 0}, {2, 1}}},
                                  {3, {{1, 1}, {2, 0}, {3, 2}}},
                                  {2, {{2, 2}, {3, 0}, {0, 0}}},
                                  {2, {{3, 3}, {3, 1}, {0, 0}}}};
constexpr CwTiles kCwTiles8[8] = {{1, {{0, 0}, {0, 0}, {0, 0}}}, {1, {{1, 1}, {0, 0}, {0, 0}}},
                                  {1, {{2, 2}, {0, 0}, {0, 0}}}, {1, {{3, 3}, {0, 0}, {0, 0}}},
                                  {2, {{1, 0}, {2, 1}, {0, 0}}}, {2, {{2, 0}, {3, 2}, {0, 0}}},
                                  {1, {{3, 0}, {0, 0}, {0, 0}}}, {1, {{3, 1}, {0, 0}, {0, 0}}}};
// Largest decay span (log2 units) of a diagonal tile formed by MFMA: column
// factors up to 2^100, products of unit-norm rows far below FP32's 2^128.
constexpr float kCwDiagSpan = 100.f;

// Waves of the channel-wise chain: 8 (two per SIMD) where each wave's
// registers fit in half a SIMD's file, else 4.
template <int DK, int DV, bool F32>
constexpr int kCwWaves = 8;

template <bool SB, bool AB, int DK, int DV, bool F32, bool CK = false>
__device__ __forceinline__ void prefill_chain_cw(const PrefillParams &p, int chain, char *smem) {
  constexpr int NW = kCwWaves<DK, DV, F32>, NT = 64 * NW;
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  using L = CwLayout<DK, DV, F32, AB>;
  using IT = typename L::IT;
  using OT = typename L::OT;
  using AT = typename Elem<AB>::T;
  static_assert(sizeof(AT) == sizeof(IT), "inputs are staged in the activation dtype");
  constexpr int C = L::C, DKP = L::DKP;
  constexpr int LDKO = L::LDKO, LDV = L::LDV, LDG = L::LDG, LDC = L::LDC;
  constexpr int NKB = DKP / 32;    // MFMA K-steps over d_k
  constexpr int DKB = DK / 16;     // 16-row blocks of d_k
  constexpr int DVB = DV / 16;     // 16-column blocks of d_v
  constexpr int NA = DVB >= NW ? DVB / NW : 1;
  constexpr int RING = 4;
  constexpr int EW = 8 * (int)sizeof(AT) / 16;
  constexpr int KQ_GROUPS = C * (DK / 8), KQ_PER = (KQ_GROUPS + NT - 1) / NT;
  constexpr int V_GROUPS = C * (DV / 8), V_PER = (V_GROUPS + NT - 1) / NT;
  constexpr int TPC = NT / DK, TOK = C / TPC;  // decay scan: threads per channel, tokens each
  constexpr int G_GROUPS = C * (DK / 4), G_PER = (G_GROUPS + NT - 1) / NT;  // decays, 4 per load
  static_assert(TPC * DK == NT && TPC * TOK == C, "whole channel columns per scan thread");
  constexpr float LOG2E = 1.4426950408889634f;

  IT *const Kh = reinterpret_cast<IT *>(smem + L::KH);
  IT *const Qh = reinterpret_cast<IT *>(smem + L::QH);
  IT *const Vh = reinterpret_cast<IT *>(smem + L::VH);
  OT *const Kg = reinterpret_cast<OT *>(smem + L::KG);
  OT *const Qg = reinterpret_cast<OT *>(smem + L::QG);
  OT *const Ke = reinterpret_cast<OT *>(smem + L::KE);
  float *const Gc = reinterpret_cast<float *>(smem + L::GC);
  float *const bet = reinterpret_cast<float *>(smem + L::BETA);
  float *const tot = reinterpret_cast<float *>(smem + L::TOT);
  OT *const Sq = reinterpret_cast<OT *>(smem + L::SQ);
  OT *const Ab = reinterpret_cast<OT *>(smem + L::AB_);
  OT *const Tb = reinterpret_cast<OT *>(smem + L::TB);
  float *const Ad = reinterpret_cast<float *>(smem + L::AD);

  const int seq = chain / p.H_v, h = chain % p.H_v, hq = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, rq = 4 * (lane >> 4);  // accumulator layout: rows rq..rq+3, column col
  const int64_t t_begin = p.cu[seq], t_end = p.cu[seq + 1];
  const int64_t rs = p.read_slot ? (int64_t)p.read_slot[seq] : seq;
  const int64_t ws = p.write_slot ? (int64_t)p.write_slot[seq] : seq;
  if (rs < -1 || rs >= p.n_slots || ws < -1 || ws >= p.n_slots) {
    if (tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
    return;
  }
  if (t_begin < 0 || t_end < t_begin || t_end > p.n_tokens) {
    if (tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SEQ);
    return;
  }
  const bool decay = (p.rule & kRuleDecay) != 0;
  const bool erase = (p.rule & kRuleErase) != 0;
  const float ef = erase ? 1.f : 0.f;

  // ---- prefetch of one chunk's inputs into registers ----
  // Rows past the sequence's end re-read its last token; staging gives them
  // beta = 0 and no decay, so they reach neither M nor a stored O row.
  u32x4_t pk[KQ_PER][EW], pq[KQ_PER][EW], pv[V_PER][EW];
  float4 pg4[G_PER];          // log-decays, 4 channels of a token per entry
  float pb = 0.f;             // wave 0: write strength of token `lane`
  const int gch = tid % DK, gpart = tid / DK;
  const int64_t kq_row = (int64_t)p.H_qk * DK, v_row = (int64_t)p.H_v * DV;
  auto fetch = [&](int64_t t0) {
    const int64_t last = t_end - 1;
    const AT *const kb = static_cast<const AT *>(p.k) + hq * DK;
    const AT *const qb = static_cast<const AT *>(p.q) + hq * DK;
    const AT *const vb = static_cast<const AT *>(p.v) + h * DV;
#pragma unroll
    for (int i = 0; i < KQ_PER; ++i) {
      const int gi = tid + NT * i;
      if (KQ_GROUPS % NT != 0 && gi >= KQ_GROUPS) continue;
      const int64_t t = std::min<int64_t>(t0 + gi / (DK / 8), last);
      const int64_t off = t * kq_row + (gi % (DK / 8)) * 8;
      const u32x4_t *sk = reinterpret_cast<const u32x4_t *>(kb + off);
      const u32x4_t *sq = reinterpret_cast<const u32x4_t *>(qb + off);
#pragma unroll
      for (int e = 0; e < EW; ++e) { pk[i][e] = sk[e]; pq[i][e] = sq[e]; }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int gi = tid + NT * i;
      if (V_GROUPS % NT != 0 && gi >= V_GROUPS) continue;
      const int64_t t = std::min<int64_t>(t0 + gi / (DV / 8), last);
      const u32x4_t *sv = reinterpret_cast<const u32x4_t *>(vb + t * v_row + (gi % (DV / 8)) * 8);
#pragma unroll
      for (int e = 0; e < EW; ++e) pv[i][e] = sv[e];
    }
#pragma unroll
    for (int i = 0; i < G_PER; ++i) {
      const int gi = tid + NT * i;
      if (G_GROUPS % NT != 0 && gi >= G_GROUPS) continue;
      const int64_t t = std::min<int64_t>(t0 + gi / (DK / 4), last);
      pg4[i] = decay ? *reinterpret_cast<const float4 *>(p.g + (t * p.H_v + h) * DK + (gi % (DK / 4)) * 4)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (wave == 0) {
      const int64_t t = std::min<int64_t>(t0 + lane, last);
      pb = erase ? p.beta[t * p.H_v + h] : 1.f;
    }
  };

  // ---- staging of the prefetched chunk (n real rows) and the decay scan ----
  auto stage = [&](int n) {
#pragma unroll
    for (int i = 0; i < KQ_PER; ++i) {
      const int gi = tid + NT * i;
      if (KQ_GROUPS % NT != 0 && gi >= KQ_GROUPS) continue;
      const int r = gi / (DK / 8), d = (gi % (DK / 8)) * 8;
      u32x4_t *dk = reinterpret_cast<u32x4_t *>(Kh + L::ak(r, d));
      u32x4_t *dq = reinterpret_cast<u32x4_t *>(Qh + L::ak(r, d));
#pragma unroll
      for (int e = 0; e < EW; ++e) { dk[e] = pk[i][e]; dq[e] = pq[i][e]; }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int gi = tid + NT * i;
      if (V_GROUPS % NT != 0 && gi >= V_GROUPS) continue;
      const int r = gi / (DV / 8), c = (gi % (DV / 8)) * 8;
      u32x4_t *dv = reinterpret_cast<u32x4_t *>(Vh + L::av(r, c));
#pragma unroll
      for (int e = 0; e < EW; ++e) dv[e] = pv[i][e];
    }
    if (wave == 0) bet[lane] = lane < n ? pb : 0.f;
    // the log2 decays into G's rows (rows past the end decay nothing), then
    // per channel an inclusive scan down the column: each thread its TOK
    // tokens, then the totals of the parts above it
#pragma unroll
    for (int i = 0; i < G_PER; ++i) {
      const int gi = tid + NT * i;
      if (G_GROUPS % NT != 0 && gi >= G_GROUPS) continue;
      const int r = gi / (DK / 4);
      const float m = r < n ? LOG2E : 0.f;
      reinterpret_cast<float4 *>(Gc + r * LDG)[gi % (DK / 4)] =
          make_float4(pg4[i].x * m, pg4[i].y * m, pg4[i].z * m, pg4[i].w * m);
    }
    __syncthreads();
    float part[TOK];
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < TOK; ++j) {
      acc += Gc[(gpart * TOK + j) * LDG + gch];
      part[j] = acc;
    }
    tot[gpart * DK + gch] = acc;
    __syncthreads();
    float pre = 0.f;
    for (int pp = 0; pp < gpart; ++pp) pre += tot[pp * DK + gch];
#pragma unroll
    for (int j = 0; j < TOK; ++j) Gc[(gpart * TOK + j) * LDG + gch] = pre + part[j];
  };

  // O rows of the chunk from the accumulator layout (the plain chain's store)
  AT *const o_head = static_cast<AT *>(p.o) + (int64_t)h * DV;
  const int64_t o_row = (int64_t)p.H_v * DV;
  const bool o_odd = (col & 1) != 0;
  const uint32_t o_lane = AB ? (uint32_t)((rq + (o_odd ? 2 : 0)) * o_row + (col & ~1))
                             : (uint32_t)(rq * o_row + col);
  AT *o_base = o_head;
  int o_n = 0;
  auto store_o_tile = [&](int r0, int c0, const f32x4_t &acc, bool whole) {
    AT *const dst = o_base + r0 * o_row + c0 + o_lane;
    if constexpr (AB) {
      const uint32_t a = pack_bf16x2(acc[0], acc[1]);
      const uint32_t b = pack_bf16x2(acc[2], acc[3]);
      const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o_odd ? a : b), 0xB1, 0xf, 0xf, false);
      const uint32_t own = o_odd ? b : a;
      const uint32_t left = o_odd ? other : own, right = o_odd ? own : other;
      const uint32_t w0 = __builtin_amdgcn_perm(right, left, 0x05040100u);
      const uint32_t w1 = __builtin_amdgcn_perm(right, left, 0x07060302u);
      const int r = r0 + rq + (o_odd ? 2 : 0);
      if (whole || r < o_n) *reinterpret_cast<uint32_t *>(dst) = w0;
      if (whole || r + 1 < o_n) *reinterpret_cast<uint32_t *>(dst + o_row) = w1;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (whole || r0 + rq + e < o_n) dst[e * o_row] = acc[e];
    }
  };

  // ---- set-up: zero the padding that no chunk writes ----
  // K columns past d_k (d_k < 32), G columns past d_k, and the two tiles above
  // the diagonal that the read-out's 32-wide slabs of L o P read
  if constexpr (DKP > DK) {
    for (int i = tid; i < C * (DKP - DK); i += NT) {
      const int r = i / (DKP - DK), c = DK + i % (DKP - DK);
      put(Kh + L::ak(r, c), 0.f);
      put(Qh + L::ak(r, c), 0.f);
      Gc[r * LDG + c] = 0.f;
    }
  }
  for (int i = tid; i < 2 * 256; i += NT) {
    const int t = i >> 8, r = 32 * t + ((i >> 4) & 15), c = 32 * t + 16 + (i & 15);
    put(Sq + r * LDC + c, 0.f);
  }

  // ---- initial state (a8): read slot -> FP32 accumulators ----
  f32x4_t macc[DKB][NA];
  const int64_t state_base = (rs * p.H_v + h) * (int64_t)DK * DV;
#pragma unroll
  for (int b = 0; b < DKB; ++b)
#pragma unroll
    for (int ia = 0; ia < NA; ++ia)
#pragma unroll
      for (int e = 0; e < 4; ++e) macc[b][ia][e] = 0.f;
  const bool mwave = DVB >= NW || wave < DVB;
  if (mwave && rs >= 0) {
#pragma unroll
    for (int b = 0; b < DKB; ++b)
#pragma unroll
      for (int ia = 0; ia < NA; ++ia) {
        const int d = 16 * b + rq, c = 16 * (wave * NA + ia) + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          macc[b][ia][e] = Elem<SB>::load1(p.pool, state_base + (int64_t)(d + e) * DV + c);
      }
  }
  auto store_state = [&](int64_t slot) {
    const int64_t out_base = (slot * p.H_v + h) * (int64_t)DK * DV;
#pragma unroll
    for (int b = 0; b < DKB; ++b)
#pragma unroll
      for (int ia = 0; ia < NA; ++ia) {
        const int d = 16 * b + rq, c = 16 * (wave * NA + ia) + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Elem<SB>::store1(p.pool, out_base + (int64_t)(d + e) * DV + c, macc[b][ia][e]);
      }
  };

  if (t_begin < t_end) fetch(t_begin);
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t t0 = t_begin; t0 < t_end; t0 += C) {
    const int64_t t1 = t0 + C;
    const int n = (int)std::min<int64_t>(C, t_end - t0);
    o_base = o_head + t0 * o_row;
    o_n = n;

    // 1: this chunk's inputs into LDS, G = per-channel cumulative log2 decays
    stage(n);
    __syncthreads();
    // the next chunk's inputs, in flight while this one computes (clamped to
    // the last token on the last chunk: no branch around the loads)
    fetch(t1);

    // 2: chunk-local products, one MFMA product per tile from fragments
    // scaled through the tile's reference token m; the wave's diagonal tile
    // only while its decay span allows (a wave-uniform decision)
    const bool dwave = wave < 4;  // owns diagonal tile `wave`
    float span = 0.f;
    if (dwave)
      for (int c = lane; c < DK; c += 64)
        span = fmaxf(span, Gc[(16 * wave) * LDG + c] - Gc[(16 * wave + 15) * LDG + c]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) span = fmaxf(span, __shfl_xor(span, off));
    const bool diag_mfma = span <= kCwDiagSpan;
    const CwTiles &tw = NW == 8 ? kCwTiles8[wave] : kCwTiles4[wave];
#pragma unroll
    for (int ti = 0; ti < 3; ++ti) {
      if (ti >= tw.n) break;
      const int I = tw.ij[ti][0], J = tw.ij[ti][1];
      const bool dg = I == J;
      if (dg && !diag_mfma) continue;
      const int m = dg ? 16 * J : 16 * J + 15;
      const int rl = 16 * I + (lane & 15), rr = 16 * J + (lane & 15);
      f32x4_t sa, pa;
#pragma unroll
      for (int kk = 0; kk < NKB; ++kk) {
        const int ch = 32 * kk + 8 * (lane >> 4);
        float gl[8], gr[8], gm[8], fl[8], fr[8];
        load8f(Gc + rl * LDG + ch, gl);
        load8f(Gc + rr * LDG + ch, gr);
        load8f(Gc + m * LDG + ch, gm);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          fl[e] = fast_exp2(gl[e] - gm[e]);  // <= 1: r at or after m
          fr[e] = fast_exp2(gm[e] - gr[e]);  // <= 1 below the diagonal, <= 2^span on it
        }
        const Frag<F32> fkl = scaled_frag<F32>(Kh + L::ak(16 * I, 32 * kk, lane & 15, 8 * (lane >> 4)), fl);
        const Frag<F32> fql = scaled_frag<F32>(Qh + L::ak(16 * I, 32 * kk, lane & 15, 8 * (lane >> 4)), fl);
        const Frag<F32> fkr = scaled_frag<F32>(Kh + L::ak(16 * J, 32 * kk, lane & 15, 8 * (lane >> 4)), fr);
        sa = mma<F32>(kk == 0 ? z : sa, fkl, fkr);
        pa = mma<F32>(kk == 0 ? z : pa, fql, fkr);
      }
      const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * I + rq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * I + rq + e, s = 16 * J + col;
        if (dg) {
          // strictly lower entries of A, lower entries and the diagonal of P
          const float a = s < r ? ef * br[e] * sa[e] : 0.f;
          put(Ab + r * L::LDAB + s, -a);
          put(Sq + r * LDC + s, s <= r ? p.scale * pa[e] : 0.f);
          Ad[(16 * I + col) * L::LDD + rq + e] = a;
        } else {
          put(Ab + r * L::LDAB + s, -(ef * br[e]) * sa[e]);
          put(Sq + r * LDC + s, p.scale * pa[e]);
        }
      }
    }
    // 3: a diagonal tile whose span is too wide for the scaled product,
    // entry by entry: lane (r, cg) sums channels cg*8 + 32 j .. +8 of every
    // column s; the four cg lanes of a row then add
    if (dwave && !diag_mfma) {
      const int b = wave, r = lane & 15, cg = lane >> 4;
      float accA[16], accP[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) accA[s] = accP[s] = 0.f;
      for (int c0 = 8 * cg; c0 < DK; c0 += 32) {
        float kr[8], qr[8], gr[8];
        load8(Kh + L::ak(16 * b + r, c0), kr);
        load8(Qh + L::ak(16 * b + r, c0), qr);
        load8f(Gc + (16 * b + r) * LDG + c0, gr);
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          float ks[8], gs[8];
          load8(Kh + L::ak(16 * b + s, c0), ks);
          load8f(Gc + (16 * b + s) * LDG + c0, gs);
          float ta = 0.f, tp = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            // e^(G_r - G_s) <= 1 for s <= r; the entries above are not used
            const float kw = ks[e] * fast_exp2(fminf(gr[e] - gs[e], 0.f));
            ta = fmaf(kr[e], kw, ta);
            tp = fmaf(qr[e], kw, tp);
          }
          accA[s] += ta;
          accP[s] += tp;
        }
      }
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        accA[s] += __shfl_xor(accA[s], 16);
        accA[s] += __shfl_xor(accA[s], 32);
        accP[s] += __shfl_xor(accP[s], 16);
        accP[s] += __shfl_xor(accP[s], 32);
      }
      if (cg == 0) {
        const float bw = ef * bet[16 * b + r];
        float a16[16], p16[16];
#pragma unroll
        for (int s = 0; s < 16; ++s) {
          a16[s] = s < r ? -bw * accA[s] : 0.f;   // -A
          p16[s] = s <= r ? p.scale * accP[s] : 0.f;
          Ad[(16 * b + s) * L::LDD + r] = -a16[s];
        }
        put_row16(Ab + (16 * b + r) * L::LDAB + 16 * b, a16);
        put_row16(Sq + (16 * b + r) * LDC + 16 * b, p16);
      }
    }
    __syncthreads();

    // 4: T_bb = (I + A_bb)^-1 by forward substitution (wave b, lane c <
    // 16: column c) in right-looking order: once x_s is final, every later
    // row takes its term -A[r][s] x_s, so a step waits on one FMA rather than
    // on a row's chain, and each row still adds its terms in the order
    // s = 0, 1, ...  A_bb is stored transposed (row 16 b + s of Ad holds
    // column s of the block), so step s reads its column as 16-byte loads.
    // Then the per-channel scalings of K and Q.
    {
      const int b = wave, c = lane;
      if (dwave && c < 16) {
        const float *const At = Ad + 16 * b * L::LDD;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = r == c ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < 15; ++s) {
          float ac[16];
#pragma unroll
          for (int q4 = (s + 1) / 4; q4 < 4; ++q4) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t *>(At + s * L::LDD + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) ac[4 * q4 + e] = v[e];
          }
#pragma unroll
          for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-ac[r], x[s], x[r]);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) put(Tb + (16 * b + r) * L::LDT + c, x[r]);
      }
    }
    // with 8 waves the scalings run on waves 4-7 alone, beside waves 0-3's
    // substitutions (0.4% faster than sharing them out over all eight)
    constexpr int XT = NW == 8 ? NT - 256 : NT;  // threads that scale
    for (int i = NW == 8 ? tid - 256 : tid; i < C * (DKP / 8); i += XT) {
      if (i < 0) break;
      const int r = i / (DKP / 8), c = (i % (DKP / 8)) * 8;
      float kx[8], qx[8], g8[8], gl8[8];
      load8(Kh + L::ak(r, c), kx);
      load8(Qh + L::ak(r, c), qx);
      load8f(Gc + r * LDG + c, g8);
      load8f(Gc + (C - 1) * LDG + c, gl8);
      float kg[8], qg[8], ke[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float eg = fast_exp2(g8[e]);
        kg[e] = kx[e] * eg;
        qg[e] = qx[e] * eg;
        ke[e] = kx[e] * fast_exp2(gl8[e] - g8[e]);
      }
      put_row8(Kg + L::ako(r, c), kg);
      put_row8(Qg + L::ako(r, c), qg);
      put_row8(Ke + L::ako(r, c), ke);
    }
    __syncthreads();

    // 5-8: the wave's d_v columns, in registers (the plain chain's steps)
    f32x4_t qm[4][NA], um[4][NA];
    if (mwave) {
      constexpr int NF = NKB * 8;  // (slab, row block, q or k)
      Frag<F32> fa[RING];
      Frag<F32> fm[NA];
      auto load_a = [&](int f) {
        if constexpr (L::SWK) return rows_afrag<typename L::RS>((f & 1) ? Kg : Qg, 16 * ((f >> 1) & 3), 32 * (f >> 3));
        else return load_afrag<F32>((f & 1) ? Kg : Qg, LDKO, 16 * ((f >> 1) & 3), 32 * (f >> 3));
      };
#pragma unroll
      for (int f = 0; f < RING - 1; ++f) fa[f] = load_a(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kk = f >> 3, tb = (f >> 1) & 3, isk = f & 1;
        if (f + RING - 1 < NF) fa[(f + RING - 1) % RING] = load_a(f + RING - 1);
        if ((f & 7) == 0) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia)
            fm[ia] = bfrag<F32>(macc[2 * kk][ia], 2 * kk + 1 < DKB ? macc[2 * kk + 1][ia] : z);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
          if (isk) um[tb][ia] = mma<F32>(kk == 0 ? z : um[tb][ia], fa[f % RING], fm[ia]);
          else qm[tb][ia] = mma<F32>(kk == 0 ? z : qm[tb][ia], fa[f % RING], fm[ia]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // R = beta (V - K_g M) (delta rules) or V; in place in um
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        float vv[NA][4];
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
          if constexpr (L::SWV) rows_col4<typename L::RS>(Vh, 16 * tb, 16 * (wave * NA + ia), vv[ia]);
          else load_col4(Vh, LDV, 16 * tb, 16 * (wave * NA + ia), vv[ia]);
        }
        const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * tb + rq);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) um[tb][ia][e] = br[e] * (vv[ia][e] - ef * um[tb][ia][e]);
      }
      // U = (I + A)^-1 R by block forward substitution (delta rules)
      if (erase) {
        Frag16<F32> fa16[6], ft[4];
#pragma unroll
        for (int i = 1, nn = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < i; ++j, ++nn) {
            if constexpr (F32) fa16[nn] = load_afrag16<F32>(Ab, L::LDAB, 16 * i, 16 * j, 1.f);
            else fa16[nn] = load_afrag16(Ab, L::LDAB, 16 * i, 16 * j);
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (F32) ft[i] = load_afrag16<F32>(Tb, L::LDT, 16 * i, 0, 1.f);
          else ft[i] = load_afrag16(Tb, L::LDT, 16 * i, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0, nn = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < i; ++j, ++nn)
#pragma unroll
            for (int ia = 0; ia < NA; ++ia)
              um[i][ia] = mma16<F32>(um[i][ia], fa16[nn], bfrag16<F32>(um[j][ia]));
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) um[i][ia] = mma16<F32>(z, ft[i], bfrag16<F32>(um[i][ia]));
        }
      }
      // O = scale Q_g M + (scale L o P) U, stored from the accumulator layout
      Frag<F32> fu[2][NA];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) fu[s2][ia] = bfrag<F32>(um[2 * s2][ia], um[2 * s2 + 1][ia]);
      Frag<F32> fs[6];
#pragma unroll
      for (int tb = 0, nn = 0; tb < 4; ++tb)
#pragma unroll
        for (int s2 = 0; s2 <= tb / 2; ++s2, ++nn) fs[nn] = load_afrag<F32>(Sq, LDC, 16 * tb, 32 * s2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0, nn = 0; tb < 4; ++tb) {
#pragma unroll
        for (int ia = 0; ia < NA; ++ia)
#pragma unroll
          for (int e = 0; e < 4; ++e) qm[tb][ia][e] *= p.scale;
#pragma unroll
        for (int s2 = 0; s2 <= tb / 2; ++s2, ++nn)
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) qm[tb][ia] = mma<F32>(qm[tb][ia], fs[nn], fu[s2][ia]);
        if (o_n == C) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) store_o_tile(16 * tb, 16 * (wave * NA + ia), qm[tb][ia], true);
        } else {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) store_o_tile(16 * tb, 16 * (wave * NA + ia), qm[tb][ia], false);
        }
      }
      // M <- Diag(e^G_last) M + K_e^T U: rows of M decay by their channel's
      // whole-chunk decay, then the chunk's writes
#pragma unroll
      for (int b = 0; b < DKB; ++b) {
        const f32x4_t gl = *reinterpret_cast<const f32x4_t *>(Gc + (C - 1) * LDG + 16 * b + rq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = fast_exp2(gl[e]);
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) macc[b][ia][e] *= a;
        }
      }
      {
        constexpr int NF = DKB * 2;  // (d_k block, token slab)
        constexpr int RK = RING < NF ? RING : NF;
        Frag<F32> fk[RK];
        auto load_k = [&](int f) {
          if constexpr (L::SWK) return rows_afrag_t<typename L::RS>(Ke, 16 * (f >> 1), 32 * (f & 1));
          else return load_afrag_t<F32>(Ke, LDKO, 16 * (f >> 1), 32 * (f & 1));
        };
#pragma unroll
        for (int f = 0; f < RK - 1; ++f) fk[f] = load_k(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + RK - 1 < NF) fk[(f + RK - 1) % RK] = load_k(f + RK - 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ia = 0; ia < NA; ++ia)
            macc[f >> 1][ia] = mma<F32>(macc[f >> 1][ia], fk[f % RK], fu[f & 1][ia]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // an intermediate checkpoint after this chunk (a uniform branch)
    if (CK && p.ckpt_chunks > 0 && t1 <= t_end && ((t1 - t_begin) / C) % p.ckpt_chunks == 0) {
      const int j = (int)((t1 - t_begin) / C / p.ckpt_chunks) - 1;
      if (j < p.ckpt_per_seq) {
        const int64_t cs = p.ckpt_slot[(int64_t)seq * p.ckpt_per_seq + j];
        if (cs >= 0 && cs < p.n_slots) {
          if (mwave) store_state(cs);
        } else if (cs != -1 && tid == 0 && p.status) {
          atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
        }
      }
    }
    __syncthreads();  // every reader of this chunk's LDS is done before the next staging
  }

  // ---- final state (a8): FP32 -> state dtype (RNE for BF16) -> write slot ----
  if (ws >= 0 && mwave) store_state(ws);
}

// LDS bytes of the channel-wise chain
template <int DK, int DV, bool F32, bool AB>
constexpr size_t kCwChainLds = CwLayout<DK, DV, F32, AB>::BYTES;

}  // namespace gdn
