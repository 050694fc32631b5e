// prefill_chain.cuh -- one (sequence, state head) chain of the chunked
// prefill, as a device function shared by the prefill kernel and the mixed
// launcher.  The algebra and the LDS layout are described in prefill.cuh.
//
// Latency: every global input of chunk c+1 (K and Q rows, V rows, gates) is
// loaded into registers while chunk c computes, and written to LDS at the
// end of chunk c, so no chunk waits on a global-memory round trip.  The
// workgroup barriers wait only on LDS (lgkmcnt), not on these loads.
//
// Work split over NW waves (4 or 8): the chunk-local half (S, P, A, L o P,
// T) is shared through LDS -- wave w forms the S and P tiles of row block
// w % 4 in 16 / NW of the four column blocks; the M-dependent half runs per
// wave on the wave's own d_v columns (NA column blocks of 16), entirely in
// registers.  With 8 waves two share each SIMD, so one's LDS and MFMA
// latencies are covered by the other's work.
#pragma once

#include <algorithm>

#include "prefill.cuh"

namespace gdn {

// Chain c of blockIdx b: inside each group of 16 blocks, chains 2m and 2m+1
// (the two state heads that share a q/k head when H_v = 2 H_qk) go to blocks
// m and m + 8, which the dispatcher places on the same XCD (blocks are dealt
// to the 8 XCDs round-robin), so their shared q/k rows meet in one L2.
__device__ __forceinline__ int chain_of_block(int b) {
  const int w = b & 15;
  return (b & ~15) + 2 * (w & 7) + (w >> 3);
}

// Waves per plain chain: 8 (two per SIMD, each covering the other's
// latencies) where the chain's registers fit in the 256 a wave then gets
// without spilling -- a spill reload inside the chunk loop would wait on the
// in-flight prefetch of the next chunk -- else 4.
template <int DK, int DV, bool F32>
constexpr int kPlainWaves = (!F32 && (DK <= 64 || DV == 128)) ? 8 : 4;

// Shapes that run the pipelined chain (prefill_pipe.cuh, always 8 waves):
// BF16 activations, whole 32-wide K slabs, and d_v a multiple of 64 so each
// of its four consumer waves owns whole 16-column blocks.
template <int DK, int DV, bool F32>
constexpr bool kPrefillPipe = !F32 && DK >= 32 && DV % 64 == 0;

// Waves per chain, whichever design runs it.
template <int DK, int DV, bool F32>
constexpr int kPrefillWaves = kPrefillPipe<DK, DV, F32> ? 8 : kPlainWaves<DK, DV, F32>;

// Chunk-local tiles of the 8-wave chain's product waves 4-7.  A fragment id
// is 2 b for block b (16 rows) of K and 2 b + 1 for block b of Q, one 32-wide
// slab at a time; a wave loads each fragment it needs once per slab, into the
// slot of its position in `frag`.
struct LocalTiles {
  int nf;        // fragments per slab
  int frag[6];   // fragment id of each slot
  int nod;       // tiles below the diagonal: S and P of (i, j)
  int od[2][5];  // i, j, and the slots of K_i, Q_i, K_j
  int ndp;       // diagonal tiles: P of (b, b)
  int dp[2][3];  // b, and the slots of Q_b, K_b
};
constexpr LocalTiles kLocalTiles[4] = {
    // wave 4: (1,0) (2,0) from K0 K1 Q1 K2 Q2
    {5, {0, 2, 3, 4, 5, 0}, 2, {{1, 0, 1, 2, 0}, {2, 0, 3, 4, 0}}, 0, {{0, 0, 0}, {0, 0, 0}}},
    // wave 5: (2,1) (3,0) from K1 K2 Q2 K0 K3 Q3
    {6, {2, 4, 5, 0, 6, 7}, 2, {{2, 1, 1, 2, 0}, {3, 0, 4, 5, 3}}, 0, {{0, 0, 0}, {0, 0, 0}}},
    // wave 6: (3,1), P of (1,1) and (0,0) from K3 Q3 K1 Q1 K0 Q0
    {6, {6, 7, 2, 3, 0, 1}, 1, {{3, 1, 0, 1, 2}, {0, 0, 0, 0, 0}}, 2, {{1, 3, 2}, {0, 5, 4}}},
    // wave 7: (3,2), P of (2,2) and (3,3) from K3 Q3 K2 Q2
    {4, {6, 7, 4, 5, 0, 0}, 1, {{3, 2, 0, 1, 2}, {0, 0, 0, 0, 0}}, 2, {{2, 3, 2}, {3, 1, 0}}},
};

// One (sequence, state head) chain; all 64 NW threads of the workgroup call
// it.  `smem` holds PrefillLayout<DK, DV, F32>::BYTES bytes, 16-byte aligned.
// CK: the instance that stores intermediate checkpoints (the launcher picks
// it only when they are asked for, so the others carry none of its code).
template <bool SB, bool AB, int DK, int DV, bool F32, int NW, bool CK = false>
__device__ __forceinline__ void prefill_chain(const PrefillParams &p, int chain, char *smem) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves per chain");
  constexpr int NT = 64 * NW;
  using L = PrefillLayout<DK, DV, F32, AB>;
  using OT = typename L::OT;  // L o P
  using IT = typename L::IT;  // staged K, Q, V rows
  using AT = typename Elem<AB>::T;
  static_assert(sizeof(AT) == sizeof(IT), "inputs are staged in the activation dtype");
  constexpr int C = L::C;
  constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF, LDV = L::LDV;
  constexpr int NKB = L::DKP / 32;  // MFMA K-steps over d_k
  constexpr int DKB = DK / 16;      // 16-row blocks of d_k
  constexpr int DVB = DV / 16;      // 16-column blocks of d_v
  constexpr int NA = DVB >= NW ? DVB / NW : 1;  // d_v blocks per wave
  constexpr int NCB = 16 / NW;                   // S / P column blocks per wave
  // With 4 waves the wave's T rows ride along the Q M / K M MFMA steps; with 8
  // the partner wave on the SIMD fills those gaps instead.
  constexpr bool kInterleaveT = NW == 4;
  // LDS operand fragments kept in flight ahead of the MFMA that uses them: one
  // 16x16x32 MFMA is 16 cycles, an LDS round trip several times that
  constexpr int RING = 4;
  // BF16 operands: -A and T_ii are stored in BF16 ready for the
  // substitution's MFMAs (no FP32 reader needs them)
  constexpr bool kBfAT = !F32;
  constexpr int EW = 8 * (int)sizeof(AT) / 16;  // 16-byte vectors per 8 elements
  constexpr int KQ_GROUPS = C * (DK / 8), KQ_PER = (KQ_GROUPS + NT - 1) / NT;
  constexpr int V_GROUPS = C * (DV / 8), V_PER = (V_GROUPS + NT - 1) / NT;
  constexpr float LOG2E = 1.4426950408889634f;
  // this chunk's input set (K, Q, V rows and gates); the sets alternate
  IT *Kh, *Qh, *Vh;
  float *Gs, *gam, *bet, *eGn;  // cumulative log2 decay, gamma, beta, exp(G_last - G)
  float *gsc, *gme;             // scale * gamma (the read-out), e * gamma (R's K M term)
  auto use_set = [&](int b) {
    char *base = smem + b * L::SET;
    Kh = reinterpret_cast<IT *>(base + L::KH);
    Qh = reinterpret_cast<IT *>(base + L::QH);
    Vh = reinterpret_cast<IT *>(base + L::VH);
    Gs = reinterpret_cast<float *>(base + L::GATES);
    gam = Gs + C; bet = Gs + 2 * C; eGn = Gs + 3 * C; gsc = Gs + 4 * C; gme = Gs + 5 * C;
  };
  OT *Sq = reinterpret_cast<OT *>(smem + L::SQ);
  float *Af = reinterpret_cast<float *>(smem + L::AF);
  float *Tf = reinterpret_cast<float *>(smem + L::TF);  // T_ii = (I + A_ii)^-1, stacked
  uint16_t *Ab = reinterpret_cast<uint16_t *>(smem + L::AF);  // kBfAT: -A in BF16
  uint16_t *Tb = reinterpret_cast<uint16_t *>(smem + L::TF);  // kBfAT: T_ii in BF16

  const int seq = chain / p.H_v, h = chain % p.H_v, hq = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, rq = 4 * (lane >> 4);  // accumulator layout: rows rq..rq+3, column col
  const int RB = wave & 3, cb0 = (wave >> 2) * NCB;  // the wave's S / P row block and column blocks
  // the wave forms T_RB,RB = (I + A_RB,RB)^-1: with 8 waves waves 0-3, with 4
  // every wave (it holds diagonal block RB of A)
  const bool diag = NW == 8 ? wave < 4 : (cb0 <= RB && RB < cb0 + NCB);
  const int64_t t_begin = p.cu[seq], t_end = p.cu[seq + 1];
  const int64_t rs = p.read_slot ? (int64_t)p.read_slot[seq] : seq;
  const int64_t ws = p.write_slot ? (int64_t)p.write_slot[seq] : seq;
  if (rs < -1 || rs >= p.n_slots || ws < -1 || ws >= p.n_slots) {
    if (tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
    return;
  }
  if (t_begin < 0 || t_end < t_begin || t_end > p.n_tokens) {  // offsets break the contract
    if (tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SEQ);
    return;
  }
  const bool decay = (p.rule & kRuleDecay) != 0;
  const bool erase = (p.rule & kRuleErase) != 0;
  // 1 for the delta rules, else 0: a factor rather than a branch, so no LDS
  // load ends up inside a branch of its own (that costs a round trip each)
  const float ef = erase ? 1.f : 0.f;

  // ---- prefetch of one chunk's inputs into registers, and their staging ----
  // The loads are unconditional: a row past the sequence's end re-reads its
  // last token.  Such padded rows are harmless because their beta factor is
  // zero: their rows of A and U vanish, so they reach neither M nor a stored
  // O row.  (Held as vector values, so they stay in registers.)
  u32x4_t pk[KQ_PER][EW], pq[KQ_PER][EW], pv[V_PER][EW];
  float pg = 0.f, pb = 0.f;  // wave 0: gate inputs of token `lane`
  bool p_valid = false;       // wave 0: token `lane` lies inside the sequence
  // Addressing: a thread's load i of a chunk reads row r0 + i * RS (RS rows
  // between the thread's loads), so its offset is a per-thread part fixed for
  // the chain plus a uniform one; only a sequence's last chunk clamps rows.
  constexpr int KQ_RS = NT / (DK / 8), V_RS = NT / (DV / 8);
  const int64_t kq_row = (int64_t)p.H_qk * DK, v_row = (int64_t)p.H_v * DV;  // elements per token
  const int kq_r0 = tid / (DK / 8), v_r0 = tid / (DV / 8);
  const uint32_t kq_lane = (uint32_t)(kq_r0 * kq_row + (tid % (DK / 8)) * 8);
  const uint32_t v_lane = (uint32_t)(v_r0 * v_row + (tid % (DV / 8)) * 8);
  const uint32_t g_lane = (uint32_t)(lane * p.H_v);
  auto fetch = [&](int64_t t0) {
    const int64_t last = t_end - 1;
    const AT *const kb = static_cast<const AT *>(p.k) + t0 * kq_row + hq * DK;
    const AT *const qb = static_cast<const AT *>(p.q) + t0 * kq_row + hq * DK;
    const AT *const vb = static_cast<const AT *>(p.v) + t0 * v_row + h * DV;
    if (t0 + C - 1 <= last) {  // a whole chunk: no clamping
#pragma unroll
      for (int i = 0; i < KQ_PER; ++i) {
        // threads past the chunk's groups (small d_k only) load nothing: their
        // rows would lie past the chunk, and stage() skips them
        if (KQ_GROUPS % NT != 0 && tid + NT * i >= KQ_GROUPS) continue;
        const int64_t off = kq_lane + (int64_t)i * KQ_RS * kq_row;
        const u32x4_t *sk = reinterpret_cast<const u32x4_t *>(kb + off);
        const u32x4_t *sq = reinterpret_cast<const u32x4_t *>(qb + off);
#pragma unroll
        for (int e = 0; e < EW; ++e) { pk[i][e] = sk[e]; pq[i][e] = sq[e]; }
      }
#pragma unroll
      for (int i = 0; i < V_PER; ++i) {
        if (V_GROUPS % NT != 0 && tid + NT * i >= V_GROUPS) continue;
        const u32x4_t *sv = reinterpret_cast<const u32x4_t *>(vb + v_lane + (int64_t)i * V_RS * v_row);
#pragma unroll
        for (int e = 0; e < EW; ++e) pv[i][e] = sv[e];
      }
    } else {
      const int rmax = (int)(last - t0);
#pragma unroll
      for (int i = 0; i < KQ_PER; ++i) {
        const int gi = tid + NT * i;
        const int r = std::min(gi / (DK / 8), rmax), d = (gi % (DK / 8)) * 8;
        const int64_t off = r * kq_row + d;
        const u32x4_t *sk = reinterpret_cast<const u32x4_t *>(kb + off);
        const u32x4_t *sq = reinterpret_cast<const u32x4_t *>(qb + off);
#pragma unroll
        for (int e = 0; e < EW; ++e) { pk[i][e] = sk[e]; pq[i][e] = sq[e]; }
      }
#pragma unroll
      for (int i = 0; i < V_PER; ++i) {
        const int gi = tid + NT * i;
        const int r = std::min(gi / (DV / 8), rmax), c = (gi % (DV / 8)) * 8;
        const u32x4_t *sv = reinterpret_cast<const u32x4_t *>(vb + r * v_row + c);
#pragma unroll
        for (int e = 0; e < EW; ++e) pv[i][e] = sv[e];
      }
    }
    if (wave == 0) {
      // raw values only: any arithmetic on them here would wait for the whole
      // fetch (loads retire in order); stage() masks them.  g and beta may be
      // NULL under the rules that do not use them.
      const int64_t gt = t0 * p.H_v + h + (t0 + lane <= last ? (int64_t)g_lane : (last - t0) * p.H_v);
      if (decay) pg = p.g[gt];
      if (erase) pb = p.beta[gt];
      p_valid = t0 + lane <= last;
    }
  };
  auto stage = [&](int b) {  // into input set b
    char *base = smem + b * L::SET;
    IT *const sK = reinterpret_cast<IT *>(base + L::KH), *const sQ = reinterpret_cast<IT *>(base + L::QH);
    IT *const sV = reinterpret_cast<IT *>(base + L::VH);
    float *const sG = reinterpret_cast<float *>(base + L::GATES);
#pragma unroll
    for (int i = 0; i < KQ_PER; ++i) {
      const int gi = tid + NT * i;
      if (KQ_GROUPS % NT != 0 && gi >= KQ_GROUPS) continue;
      const int r = gi / (DK / 8), d = (gi % (DK / 8)) * 8;
      u32x4_t *dk = reinterpret_cast<u32x4_t *>(sK + r * LDK + d);
      u32x4_t *dq = reinterpret_cast<u32x4_t *>(sQ + r * LDK + d);
#pragma unroll
      for (int e = 0; e < EW; ++e) { dk[e] = pk[i][e]; dq[e] = pq[i][e]; }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int gi = tid + NT * i;
      if (V_GROUPS % NT != 0 && gi >= V_GROUPS) continue;
      const int r = gi / (DV / 8), c = (gi % (DV / 8)) * 8;
      u32x4_t *dv = reinterpret_cast<u32x4_t *>(sV + r * LDV + c);
#pragma unroll
      for (int e = 0; e < EW; ++e) dv[e] = pv[i][e];
    }
    if (wave == 0) {
      // inclusive prefix sum of the log2 decays over the chunk's 64 tokens
      const float G = wave_inclusive_sum(p_valid && decay ? pg * LOG2E : 0.f);
      const float G_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
      sG[lane] = G;
      sG[C + lane] = fast_exp2(G);                                     // gamma
      sG[2 * C + lane] = p_valid ? (erase ? pb : 1.f) : 0.f;           // beta (plain rules: R = beta V)
      sG[3 * C + lane] = fast_exp2(G_last - G);                        // exp(G_last - G)
      sG[4 * C + lane] = p.scale * fast_exp2(G);                       // scale * gamma
      sG[5 * C + lane] = ef * fast_exp2(G);                            // e * gamma
    }
  };

  // O rows r0 + rq .. r0 + rq + 3 of column c0 + col, held by this lane in
  // the accumulator layout (already scaled: the read-out scale rides on
  // scale * gamma and on L o P), stored (only rows inside the chunk).
  // BF16: each lane swaps halves with its neighbour column (lane ^ 1), so a
  // lane stores two rows of a column pair as 4-byte words.
  // Addresses: a uniform base per chunk, a per-lane offset fixed for the
  // chain (32-bit: it spans at most 16 token rows) and a uniform per-tile part.
  AT *const o_head = static_cast<AT *>(p.o) + (int64_t)h * DV;
  const int64_t o_row = (int64_t)p.H_v * DV;  // elements between tokens
  const bool o_odd = (col & 1) != 0;
  const uint32_t o_lane = AB ? (uint32_t)((rq + (o_odd ? 2 : 0)) * o_row + (col & ~1))
                             : (uint32_t)(rq * o_row + col);  // elements
  AT *o_base = o_head;  // row 0 of the chunk
  int o_n = 0;          // tokens in the chunk
  auto store_o_tile = [&](int r0, int c0, const f32x4_t &acc, bool whole) {
    AT *const dst = o_base + r0 * o_row + c0 + o_lane;
    if constexpr (AB) {
      const uint32_t a = pack_bf16x2(acc[0], acc[1]);  // rows 0, 1
      const uint32_t b = pack_bf16x2(acc[2], acc[3]);  // rows 2, 3
      const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)(o_odd ? a : b), 0xB1, 0xf, 0xf, false);
      const uint32_t own = o_odd ? b : a;
      const uint32_t left = o_odd ? other : own, right = o_odd ? own : other;  // columns c, c + 1
      const uint32_t w0 = __builtin_amdgcn_perm(right, left, 0x05040100u);
      const uint32_t w1 = __builtin_amdgcn_perm(right, left, 0x07060302u);
      const int r = r0 + rq + (o_odd ? 2 : 0);
      if (whole || r < o_n) *reinterpret_cast<uint32_t *>(dst) = w0;
      if (whole || r + 1 < o_n) *reinterpret_cast<uint32_t *>(dst + o_row) = w1;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (whole || r0 + rq + e < o_n) dst[e * o_row] = acc[e];
      }
    }
  };

  // padded K columns (d_k < 32 only) stay zero for the whole chain, in both sets
  if constexpr (L::DKP > DK) {
    constexpr int PADC = L::DKP - DK;
    for (int i = tid; i < 4 * C * PADC; i += NT) {
      const int row = i / PADC, c = DK + i % PADC;  // rows of K0, Q0, K1, Q1
      IT *rowp = reinterpret_cast<IT *>(smem + (row / (2 * C)) * L::SET + ((row / C) & 1 ? L::QH : L::KH));
      put(rowp + (row % C) * LDK + c, 0.f);
    }
  }

  // ---- initial state (a8): read slot -> FP32 accumulators ----
  // macc[b][ia]: rows 16b.. of d_k, columns 16 (wave NA + ia).. of d_v, in the
  // accumulator layout (lane (g, n): rows 4g..4g+3 of column n)
  const bool mwave = DVB >= NW || wave < DVB;  // waves that own d_v columns
  f32x4_t macc[DKB][NA];
  const int64_t state_base = (rs * p.H_v + h) * (int64_t)DK * DV;
#pragma unroll
  for (int b = 0; b < DKB; ++b) {
#pragma unroll
    for (int ia = 0; ia < NA; ++ia) {
#pragma unroll
      for (int e = 0; e < 4; ++e) macc[b][ia][e] = 0.f;
    }
  }
  if (mwave && rs >= 0) {  // one branch around all the loads, so they overlap
#pragma unroll
    for (int b = 0; b < DKB; ++b) {
#pragma unroll
      for (int ia = 0; ia < NA; ++ia) {
        const int d = 16 * b + rq, c = 16 * (wave * NA + ia) + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          macc[b][ia][e] = Elem<SB>::load1(p.pool, state_base + (int64_t)(d + e) * DV + c);
      }
    }
  }
  // FP32 state -> state dtype (RNE for BF16) -> a slot (waves that own d_v
  // columns): the final state, and the intermediate checkpoints
  auto store_state = [&](int64_t slot) {
    const int64_t out_base = (slot * p.H_v + h) * (int64_t)DK * DV;
#pragma unroll
    for (int b = 0; b < DKB; ++b) {
#pragma unroll
      for (int ia = 0; ia < NA; ++ia) {
        const int d = 16 * b + rq, c = 16 * (wave * NA + ia) + col;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Elem<SB>::store1(p.pool, out_base + (int64_t)(d + e) * DV + c, macc[b][ia][e]);
      }
    }
  };
  if (t_begin < t_end) {
    fetch(t_begin);
    stage(0);
  }
  __syncthreads();

  if constexpr (NW == 8) {
    // the two tiles above the diagonal that the O step's 32-wide slabs read,
    // (0, 1) and (2, 3) of L o P, stay zero for the whole chain
    for (int i = tid; i < 2 * 256; i += NT) {
      const int t = i >> 8, r = 32 * t + ((i >> 4) & 15), c = 32 * t + 16 + (i & 15);
      put(Sq + r * LDC + c, 0.f);
    }
  }

  int cur = 0;  // input set of the current chunk
  for (int64_t t0 = t_begin; t0 < t_end; t0 += C, cur ^= 1) {
    const int64_t t1 = t0 + C;
    o_base = o_head + t0 * o_row;
    o_n = (int)std::min<int64_t>(C, t_end - t0);
    use_set(cur);

    // T_RB,RB = (I + A_RB,RB)^-1 from diagonal block RB of A, which this wave
    // holds in registers (ab; lane (g, n): rows 4g .. 4g+3 of column n): lane
    // (g, c) forms column c by forward substitution (the four lane groups
    // alike), one row per call, each A entry broadcast from the lane that
    // holds it (v_readlane), so there is no LDS round trip.  Without erase
    // A = 0 and T = I: formed all the same, branch-free.
    float tc[16];
    f32x4_t ab = {0.f, 0.f, 0.f, 0.f};
    auto t_row = [&](int r) {
      float x = r == col ? 1.f : 0.f;
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2) {
        const int a = __builtin_amdgcn_readlane(__float_as_int(ab[r & 3]), 16 * (r >> 2) + s2);
        x = fmaf(-__int_as_float(a), tc[s2], x);
      }
      tc[r] = x;
    };

    // 8 waves: the chunk-local products of the tiles that are used (the lower
    // triangle; the upper tiles of S and P are never formed).  Waves 0-3: S of
    // diagonal block b = wave, its A block and T_bb, a vector-ALU chain; waves
    // 4-7: S and P of the six tiles below the diagonal (two, two, one, one),
    // waves 6 and 7 also P of two diagonal tiles each (kLocalTiles).  So every
    // SIMD pairs a T wave with a product wave.
    auto chunk_local_w8 = [&]() {
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      // Product wave W: its tiles' S and P over the 32-wide slabs, every
      // fragment of slab kk + 1 loaded during slab kk's MFMAs; then A and L o P
      // of the tiles below the diagonal (s < r throughout) and L o P of the
      // diagonal tiles (masked to s <= r) into LDS.
      auto products = [&](auto wi) {
        constexpr LocalTiles c = kLocalTiles[decltype(wi)::value];
        Frag<F32> fr[2][6];
        f32x4_t sa[2], pa[2], pd[2];  // set by their first MFMA
        auto load_slab = [&](int kk, Frag<F32>(&dst)[6]) {
#pragma unroll
          for (int f = 0; f < c.nf; ++f) {
            const int id = c.frag[f];
            dst[f] = load_frag<F32>((id & 1) ? Qh : Kh, LDK, 16 * (id >> 1), 32 * kk);
          }
        };
        load_slab(0, fr[0]);
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) {
          if (kk + 1 < NKB) load_slab(kk + 1, fr[(kk + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < c.nod; ++t) {
            sa[t] = mma<F32>(kk == 0 ? z : sa[t], fr[kk & 1][c.od[t][2]], fr[kk & 1][c.od[t][4]]);
            pa[t] = mma<F32>(kk == 0 ? z : pa[t], fr[kk & 1][c.od[t][3]], fr[kk & 1][c.od[t][4]]);
          }
#pragma unroll
          for (int t = 0; t < c.ndp; ++t)
            pd[t] = mma<F32>(kk == 0 ? z : pd[t], fr[kk & 1][c.dp[t][1]], fr[kk & 1][c.dp[t][2]]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int t = 0; t < c.nod; ++t) {
          const int ti = c.od[t][0], tj = c.od[t][1];
          const float Gc = Gs[16 * tj + col];
          const f32x4_t Gr = *reinterpret_cast<const f32x4_t *>(Gs + 16 * ti + rq);
          const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * ti + rq);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * ti + rq + e, s = 16 * tj + col;
            const float dec = fast_exp2(Gr[e] - Gc);
            const float a = (ef * br[e]) * dec * sa[t][e];
            if constexpr (kBfAT) put(Ab + r * L::LDAB + s, -a);
            else Af[r * LDF + s] = a;
            put(Sq + r * LDC + s, p.scale * (dec * pa[t][e]));
          }
        }
#pragma unroll
        for (int t = 0; t < c.ndp; ++t) {
          const int b = c.dp[t][0];
          const float Gc = Gs[16 * b + col];
          const f32x4_t Gr = *reinterpret_cast<const f32x4_t *>(Gs + 16 * b + rq);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * b + rq + e;
            const float x = p.scale * (fast_exp2(Gr[e] - Gc) * pd[t][e]);
            put(Sq + r * LDC + 16 * b + col, col <= rq + e ? x : 0.f);
          }
        }
      };
      if (wave < 4) {
        // diagonal block b = wave: S_bb = K_b K_b^T, both operands the same fragment
        const int b = wave;
        f32x4_t sd;
        Frag<F32> fk[NKB];
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) fk[kk] = load_frag<F32>(Kh, LDK, 16 * b, 32 * kk);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < NKB; ++kk) sd = mma<F32>(kk == 0 ? z : sd, fk[kk], fk[kk]);
        // A_bb stays in registers (no other wave reads the diagonal block):
        // lane (g, n) holds rows 4g .. 4g+3 of column n
        const float Gc = Gs[16 * b + col];
        const f32x4_t Gr = *reinterpret_cast<const f32x4_t *>(Gs + 16 * b + rq);
        const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * b + rq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = (ef * br[e]) * fast_exp2(Gr[e] - Gc) * sd[e];
          ab[e] = col < rq + e ? a : 0.f;  // row rq + e inside the block
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) t_row(r);
      } else if (wave == 4) {
        products(std::integral_constant<int, 0>());
      } else if (wave == 5) {
        products(std::integral_constant<int, 1>());
      } else if (wave == 6) {
        products(std::integral_constant<int, 2>());
      } else {
        products(std::integral_constant<int, 3>());
      }
    };


    f32x4_t qm[4][NA], um[4][NA];  // set by their first MFMA (K-step 0 starts from zero)
    if constexpr (NW == 8) {
      chunk_local_w8();
    } else {
      // ---- 2: S = K K^T, P = Q K^T (a6), the wave's tiles: row block RB,
      // column blocks cb0 .. cb0 + NCB - 1 ----
      f32x4_t sacc[NCB], pacc[NCB];  // set by their first MFMA
      const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
      // S and P (S unused without erase: no branch, straight-line code), the
      // fragments of step f + 1 loaded during step f's MFMAs
      {
        constexpr int NF = NKB * NCB;  // (slab, column block)
        Frag<F32> fk[2], fq[2], fb[2];
        fk[0] = load_frag<F32>(Kh, LDK, 16 * RB, 0);
        fq[0] = load_frag<F32>(Qh, LDK, 16 * RB, 0);
        fb[0] = load_frag<F32>(Kh, LDK, 16 * cb0, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int kk = f / NCB, cb = f % NCB;
          if (f + 1 < NF) {
            const int kn = (f + 1) / NCB;
            if ((f + 1) % NCB == 0) {
              fk[kn & 1] = load_frag<F32>(Kh, LDK, 16 * RB, 32 * kn);
              fq[kn & 1] = load_frag<F32>(Qh, LDK, 16 * RB, 32 * kn);
            }
            fb[(f + 1) & 1] = load_frag<F32>(Kh, LDK, 16 * (cb0 + (f + 1) % NCB), 32 * kn);
          }
          __builtin_amdgcn_sched_barrier(0);
          sacc[cb] = mma<F32>(kk == 0 ? z : sacc[cb], fk[kk & 1], fb[f & 1]);
          pacc[cb] = mma<F32>(kk == 0 ? z : pacc[cb], fq[kk & 1], fb[f & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- 3: A = strict_lower(beta_r e^{G_r-G_s} S), Sq = lower(e^{G_r-G_s} P),
      // the wave's tiles ----
      {
        // gate rows as 16-byte loads and masks as selects, so no LDS load sits
        // in a branch of its own
        const f32x4_t Gr = *reinterpret_cast<const f32x4_t *>(Gs + 16 * RB + rq);
        const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * RB + rq);
        float Gc[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Gc[cb] = Gs[16 * (cb0 + cb) + col];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 16 * RB + rq + e, s = 16 * (cb0 + cb) + col;
            const float e2 = fast_exp2(Gr[e] - Gc[cb]);
            const float dec = s <= r ? e2 : 0.f;
            const float a = s < r ? (ef * br[e]) * dec * sacc[cb][e] : 0.f;
            if constexpr (kBfAT) put(Ab + r * L::LDAB + s, -a);
            else Af[r * LDF + s] = a;
            put(Sq + r * LDC + s, p.scale * (dec * pacc[cb][e]));
            if (cb0 + cb == RB) ab[e] = a;  // the wave's diagonal block, for its T
          }
        }
      }
    }
    // The next chunk's inputs, in flight while this chunk computes (issued
    // after the chunk-local products, when the previous chunk's O stores have
    // drained).  Fetched and staged on the last chunk too (clamped to the last
    // token, into the set nobody reads next): with no branch around them, the
    // register reuse at the loop head does not make the compiler wait for
    // every outstanding memory operation.
    fetch(t1);
    // ---- 5: Q M and K M (a7) for the wave's d_v columns, the A fragments in a
    // ring: the load of fragment f + RING - 1 is issued before the MFMAs of
    // fragment f (scheduling barriers keep the compiler from moving it back
    // next to its use) ----
    if (mwave) {
      constexpr int NF = NKB * 8;  // (slab, row block, q or k)
      Frag<F32> fa[RING];
      Frag<F32> fm[NA];
      auto load_a = [&](int f) {
        return load_afrag<F32>((f & 1) ? Kh : Qh, LDK, 16 * ((f >> 1) & 3), 32 * (f >> 3));
      };
#pragma unroll
      for (int f = 0; f < RING - 1; ++f) fa[f] = load_a(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kk = f >> 3, tb = (f >> 1) & 3, isk = f & 1;
        if (f + RING - 1 < NF) fa[(f + RING - 1) % RING] = load_a(f + RING - 1);
        if ((f & 7) == 0) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            fm[ia] = bfrag<F32>(macc[2 * kk][ia], 2 * kk + 1 < DKB ? macc[2 * kk + 1][ia] : z);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
          const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          if (isk) um[tb][ia] = mma<F32>(kk == 0 ? z : um[tb][ia], fa[f % RING], fm[ia]);
          else qm[tb][ia] = mma<F32>(kk == 0 ? z : qm[tb][ia], fa[f % RING], fm[ia]);
        }
        if constexpr (kInterleaveT) {
#pragma unroll
          for (int r = 16 * f / NF; r < 16 * (f + 1) / NF; ++r) t_row(r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if constexpr (kInterleaveT) {
#pragma unroll
      for (int r = 0; r < 16; ++r) t_row(r);
    }
    if (diag && lane < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (kBfAT) put(Tb + (16 * RB + r) * L::LDTB + col, tc[r]);
        else Tf[(16 * RB + r) * L::LDT + col] = tc[r];
      }
    }
    __syncthreads();  // A, L o P and T are visible; every wave is done with the previous chunk
    // the next chunk's inputs into the other set (every wave finished reading
    // it, in the previous chunk, before the barrier above).  Staged before
    // this chunk's O stores are issued, so waiting for the prefetch does not
    // wait for them too.
    stage(cur ^ 1);

    // ---- 5-8: the wave's d_v columns, in registers ----
    if (mwave) {
      // R = beta (V - gamma K M) for the delta rules, else R = V (beta holds 1 on
      // the chunk's tokens and 0 on its padded rows); um holds R.  Branch-free:
      // without erase ef = 0 and the K M term is an exact zero.  The lane's four
      // rows of beta and gamma are one 16-byte load each.
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        float vv[NA][4];
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) load_col4(Vh, LDV, 16 * tb, 16 * (wave * NA + ia), vv[ia]);
        const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * tb + rq);
        const f32x4_t gr = *reinterpret_cast<const f32x4_t *>(gme + 16 * tb + rq);  // e * gamma
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) um[tb][ia][e] = br[e] * (vv[ia][e] - gr[e] * um[tb][ia][e]);
        }
      }
      // 6: U = (I + A)^-1 R (delta rules), block forward substitution in
      // place: um[i] <- T_ii (R_i - sum_{j<i} A_ij U_j), 16-row blocks i = 0..3
      if (erase) {
        // every A_ij and T_ii fragment is loaded up front (none depends on U),
        // so the serial chain below waits only on its own MFMAs
        Frag16<F32> fa[6], ft[4];
#pragma unroll
        for (int i = 1, n = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < i; ++j, ++n) {
            if constexpr (kBfAT) fa[n] = load_afrag16(Ab, L::LDAB, 16 * i, 16 * j);
            else fa[n] = load_afrag16<F32>(Af, LDF, 16 * i, 16 * j, -1.f);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (kBfAT) ft[i] = load_afrag16(Tb, L::LDTB, 16 * i, 0);
          else ft[i] = load_afrag16<F32>(Tf, L::LDT, 16 * i, 0, 1.f);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0, n = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < i; ++j, ++n) {
#pragma unroll
            for (int ia = 0; ia < NA; ++ia)
              um[i][ia] = mma16<F32>(um[i][ia], fa[n], bfrag16<F32>(um[j][ia]));
          }
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
            um[i][ia] = mma16<F32>(z, ft[i], bfrag16<F32>(um[i][ia]));
          }
        }
      }
      // 7: O = scale (gamma Q M + (L o P) U) (a7), as (scale gamma) Q M +
      // (scale L o P) U, stored to HBM straight from the accumulator layout
      Frag<F32> fu[2][NA];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) fu[s2][ia] = bfrag<F32>(um[2 * s2][ia], um[2 * s2 + 1][ia]);
      }
      // the six (L o P) fragments below the diagonal, loaded together
      Frag<F32> fs[6];
#pragma unroll
      for (int tb = 0, n = 0; tb < 4; ++tb) {
#pragma unroll
        for (int s2 = 0; s2 <= tb / 2; ++s2, ++n) fs[n] = load_afrag<F32>(Sq, LDC, 16 * tb, 32 * s2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int tb = 0, n = 0; tb < 4; ++tb) {
        const f32x4_t gr = *reinterpret_cast<const f32x4_t *>(gsc + 16 * tb + rq);  // scale * gamma
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
#pragma unroll
          for (int e = 0; e < 4; ++e) qm[tb][ia][e] *= gr[e];
        }
#pragma unroll
        for (int s2 = 0; s2 <= tb / 2; ++s2, ++n) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) qm[tb][ia] = mma<F32>(qm[tb][ia], fs[n], fu[s2][ia]);
        }
        // whole chunks store without row checks (a uniform branch)
        if (o_n == C) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) store_o_tile(16 * tb, 16 * (wave * NA + ia), qm[tb][ia], true);
        } else {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) store_o_tile(16 * tb, 16 * (wave * NA + ia), qm[tb][ia], false);
        }
      }
    }
    if (mwave) {
      // 8: M <- gamma_last M + K^T diag(exp(G_last - G)) U: the decay weights
      // scale U's rows; K^T's fragments are read down the columns of the K rows
      Frag<F32> fe[2][NA];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const f32x4_t elo = *reinterpret_cast<const f32x4_t *>(eGn + 32 * s2 + rq);
        const f32x4_t ehi = *reinterpret_cast<const f32x4_t *>(eGn + 32 * s2 + 16 + rq);
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
          f32x4_t lo = um[2 * s2][ia], hi = um[2 * s2 + 1][ia];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] *= elo[e];
            hi[e] *= ehi[e];
          }
          fe[s2][ia] = bfrag<F32>(lo, hi);
        }
      }
      const float gl = gam[C - 1];
#pragma unroll
      for (int b = 0; b < DKB; ++b) {
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
#pragma unroll
          for (int e = 0; e < 4; ++e) macc[b][ia][e] *= gl;
        }
      }
      // K^T fragments in a ring, RING - 1 loads ahead of their MFMAs
      {
        constexpr int NF = DKB * 2;  // (d_k block, token slab)
        constexpr int RK = RING < NF ? RING : NF;
        Frag<F32> fk[RK];
        auto load_k = [&](int f) { return load_afrag_t<F32>(Kh, LDK, 16 * (f >> 1), 32 * (f & 1)); };
#pragma unroll
        for (int f = 0; f < RK - 1; ++f) fk[f] = load_k(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + RK - 1 < NF) fk[(f + RK - 1) % RK] = load_k(f + RK - 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ia = 0; ia < NA; ++ia)
            macc[f >> 1][ia] = mma<F32>(macc[f >> 1][ia], fk[f % RK], fe[f & 1][ia]);
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
    __syncthreads();  // the next chunk's set is written; this chunk's reads are done
  }

  // ---- final state (a8): FP32 -> state dtype (RNE for BF16) -> write slot ----
  if (ws >= 0 && mwave) store_state(ws);
}

}  // namespace gdn
