// prefill_pipe.cuh -- the chunked-prefill chain as a two-stage pipeline over
// chunks ("Gated DeltaNet" page, chunkwise parallel form; the same products
// as prefill_chain.cuh, in the same order per element).
//
// The chunk-local products of a chunk (S = K K^T and P = Q K^T over its
// tokens, A, L o P, T_ii = (I + A_ii)^-1) do not depend on the state M; the
// rest (Q M, K M, R, the block substitution for U, O, the update of M) does.
// So four consumer waves (0-3, d_v / 4 state columns each) run chunk c's
// state-dependent steps while four producer waves (4-7, one 16-row block of
// the chunk each) stage chunk c + 1's inputs, start fetching chunk c + 2, and
// form chunk c + 1's chunk-local products into the other of two chunk-local
// LDS sets.  Every product's operands and order are those of the 4-wave
// chain, so results are bitwise equal to it.
//
// Per iteration c there are two barriers, Y and X:
//   producers: stage chunk c+1 (input set (c+1)%2), fetch chunk c+2, Y,
//              chunk-local products of c+1 (local set (c+1)%2), X
//   consumers: Q M and K M of chunk c, Y, R, U, O, M update of chunk c, X
// Input set (c+1)%2 last held chunk c-1, whose readers all passed X of
// iteration c-1; local set (c+1)%2 likewise.  The consumers need nothing
// from Y: they meet it after their Q M / K M, by which time the producers
// have staged, so neither side idles there.  Barriers wait for LDS only,
// not for the producers' in-flight loads or the consumers' O stores (and
// the two are now in different waves' counters).
#pragma once

#include "prefill_chain.cuh"

namespace gdn {

// LDS layout of the pipelined chain (byte offsets): two input sets (K, Q, V
// rows and the six per-token gate arrays), two chunk-local sets of BF16 L o P
// (scaled), -A and T_ii, and one FP32 diagonal block of A per producer wave.
template <int DK, int DV>
struct PipeLayout {
  using B = PrefillLayout<DK, DV, false>;
  // K and Q rows (the pipelined chain has d_k >= 32), V rows
  using RK = LdsRows<DK, DK == 128 ? kRowsXor : kRowsPadded>;
  using RV = LdsRows<DV, DV == 128 ? kRowsXor : kRowsPadded>;
  static constexpr int C = B::C;
  static constexpr size_t KH = 0;
  static constexpr size_t QH = KH + (size_t)C * RK::LD * 2;
  static constexpr size_t VH = QH + (size_t)C * RK::LD * 2;
  static constexpr size_t GATES = VH + (size_t)C * RV::LD * 2;
  static constexpr size_t SET = GATES + 6 * C * 4;
  static constexpr size_t L_SQ = 0;
  static constexpr size_t L_AB = L_SQ + (size_t)C * B::LDC * 2;
  static constexpr size_t L_TB = L_AB + (size_t)C * B::LDAB * 2;
  static constexpr size_t LOC = L_TB + (size_t)C * B::LDTB * 2;  // one chunk-local set
  static constexpr size_t LOC0 = 2 * SET;
  // per producer wave: its FP32 diagonal block of A, transposed (row c holds
  // column c of A; rows of LDA floats, 16-byte aligned)
  static constexpr int LDA = 20;
  static constexpr size_t ADIAG = LOC0 + 2 * LOC;
  static constexpr size_t ADIAG_WAVE = 16 * LDA * 4;
  static constexpr size_t BYTES = ADIAG + 4 * ADIAG_WAVE;
  static_assert(SET % 16 == 0 && LOC % 16 == 0, "16-byte aligned sets");
};

// Chunk-local tiles of producer wave b (waves 4 + b): its diagonal block b
// (S_bb for A_bb and T_bb, and P_bb) and some tiles below the diagonal, from
// fragments loaded once per 32-wide slab.  A fragment id is 2 j for block j
// (16 rows) of K and 2 j + 1 for block j of Q; a slot is a position in `frag`.
struct PipeTiles {
  int nf;        // fragments per slab
  int frag[6];   // fragment id of each slot (slots 0, 1: K_b, Q_b)
  int nod;       // tiles below the diagonal: S and P of (i, j)
  int od[2][5];  // i, j, and the slots of K_i, Q_i, K_j
};
constexpr PipeTiles kPipeTiles[4] = {
    {6, {0, 1, 2, 3, 4, 5}, 2, {{1, 0, 2, 3, 0}, {2, 0, 4, 5, 0}}},  // (0,0) (1,0) (2,0)
    {4, {2, 3, 6, 7, 0, 0}, 1, {{3, 1, 2, 3, 0}, {0, 0, 0, 0, 0}}},  // (1,1) (3,1)
    {4, {4, 5, 6, 7, 0, 0}, 1, {{3, 2, 2, 3, 0}, {0, 0, 0, 0, 0}}},  // (2,2) (3,2)
    {6, {6, 7, 4, 5, 2, 0}, 2, {{2, 1, 2, 3, 4}, {3, 0, 0, 1, 5}}},  // (3,3) (2,1) (3,0)
};

// CK: the instance that stores intermediate checkpoints.
template <bool SB, bool AB, int DK, int DV, bool CK = false>
__device__ __forceinline__ void prefill_chain_pipe(const PrefillParams &p, int chain, char *smem) {
  static_assert(AB, "BF16 activations");
  constexpr bool F32 = false;
  constexpr int NT = 512, PT = 256;  // threads; producer threads (waves 4-7)
  using L = PipeLayout<DK, DV>;
  using BL = PrefillLayout<DK, DV, false>;
  using OT = uint16_t;
  using AT = typename Elem<AB>::T;
  constexpr int C = L::C;
  constexpr int LDC = BL::LDC;
  using RowK = typename L::RK;
  using RowV = typename L::RV;
  constexpr int NKB = BL::DKP / 32;  // MFMA K-steps over d_k
  constexpr int DKB = DK / 16;       // 16-row blocks of d_k
  constexpr int DVB = DV / 16;       // 16-column blocks of d_v
  constexpr int NA = DVB / 4;        // d_v blocks per consumer wave
  static_assert(DK >= 32 && DVB % 4 == 0, "whole K slabs, d_v blocks per consumer");
  constexpr int RING = 4;  // LDS operand fragments in flight ahead of their MFMA
  constexpr int KQ_GROUPS = C * (DK / 8), KQ_PER = (KQ_GROUPS + PT - 1) / PT;
  constexpr int V_GROUPS = C * (DV / 8), V_PER = (V_GROUPS + PT - 1) / PT;
  constexpr float LOG2E = 1.4426950408889634f;

  OT *Kh, *Qh, *Vh;
  float *Gs, *gam, *bet, *eGn;  // cumulative log2 decay, gamma, beta, exp(G_last - G)
  float *gsc, *gme;             // scale * gamma (the read-out), e * gamma (R's K M term)
  auto use_set = [&](int b) {
    char *base = smem + b * L::SET;
    Kh = reinterpret_cast<OT *>(base + L::KH);
    Qh = reinterpret_cast<OT *>(base + L::QH);
    Vh = reinterpret_cast<OT *>(base + L::VH);
    Gs = reinterpret_cast<float *>(base + L::GATES);
    gam = Gs + C; bet = Gs + 2 * C; eGn = Gs + 3 * C; gsc = Gs + 4 * C; gme = Gs + 5 * C;
  };
  OT *Sq;        // L o P, scaled
  uint16_t *Ab;  // -A
  uint16_t *Tb;  // T_ii, stacked
  auto use_loc = [&](int b) {
    char *base = smem + L::LOC0 + b * L::LOC;
    Sq = reinterpret_cast<OT *>(base + L::L_SQ);
    Ab = reinterpret_cast<uint16_t *>(base + L::L_AB);
    Tb = reinterpret_cast<uint16_t *>(base + L::L_TB);
  };

  const int seq = chain / p.H_v, h = chain % p.H_v, hq = h / p.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool consumer = wave < 4;  // uniform in a wave
  const int cw = wave & 3;         // consumer: column group; producer: row block
  const int col = lane & 15, rq = 4 * (lane >> 4);  // accumulator layout: rows rq..rq+3, column col
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
  const float ef = erase ? 1.f : 0.f;  // a factor, not a branch

  // ---- producers: prefetch of one chunk's inputs into registers, staging ----
  // Unconditional loads; rows past the sequence's end re-read its last token
  // and get beta = 0, so they reach neither M nor a stored O row.
  u32x4_t pk[KQ_PER], pq[KQ_PER], pv[V_PER];
  float pg = 0.f, pb = 0.f;  // wave 4: gate inputs of token `lane`
  bool p_valid = false;       // wave 4: token `lane` lies inside the sequence
  const int ptid = tid - PT;  // producers: 0..PT-1
  constexpr int KQ_RS = PT / (DK / 8), V_RS = PT / (DV / 8);
  const int64_t kq_row = (int64_t)p.H_qk * DK, v_row = (int64_t)p.H_v * DV;  // elements per token
  const uint32_t kq_lane = (uint32_t)((ptid / (DK / 8)) * kq_row + (ptid % (DK / 8)) * 8);
  const uint32_t v_lane = (uint32_t)((ptid / (DV / 8)) * v_row + (ptid % (DV / 8)) * 8);
  const uint32_t g_lane = (uint32_t)(lane * p.H_v);
  auto fetch = [&](int64_t t0) {
    const int64_t last = t_end - 1;
    const AT *const kb = static_cast<const AT *>(p.k) + t0 * kq_row + hq * DK;
    const AT *const qb = static_cast<const AT *>(p.q) + t0 * kq_row + hq * DK;
    const AT *const vb = static_cast<const AT *>(p.v) + t0 * v_row + h * DV;
    if (t0 + C - 1 <= last) {  // a whole chunk: no clamping
#pragma unroll
      for (int i = 0; i < KQ_PER; ++i) {
        if (KQ_GROUPS % PT != 0 && ptid + PT * i >= KQ_GROUPS) continue;
        const int64_t off = kq_lane + (int64_t)i * KQ_RS * kq_row;
        pk[i] = *reinterpret_cast<const u32x4_t *>(kb + off);
        pq[i] = *reinterpret_cast<const u32x4_t *>(qb + off);
      }
#pragma unroll
      for (int i = 0; i < V_PER; ++i) {
        if (V_GROUPS % PT != 0 && ptid + PT * i >= V_GROUPS) continue;
        pv[i] = *reinterpret_cast<const u32x4_t *>(vb + v_lane + (int64_t)i * V_RS * v_row);
      }
    } else {  // rows clamped to the last token (also chunks wholly past the end)
      const int64_t rmax = last - t0;
#pragma unroll
      for (int i = 0; i < KQ_PER; ++i) {
        const int gi = ptid + PT * i;
        const int64_t r = std::min<int64_t>(gi / (DK / 8), rmax);
        const int64_t off = r * kq_row + (gi % (DK / 8)) * 8;
        pk[i] = *reinterpret_cast<const u32x4_t *>(kb + off);
        pq[i] = *reinterpret_cast<const u32x4_t *>(qb + off);
      }
#pragma unroll
      for (int i = 0; i < V_PER; ++i) {
        const int gi = ptid + PT * i;
        const int64_t r = std::min<int64_t>(gi / (DV / 8), rmax);
        pv[i] = *reinterpret_cast<const u32x4_t *>(vb + r * v_row + (gi % (DV / 8)) * 8);
      }
    }
    if (wave == 4) {
      // raw values only (masked at staging); g and beta may be NULL under the
      // rules that do not use them
      const int64_t gt = t0 + lane <= last ? t0 * p.H_v + h + (int64_t)g_lane : last * p.H_v + h;
      if (decay) pg = p.g[gt];
      if (erase) pb = p.beta[gt];
      p_valid = t0 + lane <= last;
    }
  };
  auto stage = [&](int b) {  // into input set b
    char *base = smem + b * L::SET;
    OT *const sK = reinterpret_cast<OT *>(base + L::KH), *const sQ = reinterpret_cast<OT *>(base + L::QH);
    OT *const sV = reinterpret_cast<OT *>(base + L::VH);
    float *const sG = reinterpret_cast<float *>(base + L::GATES);
#pragma unroll
    for (int i = 0; i < KQ_PER; ++i) {
      const int gi = ptid + PT * i;
      if (KQ_GROUPS % PT != 0 && gi >= KQ_GROUPS) continue;
      const int r = gi / (DK / 8), d = (gi % (DK / 8)) * 8;
      *reinterpret_cast<u32x4_t *>(sK + RowK::at(r, d)) = pk[i];
      *reinterpret_cast<u32x4_t *>(sQ + RowK::at(r, d)) = pq[i];
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int gi = ptid + PT * i;
      if (V_GROUPS % PT != 0 && gi >= V_GROUPS) continue;
      const int r = gi / (DV / 8), c = (gi % (DV / 8)) * 8;
      *reinterpret_cast<u32x4_t *>(sV + RowV::at(r, c)) = pv[i];
    }
    if (wave == 4) {
      // inclusive prefix sum of the log2 decays over the chunk's 64 tokens
      const float G = wave_inclusive_sum(p_valid && decay ? pg * LOG2E : 0.f);
      const float G_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
      sG[lane] = G;
      sG[C + lane] = fast_exp2(G);                            // gamma
      sG[2 * C + lane] = p_valid ? (erase ? pb : 1.f) : 0.f;  // beta (plain rules: R = beta V)
      sG[3 * C + lane] = fast_exp2(G_last - G);               // exp(G_last - G)
      sG[4 * C + lane] = p.scale * fast_exp2(G);              // scale * gamma
      sG[5 * C + lane] = ef * fast_exp2(G);                   // e * gamma
    }
  };

  // ---- producers: chunk-local products of the current input set ----------
  // Producer wave b: S and P of its tiles (kPipeTiles) into -A and L o P, the
  // fragments of slab kk + 1 loaded during slab kk's MFMAs; then T_bb by
  // forward substitution from the diagonal block of A, passed through a small
  // LDS area of the wave's own so every lane reads its rows.  Only tiles
  // on or below the diagonal are formed; the substitution reads -A below the
  // diagonal blocks only, and the two tiles above it that the O step's slabs
  // read, (0,1) and (2,3) of L o P, are zeroed once per chain.
  auto local_tiles = [&](auto wi) {
    constexpr PipeTiles c = kPipeTiles[decltype(wi)::value];
    constexpr int b = decltype(wi)::value;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    Frag<F32> fr[2][6];
    f32x4_t sa[2], pa[2], sd, pd;  // set by their first MFMA
    auto load_slab = [&](int kk, Frag<F32>(&dst)[6]) {
#pragma unroll
      for (int f = 0; f < c.nf; ++f) {
        const int id = c.frag[f];
        dst[f] = rows_frag<RowK>((id & 1) ? Qh : Kh, 16 * (id >> 1), 32 * kk);
      }
    };
    load_slab(0, fr[0]);
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      if (kk + 1 < NKB) load_slab(kk + 1, fr[(kk + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      sd = mma<F32>(kk == 0 ? z : sd, fr[kk & 1][0], fr[kk & 1][0]);
      pd = mma<F32>(kk == 0 ? z : pd, fr[kk & 1][1], fr[kk & 1][0]);
#pragma unroll
      for (int t = 0; t < c.nod; ++t) {
        sa[t] = mma<F32>(kk == 0 ? z : sa[t], fr[kk & 1][c.od[t][2]], fr[kk & 1][c.od[t][4]]);
        pa[t] = mma<F32>(kk == 0 ? z : pa[t], fr[kk & 1][c.od[t][3]], fr[kk & 1][c.od[t][4]]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the diagonal block: A_bb stays in registers (lane (g, n): rows 4g..
    // of column n), L o P masked to s <= r
    f32x4_t ab;
    {
      const float Gc = Gs[16 * b + col];
      const f32x4_t Gr = *reinterpret_cast<const f32x4_t *>(Gs + 16 * b + rq);
      const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * b + rq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * b + rq + e;
        const float e2 = fast_exp2(Gr[e] - Gc);
        const float a = (ef * br[e]) * e2 * sd[e];
        ab[e] = col < rq + e ? a : 0.f;
        const float x = p.scale * (e2 * pd[e]);
        put(Sq + r * LDC + 16 * b + col, col <= rq + e ? x : 0.f);
      }
    }
#pragma unroll
    for (int t = 0; t < c.nod; ++t) {
      const int ti = c.od[t][0], tj = c.od[t][1];
      const float Gc = Gs[16 * tj + col];
      const f32x4_t Gr = *reinterpret_cast<const f32x4_t *>(Gs + 16 * ti + rq);
      const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * ti + rq);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * ti + rq + e, s2 = 16 * tj + col;
        const float dec = fast_exp2(Gr[e] - Gc);
        const float a = (ef * br[e]) * dec * sa[t][e];
        put(Ab + r * BL::LDAB + s2, -a);
        put(Sq + r * LDC + s2, p.scale * (dec * pa[t][e]));
      }
    }
    // T_bb column `col` by forward substitution in right-looking order: once
    // x_s is final, every later row's sum takes its term -A[r][s] x_s, so a
    // step waits on one FMA instead of a row's whole chain.  Each row still
    // adds its terms in the order s = 0, 1, ..., so T is bitwise the
    // row-by-row result.  A_bb is written transposed to the wave's LDS area (one 16-byte store
    // per lane: row c holds column c of A), and step s reads column s back as
    // 16-byte broadcast loads (every lane reads the same row).
    float *const At = reinterpret_cast<float *>(smem + L::ADIAG + b * L::ADIAG_WAVE);
    *reinterpret_cast<f32x4_t *>(At + col * L::LDA + rq) = ab;
    float tc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) tc[r] = r == col ? 1.f : 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 15; ++s2) {
      float ac[16];
#pragma unroll
      for (int q4 = (s2 + 1) / 4; q4 < 4; ++q4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t *>(At + s2 * L::LDA + 4 * q4);
#pragma unroll
        for (int e = 0; e < 4; ++e) ac[4 * q4 + e] = v[e];
      }
#pragma unroll
      for (int r = s2 + 1; r < 16; ++r) tc[r] = fmaf(-ac[r], tc[s2], tc[r]);
    }
    if (lane < 16) {
#pragma unroll
      for (int r = 0; r < 16; ++r) put(Tb + (16 * b + r) * BL::LDTB + col, tc[r]);
    }
  };
  auto local = [&]() {
    if (cw == 0) local_tiles(std::integral_constant<int, 0>());
    else if (cw == 1) local_tiles(std::integral_constant<int, 1>());
    else if (cw == 2) local_tiles(std::integral_constant<int, 2>());
    else local_tiles(std::integral_constant<int, 3>());
  };

  // ---- consumers: O stores straight from the accumulator layout ----------
  AT *const o_head = static_cast<AT *>(p.o) + (int64_t)h * DV;
  const int64_t o_row = (int64_t)p.H_v * DV;  // elements between tokens
  const bool o_odd = (col & 1) != 0;
  const uint32_t o_lane = (uint32_t)((rq + (o_odd ? 2 : 0)) * o_row + (col & ~1));  // elements
  AT *o_base = o_head;  // row 0 of the chunk
  int o_n = 0;          // tokens in the chunk
  auto store_o_tile = [&](int r0, int c0, const f32x4_t &acc, bool whole) {
    AT *const dst = o_base + r0 * o_row + c0 + o_lane;
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
  };

  // (0,1) and (2,3) of L o P in both local sets stay zero for the whole chain
  for (int i = tid; i < 2 * 2 * 256; i += NT) {
    const int set = i >> 9, t = (i >> 8) & 1, r = 32 * t + ((i >> 4) & 15), c = 32 * t + 16 + (i & 15);
    put(reinterpret_cast<OT *>(smem + L::LOC0 + set * L::LOC + L::L_SQ) + r * LDC + c, 0.f);
  }

  // Each role runs its own loop, so neither carries the other's registers
  // (the producers' prefetch, the consumers' state) through its iterations.
  // Both meet the same barriers: two in the prologue, two per chunk.
  const int n_chunks = (int)((t_end - t_begin + C - 1) / C);
  if (consumer) {
    // when both waves of a SIMD can issue, the consumer goes first, except
    // while its producer stages the next chunk's inputs (see there)
    __builtin_amdgcn_s_setprio(1);
    // ---- consumers: initial state (a8), read slot -> FP32 accumulators ------
    // macc[b][ia]: rows 16b.. of d_k, columns 16 (cw NA + ia).. of d_v
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
    if (rs >= 0) {  // one branch around all the loads, so they overlap
#pragma unroll
      for (int b = 0; b < DKB; ++b) {
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
          const int d = 16 * b + rq, c = 16 * (cw * NA + ia) + col;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            macc[b][ia][e] = Elem<SB>::load1(p.pool, state_base + (int64_t)(d + e) * DV + c);
        }
      }
    }

    // FP32 state -> state dtype (RNE for BF16) -> a slot: the final state, and
    // the intermediate checkpoints
    auto store_state = [&](int64_t slot) {
      const int64_t out_base = (slot * p.H_v + h) * (int64_t)DK * DV;
#pragma unroll
      for (int b = 0; b < DKB; ++b) {
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
          const int d = 16 * b + rq, c = 16 * (cw * NA + ia) + col;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Elem<SB>::store1(p.pool, out_base + (int64_t)(d + e) * DV + c, macc[b][ia][e]);
        }
      }
    };
    __syncthreads();  // prologue: chunk 0 staged
    __syncthreads();  // prologue: chunk 0's chunk-local set formed
    f32x4_t qm[4][NA], um[4][NA];  // set by their first MFMA (K-step 0 starts from zero)
    for (int c = 0; c < n_chunks; ++c) {
      const int64_t t0 = t_begin + (int64_t)c * C;
      use_set(c & 1);
      use_loc(c & 1);
      o_base = o_head + t0 * o_row;
      o_n = (int)std::min<int64_t>(C, t_end - t0);
      // ---- Q M and K M (a7) for the wave's d_v columns, the A fragments in
      // a ring RING - 1 loads ahead of their MFMAs ----
      {
        constexpr int NF = NKB * 8;  // (slab, row block, q or k)
        Frag<F32> fa[RING];
        Frag<F32> fm[NA];
        auto load_a = [&](int f) {
          return rows_afrag<RowK>((f & 1) ? Kh : Qh, 16 * ((f >> 1) & 3), 32 * (f >> 3));
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
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();  // Y (the consumers need nothing from it)

      // ---- R = beta (V - (e gamma) K M); um holds R ----
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        float vv[NA][4];
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) rows_col4<RowV>(Vh, 16 * tb, 16 * (cw * NA + ia), vv[ia]);
        const f32x4_t br = *reinterpret_cast<const f32x4_t *>(bet + 16 * tb + rq);
        const f32x4_t gr = *reinterpret_cast<const f32x4_t *>(gme + 16 * tb + rq);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) um[tb][ia][e] = br[e] * (vv[ia][e] - gr[e] * um[tb][ia][e]);
        }
      }
      // ---- U = (I + A)^-1 R (delta rules): um[i] <- T_ii (R_i - sum_{j<i} A_ij U_j) ----
      if (erase) {
        Frag16<F32> fa[6], ft[4];
#pragma unroll
        for (int i = 1, n = 0; i < 4; ++i) {
#pragma unroll
          for (int j = 0; j < i; ++j, ++n) fa[n] = load_afrag16(Ab, BL::LDAB, 16 * i, 16 * j);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ft[i] = load_afrag16(Tb, BL::LDTB, 16 * i, 0);
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
      // ---- O = (scale gamma) Q M + (scale L o P) U (a7), stored ----
      {
        Frag<F32> fu[2][NA];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) fu[s2][ia] = bfrag<F32>(um[2 * s2][ia], um[2 * s2 + 1][ia]);
        }
        Frag<F32> fs[6];
#pragma unroll
        for (int tb = 0, n = 0; tb < 4; ++tb) {
#pragma unroll
          for (int s2 = 0; s2 <= tb / 2; ++s2, ++n) fs[n] = load_afrag<F32>(Sq, LDC, 16 * tb, 32 * s2);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tb = 0, n = 0; tb < 4; ++tb) {
          const f32x4_t gr = *reinterpret_cast<const f32x4_t *>(gsc + 16 * tb + rq);
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
          if (o_n == C) {
#pragma unroll
            for (int ia = 0; ia < NA; ++ia) store_o_tile(16 * tb, 16 * (cw * NA + ia), qm[tb][ia], true);
          } else {
#pragma unroll
            for (int ia = 0; ia < NA; ++ia) store_o_tile(16 * tb, 16 * (cw * NA + ia), qm[tb][ia], false);
          }
        }
      }
      // ---- M <- gamma_last M + K^T diag(exp(G_last - G)) U ----
      {
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
        constexpr int NF = DKB * 2;  // (d_k block, token slab)
        constexpr int RK = RING < NF ? RING : NF;
        Frag<F32> fk[RK];
        auto load_k = [&](int f) { return rows_afrag_t<RowK>(Kh, 16 * (f >> 1), 32 * (f & 1)); };
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
      // an intermediate checkpoint after this chunk (a uniform branch)
      if (CK && p.ckpt_chunks > 0 && (c + 1) % p.ckpt_chunks == 0) {
        const int j = (c + 1) / p.ckpt_chunks - 1;
        if (j < p.ckpt_per_seq && (int64_t)(c + 1) * C <= t_end - t_begin) {
          const int64_t cs = p.ckpt_slot[(int64_t)seq * p.ckpt_per_seq + j];
          if (cs >= 0 && cs < p.n_slots) store_state(cs);
          else if (cs != -1 && tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
        }
      }
      __syncthreads();  // X: chunk c's sets are free; chunk c + 1's local set is written
    }
    // ---- final state (a8): FP32 -> state dtype (RNE for BF16) -> write slot ----
    if (ws >= 0) store_state(ws);
  } else {
    // prologue: chunk 0 staged and its chunk-local set formed, chunk 1 in flight
    if (n_chunks > 0) {
      fetch(t_begin);
      stage(0);
      fetch(t_begin + C);
    }
    __syncthreads();
    if (n_chunks > 0) {
      use_set(0);
      use_loc(0);
      local();
    }
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
      const int64_t t0 = t_begin + (int64_t)c * C;
        // chunk c + 1 staged, chunk c + 2 fetched, then chunk
        // c + 1's chunk-local products (on the last iterations these run on
        // clamped rows that no consumer reads) ----
        // staged above the consumers' issue priority: they wait for it at Y,
        // and at their priority the staging trailed their QM and KM (cycle
        // stamps, varlen workload: 8.25k-8.77k -> 8.11k-8.30k cycles per chunk)
        __builtin_amdgcn_s_setprio(2);
        stage((c + 1) & 1);
        __builtin_amdgcn_s_setprio(0);
        fetch(t0 + 2 * C);
        __syncthreads();  // Y: chunk c + 1's inputs are visible
        use_set((c + 1) & 1);
        use_loc((c + 1) & 1);
        local();
      __syncthreads();  // X
    }
  }
}

// The chain a shape runs, and its LDS bytes.
template <int DK, int DV, bool F32, bool AB>
constexpr size_t kChainLds =
    kPrefillPipe<DK, DV, F32> ? PipeLayout<DK, DV>::BYTES : PrefillLayout<DK, DV, F32, AB>::BYTES;

template <bool SB, bool AB, int DK, int DV, bool F32, bool CK = false>
__device__ __forceinline__ void run_chain(const PrefillParams &p, int chain, char *smem) {
  if constexpr (kPrefillPipe<DK, DV, F32>) {
    static_assert(kPrefillWaves<DK, DV, F32> == 8, "the pipelined chain runs 8 waves");
    prefill_chain_pipe<SB, AB, DK, DV, CK>(p, chain, smem);
  } else {
    prefill_chain<SB, AB, DK, DV, F32, kPlainWaves<DK, DV, F32>, CK>(p, chain, smem);
  }
}

}  // namespace gdn
