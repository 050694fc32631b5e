// prefill_chain.cuh -- one (sequence, state head) chain of the chunked
// prefill, as a device function shared by the prefill kernel and the mixed
// launcher.  The algebra and the LDS layout are described in prefill.cuh.
//
// Latency: every global input of chunk c+1 (K and Q rows, V rows, gates) is
// loaded into registers while chunk c computes, and written to LDS at the
// end of chunk c, so no chunk waits on a global-memory round trip.  The
// workgroup barriers wait only on LDS (lgkmcnt), not on these loads.
//
// Work split: the chunk-local half (S, P, A, L o P, the scaled K^T, T) is
// shared by the 4 waves through LDS; the M-dependent half runs per wave on
// the wave's own d_v columns (NA column blocks of 16), entirely in registers.
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

// One (sequence, state head) chain; all 256 threads of the workgroup call it.
// `smem` holds PrefillLayout<DK, DV, F32>::BYTES bytes, 16-byte aligned.
template <bool SB, bool AB, int DK, int DV, bool F32>
__device__ __forceinline__ void prefill_chain(const PrefillParams &p, int chain, char *smem) {
  using L = PrefillLayout<DK, DV, F32>;
  using OT = typename L::OT;
  using AT = typename Elem<AB>::T;
  static_assert(sizeof(AT) == sizeof(OT), "operands are staged in the activation dtype");
  constexpr int C = L::C;
  constexpr int LDK = L::LDK, LDC = L::LDC, LDF = L::LDF, LDV = L::LDV;
  constexpr int NKB = L::DKP / 32;  // MFMA K-steps over d_k
  constexpr int DKB = DK / 16;      // 16-row blocks of d_k
  constexpr int DVB = DV / 16;      // 16-column blocks of d_v
  constexpr int NA = DVB >= 4 ? DVB / 4 : 1;  // d_v blocks per wave
  constexpr int EW = 8 * (int)sizeof(AT) / 16;  // 16-byte vectors per 8 elements
  constexpr int KQ_GROUPS = C * (DK / 8), KQ_PER = (KQ_GROUPS + 255) / 256;
  constexpr int V_GROUPS = C * (DV / 8), V_PER = (V_GROUPS + 255) / 256;
  constexpr float LOG2E = 1.4426950408889634f;
  OT *Kh = reinterpret_cast<OT *>(smem + L::KH);
  OT *Qh = reinterpret_cast<OT *>(smem + L::QH);
  OT *Sq = reinterpret_cast<OT *>(smem + L::SQ);
  OT *Vh = reinterpret_cast<OT *>(smem + L::VH);  // V rows, then the chunk's O rows
  float *Af = reinterpret_cast<float *>(smem + L::AF);
  float *Tw = reinterpret_cast<float *>(smem + L::TW) + (threadIdx.x >> 6) * L::TW_WAVE;  // this wave's T_ii
  float *Gs = reinterpret_cast<float *>(smem + L::GATES);  // cumulative log2 decay
  float *gam = Gs + C, *bet = Gs + 2 * C, *eGn = Gs + 3 * C;

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
  if (t_begin < 0 || t_end < t_begin || t_end > p.n_tokens) {  // offsets break the contract
    if (tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SEQ);
    return;
  }
  const bool decay = (p.rule & kRuleDecay) != 0;
  const bool erase = (p.rule & kRuleErase) != 0;

  // ---- prefetch of one chunk's inputs into registers, and their staging ----
  // The loads are unconditional: a row past the sequence's end re-reads its
  // last token.  Such padded rows are harmless because their beta factor is
  // zero: their rows of A and U vanish, so they reach neither M nor a stored
  // O row.  (Held as vector values, so they stay in registers.)
  u32x4_t pk[KQ_PER][EW], pq[KQ_PER][EW], pv[V_PER][EW];
  float pg = 0.f, pb = 0.f;  // wave 0: gate inputs of token `lane`
  bool p_valid = false;       // wave 0: token `lane` lies inside the sequence
  auto fetch = [&](int64_t t0) {
    const int64_t last = t_end - 1;
#pragma unroll
    for (int i = 0; i < KQ_PER; ++i) {
      const int gi = tid + 256 * i;
      const int r = gi / (DK / 8), d = (gi % (DK / 8)) * 8;
      const int64_t off = (std::min(t0 + r, last) * p.H_qk + hq) * DK + d;
      const u32x4_t *sk = reinterpret_cast<const u32x4_t *>(static_cast<const AT *>(p.k) + off);
      const u32x4_t *sq = reinterpret_cast<const u32x4_t *>(static_cast<const AT *>(p.q) + off);
#pragma unroll
      for (int e = 0; e < EW; ++e) { pk[i][e] = sk[e]; pq[i][e] = sq[e]; }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int gi = tid + 256 * i;
      const int r = gi / (DV / 8), c = (gi % (DV / 8)) * 8;
      const u32x4_t *sv = reinterpret_cast<const u32x4_t *>(
          static_cast<const AT *>(p.v) + (std::min(t0 + r, last) * p.H_v + h) * DV + c);
#pragma unroll
      for (int e = 0; e < EW; ++e) pv[i][e] = sv[e];
    }
    if (wave == 0) {
      // raw values only: any arithmetic on them here would wait for the whole
      // fetch (loads retire in order); stage() masks them.  g and beta may be
      // NULL under the rules that do not use them.
      const int64_t gt = std::min(t0 + lane, last) * p.H_v + h;
      if (decay) pg = p.g[gt];
      if (erase) pb = p.beta[gt];
      p_valid = t0 + lane <= last;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < KQ_PER; ++i) {
      const int gi = tid + 256 * i;
      if (KQ_GROUPS % 256 != 0 && gi >= KQ_GROUPS) continue;
      const int r = gi / (DK / 8), d = (gi % (DK / 8)) * 8;
      u32x4_t *dk = reinterpret_cast<u32x4_t *>(Kh + r * LDK + d);
      u32x4_t *dq = reinterpret_cast<u32x4_t *>(Qh + r * LDK + d);
#pragma unroll
      for (int e = 0; e < EW; ++e) { dk[e] = pk[i][e]; dq[e] = pq[i][e]; }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int gi = tid + 256 * i;
      if (V_GROUPS % 256 != 0 && gi >= V_GROUPS) continue;
      const int r = gi / (DV / 8), c = (gi % (DV / 8)) * 8;
      u32x4_t *dv = reinterpret_cast<u32x4_t *>(Vh + r * LDV + c);
#pragma unroll
      for (int e = 0; e < EW; ++e) dv[e] = pv[i][e];
    }
    if (wave == 0) {
      // inclusive prefix sum of the log2 decays over the chunk's 64 tokens
      const float G = wave_inclusive_sum(p_valid && decay ? pg * LOG2E : 0.f);
      const float G_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), 63));
      Gs[lane] = G;
      gam[lane] = fast_exp2(G);
      bet[lane] = p_valid ? (erase ? pb : 1.f) : 0.f;  // the plain rules take R = beta V
      eGn[lane] = fast_exp2(G_last - G);
    }
  };

  // O rows r0 + rq .. r0 + rq + 3 of column c0 + col, held by this lane in
  // the accumulator layout, scaled and stored (only rows inside the chunk).
  // BF16: each lane swaps halves with its neighbour column (lane ^ 1), so a
  // lane stores two rows of a column pair as 4-byte words.
  AT *const o_head = static_cast<AT *>(p.o) + (int64_t)h * DV;
  const int64_t o_row = (int64_t)p.H_v * DV;  // elements between tokens
  int64_t o_t0 = 0;                           // first token of the chunk
  int o_n = 0;                                // tokens in the chunk
  auto store_o_tile = [&](int r0, int c0, const f32x4_t &acc) {
    if constexpr (AB) {
      const bool odd = (col & 1) != 0;
      const uint32_t a = pack_bf16x2(p.scale * acc[0], p.scale * acc[1]);  // rows 0, 1
      const uint32_t b = pack_bf16x2(p.scale * acc[2], p.scale * acc[3]);  // rows 2, 3
      const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? a : b), 0xB1, 0xf, 0xf, false);
      const uint32_t own = odd ? b : a;
      const uint32_t left = odd ? other : own, right = odd ? own : other;  // columns c, c + 1
      const int r = r0 + rq + (odd ? 2 : 0);
      AT *dst = o_head + (o_t0 + r) * o_row + c0 + (col & ~1);
      if (r < o_n) *reinterpret_cast<uint32_t *>(dst) = __builtin_amdgcn_perm(right, left, 0x05040100u);
      if (r + 1 < o_n)
        *reinterpret_cast<uint32_t *>(dst + o_row) = __builtin_amdgcn_perm(right, left, 0x07060302u);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = r0 + rq + e;
        if (r < o_n) o_head[(o_t0 + r) * o_row + c0 + col] = p.scale * acc[e];
      }
    }
  };

  // padded K columns (d_k < 32 only) stay zero for the whole chain
  if constexpr (L::DKP > DK) {
    constexpr int PADC = L::DKP - DK;
    for (int i = tid; i < 2 * C * PADC; i += 256) {
      const int row = i / PADC, c = DK + i % PADC;
      if (row < C) put(Kh + row * LDK + c, 0.f);
      else put(Qh + (row - C) * LDK + c, 0.f);
    }
  }

  // ---- initial state (a8): read slot -> FP32 accumulators ----
  // macc[b][ia]: rows 16b.. of d_k, columns 16 (wave NA + ia).. of d_v, in the
  // accumulator layout (lane (g, n): rows 4g..4g+3 of column n)
  const bool mwave = DVB >= 4 || wave < DVB;  // waves that own d_v columns
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
  if (t_begin < t_end) {
    fetch(t_begin);
    stage();
  }
  __syncthreads();

  for (int64_t t0 = t_begin; t0 < t_end; t0 += C) {
    const int n = (int)std::min<int64_t>(C, t_end - t0);
    const int64_t t1 = t0 + C;
    const bool more = t1 < t_end;
    o_t0 = t0;
    o_n = n;

    // ---- 2 and 5: S = K K^T, P = Q K^T for row block `wave` (a6), and Q M,
    // K M (a7) for the wave's d_v columns.  All of them read only this chunk's
    // K and Q rows and the state, so they share one pass over the d_k slabs
    // and their MFMAs interleave. ----
    f32x4_t sacc[4], pacc[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sacc[cb][e] = pacc[cb][e] = 0.f;
    }
    f32x4_t qm[4][NA], um[4][NA];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int ia = 0; ia < NA; ++ia) {
#pragma unroll
        for (int e = 0; e < 4; ++e) qm[tb][ia][e] = um[tb][ia][e] = 0.f;
      }
    }
    // S and P (S unused without erase: no branch, straight-line code), the
    // fragments of step f + 1 loaded during step f's MFMAs
    {
      constexpr int NF = NKB * 4;  // (slab, column block)
      Frag<F32> fk[2], fq[2], fb[2];
      fk[0] = load_frag<F32>(Kh, LDK, 16 * wave, 0);
      fq[0] = load_frag<F32>(Qh, LDK, 16 * wave, 0);
      fb[0] = load_frag<F32>(Kh, LDK, 0, 0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kk = f >> 2, cb = f & 3;
        if (f + 1 < NF) {
          const int kn = (f + 1) >> 2;
          if (((f + 1) & 3) == 0) {
            fk[kn & 1] = load_frag<F32>(Kh, LDK, 16 * wave, 32 * kn);
            fq[kn & 1] = load_frag<F32>(Qh, LDK, 16 * wave, 32 * kn);
          }
          fb[(f + 1) & 1] = load_frag<F32>(Kh, LDK, 16 * ((f + 1) & 3), 32 * kn);
        }
        __builtin_amdgcn_sched_barrier(0);
        sacc[cb] = mma<F32>(sacc[cb], fk[kk & 1], fb[f & 1]);
        pacc[cb] = mma<F32>(pacc[cb], fq[kk & 1], fb[f & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Q M and K M with the A fragments double-buffered by hand: the load of
    // fragment f+1 is issued before the MFMAs of fragment f (scheduling
    // barriers keep the compiler from moving it back next to its use)
    if (mwave) {
      constexpr int NF = NKB * 8;  // (slab, row block, q or k)
      Frag<F32> fa[2];
      Frag<F32> fm[NA];
      fa[0] = load_afrag<F32>(Qh, LDK, 0, 0);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kk = f >> 3, tb = (f >> 1) & 3, isk = f & 1;
        if (f + 1 < NF) {
          const int kn = (f + 1) >> 3, tn = ((f + 1) >> 1) & 3, kn_isk = (f + 1) & 1;
          fa[(f + 1) & 1] = load_afrag<F32>(kn_isk ? Kh : Qh, LDK, 16 * tn, 32 * kn);
        }
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
          if (isk) um[tb][ia] = mma<F32>(um[tb][ia], fa[f & 1], fm[ia]);
          else qm[tb][ia] = mma<F32>(qm[tb][ia], fa[f & 1], fm[ia]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // ---- 3: A = strict_lower(beta_r e^{G_r-G_s} S), Sq = lower(e^{G_r-G_s} P) ----
    {
      float Gr[4], br[4], Gc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Gr[e] = Gs[16 * wave + rq + e];
        br[e] = bet[16 * wave + rq + e];
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) Gc[cb] = Gs[16 * cb + col];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * wave + rq + e, s = 16 * cb + col;
          const float dec = s <= r ? fast_exp2(Gr[e] - Gc[cb]) : 0.f;
          Af[r * LDF + s] = (erase && s < r) ? br[e] * dec * sacc[cb][e] : 0.f;
          put(Sq + r * LDC + s, dec * pacc[cb][e]);
        }
      }
    }
    __syncthreads();
    // the next chunk's inputs, in flight through the rest of this chunk (issued
    // only now so the prefetch registers are free during the MFMA pass above)
    if (more) fetch(t1);

    // ---- 5-8: the wave's d_v columns, in registers ----
    if (mwave) {
      // T_bb = (I + A_bb)^-1 for the four diagonal 16 x 16 blocks, by forward
      // substitution: lane (bb, c) forms column c of T_bb; into this wave's Tw
      if (erase) {
        const int bb = lane >> 4, c = lane & 15;
        float tc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = r == c ? 1.f : 0.f;
          const float *arow = Af + (16 * bb + r) * LDF + 16 * bb;
#pragma unroll
          for (int s2 = 0; s2 < r; ++s2) x = fmaf(-arow[s2], tc[s2], x);
          tc[r] = x;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tw[(16 * bb + r) * L::LDT + c] = tc[r];
      }
      // R = beta (V - gamma K M) for the delta rules, else R = V (beta holds 1 on
      // the chunk's tokens and 0 on its padded rows); um holds R
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        float vv[NA][4];
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) load_col4(Vh, LDV, 16 * tb, 16 * (wave * NA + ia), vv[ia]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tb + rq + e;
          const float br = bet[r], gr = gam[r];
#pragma unroll
          for (int ia = 0; ia < NA; ++ia)
            um[tb][ia][e] = br * (erase ? vv[ia][e] - gr * um[tb][ia][e] : vv[ia][e]);
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
          for (int j = 0; j < i; ++j, ++n) fa[n] = load_afrag16<F32>(Af, LDF, 16 * i, 16 * j, -1.f);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) ft[i] = load_afrag16<F32>(Tw, L::LDT, 16 * i, 0, 1.f);
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
      // 7: O = gamma Q M + (L o P) U (a7), scaled, stored to HBM straight from
      // the accumulator layout
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
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
#pragma unroll
          for (int e = 0; e < 4; ++e) qm[tb][ia][e] *= gam[16 * tb + rq + e];
        }
#pragma unroll
        for (int s2 = 0; s2 <= tb / 2; ++s2, ++n) {
#pragma unroll
          for (int ia = 0; ia < NA; ++ia) qm[tb][ia] = mma<F32>(qm[tb][ia], fs[n], fu[s2][ia]);
        }
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) store_o_tile(16 * tb, 16 * (wave * NA + ia), qm[tb][ia]);
      }
      // 8: M <- gamma_last M + K^T diag(exp(G_last - G)) U: the decay weights
      // scale U's rows; K^T's fragments are read down the columns of the K rows
      Frag<F32> fe[2][NA];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int ia = 0; ia < NA; ++ia) {
          f32x4_t lo = um[2 * s2][ia], hi = um[2 * s2 + 1][ia];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] *= eGn[32 * s2 + rq + e];
            hi[e] *= eGn[32 * s2 + 16 + rq + e];
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
      // K^T fragments double-buffered: the next one loads during this one's MFMAs
      {
        constexpr int NF = DKB * 2;  // (d_k block, token slab)
        Frag<F32> fk[2];
        fk[0] = load_afrag_t<F32>(Kh, LDK, 0, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + 1 < NF) fk[(f + 1) & 1] = load_afrag_t<F32>(Kh, LDK, 16 * ((f + 1) >> 1), 32 * ((f + 1) & 1));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ia = 0; ia < NA; ++ia)
            macc[f >> 1][ia] = mma<F32>(macc[f >> 1][ia], fk[f & 1], fe[f & 1][ia]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    __syncthreads();  // all reads of this chunk's LDS operands are done
    if (more) stage();  // next chunk's K, Q, V and gates into LDS
    __syncthreads();
  }

  // ---- final state (a8): FP32 -> state dtype (RNE for BF16) -> write slot ----
  if (ws >= 0 && mwave) {
    const int64_t out_base = (ws * p.H_v + h) * (int64_t)DK * DV;
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
  }
}

}  // namespace gdn
