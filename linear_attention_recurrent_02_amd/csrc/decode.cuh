// decode.cuh -- the decode state-update tile: one (request, state head) pair.
//
// Per tile the state M (d_k x d_v, rows = key index) is read once from its
// read slot, kept in registers, updated and written once to its write slot:
//
//   u = M^T k,  w = M^T q,  kq = k . q        (reductions over the d_k rows)
//   delta = bw * (v - c * a * u)             (c = 1 for the delta rules)
//   o     = scale * (a * w + kq * delta)     (= scale * M'^T q)
//   M'    = a * M + k delta^T
//
// This is the residual form of the update given in the Kimi Linear section of
// "Seven Architectures Replacing KV Cache With Bounded Mutable State" with a
// scalar decay (which the Gated DeltaNet-2 section says is Gated DeltaNet),
// and the read-out is the rearrangement in the "Gated DeltaNet" glossary
// entry, Engineering details: the decayed old state read by the query plus,
// for the current token, a per-head scalar (k . q) times a small vector.  The
// read-out therefore never waits for the new state.
//
// With a per-key-channel decay (CW: Kimi Delta Attention, the same Kimi
// Linear section) the decay multiplies row i by a_i = exp(g_i) before the
// delta correction reads the state, so the reductions take a_i k_i and
// a_i q_i, a = 1 in delta and o, and the update is M'_i = a_i M_i + k_i delta.
//
// With 8-bit storage (Q8: DAMP's mixed precision, "Seven Architectures ...",
// ONNX LinearAttention / FlashInfer section) the first hi_rows key channels
// (rows) of a tile are BF16 and the others INT8 with one binary32 scale per
// row: the tile is [hi_rows, d_v] BF16 | [d_k - hi_rows, d_v] int8 codes |
// [d_k - hi_rows] scales.  A row is read as code * scale; on store it is
// requantised against its own largest magnitude (code = rne(x * 127 / rowmax),
// scale = rowmax / 127), the maximum taken across the LPR lanes of the row.
// hi_rows is a multiple of the rows one wave holds (or 0 or d_k), so a wave's
// rows are all BF16 or all INT8: the kernel branches once per wave and runs
// an instance of one row kind (I8), which keeps the registers of one kind.
//
// Work split (gfx950, wave64): every column j of the update is independent
// given k, q and v, so a lane owns VEC consecutive columns (one 16-byte
// vector per row) and RPT consecutive rows; LPR lanes cover one row, so each
// wave-wide load instruction moves whole contiguous 256-byte rows.  The only
// cross-lane work is the sum over rows: a butterfly across the lanes of a
// wave that share columns, then NW partials through LDS.
#pragma once

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace gdn {

// Workgroup size cap for the decode tile.
constexpr int kDecodeMaxThreads = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// The state stream: every state byte is touched exactly once per call, so its
// loads and stores are non-temporal (nothing to keep in the caches; measured
// 202 against 216 us per B = 512 launch with plain loads in request order).
__device__ __forceinline__ uint4 stream_load(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void stream_store(uint4 *p, const uint4 &v) {
  u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t *>(p));
}
// the same for the 8-byte pieces of INT8 rows
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 stream_load8(const uint2 *p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void stream_store8(uint2 *p, uint32_t lo, uint32_t hi) {
  u32x2_t w = {lo, hi};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t *>(p));
}

// The largest value over each aligned group of L lanes (L = 2, 4, 8, 16: the
// lanes of one state row), left in every lane of the group: DPP moves inside
// a 16-lane row, no LDS round trip -- swap neighbours, swap pairs, mirror each
// half-row, mirror the row.
template <int L>
__device__ __forceinline__ float lane_group_max(float m) {
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "a row spans 1..16 lanes");
  auto mv = [](float x, auto ctrl) {
    return __int_as_float(
        __builtin_amdgcn_mov_dpp(__float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  if constexpr (L >= 2) m = fmaxf(m, mv(m, std::integral_constant<int, 0xB1>()));   // quad_perm 1,0,3,2
  if constexpr (L >= 4) m = fmaxf(m, mv(m, std::integral_constant<int, 0x4E>()));   // quad_perm 2,3,0,1
  if constexpr (L >= 8) m = fmaxf(m, mv(m, std::integral_constant<int, 0x141>()));  // row_half_mirror
  if constexpr (L >= 16) m = fmaxf(m, mv(m, std::integral_constant<int, 0x140>()));  // row_mirror
  return m;
}

// eight INT8 codes (the low 8 bytes of m) times their row's scale
__device__ __forceinline__ void unpack_i8(const uint2 &m, float sc, float *f) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w = j < 4 ? m.x : m.y;
    f[j] = (float)(int8_t)(w >> (8 * (j & 3))) * sc;
  }
}

struct DecodeParams {
  int32_t B, H_qk, H_v, group;  // group = H_v / H_qk
  int64_t n_slots;
  float scale;
  int32_t rule;
  const void *q, *k, *v;
  const float *g, *beta;
  void *pool;
  const int32_t *read_slot, *write_slot;
  void *o;
  uint32_t *status;
  // 8-bit storage: BF16 rows at the head of each tile, and the tile's bytes
  int32_t hi_rows;
  int64_t tile_bytes;
};

template <bool SB, int DK, int DV, int NT>
struct DecodeShape {
  static constexpr int VEC = Elem<SB>::kPer16B;  // state elements per 16-byte vector
  static constexpr int LPR = DV / VEC;           // lanes per state row
  static_assert(DV % VEC == 0 && LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "bad d_v");
  static constexpr int RG = NT / LPR;            // row groups in the workgroup
  static constexpr int RPT = (DK + RG - 1) / RG; // rows per thread
  static constexpr int NW = NT / 64;             // waves
  static constexpr int LDS_FLOATS = (NW + 1) * (2 * DV + 1);
  // every row group owns rows (true unless the tile is tiny)
  static constexpr bool ALL_LIVE = RG * RPT == DK;
};

// Registers of one (request, state head) tile between its two phases.  When
// the thread's runs of k, q (RPT rows) and v (VEC columns) are whole 16-byte
// vectors they are kept packed as loaded (half the registers for BF16) and
// unpacked in phase 2.
template <bool SB, bool AB, int DK, int DV, int NT, bool CW = false, bool Q8 = false,
          bool I8 = false>
struct DecodeTileRegs {
  using S = DecodeShape<SB, DK, DV, NT>;
  static constexpr int AV = Elem<AB>::kPer16B;  // activation elements per 16 bytes
  static constexpr bool PACKED =
      S::ALL_LIVE && DK % S::RPT == 0 && S::RPT % AV == 0 && S::VEC % AV == 0;
  static constexpr int KN = PACKED ? S::RPT / AV : 1;
  static constexpr int VN = PACKED ? S::VEC / AV : 1;
  // the packed state rows of this thread: 16-byte pieces, or the 8-byte
  // pieces of INT8 rows
  std::conditional_t<I8, uint2, uint4> m[S::RPT];
  uint4 kp[KN], qp[KN], vp[VN];     // packed k, q, v (PACKED)
  float kr[PACKED ? 1 : S::RPT], qr[PACKED ? 1 : S::RPT], vv[PACKED ? 1 : S::VEC];
  float a, bw;                      // decay and write strength
  float ar[CW ? S::RPT : 1];        // CW: the decay of each of this thread's rows
  float sc[I8 ? S::RPT : 1];        // INT8 rows: the scale of each
  int64_t r, ws;                    // request, write slot
  int h;
  bool valid;                       // false: a bad slot (the tile is skipped)
};

// Phase 1 of a tile: resolve the slots (a1) and issue every load -- this
// token's q, k, v first, then the state tile -- without waiting for any of
// them, so the caller can overlap them with the previous tile's phase 2.  All
// NT threads of a group call it with the same (r, h), each passing its index
// in the group as `tid`: the workgroup, or one of its aligned NT-thread parts
// (each with its own `red`).
template <bool SB, bool AB, int DK, int DV, int NT, bool CW = false, bool Q8 = false,
          bool I8 = false>
__device__ __forceinline__ void decode_tile_load(const DecodeParams &p, int64_t r, int h,
                                                 DecodeTileRegs<SB, AB, DK, DV, NT, CW, Q8, I8> &t,
                                                 int tid) {
  static_assert(!Q8 || SB, "8-bit storage uses the BF16 tile shape");
  static_assert(Q8 || !I8, "INT8 rows exist in the 8-bit format only");
  using S = DecodeShape<SB, DK, DV, NT>;
  constexpr int VEC = S::VEC, LPR = S::LPR, RPT = S::RPT;
  constexpr bool ALL_LIVE = S::ALL_LIVE;
  using SE = Elem<SB>;
  const int cv = tid % LPR;  // column vector: columns [cv*VEC, cv*VEC + VEC)
  const int row0 = (tid / LPR) * RPT;  // rows [row0, row0 + RPT)

  t.r = r;
  t.h = h;
  const int64_t rs = p.read_slot ? (int64_t)p.read_slot[r] : r;
  t.ws = p.write_slot ? (int64_t)p.write_slot[r] : r;
  t.valid = !(rs < -1 || rs >= p.n_slots || t.ws < -1 || t.ws >= p.n_slots);
  if (!t.valid) {
    if (tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
    return;
  }
  const int hq = h / p.group;
  constexpr int64_t TILE = (int64_t)DK * DV;

  // this token's q, k (rows of this thread), v (its columns); issued before
  // the state tile: loads return in order, so waiting for these leaves the
  // state loads in flight
  using Regs = DecodeTileRegs<SB, AB, DK, DV, NT, CW, Q8, I8>;
  using AT = typename Elem<AB>::T;
  if constexpr (Regs::PACKED) {
    const uint4 *kp = reinterpret_cast<const uint4 *>(static_cast<const AT *>(p.k) +
                                                      (r * p.H_qk + hq) * DK + row0);
    const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const AT *>(p.q) +
                                                      (r * p.H_qk + hq) * DK + row0);
    const uint4 *vp = reinterpret_cast<const uint4 *>(static_cast<const AT *>(p.v) +
                                                      (r * p.H_v + h) * DV + cv * VEC);
#pragma unroll
    for (int j = 0; j < Regs::KN; ++j) { t.kp[j] = kp[j]; t.qp[j] = qp[j]; }
#pragma unroll
    for (int j = 0; j < Regs::VN; ++j) t.vp[j] = vp[j];
  } else {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const bool ok = row0 + i < DK;
      t.kr[i] = ok ? Elem<AB>::load1(p.k, (r * p.H_qk + hq) * DK + row0 + i) : 0.f;
      t.qr[i] = ok ? Elem<AB>::load1(p.q, (r * p.H_qk + hq) * DK + row0 + i) : 0.f;
    }
    load_run<AB, VEC>(p.v, (r * p.H_v + h) * DV + cv * VEC, t.vv);
  }

  // the gates, issued before the state tile like q, k, v, so their
  // exponentials overlap the state's loads: g per head, or (CW, g is
  // [B, H_v, d_k]) the run of RPT log-decays as 16-byte loads (host-checked
  // alignment), and beta
  const bool decay = (p.rule & kRuleDecay) != 0;
  const bool erase = (p.rule & kRuleErase) != 0;
  constexpr int G4 = CW && ALL_LIVE && RPT % 4 == 0 ? RPT / 4 : 1;
  float4 g4s[G4];
  float g1 = 0.f;
  if constexpr (CW && ALL_LIVE && RPT % 4 == 0) {
    const float4 *gr4 = reinterpret_cast<const float4 *>(p.g + (r * p.H_v + h) * DK + row0);
#pragma unroll
    for (int i = 0; i < G4; ++i) g4s[i] = decay ? gr4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
  } else if constexpr (!CW) {
    g1 = decay ? p.g[r * p.H_v + h] : 0.f;
  }
  const float b1 = erase ? p.beta[r * p.H_v + h] : 1.0f;

  // the state tile: RPT 16-byte vectors per thread (a1); 8-byte pieces and
  // one scale per row for the INT8 rows of an 8-bit tile
  if constexpr (Q8) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      t.m[i] = {};
      if constexpr (I8) t.sc[i] = 0.f;
    }
    if (rs >= 0) {
      const char *tile = static_cast<const char *>(p.pool) + (rs * p.H_v + h) * p.tile_bytes;
      if constexpr (!I8) {
        const uint4 *src = reinterpret_cast<const uint4 *>(tile);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
          if (ALL_LIVE || row0 + i < DK) t.m[i] = stream_load(src + (int64_t)(row0 + i) * LPR + cv);
      } else {
        const int lo = row0 - p.hi_rows;  // INT8 row index of the thread's first row
        const int64_t hi_b = (int64_t)p.hi_rows * DV * 2;
        const uint2 *src = reinterpret_cast<const uint2 *>(tile + hi_b);
        const float *scl = reinterpret_cast<const float *>(tile + hi_b + (int64_t)(DK - p.hi_rows) * DV);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          if (ALL_LIVE || row0 + i < DK) t.m[i] = stream_load8(src + (int64_t)(lo + i) * LPR + cv);
        }
        // the run's scales: contiguous, and 16-byte aligned when RPT is a
        // multiple of 4 (lo is a multiple of RPT, the scale area of 16)
        if constexpr (ALL_LIVE && RPT % 4 == 0) {
#pragma unroll
          for (int i = 0; i < RPT; i += 4) {
            const float4 s4 = *reinterpret_cast<const float4 *>(scl + lo + i);
            t.sc[i] = s4.x; t.sc[i + 1] = s4.y; t.sc[i + 2] = s4.z; t.sc[i + 3] = s4.w;
          }
        } else {
#pragma unroll
          for (int i = 0; i < RPT; ++i)
            if (ALL_LIVE || row0 + i < DK) t.sc[i] = scl[lo + i];
        }
      }
    }
  } else if (rs >= 0) {
    const uint4 *src = reinterpret_cast<const uint4 *>(
        static_cast<const typename SE::T *>(p.pool) + ((rs * p.H_v + h) * TILE));
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if (ALL_LIVE || row0 + i < DK) t.m[i] = stream_load(src + (int64_t)(row0 + i) * LPR + cv);
      else t.m[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < RPT; ++i) t.m[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if constexpr (CW) {
    // this thread's rows' decays, through the hardware exponential (expf
    // measured 0.8% slower per B=512 launch); their loads were issued with
    // q, k, v, ahead of the state
    t.a = 1.0f;
    if constexpr (ALL_LIVE && RPT % 4 == 0) {
#pragma unroll
      for (int i = 0; i < RPT; i += 4) {
        const float4 g4 = g4s[i / 4];
        t.ar[i] = __expf(g4.x); t.ar[i + 1] = __expf(g4.y);
        t.ar[i + 2] = __expf(g4.z); t.ar[i + 3] = __expf(g4.w);
      }
    } else {
      const float *gr = p.g + (r * p.H_v + h) * DK + row0;
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        t.ar[i] = decay && (ALL_LIVE || row0 + i < DK) ? __expf(gr[i]) : 1.0f;
    }
  } else {
    t.a = decay ? expf(g1) : 1.0f;
  }
  t.bw = b1;
}

// Phase 2 of a tile: the reductions over rows, the read-out (a4), the update
// and the store to the write slot (a5).  `red` is LDS of
// DecodeShape::LDS_FLOATS floats.  For NW > 1 it has three barriers (the last
// lets the caller reuse `red`); a skipped tile has none, uniformly.
template <bool SB, bool AB, int DK, int DV, int NT, bool CW = false, bool Q8 = false,
          bool I8 = false>
__device__ __forceinline__ void decode_tile_finish(const DecodeParams &p,
                                                   DecodeTileRegs<SB, AB, DK, DV, NT, CW, Q8, I8> &t,
                                                   float *red, int tid) {
  using S = DecodeShape<SB, DK, DV, NT>;
  constexpr int VEC = S::VEC, LPR = S::LPR, RPT = S::RPT, NW = S::NW;
  constexpr bool ALL_LIVE = S::ALL_LIVE;
  using SE = Elem<SB>;
  if (!t.valid) return;
  const int cv = tid % LPR;
  const int row0 = (tid / LPR) * RPT;
  const bool rows_live = ALL_LIVE || row0 < DK;
  const bool erase = (p.rule & kRuleErase) != 0;
  const float a = t.a;
  const int64_t r = t.r;
  const int h = t.h;
  constexpr int64_t TILE = (int64_t)DK * DV;
  using Regs = DecodeTileRegs<SB, AB, DK, DV, NT, CW, Q8, I8>;
  // Q8: the thread's rows are INT8 (I8) or BF16 (the tile's head); the kind
  // is fixed per wave (the caller's branch), so each instance has one kind
  auto unpack_row = [&](int i, float *f) {
    if constexpr (I8) unpack_i8(t.m[i], t.sc[i], f);
    else SE::unpack(t.m[i], f);
  };
  float kr[RPT], qr[RPT], vv[VEC];
  if constexpr (Regs::PACKED) {
#pragma unroll
    for (int j = 0; j < Regs::KN; ++j) {
      Elem<AB>::unpack(t.kp[j], kr + j * Regs::AV);
      Elem<AB>::unpack(t.qp[j], qr + j * Regs::AV);
    }
#pragma unroll
    for (int j = 0; j < Regs::VN; ++j) Elem<AB>::unpack(t.vp[j], vv + j * Regs::AV);
  } else {
#pragma unroll
    for (int i = 0; i < RPT; ++i) { kr[i] = t.kr[i]; qr[i] = t.qr[i]; }
#pragma unroll
    for (int e = 0; e < VEC; ++e) vv[e] = t.vv[e];
  }

  // ---- partial reductions over this thread's rows ----
  float u[VEC], w[VEC];
  float kq = 0.f;
#pragma unroll
  for (int e = 0; e < VEC; ++e) u[e] = w[e] = 0.f;
  auto partials = [&]() {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float f[VEC];
      unpack_row(i, f);
      // CW: the decayed row a_i M_i is what k and q read
      const float kd = CW ? t.ar[i] * kr[i] : kr[i], qd = CW ? t.ar[i] * qr[i] : qr[i];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        u[e] = fmaf(f[e], kd, u[e]);
        w[e] = fmaf(f[e], qd, w[e]);
      }
      kq = fmaf(kr[i], qr[i], kq);
    }
  };
  partials();
  // butterfly over the lanes of this wave that share column vector cv
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      u[e] += __shfl_xor(u[e], off);
      w[e] += __shfl_xor(w[e], off);
    }
    kq += __shfl_xor(kq, off);
  }
  const int lane = tid & 63, wave = tid >> 6;
  if constexpr (NW > 1) {
    // two levels through LDS: each wave's totals, then thread j sums value j
    // over the waves, then every thread reads back only what it needs
    constexpr int NV = 2 * DV + 1;  // u[0..DV), w[0..DV), kq
    float *mine = red + wave * NV;
    if (lane < LPR) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        mine[cv * VEC + e] = u[e];
        mine[DV + cv * VEC + e] = w[e];
      }
      if (lane == 0) mine[2 * DV] = kq;
    }
    __syncthreads();
    float *tot = red + NW * NV;
    for (int j = tid; j < NV; j += NT) {
      float sum = 0.f;
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) sum += red[wv * NV + j];
      tot[j] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < VEC; ++e) u[e] = tot[cv * VEC + e];
    if (tid < LPR) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) w[e] = tot[DV + cv * VEC + e];
      kq = tot[2 * DV];
    }
  }
  // keep the tile packed across the reduction instead of holding it unpacked
#pragma unroll
  for (int i = 0; i < RPT; ++i) opaque(t.m[i]);

  // ---- delta, read-out (a4) ----
  float d[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) d[e] = erase ? t.bw * (vv[e] - a * u[e]) : vv[e];
  if (tid < LPR) {
    float o[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = p.scale * fmaf(a, w[e], kq * d[e]);
    store_run<AB, VEC>(p.o, (r * p.H_v + h) * DV + cv * VEC, o);
  }

  // ---- update and scatter to the write slot (a5) ----
  if constexpr (Q8) {
    if (t.ws >= 0) {  // uniform over the tile: every lane takes part in the row maxima
      char *tile = static_cast<char *>(p.pool) + (t.ws * p.H_v + h) * p.tile_bytes;
      if constexpr (!I8) {
        uint4 *dst = reinterpret_cast<uint4 *>(tile);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          if (!ALL_LIVE && row0 + i >= DK) continue;
          float f[VEC];
          unpack_row(i, f);
          const float ai = CW ? t.ar[i] : a;
#pragma unroll
          for (int e = 0; e < VEC; ++e) f[e] = fmaf(kr[i], d[e], ai * f[e]);
          stream_store(dst + (int64_t)(row0 + i) * LPR + cv, SE::pack(f));
        }
      } else {
        const int lo = row0 - p.hi_rows;
        const int64_t hi_b = (int64_t)p.hi_rows * DV * 2;
        uint2 *dst = reinterpret_cast<uint2 *>(tile + hi_b);
        float *scl = reinterpret_cast<float *>(tile + hi_b + (int64_t)(DK - p.hi_rows) * DV);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const bool live = ALL_LIVE || row0 + i < DK;
          float f[VEC];
          unpack_row(i, f);
          const float ai = CW ? t.ar[i] : a;
          float m = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            f[e] = fmaf(kr[i], d[e], ai * f[e]);
            m = fmaxf(m, fabsf(f[e]));
          }
          // the row's largest magnitude over its LPR lanes (an aligned lane group)
          m = lane_group_max<LPR>(m);
          const float inv = m > 0.f ? 127.f / m : 0.f;
          uint32_t w[2] = {0u, 0u};
#pragma unroll
          for (int e = 0; e < VEC; ++e) {
            const float y = fminf(fmaxf(f[e] * inv, -127.f), 127.f);
            w[e >> 2] |= ((uint32_t)(int)rintf(y) & 0xffu) << (8 * (e & 3));
          }
          if (live) {
            stream_store8(dst + (int64_t)(lo + i) * LPR + cv, w[0], w[1]);
            if (cv == 0) scl[lo + i] = m / 127.f;
          }
        }
      }
    }
  } else if (t.ws >= 0 && rows_live) {
    uint4 *dst = reinterpret_cast<uint4 *>(static_cast<typename SE::T *>(p.pool) +
                                           ((t.ws * p.H_v + h) * TILE));
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      if (!ALL_LIVE && row0 + i >= DK) continue;
      float f[VEC];
      unpack_row(i, f);
      const float ai = CW ? t.ar[i] : a;
#pragma unroll
      for (int e = 0; e < VEC; ++e) f[e] = fmaf(kr[i], d[e], ai * f[e]);
      stream_store(dst + (int64_t)(row0 + i) * LPR + cv, SE::pack(f));
    }
  }
  if constexpr (NW > 1) __syncthreads();  // `red` may be reused by the next tile
}

// One whole tile (both phases, no overlap).
template <bool SB, bool AB, int DK, int DV, int NT>
__device__ __forceinline__ void decode_tile(const DecodeParams &p, int64_t r, int h, float *red) {
  DecodeTileRegs<SB, AB, DK, DV, NT> t;
  decode_tile_load<SB, AB, DK, DV, NT>(p, r, h, t, (int)threadIdx.x);
  decode_tile_finish<SB, AB, DK, DV, NT>(p, t, red, (int)threadIdx.x);
}

// Threads per workgroup for a tile of d_k rows of lpr lanes each: enough
// lanes for every row group to own at least one row, at most 256.
__host__ __device__ constexpr int decode_threads_for(int lpr, int dk) {
  return lpr * dk >= kDecodeMaxThreads ? kDecodeMaxThreads : (lpr * dk <= 64 ? 64 : lpr * dk);
}
template <bool SB, int DK, int DV>
constexpr int decode_threads() {
  return decode_threads_for(DV / Elem<SB>::kPer16B, DK);
}

// The rows one wave of the BF16-shaped tile holds (64 / LPR row groups of RPT
// rows), capped at d_k.  The 8-bit format's BF16 head must be a multiple of
// it (and of 8) so that every wave's rows are of one kind: 32 at d_k = d_v =
// 128.
__host__ __device__ constexpr int q8_row_quantum(int dk, int dv) {
  const int lpr = dv / 8, nt = decode_threads_for(lpr, dk), rg = nt / lpr;
  const int rows = (64 / lpr) * ((dk + rg - 1) / rg);
  const int q = rows < dk ? rows : dk;
  return q < 8 ? 8 : q;
}

}  // namespace gdn
