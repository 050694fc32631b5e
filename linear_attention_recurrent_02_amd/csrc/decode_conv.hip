// decode_conv.hip -- one decode token with the layer's short conv fused into
// the state update: the Conv1D and the recurrence in one kernel, as the
// "Gated DeltaNet" glossary entry (Engineering details) does for decode.
//
// A work unit is one request and one q/k head.  The `group` state heads of
// that q/k head share its q and k, so one workgroup runs the conv for the
// unit once and then the group's decode tiles, two at a time: the workgroup
// is two decode-tile workers side by side (two 256-thread tiles at d = 128),
// so a unit of the workloads' group of two runs both its tiles at once and
// the units in flight cover the same requests and heads as the decode
// kernel's tiles (one workgroup per unit running the tiles one after the
// other measured 225 against 192 us per B = 512 launch).  Per unit:
//  1. the stage threads, one per 16-byte piece of the unit's q, k and v rows
//     (2 d_k / CH + group d_v / CH of them), issue the loads of the raw
//     piece, its three window rows and its taps; the first `group` threads
//     also load a_raw and b_raw;
//  2. each worker issues its first tile's state loads, so they are in
//     flight while the stage computes;
//  3. the stage computes conv + SiLU (+ the L2 norm of q and k per head,
//     by DPP across the head's lanes) with frontend.cuh's arithmetic, rounds
//     to the activation dtype into LDS, and slides its pieces of the window
//     into the conv write slot; each piece is read and written by the same
//     thread, so a slot updated in place is safe;
//  4. one barrier; then each worker's tile takes q, k, v, g, beta from LDS
//     and runs decode_tile_finish (a group of more than two takes rounds).
// The per-channel arithmetic and the rounding point are those of
// gdn_conv_decode, and the tile is gdn_decode's, so results are bitwise those
// of the two calls in sequence.  What the fusion saves is the round trip of
// q, k, v, g, beta through HBM (32 KiB per request at 16 q/k and 32 state
// heads of 128 in BF16) and one launch per layer.
//
// Units are walked in ascending write-slot order of their requests, as the
// decode kernel walks tiles (order.cuh).  The grid is a multiple of H_qk, so
// a workgroup always serves the same q/k head: its taps (q and k of that
// head, v of its state heads) are staged in LDS once, and each stage thread
// reads its own when it computes rather than holding them in registers while
// the state tile's loads are in flight.
#include <algorithm>

#include "decode.cuh"
#include "frontend.cuh"
#include "order.cuh"

namespace gdn {

extern __shared__ __align__(16) int order_lds[];  // the slot order, then the taps (dynamic LDS)

DecodeParams make_decode_params(const gdn_decode_args &a);  // decode.hip

struct DecodeConvParams {
  const char *xq, *xk, *xv;   // raw [B, H_qk d_k], [B, H_qk d_k], [B, H_v d_v]
  const float *wq, *wk, *wv;  // taps [channels, 4]
  const float *a_raw, *b_raw; // [B, H_v]
  char *pool;                 // conv pool [n_slots, 3, C]
  int64_t n_slots;
  const int32_t *read_slot, *write_slot;
  float eps;
  int64_t taps_off;           // byte offset of the taps in dynamic LDS (after the slot order)
};

constexpr int kFusedMaxGroup = 8;  // state heads per q/k head
constexpr int kFusedWorkers = 2;   // decode tiles a workgroup runs side by side
constexpr int kWindow = 3;         // raw tokens a window keeps (conv width 4)

// The state a fresh request (read slot -1) starts from: a zero tile of the
// largest size (128 x 128 FP32), read in place of a slot so that the state
// loads never sit in a branch (a branch around them made the compiler wait
// for their data where the two paths join).
static __device__ __align__(256) uint4 kZeroTile[128 * 128 * 4 / 16];

// The token's inputs of a tile from LDS, for the fused conv step (per-head
// decay, BF16 or FP32 state), once the conv stage has written them there in
// the activation dtype (q, k: the tile's q/k head; v: its state head) with
// the head's g and beta.  The values are those decode_tile_load would read
// from gdn_conv_decode's outputs; the state loads are the caller's.
template <bool SB, bool AB, int DK, int DV, int NT>
__device__ __forceinline__ void decode_tile_inputs_local(
    const DecodeParams &p, DecodeTileRegs<SB, AB, DK, DV, NT> &t,
    const typename Elem<AB>::T *q, const typename Elem<AB>::T *k, const typename Elem<AB>::T *v,
    float g, float beta, int tid) {
  using S = DecodeShape<SB, DK, DV, NT>;
  constexpr int VEC = S::VEC, LPR = S::LPR, RPT = S::RPT;
  using Regs = DecodeTileRegs<SB, AB, DK, DV, NT>;
  if (!t.valid) return;
  const int cv = tid % LPR;
  const int row0 = (tid / LPR) * RPT;
  if constexpr (Regs::PACKED) {
    const uint4 *kp = reinterpret_cast<const uint4 *>(k + row0);
    const uint4 *qp = reinterpret_cast<const uint4 *>(q + row0);
    const uint4 *vp = reinterpret_cast<const uint4 *>(v + cv * VEC);
#pragma unroll
    for (int j = 0; j < Regs::KN; ++j) { t.kp[j] = kp[j]; t.qp[j] = qp[j]; }
#pragma unroll
    for (int j = 0; j < Regs::VN; ++j) t.vp[j] = vp[j];
  } else {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const bool ok = row0 + i < DK;
      t.kr[i] = ok ? Elem<AB>::load1(k, row0 + i) : 0.f;
      t.qr[i] = ok ? Elem<AB>::load1(q, row0 + i) : 0.f;
    }
    load_run<AB, VEC>(v, cv * VEC, t.vv);
  }
  const bool decay = (p.rule & kRuleDecay) != 0;
  const bool erase = (p.rule & kRuleErase) != 0;
  t.a = decay ? expf(g) : 1.0f;
  t.bw = erase ? beta : 1.0f;
}

// The state loads of one tile from resolved, in-range slots.
template <bool SB, int DK, int DV, int NT, class Regs>
__device__ __forceinline__ void fused_tile_state(const DecodeParams &p, int64_t r, int h,
                                                 int64_t rs, int64_t ws, Regs &t, int tid) {
  using S = DecodeShape<SB, DK, DV, NT>;
  constexpr int LPR = S::LPR, RPT = S::RPT;
  using ST = typename Elem<SB>::T;
  const int cv = tid % LPR;
  const int row0 = (tid / LPR) * RPT;
  t.r = r;
  t.h = h;
  t.ws = ws;
  t.valid = true;
  const uint4 *src = rs >= 0 ? reinterpret_cast<const uint4 *>(static_cast<const ST *>(p.pool) +
                                                              (rs * p.H_v + h) * (int64_t)DK * DV)
                             : kZeroTile;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    if (S::ALL_LIVE || row0 + i < DK) t.m[i] = stream_load(src + (int64_t)(row0 + i) * LPR + cv);
    else t.m[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}

template <bool SB, bool AB, int DK, int DV>
__device__ __forceinline__ void decode_conv_body(const DecodeParams &p, const DecodeConvParams &c,
                                                 int ordered) {
  constexpr int NT = decode_threads<SB, DK, DV>();
  using S = DecodeShape<SB, DK, DV, NT>;
  using E = Elem<AB>;
  using AT = typename E::T;
  using Regs = DecodeTileRegs<SB, AB, DK, DV, NT>;
  constexpr int WT = kFusedWorkers * NT;      // threads of the workgroup
  constexpr int CH = E::kPer16B;              // channels per 16-byte piece
  constexpr int PQ = DK / CH, PV = DV / CH;   // pieces per q/k head, per v head
  __shared__ float red[kFusedWorkers][S::LDS_FLOATS];  // one reduction area per worker
  __shared__ uint4 st_qk[2 * PQ];             // q, then k, of the unit's q/k head
  __shared__ uint4 st_v[kFusedMaxGroup * PV]; // v of its state heads
  __shared__ float st_g[kFusedMaxGroup], st_b[kFusedMaxGroup];
  const int wtid = (int)threadIdx.x;          // thread in the workgroup (the stage's index)
  const int worker = wtid / NT;               // uniform in a wave
  const int tid = wtid % NT;                  // thread in its worker's tile
  const int G = p.group;
  const int NS = 2 * PQ + G * PV;  // stage threads (host-checked: at most WT)
  // this workgroup's taps, one float4 per channel: q, k of head hq, then v of
  // its G state heads (channel tid CH + cc is stage thread tid's tap cc)
  const int hq = (int)(blockIdx.x % (unsigned)p.H_qk);
  float4 *const taps = reinterpret_cast<float4 *>(order_lds) + c.taps_off / 16;
  for (int e = wtid; e < NS * CH; e += WT) {
    const float4 *src = e < DK ? reinterpret_cast<const float4 *>(c.wq) + (int64_t)hq * DK + e
                      : e < 2 * DK ? reinterpret_cast<const float4 *>(c.wk) + (int64_t)hq * DK + (e - DK)
                      : reinterpret_cast<const float4 *>(c.wv) + (int64_t)hq * G * DV + (e - 2 * DK);
    taps[e] = *src;
  }
  if (ordered) build_slot_order<WT>(p.write_slot, p.B, p.n_slots, order_lds);  // ends with a barrier
  else __syncthreads();
  const int64_t P = (2 * (int64_t)p.H_qk * DK + (int64_t)p.H_v * DV) / CH;  // pieces per row
  const int64_t slot_b = (int64_t)kWindow * P * 16;
  // this thread's stage piece: q, k or v of state head hq G + vj; piece li of its head
  const bool stager = wtid < NS;
  const int region = wtid < PQ ? 0 : wtid < 2 * PQ ? 1 : 2;
  const int vj = region == 2 ? (wtid - 2 * PQ) / PV : 0;
  const int li = region == 0 ? wtid : region == 1 ? wtid - PQ : (wtid - 2 * PQ) % PV;
  const int64_t qk_row_b = (int64_t)p.H_qk * DK * sizeof(AT), v_row_b = (int64_t)p.H_v * DV * sizeof(AT);
  // the piece's index in a window row
  const int64_t wpiece = region == 0   ? (int64_t)hq * PQ + li
                         : region == 1 ? (int64_t)p.H_qk * PQ + (int64_t)hq * PQ + li
                                       : 2 * (int64_t)p.H_qk * PQ + ((int64_t)hq * G + vj) * PV + li;
  const AT *const q_lds = reinterpret_cast<const AT *>(st_qk);
  const AT *const k_lds = reinterpret_cast<const AT *>(st_qk + PQ);
  const AT *const v_lds = reinterpret_cast<const AT *>(st_v);

  const int64_t n_units = (int64_t)p.B * p.H_qk;
  for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {
    const int pos = (int)(u / p.H_qk);  // u % H_qk == hq: the grid is a multiple of H_qk
    const int64_t r = ordered ? order_lds[pos] : pos;
    // the four slot indices, loaded together and compared as loaded
    int32_t rs32 = (int32_t)r, ws32 = rs32, crs32 = rs32, cws32 = rs32;
    if (p.read_slot) rs32 = p.read_slot[r];
    if (p.write_slot) ws32 = p.write_slot[r];
    if (c.read_slot) crs32 = c.read_slot[r];
    if (c.write_slot) cws32 = c.write_slot[r];
    const int64_t rs = rs32, ws = ws32, crs = crs32, cws = cws32;
    // any slot out of range skips the whole unit: no o, state or window
    if (rs < -1 || rs >= p.n_slots || ws < -1 || ws >= p.n_slots || crs < -1 ||
        crs >= c.n_slots || cws < -1 || cws >= c.n_slots) {
      if (wtid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
      continue;
    }

    // 1. the stage's loads: raw piece, window rows (h[0] = token t-3), gates
    uint4 x0 = make_uint4(0u, 0u, 0u, 0u);
    uint4 hw[kWindow];
#pragma unroll
    for (int j = 0; j < kWindow; ++j) hw[j] = make_uint4(0u, 0u, 0u, 0u);
    float ar = 0.f, br = 0.f;
    if (stager) {
      const char *raw;
      int64_t ch0;  // first channel of the piece in its tensor
      if (region == 0) {
        raw = c.xq + r * qk_row_b; ch0 = (int64_t)hq * DK + li * CH;
      } else if (region == 1) {
        raw = c.xk + r * qk_row_b; ch0 = (int64_t)hq * DK + li * CH;
      } else {
        raw = c.xv + r * v_row_b; ch0 = ((int64_t)hq * G + vj) * DV + li * CH;
      }
      x0 = nt_load16(raw + ch0 * (int64_t)sizeof(AT));
      if (crs >= 0) {
#pragma unroll
        for (int j = 0; j < kWindow; ++j)
          hw[j] = nt_load16(c.pool + crs * slot_b + ((int64_t)j * P + wpiece) * 16);
      }
      if (wtid < G) {
        const int64_t gi = r * p.H_v + (int64_t)hq * G + wtid;
        ar = c.a_raw[gi];
        br = c.b_raw[gi];
      }
    }

    // 2. each worker's first tile's state loads, in flight while the stage
    // computes (zero-initialised: nothing of the previous unit's tile stays live)
    Regs t{};
    if (worker < G) fused_tile_state<SB, DK, DV, NT>(p, r, hq * G + worker, rs, ws, t, tid);

    // 3. the stage: conv + SiLU (+ L2 norm), rounded into LDS; the window slid
    if (stager) {
      float f0[CH], f1[CH], f2[CH], f3[CH], y[CH];
      E::unpack(x0, f0); E::unpack(hw[2], f1); E::unpack(hw[1], f2); E::unpack(hw[0], f3);
#pragma unroll
      for (int cc = 0; cc < CH; ++cc)
        y[cc] = conv4_silu(taps[wtid * CH + cc], f3[cc], f2[cc], f1[cc], f0[cc]);
      // q's lanes and k's lanes are aligned groups of PQ lanes in wave 0
      if (region < 2) l2_scale<PQ>(y, c.eps);
      const uint4 packed = E::pack(y);
      if (region < 2) st_qk[wtid] = packed;
      else st_v[wtid - 2 * PQ] = packed;
      if (cws >= 0) {
        char *dst = c.pool + cws * slot_b + wpiece * 16;
        nt_store16(dst, hw[1]);
        nt_store16(dst + P * 16, hw[2]);
        nt_store16(dst + 2 * P * 16, x0);
      }
      if (wtid < G) {
        st_g[wtid] = gate_g(ar);
        st_b[wtid] = gate_beta(br);
      }
    }
    __syncthreads();

    // 4. the group's tiles, one per worker per round; the workers meet the
    // same barriers (three per tile, none for a one-wave tile), a worker
    // without a tile in the last round of an odd group meets them alone, and
    // the last barrier of each round lets the next unit's stage overwrite LDS
    for (int j0 = 0; j0 < G; j0 += kFusedWorkers) {
      const int j = j0 + worker;
      if (j < G) {
        if (j0 > 0) fused_tile_state<SB, DK, DV, NT>(p, r, hq * G + j, rs, ws, t, tid);
        decode_tile_inputs_local<SB, AB, DK, DV, NT>(p, t, q_lds, k_lds, v_lds + j * DV, st_g[j],
                                                     st_b[j], tid);
        decode_tile_finish<SB, AB, DK, DV, NT>(p, t, red[worker], tid);
      } else if constexpr (S::NW > 1) {
        __syncthreads();
        __syncthreads();
        __syncthreads();
      }
    }
    // one-wave tiles have no barrier of their own: the workers' LDS reads of
    // this unit's inputs end before the next unit's stage writes them
    if constexpr (S::NW == 1) __syncthreads();
  }
}

template <bool SB, bool AB, int DK, int DV>
__global__ __launch_bounds__(kFusedWorkers * kDecodeMaxThreads) void decode_conv_kernel(
    DecodeParams p, DecodeConvParams c, int ordered) {
  decode_conv_body<SB, AB, DK, DV>(p, c, ordered);
}

// BF16 state and activations at four waves per SIMD, the decode kernel's
// occupancy (two workgroups of eight waves per CU): unbounded, d = 128 takes
// 139 registers, and bounded to 128 it spills ten.  The launcher takes this
// instance when a CU must hold more than one workgroup, the unbounded one
// otherwise (measured over 48 layers at d = 128: B = 16, 0.58 ms unbounded
// against 0.69 bounded; B = 64, 1.76 against 1.64; B = 512, 12.1 against
// 10.9).
template <int DK, int DV>
__global__ __launch_bounds__(kFusedWorkers * kDecodeMaxThreads)
__attribute__((amdgpu_waves_per_eu(4))) void decode_conv_bf16_kernel(DecodeParams p,
                                                                      DecodeConvParams c,
                                                                      int ordered) {
  decode_conv_body<true, true, DK, DV>(p, c, ordered);
}

// Stage threads a shape needs: one per 16-byte piece of q, k and the group's v.
int decode_conv_stage_threads(int d_k, int d_v, int group, bool act_bf16) {
  const int ch = act_bf16 ? 8 : 4;
  return 2 * d_k / ch + group * d_v / ch;
}

int decode_conv_max_group() { return kFusedMaxGroup; }

// Threads of the fused kernel's workgroup: kFusedWorkers decode tiles.
int decode_conv_block_threads(int d_k, int d_v, bool state_bf16) {
  return kFusedWorkers * decode_threads_for(d_v / (state_bf16 ? 8 : 4), d_k);
}

template <bool SB, bool AB, int DK, int DV>
static gdn_status launch_t(const DecodeParams &p, const DecodeConvParams &c, hipStream_t s) {
  constexpr int WT = kFusedWorkers * decode_threads<SB, DK, DV>();
  constexpr int CH = Elem<AB>::kPer16B;
  const int64_t units = (int64_t)p.B * p.H_qk;
  const int ordered =
      p.write_slot != nullptr && p.B <= kOrderMaxB && p.n_slots <= kOrderMaxSlots ? 1 : 0;
  DecodeConvParams cp = c;
  cp.taps_off = ordered ? (int64_t)((slot_order_lds_bytes(p.B, p.n_slots, WT) + 15) / 16 * 16) : 0;
  const size_t lds = (size_t)cp.taps_off +
                     (size_t)decode_conv_stage_threads(DK, DV, p.group, AB) * CH * sizeof(float4);
  auto kern = decode_conv_kernel<SB, AB, DK, DV>;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return GDN_ERR_LAUNCH;
  if constexpr (SB && AB) {
    if (units > (int64_t)cus) kern = decode_conv_bf16_kernel<DK, DV>;
  }
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WT, lds) != hipSuccess)
    return GDN_ERR_LAUNCH;
  // one resident wave of workgroups, rounded down to a multiple of H_qk (each
  // workgroup keeps one q/k head's taps); all units when there are fewer
  const int64_t resident = (int64_t)std::max(1, cus) * std::max(1, per_cu);
  const int64_t grid = units <= resident ? units : std::max<int64_t>(p.H_qk, resident / p.H_qk * p.H_qk);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WT), lds, s, p, cp, ordered);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <bool SB, bool AB, int DK>
static gdn_status launch_dv(const DecodeParams &p, const DecodeConvParams &c, int dv,
                            hipStream_t s) {
  switch (dv) {
    case 16: return launch_t<SB, AB, DK, 16>(p, c, s);
    case 32: return launch_t<SB, AB, DK, 32>(p, c, s);
    case 64: return launch_t<SB, AB, DK, 64>(p, c, s);
    case 128: return launch_t<SB, AB, DK, 128>(p, c, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

template <bool SB, bool AB>
static gdn_status launch_dk(const DecodeParams &p, const DecodeConvParams &c, int dk, int dv,
                            hipStream_t s) {
  switch (dk) {
    case 16: return launch_dv<SB, AB, 16>(p, c, dv, s);
    case 32: return launch_dv<SB, AB, 32>(p, c, dv, s);
    case 64: return launch_dv<SB, AB, 64>(p, c, dv, s);
    case 128: return launch_dv<SB, AB, 128>(p, c, dv, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

gdn_status launch_decode_conv(const gdn_decode_args &d, const gdn_conv_args &a, hipStream_t s) {
  const DecodeParams p = make_decode_params(d);
  DecodeConvParams c;
  c.xq = static_cast<const char *>(a.q);
  c.xk = static_cast<const char *>(a.k);
  c.xv = static_cast<const char *>(a.v);
  c.wq = a.conv_wq; c.wk = a.conv_wk; c.wv = a.conv_wv;
  c.a_raw = a.a_raw; c.b_raw = a.b_raw;
  c.pool = static_cast<char *>(a.conv_pool);
  c.n_slots = a.n_slots;
  c.read_slot = a.read_slot; c.write_slot = a.write_slot;
  c.eps = a.eps;
  const bool sb = d.state_dtype == GDN_BF16, ab = d.act_dtype == GDN_BF16;
  if (sb && ab) return launch_dk<true, true>(p, c, d.d_k, d.d_v, s);
  if (sb && !ab) return launch_dk<true, false>(p, c, d.d_k, d.d_v, s);
  if (!sb && ab) return launch_dk<false, true>(p, c, d.d_k, d.d_v, s);
  return launch_dk<false, false>(p, c, d.d_k, d.d_v, s);
}

}  // namespace gdn
