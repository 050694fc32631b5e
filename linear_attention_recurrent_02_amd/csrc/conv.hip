// conv.hip -- the front-end's conv window across calls.
//
// The short conv is part of a GDN layer ("Gated DeltaNet" glossary,
// Engineering details), so a decode token's window holds the raw inputs of
// the three tokens before it.  Those live per request in a conv-state slot
// ([3, C] raw values, oldest first, C = 2*H_qk*d_k + H_v*d_v channels in
// q|k|v order) with the recurrent state's read/write slot rules ("Recurrent
// state" glossary, Why it matters: a checkpoint read slot may differ from the
// live write slot).
//
//  - conv_decode_kernel: one token per request -- window = slot history +
//    this token, conv + SiLU (+ L2 norm for q, k), gates, and the window slid
//    by one token into the write slot.  The arithmetic is frontend.cuh's, so
//    the outputs are bitwise those of the prefill front-end for the same
//    token and window.
//  - conv_store_kernel: the window a prefilled sequence leaves behind (its
//    last three raw inputs; before its first token, the rows of the window
//    it resumed, or zeros) into a slot, and for gdn_prefill also the window
//    at each intermediate checkpoint.
//
// HBM-bound and tiny next to the recurrent state (48 KiB of window per
// request against 1 MiB of state at 32 heads of 128 x 128 BF16): one thread
// per 16-byte piece of a row (8 BF16 or 4 FP32 channels), blockIdx.x = the
// group of requests, blockIdx.y = a 256-piece span of the row, so every load
// and store is contiguous across lanes.  A head's pieces are neighbouring lanes, so its
// L2 norm is frontend.cuh's DPP butterfly.
#include <algorithm>

#include "device.h"
#include "frontend.cuh"
#include "internal.h"

namespace gdn {

constexpr int kConvThreads = 256;
constexpr int kConvHist = 3;  // raw tokens a window keeps (conv width 4)

struct ConvParams {
  int32_t n;          // requests (decode) or sequences (store)
  int32_t H_v;
  int32_t pq, pv;     // 16-byte pieces per row of q (= of k) and of v
  int64_t n_slots;
  int64_t n_tokens;   // store: rows of the raw inputs
  float eps;
  const char *q, *k, *v;
  const float *wq, *wk, *wv;  // [channels, 4]
  const float *a_raw, *b_raw;
  char *pool;         // [n_slots, 3, C] in the input dtype
  const int32_t *read_slot, *write_slot, *cu;
  char *q_out, *k_out, *v_out;
  float *g_out, *beta_out;
  uint32_t *status;
  // store: a NULL write_slot means slot s (gdn_conv_store) or none (gdn_prefill)
  int32_t write_identity;
  // store from gdn_prefill: windows at intermediate checkpoints
  int32_t ckpt_per_seq, ckpt_interval;
  const int32_t *ckpt_slot;
};

// which of q, k, v a piece of the concatenated row belongs to, and where
struct PieceOf {
  int region;      // 0 q, 1 k, 2 v
  int local;       // piece index inside that tensor's row
  int64_t row_b;   // bytes per row of that tensor
};

__device__ __forceinline__ PieceOf piece_of(const ConvParams &p, int piece) {
  PieceOf r;
  if (piece < p.pq) { r.region = 0; r.local = piece; r.row_b = (int64_t)p.pq * 16; }
  else if (piece < 2 * p.pq) { r.region = 1; r.local = piece - p.pq; r.row_b = (int64_t)p.pq * 16; }
  else { r.region = 2; r.local = piece - 2 * p.pq; r.row_b = (int64_t)p.pv * 16; }
  return r;
}

// requests per workgroup of the decode step: each lane loads its conv taps
// once and keeps the loads of all RB requests in flight together (at B = 512,
// H_qk = 16, H_v = 32, d = 128: 21.1 us per launch with one request, 16.7 with
// two or four, 21.1 with eight, which leaves too few workgroups)
constexpr int kConvReqs = 2;

template <bool AB, int DK, int RB>
__global__ __launch_bounds__(kConvThreads) void conv_decode_kernel(ConvParams p) {
  using E = Elem<AB>;
  constexpr int CH = E::kPer16B;
  constexpr int PPH = DK / CH;  // pieces per q/k head: a power of two, at most 32
  const int P = 2 * p.pq + p.pv;
  const int r0 = blockIdx.x * RB;
  // per request: its slots, or skipped (past the batch end, or a slot out of range)
  int64_t rs[RB], ws[RB];
  bool live[RB];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int r = r0 + i;
    live[i] = r < p.n;
    rs[i] = ws[i] = -1;
    if (live[i]) {
      rs[i] = p.read_slot ? p.read_slot[r] : r;
      ws[i] = p.write_slot ? p.write_slot[r] : r;
      if (rs[i] < -1 || rs[i] >= p.n_slots || ws[i] < -1 || ws[i] >= p.n_slots) {
        live[i] = false;
        if (blockIdx.y == 0 && threadIdx.x == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
      }
    }
  }
  if (blockIdx.y == 0)
#pragma unroll
    for (int i = 0; i < RB; ++i)
      if (live[i])
        for (int h = threadIdx.x; h < p.H_v; h += kConvThreads) {
          const int64_t gi = (int64_t)(r0 + i) * p.H_v + h;
          p.g_out[gi] = gate_g(p.a_raw[gi]);
          p.beta_out[gi] = gate_beta(p.b_raw[gi]);
        }
  const int piece = blockIdx.y * kConvThreads + threadIdx.x;
  // pieces past the row end are whole heads of v or nothing (q and k end on a head boundary)
  if (piece >= P) return;
  const PieceOf at = piece_of(p, piece);
  const char *raw = at.region == 0 ? p.q : at.region == 1 ? p.k : p.v;
  const float *wt = at.region == 0 ? p.wq : at.region == 1 ? p.wk : p.wv;
  char *out = at.region == 0 ? p.q_out : at.region == 1 ? p.k_out : p.v_out;
  const int64_t slot_b = (int64_t)kConvHist * P * 16;

  // every load of the RB requests first: the raw piece and the window (h[.][0] = token t-3)
  uint4 x0[RB], h[RB][kConvHist];
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    x0[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kConvHist; ++j) h[i][j] = make_uint4(0, 0, 0, 0);
    if (live[i]) {
      x0[i] = nt_load16(raw + (int64_t)(r0 + i) * at.row_b + (int64_t)at.local * 16);
      if (rs[i] >= 0)
#pragma unroll
        for (int j = 0; j < kConvHist; ++j)
          h[i][j] = nt_load16(p.pool + rs[i] * slot_b + ((int64_t)j * P + piece) * 16);
    }
  }
  float4 w[CH];
  const float4 *wsrc = reinterpret_cast<const float4 *>(wt) + (int64_t)at.local * CH;
#pragma unroll
  for (int c = 0; c < CH; ++c) w[c] = wsrc[c];

#pragma unroll
  for (int i = 0; i < RB; ++i) {
    if (!live[i]) continue;
    float f0[CH], f1[CH], f2[CH], f3[CH], y[CH];
    E::unpack(x0[i], f0); E::unpack(h[i][2], f1); E::unpack(h[i][1], f2); E::unpack(h[i][0], f3);
#pragma unroll
    for (int c = 0; c < CH; ++c) y[c] = conv4_silu(w[c], f3[c], f2[c], f1[c], f0[c]);
    // a head's lanes are all q, all k or all v (regions start on head boundaries)
    if (at.region < 2) l2_scale<PPH>(y, p.eps);
    nt_store16(out + (int64_t)(r0 + i) * at.row_b + (int64_t)at.local * 16, E::pack(y));
    // slide the window into the write slot (raw values, copied bit for bit); a
    // slot read and written by the same request is safe: each lane reads its
    // own pieces before it stores them
    if (ws[i] >= 0) {
      char *dst = p.pool + ws[i] * slot_b + (int64_t)piece * 16;
      nt_store16(dst, h[i][1]);
      nt_store16(dst + (int64_t)P * 16, h[i][2]);
      nt_store16(dst + (int64_t)2 * P * 16, x0[i]);
    }
  }
}

__global__ __launch_bounds__(kConvThreads) void conv_store_kernel(ConvParams p) {
  const int s = blockIdx.x;
  const int P = 2 * p.pq + p.pv;
  const bool reporter = blockIdx.y == 0 && threadIdx.x == 0;  // reports a bad index once
  const int64_t t0 = p.cu[s], t1 = p.cu[s + 1];
  if (t0 < 0 || t1 < t0 || t1 > p.n_tokens) {
    if (reporter && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SEQ);
    return;
  }
  const int piece = blockIdx.y * kConvThreads + threadIdx.x;
  if (piece >= P) return;
  const PieceOf at = piece_of(p, piece);
  const char *raw = (at.region == 0 ? p.q : at.region == 1 ? p.k : p.v) + (int64_t)at.local * 16;
  const int64_t slot_b = (int64_t)kConvHist * P * 16;
  auto bad = [&](int64_t slot) { return slot < -1 || slot >= p.n_slots; };
  const int64_t rs = p.read_slot ? p.read_slot[s] : -1;
  if (bad(rs) && reporter && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
  const bool resumed = rs >= 0 && !bad(rs);
  // this piece of token t's raw input, t >= t0 - 3: the input row, or before
  // the first token the resumed window's row t - t0 + 3 (zeros without one)
  auto row = [&](int64_t t) {
    if (t >= t0) return nt_load16(raw + t * at.row_b);
    if (resumed)
      return *reinterpret_cast<const uint4 *>(p.pool + rs * slot_b + (t - t0 + kConvHist) * P * 16 +
                                              (int64_t)piece * 16);
    return make_uint4(0, 0, 0, 0);
  };
  // the window of the kConvHist tokens before token `end`, into `slot`; all
  // loads first, so a sequence may write the slot it read
  auto store_window = [&](int64_t end, int64_t slot) {
    uint4 x[kConvHist];
#pragma unroll
    for (int j = 0; j < kConvHist; ++j) x[j] = row(end - kConvHist + j);
    char *dst = p.pool + slot * slot_b + (int64_t)piece * 16;
#pragma unroll
    for (int j = 0; j < kConvHist; ++j) nt_store16(dst + (int64_t)j * P * 16, x[j]);
  };
  const int64_t ws = p.write_slot ? p.write_slot[s] : p.write_identity ? s : -1;
  if (bad(ws)) {
    if (reporter && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
  } else if (ws >= 0) {
    store_window(t1, ws);
  }
  if (p.ckpt_slot) {
    for (int j = 0; j < p.ckpt_per_seq; ++j) {
      const int64_t tc = t0 + (int64_t)(j + 1) * p.ckpt_interval;
      if (tc > t1) break;
      const int64_t cs = p.ckpt_slot[(int64_t)s * p.ckpt_per_seq + j];
      if (bad(cs)) {
        if (reporter && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
      } else if (cs >= 0) {
        store_window(tc, cs);
      }
    }
  }
}

static ConvParams make_conv_params(const gdn_conv_args &a) {
  const int per = a.act_dtype == GDN_BF16 ? 8 : 4;
  ConvParams p;
  p.n = a.B; p.H_v = a.H_v;
  p.pq = a.H_qk * a.d_k / per; p.pv = a.H_v * a.d_v / per;
  p.n_slots = a.n_slots; p.n_tokens = a.n_tokens; p.eps = a.eps;
  p.q = static_cast<const char *>(a.q); p.k = static_cast<const char *>(a.k);
  p.v = static_cast<const char *>(a.v);
  p.wq = a.conv_wq; p.wk = a.conv_wk; p.wv = a.conv_wv;
  p.a_raw = a.a_raw; p.b_raw = a.b_raw;
  p.pool = static_cast<char *>(a.conv_pool);
  p.read_slot = a.read_slot; p.write_slot = a.write_slot; p.cu = a.cu_seqlens;
  p.q_out = static_cast<char *>(a.q_out); p.k_out = static_cast<char *>(a.k_out);
  p.v_out = static_cast<char *>(a.v_out);
  p.g_out = a.g_out; p.beta_out = a.beta_out; p.status = a.status;
  p.write_identity = 1;
  p.ckpt_per_seq = 0; p.ckpt_interval = 0; p.ckpt_slot = nullptr;
  return p;
}

// the grid: one column per `per_col` requests / sequences, ceil(pieces / 256) rows
static dim3 conv_grid(const ConvParams &p, int per_col) {
  const int P = 2 * p.pq + p.pv;
  return dim3((unsigned)((p.n + per_col - 1) / per_col),
              (unsigned)((P + kConvThreads - 1) / kConvThreads));
}

int64_t conv_grid_rows(const gdn_conv_args &a) {
  const int per = a.act_dtype == GDN_BF16 ? 8 : 4;
  const int64_t P = (2 * (int64_t)a.H_qk * a.d_k + (int64_t)a.H_v * a.d_v) / per;
  return (P + kConvThreads - 1) / kConvThreads;
}

gdn_status launch_conv_decode(const gdn_conv_args &a, hipStream_t s) {
  const ConvParams p = make_conv_params(a);
  const dim3 grid = conv_grid(p, kConvReqs);
  const bool ab = a.act_dtype == GDN_BF16;
#define GDN_CONV_CASE(AB_, DK_) \
  hipLaunchKernelGGL((conv_decode_kernel<AB_, DK_, kConvReqs>), grid, dim3(kConvThreads), 0, s, p)
#define GDN_CONV_DK(AB_)                          \
  switch (a.d_k) {                                \
    case 16: GDN_CONV_CASE(AB_, 16); break;       \
    case 32: GDN_CONV_CASE(AB_, 32); break;       \
    case 64: GDN_CONV_CASE(AB_, 64); break;       \
    case 128: GDN_CONV_CASE(AB_, 128); break;     \
    default: return GDN_ERR_UNSUPPORTED;          \
  }
  if (ab) { GDN_CONV_DK(true) } else { GDN_CONV_DK(false) }
#undef GDN_CONV_DK
#undef GDN_CONV_CASE
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status launch_conv_store(const gdn_conv_args &a, hipStream_t s) {
  const ConvParams p = make_conv_params(a);
  hipLaunchKernelGGL(conv_store_kernel, conv_grid(p, 1), dim3(kConvThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// The windows a prefill leaves (conv_write_slot) and those at its
// intermediate checkpoints (conv_ckpt_slot), after its front-end has read
// the windows it resumes (stream order).
gdn_status launch_prefill_conv_store(const gdn_prefill_args &a, hipStream_t s) {
  const bool ckpt = a.conv_ckpt_slot && a.ckpt_interval > 0 && a.ckpt_per_seq > 0;
  if (a.n_seq == 0 || (!a.conv_write_slot && !ckpt)) return GDN_OK;
  const int per = a.act_dtype == GDN_BF16 ? 8 : 4;
  ConvParams p = {};
  p.n = a.n_seq; p.H_v = a.H_v;
  p.pq = a.H_qk * a.d_k / per; p.pv = a.H_v * a.d_v / per;
  p.n_slots = a.conv_n_slots; p.n_tokens = a.n_tokens;
  p.q = static_cast<const char *>(a.q); p.k = static_cast<const char *>(a.k);
  p.v = static_cast<const char *>(a.v);
  p.pool = static_cast<char *>(a.conv_pool);
  p.read_slot = a.conv_read_slot; p.write_slot = a.conv_write_slot; p.cu = a.cu_seqlens;
  p.status = a.status;
  p.write_identity = 0;
  p.ckpt_slot = ckpt ? a.conv_ckpt_slot : nullptr;
  p.ckpt_per_seq = ckpt ? a.ckpt_per_seq : 0;
  p.ckpt_interval = ckpt ? a.ckpt_interval : 0;
  hipLaunchKernelGGL(conv_store_kernel, conv_grid(p, 1), dim3(kConvThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace gdn
