// frontend.hip -- the fused front-end of a GDN layer: per channel a causal
// depthwise conv of width 4 and SiLU; q and k then scaled to unit L2 norm per
// (token, head); gates g = -softplus(a_raw), beta = sigmoid(b_raw).
//
// The "Gated DeltaNet" glossary entry (Engineering details) lists fusing the
// short Conv1D with the layer among the optimisations; the width, SiLU and
// the q/k normalisation follow the prefill workload description.  Tap j
// multiplies x[t - 3 + j]; tokens before a sequence's first token are the
// rows of the conv window it resumes (a conv-state slot: the raw inputs of
// the three tokens before it), or 0 without one.
//
// HBM-bound elementwise work, laid out so that every raw byte is read once
// and every load and store is a whole-row stream.  A thread owns one 16-byte
// piece of a row (8 BF16 or 4 FP32 channels) and walks a contiguous range of
// 64-token runs, keeping the three previous tokens of its channels in
// registers, so the conv window costs no re-reads beyond a 3-token halo per
// range.  The ranges are balanced across the grid.  The threads of a workgroup cover a
// contiguous span of a row (q, k or v; several row groups per workgroup when
// the row is shorter than 256 pieces), so each token's loads and stores are
// contiguous across lanes.  A head's pieces sit in neighbouring lanes of one
// wave, so its L2 norm is a butterfly of xor shuffles.  Each thread keeps the
// loads of its next 8 tokens in flight while it computes.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "device.h"
#include "frontend.cuh"
#include "internal.h"

namespace gdn {

constexpr int kFeThreads = 256;
constexpr int kFeRun = 64;    // tokens per run (one 64-bit mask of sequence starts)
constexpr int kFeCuLds = 4096;  // sequence offsets kept in LDS (more: read from global memory)
constexpr int kFeDepth = 8;   // tokens loaded ahead per thread
// workgroups per CU the grid aims at: more than are resident at once, so at
// the workloads' sizes each takes a single 64-token run (measured 2-6% faster
// than three resident workgroups per CU walking longer ranges)
constexpr int kFeBlocksPerCU = 12;
static_assert(kFeRun <= 64, "sequence starts in a run are a 64-bit mask");
static_assert(kFeRun % kFeDepth == 0, "a whole run is a whole number of ring turns");
static_assert(kFeDepth % 4 == 0, "the conv window ring has four token slots");

// One of the three tensors of the front-end, split into chunks of `lpr`
// 16-byte pieces (a power of two; a chunk holds whole heads).
struct FeTensor {
  const void *raw;
  void *out;
  const float *w;    // [H * D, 4] conv taps
  int32_t H;         // heads
  int32_t pieces;    // 16-byte pieces per row = H * D / channels-per-piece
  int32_t lpr_log2;  // log2 of the lanes per row group
  int32_t chunks;    // ceil(pieces / lanes per row group)
  int32_t win_off;   // first piece of this tensor in a conv-window row (q|k|v order)
};

struct FrontendParams {
  int32_t n_seq, H_v;
  int64_t n_tokens;
  float eps;
  const int32_t *cu;
  FeTensor t[3];      // q, k, v
  int32_t y0[4];      // first blockIdx.y of q, k, v; y0[3] = total
  int32_t x_blocks[3];  // blockIdx.x extent of each tensor (row groups differ)
  int32_t runs_per[3];  // 64-token runs per row group
  const float *a_raw, *b_raw;
  float *g_out, *beta_out;
  // the conv windows the sequences resume: [win_slots, 3, win_pieces] 16-byte
  // pieces, win_read[s] the slot of sequence s (NULL: none)
  const char *win;
  int64_t win_slots;
  const int32_t *win_read;
  int32_t win_pieces;
  uint32_t *status;
};

// index of the sequence holding token t: the last s with cu[s] <= t
__device__ __forceinline__ int seq_of(const int32_t *cu, int n_seq, int64_t t) {
  int lo = 0, hi = n_seq - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Returns v unchanged, but only after the CH values in x exist: an empty asm
// that claims to read x and rewrite v, so nothing computed from v (a load
// address) can be scheduled before x.
template <int CH>
__device__ __forceinline__ int64_t ordered_after(float (&x)[CH], int64_t v) {
#pragma unroll
  for (int c = 0; c < CH; ++c) asm volatile("" : "+v"(x[c]), "+v"(v));
  return v;
}

template <bool AB, int D, bool NORM, bool GATES>
__device__ __forceinline__ void fe_run(const FrontendParams &p, const FeTensor &T, int chunk,
                                       int runs_per, const int32_t *cu) {
  using E = Elem<AB>;
  constexpr int CH = E::kPer16B;  // channels per piece
  constexpr int PPH = D / CH;     // pieces per head (power of two, at most 32)
  const int lpr = 1 << T.lpr_log2;
  const int lane = threadIdx.x & (lpr - 1);
  const int R = kFeThreads >> T.lpr_log2;  // row groups per workgroup
  const int rg = threadIdx.x >> T.lpr_log2;
  const int piece = chunk * lpr + lane;
  // whole heads are active or not: lpr and pieces are multiples of PPH
  if (piece >= T.pieces) return;
  const int64_t ts = ((int64_t)blockIdx.x * R + rg) * runs_per * kFeRun;
  const int64_t te = min(ts + (int64_t)runs_per * kFeRun, p.n_tokens);
  if (ts >= te) return;

  const int64_t row_bytes = (int64_t)T.pieces * 16;
  const char *src = static_cast<const char *>(T.raw) + (int64_t)piece * 16;
  char *dst = static_cast<char *>(T.out) + (int64_t)piece * 16;
  // every raw byte is read once and every output byte written once: stream them
  auto ld = [&](int64_t t) { return nt_load16(src + t * row_bytes); };

  // first the loads that do not depend on the sequence bounds: the ring of
  // the next kFeDepth tokens, the three tokens before ts and the conv taps
  const int64_t tl = te - 1;
  uint4 ring[kFeDepth];
#pragma unroll
  for (int u = 0; u < kFeDepth; ++u) ring[u] = ld(min(ts + u, tl));
  uint4 h1 = make_uint4(0, 0, 0, 0), h2 = h1, h3 = h1;
  if (ts >= 1) h1 = ld(ts - 1);
  if (ts >= 2) h2 = ld(ts - 2);
  if (ts >= 3) h3 = ld(ts - 3);
  float4 w[CH];
  const float4 *wsrc = reinterpret_cast<const float4 *>(T.w) + (int64_t)piece * CH;
#pragma unroll
  for (int c = 0; c < CH; ++c) w[c] = wsrc[c];

  // the sequence holding ts, and the offsets of the sequences that follow
  int s = seq_of(cu, p.n_seq, ts);
  const int64_t s_start = cu[s];
  // this piece of the raw input of token t, t before the first token `start`
  // of sequence sq (t >= start - 3): row t - start + 3 of the window the
  // sequence resumes, or 0
  auto before = [&](int sq, int64_t start, int64_t t) {
    uint4 x = make_uint4(0, 0, 0, 0);
    if (p.win_read) {
      const int64_t slot = p.win_read[sq];
      if (slot >= 0 && slot < p.win_slots)
        x = *reinterpret_cast<const uint4 *>(
            p.win + ((slot * 3 + (t - start + 3)) * p.win_pieces + T.win_off + piece) * 16);
      else if (slot != -1 && p.status)
        atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
    }
    return x;
  };
  // bit i of the mask is set when token r0 + i opens a sequence (equals an
  // offset cu[j], j >= 1): the conv window is cleared there
  auto starts_mask = [&](int64_t r0, int64_t r1) {
    while (s + 1 < p.n_seq && cu[s + 1] < r0) ++s;  // a start at r0 itself stays ahead
    uint64_t m = 0;
    for (int j = s + 1; j < p.n_seq; ++j) {
      const int64_t c = cu[j];
      if (c >= r1) break;
      if (c >= r0) m |= 1ull << (c - r0);  // (offsets below r0 only if they decrease)
    }
    return m;
  };

  // The conv window is a ring of four token slots: token ts + j lives in slot
  // j % 4 (runs and the unrolled steps are multiples of 4 tokens, so every
  // slot index is a constant and the window slides without register copies).
  // Slots 3, 2, 1 start as tokens ts - 1, ts - 2, ts - 3 (before the
  // sequence: its resumed window, or 0).
  float xw[4][CH];
  if (ts - 1 < s_start) h1 = before(s, s_start, ts - 1);
  if (ts - 2 < s_start) h2 = before(s, s_start, ts - 2);
  if (ts - 3 < s_start) h3 = before(s, s_start, ts - 3);
  E::unpack(h1, xw[3]); E::unpack(h2, xw[2]); E::unpack(h3, xw[1]);

  // one token t, slot u % 4: conv + SiLU (+ L2 norm) of x0 given the window;
  // `check` = the run holds a sequence start (bit i of resets: token t opens
  // a sequence, whose window replaces the previous tokens)
  auto step = [&](const float (&x0)[CH], bool check, uint64_t resets, int i, int u, int64_t t,
                  float (&y)[CH]) {
    float(&x1)[CH] = xw[(u + 3) & 3];
    float(&x2)[CH] = xw[(u + 2) & 3];
    float(&x3)[CH] = xw[(u + 1) & 3];
    if (check && ((resets >> i) & 1ull)) {
      const int sq = seq_of(cu, p.n_seq, t);
      E::unpack(before(sq, t, t - 1), x1);
      E::unpack(before(sq, t, t - 2), x2);
      E::unpack(before(sq, t, t - 3), x3);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      y[c] = conv4_silu(w[c], x3[c], x2[c], x1[c], x0[c]);
      xw[u & 3][c] = x0[c];
    }
    if constexpr (NORM) l2_scale<PPH>(y, p.eps);
  };

  // whole runs: token t comes from ring slot (t - ts) % kFeDepth, which is
  // then refilled with token t + kFeDepth (clamped to the range, so every step
  // issues one load and one store and the waits stay kFeDepth deep)
  // (runs without a sequence start -- nearly all -- skip the per-token check)
  auto whole_run = [&](int64_t r0, uint64_t resets, auto check_tag) {
    constexpr bool check = decltype(check_tag)::value;
#pragma unroll 1
    for (int b0 = 0; b0 < kFeRun; b0 += kFeDepth) {
#pragma unroll
      for (int u = 0; u < kFeDepth; ++u) {
        const int64_t t = r0 + b0 + u;
        float x0[CH], y[CH];
        E::unpack(ring[u], x0);
        // refill the slot only after it has been unpacked, so the load can
        // land in the slot's own registers (no copies, no early waits)
        ring[u] = ld(ordered_after(x0, min(t + kFeDepth, tl)));
        step(x0, check, resets, b0 + u, u, t, y);
        nt_store16(dst + t * row_bytes, E::pack(y));
      }
    }
  };
  int64_t r0 = ts;
  for (; r0 + kFeRun <= te; r0 += kFeRun) {
    const uint64_t resets = starts_mask(r0, r0 + kFeRun);
    if (resets == 0) whole_run(r0, resets, std::false_type{});
    else whole_run(r0, resets, std::true_type{});
  }
  if (r0 < te) {
    // the ragged last run of the tensor: the same steps, stores guarded
    const uint64_t resets = starts_mask(r0, te);
#pragma unroll 1
    for (int b0 = 0; b0 < kFeRun; b0 += kFeDepth) {
#pragma unroll
      for (int u = 0; u < kFeDepth; ++u) {
        const int64_t t = r0 + b0 + u;
        float x0[CH], y[CH];
        E::unpack(ring[u], x0);
        ring[u] = ld(min(t + kFeDepth, tl));
        step(x0, true, resets, b0 + u, u, t, y);
        if (t < te) nt_store16(dst + t * row_bytes, E::pack(y));
      }
    }
  }

  if constexpr (GATES) {
    // the gates of this run's tokens for the heads of this chunk, one
    // (token, head) per lane step, heads fastest (contiguous in a_raw/b_raw)
    const int h0 = chunk * (lpr / PPH);
    const int nh = min(lpr / PPH, p.H_v - h0);
    const int64_t n = (te - ts) * nh;
    for (int64_t i = lane; i < n; i += lpr) {
      const int64_t gi = (ts + i / nh) * p.H_v + h0 + (int)(i % nh);
      p.g_out[gi] = p.a_raw ? gate_g(p.a_raw[gi]) : 0.f;
      p.beta_out[gi] = p.b_raw ? gate_beta(p.b_raw[gi]) : 1.0f;
    }
  }
}

template <bool AB, int DK, int DV>
__global__ __launch_bounds__(kFeThreads) void frontend_kernel(FrontendParams p) {
  __shared__ int32_t cu_lds[kFeCuLds + 1];
  const bool in_lds = p.n_seq <= kFeCuLds;
  if (in_lds)
    for (int i = threadIdx.x; i <= p.n_seq; i += kFeThreads) cu_lds[i] = p.cu[i];
  __syncthreads();
  const int32_t *cu = in_lds ? cu_lds : p.cu;
  const int y = blockIdx.y;
  if (y < p.y0[1]) {
    if ((int)blockIdx.x < p.x_blocks[0])
      fe_run<AB, DK, true, false>(p, p.t[0], y - p.y0[0], p.runs_per[0], cu);
  } else if (y < p.y0[2]) {
    if ((int)blockIdx.x < p.x_blocks[1])
      fe_run<AB, DK, true, false>(p, p.t[1], y - p.y0[1], p.runs_per[1], cu);
  } else {
    if ((int)blockIdx.x < p.x_blocks[2])
      fe_run<AB, DV, false, true>(p, p.t[2], y - p.y0[2], p.runs_per[2], cu);
  }
}

static int ilog2_ceil(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

static FeTensor make_tensor(const void *raw, void *out, const float *w, int H, int d, bool ab) {
  FeTensor T;
  T.raw = raw; T.out = out; T.w = w; T.H = H;
  T.pieces = H * d / (ab ? 8 : 4);
  T.lpr_log2 = ilog2_ceil(T.pieces);
  if (T.lpr_log2 > 8) T.lpr_log2 = 8;  // 256 lanes
  const int lpr = 1 << T.lpr_log2;
  T.chunks = (T.pieces + lpr - 1) / lpr;
  return T;
}

gdn_status launch_frontend(const gdn_prefill_args &a, void *q_out, void *k_out, void *v_out,
                           float *g_out, float *beta_out, hipStream_t stream) {
  if (a.n_tokens == 0) return GDN_OK;
  const bool ab = a.act_dtype == GDN_BF16;
  FrontendParams p;
  p.n_seq = a.n_seq; p.H_v = a.H_v; p.n_tokens = a.n_tokens; p.eps = a.eps; p.cu = a.cu_seqlens;
  p.t[0] = make_tensor(a.q, q_out, a.conv_wq, a.H_qk, a.d_k, ab);
  p.t[1] = make_tensor(a.k, k_out, a.conv_wk, a.H_qk, a.d_k, ab);
  p.t[2] = make_tensor(a.v, v_out, a.conv_wv, a.H_v, a.d_v, ab);
  p.a_raw = a.a_raw; p.b_raw = a.b_raw; p.g_out = g_out; p.beta_out = beta_out;
  p.t[0].win_off = 0;
  p.t[1].win_off = p.t[0].pieces;
  p.t[2].win_off = 2 * p.t[0].pieces;
  p.win = static_cast<const char *>(a.conv_pool);
  p.win_slots = a.conv_n_slots;
  p.win_read = a.conv_pool ? a.conv_read_slot : nullptr;
  p.win_pieces = 2 * p.t[0].pieces + p.t[2].pieces;
  p.status = a.status;
  p.y0[0] = 0;
  for (int i = 0; i < 3; ++i) p.y0[i + 1] = p.y0[i] + p.t[i].chunks;
  // about kFeBlocksPerCU workgroups per CU in all, the runs of a tensor dealt
  // out as equal contiguous ranges
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return GDN_ERR_LAUNCH;
  const int64_t runs = (a.n_tokens + kFeRun - 1) / kFeRun;
  const int64_t x_target = std::max<int64_t>(1, (int64_t)cus * kFeBlocksPerCU / p.y0[3]);
  int xmax = 0;
  for (int i = 0; i < 3; ++i) {
    const int64_t R = kFeThreads >> p.t[i].lpr_log2;  // row groups per workgroup
    const int64_t ranges = std::max<int64_t>(1, std::min<int64_t>(runs, x_target * R));
    p.runs_per[i] = (int)((runs + ranges - 1) / ranges);
    const int64_t tokens_per_block = R * p.runs_per[i] * kFeRun;
    p.x_blocks[i] = (int)((a.n_tokens + tokens_per_block - 1) / tokens_per_block);
    xmax = p.x_blocks[i] > xmax ? p.x_blocks[i] : xmax;
  }
  const dim3 grid((unsigned)xmax, (unsigned)p.y0[3]);
  const dim3 block(kFeThreads);
#define GDN_FE_CASE(AB_, DK_, DV_) \
  hipLaunchKernelGGL((frontend_kernel<AB_, DK_, DV_>), grid, block, 0, stream, p)
#define GDN_FE_DV(AB_, DK_)                                \
  switch (a.d_v) {                                         \
    case 16: GDN_FE_CASE(AB_, DK_, 16); break;             \
    case 32: GDN_FE_CASE(AB_, DK_, 32); break;             \
    case 64: GDN_FE_CASE(AB_, DK_, 64); break;             \
    case 128: GDN_FE_CASE(AB_, DK_, 128); break;           \
    default: return GDN_ERR_UNSUPPORTED;                   \
  }
#define GDN_FE_DK(AB_)                                     \
  switch (a.d_k) {                                         \
    case 16: GDN_FE_DV(AB_, 16); break;                    \
    case 32: GDN_FE_DV(AB_, 32); break;                    \
    case 64: GDN_FE_DV(AB_, 64); break;                    \
    case 128: GDN_FE_DV(AB_, 128); break;                  \
    default: return GDN_ERR_UNSUPPORTED;                   \
  }
  if (ab) { GDN_FE_DK(true) } else { GDN_FE_DK(false) }
#undef GDN_FE_DK
#undef GDN_FE_DV
#undef GDN_FE_CASE
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace gdn
