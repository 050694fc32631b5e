// frontend.hip -- the fused front-end of a GDN layer: per channel a causal
// depthwise conv of width 4 and SiLU; q and k then scaled to unit L2 norm per
// (token, head); gates g = -softplus(a_raw), beta = sigmoid(b_raw).
//
// The "Gated DeltaNet" glossary entry (Engineering details) lists fusing the
// short Conv1D with the layer among the optimisations; the width, SiLU and
// the q/k normalisation follow the prefill workload description.  Tap j
// multiplies x[t - 3 + j]; tokens before a sequence's first token count as 0.
//
// HBM-bound elementwise work, laid out so that every raw byte is read once
// and every load and store is a whole-row stream.  A thread owns one 16-byte
// piece of a row (8 BF16 or 4 FP32 channels) and walks a run of consecutive
// tokens, keeping the three previous tokens of its channels in registers, so
// the conv window costs no re-reads.  The threads of a workgroup cover a
// contiguous span of a row (q, k or v; several row groups per workgroup when
// the row is shorter than 256 pieces), so each token's loads and stores are
// contiguous across lanes.  A head's pieces sit in neighbouring lanes of one
// wave, so its L2 norm is a butterfly of xor shuffles.  Each thread keeps the
// loads of its next 8 tokens in flight while it computes.
#include <math.h>

#include "device.h"
#include "internal.h"

namespace gdn {

constexpr int kFeThreads = 256;
constexpr int kFeRun = 64;    // consecutive tokens per row group
constexpr int kFeDepth = 8;   // tokens loaded ahead per thread
static_assert(kFeRun <= 64, "sequence starts in a run are a 64-bit mask");
static_assert(kFeRun % kFeDepth == 0, "a whole run is a whole number of ring turns");

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
};

struct FrontendParams {
  int32_t n_seq, H_v;
  int64_t n_tokens;
  float eps;
  const int32_t *cu;
  FeTensor t[3];      // q, k, v
  int32_t y0[4];      // first blockIdx.y of q, k, v; y0[3] = total
  int32_t x_blocks[3];  // blockIdx.x extent of each tensor (row groups differ)
  const float *a_raw, *b_raw;
  float *g_out, *beta_out;
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

// SiLU with the hardware exp and reciprocal: x * 1 / (1 + e^-x)
__device__ __forceinline__ float silu_fast(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

template <bool AB, int D, bool NORM, bool GATES>
__device__ __forceinline__ void fe_run(const FrontendParams &p, const FeTensor &T, int chunk) {
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
  const int64_t ts = ((int64_t)blockIdx.x * R + rg) * kFeRun;
  const int64_t te = min(ts + (int64_t)kFeRun, p.n_tokens);
  if (ts >= te) return;

  const int64_t row_bytes = (int64_t)T.pieces * 16;
  const char *src = static_cast<const char *>(T.raw) + (int64_t)piece * 16;
  char *dst = static_cast<char *>(T.out) + (int64_t)piece * 16;
  auto ld = [&](int64_t t) { return *reinterpret_cast<const uint4 *>(src + t * row_bytes); };

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

  // bit i of `resets` is set when token ts + i opens a sequence (it equals a
  // sequence offset cu[j], j >= 1); the conv window is cleared there
  const int s = seq_of(p.cu, p.n_seq, ts);
  const int64_t s_start = p.cu[s];
  uint64_t resets = 0;
  for (int j = s + 1; j < p.n_seq; ++j) {
    const int64_t c = p.cu[j];
    if (c >= te) break;
    if (c >= ts) resets |= 1ull << (c - ts);  // (offsets below ts only if they decrease)
  }

  // x1, x2, x3 = the previous three tokens of this piece (0 before the sequence)
  float x1[CH], x2[CH], x3[CH];
  if (ts - 1 < s_start) h1 = make_uint4(0, 0, 0, 0);
  if (ts - 2 < s_start) h2 = make_uint4(0, 0, 0, 0);
  if (ts - 3 < s_start) h3 = make_uint4(0, 0, 0, 0);
  E::unpack(h1, x1); E::unpack(h2, x2); E::unpack(h3, x3);

  // one token: conv + SiLU (+ L2 norm) of x0 given the window, then slide it
  auto step = [&](const float (&x0)[CH], int64_t t, float (&y)[CH]) {
    if ((resets >> (t - ts)) & 1ull) {
#pragma unroll
      for (int c = 0; c < CH; ++c) { x1[c] = 0.f; x2[c] = 0.f; x3[c] = 0.f; }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float acc = fmaf(w[c].x, x3[c], fmaf(w[c].y, x2[c], fmaf(w[c].z, x1[c], w[c].w * x0[c])));
      y[c] = silu_fast(acc);
      x3[c] = x2[c]; x2[c] = x1[c]; x1[c] = x0[c];
    }
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < CH; ++c) ss = fmaf(y[c], y[c], ss);
#pragma unroll
      for (int off = 1; off < PPH; off <<= 1) ss += __shfl_xor(ss, off);
      const float inv = 1.0f / sqrtf(ss + p.eps);
#pragma unroll
      for (int c = 0; c < CH; ++c) y[c] *= inv;
    }
  };

  if (te - ts == kFeRun) {
    // a whole run: token t comes from ring slot (t - ts) % kFeDepth, which is
    // then refilled with token t + kFeDepth (clamped to the run, so every step
    // issues one load and one store and the waits stay kFeDepth deep)
    for (int64_t b0 = ts; b0 < te; b0 += kFeDepth) {
#pragma unroll
      for (int u = 0; u < kFeDepth; ++u) {
        const int64_t t = b0 + u;
        float x0[CH], y[CH];
        E::unpack(ring[u], x0);
        // refill the slot only after it has been unpacked, so the load can
        // land in the slot's own registers (no copies, no early waits)
        ring[u] = ld(ordered_after(x0, min(t + kFeDepth, tl)));
        step(x0, t, y);
        *reinterpret_cast<uint4 *>(dst + t * row_bytes) = E::pack(y);
      }
    }
  } else {
    // the ragged last run of the tensor: plain loads, one token at a time
    for (int64_t t = ts; t < te; ++t) {
      float x0[CH], y[CH];
      E::unpack(ld(t), x0);
      step(x0, t, y);
      *reinterpret_cast<uint4 *>(dst + t * row_bytes) = E::pack(y);
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
      // g = -softplus(a) computed as -(max(a,0) + log1p(exp(-|a|))); beta = sigmoid(b)
      if (p.a_raw) {
        const float a = p.a_raw[gi];
        p.g_out[gi] = -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a))));
      } else {
        p.g_out[gi] = 0.f;
      }
      p.beta_out[gi] = p.b_raw ? 1.0f / (1.0f + expf(-p.b_raw[gi])) : 1.0f;
    }
  }
}

template <bool AB, int DK, int DV>
__global__ __launch_bounds__(kFeThreads) void frontend_kernel(FrontendParams p) {
  const int y = blockIdx.y;
  if (y < p.y0[1]) {
    if ((int)blockIdx.x < p.x_blocks[0]) fe_run<AB, DK, true, false>(p, p.t[0], y - p.y0[0]);
  } else if (y < p.y0[2]) {
    if ((int)blockIdx.x < p.x_blocks[1]) fe_run<AB, DK, true, false>(p, p.t[1], y - p.y0[1]);
  } else {
    if ((int)blockIdx.x < p.x_blocks[2]) fe_run<AB, DV, false, true>(p, p.t[2], y - p.y0[2]);
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
  int xmax = 0;
  p.y0[0] = 0;
  for (int i = 0; i < 3; ++i) {
    const int64_t tokens_per_block = (int64_t)(kFeThreads >> p.t[i].lpr_log2) * kFeRun;
    p.x_blocks[i] = (int)((a.n_tokens + tokens_per_block - 1) / tokens_per_block);
    xmax = p.x_blocks[i] > xmax ? p.x_blocks[i] : xmax;
    p.y0[i + 1] = p.y0[i] + p.t[i].chunks;
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
