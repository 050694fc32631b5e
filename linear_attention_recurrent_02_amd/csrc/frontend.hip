// frontend.hip -- the fused front-end of a GDN layer: per channel a causal
// depthwise conv of width 4 and SiLU; q and k then scaled to unit L2 norm per
// (token, head); gates g = -softplus(a_raw), beta = sigmoid(b_raw).
//
// The "Gated DeltaNet" glossary entry (Engineering details) lists fusing the
// short Conv1D with the layer among the optimisations; the width, SiLU and
// the q/k normalisation follow the prefill workload description.  Tap j
// multiplies x[t - 3 + j]; tokens before a sequence's first token count as 0.
//
// HBM-bound elementwise work: one workgroup per (64-token block, head job),
// where a head job is a q head, a k head or a v head.  A thread owns one
// token and a quarter of the head's channels (a run of d/4 consecutive
// channels, read and written as 16-byte vectors), so the L2 norm is a sum over
// 4 lanes (two xor shuffles).  The three previous tokens of the window are
// re-read from L1/L2; each raw byte comes from HBM once.
#include <math.h>

#include "device.h"
#include "internal.h"

namespace gdn {

struct FrontendParams {
  int32_t n_seq, H_qk, H_v;
  int64_t n_tokens;
  float eps;
  int32_t rule;
  const int32_t *cu;
  const void *q_raw, *k_raw, *v_raw;
  const float *wq, *wk, *wv, *a_raw, *b_raw;
  void *q_out, *k_out, *v_out;
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

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// conv + SiLU of NC consecutive channels of one head for token t (raw row
// stride ld elements, channel offset c0); w holds the NC channels' 4 taps
// (LDS, channel-major); seq_start is the first token of t's sequence.
template <bool AB, int NC>
__device__ __forceinline__ void conv_silu_run(const void *raw, int64_t ld, int64_t c0, int64_t t,
                                              int64_t seq_start, const float4 *w, float *y) {
#pragma unroll
  for (int c = 0; c < NC; ++c) y[c] = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t src = t - 3 + j;
    if (src < seq_start) continue;
    float x[NC];
    load_run<AB, NC>(raw, src * ld + c0, x);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float4 wc = w[c];
      const float wj = j == 0 ? wc.x : (j == 1 ? wc.y : (j == 2 ? wc.z : wc.w));
      y[c] = fmaf(wj, x[c], y[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) y[c] = silu(y[c]);
}

// LDS: the head's conv weights (d x 4 floats) and, for up to kFeCuLds
// sequences, the sequence offsets (binary search in LDS, not global memory)
constexpr int kFeCuLds = 2048;

template <bool AB, int DK, int DV>
__global__ __launch_bounds__(256) void frontend_kernel(FrontendParams p) {
  constexpr int DMAX = DK > DV ? DK : DV;
  __shared__ float4 w_lds[DMAX];
  __shared__ int32_t cu_lds[kFeCuLds + 1];
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * 64 + (tid >> 2);
  const int quarter = tid & 3;
  const int job = blockIdx.y;  // [0, H_qk): q head, [H_qk, 2 H_qk): k head, then v heads
  const bool is_qk = job < 2 * p.H_qk;
  const bool is_q = job < p.H_qk;
  const int D = is_qk ? DK : DV;
  const int hd = is_qk ? (is_q ? job : job - p.H_qk) : job - 2 * p.H_qk;
  const float *wsrc = (is_qk ? (is_q ? p.wq : p.wk) : p.wv) + (int64_t)hd * D * 4;
  for (int c = tid; c < D; c += 256) w_lds[c] = reinterpret_cast<const float4 *>(wsrc)[c];
  const bool cu_in_lds = p.n_seq <= kFeCuLds;
  if (cu_in_lds)
    for (int i = tid; i <= p.n_seq; i += 256) cu_lds[i] = p.cu[i];
  __syncthreads();
  const bool live = t < p.n_tokens;
  const int64_t tt = live ? t : p.n_tokens - 1;  // keep every lane in the shuffles
  const int32_t *cu = cu_in_lds ? cu_lds : p.cu;
  const int64_t s0 = cu[seq_of(cu, p.n_seq, tt)];
  if (is_qk) {
    constexpr int NC = DK / 4;
    const int64_t ld = (int64_t)p.H_qk * DK;
    const int64_t c0 = (int64_t)hd * DK + quarter * NC;
    float y[NC];
    conv_silu_run<AB, NC>(is_q ? p.q_raw : p.k_raw, ld, c0, tt, s0, w_lds + quarter * NC, y);
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) ss = fmaf(y[c], y[c], ss);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    const float inv = 1.0f / sqrtf(ss + p.eps);
#pragma unroll
    for (int c = 0; c < NC; ++c) y[c] *= inv;
    if (live) store_run<AB, NC>(is_q ? p.q_out : p.k_out, tt * ld + c0, y);
  } else {
    constexpr int NC = DV / 4;
    const int64_t ld = (int64_t)p.H_v * DV;
    const int64_t c0 = (int64_t)hd * DV + quarter * NC;
    float y[NC];
    conv_silu_run<AB, NC>(p.v_raw, ld, c0, tt, s0, w_lds + quarter * NC, y);
    if (live) {
      store_run<AB, NC>(p.v_out, tt * ld + c0, y);
      if (quarter == 0) {
        const int64_t gi = tt * p.H_v + hd;
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
}

FrontendParams make_frontend_params(const gdn_prefill_args &a, void *q_out, void *k_out,
                                    void *v_out, float *g_out, float *beta_out) {
  FrontendParams p;
  p.n_seq = a.n_seq; p.H_qk = a.H_qk; p.H_v = a.H_v; p.n_tokens = a.n_tokens;
  p.eps = a.eps; p.rule = a.rule; p.cu = a.cu_seqlens;
  p.q_raw = a.q; p.k_raw = a.k; p.v_raw = a.v;
  p.wq = a.conv_wq; p.wk = a.conv_wk; p.wv = a.conv_wv; p.a_raw = a.a_raw; p.b_raw = a.b_raw;
  p.q_out = q_out; p.k_out = k_out; p.v_out = v_out; p.g_out = g_out; p.beta_out = beta_out;
  return p;
}

template <bool AB, int DK>
static gdn_status fe_dv(const FrontendParams &p, int dv, hipStream_t s) {
  const dim3 grid((unsigned)((p.n_tokens + 63) / 64), (unsigned)(2 * p.H_qk + p.H_v));
  switch (dv) {
    case 16: hipLaunchKernelGGL((frontend_kernel<AB, DK, 16>), grid, dim3(256), 0, s, p); break;
    case 32: hipLaunchKernelGGL((frontend_kernel<AB, DK, 32>), grid, dim3(256), 0, s, p); break;
    case 64: hipLaunchKernelGGL((frontend_kernel<AB, DK, 64>), grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL((frontend_kernel<AB, DK, 128>), grid, dim3(256), 0, s, p); break;
    default: return GDN_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <bool AB>
static gdn_status fe_dk(const FrontendParams &p, int dk, int dv, hipStream_t s) {
  switch (dk) {
    case 16: return fe_dv<AB, 16>(p, dv, s);
    case 32: return fe_dv<AB, 32>(p, dv, s);
    case 64: return fe_dv<AB, 64>(p, dv, s);
    case 128: return fe_dv<AB, 128>(p, dv, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

gdn_status launch_frontend(const gdn_prefill_args &a, void *q_out, void *k_out, void *v_out,
                           float *g_out, float *beta_out, hipStream_t stream) {
  if (a.n_tokens == 0) return GDN_OK;
  const FrontendParams p = make_frontend_params(a, q_out, k_out, v_out, g_out, beta_out);
  return a.act_dtype == GDN_BF16 ? fe_dk<true>(p, a.d_k, a.d_v, stream)
                                 : fe_dk<false>(p, a.d_k, a.d_v, stream);
}

}  // namespace gdn
