// prefill.hip -- the chunked-prefill kernel (one workgroup per (sequence,
// state head) chain, the chain itself in prefill_pipe.cuh or
// prefill_chain.cuh) and the
// gdn_prefill launcher: the front-end kernel into the workspace when the
// inputs are raw, then the chains.
#include <algorithm>

#include "prefill_cw.cuh"
#include "prefill_pipe.cuh"

namespace gdn {

template <bool SB, bool AB, int DK, int DV, bool F32, bool CK>
__global__ __launch_bounds__((64 * kPrefillWaves<DK, DV, F32>)) void prefill_kernel(PrefillParams p,
                                                                                   int n_chains) {
  __shared__ __align__(16) char smem[kChainLds<DK, DV, F32, AB>];
  const int chain = chain_of_block(blockIdx.x);
  if (chain < n_chains) run_chain<SB, AB, DK, DV, F32, CK>(p, chain, smem);
}

// one (sequence, state head) chain per workgroup with a per-key-channel decay
template <bool SB, bool AB, int DK, int DV, bool F32, bool CK>
__global__ __launch_bounds__((64 * kCwWaves<DK, DV, F32>)) void prefill_cw_kernel(PrefillParams p,
                                                                                 int n_chains) {
  __shared__ __align__(16) char smem[kCwChainLds<DK, DV, F32, AB>];
  const int chain = chain_of_block(blockIdx.x);
  if (chain < n_chains) prefill_chain_cw<SB, AB, DK, DV, F32, CK>(p, chain, smem);
}

// ---- launcher --------------------------------------------------------------

PrefillParams make_prefill_params(const gdn_prefill_args &a, const void *q, const void *k,
                                  const void *v, const float *g, const float *beta) {
  PrefillParams p;
  p.n_seq = a.n_seq; p.H_qk = a.H_qk; p.H_v = a.H_v; p.group = a.H_v / a.H_qk;
  p.n_tokens = a.n_tokens; p.n_slots = a.n_slots; p.scale = a.scale; p.rule = a.rule; p.cu = a.cu_seqlens;
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
  p.pool = a.state_pool; p.read_slot = a.read_slot; p.write_slot = a.write_slot;
  p.o = a.o; p.status = a.status;
  p.ckpt_chunks = a.ckpt_interval > 0 ? a.ckpt_interval / a.chunk : 0;
  p.ckpt_per_seq = a.ckpt_per_seq;
  p.ckpt_slot = a.ckpt_slot;
  p.channel_decay = a.decay_mode == GDN_DECAY_CHANNEL ? 1 : 0;
  return p;
}

template <bool SB, bool AB, int DK, int DV>
static gdn_status launch_chains(const PrefillParams &p, hipStream_t s) {
  // FP32 arithmetic (FP32 MFMA operands) for an FP32 state or FP32
  // activations; BF16 MFMA operands only when both are BF16
  constexpr bool F32 = !AB || !SB;
  if (p.channel_decay) {
    if constexpr (kCwChainLds<DK, DV, F32, AB> > 160 * 1024) {
      return GDN_ERR_UNSUPPORTED;  // FP32 operands of the channel-wise chain at d_k = 128
    } else {
      const int n_chains = p.n_seq * p.H_v;
      const int blocks = (n_chains + 15) / 16 * 16;
      const dim3 block(64 * kCwWaves<DK, DV, F32>);
      if (p.ckpt_chunks > 0)
        hipLaunchKernelGGL((prefill_cw_kernel<SB, AB, DK, DV, F32, true>), dim3(blocks), block, 0,
                           s, p, n_chains);
      else
        hipLaunchKernelGGL((prefill_cw_kernel<SB, AB, DK, DV, F32, false>), dim3(blocks), block, 0,
                           s, p, n_chains);
      return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
    }
  }
  if constexpr (kChainLds<DK, DV, F32, AB> > 160 * 1024) {
    return GDN_ERR_UNSUPPORTED;  // FP32 activation tiles at d = 128 do not fit in LDS
  } else {
    const int n_chains = p.n_seq * p.H_v;
    const int blocks = (n_chains + 15) / 16 * 16;
    // the instance with intermediate checkpoints only when they are asked for
    if (p.ckpt_chunks > 0)
      hipLaunchKernelGGL((prefill_kernel<SB, AB, DK, DV, F32, true>), dim3(blocks),
                         dim3(64 * kPrefillWaves<DK, DV, F32>), 0, s, p, n_chains);
    else
      hipLaunchKernelGGL((prefill_kernel<SB, AB, DK, DV, F32, false>), dim3(blocks),
                         dim3(64 * kPrefillWaves<DK, DV, F32>), 0, s, p, n_chains);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
  }
}

template <bool SB, bool AB, int DK>
static gdn_status chains_dv(const PrefillParams &p, int dv, hipStream_t s) {
  switch (dv) {
    case 16: return launch_chains<SB, AB, DK, 16>(p, s);
    case 32: return launch_chains<SB, AB, DK, 32>(p, s);
    case 64: return launch_chains<SB, AB, DK, 64>(p, s);
    case 128: return launch_chains<SB, AB, DK, 128>(p, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

template <bool SB, bool AB>
static gdn_status chains_dk(const PrefillParams &p, int dk, int dv, hipStream_t s) {
  switch (dk) {
    case 16: return chains_dv<SB, AB, 16>(p, dv, s);
    case 32: return chains_dv<SB, AB, 32>(p, dv, s);
    case 64: return chains_dv<SB, AB, 64>(p, dv, s);
    case 128: return chains_dv<SB, AB, 128>(p, dv, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

// workspace: front-end outputs q, k, v (act dtype) and g, beta (FP32), each
// segment 256-byte aligned
struct FeWorkspace {
  size_t q, k, v, g, beta, bytes;
};
static FeWorkspace fe_workspace(const gdn_prefill_args &a) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t es = a.act_dtype == GDN_BF16 ? 2 : 4;
  const size_t N = (size_t)std::max<int64_t>(0, a.n_tokens);
  FeWorkspace w;
  w.q = 0;
  w.k = up(w.q + N * a.H_qk * a.d_k * es);
  w.v = up(w.k + N * a.H_qk * a.d_k * es);
  w.g = up(w.v + N * a.H_v * a.d_v * es);
  w.beta = up(w.g + N * a.H_v * 4);
  w.bytes = up(w.beta + N * a.H_v * 4);
  return w;
}

size_t prefill_workspace_bytes(const gdn_prefill_args &a) {
  if (!a.use_frontend || a.n_tokens <= 0 || a.H_qk <= 0 || a.H_v <= 0 || a.d_k <= 0 || a.d_v <= 0)
    return 0;
  return fe_workspace(a).bytes;
}

gdn_status prepare_prefill(const gdn_prefill_args &a, hipStream_t stream, PrefillParams *out) {
  const void *q = a.q, *k = a.k, *v = a.v;
  const float *g = a.g, *beta = a.beta;
  if (a.use_frontend && a.n_tokens > 0) {
    const FeWorkspace w = fe_workspace(a);
    char *base = static_cast<char *>(a.workspace);
    const gdn_status st = launch_frontend(a, base + w.q, base + w.k, base + w.v,
                                          reinterpret_cast<float *>(base + w.g),
                                          reinterpret_cast<float *>(base + w.beta), stream);
    if (st != GDN_OK) return st;
    q = base + w.q; k = base + w.k; v = base + w.v;
    g = reinterpret_cast<const float *>(base + w.g);
    beta = reinterpret_cast<const float *>(base + w.beta);
  }
  if (a.use_frontend) {
    // the conv windows the sequences leave, once the front-end has read the
    // ones they resume (an empty sequence leaves the window it resumed)
    const gdn_status st = launch_prefill_conv_store(a, stream);
    if (st != GDN_OK) return st;
  }
  *out = make_prefill_params(a, q, k, v, g, beta);
  return GDN_OK;
}

gdn_status launch_prefill(const gdn_prefill_args &a, hipStream_t stream) {
  PrefillParams p;
  const gdn_status st = prepare_prefill(a, stream, &p);
  if (st != GDN_OK) return st;
  const bool sb = a.state_dtype == GDN_BF16, ab = a.act_dtype == GDN_BF16;
  if (sb && ab) return chains_dk<true, true>(p, a.d_k, a.d_v, stream);
  if (sb && !ab) return chains_dk<true, false>(p, a.d_k, a.d_v, stream);
  if (!sb && ab) return chains_dk<false, true>(p, a.d_k, a.d_v, stream);
  return chains_dk<false, false>(p, a.d_k, a.d_v, stream);
}

}  // namespace gdn
