// mixed.hip -- one launch for a decode batch and a prefill batch.
//
// Mixed batches are where the pages' GDN v3 kernels gained the most (2.14x
// on Ironwood; "Gated DeltaNet" glossary entry, How to read it).  Here the
// grid's first blocks are the prefill chains -- the long poles, one per
// (sequence, state head), dispatched first -- and the remaining blocks are
// persistent decode workers that stream the decode tiles in write-slot
// order on the CUs the chains leave free.  Each block runs exactly the device
// code of gdn_prefill or gdn_decode, so the results equal the two calls made
// separately.  Blocks have the chain's width (64 threads per chain wave); a
// decode block splits into 256-thread workers, the width of gdn_decode's
// tiles, each with its own reduction LDS.  A block holds the prefill chain's
// LDS, so one block fits per CU; each decode worker therefore keeps two tiles
// in flight (the next tile's loads are issued before the current tile is
// reduced and stored).  The workers of a block share its barriers: a tile's
// barriers are uniform within its worker, the workers exchange no data, and
// a barrier waits only for waves that have not ended, so they may meet at any
// of one another's barriers.
//
// Both halves must describe the same layer shape (heads, d_k, d_v, state and
// activation dtypes) and the same decay (one per head, or one per key
// channel: then the chains are gdn_prefill's channel-wise chain and the
// decode tiles its channel-wise decode).  With raw prefill inputs the
// front-end kernel runs first, then the single mixed launch.
#include <algorithm>

#include "decode.cuh"
#include "order.cuh"
#include "prefill_cw.cuh"
#include "prefill_pipe.cuh"

namespace gdn {

DecodeParams make_decode_params(const gdn_decode_args &a);

template <bool SB, bool AB, int DK, int DV, bool F32, bool CW>
struct MixedLayout {
  // the chain's waves, except with FP32 state: a worker's two FP32 tiles in
  // flight need more registers than a wave of a 512-thread block gets (the
  // channel-wise chain has its own wave count)
  static constexpr int NW = CW ? kCwWaves<DK, DV, F32> : SB ? kPrefillWaves<DK, DV, F32> : 4;
  static constexpr int NT = 64 * NW;                          // threads per block
  static constexpr int DT = 256;                              // threads per decode worker
  static constexpr int NH = NT / DT;                          // decode workers per block
  static_assert(NT % DT == 0, "whole decode workers per block");
  // with the chain's own wave count the block runs gdn_prefill's chain
  static constexpr bool OWN_CHAIN = !CW && NW == kPrefillWaves<DK, DV, F32>;
  static constexpr size_t PREFILL =
      CW ? kCwChainLds<DK, DV, F32, AB>
         : OWN_CHAIN ? kChainLds<DK, DV, F32, AB> : PrefillLayout<DK, DV, F32, AB>::BYTES;
  // one worker's reduction area, rounded to 16 bytes so every worker's is aligned alike
  static constexpr size_t RED = (sizeof(float) * DecodeShape<SB, DK, DV, DT>::LDS_FLOATS + 15) / 16 * 16;
  static constexpr size_t ORDER = slot_order_lds_bytes(kOrderMaxB, kOrderMaxSlots, NT);
  static constexpr size_t DECODE = NH * RED + ORDER;
  static constexpr size_t BYTES = PREFILL > DECODE ? PREFILL : DECODE;
};

template <bool SB, bool AB, int DK, int DV, bool F32, bool CW, bool CK>
__global__ __launch_bounds__((MixedLayout<SB, AB, DK, DV, F32, CW>::NT)) void mixed_kernel(
    DecodeParams dp, PrefillParams pp, int n_chains, int prefill_blocks, int ordered) {
  using L = MixedLayout<SB, AB, DK, DV, F32, CW>;
  constexpr int NT = L::NT, DT = L::DT;
  __shared__ __align__(16) char smem[L::BYTES];
  if ((int)blockIdx.x < prefill_blocks) {
    const int chain = chain_of_block(blockIdx.x);
    if (chain < n_chains) {
      if constexpr (CW) prefill_chain_cw<SB, AB, DK, DV, F32, CK>(pp, chain, smem);
      else if constexpr (L::OWN_CHAIN) run_chain<SB, AB, DK, DV, F32, CK>(pp, chain, smem);
      else prefill_chain<SB, AB, DK, DV, F32, L::NW, CK>(pp, chain, smem);
    }
    return;
  }
  // decode workers: DT-thread parts of the block
  const int part = (int)threadIdx.x / DT;  // uniform in a wave
  const int tid = (int)threadIdx.x % DT;   // the thread within its worker
  float *red = reinterpret_cast<float *>(smem + part * L::RED);
  int *order = reinterpret_cast<int *>(smem + L::NH * L::RED);
  if (ordered) build_slot_order<NT>(dp.write_slot, dp.B, dp.n_slots, order);
  const int64_t n_tiles = (int64_t)dp.B * dp.H_v;
  const int64_t workers = ((int64_t)gridDim.x - prefill_blocks) * L::NH;
  int64_t t = ((int64_t)blockIdx.x - prefill_blocks) * L::NH + part;
  if (t >= n_tiles) return;
  using Regs = DecodeTileRegs<SB, AB, DK, DV, DT, CW>;
  auto load = [&](int64_t tile, Regs &dst) {
    const int pos = (int)(tile / dp.H_v);
    decode_tile_load<SB, AB, DK, DV, DT, CW>(dp, ordered ? order[pos] : pos,
                                             (int)(tile % dp.H_v), dst, tid);
  };
  Regs cur, nxt;
  load(t, cur);
  for (;;) {
    const int64_t tn = t + workers;
    const bool more = tn < n_tiles;
    if (more) load(tn, nxt);
    decode_tile_finish<SB, AB, DK, DV, DT, CW>(dp, cur, red, tid);
    if (!more) break;
    cur = nxt;
    t = tn;
  }
}

template <bool SB, bool AB, int DK, int DV, bool CW>
static gdn_status launch_mixed_t(const DecodeParams &dp, const PrefillParams &pp, hipStream_t s) {
  constexpr bool F32 = !AB || !SB;  // the prefill chain's arithmetic, as in gdn_prefill
  using L = MixedLayout<SB, AB, DK, DV, F32, CW>;
  if constexpr (L::BYTES > 160 * 1024) {
    return GDN_ERR_UNSUPPORTED;
  } else {
    const int n_chains = pp.n_seq * pp.H_v;
    const int prefill_blocks = (n_chains + 15) / 16 * 16;
    const int64_t tiles = (int64_t)dp.B * dp.H_v;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return GDN_ERR_LAUNCH;
    // decode workers on the CUs the chains leave free (at least a quarter of the chip)
    const int64_t free_cus = std::max<int64_t>(cus - n_chains, std::max(1, cus / 4));
    const int64_t workers = tiles > 0 ? std::min<int64_t>((tiles + L::NH - 1) / L::NH, free_cus) : 0;
    const int ordered =
        dp.write_slot != nullptr && dp.B <= kOrderMaxB && dp.n_slots <= kOrderMaxSlots ? 1 : 0;
    const int64_t grid = (n_chains > 0 ? prefill_blocks : 0) + workers;
    if (grid == 0) return GDN_OK;
    // the instance with intermediate checkpoints only when they are asked for
    if (pp.ckpt_chunks > 0)
      hipLaunchKernelGGL((mixed_kernel<SB, AB, DK, DV, F32, CW, true>), dim3((unsigned)grid),
                         dim3(L::NT), 0, s, dp, pp, n_chains,
                         n_chains > 0 ? prefill_blocks : 0, ordered);
    else
      hipLaunchKernelGGL((mixed_kernel<SB, AB, DK, DV, F32, CW, false>), dim3((unsigned)grid),
                         dim3(L::NT), 0, s, dp, pp, n_chains,
                         n_chains > 0 ? prefill_blocks : 0, ordered);
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
  }
}

template <bool SB, bool AB, int DK, int DV>
static gdn_status mixed_cw(const DecodeParams &dp, const PrefillParams &pp, bool cw,
                           hipStream_t s) {
  return cw ? launch_mixed_t<SB, AB, DK, DV, true>(dp, pp, s)
            : launch_mixed_t<SB, AB, DK, DV, false>(dp, pp, s);
}

template <bool SB, bool AB, int DK>
static gdn_status mixed_dv(const DecodeParams &dp, const PrefillParams &pp, int dv, bool cw,
                           hipStream_t s) {
  switch (dv) {
    case 16: return mixed_cw<SB, AB, DK, 16>(dp, pp, cw, s);
    case 32: return mixed_cw<SB, AB, DK, 32>(dp, pp, cw, s);
    case 64: return mixed_cw<SB, AB, DK, 64>(dp, pp, cw, s);
    case 128: return mixed_cw<SB, AB, DK, 128>(dp, pp, cw, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

template <bool SB, bool AB>
static gdn_status mixed_dk(const DecodeParams &dp, const PrefillParams &pp, int dk, int dv,
                           bool cw, hipStream_t s) {
  switch (dk) {
    case 16: return mixed_dv<SB, AB, 16>(dp, pp, dv, cw, s);
    case 32: return mixed_dv<SB, AB, 32>(dp, pp, dv, cw, s);
    case 64: return mixed_dv<SB, AB, 64>(dp, pp, dv, cw, s);
    case 128: return mixed_dv<SB, AB, 128>(dp, pp, dv, cw, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

gdn_status launch_mixed(const gdn_decode_args &d, const gdn_prefill_args &p, hipStream_t stream) {
  if (d.B > 0 && p.n_seq > 0 &&
      (d.H_qk != p.H_qk || d.H_v != p.H_v || d.d_k != p.d_k || d.d_v != p.d_v ||
       d.state_dtype != p.state_dtype || d.act_dtype != p.act_dtype ||
       d.decay_mode != p.decay_mode))
    return GDN_ERR_UNSUPPORTED;
  // shapes come from whichever half is present
  const gdn_prefill_args &shape = p;
  const int dk = d.B > 0 ? d.d_k : shape.d_k, dv = d.B > 0 ? d.d_v : shape.d_v;
  const int sdt = d.B > 0 ? d.state_dtype : shape.state_dtype;
  const int adt = d.B > 0 ? d.act_dtype : shape.act_dtype;
  const bool cw = (d.B > 0 ? d.decay_mode : shape.decay_mode) == GDN_DECAY_CHANNEL;
  PrefillParams pp = {};
  if (p.n_seq > 0) {
    const gdn_status st = prepare_prefill(p, stream, &pp);
    if (st != GDN_OK) return st;
  }
  const DecodeParams dp = d.B > 0 ? make_decode_params(d) : DecodeParams{};
  const bool sb = sdt == GDN_BF16, ab = adt == GDN_BF16;
  if (sb && ab) return mixed_dk<true, true>(dp, pp, dk, dv, cw, stream);
  if (sb && !ab) return mixed_dk<true, false>(dp, pp, dk, dv, cw, stream);
  if (!sb && ab) return mixed_dk<false, true>(dp, pp, dk, dv, cw, stream);
  return mixed_dk<false, false>(dp, pp, dk, dv, cw, stream);
}

}  // namespace gdn
