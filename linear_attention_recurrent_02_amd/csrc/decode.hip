// decode.hip -- the decode kernel: a persistent grid of workgroups that walk
// the (request, state head) tiles of a batch in write-slot order; the tile
// body is decode_tile() in decode.cuh (shared with the mixed launcher) and
// the order comes from build_slot_order() in order.cuh.
#include "decode.cuh"
#include "order.cuh"

#include <algorithm>

namespace gdn {


template <bool SB, bool AB, int DK, int DV, bool CW>
__global__ __launch_bounds__(GDN_DECODE_MAX_THREADS) void decode_kernel(DecodeParams p,
                                                                         int ordered) {
  constexpr int NT = decode_threads<SB, DK, DV>();
  __shared__ float red[DecodeShape<SB, DK, DV, NT>::LDS_FLOATS];
  extern __shared__ int order_lds[];
  if (ordered) build_slot_order<NT>(p.write_slot, p.B, p.n_slots, order_lds);
  const int64_t n_tiles = (int64_t)p.B * p.H_v;
  // software pipeline: the next tile's loads are issued before this tile's
  // reduction and store, so each workgroup keeps loads in flight throughout
  using Regs = DecodeTileRegs<SB, AB, DK, DV, NT, CW>;
  int64_t t = blockIdx.x;
  if (t >= n_tiles) return;
  auto load = [&](int64_t tile, Regs &dst) {
    const int pos = (int)(tile / p.H_v);
    decode_tile_load<SB, AB, DK, DV, NT, CW>(p, ordered ? order_lds[pos] : pos,
                                             (int)(tile % p.H_v), dst, (int)threadIdx.x);
  };
#if GDN_DECODE_PIPELINE
  Regs cur, nxt;
  load(t, cur);
  for (;;) {
    const int64_t tn = t + gridDim.x;
    const bool more = tn < n_tiles;
    if (more) load(tn, nxt);
    decode_tile_finish<SB, AB, DK, DV, NT, CW>(p, cur, red, (int)threadIdx.x);
    if (!more) break;
    cur = nxt;
    t = tn;
  }
#else
  for (; t < n_tiles; t += gridDim.x) {
    Regs cur;
    load(t, cur);
    decode_tile_finish<SB, AB, DK, DV, NT, CW>(p, cur, red, (int)threadIdx.x);
  }
#endif
}

DecodeParams make_decode_params(const gdn_decode_args &a) {
  DecodeParams p;
  p.B = a.B; p.H_qk = a.H_qk; p.H_v = a.H_v; p.group = a.H_v / a.H_qk;
  p.n_slots = a.n_slots; p.scale = a.scale; p.rule = a.rule;
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta;
  p.pool = a.state_pool; p.read_slot = a.read_slot; p.write_slot = a.write_slot;
  p.o = a.o; p.status = a.status;
  return p;
}

template <bool SB, bool AB, int DK, int DV, bool CW>
static gdn_status launch_t(const DecodeParams &p, hipStream_t s) {
  constexpr int NT = decode_threads<SB, DK, DV>();
  const int64_t tiles = (int64_t)p.B * p.H_v;
  const int ordered =
      p.write_slot != nullptr && p.B <= kOrderMaxB && p.n_slots <= kOrderMaxSlots ? 1 : 0;
  const size_t lds = ordered ? slot_order_lds_bytes(p.B, p.n_slots, NT) : 0;
  auto kern = decode_kernel<SB, AB, DK, DV, CW>;
  // one resident wave of workgroups: CUs x workgroups per CU
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, NT, lds) != hipSuccess)
    return GDN_ERR_LAUNCH;
  const int64_t grid = std::min<int64_t>(tiles, (int64_t)std::max(1, cus) * std::max(1, per_cu));
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), lds, s, p, ordered);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

template <bool SB, bool AB, int DK, int DV>
static gdn_status launch_cw(const DecodeParams &p, bool cw, hipStream_t s) {
  return cw ? launch_t<SB, AB, DK, DV, true>(p, s) : launch_t<SB, AB, DK, DV, false>(p, s);
}

template <bool SB, bool AB, int DK>
static gdn_status launch_dv(const DecodeParams &p, int dv, bool cw, hipStream_t s) {
  switch (dv) {
    case 16: return launch_cw<SB, AB, DK, 16>(p, cw, s);
    case 32: return launch_cw<SB, AB, DK, 32>(p, cw, s);
    case 64: return launch_cw<SB, AB, DK, 64>(p, cw, s);
    case 128: return launch_cw<SB, AB, DK, 128>(p, cw, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

template <bool SB, bool AB>
static gdn_status launch_dk(const DecodeParams &p, int dk, int dv, bool cw, hipStream_t s) {
  switch (dk) {
    case 16: return launch_dv<SB, AB, 16>(p, dv, cw, s);
    case 32: return launch_dv<SB, AB, 32>(p, dv, cw, s);
    case 64: return launch_dv<SB, AB, 64>(p, dv, cw, s);
    case 128: return launch_dv<SB, AB, 128>(p, dv, cw, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

gdn_status launch_decode(const gdn_decode_args &a, hipStream_t s) {
  const DecodeParams p = make_decode_params(a);
  const bool sb = a.state_dtype == GDN_BF16, ab = a.act_dtype == GDN_BF16;
  const bool cw = a.decay_mode == GDN_DECAY_CHANNEL;
  if (sb && ab) return launch_dk<true, true>(p, a.d_k, a.d_v, cw, s);
  if (sb && !ab) return launch_dk<true, false>(p, a.d_k, a.d_v, cw, s);
  if (!sb && ab) return launch_dk<false, true>(p, a.d_k, a.d_v, cw, s);
  return launch_dk<false, false>(p, a.d_k, a.d_v, cw, s);
}

}  // namespace gdn
