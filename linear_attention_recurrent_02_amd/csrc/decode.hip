// decode.hip -- the decode kernel: a persistent grid of workgroups that walk
// the (request, state head) tiles of a batch in write-slot order; the tile
// body is decode_tile() in decode.cuh (shared with the mixed launcher) and
// the order comes from build_slot_order() in order.cuh.
#include "decode.cuh"
#include "order.cuh"

#include <algorithm>

namespace gdn {

extern __shared__ int order_lds[];  // the slot order (dynamic LDS)

template <bool SB, bool AB, int DK, int DV, bool CW, bool Q8>
__device__ __forceinline__ void decode_walk(const DecodeParams &p, int ordered, float *red) {
  constexpr int NT = decode_threads<SB, DK, DV>();
  if (ordered) build_slot_order<NT>(p.write_slot, p.B, p.n_slots, order_lds);
  const int64_t n_tiles = (int64_t)p.B * p.H_v;
  // one tile at a time: a software-pipelined loop (the next tile's loads in
  // flight during this tile's reduction and store) measured slower on MI355X
  // (196 against 191 us per B = 512 launch), its extra registers costing more
  // occupancy than the overlap gains
  auto walk = [&](auto i8) {
    constexpr bool I8 = decltype(i8)::value;
    using Regs = DecodeTileRegs<SB, AB, DK, DV, NT, CW, Q8, I8>;
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
      const int pos = (int)(t / p.H_v);
      Regs cur;
      decode_tile_load<SB, AB, DK, DV, NT, CW, Q8, I8>(p, ordered ? order_lds[pos] : pos,
                                                       (int)(t % p.H_v), cur, (int)threadIdx.x);
      decode_tile_finish<SB, AB, DK, DV, NT, CW, Q8, I8>(p, cur, red, (int)threadIdx.x);
    }
  };
  if constexpr (Q8) {
    // the wave's rows are all BF16 or all INT8 (host validation: hi_rows is a
    // multiple of q8_row_quantum), so the branch is uniform per wave and every
    // wave meets the same barriers in either instance
    using S = DecodeShape<SB, DK, DV, NT>;
    const int wave_row0 = (int)(threadIdx.x >> 6) * (64 / S::LPR) * S::RPT;
    if (wave_row0 < p.hi_rows) walk(std::false_type());
    else walk(std::true_type());
  } else {
    walk(std::false_type());
  }
}

template <bool SB, bool AB, int DK, int DV, bool CW, bool Q8>
__global__ __launch_bounds__(kDecodeMaxThreads) void decode_kernel(DecodeParams p, int ordered) {
  __shared__ float red[DecodeShape<SB, DK, DV, decode_threads<SB, DK, DV>()>::LDS_FLOATS];
  decode_walk<SB, AB, DK, DV, CW, Q8>(p, ordered, red);
}

// The 8-bit format with a per-head decay at four waves per SIMD: its INT8
// instance needs 129 registers and would otherwise run three.  The forced 128
// spill 12 bytes per lane and still win (B = 512 x 48 layers, d = 128, 32
// BF16 rows: 169 against 188 us per launch); each tile's pass is latency
// bound, so waves in flight count more than the bytes of a tile.
template <bool AB, int DK, int DV>
__global__ __launch_bounds__(kDecodeMaxThreads) __attribute__((amdgpu_waves_per_eu(4)))
void decode_q8_kernel(DecodeParams p, int ordered) {
  __shared__ float red[DecodeShape<true, DK, DV, decode_threads<true, DK, DV>()>::LDS_FLOATS];
  decode_walk<true, AB, DK, DV, false, true>(p, ordered, red);
}

DecodeParams make_decode_params(const gdn_decode_args &a) {
  DecodeParams p;
  p.B = a.B; p.H_qk = a.H_qk; p.H_v = a.H_v; p.group = a.H_v / a.H_qk;
  p.n_slots = a.n_slots; p.scale = a.scale; p.rule = a.rule;
  p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta;
  p.pool = a.state_pool; p.read_slot = a.read_slot; p.write_slot = a.write_slot;
  p.o = a.o; p.status = a.status;
  p.hi_rows = a.state_dtype == GDN_Q8 ? a.state_bf16_rows : 0;
  p.tile_bytes = a.state_dtype == GDN_Q8
                     ? (int64_t)gdn_state_q8_bytes(1, a.d_k, a.d_v, a.state_bf16_rows)
                     : 0;
  return p;
}

template <bool SB, bool AB, int DK, int DV, bool CW, bool Q8>
static gdn_status launch_t(const DecodeParams &p, hipStream_t s) {
  constexpr int NT = decode_threads<SB, DK, DV>();
  const int64_t tiles = (int64_t)p.B * p.H_v;
  const int ordered =
      p.write_slot != nullptr && p.B <= kOrderMaxB && p.n_slots <= kOrderMaxSlots ? 1 : 0;
  const size_t lds = ordered ? slot_order_lds_bytes(p.B, p.n_slots, NT) : 0;
  auto kern = decode_kernel<SB, AB, DK, DV, CW, Q8>;
  if constexpr (Q8 && !CW) kern = decode_q8_kernel<AB, DK, DV>;
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
static gdn_status launch_cw(const DecodeParams &p, bool cw, bool q8, hipStream_t s) {
  if constexpr (SB) {
    if (q8)
      return cw ? launch_t<SB, AB, DK, DV, true, true>(p, s)
                : launch_t<SB, AB, DK, DV, false, true>(p, s);
  }
  return cw ? launch_t<SB, AB, DK, DV, true, false>(p, s)
            : launch_t<SB, AB, DK, DV, false, false>(p, s);
}

template <bool SB, bool AB, int DK>
static gdn_status launch_dv(const DecodeParams &p, int dv, bool cw, bool q8, hipStream_t s) {
  switch (dv) {
    case 16: return launch_cw<SB, AB, DK, 16>(p, cw, q8, s);
    case 32: return launch_cw<SB, AB, DK, 32>(p, cw, q8, s);
    case 64: return launch_cw<SB, AB, DK, 64>(p, cw, q8, s);
    case 128: return launch_cw<SB, AB, DK, 128>(p, cw, q8, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

template <bool SB, bool AB>
static gdn_status launch_dk(const DecodeParams &p, int dk, int dv, bool cw, bool q8,
                            hipStream_t s) {
  switch (dk) {
    case 16: return launch_dv<SB, AB, 16>(p, dv, cw, q8, s);
    case 32: return launch_dv<SB, AB, 32>(p, dv, cw, q8, s);
    case 64: return launch_dv<SB, AB, 64>(p, dv, cw, q8, s);
    case 128: return launch_dv<SB, AB, 128>(p, dv, cw, q8, s);
  }
  return GDN_ERR_UNSUPPORTED;
}

gdn_status launch_decode(const gdn_decode_args &a, hipStream_t s) {
  const DecodeParams p = make_decode_params(a);
  // the 8-bit format runs the BF16 tile shape
  const bool q8 = a.state_dtype == GDN_Q8;
  const bool sb = a.state_dtype == GDN_BF16 || q8, ab = a.act_dtype == GDN_BF16;
  const bool cw = a.decay_mode == GDN_DECAY_CHANNEL;
  if (sb && ab) return launch_dk<true, true>(p, a.d_k, a.d_v, cw, q8, s);
  if (sb && !ab) return launch_dk<true, false>(p, a.d_k, a.d_v, cw, q8, s);
  if (!sb && ab) return launch_dk<false, true>(p, a.d_k, a.d_v, cw, false, s);
  return launch_dk<false, false>(p, a.d_k, a.d_v, cw, false, s);
}

}  // namespace gdn
