// convert.hip -- state tiles copied between pools of different storage
// formats (FP32, BF16, or the 8-bit format of DAMP-like mixed precision,
// "Seven Architectures Replacing KV Cache With Bounded Mutable State",
// ONNX LinearAttention / FlashInfer section), slot to slot with the
// recurrent state's read/write rules ("Recurrent state" glossary entry, Why
// it matters).
//
// What it is for: a prefill stores its state in BF16 or FP32 while decode
// runs on an 8-bit pool, so a prefilled state is stored into the 8-bit pool
// here, and an 8-bit checkpoint is read back here before a prefill resumes.
//
// The 8-bit encoding is the one the decode stores: the first bf16_rows key
// channels (rows) of a tile in BF16 (round to nearest even), every other row
// as INT8 codes with one binary32 scale, code = rne(x * (127 / rowmax))
// clamped to +-127, scale = rowmax / 127, each step in binary32.  Decoding a
// row gives code * scale in binary32; storing to BF16 rounds to nearest even.
//
// One workgroup of 256 threads per (slot pair, head); a lane owns 8
// consecutive columns of a row (one 16-byte BF16 piece, two FP32 pieces or 8
// INT8 codes) and the LPR = d_v / 8 lanes of a row are an aligned group of
// one wave, so the row maximum is a DPP reduction.  The lanes of a row load
// before any stores, so a pair may read and write the same slot of one pool.
#include "decode.cuh"

namespace gdn {

constexpr int kConvertThreads = 256;

struct ConvertParams {
  int32_t n, H_v, d_k;
  int32_t src_kind, dst_kind;          // GDN_F32, GDN_BF16, GDN_Q8
  int32_t src_hi, dst_hi;              // BF16 rows of an 8-bit tile
  int64_t src_tile_bytes, dst_tile_bytes;
  int64_t src_n_slots, dst_n_slots;
  const char *src;
  char *dst;
  const int32_t *src_slot, *dst_slot;
  uint32_t *status;
};

template <int DV>
__global__ __launch_bounds__(kConvertThreads) void convert_kernel(ConvertParams p) {
  constexpr int LPR = DV / 8;                  // lanes per row
  constexpr int RPI = kConvertThreads / LPR;   // rows per pass of the workgroup
  const int pair = (int)(blockIdx.x / (unsigned)p.H_v), h = (int)(blockIdx.x % (unsigned)p.H_v);
  const int tid = (int)threadIdx.x, cv = tid % LPR;
  const int64_t ss = p.src_slot ? (int64_t)p.src_slot[pair] : pair;
  const int64_t ds = p.dst_slot ? (int64_t)p.dst_slot[pair] : pair;
  if (ss < -1 || ss >= p.src_n_slots || ds < -1 || ds >= p.dst_n_slots) {
    if (tid == 0 && p.status) atomicOr(p.status, GDN_DEVICE_BAD_SLOT);
    return;
  }
  if (ds < 0) return;  // nothing stored
  const char *src = ss >= 0 ? p.src + (ss * p.H_v + h) * p.src_tile_bytes : nullptr;
  char *dst = p.dst + (ds * p.H_v + h) * p.dst_tile_bytes;
  const int64_t src_lo = (int64_t)p.src_hi * DV * 2;  // byte offset of an 8-bit tile's codes
  const int64_t dst_lo = (int64_t)p.dst_hi * DV * 2;

  for (int row = tid / LPR; row < p.d_k; row += RPI) {
    // this lane's 8 values of the row (a read slot of -1 is the zero state)
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = 0.f;
    if (src) {
      if (p.src_kind == GDN_F32) {
        const uint4 *s = reinterpret_cast<const uint4 *>(src + ((int64_t)row * DV + cv * 8) * 4);
        Elem<false>::unpack(s[0], f);
        Elem<false>::unpack(s[1], f + 4);
      } else if (p.src_kind == GDN_BF16 || row < p.src_hi) {
        Elem<true>::unpack(
            *reinterpret_cast<const uint4 *>(src + ((int64_t)row * DV + cv * 8) * 2), f);
      } else {
        const int i = row - p.src_hi;
        const uint2 c = *reinterpret_cast<const uint2 *>(src + src_lo + (int64_t)i * DV + cv * 8);
        const float sc = reinterpret_cast<const float *>(
            src + src_lo + (int64_t)(p.d_k - p.src_hi) * DV)[i];
        unpack_i8(c, sc, f);
      }
    }
    // the row in the destination format
    if (p.dst_kind == GDN_F32) {
      uint4 *d = reinterpret_cast<uint4 *>(dst + ((int64_t)row * DV + cv * 8) * 4);
      d[0] = Elem<false>::pack(f);
      d[1] = Elem<false>::pack(f + 4);
    } else if (p.dst_kind == GDN_BF16 || row < p.dst_hi) {
      *reinterpret_cast<uint4 *>(dst + ((int64_t)row * DV + cv * 8) * 2) = Elem<true>::pack(f);
    } else {
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
      m = lane_group_max<LPR>(m);  // the row's largest magnitude
      const float inv = m > 0.f ? 127.f / m : 0.f;
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = fminf(fmaxf(f[e] * inv, -127.f), 127.f);
        w[e >> 2] |= ((uint32_t)(int)rintf(y) & 0xffu) << (8 * (e & 3));
      }
      const int i = row - p.dst_hi;
      *reinterpret_cast<uint2 *>(dst + dst_lo + (int64_t)i * DV + cv * 8) = make_uint2(w[0], w[1]);
      if (cv == 0)
        reinterpret_cast<float *>(dst + dst_lo + (int64_t)(p.d_k - p.dst_hi) * DV)[i] = m / 127.f;
    }
  }
}

gdn_status launch_state_convert(const gdn_convert_args &a, hipStream_t s) {
  auto tile = [&](int32_t kind, int32_t hi) -> int64_t {
    if (kind == GDN_Q8) return (int64_t)gdn_state_q8_bytes(1, a.d_k, a.d_v, hi);
    return (int64_t)a.d_k * a.d_v * (kind == GDN_BF16 ? 2 : 4);
  };
  ConvertParams p;
  p.n = a.n; p.H_v = a.H_v; p.d_k = a.d_k;
  p.src_kind = a.src_dtype; p.dst_kind = a.dst_dtype;
  p.src_hi = a.src_dtype == GDN_Q8 ? a.src_bf16_rows : 0;
  p.dst_hi = a.dst_dtype == GDN_Q8 ? a.dst_bf16_rows : 0;
  p.src_tile_bytes = tile(a.src_dtype, p.src_hi);
  p.dst_tile_bytes = tile(a.dst_dtype, p.dst_hi);
  p.src_n_slots = a.src_n_slots; p.dst_n_slots = a.dst_n_slots;
  p.src = static_cast<const char *>(a.src_pool);
  p.dst = static_cast<char *>(a.dst_pool);
  p.src_slot = a.src_slot; p.dst_slot = a.dst_slot; p.status = a.status;
  const dim3 grid((unsigned)((int64_t)a.n * a.H_v));
  switch (a.d_v) {
    case 16: hipLaunchKernelGGL(convert_kernel<16>, grid, dim3(kConvertThreads), 0, s, p); break;
    case 32: hipLaunchKernelGGL(convert_kernel<32>, grid, dim3(kConvertThreads), 0, s, p); break;
    case 64: hipLaunchKernelGGL(convert_kernel<64>, grid, dim3(kConvertThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(convert_kernel<128>, grid, dim3(kConvertThreads), 0, s, p); break;
    default: return GDN_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace gdn
