// device.h -- small device helpers shared by the gfx950 kernels: 16-byte
// vector loads/stores and BF16 <-> FP32 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// BF16 -> FP32 is exact: the 16 BF16 bits are the top half of the FP32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// FP32 -> BF16, round to nearest even (NaN stays NaN): the cast lowers to the
// gfx950 hardware conversion v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// An empty asm that claims to modify v: the compiler must re-derive anything it
// computed from v before this point, so values unpacked from v are not kept
// live across it (the packed form is half the registers).
__device__ __forceinline__ void opaque(uint4 &v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}
__device__ __forceinline__ void opaque(uint2 &v) { asm volatile("" : "+v"(v.x), "+v"(v.y)); }

// 16-byte loads and stores marked non-temporal (streamed once: no reason to
// keep the line in the caches).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load16(const void *p) {
  const nt_u32x4 v = __builtin_nontemporal_load(static_cast<const nt_u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store16(void *p, const uint4 &v) {
  nt_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<nt_u32x4 *>(p));
}

// Element type of a tensor: BF16 (stored as uint16) or FP32.
template <bool BF16> struct Elem;
template <> struct Elem<true> {
  using T = uint16_t;
  static constexpr int kPer16B = 8;
  __device__ static __forceinline__ void unpack(const uint4 &v, float *f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float *f) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]); v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]); v.w = pack_bf16x2(f[6], f[7]);
    return v;
  }
  __device__ static __forceinline__ float load1(const void *p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t *>(p)[i]);
  }
  __device__ static __forceinline__ void store1(void *p, int64_t i, float x) {
    static_cast<uint16_t *>(p)[i] = f32_to_bf16(x);
  }
};
template <> struct Elem<false> {
  using T = float;
  static constexpr int kPer16B = 4;
  __device__ static __forceinline__ void unpack(const uint4 &v, float *f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 pack(const float *f) {
    uint4 v;
    v.x = __float_as_uint(f[0]); v.y = __float_as_uint(f[1]);
    v.z = __float_as_uint(f[2]); v.w = __float_as_uint(f[3]);
    return v;
  }
  __device__ static __forceinline__ float load1(const void *p, int64_t i) {
    return static_cast<const float *>(p)[i];
  }
  __device__ static __forceinline__ void store1(void *p, int64_t i, float x) {
    static_cast<float *>(p)[i] = x;
  }
};

// Load N consecutive elements starting at element index i into f[0..N).
// Uses 16-byte loads when the run is a whole number of 16-byte vectors
// (callers guarantee the alignment then), element loads otherwise.
template <bool BF16, int N>
__device__ __forceinline__ void load_run(const void *base, int64_t i, float *f) {
  using E = Elem<BF16>;
  constexpr int V = E::kPer16B;
  if constexpr (N % V == 0) {
    const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const typename E::T *>(base) + i);
#pragma unroll
    for (int j = 0; j < N / V; ++j) E::unpack(p[j], f + j * V);
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) f[j] = E::load1(base, i + j);
  }
}

template <bool BF16, int N>
__device__ __forceinline__ void store_run(void *base, int64_t i, const float *f) {
  using E = Elem<BF16>;
  constexpr int V = E::kPer16B;
  if constexpr (N % V == 0) {
    uint4 *p = reinterpret_cast<uint4 *>(static_cast<typename E::T *>(base) + i);
#pragma unroll
    for (int j = 0; j < N / V; ++j) p[j] = E::pack(f + j * V);
  } else {
#pragma unroll
    for (int j = 0; j < N; ++j) E::store1(base, i + j, f[j]);
  }
}

}  // namespace gdn
