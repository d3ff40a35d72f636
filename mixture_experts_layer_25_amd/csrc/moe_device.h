// Device-side helpers shared by the libmoe kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Work split shared by the top-k, scan and assign kernels: the tokens of
// one chunk are ranked together, chunks are combined by the scan.
constexpr int kChunkTokens = 256;

// Row tiles of the grouped GEMMs (the scan kernel sizes the tile table
// with the same values).
constexpr int kGemmBM_bf16 = 256;
constexpr int kGemmBM_f32 = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  bf16 h = (bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// 16-byte global load / store through a uint4.
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Element types of the layer's tensors: bf16 (held as uint16_t bits) or
// fp32.  Elt<T> converts one element, and 16 bytes (8 bf16 or 4 fp32) at a
// time, to and from fp32; bf16 stores round to nearest even.
template <typename T>
struct Elt;
template <>
struct Elt<uint16_t> {
  static constexpr int kVec = 8;
  static __device__ __forceinline__ float ld(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void st(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
  static __device__ __forceinline__ void unpack(uint4 q, float (&f)[8]) {
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      f[2 * p] = bf16_bits_to_f32(u[p] & 0xFFFFu);
      f[2 * p + 1] = bf16_bits_to_f32(u[p] >> 16);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float (&f)[8]) {
    return uint4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
  }
};
template <>
struct Elt<float> {
  static constexpr int kVec = 4;
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ void unpack(uint4 q, float (&f)[4]) {
    f[0] = __uint_as_float(q.x);
    f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z);
    f[3] = __uint_as_float(q.w);
  }
  static __device__ __forceinline__ uint4 pack(const float (&f)[4]) {
    return uint4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};

// Monotone map of an fp32 value to uint32 (larger float -> larger integer).
// -0.0 is folded onto +0.0 first so that the two compare equal, as floats do.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Max / sum over aligned segments of G lanes (G a power of two <= 64);
// every lane of a segment gets the result.
template <int G>
__device__ __forceinline__ float seg_max_f32(float v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, G));
  return v;
}

template <int G>
__device__ __forceinline__ float seg_sum_f32(float v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, G);
  return v;
}

// Lanes per token of the segment kernels (top-k, router probabilities):
// the next power of two >= E, at most 64.
inline int seg_lanes(int E) { return E <= 8 ? 8 : (E <= 16 ? 16 : (E <= 32 ? 32 : 64)); }

}  // namespace moe
