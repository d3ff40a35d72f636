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
