// Shared device helpers of the gfx950 kernels (HIP, CDNA4 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Query rows per attention workgroup (4 waves x 32 rows) and keys per KV tile.
constexpr int kQTile = 128;
constexpr int kKTile = 64;
// Tokens per workgroup of the per-channel statistics passes (K sums, V maxima).
constexpr int kStatChunk = 256;

// log2(e) rounded to fp32.
constexpr float kLog2e = 0x1.715476p+0f;

// fp16 / bf16 -> fp32 (both exact).
__device__ __forceinline__ float load_h(uint16_t h, bool is_bf16) {
  if (is_bf16) return __uint_as_float((uint32_t)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
}

// fp32 -> bf16 / fp16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
// (The hardware f32->f16 conversion was measured to round exact ties away from
// zero, so the rounding is done here on the bit pattern.)
__device__ __forceinline__ uint32_t f16_bits_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 16) & 0x8000u, a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7E00u;                  // NaN
  if (a >= 0x477FF000u) return sign | 0x7C00u;                 // rounds to infinity
  if (a >= 0x38800000u) {                                      // normal half: rebias, round 13 bits
    const uint32_t m = a - 0x38000000u;
    return sign | ((m + 0xFFFu + ((m >> 13) & 1u)) >> 13);
  }
  // subnormal half: |x| * 2^24 < 1024 is exact in fp32; rint rounds ties to even
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 16777216.0f);
}

// Exchange with the lane 32 apart (same query row, other half of the keys /
// channels): v_permlane32_swap returns {x[l], x[l^32]} in some order for every
// lane, so a symmetric combination of the two results is the pair's combination.
__device__ __forceinline__ int pair_max_i32(int x) {
  auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  int a = (int)r[0], b = (int)r[1];
  return a > b ? a : b;
}
__device__ __forceinline__ float pair_max_f32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum_f32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace sage
