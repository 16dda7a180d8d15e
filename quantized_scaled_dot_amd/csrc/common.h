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

// ---- KV tiles in LDS (shared by the attention and decode kernels) ----

// LDS row of key kappa (0..63) of a KV tile: 32*h + m with m the MFMA row
// m = 8*(v/4) + 4*g + v%4 for kappa = 32*g + 16*h + v.  k_lds_key inverts it.
__device__ __forceinline__ int k_lds_key(int rho) {
  const int h = rho >> 5, m = rho & 31;
  const int g = (m >> 2) & 1, v = 4 * (m >> 3) + (m & 3);
  return 32 * g + 16 * h + v;
}
// LDS rows are padded by 16 bytes (K: d+16, V: 64+16).  The matrix-core
// operand reads (ds_read_b128) touch the same 16-byte chunk of 8 or 16
// consecutive rows; with these strides those rows fall on distinct banks
// whether the LDS serves 8 lanes (128 bytes) or 16 lanes (256 bytes) per
// cycle, and every read of a wave shares one base address plus an immediate
// offset.
template <int D> constexpr int kRowK = D + 16;
constexpr int kRowV = kKTile + 16;

template <int OUT>
__device__ __forceinline__ void store4(void* O, size_t idx, v4f v) {
  if (OUT == 2) {
    *(v4f*)((float*)O + idx) = v;
  } else if (OUT == 1) {
    unsigned u[4];
#pragma unroll
    for (int e = 0; e < 4; e++) u[e] = bf16_bits_rne(v[e]);
    v2i w = {(int)(u[0] | (u[1] << 16)), (int)(u[2] | (u[3] << 16))};
    *(v2i*)((uint16_t*)O + idx) = w;
  } else {
    unsigned u[4];
#pragma unroll
    for (int e = 0; e < 4; e++) u[e] = f16_bits_rne(v[e]);
    v2i w = {(int)(u[0] | (u[1] << 16)), (int)(u[2] | (u[3] << 16))};
    *(v2i*)((uint16_t*)O + idx) = w;
  }
}

// Buffer resource for raw 16-byte loads of one head's codes (out-of-range
// offsets read zero; every offset used here is in range).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes
// lds + 16 l (the LDS address must be the same for the whole wave).
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
// The same copy to the LDS byte address lds_addr (an integer, so that the
// compiler does not tie the copy to an LDS object).
__device__ __forceinline__ void lds_copy16_at(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(uintptr_t)lds_addr, 16, voff, soff, 0, 0);
}

}  // namespace sage
