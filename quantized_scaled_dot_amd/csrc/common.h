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

// Bias of the INT8 score accumulators: the integer matrix instruction starts
// from the bit pattern of B = 1.5 * 2^23, so each int32 result B_bits + S,
// read as fp32, is exactly B + S (|S| <= 127^2 * 128 < 2^21 keeps it inside
// [2^23, 2^24), where fp32 spacing is 1): the softmax needs no int-to-float
// conversion per score.
constexpr float kScoreBiasF = 12582912.0f;
constexpr int kScoreBiasBits = 0x4B400000;
constexpr v16i kScoreBias16 = {kScoreBiasBits, kScoreBiasBits, kScoreBiasBits, kScoreBiasBits,
                               kScoreBiasBits, kScoreBiasBits, kScoreBiasBits, kScoreBiasBits,
                               kScoreBiasBits, kScoreBiasBits, kScoreBiasBits, kScoreBiasBits,
                               kScoreBiasBits, kScoreBiasBits, kScoreBiasBits, kScoreBiasBits};
// The exact score S of a biased accumulator value (wrapping unsigned arithmetic:
// masked sentinels are compared before this is used, never converted).
__device__ __forceinline__ int unbias_score(int x) { return (int)((unsigned)x - (unsigned)kScoreBiasBits); }

// FP4 x FP4 scaled MFMA whose A scale is byte SEL of the word sa (the
// instruction's operand byte select: no extraction on the VALU); B scale sb.
template <int SEL>
__device__ __forceinline__ v16f mfma_fp4_sel(const v8i& a, const v8i& b, const v16f& c, unsigned sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, SEL, (int)sa, 0, sb);
}
// the same with SEL picked by a value that is a constant after unrolling
__device__ __forceinline__ v16f mfma_fp4_byte(int sel, const v8i& a, const v8i& b, const v16f& c, unsigned sa, int sb) {
  return sel == 0 ? mfma_fp4_sel<0>(a, b, c, sa, sb)
       : sel == 1 ? mfma_fp4_sel<1>(a, b, c, sa, sb)
       : sel == 2 ? mfma_fp4_sel<2>(a, b, c, sa, sb)
                  : mfma_fp4_sel<3>(a, b, c, sa, sb);
}

// Row sum of a wave's FP8 P~ codes on the matrix core.  pb is the B operand
// of the 32x32x64 P~V instruction (lane l: query l%32, keys 32(l/32) ..
// +31).  Read as the B operand of the 16x16x128 FP8 instruction, lane l is
// column l%16 of lane group l/16; with an A operand that is all ones (e4m3
// 1.0) exactly where row (l%16)/4 and lane group l/16 have the same parity,
// and zero elsewhere, row r of column n sums lane groups of r's parity: the
// 64 keys of query n (even) or n + 16 (odd).  Lane l holds rows 4(l/16) ..
// +3 of column l%16, i.e. the sum for its own query l%32 in every register.
// The same with E2M1 operands (fp4): 32 codes per lane in the low 16 bytes,
// E2M1 1.0 = code 2, and the B scale of each lane (its own block's E8M0
// byte) applied inside the instruction.
__device__ __forceinline__ v8i rowsum_ones_operand(int lane, bool fp4 = false) {
  const bool on = (((lane & 15) >> 2) & 1) == ((lane >> 4) & 1);
  const int w = on ? (fp4 ? 0x22222222 : 0x38383838) : 0;
  return fp4 ? v8i{w, w, w, w, 0, 0, 0, 0} : v8i{w, w, w, w, w, w, w, w};
}
__device__ __forceinline__ float rowsum_fp8(const v8i& ones, const v8i& pb) {
  const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pb, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0,
                                                                 127, 0, 127);
  return r[0];
}
__device__ __forceinline__ float rowsum_fp4(const v8i& ones, const v8i& pb, int pscale) {
  const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pb, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0,
                                                                 127, 0, pscale);
  return r[0];
}

// fp16 / bf16 -> fp32 (both exact).
__device__ __forceinline__ float load_h(uint16_t h, bool is_bf16) {
  if (is_bf16) return __uint_as_float((uint32_t)h << 16);
  return (float)__builtin_bit_cast(_Float16, h);
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

// Four consecutive outputs: fp32, or bf16 / fp16 rounded to nearest even by
// the packed hardware converts (v_cvt_pk_bf16_f32, v_cvt_pk_f16_f32: one
// instruction per two values).  A check over every non-NaN fp32 input on the
// MI355X found both equal to round-to-nearest-even on the bit pattern.
template <int OUT>
__device__ __forceinline__ void store4(void* O, size_t idx, v4f v) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  if (OUT == 2) {
    *(v4f*)((float*)O + idx) = v;
  } else if (OUT == 1) {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    const h2 lo = __builtin_convertvector(f2{v[0], v[1]}, h2), hi = __builtin_convertvector(f2{v[2], v[3]}, h2);
    const v2i w = {__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
    *(v2i*)((uint16_t*)O + idx) = w;
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 lo = __builtin_convertvector(f2{v[0], v[1]}, h2), hi = __builtin_convertvector(f2{v[2], v[3]}, h2);
    const v2i w = {__builtin_bit_cast(int, lo), __builtin_bit_cast(int, hi)};
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
