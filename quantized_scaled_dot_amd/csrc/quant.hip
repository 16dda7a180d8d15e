// Quantization kernels (gfx950): K smoothing + INT8 per-block Q/K, FP8 V with
// per-channel scales.  All passes stream HBM with 16-byte loads; every
// reduction is order-free (exact integer sums, max), so results do not depend
// on launch geometry.
//
// quantize_qk: pass 1 = {INT8 blocks of Q} + {per-chunk K channel sums} in one
//              launch; finalize = per-head K mean; pass 2 = INT8 blocks of the
//              smoothed K.
// quantize_v:  pass 1 = per-chunk V channel maxima; finalize = per-channel
//              scales and reciprocals; pass 2 = FP8 codes, transposed in
//              registers into the KV-tile channel-major layout.
// quantize_qk4: the K mean as above, then 4-bit E2M1 blocks of Q and of the
//              smoothed K (one thread per token and 32 channels); with Q
//              smoothing first the block means of 32 queries, and K also in
//              FP8 blocks.
#include "common.h"
#include "launch.h"

namespace sage {

// 16-byte loads and code stores.  The codes are written with non-temporal
// (streaming) stores, and the passes that read an input for the first time
// (Q blocks, K channel sums, V channel maxima) use streaming loads; the
// second passes over K and V use ordinary loads.  Measured on MI355X against
// ordinary loads and stores throughout: quantize_qk + quantize_v 9-10% faster
// at the 32k and 4k shapes, the same bits.
template <bool STREAM>
__device__ __forceinline__ v4i load16_in(const void* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load((const v4i*)p);
  else return *(const v4i*)p;
}

// Max over each group of TPB consecutive threads (TPB = 128 or 256) of a
// 256-thread workgroup.
template <int TPB>
__device__ __forceinline__ float group_max(float a, float* red4) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = a;
  __syncthreads();
  if (TPB == 256) return fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
  const int g = (threadIdx.x >> 7) * 2;
  return fmaxf(red4[g], red4[g + 1]);
}

__device__ __forceinline__ float half_of(const v4i& raw, int e, int is_bf16) {
  return load_h((uint16_t)((unsigned)raw[e >> 1] >> (16 * (e & 1))), is_bf16);
}

// Rows of d elements of an input tensor: [B,H,N,d] (head-major) or [B,N,H,d]
// (token-major).  Row n of flat head bh starts at head(bh) + n * stride.  The
// codes of a head hold P >= N rows (N rounded up to the block / tile); rows
// N..P-1 are zero codes.
struct InRows {
  int H, N, P, nhd;
  __device__ __forceinline__ size_t head(int bh, int D) const {
    return nhd ? ((size_t)(bh / H) * N * H + (size_t)(bh % H)) * D : (size_t)bh * N * D;
  }
  __device__ __forceinline__ size_t stride(int D) const { return nhd ? (size_t)H * D : (size_t)D; }
};

// Exponent of the power-of-two scale of INT8 codes for a block with
// max |x| = a: the smallest e in [-63, 52] with a * 2^-e <= 127 (a = 0: -63).
__device__ __forceinline__ int int8_pow2_exponent(float a) {
  if (a == 0.0f) return -63;
  int e = ilogbf(a) - 6;                 // a * 2^-e in [64, 128)
  if (ldexpf(a, -e) > 127.0f) e += 1;    // then in [32, 64)
  return min(max(e, -63), 52);
}

// ---------------------------------------------------------------------------
// Symmetric INT8 quantization of one block of BLK tokens x D channels:
// a = max|x| (x = K - mean when SMOOTH), scale = a/127, r = 127/a,
// code = rint(x * r) in [-127, 127]; a < 2^-120 gives scale 0 and zero codes.
// POW2: the scale is 2^e instead (int8_pow2_exponent), r = 2^-e exactly, and
// the byte e + 127 is written as the scale.
// Tokens at or past N (the shorter last block) are not read and count as 0.
// A block is held by TPB = min(256, BLK*D/8) threads, 8 values per 16-byte
// load; a 256-thread workgroup quantizes 256/TPB consecutive blocks.
// ---------------------------------------------------------------------------
template <int D, int BLK>
constexpr int blocks_per_wg() { return BLK * D / 8 >= 256 ? 1 : 256 / (BLK * D / 8); }

template <int D, int BLK, bool SMOOTH, bool POW2 = false, typename ST = float>
__device__ __forceinline__ void quant_block(const uint16_t* __restrict__ X, int is_bf16, InRows in,
                                            const float* __restrict__ mean, int8_t* __restrict__ codes,
                                            ST* __restrict__ scale, int lin, float* red4) {
  constexpr int NB = blocks_per_wg<D, BLK>();
  constexpr int TPB = 256 / NB;                // threads per block
  constexpr int LPT = BLK * D / 8 / TPB;       // 16-byte loads per thread
  constexpr int EPT = 8 * LPT;                 // values per thread
  static_assert(TPB == 128 || TPB == 256, "block sizes of 16 to 128 tokens at d = 64 or 128");
  const int nblk = in.P / BLK;
  const int gblk = lin * NB + (int)threadIdx.x / TPB;
  const int blk = gblk % nblk, bh = gblk / nblk;
  const int t = threadIdx.x % TPB;
  const size_t off = ((size_t)bh * in.P + (size_t)blk * BLK) * D;   // codes: [BH, P, D]
  const uint16_t* src = X + in.head(bh, D);
  float x[EPT];
  float a = 0.0f;
#pragma unroll
  for (int l = 0; l < LPT; l++) {
    const int ch = l * TPB + t;   // 16-byte chunk index within the block
    // a token past N reads the last real token (every load stays in bounds
    // and none is predicated) and then counts as zero
    const int tok = blk * BLK + ch / (D / 8);
    const bool valid = tok < in.N;
    v4i raw = load16_in<!SMOOTH>(src + (size_t)min(tok, in.N - 1) * in.stride(D) + (size_t)(ch % (D / 8)) * 8);
    if (!valid) raw = v4i{0, 0, 0, 0};
    const int c0 = (ch * 8) % D;
    float mu[8];
    if (SMOOTH) {
      v4f m0 = *(const v4f*)(mean + (size_t)bh * D + c0);
      v4f m1 = *(const v4f*)(mean + (size_t)bh * D + c0 + 4);
#pragma unroll
      for (int e = 0; e < 4; e++) { mu[e] = m0[e]; mu[e + 4] = m1[e]; }
    }
#pragma unroll
    for (int e = 0; e < 8; e++) {
      float v = half_of(raw, e, is_bf16);
      if (SMOOTH) v = valid ? v - mu[e] : 0.0f;
      x[l * 8 + e] = v;
      a = fmaxf(a, fabsf(v));
    }
  }
  a = group_max<TPB>(a, red4);
  const bool zero = !(a >= 0x1p-120f);
  const float dl = zero ? 0.0f : a / 127.0f;
  const int e2 = POW2 ? int8_pow2_exponent(a) : 0;
  const float r = POW2 ? ldexpf(1.0f, -e2) : zero ? 0.0f : 127.0f / a;
  int8_t* dst = codes + off;
#pragma unroll
  for (int l = 0; l < LPT; l++) {
    const int ch = l * TPB + t;
    unsigned w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      float y = __builtin_rintf(x[l * 8 + e] * r);
      y = fminf(fmaxf(y, -127.0f), 127.0f);
      w[e >> 2] |= ((unsigned)(int)y & 0xFFu) << (8 * (e & 3));
    }
    v2i pk = {(int)w[0], (int)w[1]};
    __builtin_nontemporal_store(pk, (v2i*)(dst + (size_t)ch * 8));
  }
  if (t == 0) scale[(size_t)bh * nblk + blk] = POW2 ? (ST)(e2 + 127) : (ST)dl;
}

// ---------------------------------------------------------------------------
// Per-channel fixed-point sums of K over one chunk of kStatChunk tokens:
// s_c = sum_t trunc(clamp(k, +-2^19) * 2^24).  Each term is an integer of at
// most 2^43; a thread adds at most 32 of them in fp64 (exact below 2^53),
// converts once to int64, and the threads' int64 sums are combined through
// LDS.  With at most 2^19 tokens a head's sum stays within 2^62.
// ---------------------------------------------------------------------------
template <int D, bool STREAM = true>
__device__ __forceinline__ void k_colsum(const uint16_t* __restrict__ K, int is_bf16, InRows in, int nchunk, int lin,
                                         long long* __restrict__ partial, long long (*red)[D]) {
  const int N = in.N;
  const size_t rs = in.stride(D);
  constexpr int TPR = D / 8;        // threads per token row
  constexpr int RPP = 256 / TPR;    // token rows per pass
  const int chunk = lin % nchunk, bh = lin / nchunk;
  const int t = threadIdx.x, cg = t % TPR, r0 = t / TPR;
  const int n0 = chunk * kStatChunk;
  const int nrows = min(kStatChunk, N - n0);
  double s[8];
#pragma unroll
  for (int e = 0; e < 8; e++) s[e] = 0.0;
  const uint16_t* base = K + in.head(bh, D) + (size_t)n0 * rs + cg * 8;
  auto add_row = [&](const v4i& raw) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float x = fminf(fmaxf(half_of(raw, e, is_bf16), -524288.0f), 524288.0f);
      s[e] += (double)__builtin_truncf(x * 16777216.0f);   // exact product, exact sum
    }
  };
  if (nrows == kStatChunk) {   // full chunk: issue every row load of this thread first
    constexpr int RPT = kStatChunk / RPP;
    v4i raw[RPT];
#pragma unroll
    for (int i = 0; i < RPT; i++) raw[i] = load16_in<STREAM>(base + (size_t)(r0 + i * RPP) * rs);
#pragma unroll
    for (int i = 0; i < RPT; i++) add_row(raw[i]);
  } else {
    for (int r = r0; r < nrows; r += RPP) add_row(*(const v4i*)(base + (size_t)r * rs));
  }
#pragma unroll
  for (int e = 0; e < 8; e++) red[r0][cg * 8 + e] = (long long)s[e];
  __syncthreads();
  for (int c = t; c < D; c += 256) {
    long long tot = 0;
    for (int r = 0; r < RPP; r++) tot += red[r][c];
    partial[((size_t)bh * nchunk + chunk) * D + c] = tot;
  }
}

// Pass 1 of quantize_qk.  Grid: the workgroups of the B*Hq*P/BLKQ Q blocks,
// followed by B*Hkv*nchunk K chunks.
template <int D, int BLKQ>
__global__ __launch_bounds__(256) void qk_pass1_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                        int is_bf16, InRows qin, InRows kin, int nq, int nchunk,
                                                        int8_t* __restrict__ q_codes, float* __restrict__ q_scale,
                                                        long long* __restrict__ partial) {
  __shared__ long long red[256 / (D / 8)][D];
  __shared__ float red4[4];
  const int b = blockIdx.x;
  if (b < nq) quant_block<D, BLKQ, false>(Q, is_bf16, qin, nullptr, q_codes, q_scale, b, red4);
  else k_colsum<D>(K, is_bf16, kin, nchunk, b - nq, partial, red);
}

// mean_c = fp32(fp64(sum_chunks s_c) * 2^-24 / N).  Grid: BH * D/16; a block
// of 256 = 16 channels x 16 chunk lanes.
__device__ __forceinline__ void k_mean_group(const long long* __restrict__ partial, int nchunk, int N, int D,
                                             float* __restrict__ k_mean, int lin, long long (*red)[16]) {
  const int ng = D / 16, g = lin % ng, bh = lin / ng;
  const int cl = threadIdx.x & 15, j = threadIdx.x >> 4;
  const int c = g * 16 + cl;
  long long s = 0;
  for (int ch = j; ch < nchunk; ch += 16) s += partial[((size_t)bh * nchunk + ch) * D + c];
  red[j][cl] = s;
  __syncthreads();
  if (threadIdx.x < 16) {
    long long tot = 0;
    for (int k = 0; k < 16; k++) tot += red[k][threadIdx.x];
    k_mean[(size_t)bh * D + g * 16 + threadIdx.x] = (float)(((double)tot * 0x1p-24) / (double)N);
  }
}
__global__ __launch_bounds__(256) void k_mean_kernel(const long long* __restrict__ partial, int nchunk, int N, int D,
                                                      float* __restrict__ k_mean) {
  __shared__ long long red[16][16];
  k_mean_group(partial, nchunk, N, D, k_mean, blockIdx.x, red);
}

// Pass 2 of quantize_qk: INT8 blocks of BLKK tokens of the smoothed K.
// Grid: (B*Hkv*P/BLKK) / blocks_per_wg.
template <int D, int BLKK>
__global__ __launch_bounds__(256) void k_quant_kernel(const uint16_t* __restrict__ K, int is_bf16, InRows kin,
                                                       const float* __restrict__ k_mean, int8_t* __restrict__ k_codes,
                                                       float* __restrict__ k_scale) {
  __shared__ float red4[4];
  quant_block<D, BLKK, true>(K, is_bf16, kin, k_mean, k_codes, k_scale, blockIdx.x, red4);
}

// ---------------------------------------------------------------------------
// Per-channel maxima of |V| over one chunk of tokens.  Grid: nchunk * BH.
// ---------------------------------------------------------------------------
template <int D, bool STREAM = true>
__device__ __forceinline__ void v_colmax_chunk(const uint16_t* __restrict__ V, int is_bf16, InRows in, int nchunk,
                                               float* __restrict__ partial, int lin, float (*red)[D]) {
  const int N = in.N;
  const size_t rs = in.stride(D);
  constexpr int TPR = D / 8;
  constexpr int RPP = 256 / TPR;
  const int chunk = lin % nchunk, bh = lin / nchunk;
  const int t = threadIdx.x, cg = t % TPR, r0 = t / TPR;
  const int n0 = chunk * kStatChunk;
  const int nrows = min(kStatChunk, N - n0);
  // |x| of a finite f16 / bf16 value orders exactly like its sign-cleared
  // bit pattern read as an unsigned integer, so the maxima are taken on the
  // bit patterns, two channels per 32-bit lane, and decoded once at the end.
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mx[4];
#pragma unroll
  for (int j = 0; j < 4; j++) mx[j] = u16x2{0, 0};
  const uint16_t* base = V + in.head(bh, D) + (size_t)n0 * rs + cg * 8;
  auto max_row = [&](const v4i& raw) {
#pragma unroll
    for (int j = 0; j < 4; j++)
      mx[j] = __builtin_elementwise_max(mx[j], __builtin_bit_cast(u16x2, (unsigned)raw[j] & 0x7FFF7FFFu));
  };
  if (nrows == kStatChunk) {   // full chunk: issue every row load of this thread first
    constexpr int RPT = kStatChunk / RPP;
    v4i raw[RPT];
#pragma unroll
    for (int i = 0; i < RPT; i++) raw[i] = load16_in<STREAM>(base + (size_t)(r0 + i * RPP) * rs);
#pragma unroll
    for (int i = 0; i < RPT; i++) max_row(raw[i]);
  } else {
    for (int r = r0; r < nrows; r += RPP) max_row(*(const v4i*)(base + (size_t)r * rs));
  }
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; e++) s[e] = load_h(mx[e >> 1][e & 1], is_bf16);
#pragma unroll
  for (int e = 0; e < 8; e++) red[r0][cg * 8 + e] = s[e];
  __syncthreads();
  for (int c = t; c < D; c += 256) {
    float m = 0.0f;
    for (int r = 0; r < RPP; r++) m = fmaxf(m, red[r][c]);
    partial[((size_t)bh * nchunk + chunk) * D + c] = m;
  }
}
template <int D>
__global__ __launch_bounds__(256) void v_colmax_kernel(const uint16_t* __restrict__ V, int is_bf16, InRows in,
                                                        int nchunk, float* __restrict__ partial) {
  __shared__ float red[256 / (D / 8)][D];
  v_colmax_chunk<D>(V, is_bf16, in, nchunk, partial, blockIdx.x, red);
}

// scale_c = a_c / 448, r_c = 448 / a_c (0 and 0 when a_c < 2^-120).
// Grid: BH * D/16; a block of 256 = 16 channels x 16 chunk lanes.
__device__ __forceinline__ void v_scale_group(const float* __restrict__ partial, int nchunk, int D,
                                              float* __restrict__ v_scale, float* __restrict__ v_recip, int lin,
                                              float (*red)[16]) {
  const int ng = D / 16, g = lin % ng, bh = lin / ng;
  const int cl = threadIdx.x & 15, j = threadIdx.x >> 4;
  const int c = g * 16 + cl;
  float a = 0.0f;
  for (int ch = j; ch < nchunk; ch += 16) a = fmaxf(a, partial[((size_t)bh * nchunk + ch) * D + c]);
  red[j][cl] = a;
  __syncthreads();
  if (threadIdx.x < 16) {
    float m = 0.0f;
    for (int k = 0; k < 16; k++) m = fmaxf(m, red[k][threadIdx.x]);
    const bool zero = !(m >= 0x1p-120f);
    const size_t o = (size_t)bh * D + g * 16 + threadIdx.x;
    v_scale[o] = zero ? 0.0f : m / 448.0f;
    v_recip[o] = zero ? 0.0f : 448.0f / m;
  }
}
__global__ __launch_bounds__(256) void v_scale_kernel(const float* __restrict__ partial, int nchunk, int D,
                                                       float* __restrict__ v_scale, float* __restrict__ v_recip) {
  __shared__ float red[16][16];
  v_scale_group(partial, nchunk, D, v_scale, v_recip, blockIdx.x, red);
}

// ---------------------------------------------------------------------------
// FP8 codes of one KV tile of 64 tokens, written channel-major: the 64 codes of
// channel c are contiguous (the layout the attention kernel stages into LDS).
// code = e4m3(clamp(rn(v * r_c), +-448)), round to nearest even; zero channels
// and tokens at or past N (padding of the last tile) give code 0.  A thread converts 4 consecutive tokens x 8 channels and packs
// each channel's 4 codes into one dword, so the transpose happens in registers
// and every channel row is written as 16 consecutive dwords.
// Grid: BH * P/64.  Block: 16 * D/8 threads.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void v_quant_tile(const uint16_t* __restrict__ V, int is_bf16, InRows in,
                                             const float* __restrict__ v_recip, uint8_t* __restrict__ v_codes,
                                             int lin, int t) {
  const int ntile = in.P / kKTile;
  const size_t rs = in.stride(D);
  const int tile = lin % ntile, bh = lin / ntile;
  const int cg = t >> 4, tg = t & 15;   // channels 8cg.., tokens 4tg..4tg+3
  const uint16_t* src = V + in.head(bh, D) + 8 * cg;   // channel group of this head; rows added below
  const v4f r0 = *(const v4f*)(v_recip + (size_t)bh * D + 8 * cg);
  const v4f r1 = *(const v4f*)(v_recip + (size_t)bh * D + 8 * cg + 4);
  float r[8];
#pragma unroll
  for (int e = 0; e < 4; e++) { r[e] = r0[e]; r[e + 4] = r1[e]; }
  float y[4][8];
  const int tok0 = tile * kKTile + 4 * tg;   // this thread's first token
#pragma unroll
  for (int i = 0; i < 4; i++) {
    // a token past N reads the last real token and then counts as zero
    v4i raw = *(const v4i*)(src + (size_t)min(tok0 + i, in.N - 1) * rs);
    if (tok0 + i >= in.N) raw = v4i{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; e++) y[i][e] = fminf(fmaxf(half_of(raw, e, is_bf16) * r[e], -448.0f), 448.0f);
  }
  uint8_t* dst = v_codes + ((size_t)bh * ntile + tile) * (size_t)(D * kKTile) + (size_t)(8 * cg) * kKTile + 4 * tg;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0][e], y[1][e], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2][e], y[3][e], w, true);
    __builtin_nontemporal_store(r[e] == 0.0f ? 0 : w, (int*)(dst + (size_t)e * kKTile));
  }
}
template <int D>
__global__ __launch_bounds__(16 * D / 8) void v_quant_kernel(const uint16_t* __restrict__ V, int is_bf16, InRows in,
                                                              const float* __restrict__ v_recip,
                                                              uint8_t* __restrict__ v_codes) {
  v_quant_tile<D>(V, is_bf16, in, v_recip, v_codes, blockIdx.x, threadIdx.x);
}

// ---------------------------------------------------------------------------
// quantize_qkv: the two calls above in three launches instead of six (the
// same device functions and arithmetic, so the same bits): pass 1 = Q blocks,
// K channel sums and V channel maxima; finalize = K means and V scales;
// pass 2 = V tiles, then smoothed K blocks (V was read last).  Each workgroup
// takes one item of one of the parts by its index range.  When K and V
// together are not much larger than the last-level cache (CACHED), pass 1
// reads them with ordinary loads so that pass 2 finds part of them there;
// otherwise with streaming loads (measured: 4-6% faster at 268 MB and 134 MB
// of K and V, 1% slower at 402 MB).
// ---------------------------------------------------------------------------
template <int D, int BLKQ, bool CACHED>
__global__ __launch_bounds__(256) void qkv_pass1_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V, int is_bf16, InRows qin,
                                                         InRows kin, int nq, int nk, int nchunk,
                                                         int8_t* __restrict__ q_codes, float* __restrict__ q_scale,
                                                         long long* __restrict__ ksum, float* __restrict__ vmax) {
  __shared__ long long red[256 / (D / 8)][D];   // K sums; V maxima use the first half as floats
  __shared__ float red4[4];
  const int b = blockIdx.x;
  if (b < nq) quant_block<D, BLKQ, false>(Q, is_bf16, qin, nullptr, q_codes, q_scale, b, red4);
  else if (b < nq + nk) k_colsum<D, !CACHED>(K, is_bf16, kin, nchunk, b - nq, ksum, red);
  else v_colmax_chunk<D, !CACHED>(V, is_bf16, kin, nchunk, vmax, b - nq - nk, (float (*)[D])&red[0][0]);
}

__global__ __launch_bounds__(256) void qkv_finalize_kernel(const long long* __restrict__ ksum,
                                                            const float* __restrict__ vmax, int nchunk, int N, int D,
                                                            int ng, float* __restrict__ k_mean,
                                                            float* __restrict__ v_scale, float* __restrict__ v_recip) {
  __shared__ long long red[16][16];   // V scales use it as floats
  const int b = blockIdx.x;
  if (b < ng) k_mean_group(ksum, nchunk, N, D, k_mean, b, red);
  else v_scale_group(vmax, nchunk, D, v_scale, v_recip, b - ng, (float (*)[16])&red[0][0]);
}

// pass 2: V tiles (one per workgroup at d = 128; two per workgroup of 256
// threads at d = 64, whose tiles take 128 threads), then nkq workgroups of
// smoothed K blocks
template <int D, int BLKK>
__global__ __launch_bounds__(256) void qkv_pass2_kernel(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                         int is_bf16, InRows kin, int nkq, int ntiles,
                                                         const float* __restrict__ k_mean, int8_t* __restrict__ k_codes,
                                                         float* __restrict__ k_scale, const float* __restrict__ v_recip,
                                                         uint8_t* __restrict__ v_codes) {
  __shared__ float red4[4];
  constexpr int TPT = 16 * D / 8;   // threads per V tile
  const int nvw = (ntiles + 256 / TPT - 1) / (256 / TPT);
  const int b = blockIdx.x;
  if (b >= nvw) {
    quant_block<D, BLKK, true>(K, is_bf16, kin, k_mean, k_codes, k_scale, b - nvw, red4);
  } else {
    const int tile = b * (256 / TPT) + (int)threadIdx.x / TPT;
    if (tile < ntiles) v_quant_tile<D>(V, is_bf16, kin, v_recip, v_codes, tile, (int)threadIdx.x % TPT);
  }
}

// ---------------------------------------------------------------------------
// 4-bit Q / K: E2M1 values in blocks of 32 channels of a token row, one
// power-of-two scale per block: E = floor(log2(max|x|)) - 2 clamped to
// [-127, 127] (stored as the byte E + 127), values E2M1(x / 2^E) rounded to
// nearest with ties to the even code, saturating at 6; an all-zero block gets
// scale byte 0.  Codes are packed two per byte (even channel in the low
// nibble), rows of d/2 bytes, padded with zero rows like the INT8 codes.
// One thread per (row, block).  SMOOTH: x = K - mean (fp32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ unsigned e2m1_code(float x) {
  const float y = fabsf(x);
  // thresholds between consecutive magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; at a
  // midpoint the code with the even last bit wins (strict or non-strict test)
  const unsigned m = (unsigned)(y > 0.25f) + (unsigned)(y >= 0.75f) + (unsigned)(y > 1.25f) +
                     (unsigned)(y >= 1.75f) + (unsigned)(y > 2.5f) + (unsigned)(y >= 3.5f) + (unsigned)(y > 5.0f);
  return m | ((__float_as_uint(x) >> 28) & 8u);
}

// One token row of d channels in blocks of 32, each with one power-of-two
// scale: E2M1 codes (E = ilogb(max) - 2).  MEAN: 0 none, 1 one mean per
// head (K), 2 one per block of 32 rows (Q smoothing; mean [BH, P/32, d]).
template <int D, int MEAN>
__global__ __launch_bounds__(256) void quant4_kernel(const uint16_t* __restrict__ X, int is_bf16, InRows in, int BH,
                                                     const float* __restrict__ mean, uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scale) {
  constexpr int NB = D / 32;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)BH * in.P * NB) return;
  const int b = (int)(gid % NB);
  const long long rowid = gid / NB;
  const int n = (int)(rowid % in.P), bh = (int)(rowid / in.P);
  float x[32];
  if (n < in.N) {
    const uint16_t* src = X + in.head(bh, D) + (size_t)n * in.stride(D) + 32 * b;
#pragma unroll
    for (int l = 0; l < 4; l++) {
      const v4i raw = *(const v4i*)(src + 8 * l);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        float v = half_of(raw, e, is_bf16);
        if (MEAN == 1) v = v - mean[(size_t)bh * D + 32 * b + 8 * l + e];
        if (MEAN == 2) v = v - mean[((size_t)bh * (in.P / 32) + n / 32) * D + 32 * b + 8 * l + e];
        x[8 * l + e] = v;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; k++) x[k] = 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; k++) a = fmaxf(a, fabsf(x[k]));
  unsigned sbyte = 0;
  v4i packed = {0, 0, 0, 0};
  if (a != 0.0f) {
    const int e = min(max(ilogbf(a) - 2, -127), 127);
    sbyte = (unsigned)(e + 127);
#pragma unroll
    for (int w = 0; w < 4; w++) {
      unsigned word = 0;
#pragma unroll
      for (int k = 0; k < 8; k++) word |= e2m1_code(ldexpf(x[8 * w + k], -e)) << (4 * k);
      packed[w] = (int)word;
    }
  }
  *(v4i*)(codes + (size_t)rowid * (D / 2) + 16 * b) = packed;
  scale[(size_t)rowid * NB + b] = (uint8_t)sbyte;
}

// Q smoothing, the K of the mean's term: the smoothed K in INT8 blocks of
// one KV tile (64 keys) x d channels, one power-of-two scale each (exponent
// bytes [BH, P/64]).
template <int D>
__global__ __launch_bounds__(256) void k8_quant_kernel(const uint16_t* __restrict__ K, int is_bf16, InRows kin,
                                                       const float* __restrict__ k_mean, int8_t* __restrict__ k8_codes,
                                                       uint8_t* __restrict__ k8_scale) {
  __shared__ float red4[4];
  quant_block<D, kKTile, true, true>(K, is_bf16, kin, k_mean, k8_codes, k8_scale, blockIdx.x, red4);
}

// Block means of Q for smoothing: one workgroup per (head, block of 32 query
// rows), one thread per channel.  The mean is the fp64 sum of the block's
// rows in ascending order over the number of rows (the last block may be
// short), rounded to fp32; padding blocks (past Nq) get 0.  It is written as
// fp32 and as INT8 codes with one power-of-two scale over the d channels
// (int8_pow2_exponent; exponent byte e + 127).
template <int D>
__global__ __launch_bounds__(D) void q_mean_kernel(const uint16_t* __restrict__ X, int is_bf16, InRows in,
                                                   float* __restrict__ q_mean, int8_t* __restrict__ qm_codes,
                                                   uint8_t* __restrict__ qm_scale) {
  const int nb = in.P / 32;
  const int blk = blockIdx.x % nb, bh = blockIdx.x / nb, c = threadIdx.x;
  const int n0 = 32 * blk, n = min(32, in.N - n0);
  // the block's rows into LDS with 16-byte loads (32 rows x d/8 chunks, d threads)
  constexpr int RW = D + 2;
  __shared__ uint16_t rows[32 * RW];
  const uint16_t* src = X + in.head(bh, D) + (size_t)max(n0, 0) * in.stride(D);
#pragma unroll
  for (int l = 0; l < 4; l++) {
    const int ch = l * D + c, r = ch / (D / 8), c8 = ch % (D / 8);
    v4i raw = {0, 0, 0, 0};
    if (r < n) raw = *(const v4i*)(src + (size_t)r * in.stride(D) + 8 * c8);
#pragma unroll
    for (int e = 0; e < 4; e++) {
      rows[r * RW + 8 * c8 + 2 * e] = (uint16_t)((unsigned)raw[e] & 0xFFFFu);
      rows[r * RW + 8 * c8 + 2 * e + 1] = (uint16_t)((unsigned)raw[e] >> 16);
    }
  }
  __syncthreads();
  float qm = 0.0f;
  if (n > 0) {
    double sum = 0.0;
    for (int i = 0; i < n; i++) sum += (double)load_h(rows[i * RW + c], is_bf16);   // ascending rows
    qm = (float)(sum / n);
  }
  float a = fabsf(qm);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a = fmaxf(a, __shfl_xor(a, o));   // max over the wave's 64 channels
  if constexpr (D > 64) {
    __shared__ float red[D / 64];
    if ((c & 63) == 0) red[c >> 6] = a;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < D / 64; w++) a = fmaxf(a, red[w]);
  }
  const int e = int8_pow2_exponent(a);
  const float y = fminf(fmaxf(__builtin_rintf(ldexpf(qm, -e)), -127.0f), 127.0f);
  const size_t r = (size_t)bh * nb + blk;
  q_mean[r * D + c] = qm;
  qm_codes[r * D + c] = (int8_t)(int)y;
  if (c == 0) qm_scale[r] = (uint8_t)(e + 127);
}

// FP4 V (MXFP4): a workgroup of 256 threads takes 256 / (2 d) KV tiles (one
// at d = 128, two at d = 64).  The tile's 64 token rows are read with
// 16-byte loads into LDS (rows padded by 2 values), then thread pair 2c,
// 2c + 1 takes channel c, each thread one block g of 32 tokens: the shared
// exponent E = ilogb(max) - 2 clamped to [-127, 127] (an all-zero block: byte
// 0) and the E2M1 codes of v / 2^E, written as the 16-byte half g of the
// channel's 32-byte row (so a wave's stores are contiguous); tokens past N
// count as zero.  Scales go to the per-tile array permuted for the
// attention kernel's per-lane loads.
template <int D>
__global__ __launch_bounds__(256) void v4_quant_kernel(const uint16_t* __restrict__ V, int is_bf16, InRows in, int BH,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ scale) {
  constexpr int TPT = 2 * D;            // threads per tile
  constexpr int NT = 256 / TPT;         // tiles per workgroup
  constexpr int RW = D + 2;             // LDS row of one token (u16), padded
  __shared__ uint16_t tileb[NT][kKTile * RW];
  const int nkt = in.P / kKTile;
  const int sub = (int)threadIdx.x / TPT, t_in = (int)threadIdx.x % TPT;
  const long long tg = (long long)blockIdx.x * NT + sub;          // flat (head, tile)
  const bool live = tg < (long long)BH * nkt;
  const int t = live ? (int)(tg % nkt) : 0, bh = live ? (int)(tg / nkt) : 0;
  const uint16_t* src = V + in.head(bh, D);
  const size_t stride = in.stride(D);
  // 64 rows x d values = 8 d chunks of 8 values; TPT = 2 d threads load 4 each
#pragma unroll
  for (int l = 0; l < 4; l++) {
    const int ch = l * TPT + t_in;
    const int row = ch / (D / 8), c8 = ch % (D / 8);
    const int tok = t * kKTile + row;
    v4i raw = {0, 0, 0, 0};
    if (live && tok < in.N) raw = load16_in<true>(src + (size_t)tok * stride + 8 * c8);
    uint16_t* dst = &tileb[sub][row * RW + 8 * c8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
      dst[2 * e] = (uint16_t)((unsigned)raw[e] & 0xFFFFu);
      dst[2 * e + 1] = (uint16_t)((unsigned)raw[e] >> 16);
    }
  }
  __syncthreads();
  if (!live) return;
  const int c = t_in >> 1, g = t_in & 1;
  float x[32];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) {
    x[i] = load_h(tileb[sub][(32 * g + i) * RW + c], is_bf16);
    a = fmaxf(a, fabsf(x[i]));
  }
  v4i packed = {0, 0, 0, 0};
  unsigned sbyte = 0;
  if (a != 0.0f) {
    const int e = min(max(ilogbf(a) - 2, -127), 127);
    sbyte = (unsigned)(e + 127);
#pragma unroll
    for (int w = 0; w < 4; w++) {
      unsigned word = 0;
#pragma unroll
      for (int k = 0; k < 8; k++) word |= e2m1_code(ldexpf(x[8 * w + k], -e)) << (4 * k);
      packed[w] = (int)word;
    }
  }
  __builtin_nontemporal_store(packed, (v4i*)(codes + ((size_t)(bh * nkt + t) * D + c) * 32 + 16 * g));
  scale[(size_t)(bh * nkt + t) * 64 * (D / 32) + (32 * g + c % 32) * (D / 32) + c / 32] = (uint8_t)sbyte;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
static inline int stat_chunks(int N) { return (N + kStatChunk - 1) / kStatChunk; }
static inline int round_up(int n, int m) { return (n + m - 1) / m * m; }

template <int D, int BLKQ>
static int launch_qk_pass1(const QuantQKArgs& a, InRows qin, InRows kin, int nchunk, long long* partial,
                           bool with_q, bool with_k, hipStream_t st) {
  const int nq = with_q ? a.B * a.Hq * (qin.P / BLKQ) / blocks_per_wg<D, BLKQ>() : 0;
  const int grid1 = nq + (with_k ? a.B * a.Hkv * nchunk : 0);
  hipLaunchKernelGGL((qk_pass1_kernel<D, BLKQ>), dim3(grid1), dim3(256), 0, st, (const uint16_t*)a.Q,
                     (const uint16_t*)a.K, a.is_bf16, qin, kin, nq, nchunk, a.q_codes, a.q_scale, partial);
  return nq;
}

template <int D, int BLKK>
static void launch_k_quant(const QuantQKArgs& a, InRows kin, hipStream_t st) {
  const int grid = a.B * a.Hkv * (kin.P / BLKK) / blocks_per_wg<D, BLKK>();
  hipLaunchKernelGGL((k_quant_kernel<D, BLKK>), dim3(grid), dim3(256), 0, st, (const uint16_t*)a.K, a.is_bf16, kin,
                     (const float*)a.k_mean, a.k_codes, a.k_scale);
}

template <int D>
static void launch_qk_d(const QuantQKArgs& a, hipStream_t st, bool with_q, bool with_k) {
  const int BHkv = a.B * a.Hkv;
  const int nchunk = stat_chunks(a.Nkv);
  long long* partial = (long long*)a.workspace;
  const InRows qin{a.Hq, a.Nq, round_up(a.Nq, kQTile), a.nhd}, kin{a.Hkv, a.Nkv, round_up(a.Nkv, kKTile), a.nhd};
  if (a.blk_q == 128) launch_qk_pass1<D, 128>(a, qin, kin, nchunk, partial, with_q, with_k, st);
  else if (a.blk_q == 64) launch_qk_pass1<D, 64>(a, qin, kin, nchunk, partial, with_q, with_k, st);
  else launch_qk_pass1<D, 32>(a, qin, kin, nchunk, partial, with_q, with_k, st);
  if (!with_k) return;
  hipLaunchKernelGGL(k_mean_kernel, dim3(BHkv * (D / 16)), dim3(256), 0, st, (const long long*)partial, nchunk, a.Nkv,
                     D, a.k_mean);
  if (a.blk_k == 64) launch_k_quant<D, 64>(a, kin, st);
  else if (a.blk_k == 32) launch_k_quant<D, 32>(a, kin, st);
  else launch_k_quant<D, 16>(a, kin, st);
}

void launch_quantize_qk(const QuantQKArgs& a, hipStream_t st, bool with_q, bool with_k) {
  if (a.d == 128) launch_qk_d<128>(a, st, with_q, with_k);
  else launch_qk_d<64>(a, st, with_q, with_k);
}

template <int D>
static void launch_v_d(const QuantVArgs& a, hipStream_t st) {
  const int BH = a.B * a.H;
  const int nchunk = stat_chunks(a.N);
  float* partial = (float*)a.workspace;
  float* recip = partial + (size_t)BH * nchunk * D;
  const InRows in{a.H, a.N, round_up(a.N, kKTile), a.nhd};
  hipLaunchKernelGGL(v_colmax_kernel<D>, dim3(nchunk * BH), dim3(256), 0, st, (const uint16_t*)a.V, a.is_bf16, in,
                     nchunk, partial);
  hipLaunchKernelGGL(v_scale_kernel, dim3(BH * (D / 16)), dim3(256), 0, st, (const float*)partial, nchunk, D,
                     a.v_scale, recip);
  hipLaunchKernelGGL(v_quant_kernel<D>, dim3(in.P / kKTile * BH), dim3(16 * D / 8), 0, st, (const uint16_t*)a.V,
                     a.is_bf16, in, (const float*)recip, a.v_codes);
}

template <int D, int BLKQ, int BLKK>
static void launch_qkv_d(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t st) {
  const int BHkv = a.B * a.Hkv;
  const int nchunk = stat_chunks(a.Nkv);
  long long* ksum = (long long*)a.workspace;
  float* vmax = (float*)v.workspace;
  float* recip = vmax + (size_t)BHkv * nchunk * D;
  const InRows qin{a.Hq, a.Nq, round_up(a.Nq, kQTile), a.nhd}, kin{a.Hkv, a.Nkv, round_up(a.Nkv, kKTile), a.nhd};
  const int nq = a.B * a.Hq * (qin.P / BLKQ) / blocks_per_wg<D, BLKQ>();
  const int nk = BHkv * nchunk;
  // K and V of at most 320 MB together: ordinary loads in pass 1 (the last-level cache is 256 MB;
  // measured faster at 268 MB, slower at 402 MB)
  const bool cached = 2.0 * 2.0 * BHkv * a.Nkv * D <= 320.0 * (1 << 20);
  if (cached)
    hipLaunchKernelGGL((qkv_pass1_kernel<D, BLKQ, true>), dim3(nq + 2 * nk), dim3(256), 0, st, (const uint16_t*)a.Q,
                       (const uint16_t*)a.K, (const uint16_t*)v.V, a.is_bf16, qin, kin, nq, nk, nchunk, a.q_codes,
                       a.q_scale, ksum, vmax);
  else
    hipLaunchKernelGGL((qkv_pass1_kernel<D, BLKQ, false>), dim3(nq + 2 * nk), dim3(256), 0, st, (const uint16_t*)a.Q,
                       (const uint16_t*)a.K, (const uint16_t*)v.V, a.is_bf16, qin, kin, nq, nk, nchunk, a.q_codes,
                       a.q_scale, ksum, vmax);
  const int ng = BHkv * (D / 16);
  hipLaunchKernelGGL(qkv_finalize_kernel, dim3(2 * ng), dim3(256), 0, st, (const long long*)ksum, (const float*)vmax,
                     nchunk, a.Nkv, D, ng, a.k_mean, v.v_scale, recip);
  const int nkq = BHkv * (kin.P / BLKK) / blocks_per_wg<D, BLKK>();
  const int ntiles = BHkv * (kin.P / kKTile);
  constexpr int TPW = 256 / (16 * D / 8);   // V tiles per workgroup
  hipLaunchKernelGGL((qkv_pass2_kernel<D, BLKK>), dim3(nkq + (ntiles + TPW - 1) / TPW), dim3(256), 0, st,
                     (const uint16_t*)a.K, (const uint16_t*)v.V, a.is_bf16, kin, nkq, ntiles, (const float*)a.k_mean,
                     a.k_codes, a.k_scale, (const float*)recip, v.v_codes);
}

template <int D, int BLKQ>
static void launch_qkv_q(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t st) {
  if (a.blk_k == 64) launch_qkv_d<D, BLKQ, 64>(a, v, st);
  else if (a.blk_k == 32) launch_qkv_d<D, BLKQ, 32>(a, v, st);
  else launch_qkv_d<D, BLKQ, 16>(a, v, st);
}
template <int D>
static void launch_qkv_dd(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t st) {
  if (a.blk_q == 128) launch_qkv_q<D, 128>(a, v, st);
  else if (a.blk_q == 64) launch_qkv_q<D, 64>(a, v, st);
  else launch_qkv_q<D, 32>(a, v, st);
}

void launch_quantize_qkv(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t st) {
  if (a.d == 128) launch_qkv_dd<128>(a, v, st);
  else launch_qkv_dd<64>(a, v, st);
}

void launch_quantize_v(const QuantVArgs& a, hipStream_t st) {
  if (a.d == 128) launch_v_d<128>(a, st);
  else launch_v_d<64>(a, st);
}

template <int D>
static void launch_qk4_d(const Quant4Args& a, hipStream_t st) {
  const int BHq = a.B * a.Hq, BHkv = a.B * a.Hkv;
  const int nchunk = stat_chunks(a.Nkv);
  long long* partial = (long long*)a.workspace;
  const InRows qin{a.Hq, a.Nq, round_up(a.Nq, kQTile), a.nhd}, kin{a.Hkv, a.Nkv, round_up(a.Nkv, kKTile), a.nhd};
  // K column sums (the Q part of pass 1 is not launched), then the K mean
  hipLaunchKernelGGL((qk_pass1_kernel<D, 128>), dim3(BHkv * nchunk), dim3(256), 0, st, (const uint16_t*)nullptr,
                     (const uint16_t*)a.K, a.is_bf16, qin, kin, 0, nchunk, (int8_t*)nullptr, (float*)nullptr, partial);
  hipLaunchKernelGGL(k_mean_kernel, dim3(BHkv * (D / 16)), dim3(256), 0, st, (const long long*)partial, nchunk, a.Nkv,
                     D, a.k_mean);
  const long long tq = (long long)BHq * qin.P * (D / 32), tk = (long long)BHkv * kin.P * (D / 32);
  const dim3 gq((unsigned)((tq + 255) / 256)), gk((unsigned)((tk + 255) / 256));
  if (a.q_mean) {   // Q smoothing: block means, smoothed Q, and K also in INT8 blocks for the mean's term
    hipLaunchKernelGGL(q_mean_kernel<D>, dim3(BHq * (qin.P / 32)), dim3(D), 0, st, (const uint16_t*)a.Q, a.is_bf16,
                       qin, a.q_mean, a.qm_codes, a.qm_scale);
    hipLaunchKernelGGL((quant4_kernel<D, 2>), gq, dim3(256), 0, st, (const uint16_t*)a.Q, a.is_bf16, qin, BHq,
                       (const float*)a.q_mean, a.q4_codes, a.q4_scale);
    hipLaunchKernelGGL(k8_quant_kernel<D>, dim3(BHkv * (kin.P / kKTile)), dim3(256), 0, st, (const uint16_t*)a.K,
                       a.is_bf16, kin, (const float*)a.k_mean, a.k8_codes, a.k8_scale);
  } else {
    hipLaunchKernelGGL((quant4_kernel<D, 0>), gq, dim3(256), 0, st, (const uint16_t*)a.Q, a.is_bf16, qin, BHq,
                       (const float*)nullptr, a.q4_codes, a.q4_scale);
  }
  hipLaunchKernelGGL((quant4_kernel<D, 1>), gk, dim3(256), 0, st, (const uint16_t*)a.K, a.is_bf16, kin, BHkv,
                     (const float*)a.k_mean, a.k4_codes, a.k4_scale);
}

void launch_quantize_qk4(const Quant4Args& a, hipStream_t st) {
  if (a.d == 128) launch_qk4_d<128>(a, st);
  else launch_qk4_d<64>(a, st);
}

void launch_quantize_v4(const QuantV4Args& a, hipStream_t st) {
  const InRows in{a.H, a.N, round_up(a.N, kKTile), a.nhd};
  const int BH = a.B * a.H;
  const long long tiles = (long long)BH * (in.P / kKTile);
  const int nt = 256 / (2 * a.d);   // tiles per workgroup
  const dim3 g((unsigned)((tiles + nt - 1) / nt));
  if (a.d == 128)
    hipLaunchKernelGGL(v4_quant_kernel<128>, g, dim3(256), 0, st, (const uint16_t*)a.V, a.is_bf16, in, BH, a.v4_codes,
                       a.v4_scale);
  else
    hipLaunchKernelGGL(v4_quant_kernel<64>, g, dim3(256), 0, st, (const uint16_t*)a.V, a.is_bf16, in, BH, a.v4_codes,
                       a.v4_scale);
}

size_t quantize_qk_workspace(int BHkv, int Nkv, int d) {
  return (size_t)BHkv * stat_chunks(Nkv) * d * sizeof(long long);
}
size_t quantize_v_workspace(int BH, int N, int d) {
  return ((size_t)BH * stat_chunks(N) * d + (size_t)BH * d) * sizeof(float);
}

}  // namespace sage
