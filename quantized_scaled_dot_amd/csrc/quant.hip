// Quantization kernels (gfx950): K smoothing + INT8 per-block Q/K, FP8 V with
// per-channel scales.  All passes are HBM-bound streams with 16-byte coalesced
// loads; every reduction is order-free (int64 sums, max), so results do not
// depend on launch geometry.
#include "common.h"
#include "launch.h"

namespace sage {

// ---------------------------------------------------------------------------
// Per-channel fixed-point sums of K over one chunk of kStatChunk tokens:
// s_c = sum_t trunc(clamp(k, +-2^20) * 2^24) (int64, exact).
// Grid: (nchunk * BH).  Block: 256 threads, each owning 8 channels of every
// RPP-th token of the chunk.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_colsum_kernel(const uint16_t* __restrict__ K, int is_bf16, int N,
                                                        int nchunk, long long* __restrict__ partial) {
  constexpr int TPR = D / 8;        // threads per token row
  constexpr int RPP = 256 / TPR;    // token rows per pass
  const int chunk = blockIdx.x % nchunk, bh = blockIdx.x / nchunk;
  const int t = threadIdx.x, cg = t % TPR, r0 = t / TPR;
  const int n0 = chunk * kStatChunk;
  const int nrows = min(kStatChunk, N - n0);
  long long s[8];
#pragma unroll
  for (int e = 0; e < 8; e++) s[e] = 0;
  const uint16_t* base = K + ((size_t)bh * N + n0) * D + cg * 8;
  for (int r = r0; r < nrows; r += RPP) {
    v4i raw = *(const v4i*)(base + (size_t)r * D);
#pragma unroll
    for (int e = 0; e < 8; e++) {
      float x = load_h((uint16_t)((unsigned)raw[e >> 1] >> (16 * (e & 1))), is_bf16);
      x = fminf(fmaxf(x, -1048576.0f), 1048576.0f);
      s[e] += (long long)(x * 16777216.0f);   // exact product; truncation toward zero
    }
  }
  __shared__ long long red[RPP][D];
#pragma unroll
  for (int e = 0; e < 8; e++) red[r0][cg * 8 + e] = s[e];
  __syncthreads();
  for (int c = t; c < D; c += 256) {
    long long tot = 0;
    for (int r = 0; r < RPP; r++) tot += red[r][c];
    partial[((size_t)bh * nchunk + chunk) * D + c] = tot;
  }
}

// mean_c = fp32(fp64(sum_chunks s_c) * 2^-24 / N).  Grid: BH.  Block: 128.
__global__ __launch_bounds__(128) void k_mean_kernel(const long long* __restrict__ partial, int nchunk, int N, int D,
                                                      float* __restrict__ k_mean) {
  const int bh = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    long long s = 0;
    for (int ch = 0; ch < nchunk; ch++) s += partial[((size_t)bh * nchunk + ch) * D + c];
    k_mean[(size_t)bh * D + c] = (float)(((double)s * 0x1p-24) / (double)N);
  }
}

__device__ __forceinline__ float block_max_256(float a, float* red4) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red4[threadIdx.x >> 6] = a;
  __syncthreads();
  return fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]));
}

// ---------------------------------------------------------------------------
// Symmetric INT8 quantization of one block of BLK tokens x D channels:
// a = max|x| (x = K - mean when SMOOTH), scale = a/127, r = 127/a,
// code = rint(x * r) in [-127, 127]; a < 2^-120 gives scale 0 and zero codes.
// Grid: (nblk * BH).  Block: 256 threads holding BLK*D/256 values each.
// ---------------------------------------------------------------------------
template <int D, int BLK, bool SMOOTH>
__global__ __launch_bounds__(256) void quant_block_kernel(const uint16_t* __restrict__ X, int is_bf16, int N,
                                                           const float* __restrict__ mean, int8_t* __restrict__ codes,
                                                           float* __restrict__ scale) {
  constexpr int EPT = BLK * D / 256;   // values per thread
  constexpr int LPT = EPT / 8;         // 16-byte loads per thread
  const int nblk = N / BLK;
  const int blk = blockIdx.x % nblk, bh = blockIdx.x / nblk;
  const int t = threadIdx.x;
  const size_t off = ((size_t)bh * N + (size_t)blk * BLK) * D;
  const uint16_t* src = X + off;
  float x[EPT];
  float a = 0.0f;
#pragma unroll
  for (int l = 0; l < LPT; l++) {
    const int ch = l * 256 + t;   // 16-byte chunk index within the block
    v4i raw = *(const v4i*)(src + (size_t)ch * 8);
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
      float v = load_h((uint16_t)((unsigned)raw[e >> 1] >> (16 * (e & 1))), is_bf16);
      if (SMOOTH) v = v - mu[e];
      x[l * 8 + e] = v;
      a = fmaxf(a, fabsf(v));
    }
  }
  __shared__ float red4[4];
  a = block_max_256(a, red4);
  const bool zero = !(a >= 0x1p-120f);
  const float dl = zero ? 0.0f : a / 127.0f;
  const float r = zero ? 0.0f : 127.0f / a;
  int8_t* dst = codes + off;
#pragma unroll
  for (int l = 0; l < LPT; l++) {
    const int ch = l * 256 + t;
    unsigned w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; e++) {
      float y = __builtin_rintf(x[l * 8 + e] * r);
      y = fminf(fmaxf(y, -127.0f), 127.0f);
      w[e >> 2] |= ((unsigned)(int)y & 0xFFu) << (8 * (e & 3));
    }
    v2i pk = {(int)w[0], (int)w[1]};
    *(v2i*)(dst + (size_t)ch * 8) = pk;
  }
  if (t == 0) scale[(size_t)bh * nblk + blk] = dl;
}

// ---------------------------------------------------------------------------
// Per-channel maxima of |V| over one chunk of tokens.  Grid: (nchunk * BH).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void v_colmax_kernel(const uint16_t* __restrict__ V, int is_bf16, int N, int nchunk,
                                                        float* __restrict__ partial) {
  constexpr int TPR = D / 8;
  constexpr int RPP = 256 / TPR;
  const int chunk = blockIdx.x % nchunk, bh = blockIdx.x / nchunk;
  const int t = threadIdx.x, cg = t % TPR, r0 = t / TPR;
  const int n0 = chunk * kStatChunk;
  const int nrows = min(kStatChunk, N - n0);
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; e++) s[e] = 0.0f;
  const uint16_t* base = V + ((size_t)bh * N + n0) * D + cg * 8;
  for (int r = r0; r < nrows; r += RPP) {
    v4i raw = *(const v4i*)(base + (size_t)r * D);
#pragma unroll
    for (int e = 0; e < 8; e++)
      s[e] = fmaxf(s[e], fabsf(load_h((uint16_t)((unsigned)raw[e >> 1] >> (16 * (e & 1))), is_bf16)));
  }
  __shared__ float red[RPP][D];
#pragma unroll
  for (int e = 0; e < 8; e++) red[r0][cg * 8 + e] = s[e];
  __syncthreads();
  for (int c = t; c < D; c += 256) {
    float m = 0.0f;
    for (int r = 0; r < RPP; r++) m = fmaxf(m, red[r][c]);
    partial[((size_t)bh * nchunk + chunk) * D + c] = m;
  }
}

// scale_c = a_c / 448, r_c = 448 / a_c (0 and 0 when a_c < 2^-120).  Grid: BH.
__global__ __launch_bounds__(128) void v_scale_kernel(const float* __restrict__ partial, int nchunk, int D,
                                                       float* __restrict__ v_scale, float* __restrict__ v_recip) {
  const int bh = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float a = 0.0f;
    for (int ch = 0; ch < nchunk; ch++) a = fmaxf(a, partial[((size_t)bh * nchunk + ch) * D + c]);
    const bool zero = !(a >= 0x1p-120f);
    v_scale[(size_t)bh * D + c] = zero ? 0.0f : a / 448.0f;
    v_recip[(size_t)bh * D + c] = zero ? 0.0f : 448.0f / a;
  }
}

// ---------------------------------------------------------------------------
// FP8 codes of one KV tile of 64 tokens, written channel-major: the 64 codes of
// channel c are contiguous (the layout the attention kernel stages into LDS).
// code = e4m3(clamp(rn(v * r_c), +-448)), round to nearest even; zero channels
// give code 0.  Grid: (N/64 * BH).  Transposed through LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void v_quant_kernel(const uint16_t* __restrict__ V, int is_bf16, int N,
                                                       const float* __restrict__ v_recip, uint8_t* __restrict__ v_codes) {
  constexpr int ROW = kKTile + 16;   // padded LDS row: 64 codes + 16 bytes
  __shared__ __attribute__((aligned(16))) uint8_t sT[D * ROW];
  const int ntile = N / kKTile;
  const int tile = blockIdx.x % ntile, bh = blockIdx.x / ntile;
  const int t = threadIdx.x;
  const uint16_t* src = V + ((size_t)bh * N + (size_t)tile * kKTile) * D;
  constexpr int CHUNKS = kKTile * D / 8;
  for (int ch = t; ch < CHUNKS; ch += 256) {
    const int tok = ch / (D / 8), c0 = (ch % (D / 8)) * 8;
    v4i raw = *(const v4i*)(src + (size_t)ch * 8);
    v4f r0 = *(const v4f*)(v_recip + (size_t)bh * D + c0);
    v4f r1 = *(const v4f*)(v_recip + (size_t)bh * D + c0 + 4);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float r = e < 4 ? r0[e] : r1[e - 4];
      float v = load_h((uint16_t)((unsigned)raw[e >> 1] >> (16 * (e & 1))), is_bf16) * r;
      y[e] = fminf(fmaxf(v, -448.0f), 448.0f);
    }
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[e], y[e + 1], 0, false);
      const float ra = e < 4 ? r0[e] : r1[e - 4], rb = e < 4 ? r0[e + 1] : r1[e - 3];
      sT[(c0 + e) * ROW + tok] = ra == 0.0f ? 0 : (uint8_t)(pk & 0xFF);
      sT[(c0 + e + 1) * ROW + tok] = rb == 0.0f ? 0 : (uint8_t)((pk >> 8) & 0xFF);
    }
  }
  __syncthreads();
  uint8_t* dst = v_codes + ((size_t)bh * ntile + tile) * (size_t)(D * kKTile);
  for (int ch = t; ch < D * (kKTile / 16); ch += 256) {
    const int c = ch / (kKTile / 16), part = ch % (kKTile / 16);
    *(v4i*)(dst + (size_t)c * kKTile + part * 16) = *(const v4i*)(sT + c * ROW + part * 16);
  }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <int D>
static void launch_qk_d(const QuantQKArgs& a, hipStream_t st) {
  const int nchunk = (a.N + kStatChunk - 1) / kStatChunk;
  long long* partial = (long long*)a.workspace;
  hipLaunchKernelGGL(k_colsum_kernel<D>, dim3(nchunk * a.BH), dim3(256), 0, st, (const uint16_t*)a.K, a.is_bf16, a.N,
                     nchunk, partial);
  hipLaunchKernelGGL(k_mean_kernel, dim3(a.BH), dim3(128), 0, st, (const long long*)partial, nchunk, a.N, D, a.k_mean);
  if (a.blk_q == 128)
    hipLaunchKernelGGL((quant_block_kernel<D, 128, false>), dim3(a.N / 128 * a.BH), dim3(256), 0, st,
                       (const uint16_t*)a.Q, a.is_bf16, a.N, (const float*)nullptr, a.q_codes, a.q_scale);
  else
    hipLaunchKernelGGL((quant_block_kernel<D, 64, false>), dim3(a.N / 64 * a.BH), dim3(256), 0, st,
                       (const uint16_t*)a.Q, a.is_bf16, a.N, (const float*)nullptr, a.q_codes, a.q_scale);
  hipLaunchKernelGGL((quant_block_kernel<D, 64, true>), dim3(a.N / 64 * a.BH), dim3(256), 0, st, (const uint16_t*)a.K,
                     a.is_bf16, a.N, (const float*)a.k_mean, a.k_codes, a.k_scale);
}

void launch_quantize_qk(const QuantQKArgs& a, hipStream_t st) {
  if (a.d == 128) launch_qk_d<128>(a, st);
  else launch_qk_d<64>(a, st);
}

template <int D>
static void launch_v_d(const QuantVArgs& a, hipStream_t st) {
  const int nchunk = (a.N + kStatChunk - 1) / kStatChunk;
  float* partial = (float*)a.workspace;
  float* recip = partial + (size_t)a.BH * nchunk * D;
  hipLaunchKernelGGL(v_colmax_kernel<D>, dim3(nchunk * a.BH), dim3(256), 0, st, (const uint16_t*)a.V, a.is_bf16, a.N,
                     nchunk, partial);
  hipLaunchKernelGGL(v_scale_kernel, dim3(a.BH), dim3(128), 0, st, (const float*)partial, nchunk, D, a.v_scale, recip);
  hipLaunchKernelGGL(v_quant_kernel<D>, dim3(a.N / kKTile * a.BH), dim3(256), 0, st, (const uint16_t*)a.V, a.is_bf16,
                     a.N, (const float*)recip, a.v_codes);
}

void launch_quantize_v(const QuantVArgs& a, hipStream_t st) {
  if (a.d == 128) launch_v_d<128>(a, st);
  else launch_v_d<64>(a, st);
}

size_t quantize_qk_workspace(int BH, int N, int d) {
  const size_t nchunk = (size_t)(N + kStatChunk - 1) / kStatChunk;
  return (size_t)BH * nchunk * d * sizeof(long long);
}
size_t quantize_v_workspace(int BH, int N, int d) {
  const size_t nchunk = (size_t)(N + kStatChunk - 1) / kStatChunk;
  return ((size_t)BH * nchunk * d + (size_t)BH * d) * sizeof(float);
}

}  // namespace sage
