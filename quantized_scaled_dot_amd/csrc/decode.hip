// Decode: a few queries per sequence against a long quantized KV cache
// (gfx950).  The work is bound by reading the K/V codes once, so it is split
// over the keys: every wave takes one chunk of one K/V head and the 32-row
// group of query rows that read that head (the Hq/Hkv query heads times the
// Nq queries, packed), runs the same tiled online softmax and two-level FP8
// P~V as the attention kernel over its chunk from a fresh state, and writes
// (m, l, O_acc) per row.  A second kernel merges the chunks of each row in
// ascending order with the log-sum-exp rule and applies the V scales.
//
// Per wave and KV tile (64 keys), with the tile's K and V operands in registers:
//   S^T = K_tile . Q^T    2 x (d/32) v_mfma_i32_32x32x32_i8
//   softmax on the VALU (one lane per query row, the attention kernel's
//   arithmetic: exponent argument (B + S) c2 - K, row sum of the FP8 codes on
//   the matrix core)
//   O^T += V^T . P~^T     d/32 v_mfma_scale_f32_32x32x64_f8f6f4
// Waves share nothing and never synchronise with each other.
#include "common.h"
#include "launch.h"

namespace sage {

struct DecodeK {
  const int8_t* q_codes;
  const float* q_scale;
  const int8_t* k_codes;
  const float* k_scale;
  const uint8_t* v_codes;
  float* part;          // per unit: [32][D] O_acc, then [32] m, then [32] l
  int g, Nq, Nkv, off;  // g = Hq/Hkv; off = Nkv - Nq
  int nqp, nbq, blk_q;  // Q code rows per head, Q scales per head, Q block
  int nkt, nbk, lgk;    // KV tiles per head, K scales per head, log2 K block
  int causal;
  int R, nchunk, ctiles, units;   // row groups per K/V head, chunks, tiles per chunk, waves of work
  float s2;
};

template <int D>
constexpr size_t unit_floats() { return (size_t)32 * D + 64; }

// One wave = one unit of work (K/V head, group of 32 query rows, split).  The
// K/V operands go from global memory straight into registers, two tiles
// ahead of the one being computed (three register sets in rotation; no LDS,
// one wave per SIMD with the accumulation registers): 32 KB in flight per
// wave.  Lane (i, g) loads the 16-byte pieces its MFMA operands need: K rows
// of the tile in MFMA order (key k_lds_key(i) for the first 32 rows,
// k_lds_key(32 + i) for the second), bytes 16 g + 32 s; V channel rows
// 32 ct + i, keys 32 g .. 32 g + 31 (the tile is channel-major).
__device__ __forceinline__ v4i load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <int D, bool FINEK>
__global__ __launch_bounds__(256, 1) void decode_chunk_kernel(DecodeK p) {
  constexpr int KS = D / 32, CT = D / 32;
  constexpr int TILE = kKTile * D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, lg = lane >> 5;
  const v8i ones16 = rowsum_ones_operand(lane);
  const int unit = blockIdx.x * 4 + wave;
  if (unit >= p.units) return;   // whole wave; no barrier in this kernel
  const int chunk = unit % p.nchunk, rest = unit / p.nchunk;
  const int rg = rest % p.R, bhkv = rest / p.R;

  const int f = rg * 32 + li;
  const bool valid = f < p.g * p.Nq;
  const int qi = valid ? f % p.Nq : 0;
  const int bhq = bhkv * p.g + (valid ? f / p.Nq : 0);
  v4i qreg[KS];
  float dq = 0.0f;
#pragma unroll
  for (int s = 0; s < KS; s++) qreg[s] = v4i{0, 0, 0, 0};
  if (valid) {
    const int8_t* qp = p.q_codes + ((size_t)bhq * p.nqp + qi) * D + 16 * lg;
#pragma unroll
    for (int s = 0; s < KS; s++) qreg[s] = *(const v4i*)(qp + 32 * s);
    dq = p.q_scale[(size_t)bhq * p.nbq + qi / p.blk_q];
  }
  const int lastk = p.causal ? min(qi + p.off, p.Nkv - 1) : p.Nkv - 1;
  const int lastk0 = p.causal ? min(p.off, p.Nkv - 1) : p.Nkv - 1;

  // buffer loads: one resource per head, a per-lane offset, the tile as the
  // scalar offset and the rest as immediates (few address registers)
  const __amdgpu_buffer_rsrc_t rK = head_rsrc(p.k_codes + (size_t)bhkv * p.nkt * TILE, (uint32_t)(p.nkt * TILE));
  const __amdgpu_buffer_rsrc_t rV = head_rsrc(p.v_codes + (size_t)bhkv * p.nkt * TILE, (uint32_t)(p.nkt * TILE));
  const int ka_off = k_lds_key(li) * D + 16 * lg, kb_off = k_lds_key(32 + li) * D + 16 * lg;
  const int v_off = li * kKTile + 32 * lg;
  struct Ops {
    v4i ka[KS], kb[KS], va[CT], vb[CT];
    float ks0, ks1;
  };
  const float* kscale = p.k_scale + (size_t)bhkv * p.nbk;
  auto kidx = [&](int t, int h) { return FINEK ? (t * kKTile + 32 * lg + 16 * h) >> p.lgk : t; };
  auto load = [&](int t, Ops& o) {
    const int tb = t * TILE;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      o.ka[s] = load16(rK, ka_off + 32 * s, tb);
      o.kb[s] = load16(rK, kb_off + 32 * s, tb);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ct++) {
      o.va[ct] = load16(rV, v_off + ct * 32 * kKTile, tb);
      o.vb[ct] = load16(rV, v_off + ct * 32 * kKTile + 16, tb);
    }
    o.ks0 = kscale[kidx(t, 0)];
    o.ks1 = FINEK ? kscale[kidx(t, 1)] : o.ks0;
  };

  v16f oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++)
#pragma unroll
    for (int e = 0; e < 16; e++) oacc[ct][e] = 0.0f;
  float m = -1e30f, lpart = 0.0f;

  auto compute = [&](int t, const Ops& o) {
    v16i sc0 = v16i{}, sc1 = v16i{};
#pragma unroll
    for (int s = 0; s < KS; s++) {
      sc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.ka[s], qreg[s], sc0, 0, 0, 0);
      sc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(o.kb[s], qreg[s], sc1, 0, 0, 0);
    }
    const int kv0 = t * kKTile;
    const int keyb = kv0 + 32 * lg;
    const bool diag = kv0 + kKTile - 1 > lastk0;
    int sa = INT32_MIN, sb = INT32_MIN;
#pragma unroll
    for (int v = 0; v < 16; v++) {
      sa = max(sa, diag && keyb + v > lastk ? INT32_MIN : sc0[v]);
      sb = max(sb, diag && keyb + 16 + v > lastk ? INT32_MIN : sc1[v]);
    }
    const float c2a = (dq * o.ks0) * p.s2, c2b = (dq * o.ks1) * p.s2;
    float ustar;
    if (FINEK) {
      float ua = sa == INT32_MIN ? -1e30f : (float)sa * c2a;
      float ub = sb == INT32_MIN ? -1e30f : (float)sb * c2b;
      ustar = pair_max_f32(fmaxf(ua, ub));
    } else {
      const int smax = pair_max_i32(max(sa, sb));
      ustar = smax == INT32_MIN ? -1e30f : (float)smax * c2a;
    }
    const float mnew = fmaxf(m, ustar);
    const float mm = mnew - 8.0f;
    const float ka = __builtin_fmaf(kScoreBiasF, c2a, mm), kb = FINEK ? __builtin_fmaf(kScoreBiasF, c2b, mm) : ka;
    v8i pb;
#pragma unroll
    for (int h = 0; h < 2; h++) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        float pv4[4];
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const int sv = h == 0 ? sc0[4 * q + e] : sc1[4 * q + e];
          // B + S as fp32 (an exact add): the attention kernel's argument bit for bit
          float arg = __builtin_fmaf((float)sv + kScoreBiasF, h == 0 ? c2a : c2b, h == 0 ? -ka : -kb);
          if (diag && keyb + 16 * h + 4 * q + e > lastk) arg = -__builtin_inff();
          const float x = __builtin_amdgcn_exp2f(arg);
          pv4[e] = x;
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pv4[0], pv4[1], __float_as_int(pv4[0]), false);
        pb[4 * h + q] = __builtin_amdgcn_cvt_pk_fp8_f32(pv4[2], pv4[3], w, true);
      }
    }
    const float rs = rowsum_fp8(ones16, pb);   // the row's whole 64-key sum of the FP8 codes
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    if (__builtin_amdgcn_ballot_w64(mnew > m) != 0) {
#pragma unroll
      for (int ct = 0; ct < CT; ct++)
#pragma unroll
        for (int e = 0; e < 16; e++) oacc[ct][e] *= alpha;
    }
    m = mnew;
#pragma unroll
    for (int ct = 0; ct < CT; ct++) {
      const v8i av = {o.va[ct][0], o.va[ct][1], o.va[ct][2], o.va[ct][3],
                      o.vb[ct][0], o.vb[ct][1], o.vb[ct][2], o.vb[ct][3]};
      oacc[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, oacc[ct], 0, 0, 0, 127, 0, 127);
    }
    lpart = __builtin_fmaf(alpha, lpart, rs);
  };

  const int t0 = chunk * p.ctiles, t1 = min(t0 + p.ctiles, p.nkt);
  Ops a, b, c;   // tiles t, t+1, t+2 (two tiles in flight while one is computed)
  load(t0, a);
  if (t0 + 1 < t1) load(t0 + 1, b);
  for (int t = t0; t < t1; t += 3) {
    if (t + 2 < t1) load(t + 2, c);
    compute(t, a);
    if (t + 1 >= t1) break;
    if (t + 3 < t1) load(t + 3, a);
    compute(t + 1, b);
    if (t + 2 >= t1) break;
    if (t + 4 < t1) load(t + 4, b);
    compute(t + 2, c);
  }

  float* up = p.part + (size_t)unit * unit_floats<D>();
  // lanes l and l^32 hold the same whole sum (the max of the pair is that sum; this
  // form also keeps the register allocation of this kernel free of spills)
  const float lt = pair_max_f32(lpart);
#pragma unroll
  for (int ct = 0; ct < CT; ct++)
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int c0 = 32 * ct + 8 * q + 4 * lg;
      *(v4f*)(up + (size_t)li * D + c0) = v4f{oacc[ct][4 * q], oacc[ct][4 * q + 1], oacc[ct][4 * q + 2],
                                               oacc[ct][4 * q + 3]};
    }
  if (lg == 0) {
    up[32 * D + li] = m;
    up[32 * D + 32 + li] = lt;
  }
}

// Merge of the chunks of each query row: m* = max m_c over chunks with l_c > 0
// (a chunk where the row sees no key has l_c = 0), w_c = exp2(m_c - m*),
// L = sum w_c l_c and O' = sum w_c O_c (fp32 fma, ascending chunks),
// O = O' * v_scale / L.  One workgroup per (K/V head, row group, block of 32
// channels): 8 threads per row, 4 channels each.
template <int D, int OUT>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeK p, const float* __restrict__ v_scale, void* O,
                                                           int Hq, int nhd) {
  constexpr int CPT = 4;
  const int cb = blockIdx.x % (D / 32), rest = blockIdx.x / (D / 32);
  const int rg = rest % p.R, bhkv = rest / p.R;
  const int row = threadIdx.x >> 3, c0 = 32 * cb + (threadIdx.x & 7) * CPT;
  const int f = rg * 32 + row;
  if (f >= p.g * p.Nq) return;
  const int qi = f % p.Nq, bhq = bhkv * p.g + f / p.Nq;
  const size_t u0 = ((size_t)bhkv * p.R + rg) * p.nchunk;   // first unit of this row group
  // The splits' states are loaded eight at a time, every load of a batch in
  // flight before the first is used; the arithmetic keeps its order (the
  // maximum first, then the fma chains in ascending split order).
  static_assert(CPT == 4, "one 16-byte load of O_acc per split");
  constexpr int NB = 8;
  float ms = -3.0e38f;
  int c = 0;
  for (; c + NB <= p.nchunk; c += NB) {
    float mm[NB], ll[NB];
#pragma unroll
    for (int u = 0; u < NB; u++) {
      const float* up = p.part + (u0 + c + u) * unit_floats<D>();
      mm[u] = up[32 * D + row];
      ll[u] = up[32 * D + 32 + row];
    }
#pragma unroll
    for (int u = 0; u < NB; u++)
      if (ll[u] > 0.0f) ms = fmaxf(ms, mm[u]);
  }
  for (; c < p.nchunk; c++) {
    const float* up = p.part + (u0 + c) * unit_floats<D>();
    if (up[32 * D + 32 + row] > 0.0f) ms = fmaxf(ms, up[32 * D + row]);
  }
  float L = 0.0f, o[CPT];
#pragma unroll
  for (int e = 0; e < CPT; e++) o[e] = 0.0f;
  auto add = [&](float lc, float mc, const v4f& x) {
    if (!(lc > 0.0f)) return;
    const float w = __builtin_amdgcn_exp2f(mc - ms);
    L = __builtin_fmaf(w, lc, L);
#pragma unroll
    for (int k = 0; k < 4; k++) o[k] = __builtin_fmaf(w, x[k], o[k]);
  };
  c = 0;
  for (; c + NB <= p.nchunk; c += NB) {
    float mm[NB], ll[NB];
    v4f xx[NB];
#pragma unroll
    for (int u = 0; u < NB; u++) {
      const float* up = p.part + (u0 + c + u) * unit_floats<D>();
      mm[u] = up[32 * D + row];
      ll[u] = up[32 * D + 32 + row];
      xx[u] = *(const v4f*)(up + (size_t)row * D + c0);   // in bounds; unused when the split has no key
    }
#pragma unroll
    for (int u = 0; u < NB; u++) add(ll[u], mm[u], xx[u]);
  }
  for (; c < p.nchunk; c++) {
    const float* up = p.part + (u0 + c) * unit_floats<D>();
    add(up[32 * D + 32 + row], up[32 * D + row], *(const v4f*)(up + (size_t)row * D + c0));
  }
  const float inv = 1.0f / L;
  const float* vs = v_scale + (size_t)bhkv * D;
  const size_t orow = nhd ? ((size_t)(bhq / Hq) * p.Nq + qi) * Hq + bhq % Hq : (size_t)bhq * p.Nq + qi;
#pragma unroll
  for (int e = 0; e < CPT; e += 4) {
    const v4f sc = *(const v4f*)(vs + c0 + e);
    v4f r;
#pragma unroll
    for (int k = 0; k < 4; k++) r[k] = o[e + k] * (sc[k] * inv);
    store4<OUT>(O, orow * D + c0 + e, r);
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
static DecodeK decode_params(const DecodeArgs& a) {
  DecodeK k{};
  k.q_codes = a.q_codes; k.q_scale = a.q_scale; k.k_codes = a.k_codes; k.k_scale = a.k_scale;
  k.v_codes = a.v_codes; k.part = (float*)a.workspace;
  k.g = a.Hq / a.Hkv; k.Nq = a.Nq; k.Nkv = a.Nkv; k.off = a.Nkv - a.Nq;
  k.nqp = (a.Nq + kQTile - 1) / kQTile * kQTile; k.nbq = k.nqp / a.blk_q; k.blk_q = a.blk_q;
  k.nkt = (a.Nkv + kKTile - 1) / kKTile; k.nbk = k.nkt * kKTile / a.blk_k;
  k.lgk = a.blk_k == 16 ? 4 : a.blk_k == 32 ? 5 : 6;
  k.causal = a.causal;
  k.R = (k.g * a.Nq + 31) / 32;
  k.ctiles = a.kv_chunk / kKTile;
  k.nchunk = (k.nkt + k.ctiles - 1) / k.ctiles;
  k.units = a.B * a.Hkv * k.R * k.nchunk;
  k.s2 = a.s2;
  return k;
}

int decode_default_chunk(int B, int Hq, int Hkv, int Nq, int Nkv) {
  // as many splits as fit one round of waves (one per SIMD: 1024 on 256 CUs),
  // at least one tile each
  const long long rows = (long long)B * Hkv * (((long long)(Hq / Hkv) * Nq + 31) / 32);
  const int nkt = (Nkv + kKTile - 1) / kKTile;
  long long nchunk = 1024 / rows;
  if (nchunk > nkt) nchunk = nkt;
  if (nchunk < 1) nchunk = 1;
  const int ctiles = (int)((nkt + nchunk - 1) / nchunk);
  return ctiles * kKTile;
}

size_t decode_workspace(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int kv_chunk) {
  const long long R = ((long long)(Hq / Hkv) * Nq + 31) / 32;
  const long long nkt = (Nkv + kKTile - 1) / kKTile, ctiles = kv_chunk / kKTile;
  const long long units = (long long)B * Hkv * R * ((nkt + ctiles - 1) / ctiles);
  return (size_t)units * ((size_t)32 * d + 64) * sizeof(float);
}

template <int D>
static void launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  const DecodeK k = decode_params(a);
  const int grid = (k.units + 3) / 4;
  if (a.blk_k < kKTile) hipLaunchKernelGGL((decode_chunk_kernel<D, true>), dim3(grid), dim3(256), 0, st, k);
  else hipLaunchKernelGGL((decode_chunk_kernel<D, false>), dim3(grid), dim3(256), 0, st, k);
  const int mgrid = a.B * a.Hkv * k.R * (D / 32);
  if (a.out_dtype == 2)
    hipLaunchKernelGGL((decode_merge_kernel<D, 2>), dim3(mgrid), dim3(256), 0, st, k, a.v_scale, a.O, a.Hq, a.nhd);
  else if (a.out_dtype == 1)
    hipLaunchKernelGGL((decode_merge_kernel<D, 1>), dim3(mgrid), dim3(256), 0, st, k, a.v_scale, a.O, a.Hq, a.nhd);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, 0>), dim3(mgrid), dim3(256), 0, st, k, a.v_scale, a.O, a.Hq, a.nhd);
}

void launch_attn_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.d == 128) launch_decode_d<128>(a, st);
  else launch_decode_d<64>(a, st);
}

}  // namespace sage
