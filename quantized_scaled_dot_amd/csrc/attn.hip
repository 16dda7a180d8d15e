// Fused quantized attention forward for gfx950 (CDNA4).
//
// One workgroup = 128 query rows of one query head (4 waves x 32 rows); KV
// tiles of 64 keys of its K/V head (query head h of Hq reads K/V head
// h / (Hq/Hkv)) are staged in LDS and visited in ascending order.  With fewer
// queries than keys, query row i is aligned with key i + (Nkv - Nq): under
// the causal mask it sees keys 0 .. i + Nkv - Nq.  Lengths need not be tile
// multiples: the codes are zero-padded to whole tiles, keys at or past Nkv
// are masked like causal ones, and rows at or past Nq are not stored.
//
// LDS: two K tile slots (MFMA order, rows padded to d+16 bytes) and three V
// tile slots (channel-major, rows padded to 80 bytes), filled by direct
// global -> LDS copies: K two tiles ahead of use, V one (with Q smoothing also
// two slots of the INT8 K tile).  Step t computes the scores of tile t+1, the
// softmax of tile t and the P~V of tile t-1, one barrier per step.
//
// Per wave and KV tile:
//   S^T[64 keys x 32 queries] = K_tile . Q^T          2 x (d/32) v_mfma_i32_32x32x32_i8
//   (transposed so that each lane holds one query row: lane l owns query l%32
//    and 32 of the 64 keys; lanes l and l^32 share a row)
//   (the accumulators start at the bit pattern of B = 1.5 * 2^23, so each
//    int32 result read as fp32 is exactly B + S: no conversion per score)
//   row max on the int32 scores, dequantisation c2 = dQ*dK*sm_scale*log2e,
//   P~ = exp2((B + S)*c2 - K), K = RN(B*c2 + m' - 8) (one fma, fp32
//   v_exp_f32) on the VALU, packed to FP8 e4m3 in registers
//   l += sum of the FP8 codes of the row             1 v_mfma_scale_f32_16x16x128_f8f6f4
//   O_acc^T[32 ch x 32 q] += V^T_tile . P^T             d/32 v_mfma_scale_f32_32x32x64_f8f6f4
//   (inner level: the instruction's 64-product block sum; outer level: the
//    exact fp32 accumulate into its C operand; O_acc is rescaled by alpha
//    first whenever a row's running max grew)
//
// Register layout chaining: the int8 MFMA output places key
// 32*g + 16*h + v in register v of half h of lane group g = lane/32 when K
// row sigma_h(m) feeds MFMA row m (sigma is applied when K is staged into LDS,
// "MFMA order").  Packing those 32 values in register order gives exactly the
// FP8 B operand whose byte b of lane group g is key 32*g + b, which pairs with
// byte b of the V^T operand = the 32 contiguous channel-major codes of keys
// 32*g .. 32*g+31.  No register shuffles are needed between the two MFMAs.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace sage {

struct AttnK {
  const int8_t* q_codes;
  const float* q_scale;
  const int8_t* k_codes;
  const float* k_scale;
  const uint8_t* v_codes;
  const float* v_scale;
  void* O;
  int Hq, g, Nq, Nkv, off, nqt, nbq, blk_q, nhd;   // g = Hq/Hkv; off = Nkv - Nq
  int nqp, nkt;   // Q code rows per head (Nq rounded up to 128); KV tiles per head
  int nbk, lgk;   // K scales per head; log2 of the K block size
  // 4-bit QK^T: E2M1 codes (two per byte, rows of d/2 bytes) and one E8M0
  // scale byte per 32 channels of a row
  const uint8_t* q4_codes;
  const uint8_t* q4_scale;
  const uint8_t* k4_codes;
  const uint8_t* k4_scale;
  // Q smoothing of the 4-bit scores: INT8 block means of 32 queries (nqp/32
  // blocks per head, rows of d codes) with one exponent byte each, and the
  // smoothed K in INT8 tiles (rows of d codes, one exponent byte per tile)
  const int8_t* qm_codes;
  const uint8_t* qm_scale;
  const int8_t* k8_codes;
  const uint8_t* k8_scale;
  // FP4 P~V: V in E2M1 (tiles of d channel rows of 32 bytes, two keys per
  // byte) with E8M0 scales per channel and 32 keys (per tile: 2 x 32 x d/32
  // bytes, byte (g, m, c) for channel 32c + m and keys 32g .. 32g+31)
  const uint8_t* v4_codes;
  const uint8_t* v4_scale;
  float s2;
  const int32_t* sel;
  int n_sel;
  int32_t* s_dump;
  uint8_t* p_dump;
};

// RAGGED: Nq or Nkv is not a multiple of 128 (masked partial last KV tile,
// unstored padding rows, 1 to 4 masked steps at the end; at d = 64 it runs 2
// workgroups per CU, where the 3 of the other d = 64 kernels would spill;
// so does the causal FP4 P~V kernel at d = 64).
// Otherwise the masked steps are exactly the two causal diagonal tiles and
// none at all without the mask.
// FINEK: K blocks of 16 or 32 keys.  A lane's 32 keys of a tile are two runs
// of 16 (keys 32g + v and 32g + 16 + v), each inside one K block, so a lane
// dequantizes each run with its own factor and the row max combines the two
// scaled run maxima.  Otherwise one K block is one KV tile.
// QK4: 4-bit QK^T.  Q and K are E2M1 with a power-of-two scale per 32
// channels; the scores come from the scaled FP4 matrix instruction as fp32
// (the block scales applied inside it), so the dequantization factor is
// sm_scale * log2(e) alone and the row max runs on fp32.  K tiles are d/2
// bytes per key; each lane loads the scale bytes of its two MFMA rows' keys
// one step ahead.  QK4 = 3: the same 4-bit scores with P~V in FP4 as well:
// each lane's 32 keys of a row are one MX block, whose E8M0 exponent is
// floor(max exponent argument) - 2; the hardware converts P~ / 2^E to E2M1
// (round to nearest even, saturating), the row sum of the decoded P^ comes
// from one 16x16x128 FP4 instruction, the P~V instructions take both
// operands in FP4 with their block scales, and O = O_acc / l (the V scales
// are inside the products).  QK4 = 2 adds Q smoothing: the scores also take the mean
// of the wave's 32 queries (one block) against the smoothed K, both INT8
// with power-of-two block scales: the INT8 matrix instruction sums the
// integer products exactly, one fma per score turns that sum into the exact
// fp32 term, and the FP4 products are added on top (the INT8 K tile is
// staged next to the 4-bit one, rows of d + 16 bytes in the same MFMA order).
// Workgroups per CU (launch bounds): 3 for the aligned d = 64 kernels (but
// the causal FP4 one) and the aligned non-causal FP4 kernel at d = 128 (168
// VGPRs, a few spilled; measured 4.7% faster than 2 at the video shape),
// otherwise 2 (1 for NW = 8).
// NW: waves per workgroup (query rows 32 NW).  4 everywhere; 8 for the
// aligned INT8 d = 128 kernels on whole 256-row query tiles, where one
// workgroup then fills a CU and each K/V tile copy serves twice the rows
// (causal: only for long key ranges, since its four diagonal steps leave more
// waves idle than the two of a 128-row workgroup).
template <int D, bool CAUSAL, bool RAGGED, bool FINEK, int QK4, int OUT, bool DUMP, int NW = 4>
__global__ __launch_bounds__(64 * NW, NW == 8                                              ? 1
                                       : D == 64 && !RAGGED && !(QK4 == 3 && CAUSAL)        ? 3
                                       : QK4 == 3 && !CAUSAL && !RAGGED                     ? 3
                                                                                            : 2) void
attn_fwd_kernel(AttnK p) {
  static_assert(NW == 4 || (NW == 8 && D == 128 && !RAGGED && !DUMP && QK4 == 0), "wide tiles");
  constexpr int QT = 32 * NW;   // query rows per workgroup
  constexpr bool QSM = QK4 == 2;
  constexpr bool PV4 = QK4 == 3;               // FP4 P~V
  constexpr int KB = QK4 ? D / 2 : D;          // K code bytes per key
  constexpr int KS = KB / 32;                  // k-steps of the score MFMA over d (32 code bytes a lane pair)
  constexpr int CT = D / 32;                   // 32-channel tiles of the FP8 MFMA
  constexpr int VB = PV4 ? kKTile / 2 : kKTile;  // V code bytes per channel row of a tile
  constexpr int TILE = VB * D;                 // bytes of one V tile in HBM
  constexpr int RV = VB + 16;                  // V rows in LDS, padded by 16 bytes
  constexpr int KTILE = kKTile * KB;           // bytes of one K tile in HBM
  constexpr int RK = QK4 ? KB + 16 : kRowK<D>;
  using SV = typename std::conditional<(QK4 != 0), v16f, v16i>::type;   // score registers
  constexpr int RK8 = kRowK<D>;                 // INT8 K rows of the mean term (Q smoothing), padded like INT8 K
  __shared__ __attribute__((aligned(16))) int8_t sK[2][kKTile * RK];
  __shared__ __attribute__((aligned(16))) uint8_t sV[3][D * RV];
  __shared__ __attribute__((aligned(16))) uint8_t sK8[2][QSM ? kKTile * RK8 : 16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int li = lane & 31, lg = lane >> 5;
  const v8i ones16 = rowsum_ones_operand(lane, PV4);   // row sums of P^ (see rowsum_fp8)
  // INT8 scores: the score bias held in 16 VGPRs for the whole kernel (an
  // opaque value, so that it is not rebuilt from SGPRs with 8 moves per tile)
  // and read as the C operand of each tile's first score MFMAs, wherever those
  // registers fit without spills: not at d = 64 with three workgroups per CU,
  // nor in the non-causal ragged d = 128 kernel (256 VGPRs already)
  constexpr bool KEEPB = QK4 == 0 && (D == 128 ? CAUSAL || !RAGGED : RAGGED);
  v16i kbias = kScoreBias16;
  if constexpr (KEEPB) asm volatile("" : "+v"(kbias));
  // Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs
  // on XCD b % 8).  Flat query head bh = b*Hq + h reads flat K/V head
  // bh / g (the g query heads of a K/V head are consecutive).  When the K/V
  // heads divide evenly, XCD x owns K/V heads x, x+8, ... with all of their
  // query heads, so each K/V head stays in one L2.  Non-causal: an XCD walks
  // its K/V heads one after another.  Causal (work grows with the query
  // tile): an XCD walks its query tiles heaviest first across all of its
  // heads, so the long tiles never start last.
  const int G = gridDim.x, b = blockIdx.x;
  const int BHq = G / p.nqt, BHkv = BHq / p.g;
  int bh, qt;
  if (BHkv % 8 == 0) {
    const int x = b % 8, j = b / 8, hpx = BHkv / 8;   // XCD, its j-th item, K/V heads per XCD
    if (CAUSAL) {
      const int r = j % (hpx * p.g);
      bh = ((r % hpx) * 8 + x) * p.g + r / hpx;
      qt = p.nqt - 1 - j / (hpx * p.g);
    } else {
      const int u = p.g * p.nqt, r = j % u;           // units of one K/V head
      bh = ((j / u) * 8 + x) * p.g + r / p.nqt;
      qt = r % p.nqt;
    }
  } else if (CAUSAL) {
    bh = b % BHq; qt = p.nqt - 1 - b / BHq;          // heaviest first overall
  } else {
    bh = b / p.nqt; qt = b % p.nqt;
  }
  const int bhkv = bh / p.g;
  const int Nq = p.Nq, Nkv = p.Nkv, off = p.off;
  const int q0 = qt * QT, qrow0 = q0 + wave * 32, row = qrow0 + li;
  // the last key this row sees, and the smallest such key over the wave
  // (only read in masked steps)
  const int lastk = !RAGGED ? row + off : CAUSAL ? min(row + off, Nkv - 1) : Nkv - 1;
  const int lastk0 = !RAGGED ? qrow0 + off : CAUSAL ? min(qrow0 + off, Nkv - 1) : Nkv - 1;

  int dump_idx = -1;
  if (DUMP) {
    for (int k = 0; k < p.n_sel; k++)
      if (p.sel[k] == bh * p.nqt + qt) { dump_idx = k; break; }
  }

  v4i qreg[KS];
  int qsc[KS];   // QK4: the E8M0 scale byte of each of this lane's Q blocks
  {
    const int8_t* qp = (QK4 ? (const int8_t*)p.q4_codes : p.q_codes) + ((size_t)bh * p.nqp + row) * KB + 16 * lg;
#pragma unroll
    for (int s = 0; s < KS; s++) qreg[s] = *(const v4i*)(qp + 32 * s);
    if (QK4) {
#pragma unroll
      for (int s = 0; s < KS; s++) qsc[s] = p.q4_scale[((size_t)bh * p.nqp + row) * (D / 32) + 2 * s + lg];
    }
  }
  const float dq = QK4 ? 0.0f : p.q_scale[(size_t)bh * p.nbq + qrow0 / p.blk_q];
  // Q smoothing: the INT8 mean of this wave's 32 queries as the B operand of
  // every column (lane group g holds channels 32s + 16g .. +15 of k-step s,
  // as the INT8 Q codes), and its scale exponent
  v4i qm8[QSM ? CT : 1];
  int qme = 0;
  if (QSM) {
    const size_t r = (size_t)bh * (p.nqp / 32) + qrow0 / 32;
#pragma unroll
    for (int s = 0; s < CT; s++) qm8[s] = *(const v4i*)(p.qm_codes + r * D + 32 * s + 16 * lg);
    qme = (int)p.qm_scale[r] - 127;
  }

  // ---- staging: direct global -> LDS copies (buffer loads with the LDS
  // destination, 16 bytes per lane, 1 KiB per wave instruction) ----
  // Instruction i of a tile fills LDS bytes [1024 i, 1024 i + 1024) of its
  // slot: lane l writes bytes 1024 i + 16 l onward, and its global source is
  // chosen so that the padded LDS layout comes out directly (K rows in MFMA
  // order, d + 16 bytes; V channel rows, 80 bytes).  Padding chunks re-read
  // the last data chunk of their row.  A step copies one K and one V tile:
  // wave w issues K and V instructions w, w+NW, ... of the whole rounds of
  // four, then one of the leftover instructions (K first, then V; none when
  // w is past them), so that no copy depends on a branch per instruction.
  // K tile t lives in sK[t%2], V tile t in sV[t%3]; K is staged one tile
  // ahead of V (see the loop).  The K and V tiles are contiguous blocks in
  // HBM (K: 64 rows of KB code bytes; V: d rows of 64 codes).
  constexpr int NKI = kKTile * RK / 1024, NVI = D * RV / 1024;   // 9, 10 (d = 128); 5, 5 (d = 64); FP4 V: 6, 3
  constexpr int N8I = QSM ? kKTile * RK8 / 1024 : 0;                 // INT8 K tile (Q smoothing)
  constexpr int KTILE8 = kKTile * D;                                 // bytes of one INT8 K tile in HBM
  static_assert(kKTile * RK % 1024 == 0 && D * RV % 1024 == 0 && kKTile * RK8 % 1024 == 0,
                "whole DMA instructions per tile");
  constexpr int FK = NKI / NW, F8 = N8I / NW, FV = NVI / NW;         // whole rounds
  constexpr int XK = NKI % NW, X8 = N8I % NW, XR = NKI % NW + N8I % NW + NVI % NW;   // leftovers: K, INT8 K, all
  constexpr int NXR = (XR + NW - 1) / NW;                             // leftover rounds
  static_assert(NXR <= 2, "at most two leftover rounds");
  __builtin_assume(wave >= 0 && wave < NW);
  const __amdgpu_buffer_rsrc_t rK =
      head_rsrc((QK4 ? (const int8_t*)p.k4_codes : p.k_codes) + (size_t)bhkv * p.nkt * KTILE, (uint32_t)(p.nkt * KTILE));
  const __amdgpu_buffer_rsrc_t rV =
      head_rsrc((PV4 ? p.v4_codes : p.v_codes) + (size_t)bhkv * p.nkt * TILE, (uint32_t)(p.nkt * TILE));
  const __amdgpu_buffer_rsrc_t rK8 =
      QSM ? head_rsrc(p.k8_codes + (size_t)bhkv * p.nkt * KTILE8, (uint32_t)(p.nkt * KTILE8)) : rK;
  auto k_src = [&](int i, int rk, int kb) {
    const int o = 1024 * i + 16 * lane;
    const int rho = o / rk, c = min((o % rk) / 16, kb / 16 - 1);
    return (uint32_t)(k_lds_key(rho) * kb + 16 * c);
  };
  auto v_src = [&](int i) {
    const int o = 1024 * i + 16 * lane;
    const int r = o / RV, c = min((o % RV) / 16, VB / 16 - 1);
    return (uint32_t)(r * VB + 16 * c);
  };
  uint32_t koff[FK > 0 ? FK : 1], k8off[F8 > 0 ? F8 : 1], voff[FV > 0 ? FV : 1];
#pragma unroll
  for (int j = 0; j < FK; j++) koff[j] = k_src(wave + NW * j, RK, KB);
#pragma unroll
  for (int j = 0; j < F8; j++) k8off[j] = k_src(wave + NW * j, RK8, D);
#pragma unroll
  for (int j = 0; j < FV; j++) voff[j] = v_src(wave + NW * j);
  // this wave's leftover of round r: entry e = 4 r + wave of the list (K ones,
  // then INT8 K, then V); xt = 0 K, 1 INT8 K, 2 V, -1 none
  int xt[NXR > 0 ? NXR : 1], xi[NXR > 0 ? NXR : 1];
  uint32_t xoff[NXR > 0 ? NXR : 1];
#pragma unroll
  for (int r = 0; r < NXR; r++) {
    const int e = NW * r + wave;
    xt[r] = e < XK ? 0 : e < XK + X8 ? 1 : e < XR ? 2 : -1;
    xi[r] = xt[r] == 0 ? NW * FK + e : xt[r] == 1 ? NW * F8 + e - XK : NW * FV + e - XK - X8;
    xoff[r] = xt[r] == 0 ? k_src(xi[r], RK, KB) : xt[r] == 1 ? k_src(min(xi[r], N8I - 1), RK8, D) : v_src(min(xi[r], NVI - 1));
  }
  // The copies take their LDS destination as a plain address: the compiler
  // then does not relate them to the operand reads of the other slots (it
  // would wait for every copy before a step's first read), and the kernel
  // orders them itself (wait for this wave's copies, then the barrier,
  // before any read of a slot).
  const uint32_t kbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const void __attribute__((address_space(3)))*)&sK[0][0]);
  const uint32_t vbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const void __attribute__((address_space(3)))*)&sV[0][0]);
  const uint32_t k8base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const void __attribute__((address_space(3)))*)&sK8[0][0]);
  // K tile tk (and its FP8 form) into K slot kslot, V tile tv into V slot vslot
  auto stageKV = [&](int tk, int kslot, int tv, int vslot) {
    const uint32_t kd = kbase + (uint32_t)(kslot * (kKTile * RK)), vd = vbase + (uint32_t)(vslot * (D * RV));
    const uint32_t k8d = k8base + (uint32_t)(kslot * (kKTile * RK8));
#pragma unroll
    for (int j = 0; j < FK; j++) lds_copy16_at(rK, kd + 1024 * (wave + NW * j), koff[j], tk * KTILE);
#pragma unroll
    for (int j = 0; j < F8; j++) lds_copy16_at(rK8, k8d + 1024 * (wave + NW * j), k8off[j], tk * KTILE8);
#pragma unroll
    for (int j = 0; j < FV; j++) lds_copy16_at(rV, vd + 1024 * (wave + NW * j), voff[j], tv * TILE);
#pragma unroll
    for (int r = 0; r < NXR; r++)
      if (NW * (r + 1) <= XR || xt[r] >= 0)
        lds_copy16_at(xt[r] == 0 ? rK : xt[r] == 1 ? rK8 : rV, (xt[r] == 0 ? kd : xt[r] == 1 ? k8d : vd) + 1024 * xi[r],
                      xoff[r], xt[r] == 0 ? tk * KTILE : xt[r] == 1 ? tk * KTILE8 : tv * TILE);
  };
  // this wave's copies have landed in LDS (the barrier that follows makes
  // them visible to the other waves)
  auto staged = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };   // vmcnt(0)

  v16f oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ct++)
#pragma unroll
    for (int e = 0; e < 16; e++) oacc[ct][e] = 0.0f;
  float m = -1e30f, lpart = 0.0f;

  // tiles up to the one holding the workgroup's last visible key
  const int ntiles = CAUSAL ? min((q0 + QT - 1 + off) / kKTile + 1, p.nkt) : p.nkt;
  const float* kscale = p.k_scale + (size_t)bhkv * p.nbk;
  // K scale index of the run of 16 keys of half h of this lane in tile t
  auto kidx = [&](int t, int h) { return FINEK ? (t * kKTile + 32 * lg + 16 * h) >> p.lgk : t; };

  // QK4: K scale words of this lane's two MFMA rows (keys k_lds_key(li) and
  // k_lds_key(32 + li) of a tile): byte b is the scale of channels 32b..32b+31
  auto kscale4 = [&](int t, int h) -> unsigned {
    const uint8_t* ksp =
        p.k4_scale + ((size_t)bhkv * p.nkt * kKTile + (size_t)t * kKTile + k_lds_key(32 * h + li)) * (D / 32);
    return D == 128 ? *(const unsigned*)ksp : (unsigned)*(const uint16_t*)ksp;
  };
  unsigned ksw_next[2] = {QK4 ? kscale4(0, 0) : 0u, QK4 ? kscale4(0, 1) : 0u};
  unsigned ksw[2] = {0u, 0u};
  // the scale exponent byte of the INT8 K tile (Q smoothing)
  auto kscale8 = [&](int t) -> int { return (int)p.k8_scale[(size_t)bhkv * p.nkt + t]; };
  int ke8_next = QSM ? kscale8(0) : 0, ke8 = 0;
  // the scale words of tile t+1 become current; those of tile t+2 are loaded
  auto next_kscales = [&](int tn) {
    ksw[0] = ksw_next[0]; ksw[1] = ksw_next[1];
    ksw_next[0] = kscale4(tn, 0);
    ksw_next[1] = kscale4(tn, 1);
    if (QSM) {
      ke8 = ke8_next;
      ke8_next = kscale8(tn);
    }
  };
  // S^T = K_t . Q^T for KV tile t, into (a0: keys 32*lg + v, a1: keys 32*lg + 16 + v):
  // int32 (INT8 codes) or fp32 (QK4, scales applied in the instruction)
  auto qk = [&](int t, SV& a0, SV& a1) {
    const int8_t* kb0 = sK[t & 1] + li * RK + 16 * lg;   // MFMA rows li and 32 + li
    if constexpr (QSM) {
      // the block mean of Q against the INT8 K: n = exact int32 sum, in the
      // accumulator biased by B (its bits read as fp32 are B + n exactly,
      // |n| <= d 127^2 < 2^21); then fma((B + n), 2^e, -B 2^e) = n 2^e exactly,
      // e = Em + Ek8 in [-126, 104]
      v16i i0 = kScoreBias16, i1 = kScoreBias16;
      const int8_t* k8b = (const int8_t*)sK8[t & 1] + li * RK8 + 16 * lg;
#pragma unroll
      for (int s = 0; s < CT; s++) {
        const v4i x0 = *(const v4i*)(k8b + 32 * s), x1 = *(const v4i*)(k8b + 32 * RK8 + 32 * s);
        i0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(x0, qm8[s], i0, 0, 0, 0);
        i1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(x1, qm8[s], i1, 0, 0, 0);
      }
      const int e = qme + ke8 - 127;
      const float sc = __builtin_amdgcn_ldexpf(1.0f, e), bs = __builtin_amdgcn_ldexpf(kScoreBiasF, e);
      // (each element is copied out before the bit cast: this compiler's
      // __builtin_bit_cast of a vector element expression reads element 0)
#pragma unroll
      for (int v = 0; v < 16; v++) {
        const int n0 = i0[v], n1 = i1[v];
        a0[v] = __builtin_fmaf(__builtin_bit_cast(float, n0), sc, -bs);
        a1[v] = __builtin_fmaf(__builtin_bit_cast(float, n1), sc, -bs);
      }
    } else if constexpr (QK4) {
      a0 = SV{}; a1 = SV{};
    } else {
      a0 = KEEPB ? kbias : kScoreBias16; a1 = a0;   // int32 results read as fp32 give B + S exactly
    }
    // QK4: this lane's 32 channels of k-step s are block 2s + lg.  With FP4
    // P~V that is byte 2s of its scale words shifted by lg bytes, which the
    // instruction selects (measured: 4% faster there); the other 4-bit kernels
    // extract the byte on the VALU (selecting it cost them registers: 166 ->
    // 170 VGPRs and the third wave of the plain 4-bit kernel, 5% slower)
    const unsigned kw0 = PV4 ? ksw[0] >> (8 * lg) : 0u, kw1 = PV4 ? ksw[1] >> (8 * lg) : 0u;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      const v4i k0 = *(const v4i*)(kb0 + 32 * s);
      const v4i k1 = *(const v4i*)(kb0 + 32 * RK + 32 * s);
      if constexpr (QK4) {
        const v8i q8 = {qreg[s][0], qreg[s][1], qreg[s][2], qreg[s][3], 0, 0, 0, 0};
        const v8i a8 = {k0[0], k0[1], k0[2], k0[3], 0, 0, 0, 0};
        const v8i b8 = {k1[0], k1[1], k1[2], k1[3], 0, 0, 0, 0};
        if constexpr (PV4) {
          a0 = mfma_fp4_byte(2 * s, a8, q8, a0, kw0, qsc[s]);
          a1 = mfma_fp4_byte(2 * s, b8, q8, a1, kw1, qsc[s]);
        } else {
          const int s0 = (int)((ksw[0] >> (8 * (2 * s + lg))) & 0xFFu), s1 = (int)((ksw[1] >> (8 * (2 * s + lg))) & 0xFFu);
          a0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, q8, a0, 4, 4, 0, s0, 0, qsc[s]);
          a1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, q8, a1, 4, 4, 0, s1, 0, qsc[s]);
        }
      } else {
        a0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0, qreg[s], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1, qreg[s], a1, 0, 0, 0);
      }
    }
  };
  // ---- two-level P~V for the tile whose V codes are in slot vslot: the
  // matrix core sums the 64 FP8 products of the tile (inner level) and adds
  // that block sum into the fp32 accumulator O_acc passed as its C operand
  // (outer level; the C addition is an fp32 add outside the instruction's
  // product-alignment window) ----
  // FP4 P~V: pb holds 32 E2M1 codes in its low 16 bytes, pscale the lane's
  // E8M0 byte of them, vsw the V scale bytes of the lane's rows (byte ct:
  // channel 32ct + li, keys 32lg ..)
  auto pv = [&](const v8i& pb, int vslot, int pscale, unsigned vsw) {
#pragma unroll
    for (int ct = 0; ct < CT; ct++) {
      const uint8_t* vb = sV[vslot] + (32 * ct + li) * RV + (PV4 ? 16 : 32) * lg;   // channel row, keys 32*lg..
      const v4i v0 = *(const v4i*)(vb);
      if constexpr (PV4) {
        const v8i av = {v0[0], v0[1], v0[2], v0[3], 0, 0, 0, 0};
        oacc[ct] = mfma_fp4_byte(ct, av, pb, oacc[ct], vsw, pscale);   // V scale: byte ct of vsw
      } else {
        const v4i v1 = *(const v4i*)(vb + 16);
        const v8i av = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        oacc[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, oacc[ct], 0, 0, 0, 127, 0, 127);
      }
    }
  };
  // FP4 P~V: the V scale bytes of this lane's rows in tile t
  auto vscale4 = [&](int t) -> unsigned {
    const uint8_t* vsp = p.v4_scale + ((size_t)(bhkv * p.nkt + t) * 64 + 32 * lg + li) * (D / 32);
    return D == 128 ? *(const unsigned*)vsp : (unsigned)*(const uint16_t*)vsp;
  };
  // whole tile t after every row of this wave (causal): nothing to compute
  auto future = [&](int t) { return CAUSAL && t * kKTile > qrow0 + 31 + off; };

  // P~ codes of the last visited tile whose P~V is still to be issued, and
  // that tile's rescale of the running state (alpha_prev, applied before
  // the pending P~V when some row of the wave got a larger max).
  v8i pprev;
  int pscale_prev = 127;        // FP4 P~V: E8M0 byte of pprev
  unsigned vsw_prev = 0u;       // FP4 P~V: V scale bytes of the tile of pprev
  bool pend = false, grew = false;
  float alpha_prev = 1.0f;
  // K scales (of this lane's two runs) of the tile whose softmax comes next
  float ks_next[2] = {QK4 ? 0.0f : kscale[kidx(0, 0)], FINEK ? kscale[kidx(0, 1)] : 0.0f};
  auto rescale = [&]() {
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
      for (int e = 0; e < 16; e++) oacc[ct][e] *= alpha_prev;
  };

  // One KV tile t whose scores sc0/sc1 were issued in the previous step.
  // The step issues the P~V of the previous tile and the scores of tile t+1
  // (when NEXT) between the VALU instructions of tile t's softmax, so the
  // matrix core runs while the VALU computes.  The previous tile's rescale
  // comes first: after the P~V of the tile before it (issued one step
  // earlier) and before its own, so O_t = alpha_t * O_{t-1} + P~_t V_t holds
  // exactly as in the sequential form.
  // DIAG: the tile may hold keys after some row (causal diagonal region).
  // HAD: 1 = a P~V is pending (every step after the first in the interior),
  // 0 = none (first step), 2 = decided at run time (causal diagonal steps).
  auto tile_step = [&](const int t, SV& sc0, SV& sc1, SV& nx0, SV& nx1, auto diag_tag, auto had_tag,
                       bool next) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    constexpr int HAD = decltype(had_tag)::value;
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();          // K_{t+1}, V_t staged; every wave is done with tile t-1
    __builtin_amdgcn_sched_barrier(0);
    const bool had = HAD == 2 ? pend : HAD == 1;
    if (had && grew) rescale();   // rare
    // The K scale of tile t+1 is read one step ahead, before the tile
    // copies, so waiting for it never waits for them.
    const float ks0 = ks_next[0], ks1 = ks_next[1];
    if (QK4) {
      next_kscales(min(t + 2, ntiles - 1));   // tile t+1's scores are computed in this step
    } else {
      ks_next[0] = kscale[kidx(min(t + 1, ntiles - 1), 0)];
      if (FINEK) ks_next[1] = kscale[kidx(min(t + 1, ntiles - 1), 1)];
    }
    // In flight while tile t is computed: K_{t+2} replaces K_t (read by the
    // previous step's score MFMAs), V_{t+1} replaces V_{t-2} (read by the
    // previous step's P~V).  Past the last tile the index is clamped: the
    // extra copy lands in a slot that is never read again.
    stageKV(min(t + 2, ntiles - 1), t & 1, min(t + 1, ntiles - 1), (t + 1) % 3);
    __builtin_amdgcn_sched_barrier(0);   // issue the copies first
    const int kv0 = t * kKTile;
    const int keyb = kv0 + 32 * lg;   // sc0[v] is key keyb + v, sc1[v] is key keyb + 16 + v
    if (had) pv(pprev, (t + 2) % 3, pscale_prev, vsw_prev);   // slot of tile t-1
    if (PV4) vsw_prev = vscale4(min(t, ntiles - 1));   // for the P~V of tile t (next step)

    if (!(DIAG && future(t))) {
      if (DUMP && dump_idx >= 0) {
        int32_t* sd = p.s_dump + ((size_t)dump_idx * QT + (row - q0)) * Nkv + keyb;
        // INT8: the exact int32 scores (the accumulator started at the bias); QK4: fp32 bits
        const v16i si0 = __builtin_bit_cast(v16i, sc0) - (QK4 ? 0 : kScoreBiasBits);   // no wrap: B + S > 0
        const v16i si1 = __builtin_bit_cast(v16i, sc1) - (QK4 ? 0 : kScoreBiasBits);
#pragma unroll
        for (int v = 0; v < 16; v++) {
          if (!RAGGED || keyb + v < Nkv) sd[v] = si0[v];
          if (!RAGGED || keyb + 16 + v < Nkv) sd[16 + v] = si1[v];
        }
      }
      const bool diag = DIAG && (kv0 + kKTile - 1 > lastk0);
      // ---- online softmax state (the max runs over visible keys only) ----
      float ustar, c2a, c2b;   // c2a, c2b: dequantization factors of the two runs
      float smx_lane = 0.0f;   // 4-bit: the max over this lane's visible keys
      if constexpr (QK4) {
        float smx = -__builtin_inff();
        if (diag) {
#pragma unroll
          for (int v = 0; v < 16; v++)
            smx = fmaxf(fmaxf(smx, keyb + v > lastk ? -__builtin_inff() : sc0[v]),
                        keyb + 16 + v > lastk ? -__builtin_inff() : sc1[v]);
        } else {
#pragma unroll
          for (int v = 0; v < 16; v++) smx = fmaxf(fmaxf(smx, sc0[v]), sc1[v]);   // v_max3_f32 chain
        }
        smx_lane = smx;
        smx = pair_max_f32(smx);
        c2a = c2b = p.s2;
        ustar = smx * c2a;
        if (DIAG && smx == -__builtin_inff()) ustar = -1e30f;   // no visible key in this tile for this row
      } else if (!FINEK) {
        int smax = INT32_MIN;
        if (diag) {
#pragma unroll
          for (int v = 0; v < 16; v++)
            smax = max(max(smax, keyb + v > lastk ? INT32_MIN : sc0[v]), keyb + 16 + v > lastk ? INT32_MIN : sc1[v]);
        } else {
#pragma unroll
          for (int v = 0; v < 16; v++) smax = max(max(smax, sc0[v]), sc1[v]);   // v_max3_i32 chain
        }
        smax = pair_max_i32(smax);
        c2a = c2b = (dq * ks0) * p.s2;
        ustar = DIAG && smax == INT32_MIN ? -1e30f   // no visible key in this tile for this row
                                          : (float)unbias_score(smax) * c2a;
      } else {
        int sa = INT32_MIN, sb = INT32_MIN;
#pragma unroll
        for (int v = 0; v < 16; v++) {
          sa = max(sa, diag && keyb + v > lastk ? INT32_MIN : sc0[v]);
          sb = max(sb, diag && keyb + 16 + v > lastk ? INT32_MIN : sc1[v]);
        }
        c2a = (dq * ks0) * p.s2;
        c2b = (dq * ks1) * p.s2;
        const float ua = DIAG && sa == INT32_MIN ? -1e30f : (float)unbias_score(sa) * c2a;
        const float ub = DIAG && sb == INT32_MIN ? -1e30f : (float)unbias_score(sb) * c2b;
        ustar = pair_max_f32(fmaxf(ua, ub));
      }
      const float mnew = fmaxf(m, ustar);
      const float mm = mnew - 8.0f;
      // INT8: the argument is one fma of the biased score, (B + S) c2 - K with
      // K = RN(B c2 + mm): the offset mm taken at the precision of B c2
      const float ka = QK4 ? mm : __builtin_fmaf(kScoreBiasF, c2a, mm);
      const float kb = QK4 ? mm : (FINEK ? __builtin_fmaf(kScoreBiasF, c2b, mm) : ka);
      if (next) qk(t + 1, nx0, nx1);

      // ---- P~ (fp32) -> FP8 B operand, packed in place ----
      // exp2 is the hardware's fp32 exp2 (v_exp_f32): any argument is valid,
      // and masked (future) keys get -inf, whose exp2 is exactly 0.
      v8i pb;
      float rs = 0.0f;   // 4-bit scores with FP8 P~V: the fp32 row sum of P~ on the VALU
      // FP4 P~V: this lane's block exponent E = floor(max arg) - 2 in
      // [-126, 127] (no visible key: -126), the convert's divisor 2^E and
      // the E8M0 byte E + 127
      int pscale = 127;
      float pdiv = 1.0f;
      if constexpr (PV4) {
        const float fe = fminf(fmaxf(__builtin_floorf(__builtin_fmaf(smx_lane, c2a, -ka)) - 2.0f, -126.0f), 127.0f);
        const int e = (int)fe;
        pscale = e + 127;
        pdiv = __builtin_amdgcn_ldexpf(1.0f, e);
      }
#pragma unroll
      for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          float pv4[4];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const auto sv = h == 0 ? sc0[4 * q + e] : sc1[4 * q + e];   // biased int32 or fp32 score
            float sf;
            if constexpr (QK4) sf = sv;
            else sf = __builtin_bit_cast(float, sv);
            float arg = __builtin_fmaf(sf, h == 0 ? c2a : c2b, h == 0 ? -ka : -kb);
            if (diag && keyb + 16 * h + 4 * q + e > lastk) arg = -__builtin_inff();
            const float x = __builtin_amdgcn_exp2f(arg);
            pv4[e] = x;
            if constexpr (QK4 == 1 || QK4 == 2) rs += x;
          }
          if constexpr (PV4) {
            // keys 16h + 4q .. +3 are E2M1 elements 16h + 4q .. of the lane's
            // block: bytes 2(q%2), 2(q%2)+1 of dword 2h + q/2, low nibble first
            unsigned w;
            if (q % 2 == 0) {
              // (the first convert's "old" operand is a register that dies
              // here: the four converts of a dword write all of its bytes)
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(pv4[0]), pv4[0], pv4[1], pdiv, 0);
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pv4[2], pv4[3], pdiv, 1);
            } else {
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((unsigned)pb[2 * h + q / 2], pv4[0], pv4[1], pdiv, 2);
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, pv4[2], pv4[3], pdiv, 3);
            }
            pb[2 * h + q / 2] = (int)w;
          } else {
            // the low-half convert's "old" operand is a register that dies here
            // (its high half is overwritten by the second convert)
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(pv4[0], pv4[1], __float_as_int(pv4[0]), false);
            pb[4 * h + q] = __builtin_amdgcn_cvt_pk_fp8_f32(pv4[2], pv4[3], w, true);
          }
        }
      }
      if constexpr (PV4) { pb[4] = 0; pb[5] = 0; pb[6] = 0; pb[7] = 0; }
      // keep the softmax in this block: without a use here the compiler
      // moves it below the rescale branch, away from the MFMAs it should
      // overlap (an empty statement that reads the packed codes and the sum)
      asm volatile("" : "+v"(pb), "+v"(rs));
      // INT8 scores: the row sum of the FP8 codes P^ on the matrix core (each
      // lane gets its row's whole 64-key sum); FP4 P~V: of the E2M1 codes
      // with their block scales
      if constexpr (QK4 == 0) rs = rowsum_fp8(ones16, pb);
      if constexpr (PV4) rs = rowsum_fp4(ones16, pb, pscale);
      if (DUMP && dump_idx >= 0) {
        uint8_t* pd = p.p_dump + ((size_t)dump_idx * QT + (row - q0)) * Nkv + keyb;
#pragma unroll
        for (int k = 0; k < 32; k++)
          if (!RAGGED || keyb + k < Nkv)
            pd[k] = PV4 ? (uint8_t)(((unsigned)pb[k >> 3] >> (4 * (k & 7))) & 0xF)
                        : (uint8_t)(((unsigned)pb[k >> 2] >> (8 * (k & 3))) & 0xFF);
      }
      // alpha = exp2(m - m'): 1 exactly where the max did not grow, 0 on the
      // first visited tile (m = -1e30, the state is still zero)
      const float alpha = __builtin_amdgcn_exp2f(m - mnew);
      lpart = __builtin_fmaf(alpha, lpart, rs);
      grew = __builtin_amdgcn_ballot_w64(mnew > m) != 0;
      alpha_prev = alpha;
      m = mnew;
      pprev = pb;
      pscale_prev = pscale;
      pend = true;
    } else {
      if (next) qk(t + 1, nx0, nx1);
      pend = false;
    }
    if constexpr (!DIAG && HAD == 1 && (QK4 == 1 || (D == 64 && QK4 == 0))) {
      // Interior step of the plain 4-bit and the d = 64 INT8 kernels: spread
      // the matrix instructions evenly through the softmax (one MFMA, then its
      // share of VALU instructions; for INT8 with the step's operand reads
      // first).  Measured per variant: 4-bit 5-6% and d = 64 3-4% faster; the
      // d = 128 INT8 and the Q-smoothing kernels are faster in the
      // compiler's own order.
      constexpr int NM = 2 * KS * (QSM ? 2 : 1) + CT;
      constexpr int NV = QK4 ? 150 / NM : 175 / NM;
      if constexpr (!QK4) __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS + 2 * CT, 0);
#pragma unroll
      for (int i = 0; i < NM; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
      }
    }
    staged();
  };

  // prologue: K_0, V_0, K_1 (and V_1) staged, scores of tile 0 issued
  stageKV(0, 0, 0, 0);
  stageKV(min(1, ntiles - 1), 1, min(1, ntiles - 1), 1);   // V_1 early: step 0 copies it to the same slot again
  staged();
  __syncthreads();
  SV sa0, sa1, sb0, sb1;
  if (QK4) next_kscales(min(1, ntiles - 1));   // scale words of tiles 0 and 1
  qk(0, sa0, sa1);

  // Tiles fully visible to every row of the workgroup (before the causal
  // diagonal and before a partial last tile), rounded down to an even count,
  // take the unmasked steps in pairs.  The pipelined step always computes the
  // next tile's scores there: after the last tile of a non-causal pass that
  // reads a stale (but in-bounds) K slot and is unused.  The remaining 0 to 4
  // tiles take the masked steps.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  const int nint = (CAUSAL ? (q0 + off + 1) / kKTile : Nkv / kKTile) & ~1;
  int t = 0;
  if (nint > 0) {
    tile_step(0, sa0, sa1, sb0, sb1, std::false_type{}, I0{}, true);
    for (t = 1; t + 1 < nint; t += 2) {
      tile_step(t, sb0, sb1, sa0, sa1, std::false_type{}, I1{}, true);
      tile_step(t + 1, sa0, sa1, sb0, sb1, std::false_type{}, I1{}, true);
    }
    tile_step(t, sb0, sb1, sa0, sa1, std::false_type{}, I1{}, true);   // t = nint - 1
    t = nint;
  }
  if (RAGGED) {
    for (; t < ntiles; t += 2) {   // masked steps (scores of tile t are in sa)
      tile_step(t, sa0, sa1, sb0, sb1, std::true_type{}, I2{}, t + 1 < ntiles && !future(t + 1));
      if (t + 1 == ntiles) { t = ntiles; break; }
      tile_step(t + 1, sb0, sb1, sa0, sa1, std::true_type{}, I2{}, t + 2 < ntiles && !future(t + 2));
    }
  } else if (CAUSAL && NW == 8) {   // the four diagonal tiles of 256 rows (scores of tile t are in sa)
    for (; t < ntiles; t += 2) {
      tile_step(t, sa0, sa1, sb0, sb1, std::true_type{}, I2{}, t + 1 < ntiles && !future(t + 1));
      if (t + 1 == ntiles) { t = ntiles; break; }
      tile_step(t + 1, sb0, sb1, sa0, sa1, std::true_type{}, I2{}, t + 2 < ntiles && !future(t + 2));
    }
  } else if (CAUSAL) {   // the two diagonal tiles (q0 + off)/64 and the next (scores of tile t are in sa)
    tile_step(t, sa0, sa1, sb0, sb1, std::true_type{}, I2{}, !future(t + 1));
    tile_step(t + 1, sb0, sb1, sa0, sa1, std::true_type{}, I2{}, false);
    t += 2;
  }
  if (pend) {   // the last visited tile is t-1
    if (grew) rescale();
    pv(pprev, (t + 2) % 3, pscale_prev, vsw_prev);
  }

  // ---- epilogue: O = O_acc * v_scale / l ----
  // INT8 and FP4 P~V: every lane holds its row's whole sum; 4-bit with FP8 P~V:
  // each lane summed half the keys
  const float lt = QK4 == 1 || QK4 == 2 ? pair_sum_f32(lpart) : lpart;
  const float inv = 1.0f / lt;
  const float* vs = p.v_scale + (size_t)bhkv * D;
  const size_t orow = p.nhd ? ((size_t)(bh / p.Hq) * Nq + row) * p.Hq + bh % p.Hq : (size_t)bh * Nq + row;
  const bool store = !RAGGED || row < Nq;
  // every V scale of the lane's channels is loaded before the first store (the
  // compiler may not move a load past a store to O), so the epilogue waits for
  // one round trip instead of one per group of four channels
  v4f vsc[PV4 ? 1 : CT][4];
  if constexpr (!PV4) {
#pragma unroll
    for (int ct = 0; ct < CT; ct++)
#pragma unroll
      for (int q = 0; q < 4; q++) vsc[ct][q] = *(const v4f*)(vs + 32 * ct + 8 * q + 4 * lg);
  }
#pragma unroll
  for (int ct = 0; ct < CT; ct++) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int c0 = 32 * ct + 8 * q + 4 * lg;   // O^T register 4q+e holds channel c0 + e
      const v4f sc = PV4 ? v4f{1.0f, 1.0f, 1.0f, 1.0f} : vsc[PV4 ? 0 : ct][q];
      v4f o;
#pragma unroll
      for (int e = 0; e < 4; e++) o[e] = PV4 ? oacc[ct][4 * q + e] * inv : oacc[ct][4 * q + e] * (sc[e] * inv);
      if (store) store4<OUT>(p.O, orow * D + c0, o);
    }
  }
}

// wide: the 8-wave workgroups of 256 query rows (see attn_fwd_kernel); the
// launcher only asks for them where that instance exists
template <int D, bool CAUSAL, bool RAGGED, bool FINEK, int QK4, int OUT>
static void launch5(const AttnK& k, int grid, bool dump, bool wide, hipStream_t st) {
  if constexpr (D == 128 && !RAGGED && QK4 == 0) {
    if (wide) {
      hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, RAGGED, FINEK, QK4, OUT, false, 8>), dim3(grid), dim3(512), 0,
                         st, k);
      return;
    }
  }
  if (dump)
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, RAGGED, FINEK, QK4, OUT, true>), dim3(grid), dim3(256), 0, st, k);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL, RAGGED, FINEK, QK4, OUT, false>), dim3(grid), dim3(256), 0, st, k);
}
template <int D, bool CAUSAL, bool RAGGED, bool FINEK, int QK4>
static void launch4(const AttnK& k, int grid, int out, bool dump, bool wide, hipStream_t st) {
  if (out == 2) launch5<D, CAUSAL, RAGGED, FINEK, QK4, 2>(k, grid, dump, wide, st);
  else if (out == 1) launch5<D, CAUSAL, RAGGED, FINEK, QK4, 1>(k, grid, dump, wide, st);
  else launch5<D, CAUSAL, RAGGED, FINEK, QK4, 0>(k, grid, dump, wide, st);
}
// the score variant: INT8 with K blocks of a tile, INT8 with finer K blocks,
// 4-bit, 4-bit with Q smoothing, or 4-bit with FP4 P~V
template <int D, bool CAUSAL, bool RAGGED>
static void launch3(const AttnK& k, int grid, int variant, int out, bool dump, bool wide, hipStream_t st) {
  if (variant == 4) launch4<D, CAUSAL, RAGGED, false, 3>(k, grid, out, dump, wide, st);
  else if (variant == 3) launch4<D, CAUSAL, RAGGED, false, 2>(k, grid, out, dump, wide, st);
  else if (variant == 2) launch4<D, CAUSAL, RAGGED, false, 1>(k, grid, out, dump, wide, st);
  else if (variant == 1) launch4<D, CAUSAL, RAGGED, true, 0>(k, grid, out, dump, wide, st);
  else launch4<D, CAUSAL, RAGGED, false, 0>(k, grid, out, dump, wide, st);
}
// The kernel instances are compiled in eight parts, one per (head size,
// causal, ragged) combination, so that the build can run them in parallel:
// SAGE_ATTN_PART = 0..7 compiles part p only (D = 128 for p < 4, causal for
// p % 4 < 2, ragged for odd p); part 0 also holds the dispatcher.  Without
// the macro everything is compiled in one unit.
#ifndef SAGE_ATTN_PART
#define SAGE_ATTN_PART -1
#endif
#define SAGE_PART_DEF(P, D, C, R)                                                                         \
  void launch_attn_part##P(const AttnK& k, int grid, int variant, int out, bool dump, bool wide, hipStream_t st)
SAGE_PART_DEF(0, 128, true, false);
SAGE_PART_DEF(1, 128, true, true);
SAGE_PART_DEF(2, 128, false, false);
SAGE_PART_DEF(3, 128, false, true);
SAGE_PART_DEF(4, 64, true, false);
SAGE_PART_DEF(5, 64, true, true);
SAGE_PART_DEF(6, 64, false, false);
SAGE_PART_DEF(7, 64, false, true);
#define SAGE_PART_BODY(P, D, C, R)                                                                        \
  SAGE_PART_DEF(P, D, C, R) { launch3<D, C, R>(k, grid, variant, out, dump, wide, st); }
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 0
SAGE_PART_BODY(0, 128, true, false)
#endif
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 1
SAGE_PART_BODY(1, 128, true, true)
#endif
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 2
SAGE_PART_BODY(2, 128, false, false)
#endif
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 3
SAGE_PART_BODY(3, 128, false, true)
#endif
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 4
SAGE_PART_BODY(4, 64, true, false)
#endif
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 5
SAGE_PART_BODY(5, 64, true, true)
#endif
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 6
SAGE_PART_BODY(6, 64, false, false)
#endif
#if SAGE_ATTN_PART < 0 || SAGE_ATTN_PART == 7
SAGE_PART_BODY(7, 64, false, true)
#endif

#if SAGE_ATTN_PART <= 0
// average keys per query row (Nkv - Nq/2) from which causal runs 256-row workgroups
constexpr int kWideCausalKeys = 16384;

void launch_attn_fwd(const AttnArgs& a, bool dump, hipStream_t st) {
  AttnK k;
  k.q_codes = a.q_codes; k.q_scale = a.q_scale; k.k_codes = a.k_codes; k.k_scale = a.k_scale;
  k.v_codes = a.v_codes; k.v_scale = a.v_scale; k.O = a.O;
  k.Hq = a.Hq; k.g = a.Hq / a.Hkv; k.Nq = a.Nq; k.Nkv = a.Nkv; k.off = a.Nkv - a.Nq;
  // Q code rows per head: Nq rounded up to 128 (the layout of the quantized Q)
  k.nqp = (a.Nq + kQTile - 1) / kQTile * kQTile; k.nbq = k.nqp / a.blk_q;
  k.nkt = (a.Nkv + kKTile - 1) / kKTile; k.blk_q = a.blk_q; k.nhd = a.nhd; k.s2 = a.s2;
  k.nbk = k.nkt * kKTile / a.blk_k; k.lgk = a.blk_k == 16 ? 4 : a.blk_k == 32 ? 5 : 6;
  k.sel = a.sel; k.n_sel = a.n_sel; k.s_dump = a.s_dump; k.p_dump = a.p_dump;
  const bool ragged = a.Nq % kQTile != 0 || a.Nkv % kQTile != 0;
  k.q4_codes = a.q4_codes; k.q4_scale = a.q4_scale; k.k4_codes = a.k4_codes; k.k4_scale = a.k4_scale;
  k.qm_codes = a.qm_codes; k.qm_scale = a.qm_scale; k.k8_codes = a.k8_codes; k.k8_scale = a.k8_scale;
  k.v4_codes = a.v4_codes; k.v4_scale = a.v4_scale;
  const int variant = a.q4_codes ? (a.v4_codes ? 4 : a.qm_codes ? 3 : 2) : a.blk_k < kKTile ? 1 : 0;
  // 256-row workgroups: INT8 at d = 128 on whole 256-row query tiles (not for
  // the test dumps, which address 128-row tiles); causal only where a query
  // row sees 16384 keys or more on average (Nkv - Nq/2): measured 0.8-2% faster
  // at 30k-64k keys, 2-4% slower at 4k-8k, the same bits
  const bool wide = !dump && a.d == 128 && !ragged && variant <= 1 && a.Nq % 256 == 0 &&
                    (!a.causal || a.Nkv - a.Nq / 2 >= kWideCausalKeys);
  const int qtile = wide ? 256 : kQTile;
  k.nqt = (a.Nq + qtile - 1) / qtile;   // query tiles (workgroups) per head
  const int grid = a.B * a.Hq * k.nqt;
  const int part = (a.d == 128 ? 0 : 4) + (a.causal ? 0 : 2) + (ragged ? 1 : 0);
  void (*const parts[8])(const AttnK&, int, int, int, bool, bool, hipStream_t) = {
      launch_attn_part0, launch_attn_part1, launch_attn_part2, launch_attn_part3,
      launch_attn_part4, launch_attn_part5, launch_attn_part6, launch_attn_part7};
  parts[part](k, grid, variant, a.out_dtype, dump, wide, st);
}
#endif

}  // namespace sage
