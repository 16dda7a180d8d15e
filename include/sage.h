/*
 * sage.h -- C ABI of libsage.so, the MI355X (gfx950) quantized attention
 * forward: K smoothing, INT8 per-block Q/K, INT8 QK^T with int32 accumulation,
 * fp32 online softmax, FP8 (OCP e4m3) P~ and per-channel-scaled FP8 V, and a
 * two-level P~V accumulation (an FP8 matrix-core inner block added into an fp32
 * running accumulator).
 *
 * Method sources (web pages, by title and section):
 *  - "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
 *    Acceleration", abstract (dblp author listing on taxoreview.com): attention
 *    with 8-bit quantized Q and K.
 *  - The SageAttention2 abstract (same listing): P~
 *    and V quantized to FP8, and a two-level accumulation strategy for P~V.
 *  - "Flash Attention vs Sage Attention: Kernel Comparison", sections "How
 *    SageAttention uses quantization for more throughput" (Q, K to 8-bit before
 *    the matrix multiply, then precision-aware scaling), "How FlashAttention
 *    reduces memory traffic" (tiled online softmax) and the list of variables
 *    under "Attention kernel benchmarks" (causal masking changes which blocks are
 *    skipped).
 *
 * Entry points, by group
 *  - the path: sage_quantize_qk, sage_quantize_v, sage_attn_fwd (and their
 *    workspace queries); sage_attn_fwd_dump for tests; sage_quantize_qkv,
 *    the two quantize calls in one;
 *  - the extended shapes (_ex: layouts, grouped heads, Nq != Nkv);
 *  - decode over a quantized KV cache (blog section "FlashAttention for
 *    training and inference: where SageAttention fits": decode is bound by
 *    reading the cache): sage_quantize_q, sage_quantize_k,
 *    sage_decode_kv_chunk, sage_attn_decode_workspace_bytes, sage_attn_decode,
 *    sage_attn_decode_noalloc;
 *  - 4-bit QK^T (the SageAttention3 abstract: attention on FP4 matrix cores):
 *    sage_quantize_qk4, sage_attn_fwd_qk4(_dump), and with Q smoothing (the
 *    SageAttention2 abstract) sage_quantize_qk4_smooth_q,
 *    sage_attn_fwd_qk4_smooth_q(_dump); FP4 P~V as well: sage_quantize_v4,
 *    sage_attn_fwd_fp4(_dump).
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers owned by the caller; the library allocates
 *    nothing and keeps no state between calls (sage_attn_decode_noalloc
 *    alone uses a device array of the library's own, see there).  Every pointer must be 16-byte
 *    aligned; outputs must not alias inputs.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue
 *    work on it and return; no host synchronisation happens inside.
 *  - Return value: a sage_status.  Argument errors are detected before any work
 *    is enqueued; then no output is touched.  A failed kernel launch returns
 *    SAGE_ERR_HIP.  Faults during execution surface at the caller's next
 *    synchronisation, as for any HIP work.
 *  - Tensors are contiguous and row-major.  The plain entry points take
 *    self-attention shaped [B, H, N, d] tensors (the layout of PyTorch's
 *    scaled_dot_product_attention).  The _ex entry points also take
 *    [B, N, H, d] inputs and outputs (layout SAGE_LAYOUT_BNHD), Hq query heads
 *    sharing Hkv K/V heads (grouped heads: query head h reads K/V head
 *    h / (Hq/Hkv)), and Nq queries against Nkv keys.  The quantized codes and
 *    scales are always head-major, as documented below for H, N.
 *  - Lengths need not be block multiples.  Quantization blocks are runs of
 *    blk tokens from token 0 and the last one holds the N mod blk remaining
 *    tokens.  The code buffers are padded with zero codes: Q codes to
 *    Np = N rounded up to 128 rows, K and V codes to Nt = N rounded up to 64
 *    (one KV tile); a padding block gets scale 0.
 *  - Supported: d in {64, 128}; 1 <= N (Nq and Nkv) <= 524288; blk_q in
 *    {32, 64, 128}; blk_k in {16, 32, 64}; B*H >= 1; Hq a multiple of Hkv; causal only with
 *    Nkv >= Nq; sm_scale finite and > 0; inputs finite.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad dtype, bad sm_scale */
  SAGE_ERR_UNSUPPORTED = 2,   /* shape outside the supported set above */
  SAGE_ERR_MISALIGNED = 3,    /* a pointer is not 16-byte aligned */
  SAGE_ERR_HIP = 4,           /* a HIP call failed (launch error) */
  SAGE_ERR_WORKSPACE = 5      /* workspace too small */
};

enum { SAGE_F16 = 0, SAGE_BF16 = 1, SAGE_F32 = 2 };

/* Memory layout of the fp16/bf16 inputs and of O in the _ex entry points. */
enum { SAGE_LAYOUT_BHND = 0, SAGE_LAYOUT_BNHD = 1 };

/* Human-readable text of a status code (static storage). */
const char* sage_status_string(int status);

/* Width, in keys, of the KV tile of the online softmax: the running max is
 * updated and one FP8 inner P~V block is accumulated per tile. */
int sage_kv_tile(void);

/* Bytes of scratch memory sage_quantize_qk needs (int64 per-channel partial
 * sums of K, one row of d per 256 tokens of every head).  It depends on K
 * only: for sage_quantize_qk_ex pass H = Hkv and N = Nkv. */
size_t sage_quantize_qk_workspace_bytes(int B, int H, int N, int d);

/*
 * sage_quantize_qk -- smooth K and quantize Q and K to INT8 per block.
 * (SageAttention abstract; blog section "How SageAttention uses quantization
 * for more throughput".)
 *   k_mean[b,h,c] = mean over all N tokens of K[b,h,:,c], computed from the
 *     exact int64 sum of trunc(clamp(k, +-2^19) * 2^24) (order-free; at most
 *     2^62 in magnitude for N <= 2^19), divided in fp64 and rounded to fp32.
 *   Smoothed K: ks = fp32(k) - k_mean (fp32).
 *   Blocks of blk_q tokens of Q / blk_k tokens of ks, all d channels: a = max|x|;
 *     scale = a/127, r = 127/a (fp32, correctly rounded), code = rint(x*r)
 *     (ties to even) in [-127, 127]; a block with a < 2^-120 gets scale 0 and
 *     all-zero codes.
 * In:  Q, K        [B,H,N,d] float16 (in_dtype SAGE_F16) or bfloat16 (SAGE_BF16).
 * Out: q_codes     [B,H,Np,d] int8;  q_scale [B,H,Np/blk_q] fp32;
 *      k_codes     [B,H,Nt,d] int8;  k_scale [B,H,Nt/blk_k] fp32;
 *      k_mean      [B,H,d] fp32 (mean over the N tokens).
 *      (Np = N rounded up to 128, Nt = N rounded up to 64; padding rows hold
 *      zero codes.)
 * workspace: device scratch of at least sage_quantize_qk_workspace_bytes(...);
 *      contents on entry are ignored.
 */
int sage_quantize_qk(const void* Q, const void* K, int in_dtype, int B, int H, int N, int d, int blk_q,
                     int blk_k, int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale,
                     float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_quantize_qk_ex -- sage_quantize_qk for Q of Hq heads and Nq tokens, K of
 * Hkv heads and Nkv tokens (the mean of K runs over its own Nkv tokens), both
 * in `layout` (same quantization as above).
 * In:  Q [B,Hq,Nq,d] or [B,Nq,Hq,d]; K [B,Hkv,Nkv,d] or [B,Nkv,Hkv,d].
 * Out: q_codes [B,Hq,Nqp,d], q_scale [B,Hq,Nqp/blk_q], k_codes [B,Hkv,Nkt,d],
 *      k_scale [B,Hkv,Nkt/blk_k], k_mean [B,Hkv,d] (head-major whatever the
 *      layout; Nqp = Nq rounded up to 128, Nkt = Nkv rounded up to 64).
 *      workspace: sage_quantize_qk_workspace_bytes(B, Hkv, Nkv, d).
 */
int sage_quantize_qk_ex(const void* Q, const void* K, int in_dtype, int layout, int B, int Hq, int Hkv, int Nq,
                        int Nkv, int d, int blk_q, int blk_k, int8_t* q_codes, float* q_scale, int8_t* k_codes,
                        float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch memory sage_quantize_v needs (fp32 per-channel partial
 * maxima, one row of d per 256 tokens of every head, plus one row per head). */
size_t sage_quantize_v_workspace_bytes(int B, int H, int N, int d);

/*
 * sage_quantize_v -- V to FP8 e4m3 with one scale per channel of each head.
 * (SageAttention2 abstract: V quantized to FP8.)
 *   a_c = max over all N tokens of |V[b,h,:,c]|; v_scale = a_c/448,
 *   r_c = 448/a_c; code = e4m3(rn(v * r_c)) with round-to-nearest-even
 *   (a channel with a_c < 2^-120 gets scale 0 and zero codes).
 * In:  V       [B,H,N,d] float16 / bfloat16.
 * Out: v_codes e4m3 bytes in KV-tile channel-major order: for head (b,h),
 *              tile t of 64 consecutive tokens and channel c, the 64 codes of
 *              tokens 64t..64t+63 are contiguous at byte offset
 *              (((b*H + h)*Nt/64 + t)*d + c)*64 (Nt = N rounded up to 64;
 *              tokens at or past N get code 0).
 *      v_scale [B,H,d] fp32.
 */
int sage_quantize_v(const void* V, int in_dtype, int B, int H, int N, int d, uint8_t* v_codes, float* v_scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_quantize_v_ex -- sage_quantize_v with V in `layout`: [B,H,N,d] or
 * [B,N,H,d] (H = Hkv, N = Nkv of the attention).  v_codes and v_scale as above.
 */
int sage_quantize_v_ex(const void* V, int in_dtype, int layout, int B, int H, int N, int d, uint8_t* v_codes,
                       float* v_scale, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of scratch memory sage_quantize_qkv needs: the K channel sums of
 * sage_quantize_qk and the V channel maxima of sage_quantize_v (0 for a bad
 * shape). */
size_t sage_quantize_qkv_workspace_bytes(int B, int Hkv, int Nkv, int d);

/*
 * sage_quantize_qkv -- sage_quantize_qk_ex and sage_quantize_v_ex of the same
 * K/V heads in one call: the same outputs bit for bit (the same kernels'
 * arithmetic) in three launches instead of six.  Pass 1 quantizes the Q
 * blocks and takes the per-chunk K channel sums and V channel maxima, the
 * finalize step the K means and V scales, pass 2 the smoothed K blocks and
 * the V tiles; fewer, larger launches keep the HBM-bound passes busy on short
 * sequences.  Arguments as the two calls (V in `layout` with Hkv heads of Nkv
 * tokens, like K); workspace: sage_quantize_qkv_workspace_bytes(B, Hkv, Nkv,
 * d) bytes, contents ignored.
 */
int sage_quantize_qkv(const void* Q, const void* K, const void* V, int in_dtype, int layout, int B, int Hq, int Hkv,
                      int Nq, int Nkv, int d, int blk_q, int blk_k, int8_t* q_codes, float* q_scale, int8_t* k_codes,
                      float* k_scale, float* k_mean, uint8_t* v_codes, float* v_scale, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd -- attention forward on the quantized operands.
 * (Tiled online softmax: blog section "How FlashAttention reduces memory
 * traffic"; FP8 P~ and two-level P~V accumulation: SageAttention2 abstract;
 * causal block skipping: blog, variables under "Attention kernel benchmarks".)
 * For query row i, KV tiles of sage_kv_tile() keys are visited in ascending
 * order (the last one may be partial; causal: only tiles holding a key
 * j <= i; key j is visible iff j <= i):
 *   S_j    = sum_c q_codes[i,c] k_codes[j,c]               (int32, exact)
 *   c2     = (q_scale * k_scale_j) * (sm_scale * log2 e)   (fp32, in this order)
 *   m'     = max(m, max_j fp32(S_j) * c2)
 *   alpha  = exp2(m - m')   (0 on the first tile)
 *   K      = fma(B, c2, m' - 8),  B = 1.5 * 2^23            (fp32)
 *   P~_j   = exp2(fma(B + S_j, c2, -K))                    (P~ scaled by 2^8)
 *            (= exp2 of S_j c2 - (m' - 8), the offset rounded at the size of
 *            B c2: B + S_j is exact in fp32, and the score accumulators start
 *            at the bits of B so that no conversion per score is needed)
 *   P^_j   = e4m3(P~_j)
 *   l      = fma(alpha, l, sum_j P^_j)                     (FP8 matrix cores)
 *   O_blk  = sum_j P^_j * v_code_j                         (FP8 matrix cores)
 *   O_acc  = alpha * O_acc + O_blk;  m = m'
 *   O[i,c] = O_acc[c] * v_scale[c] / l
 * exp2 is the hardware's fp32 exp2 instruction (v_exp_f32, about 1 ulp), so
 *   an FP8 code of P~ may differ by one step from one computed with exp2
 *   rounded once from the exact value.  O_blk and the row sum of the codes
 *   are the FP8 instruction's sums of the tile's 64 products: it adds each
 *   group of 8 within about 13 bits of the group's largest product, then the
 *   block sum enters the fp32 accumulator (O_acc is its C operand).
 * In:  the outputs of sage_quantize_qk (q_codes, q_scale, k_codes, k_scale)
 *      and sage_quantize_v (v_codes, v_scale), same B, H, N, d, blk_q, blk_k.
 * Out: O [B,H,N,d] of out_dtype (SAGE_F32, SAGE_F16 or SAGE_BF16; rounded to
 *      nearest even from fp32).
 */
int sage_attn_fwd(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                  const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int B, int H, int N, int d,
                  int blk_q, int blk_k, int causal, float sm_scale, void* stream);

/*
 * sage_attn_fwd_ex -- sage_attn_fwd with Hq query heads on Hkv K/V heads
 * (query head h reads K/V head h / (Hq/Hkv)), Nq queries on Nkv keys, and O
 * in `layout`.  Query row i is aligned with key i + (Nkv - Nq) (the queries
 * are the last Nq positions of the sequence): under the causal mask key j is
 * visible iff j <= i + Nkv - Nq, which needs Nkv >= Nq.
 * In:  the outputs of sage_quantize_qk_ex and sage_quantize_v_ex for the same
 *      B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k.
 * Out: O [B,Hq,Nq,d] (SAGE_LAYOUT_BHND) or [B,Nq,Hq,d] (SAGE_LAYOUT_BNHD).
 */
int sage_attn_fwd_ex(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                     const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq,
                     int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale, void* stream);

/*
 * sage_attn_fwd_dump -- sage_attn_fwd through the same kernel code, which in
 * addition writes the int32 scores and the FP8 codes of P~ of selected
 * 128-query tiles (test and diagnostic use).
 * sel:    n_sel device int32 ids (b*H + h) * ceil(N/128) + qt of query tiles.
 * s_dump: [n_sel, 128, N] int32; entry (k, r, j) = S for query qt*128 + r and
 *         key j, for every key of every KV tile the kernel computed for that
 *         query's 32-row group (other entries are left untouched).
 * p_dump: [n_sel, 128, N] uint8 e4m3 codes of P~ (0 for keys not visible),
 *         same coverage.
 */
int sage_attn_fwd_dump(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                       const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int B, int H, int N,
                       int d, int blk_q, int blk_k, int causal, float sm_scale, const int32_t* sel, int n_sel,
                       int32_t* s_dump, uint8_t* p_dump, void* stream);

/*
 * sage_attn_fwd_ex_dump -- sage_attn_fwd_ex with the dumps of
 * sage_attn_fwd_dump: sel ids are (b*Hq + h) * ceil(Nq/128) + qt; s_dump and
 * p_dump are [n_sel, 128, Nkv].
 */
int sage_attn_fwd_ex_dump(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                          const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B,
                          int Hq, int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale,
                          const int32_t* sel, int n_sel, int32_t* s_dump, uint8_t* p_dump, void* stream);

/*
 * sage_quantize_q -- the Q part of sage_quantize_qk_ex alone: INT8 blocks of
 * blk_q tokens of Q [B,Hq,Nq,d] or [B,Nq,Hq,d].  Out: q_codes [B,Hq,Nqp,d],
 * q_scale [B,Hq,Nqp/blk_q] as there.  No workspace.  (For decode: the new
 * queries are quantized on their own, the K/V cache once.)
 */
int sage_quantize_q(const void* Q, int in_dtype, int layout, int B, int Hq, int Nq, int d, int blk_q,
                    int8_t* q_codes, float* q_scale, void* stream);

/*
 * sage_quantize_k -- the K part of sage_quantize_qk_ex alone (mean over the
 * Nkv tokens, smoothed INT8 blocks of blk_k keys).  Out: k_codes
 * [B,Hkv,Nkt,d], k_scale [B,Hkv,Nkt/blk_k], k_mean [B,Hkv,d].  workspace:
 * sage_quantize_qk_workspace_bytes(B, Hkv, Nkv, d).
 */
int sage_quantize_k(const void* K, int in_dtype, int layout, int B, int Hkv, int Nkv, int d, int blk_k,
                    int8_t* k_codes, float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Default keys per split of sage_attn_decode for this shape: a multiple of
 * sage_kv_tile(), giving as many splits as fit one round of waves (one wave
 * per SIMD, 1024 on MI355X), at least one tile each; 0 for a bad shape. */
int sage_decode_kv_chunk(int B, int Hq, int Hkv, int Nq, int Nkv, int d);

/* Bytes of scratch memory sage_attn_decode needs (fp32 partial states, one
 * [32][d + 2] block per wave of work); kv_chunk 0 = the default.  0 for a bad
 * shape or chunk. */
size_t sage_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int kv_chunk);

/*
 * sage_attn_decode -- sage_attn_fwd_ex for few queries against a long
 * quantized K/V cache, split over the keys (the pages note that decode is
 * bound by reading the KV cache).  The Nkv keys are cut into splits of
 * kv_chunk keys (a multiple of sage_kv_tile(); 0 = sage_decode_kv_chunk).
 * For every query row each split runs the tiled online softmax of
 * sage_attn_fwd from a fresh state, giving (m_c, l_c, O_acc,c); the splits
 * with a visible key are then merged in ascending order:
 *   m* = max m_c,  w_c = exp2(m_c - m*),  L = sum w_c l_c,
 *   O' = sum w_c O_acc,c  (fp32 fma),  O = O' * v_scale / L.
 * The FP8 codes of P~ therefore depend on kv_chunk (each split has its own
 * running max); with one split the result is that of sage_attn_fwd_ex.
 * Work: one wave per (batch, K/V head, group of 32 query rows, split); the
 * Hq/Hkv query heads of a K/V head and their Nq queries share the group, so
 * each K/V byte is read once per group.  Arguments as sage_attn_fwd_ex, plus
 * workspace: sage_attn_decode_workspace_bytes(...) bytes, contents ignored.
 */
int sage_attn_decode(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                     const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq,
                     int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale,
                     int kv_chunk, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device scratch array of sage_attn_decode_noalloc (one per
 * device): the chunk states of 2016 waves of work at d = 128, 3968 at d = 64. */
#define SAGE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * sage_attn_decode_noalloc -- sage_attn_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments and result as
 * sage_attn_decode without the workspace: the chunk states go to a device
 * array inside the library, SAGE_NOALLOC_SCRATCH_BYTES on each device, which
 * that device holds until the process ends.  Its address is looked up on the
 * first call on each device; nothing is allocated, set or synchronised.
 * Errors: SAGE_ERR_WORKSPACE (before anything is enqueued) when
 * sage_attn_decode_workspace_bytes(...) of the shape and kv_chunk exceeds
 * SAGE_NOALLOC_SCRATCH_BYTES; SAGE_ERR_INVALID_ARG when `stream` is not a
 * stream of the current device; the argument errors of sage_attn_decode.
 * The array keeps the last call's contents and needs no clearing (a call
 * writes every state before reading it).  All calls on one GPU share it:
 * calls that overlap on one GPU (on different streams or host threads) race
 * and give wrong results, so issue them in order on one stream.
 */
int sage_attn_decode_noalloc(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                             const float* k_scale, const uint8_t* v_codes, const float* v_scale, void* O,
                             int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int blk_q,
                             int blk_k, int causal, float sm_scale, int kv_chunk, void* stream);

/*
 * sage_quantize_qk4 -- Q and smoothed K to 4-bit E2M1 for sage_attn_fwd_qk4
 * (SageAttention3 abstract: attention on FP4 matrix cores; here the FP4
 * matrix instruction multiplies E2M1 values with one power-of-two scale per
 * 32 values along d).  The K mean is that of sage_quantize_qk.  Every token
 * row is cut into blocks of 32 channels: E = floor(log2(max|x|)) - 2 clamped
 * to [-127, 127], stored as the scale byte E + 127 (E8M0); codes =
 * E2M1(x / 2^E), round to nearest with ties to the even code, saturating at 6
 * (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 by code 0..7, bit 3 the sign); an
 * all-zero block gets scale byte 0.
 * Out: q4_codes [B,Hq,Nqp,d/2] bytes (two codes per byte, the even channel in
 *      the low nibble), q4_scale [B,Hq,Nqp,d/32] bytes, k4_codes [B,Hkv,Nkt,d/2],
 *      k4_scale [B,Hkv,Nkt,d/32], k_mean [B,Hkv,d] fp32; padding rows zero.
 * workspace: sage_quantize_qk_workspace_bytes(B, Hkv, Nkv, d).
 */
int sage_quantize_qk4(const void* Q, const void* K, int in_dtype, int layout, int B, int Hq, int Hkv, int Nq,
                      int Nkv, int d, uint8_t* q4_codes, uint8_t* q4_scale, uint8_t* k4_codes, uint8_t* k4_scale,
                      float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd_qk4 -- sage_attn_fwd_ex with the scores from the 4-bit codes:
 *   S_j = sum over blocks b of 2^(Eq_b + Ek_b) * sum_{c in b} q_c k_c
 * on the FP4 matrix cores (fp32; exact products, fp32 accumulation), and the
 * dequantization factor c2 = sm_scale * log2 e for every key; FP8 P~ (V from
 * sage_quantize_v_ex) and the two-level P~V as in sage_attn_fwd.  The scores
 * are fp32 already, so P~_j = exp2(fma(S_j, c2, -(m' - 8))), and l sums the
 * fp32 P~ on the vector ALU: l = fma(alpha, l, sum_j P~_j).
 * The 4-bit scores are coarser than INT8 (about three bits fewer).
 */
int sage_attn_fwd_qk4(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                      const uint8_t* k4_scale, const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype,
                      int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal, float sm_scale,
                      void* stream);

/* sage_attn_fwd_qk4_dump -- sage_attn_fwd_qk4 with the dumps of
 * sage_attn_fwd_ex_dump; s_dump holds the fp32 scores' bit patterns. */
int sage_attn_fwd_qk4_dump(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                           const uint8_t* k4_scale, const uint8_t* v_codes, const float* v_scale, void* O,
                           int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                           float sm_scale, const int32_t* sel, int n_sel, int32_t* s_dump, uint8_t* p_dump,
                           void* stream);

/*
 * sage_quantize_qk4_smooth_q -- sage_quantize_qk4 with Q smoothing
 * (SageAttention2 abstract: Q is smoothed to make the low-bit QK^T
 * accurate).  The queries of each head are cut into blocks of 32 rows (the
 * last block holds the Nq mod 32 remaining rows); the block mean
 *   q_mean[c] = fp32( (fp64 sum over the block's rows, ascending) / rows )
 * is subtracted in fp32 before the E2M1 blocks are formed, and returns in
 * the scores (sage_attn_fwd_qk4_smooth_q) as the mean against K, both in
 * INT8 with one power-of-two scale 2^E per block: the mean per block of 32
 * queries over all d channels, the smoothed K (the values of k4_codes) per
 * block of 64 keys (one KV tile) over all d channels;
 *   E = the smallest exponent in [-63, 52] with max|x| * 2^-E <= 127 (an
 *   all-zero block: -63), exponent byte E + 127, codes = RN(x * 2^-E) ties
 *   to even, saturated at +-127 (reached only at the upper clamp).
 * Out, besides those of sage_quantize_qk4:
 *   q_mean [B,Hq,Nqp/32,d] fp32 (Nqp = Nq rounded up to 128; padding blocks 0),
 *   qm_codes [B,Hq,Nqp/32,d] int8, qm_scale [B,Hq,Nqp/32] exponent bytes,
 *   k8_codes [B,Hkv,Nkt,d] int8 (padding keys 0), k8_scale [B,Hkv,Nkt/64]
 *   exponent bytes.
 * The five smoothing pointers are all null (plain sage_quantize_qk4) or all
 * valid (SAGE_ERR_INVALID_ARG otherwise).
 */
int sage_quantize_qk4_smooth_q(const void* Q, const void* K, int in_dtype, int layout, int B, int Hq, int Hkv,
                               int Nq, int Nkv, int d, uint8_t* q4_codes, uint8_t* q4_scale, uint8_t* k4_codes,
                               uint8_t* k4_scale, float* k_mean, float* q_mean, int8_t* qm_codes,
                               uint8_t* qm_scale, int8_t* k8_codes, uint8_t* k8_scale, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd_qk4_smooth_q -- sage_attn_fwd_qk4 on smoothed codes: the
 * score of query row i (block m = i / 32) and key j (block t = j / 64) is
 *   S_ij = sum_b 2^(Eq_b + Ek_b) q4_i . k4_j over block b
 *        + 2^(Em + Ek8_t) qm_m . k8_j
 * where the second dot product is the exact int32 sum of the INT8 codes
 * (INT8 matrix core), made fp32 exactly, and the first is added to it on the
 * FP4 matrix core (fp32 accumulation); the rest as sage_attn_fwd_qk4.  Null
 * smoothing pointers: SAGE_ERR_INVALID_ARG.
 */
int sage_attn_fwd_qk4_smooth_q(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                               const uint8_t* k4_scale, const int8_t* qm_codes, const uint8_t* qm_scale,
                               const int8_t* k8_codes, const uint8_t* k8_scale, const uint8_t* v_codes,
                               const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq, int Hkv,
                               int Nq, int Nkv, int d, int causal, float sm_scale, void* stream);

/* sage_attn_fwd_qk4_smooth_q_dump -- sage_attn_fwd_qk4_smooth_q with the
 * dumps of sage_attn_fwd_qk4_dump. */
int sage_attn_fwd_qk4_smooth_q_dump(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                                    const uint8_t* k4_scale, const int8_t* qm_codes, const uint8_t* qm_scale,
                                    const int8_t* k8_codes, const uint8_t* k8_scale, const uint8_t* v_codes,
                                    const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq, int Hkv,
                                    int Nq, int Nkv, int d, int causal, float sm_scale, const int32_t* sel, int n_sel,
                                    int32_t* s_dump, uint8_t* p_dump, void* stream);

/*
 * sage_quantize_v4 -- V to FP4 for FP4 P~V (SageAttention3 abstract:
 * attention on FP4 matrix cores), in the OCP Microscaling formats' MXFP4:
 * E2M1 elements with one E8M0 scale per channel and block of 32 consecutive
 * tokens of a head (the last block holds the rest, padding tokens zero):
 *   E = floor(log2(max|v|)) - 2 clamped to [-127, 127], scale byte E + 127,
 *   codes = E2M1(v / 2^E) round to nearest even, saturating at 6 (sign
 *   kept); an all-zero block gets scale byte 0 and zero codes.
 * In:  V [B,H,N,d] or [B,N,H,d] (layout), fp16/bf16 (in_dtype).
 * Out: v4_codes [B,H,Nkt,d,32] bytes (Nkt = N rounded up to the KV tile of
 *      64 tokens: per tile, d channel rows of its 64 codes, two tokens per
 *      byte, the lower token in the low nibble);
 *      v4_scale [B,H,Nkt/64,2,32,d/32] bytes (per tile, byte (g, m, c) is
 *      the scale of channel 32c + m over tokens 32g .. 32g+31).
 * Allocates nothing; no workspace.  Errors as sage_quantize_v.
 */
int sage_quantize_v4(const void* V, int in_dtype, int layout, int B, int H, int N, int d, uint8_t* v4_codes,
                     uint8_t* v4_scale, void* stream);

/*
 * sage_attn_fwd_fp4 -- FP4 attention: the 4-bit scores of sage_attn_fwd_qk4
 * and P~V in FP4 as well (all matrix work on the FP4 instructions).  Per
 * row and KV tile, each 32-key half is one MX block of P~ with exponent
 *   E = floor(max over its visible keys of the exp2 argument) - 2
 *   clamped to [-126, 127] (no visible key: -126),
 * P^ = E2M1(P~ / 2^E) (round to nearest even, saturating; the hardware's
 * fp32 exp2), the tile's row sum is that of the decoded P^ 2^E (as the
 * weights of the product), P^V accumulates in fp32 with the block sum as
 * the inner level, and O = O_acc / l.  V from sage_quantize_v4 (the K/V
 * head of each query head as sage_attn_fwd_ex).  Other arguments and
 * errors as sage_attn_fwd_qk4; null V pointers: SAGE_ERR_INVALID_ARG.
 */
int sage_attn_fwd_fp4(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                      const uint8_t* k4_scale, const uint8_t* v4_codes, const uint8_t* v4_scale, void* O,
                      int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                      float sm_scale, void* stream);

/* sage_attn_fwd_fp4_dump -- sage_attn_fwd_fp4 with the dumps of
 * sage_attn_fwd_qk4_dump, the P~ codes as E2M1 codes (0..15). */
int sage_attn_fwd_fp4_dump(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                           const uint8_t* k4_scale, const uint8_t* v4_codes, const uint8_t* v4_scale, void* O,
                           int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                           float sm_scale, const int32_t* sel, int n_sel, int32_t* s_dump, uint8_t* p_dump,
                           void* stream);

/*
 * sage_probe_mfma_peak -- a measurement aid, not a step of the method: each of
 * `workgroups` workgroups of 256 threads (2 per CU, the attention kernel's
 * occupancy at d = 128) runs `iters` iterations of the matrix instructions
 * one d = 128 KV tile costs a wave of the attention kernel (8 INT8
 * 32x32x32 and 4 FP8 32x32x64 instructions, 2^20 operations a wave) and
 * nothing else.  Operation count 4 * 2^20 * workgroups * iters; divided by
 * the launch's time it gives the sustained dense INT8/FP8 matrix rate of the
 * chip.  sink: null, or device memory for workgroups * 256 ints that
 * receives a checksum per thread.  Enqueued on `stream`;
 * errors: SAGE_ERR_INVALID_ARG (workgroups outside 1..65536, iters outside
 * 1..2^24), SAGE_ERR_MISALIGNED, SAGE_ERR_HIP.
 */
int sage_probe_mfma_peak(int workgroups, int iters, int* sink, void* stream);

/*
 * sage_probe_hbm_read -- a measurement aid, not a step of the method: reads
 * `bytes` of device memory at `buf` once with 16-byte streaming loads (1024
 * workgroups of 256 threads, each over one contiguous span, eight loads in
 * flight per thread) and writes one checksum per thread to sink (device
 * memory for 1024 * 256 ints).  bytes / the
 * launch's time is the sustained HBM read bandwidth when bytes is well above
 * the caches (1 GiB and more): the measured ceiling for the HBM-bound passes
 * (quantization, decode).  Enqueued on `stream`; errors: SAGE_ERR_INVALID_ARG
 * (null pointer, bytes not a positive multiple of 16), SAGE_ERR_MISALIGNED,
 * SAGE_ERR_HIP.
 */
int sage_probe_hbm_read(const void* buf, size_t bytes, int* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H */
