// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sage {

// Input tensors are [B,H,N,d] (nhd = 0) or [B,N,H,d] (nhd = 1); Q has Hq
// heads of Nq tokens, K and V have Hkv heads of Nkv tokens.  Codes and scales
// are always head-major.
struct QuantQKArgs {
  const void* Q;
  const void* K;
  int is_bf16, nhd;
  int B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k;
  int8_t* q_codes;
  float* q_scale;
  int8_t* k_codes;
  float* k_scale;
  float* k_mean;
  void* workspace;
};

struct QuantVArgs {
  const void* V;
  int is_bf16, nhd;
  int B, H, N, d;
  uint8_t* v_codes;
  float* v_scale;
  void* workspace;
};

struct AttnArgs {
  const int8_t* q_codes;
  const float* q_scale;
  const int8_t* k_codes;
  const float* k_scale;
  const uint8_t* v_codes;
  const float* v_scale;
  void* O;
  int out_dtype, nhd;   // O layout: [B,Hq,Nq,d] (0) or [B,Nq,Hq,d] (1)
  int B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, causal;
  float s2;   // fp32(sm_scale * log2 e)
  // 4-bit QK^T instead of INT8 (q4_codes != nullptr): codes and scales as in Quant4Args
  const uint8_t* q4_codes = nullptr;
  const uint8_t* q4_scale = nullptr;
  const uint8_t* k4_codes = nullptr;
  const uint8_t* k4_scale = nullptr;
  // with Q smoothing of the 4-bit scores (qm_codes != nullptr): the INT8 block
  // means of Q [B,Hq,Nqp/32,d] with exponent bytes [B,Hq,Nqp/32], and the
  // smoothed K in INT8 [B,Hkv,Nkt,d] with one exponent byte per 64-key tile
  // [B,Hkv,Nkt/64] (scale 2^(byte - 127))
  const int8_t* qm_codes = nullptr;
  const uint8_t* qm_scale = nullptr;
  const int8_t* k8_codes = nullptr;
  const uint8_t* k8_scale = nullptr;
  // FP4 P~V (v4_codes != nullptr, with the 4-bit scores): V in E2M1 tiles and
  // their E8M0 scales as in QuantV4Args; v_codes / v_scale unused
  const uint8_t* v4_codes = nullptr;
  const uint8_t* v4_scale = nullptr;
  // dump (test) mode
  const int32_t* sel;
  int n_sel;
  int32_t* s_dump;
  uint8_t* p_dump;
};

// 4-bit Q and smoothed K (E2M1, one power-of-two scale per 32 channels).
struct Quant4Args {
  const void* Q;
  const void* K;
  int is_bf16, nhd;
  int B, Hq, Hkv, Nq, Nkv, d;
  uint8_t* q4_codes;   // [B,Hq,Nqp,d/2] packed nibbles
  uint8_t* q4_scale;   // [B,Hq,Nqp,d/32]
  uint8_t* k4_codes;   // [B,Hkv,Nkt,d/2]
  uint8_t* k4_scale;   // [B,Hkv,Nkt,d/32]
  float* k_mean;
  // Q smoothing (all null: none): block means of 32 queries [B,Hq,Nqp/32,d]
  // fp32, their INT8 codes [B,Hq,Nqp/32,d] and exponent bytes [B,Hq,Nqp/32],
  // and the smoothed K in INT8 [B,Hkv,Nkt,d] with one exponent byte per
  // 64-key tile [B,Hkv,Nkt/64]
  float* q_mean = nullptr;
  int8_t* qm_codes = nullptr;
  uint8_t* qm_scale = nullptr;
  int8_t* k8_codes = nullptr;
  uint8_t* k8_scale = nullptr;
  void* workspace;     // quantize_qk_workspace(B*Hkv, Nkv, d) bytes
};
void launch_quantize_qk4(const Quant4Args& a, hipStream_t st);

// V in E2M1 (MXFP4) for FP4 P~V: per channel and block of 32 tokens one E8M0
// scale; codes as KV tiles of d channel rows of 32 bytes (two tokens per
// byte, low nibble first) [B,H,Nkt,d,32]; scales per tile permuted for the
// attention kernel, [B,H,Nkt/64,2,32,d/32] (byte (g, m, c) for channel
// 32c + m and tokens 32g .. 32g+31 of the tile); padding tokens zero.
struct QuantV4Args {
  const void* V;
  int is_bf16, nhd;
  int B, H, N, d;
  uint8_t* v4_codes;
  uint8_t* v4_scale;
};
void launch_quantize_v4(const QuantV4Args& a, hipStream_t st);

// Decode over a quantized KV cache: split-KV chunks of kv_chunk keys, merged.
struct DecodeArgs {
  const int8_t* q_codes;
  const float* q_scale;
  const int8_t* k_codes;
  const float* k_scale;
  const uint8_t* v_codes;
  const float* v_scale;
  void* O;
  int out_dtype, nhd;
  int B, Hq, Hkv, Nq, Nkv, d, blk_q, blk_k, causal, kv_chunk;
  float s2;
  void* workspace;   // decode_workspace(...) bytes of partial chunk states
};

// with_q / with_k: quantize Q (blocks), K (mean, smoothed blocks), or both
void launch_quantize_qk(const QuantQKArgs& a, hipStream_t st, bool with_q = true, bool with_k = true);
void launch_quantize_v(const QuantVArgs& a, hipStream_t st);
// quantize_qk and quantize_v of one K/V (v.H = a.Hkv, v.N = a.Nkv, same layout and
// dtype) in three launches; a.workspace and v.workspace as for the two calls
void launch_quantize_qkv(const QuantQKArgs& a, const QuantVArgs& v, hipStream_t st);
void launch_attn_fwd(const AttnArgs& a, bool dump, hipStream_t st);
size_t quantize_qk_workspace(int BHkv, int Nkv, int d);
size_t quantize_v_workspace(int BH, int N, int d);
void launch_attn_decode(const DecodeArgs& a, hipStream_t st);
int decode_default_chunk(int B, int Hq, int Hkv, int Nq, int Nkv);
size_t decode_workspace(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int kv_chunk);

}  // namespace sage
