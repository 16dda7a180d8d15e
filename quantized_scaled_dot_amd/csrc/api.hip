// C ABI of libsage.so: argument validation, then kernel launches on the
// caller's stream.  No allocation and no host synchronisation; the only
// global state is the per-device address of the allocation-free decode's
// scratch array.
#include <math.h>

#include <mutex>

#include "../../include/sage.h"
#include "common.h"
#include "launch.h"

namespace {

#define SAGE_TRY(x)          \
  do {                       \
    int _s = (x);            \
    if (_s != SAGE_OK) return _s; \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return SAGE_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SAGE_ERR_UNSUPPORTED;
  if (N > (1 << 19)) return SAGE_ERR_UNSUPPORTED;
  const long long bh = (long long)B * H;
  // flattened 1-D grids: ceil(N/64) * B*H workgroups must fit in a grid dimension
  if (bh * ((N + sage::kKTile - 1) / sage::kKTile) > 0x7fffffffLL) return SAGE_ERR_UNSUPPORTED;
  return SAGE_OK;
}

// Query heads Hq of Nq tokens, K/V heads Hkv of Nkv tokens, one memory layout.
int check_shapes(int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d) {
  if (layout != SAGE_LAYOUT_BHND && layout != SAGE_LAYOUT_BNHD) return SAGE_ERR_INVALID_ARG;
  SAGE_TRY(check_shape(B, Hq, Nq, d));
  SAGE_TRY(check_shape(B, Hkv, Nkv, d));
  if (Hq % Hkv != 0) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

// Quantization block sizes: Q blocks of 32 (one wave's rows), 64 or 128
// tokens; K blocks of 16, 32 or 64 keys (a quarter, half or whole KV tile).
int check_blocks(int blk_q, int blk_k) {
  if (blk_q != 32 && blk_q != 64 && blk_q != 128) return SAGE_ERR_UNSUPPORTED;
  if (blk_k != 16 && blk_k != 32 && blk_k != 64) return SAGE_ERR_UNSUPPORTED;
  return SAGE_OK;
}

int check_in_dtype(int dt) { return (dt == SAGE_F16 || dt == SAGE_BF16) ? SAGE_OK : SAGE_ERR_INVALID_ARG; }

int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

#define SAGE_PTR(p)                                    \
  do {                                                 \
    if ((p) == nullptr) return SAGE_ERR_INVALID_ARG;   \
    if (!aligned16(p)) return SAGE_ERR_MISALIGNED;     \
  } while (0)

// q4 (4-bit QK^T): q_codes/k_codes/q_scale/k_scale are unused and the four q4 pointers are the operands
struct Q4Ptrs {
  const uint8_t* q4_codes;
  const uint8_t* q4_scale;
  const uint8_t* k4_codes;
  const uint8_t* k4_scale;
  // Q smoothing (all four or none)
  const int8_t* qm_codes = nullptr;
  const uint8_t* qm_scale = nullptr;
  const int8_t* k8_codes = nullptr;
  const uint8_t* k8_scale = nullptr;
  // FP4 P~V (both or none; v_codes / v_scale are then unused)
  const uint8_t* v4_codes = nullptr;
  const uint8_t* v4_scale = nullptr;
};

int attn_common(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq,
                int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale,
                const int32_t* sel, int n_sel, int32_t* s_dump, uint8_t* p_dump, bool dump, void* stream,
                const Q4Ptrs* q4 = nullptr) {
  SAGE_TRY(check_shapes(layout, B, Hq, Hkv, Nq, Nkv, d));
  SAGE_TRY(check_blocks(blk_q, blk_k));
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (causal && Nkv < Nq) return SAGE_ERR_INVALID_ARG;   // the first rows would see no key
  if (!(sm_scale > 0.0f) || isinf(sm_scale)) return SAGE_ERR_INVALID_ARG;
  if (q4) {
    SAGE_PTR(q4->q4_codes); SAGE_PTR(q4->q4_scale); SAGE_PTR(q4->k4_codes); SAGE_PTR(q4->k4_scale);
    if (q4->qm_codes || q4->qm_scale || q4->k8_codes || q4->k8_scale) {
      SAGE_PTR(q4->qm_codes); SAGE_PTR(q4->qm_scale); SAGE_PTR(q4->k8_codes); SAGE_PTR(q4->k8_scale);
    }
  } else {
    SAGE_PTR(q_codes); SAGE_PTR(q_scale); SAGE_PTR(k_codes); SAGE_PTR(k_scale);
  }
  if (q4 && q4->v4_codes) {
    SAGE_PTR(q4->v4_codes); SAGE_PTR(q4->v4_scale);
  } else {
    SAGE_PTR(v_codes); SAGE_PTR(v_scale);
  }
  SAGE_PTR(O);
  if (dump) {
    if (n_sel < 0) return SAGE_ERR_INVALID_ARG;
    if (n_sel > 0) { SAGE_PTR(sel); SAGE_PTR(s_dump); SAGE_PTR(p_dump); }
  }
  sage::AttnArgs a;
  a.q_codes = q_codes; a.q_scale = q_scale; a.k_codes = k_codes; a.k_scale = k_scale;
  a.v_codes = v_codes; a.v_scale = v_scale; a.O = O; a.out_dtype = out_dtype; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv; a.d = d; a.blk_q = blk_q; a.blk_k = blk_k;
  a.causal = causal;
  a.s2 = sm_scale * sage::kLog2e;
  a.sel = dump ? sel : nullptr; a.n_sel = dump ? n_sel : 0; a.s_dump = s_dump; a.p_dump = p_dump;
  if (q4) {
    a.q4_codes = q4->q4_codes; a.q4_scale = q4->q4_scale; a.k4_codes = q4->k4_codes; a.k4_scale = q4->k4_scale;
    a.qm_codes = q4->qm_codes; a.qm_scale = q4->qm_scale; a.k8_codes = q4->k8_codes; a.k8_scale = q4->k8_scale;
    a.v4_codes = q4->v4_codes; a.v4_scale = q4->v4_scale;
  }
  (void)hipGetLastError();
  sage::launch_attn_fwd(a, dump, (hipStream_t)stream);
  return launch_status();
}

}  // namespace

extern "C" {

const char* sage_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID_ARG:
      return "SAGE_ERR_INVALID_ARG: null pointer, bad size, dtype, layout or sm_scale, Hq not a multiple of Hkv, "
             "or causal with Nq > Nkv";
    case SAGE_ERR_UNSUPPORTED:
      return "SAGE_ERR_UNSUPPORTED: shape outside d in {64,128}, N <= 2^19 (Nq and Nkv), blk_q in {32,64,128}, "
             "blk_k in {16,32,64}";
    case SAGE_ERR_MISALIGNED: return "SAGE_ERR_MISALIGNED: pointer not 16-byte aligned";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP: kernel launch failed";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE: workspace too small";
    default: return "SAGE_ERR_UNKNOWN";
  }
}

int sage_kv_tile(void) { return sage::kKTile; }

size_t sage_quantize_qk_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != SAGE_OK) return 0;
  return sage::quantize_qk_workspace(B * H, N, d);
}

size_t sage_quantize_v_workspace_bytes(int B, int H, int N, int d) {
  if (check_shape(B, H, N, d) != SAGE_OK) return 0;
  return sage::quantize_v_workspace(B * H, N, d);
}

int sage_quantize_qk_ex(const void* Q, const void* K, int in_dtype, int layout, int B, int Hq, int Hkv, int Nq,
                        int Nkv, int d, int blk_q, int blk_k, int8_t* q_codes, float* q_scale, int8_t* k_codes,
                        float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes, void* stream) {
  SAGE_TRY(check_shapes(layout, B, Hq, Hkv, Nq, Nkv, d));
  SAGE_TRY(check_in_dtype(in_dtype));
  SAGE_TRY(check_blocks(blk_q, blk_k));
  SAGE_PTR(Q); SAGE_PTR(K); SAGE_PTR(q_codes); SAGE_PTR(q_scale); SAGE_PTR(k_codes); SAGE_PTR(k_scale);
  SAGE_PTR(k_mean); SAGE_PTR(workspace);
  if (workspace_bytes < sage::quantize_qk_workspace(B * Hkv, Nkv, d)) return SAGE_ERR_WORKSPACE;
  sage::QuantQKArgs a;
  a.Q = Q; a.K = K; a.is_bf16 = in_dtype == SAGE_BF16; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv; a.d = d; a.blk_q = blk_q; a.blk_k = blk_k;
  a.q_codes = q_codes; a.q_scale = q_scale; a.k_codes = k_codes; a.k_scale = k_scale; a.k_mean = k_mean;
  a.workspace = workspace;
  (void)hipGetLastError();
  sage::launch_quantize_qk(a, (hipStream_t)stream);
  return launch_status();
}

int sage_quantize_qk(const void* Q, const void* K, int in_dtype, int B, int H, int N, int d, int blk_q, int blk_k,
                     int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale, float* k_mean, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return sage_quantize_qk_ex(Q, K, in_dtype, SAGE_LAYOUT_BHND, B, H, H, N, N, d, blk_q, blk_k, q_codes, q_scale,
                             k_codes, k_scale, k_mean, workspace, workspace_bytes, stream);
}

int sage_quantize_v_ex(const void* V, int in_dtype, int layout, int B, int H, int N, int d, uint8_t* v_codes,
                       float* v_scale, void* workspace, size_t workspace_bytes, void* stream) {
  SAGE_TRY(check_shapes(layout, B, H, H, N, N, d));
  SAGE_TRY(check_in_dtype(in_dtype));
  SAGE_PTR(V); SAGE_PTR(v_codes); SAGE_PTR(v_scale); SAGE_PTR(workspace);
  if (workspace_bytes < sage::quantize_v_workspace(B * H, N, d)) return SAGE_ERR_WORKSPACE;
  sage::QuantVArgs a;
  a.V = V; a.is_bf16 = in_dtype == SAGE_BF16; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.v_codes = v_codes; a.v_scale = v_scale; a.workspace = workspace;
  (void)hipGetLastError();
  sage::launch_quantize_v(a, (hipStream_t)stream);
  return launch_status();
}

size_t sage_quantize_qkv_workspace_bytes(int B, int Hkv, int Nkv, int d) {
  if (B < 1 || Hkv < 1 || Nkv < 1 || d < 1) return 0;
  return (sage::quantize_qk_workspace(B * Hkv, Nkv, d) + 255) / 256 * 256 + sage::quantize_v_workspace(B * Hkv, Nkv, d);
}

int sage_quantize_qkv(const void* Q, const void* K, const void* V, int in_dtype, int layout, int B, int Hq, int Hkv,
                      int Nq, int Nkv, int d, int blk_q, int blk_k, int8_t* q_codes, float* q_scale, int8_t* k_codes,
                      float* k_scale, float* k_mean, uint8_t* v_codes, float* v_scale, void* workspace,
                      size_t workspace_bytes, void* stream) {
  SAGE_TRY(check_shapes(layout, B, Hq, Hkv, Nq, Nkv, d));
  SAGE_TRY(check_in_dtype(in_dtype));
  SAGE_TRY(check_blocks(blk_q, blk_k));
  SAGE_PTR(Q); SAGE_PTR(K); SAGE_PTR(V); SAGE_PTR(q_codes); SAGE_PTR(q_scale); SAGE_PTR(k_codes); SAGE_PTR(k_scale);
  SAGE_PTR(k_mean); SAGE_PTR(v_codes); SAGE_PTR(v_scale); SAGE_PTR(workspace);
  if (workspace_bytes < sage_quantize_qkv_workspace_bytes(B, Hkv, Nkv, d)) return SAGE_ERR_WORKSPACE;
  sage::QuantQKArgs a;
  a.Q = Q; a.K = K; a.is_bf16 = in_dtype == SAGE_BF16; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv; a.d = d; a.blk_q = blk_q; a.blk_k = blk_k;
  a.q_codes = q_codes; a.q_scale = q_scale; a.k_codes = k_codes; a.k_scale = k_scale; a.k_mean = k_mean;
  a.workspace = workspace;
  sage::QuantVArgs v;
  v.V = V; v.is_bf16 = a.is_bf16; v.nhd = a.nhd; v.B = B; v.H = Hkv; v.N = Nkv; v.d = d;
  v.v_codes = v_codes; v.v_scale = v_scale;
  v.workspace = (char*)workspace + (sage::quantize_qk_workspace(B * Hkv, Nkv, d) + 255) / 256 * 256;
  (void)hipGetLastError();
  sage::launch_quantize_qkv(a, v, (hipStream_t)stream);
  return launch_status();
}

int sage_quantize_v(const void* V, int in_dtype, int B, int H, int N, int d, uint8_t* v_codes, float* v_scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return sage_quantize_v_ex(V, in_dtype, SAGE_LAYOUT_BHND, B, H, N, d, v_codes, v_scale, workspace, workspace_bytes,
                            stream);
}

int sage_quantize_qk4(const void* Q, const void* K, int in_dtype, int layout, int B, int Hq, int Hkv, int Nq,
                      int Nkv, int d, uint8_t* q4_codes, uint8_t* q4_scale, uint8_t* k4_codes, uint8_t* k4_scale,
                      float* k_mean, void* workspace, size_t workspace_bytes, void* stream) {
  return sage_quantize_qk4_smooth_q(Q, K, in_dtype, layout, B, Hq, Hkv, Nq, Nkv, d, q4_codes, q4_scale, k4_codes,
                                    k4_scale, k_mean, nullptr, nullptr, nullptr, nullptr, nullptr, workspace,
                                    workspace_bytes, stream);
}

int sage_quantize_qk4_smooth_q(const void* Q, const void* K, int in_dtype, int layout, int B, int Hq, int Hkv,
                               int Nq, int Nkv, int d, uint8_t* q4_codes, uint8_t* q4_scale, uint8_t* k4_codes,
                               uint8_t* k4_scale, float* k_mean, float* q_mean, int8_t* qm_codes,
                               uint8_t* qm_scale, int8_t* k8_codes, uint8_t* k8_scale, void* workspace,
                               size_t workspace_bytes, void* stream) {
  SAGE_TRY(check_shapes(layout, B, Hq, Hkv, Nq, Nkv, d));
  SAGE_TRY(check_in_dtype(in_dtype));
  SAGE_PTR(Q); SAGE_PTR(K); SAGE_PTR(q4_codes); SAGE_PTR(q4_scale); SAGE_PTR(k4_codes); SAGE_PTR(k4_scale);
  SAGE_PTR(k_mean); SAGE_PTR(workspace);
  const bool smooth = q_mean || qm_codes || qm_scale || k8_codes || k8_scale;
  if (smooth) { SAGE_PTR(q_mean); SAGE_PTR(qm_codes); SAGE_PTR(qm_scale); SAGE_PTR(k8_codes); SAGE_PTR(k8_scale); }
  if (workspace_bytes < sage::quantize_qk_workspace(B * Hkv, Nkv, d)) return SAGE_ERR_WORKSPACE;
  sage::Quant4Args a{};
  a.Q = Q; a.K = K; a.is_bf16 = in_dtype == SAGE_BF16; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv; a.d = d;
  a.q4_codes = q4_codes; a.q4_scale = q4_scale; a.k4_codes = k4_codes; a.k4_scale = k4_scale; a.k_mean = k_mean;
  if (smooth) { a.q_mean = q_mean; a.qm_codes = qm_codes; a.qm_scale = qm_scale; a.k8_codes = k8_codes; a.k8_scale = k8_scale; }
  a.workspace = workspace;
  (void)hipGetLastError();
  sage::launch_quantize_qk4(a, (hipStream_t)stream);
  return launch_status();
}

int sage_attn_fwd_qk4(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                      const uint8_t* k4_scale, const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype,
                      int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal, float sm_scale,
                      void* stream) {
  const Q4Ptrs q4{q4_codes, q4_scale, k4_codes, k4_scale};
  return attn_common(nullptr, nullptr, nullptr, nullptr, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, 128, 64, causal, sm_scale, nullptr, 0, nullptr, nullptr, false, stream, &q4);
}

int sage_attn_fwd_qk4_dump(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                           const uint8_t* k4_scale, const uint8_t* v_codes, const float* v_scale, void* O,
                           int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                           float sm_scale, const int32_t* sel, int n_sel, int32_t* s_dump, uint8_t* p_dump,
                           void* stream) {
  const Q4Ptrs q4{q4_codes, q4_scale, k4_codes, k4_scale};
  return attn_common(nullptr, nullptr, nullptr, nullptr, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, 128, 64, causal, sm_scale, sel, n_sel, s_dump, p_dump, true, stream, &q4);
}

int sage_attn_fwd_qk4_smooth_q(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                               const uint8_t* k4_scale, const int8_t* qm_codes, const uint8_t* qm_scale,
                               const int8_t* k8_codes, const uint8_t* k8_scale, const uint8_t* v_codes,
                               const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq, int Hkv,
                               int Nq, int Nkv, int d, int causal, float sm_scale, void* stream) {
  if (!qm_codes || !qm_scale || !k8_codes || !k8_scale) return SAGE_ERR_INVALID_ARG;
  const Q4Ptrs q4{q4_codes, q4_scale, k4_codes, k4_scale, qm_codes, qm_scale, k8_codes, k8_scale};
  return attn_common(nullptr, nullptr, nullptr, nullptr, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, 128, 64, causal, sm_scale, nullptr, 0, nullptr, nullptr, false, stream, &q4);
}

int sage_attn_fwd_qk4_smooth_q_dump(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                                    const uint8_t* k4_scale, const int8_t* qm_codes, const uint8_t* qm_scale,
                                    const int8_t* k8_codes, const uint8_t* k8_scale, const uint8_t* v_codes,
                                    const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq, int Hkv,
                                    int Nq, int Nkv, int d, int causal, float sm_scale, const int32_t* sel, int n_sel,
                                    int32_t* s_dump, uint8_t* p_dump, void* stream) {
  if (!qm_codes || !qm_scale || !k8_codes || !k8_scale) return SAGE_ERR_INVALID_ARG;
  const Q4Ptrs q4{q4_codes, q4_scale, k4_codes, k4_scale, qm_codes, qm_scale, k8_codes, k8_scale};
  return attn_common(nullptr, nullptr, nullptr, nullptr, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, 128, 64, causal, sm_scale, sel, n_sel, s_dump, p_dump, true, stream, &q4);
}

int sage_quantize_v4(const void* V, int in_dtype, int layout, int B, int H, int N, int d, uint8_t* v4_codes,
                     uint8_t* v4_scale, void* stream) {
  SAGE_TRY(check_shapes(layout, B, H, H, N, N, d));
  SAGE_TRY(check_in_dtype(in_dtype));
  SAGE_PTR(V); SAGE_PTR(v4_codes); SAGE_PTR(v4_scale);
  sage::QuantV4Args a{};
  a.V = V; a.is_bf16 = in_dtype == SAGE_BF16; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.H = H; a.N = N; a.d = d; a.v4_codes = v4_codes; a.v4_scale = v4_scale;
  (void)hipGetLastError();
  sage::launch_quantize_v4(a, (hipStream_t)stream);
  return launch_status();
}

int sage_attn_fwd_fp4(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                      const uint8_t* k4_scale, const uint8_t* v4_codes, const uint8_t* v4_scale, void* O,
                      int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                      float sm_scale, void* stream) {
  if (!v4_codes || !v4_scale) return SAGE_ERR_INVALID_ARG;
  Q4Ptrs q4{q4_codes, q4_scale, k4_codes, k4_scale};
  q4.v4_codes = v4_codes; q4.v4_scale = v4_scale;
  return attn_common(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, 128, 64, causal, sm_scale, nullptr, 0, nullptr, nullptr, false, stream, &q4);
}

int sage_attn_fwd_fp4_dump(const uint8_t* q4_codes, const uint8_t* q4_scale, const uint8_t* k4_codes,
                           const uint8_t* k4_scale, const uint8_t* v4_codes, const uint8_t* v4_scale, void* O,
                           int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int causal,
                           float sm_scale, const int32_t* sel, int n_sel, int32_t* s_dump, uint8_t* p_dump,
                           void* stream) {
  if (!v4_codes || !v4_scale) return SAGE_ERR_INVALID_ARG;
  Q4Ptrs q4{q4_codes, q4_scale, k4_codes, k4_scale};
  q4.v4_codes = v4_codes; q4.v4_scale = v4_scale;
  return attn_common(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, 128, 64, causal, sm_scale, sel, n_sel, s_dump, p_dump, true, stream, &q4);
}

int sage_quantize_q(const void* Q, int in_dtype, int layout, int B, int Hq, int Nq, int d, int blk_q,
                    int8_t* q_codes, float* q_scale, void* stream) {
  SAGE_TRY(check_shapes(layout, B, Hq, Hq, Nq, Nq, d));
  SAGE_TRY(check_in_dtype(in_dtype));
  SAGE_TRY(check_blocks(blk_q, 64));
  SAGE_PTR(Q); SAGE_PTR(q_codes); SAGE_PTR(q_scale);
  sage::QuantQKArgs a{};
  a.Q = Q; a.is_bf16 = in_dtype == SAGE_BF16; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.Hq = Hq; a.Hkv = Hq; a.Nq = Nq; a.Nkv = Nq; a.d = d; a.blk_q = blk_q; a.blk_k = 64;
  a.q_codes = q_codes; a.q_scale = q_scale;
  (void)hipGetLastError();
  sage::launch_quantize_qk(a, (hipStream_t)stream, true, false);
  return launch_status();
}

int sage_quantize_k(const void* K, int in_dtype, int layout, int B, int Hkv, int Nkv, int d, int blk_k,
                    int8_t* k_codes, float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes,
                    void* stream) {
  SAGE_TRY(check_shapes(layout, B, Hkv, Hkv, Nkv, Nkv, d));
  SAGE_TRY(check_in_dtype(in_dtype));
  SAGE_TRY(check_blocks(64, blk_k));
  SAGE_PTR(K); SAGE_PTR(k_codes); SAGE_PTR(k_scale); SAGE_PTR(k_mean); SAGE_PTR(workspace);
  if (workspace_bytes < sage::quantize_qk_workspace(B * Hkv, Nkv, d)) return SAGE_ERR_WORKSPACE;
  sage::QuantQKArgs a{};
  a.K = K; a.is_bf16 = in_dtype == SAGE_BF16; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.Hq = Hkv; a.Hkv = Hkv; a.Nq = Nkv; a.Nkv = Nkv; a.d = d; a.blk_q = 64; a.blk_k = blk_k;
  a.k_codes = k_codes; a.k_scale = k_scale; a.k_mean = k_mean; a.workspace = workspace;
  (void)hipGetLastError();
  sage::launch_quantize_qk(a, (hipStream_t)stream, false, true);
  return launch_status();
}

int sage_decode_kv_chunk(int B, int Hq, int Hkv, int Nq, int Nkv, int d) {
  if (check_shapes(SAGE_LAYOUT_BHND, B, Hq, Hkv, Nq, Nkv, d) != SAGE_OK) return 0;
  return sage::decode_default_chunk(B, Hq, Hkv, Nq, Nkv);
}

size_t sage_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nkv, int d, int kv_chunk) {
  if (check_shapes(SAGE_LAYOUT_BHND, B, Hq, Hkv, Nq, Nkv, d) != SAGE_OK) return 0;
  if (kv_chunk == 0) kv_chunk = sage::decode_default_chunk(B, Hq, Hkv, Nq, Nkv);
  if (kv_chunk < sage::kKTile || kv_chunk % sage::kKTile) return 0;
  return sage::decode_workspace(B, Hq, Hkv, Nq, Nkv, d, kv_chunk);
}

}  // extern "C"

// Chunk states of sage_attn_decode_noalloc: one copy of this array per device,
// held until the process ends.  In host code its name is only a handle for
// hipGetSymbolAddress: the device address of each device's copy is looked up
// once, with that device current, and only that pointer reaches the kernels.
static __device__ __align__(256) unsigned char scratch[SAGE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current device's scratch array (looked up on the
// first call on that device).  The stream must belong to the current device.
int noalloc_scratch(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return SAGE_ERR_HIP;
  }
  if (dev >= kMaxDevices) return SAGE_ERR_UNSUPPORTED;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) {
      (void)hipGetLastError();
      return SAGE_ERR_HIP;
    }
    if (sdev != dev) return SAGE_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return SAGE_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SAGE_OK;
}

// sage_attn_decode with the workspace given (noalloc = false) or the
// library's scratch array (noalloc = true; workspace and workspace_bytes unused).
int decode_common(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                  const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq,
                  int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale, int kv_chunk,
                  void* workspace, size_t workspace_bytes, bool noalloc, void* stream) {
  SAGE_TRY(check_shapes(layout, B, Hq, Hkv, Nq, Nkv, d));
  SAGE_TRY(check_blocks(blk_q, blk_k));
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (causal && Nkv < Nq) return SAGE_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || isinf(sm_scale)) return SAGE_ERR_INVALID_ARG;
  if (kv_chunk == 0) kv_chunk = sage::decode_default_chunk(B, Hq, Hkv, Nq, Nkv);
  if (kv_chunk < sage::kKTile || kv_chunk % sage::kKTile) return SAGE_ERR_INVALID_ARG;
  // waves of work: B*Hkv * ceil(g*Nq/32) * chunks, four per workgroup of a 1-D grid
  const long long units = (long long)B * Hkv * (((long long)(Hq / Hkv) * Nq + 31) / 32) *
                          (((Nkv + sage::kKTile - 1) / sage::kKTile + kv_chunk / sage::kKTile - 1) /
                           (kv_chunk / sage::kKTile));
  if (units / 4 + 1 > 0x7fffffffLL) return SAGE_ERR_UNSUPPORTED;
  SAGE_PTR(q_codes); SAGE_PTR(q_scale); SAGE_PTR(k_codes); SAGE_PTR(k_scale);
  SAGE_PTR(v_codes); SAGE_PTR(v_scale); SAGE_PTR(O);
  const size_t need = sage::decode_workspace(B, Hq, Hkv, Nq, Nkv, d, kv_chunk);
  if (noalloc) {
    if (need > SAGE_NOALLOC_SCRATCH_BYTES) return SAGE_ERR_WORKSPACE;
    SAGE_TRY(noalloc_scratch(stream, &workspace));
  } else {
    SAGE_PTR(workspace);
    if (workspace_bytes < need) return SAGE_ERR_WORKSPACE;
  }
  sage::DecodeArgs a;
  a.q_codes = q_codes; a.q_scale = q_scale; a.k_codes = k_codes; a.k_scale = k_scale;
  a.v_codes = v_codes; a.v_scale = v_scale; a.O = O; a.out_dtype = out_dtype; a.nhd = layout == SAGE_LAYOUT_BNHD;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Nq = Nq; a.Nkv = Nkv; a.d = d; a.blk_q = blk_q; a.blk_k = blk_k;
  a.causal = causal; a.kv_chunk = kv_chunk; a.s2 = sm_scale * sage::kLog2e; a.workspace = workspace;
  (void)hipGetLastError();
  sage::launch_attn_decode(a, (hipStream_t)stream);
  return launch_status();
}

}  // namespace

extern "C" {

int sage_attn_decode(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                     const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq,
                     int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale,
                     int kv_chunk, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq,
                       Nkv, d, blk_q, blk_k, causal, sm_scale, kv_chunk, workspace, workspace_bytes, false, stream);
}

int sage_attn_decode_noalloc(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes,
                             const float* k_scale, const uint8_t* v_codes, const float* v_scale, void* O,
                             int out_dtype, int layout, int B, int Hq, int Hkv, int Nq, int Nkv, int d, int blk_q,
                             int blk_k, int causal, float sm_scale, int kv_chunk, void* stream) {
  return decode_common(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq,
                       Nkv, d, blk_q, blk_k, causal, sm_scale, kv_chunk, nullptr, 0, true, stream);
}

int sage_attn_fwd_ex(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                     const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B, int Hq,
                     int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale, void* stream) {
  return attn_common(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, blk_q, blk_k, causal, sm_scale, nullptr, 0, nullptr, nullptr, false, stream);
}

int sage_attn_fwd_ex_dump(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                          const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int layout, int B,
                          int Hq, int Hkv, int Nq, int Nkv, int d, int blk_q, int blk_k, int causal, float sm_scale,
                          const int32_t* sel, int n_sel, int32_t* s_dump, uint8_t* p_dump, void* stream) {
  return attn_common(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, layout, B, Hq, Hkv, Nq, Nkv,
                     d, blk_q, blk_k, causal, sm_scale, sel, n_sel, s_dump, p_dump, true, stream);
}

int sage_attn_fwd(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                  const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int B, int H, int N, int d,
                  int blk_q, int blk_k, int causal, float sm_scale, void* stream) {
  return attn_common(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, SAGE_LAYOUT_BHND, B, H, H, N,
                     N, d, blk_q, blk_k, causal, sm_scale, nullptr, 0, nullptr, nullptr, false, stream);
}

int sage_attn_fwd_dump(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                       const uint8_t* v_codes, const float* v_scale, void* O, int out_dtype, int B, int H, int N, int d,
                       int blk_q, int blk_k, int causal, float sm_scale, const int32_t* sel, int n_sel, int32_t* s_dump,
                       uint8_t* p_dump, void* stream) {
  return attn_common(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, O, out_dtype, SAGE_LAYOUT_BHND, B, H, H, N,
                     N, d, blk_q, blk_k, causal, sm_scale, sel, n_sel, s_dump, p_dump, true, stream);
}

}  // extern "C"
