// Throughput probes for gfx950 (measurement aids next to the kernels, not
// steps of the method): the matrix cores, and HBM read bandwidth.
//
// Matrix-core probe.  Every wave issues, per loop
// iteration, the matrix instructions one d = 128 KV tile costs a wave of the
// attention kernel: 8 v_mfma_i32_32x32x32_i8 (the scores) and 4
// v_mfma_scale_f32_32x32x64_f8f6f4 in FP8 form (P~V), on six independent
// accumulators and with no other work.  The measured rate is the sustained
// dense INT8/FP8 rate of the chip at the clock it holds under that load; the
// attention kernel's rate can be read against it as well as against the
// published peak.
#include <hip/hip_runtime.h>

#include "../../include/sage.h"
#include "common.h"

namespace sage {

// 2 workgroups of 4 waves per CU: the attention kernel's occupancy at d = 128.
__global__ __launch_bounds__(256, 2) void mfma_peak_kernel(int iters, int* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  // operands that depend on the lane (nothing to fold); FP8 bytes 0x38 = 1.0
  const v4i a = {lane, lane * 3 + 1, lane * 5 + 2, lane * 7 + 3};
  const v4i b = {lane ^ 21, lane ^ 42, lane + 9, lane + 17};
  const v8i a8 = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x30383830, 0x38303038, 0x38383838, 0x38303830};
  const v8i b8 = {0x38383838, 0x30303030, 0x38383838, 0x30303030, 0x38383838, 0x30303030, 0x38383838, 0x30303030};
  v16i c0 = {}, c1 = {}, c2 = {}, c3 = {};
  v16f f0 = {}, f1 = {};
  for (int i = 0; i < iters; i++) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    f0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, f0, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    f1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, f1, 0, 0, 0, 127, 0, 127);
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
    f0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, f0, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    f1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b8, a8, f1, 0, 0, 0, 127, 0, 127);
  }
  // the accumulators are live: a checksum per thread when a sink is given
  if (sink) {
    int s = 0;
#pragma unroll
    for (int e = 0; e < 16; e++) s += c0[e] + c1[e] + c2[e] + c3[e] + (int)f0[e] + (int)f1[e];
    sink[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
  }
}

// HBM read-bandwidth probe (a measurement aid for the HBM-bound passes):
// 1024 workgroups of 256 threads read `bytes` of device memory once with
// 16-byte non-temporal (streaming) loads, eight in flight per thread, each
// workgroup over one contiguous span (measured on MI355X: contiguous spans
// and streaming loads each gain about 10% over a grid-stride loop with
// ordinary loads); the remainder past the spans is read grid-stride.  Every
// 16-byte vector is folded into one checksum per thread, written to the sink.
__global__ __launch_bounds__(256) void hbm_read_kernel(const v4i* __restrict__ src, long long nvec,
                                                       int* __restrict__ sink) {
  constexpr int U = 8;
  const long long per = nvec / gridDim.x / (256 * U) * (256 * U);   // whole iterations per span
  const v4i* p = src + (long long)blockIdx.x * per;
  v4i acc = {0, 0, 0, 0};
  for (long long base = threadIdx.x; base < per; base += 256 * U) {
    v4i x[U];
#pragma unroll
    for (int u = 0; u < U; u++) x[u] = __builtin_nontemporal_load(p + base + u * 256);
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= x[u];
  }
  for (long long i = per * gridDim.x + (long long)blockIdx.x * 256 + threadIdx.x; i < nvec;
       i += (long long)gridDim.x * 256)
    acc ^= __builtin_nontemporal_load(src + i);
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace sage

extern "C" int sage_probe_hbm_read(const void* buf, size_t bytes, int* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16) return SAGE_ERR_INVALID_ARG;
  if (((uintptr_t)buf & 15u) != 0 || ((uintptr_t)sink & 15u) != 0) return SAGE_ERR_MISALIGNED;
  (void)hipGetLastError();
  hipLaunchKernelGGL(sage::hbm_read_kernel, dim3(1024), dim3(256), 0, (hipStream_t)stream, (const sage::v4i*)buf,
                     (long long)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

extern "C" int sage_probe_mfma_peak(int workgroups, int iters, int* sink, void* stream) {
  if (workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 24)) return SAGE_ERR_INVALID_ARG;
  if (((uintptr_t)sink & 15u) != 0) return SAGE_ERR_MISALIGNED;
  (void)hipGetLastError();
  hipLaunchKernelGGL(sage::mfma_peak_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return hipGetLastError() == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}
