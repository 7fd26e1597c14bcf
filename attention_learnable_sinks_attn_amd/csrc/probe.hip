// Throughput probe of the bf16 matrix cores (gfx950), for the benchmark's roofline report: how
// many bf16 MFMA FLOP/s this GPU sustains at its running clock when nothing but MFMAs is issued.
// Built into its own library (libattn_sink_probe.so); the attention library does not use it.
//
// Every wave runs `iters` rounds of kChains independent 32x32x16 bf16 MFMA accumulation chains on
// register operands (two waves per SIMD, enough chains to cover the MFMA latency), then writes one
// float per lane so that nothing is optimised away. FLOPs = 2 * 32 * 32 * 16 per MFMA.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;

__global__ __launch_bounds__(256, 2) void attn_sink_probe_mfma_kernel(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[c][i] = 1e-3f * (float)c;  // distinct chains: none can be merged
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Enqueues `blocks` workgroups of 256 threads on `stream`; `out` must hold blocks * 256 floats.
// Returns 0, or -1 for bad arguments, -6 for a launch error. FLOPs done:
// blocks * 4 waves * iters * 8 chains * 32768.
int attn_sink_probe_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(attn_sink_probe_mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
