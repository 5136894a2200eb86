// mfma_peak.hip — a measurement aid beside the head, not part of it: the bf16 MFMA rate this GPU
// sustains at the clock it actually runs, to read the head kernels' utilisation against. Every wave
// keeps eight independent 32x32x16 bf16 accumulators (no MFMA waits on another) and cycles through
// them; its operands come from memory so that the caller chooses their bit patterns (zeros or
// random data draw different power, and so run at different clocks).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kThreads = 512;
constexpr int kChains = 8;

__global__ __launch_bounds__(kThreads) void mfma_loop(const bf16x8* src, int iters, float* out) {
  const int l = threadIdx.x & 63;
  const bf16x8 a = src[l], b = src[64 + l];
  f32x16 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}
}  // namespace

extern "C" {
// Work of one launch: n_workgroups * 8 waves * iters * 8 MFMAs * 32768 FLOP.
// src: device bf16 [128 x 8] operands (lanes' A then B fragments); out: device float
// [n_workgroups * 512]. Returns 0, or -1 for bad sizes, -4 when the launch fails.
int mfma_peak_run(int n_workgroups, int iters, const void* src, float* out, hipStream_t stream) {
  if (n_workgroups <= 0 || iters <= 0 || !src || !out) return -1;
  hipLaunchKernelGGL(mfma_loop, dim3(n_workgroups), dim3(kThreads), 0, stream, (const bf16x8*)src,
                     iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}
}
