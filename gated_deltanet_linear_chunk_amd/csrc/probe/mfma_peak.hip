// mfma_peak.hip -- measured dense bf16 matrix-core rate of the device, the
// peak the chunk kernels' MFMA share is also reported against (next to the
// published one).  Not part of the library: built into libgdn_probe.so and
// called by the benchmark only.
//
// Every wave keeps eight independent accumulators, so each
// v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 multiply-adds, 16384 flops) issues
// without waiting for the previous one, and the grid holds several waves per
// SIMD on every compute unit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChains = 8;

__global__ void __launch_bounds__(256) mfma_peak_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  // distinct start values per chain, so no two chains compute the same thing
  f32x4 acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) {
    const float s = (float)(lane * kChains + j);
    acc[j] = f32x4{s, s + 1.f, s + 2.f, s + 3.f};
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  // one store per workgroup keeps the work observable
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

}  // namespace

extern "C" {

// Flops one launch performs.
double gdn_probe_mfma_bf16_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * (double)iters * kChains * 16384.0;
}

// Launches `blocks` workgroups of 4 waves, each wave issuing iters * 8 MFMAs;
// out: device float[blocks].  Returns the hipError_t of the launch.
int gdn_probe_mfma_bf16(int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, out);
  return (int)hipGetLastError();
}

}  // extern "C"
