// gated_norm.hip -- the output norm gated by z that follows the chunk rule.
//
// The LlamaFactory PR "[v1] support GDN Ulysses cp" (Design) runs
// "chunk_gated_delta_rule + norm" with the z component before the output
// leaves the layer.  Per row (one token of one v-head, V values):
//   y = o * rsqrt(mean(o^2) + eps) * weight * z * sigmoid(z).
// A streaming step (o and z read once, y written once) with one reduction
// per row: V / 8 adjacent lanes hold a row, eight values each (16- or
// 32-byte vector loads), and sum their squares with lane exchanges inside
// the wave; all arithmetic in fp32.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int NT = 256;

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
};
template <>
struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* x) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* x) {
    *reinterpret_cast<uint4*>(p) =
        make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
  }
};

template <int V, typename To, typename Tz, typename Ty>
__global__ void __launch_bounds__(NT) gated_norm_kernel(const To* o, const Tz* z, const float* __restrict__ weight,
                                                        float eps, int64_t rows, Ty* y) {
  constexpr int TPR = V / 8;      // lanes per row
  constexpr int RPB = NT / TPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int64_t r = (int64_t)blockIdx.x * RPB + tid / TPR;
  const int c = 8 * (tid % TPR);
  const int64_t rr = r < rows ? r : rows - 1;  // the tail re-reads the last row and stores nothing
  float ov[8], zv[8], w[8];
  Vec8<To>::load(o + rr * V + c, ov);
  Vec8<Tz>::load(z + rr * V + c, zv);
  if (weight) {
    Vec8<float>::load(weight + c, w);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 1.f;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(ov[i], ov[i], ss);
#pragma unroll
  for (int off = 1; off < TPR; off <<= 1) ss += __shfl_xor(ss, off, 64);
  const float inv = 1.f / sqrtf(ss / (float)V + eps);
  float out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = ov[i] * inv * w[i] * silu_hw(zv[i]);
  if (r < rows) Vec8<Ty>::store(y + r * V + c, out);
}

template <int V, typename To, typename Tz>
hipError_t launch_y(const GatedNormArgs& a, hipStream_t stream) {
  constexpr int RPB = NT / (V / 8);
  const int64_t blocks = (a.rows + RPB - 1) / RPB;
  if (a.y_dt == 1)
    hipLaunchKernelGGL((gated_norm_kernel<V, To, Tz, uint16_t>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       (const To*)a.o, (const Tz*)a.z, a.weight, a.eps, a.rows, (uint16_t*)a.y);
  else
    hipLaunchKernelGGL((gated_norm_kernel<V, To, Tz, float>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       (const To*)a.o, (const Tz*)a.z, a.weight, a.eps, a.rows, (float*)a.y);
  return hipGetLastError();
}

template <int V>
hipError_t launch_v(const GatedNormArgs& a, hipStream_t stream) {
  if (a.o_dt == 1)
    return a.z_dt == 1 ? launch_y<V, uint16_t, uint16_t>(a, stream) : launch_y<V, uint16_t, float>(a, stream);
  return a.z_dt == 1 ? launch_y<V, float, uint16_t>(a, stream) : launch_y<V, float, float>(a, stream);
}

}  // namespace

hipError_t launch_gated_norm(const GatedNormArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  switch (a.V) {
    case 32: return launch_v<32>(a, stream);
    case 64: return launch_v<64>(a, stream);
    case 128: return launch_v<128>(a, stream);
    case 256: return launch_v<256>(a, stream);
    case 512: return launch_v<512>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
