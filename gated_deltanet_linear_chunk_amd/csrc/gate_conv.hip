// gate_conv.hip -- gates and the causal depthwise conv1d (+ SiLU, + q/k L2 norm).
//
// Both are streaming, HBM-bound steps: no matrix work, so they use plain
// coalesced 16-byte vector loads and stores and fp32 arithmetic.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

// ----------------------------------------------------------------------------
// Gates: beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias).
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) gate_kernel(const float* __restrict__ a,
                                                   const float* __restrict__ b,
                                                   const float* __restrict__ A_log,
                                                   const float* __restrict__ dt_bias,
                                                   int64_t n, int H, float* __restrict__ g,
                                                   float* __restrict__ beta) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int h = (int)(i % H);
    const float x = a[i] + dt_bias[h];
    const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
    g[i] = -expf(A_log[h]) * sp;
    beta[i] = 1.f / (1.f + expf(-b[i]));
  }
}

hipError_t launch_gate(const float* a, const float* b, const float* A_log, const float* dt_bias,
                       int64_t n_tokens, int H, float* g, float* beta, hipStream_t stream) {
  const int64_t n = n_tokens * H;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, b, A_log,
                     dt_bias, n, H, g, beta);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Causal depthwise conv1d.
//
// One thread owns 8 consecutive channels (one 16-byte bf16 vector) and walks a
// tile of TOK consecutive tokens, keeping the last 3 inputs of its channels in
// registers.  A block of 256 threads covers 2048 channels; a wave (512
// channels) is one contiguous 1 KiB row segment per token, so every load and
// store is fully coalesced.  The history is zeroed at each sample start; the
// sample of the tile's first token comes from a binary search of cu_seqlens
// (or from the batch row), later boundaries from walking the offsets.
// The per-head L2 norm reduces over head_dim / 8 adjacent lanes with xor
// shuffles, which stay inside one head because heads are 8-channel aligned.
// ----------------------------------------------------------------------------
constexpr int CONV_THREADS = 256;
constexpr int CONV_CH_PER_THREAD = 8;
constexpr int CONV_TOK = 32;

template <typename T>
struct Vec8;

template <>
struct Vec8<uint16_t> {  // bf16
  static __device__ __forceinline__ void load(const uint16_t* p, float* out) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* in) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16_bits(in[2 * i]) | ((uint32_t)f32_to_bf16_bits(in[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  static __device__ __forceinline__ float scalar(const uint16_t* p, int i) {
    return bf16_bits_to_f32(p[i]);
  }
};

template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* out) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* in) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(in[4], in[5], in[6], in[7]);
  }
  static __device__ __forceinline__ float scalar(const float* p, int i) { return p[i]; }
};

// Sample index of token t (largest n with cu[n] <= t), offsets clamped to [0, T].
__device__ __forceinline__ int find_sample(const int32_t* cu, int n_seqs, int64_t t,
                                           int64_t Ttot) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (clampi(cu[mid], 0, Ttot) <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

template <typename T>
__global__ void __launch_bounds__(CONV_THREADS) conv1d_kernel(
    const T* __restrict__ x, const T* __restrict__ w, const T* __restrict__ bias,
    const int32_t* __restrict__ cu, int n_seqs, int64_t row_len, int64_t Ttot, int C, int width,
    int apply_silu, int l2_channels, int l2_lanes_log2, float l2_eps, T* __restrict__ y) {
  const int c0 = (blockIdx.x * CONV_THREADS + threadIdx.x) * CONV_CH_PER_THREAD;
  const bool active = c0 < C;
  const int64_t t_begin = (int64_t)blockIdx.y * CONV_TOK;
  const int64_t t_end = t_begin + CONV_TOK < Ttot ? t_begin + CONV_TOK : Ttot;

  // taps aligned so that tap 3 multiplies the current token (zero-filled when width < 4)
  float wt[4][CONV_CH_PER_THREAD];
  float bs[CONV_CH_PER_THREAD];
#pragma unroll
  for (int i = 0; i < CONV_CH_PER_THREAD; ++i) {
    const int c = active ? c0 + i : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int src = j - (4 - width);
      wt[j][i] = (active && src >= 0) ? Vec8<T>::scalar(w, c * width + src) : 0.f;
    }
    bs[i] = (active && bias) ? Vec8<T>::scalar(bias, c) : 0.f;
  }

  // sample bounds of the first token
  int64_t s_start, s_end;
  int n = 0;
  if (cu) {
    n = find_sample(cu, n_seqs, t_begin, Ttot);
    s_start = clampi(cu[n], 0, Ttot);
    s_end = clampi(cu[n + 1], s_start, Ttot);
  } else {
    s_start = (t_begin / row_len) * row_len;
    s_end = s_start + row_len;
  }

  float h1[CONV_CH_PER_THREAD], h2[CONV_CH_PER_THREAD], h3[CONV_CH_PER_THREAD];  // x[t-3..t-1]
#pragma unroll
  for (int i = 0; i < CONV_CH_PER_THREAD; ++i) h1[i] = h2[i] = h3[i] = 0.f;
  if (active) {
    float tmp[CONV_CH_PER_THREAD];
    if (t_begin - 3 >= s_start) {
      Vec8<T>::load(x + (t_begin - 3) * C + c0, tmp);
#pragma unroll
      for (int i = 0; i < CONV_CH_PER_THREAD; ++i) h1[i] = tmp[i];
    }
    if (t_begin - 2 >= s_start) {
      Vec8<T>::load(x + (t_begin - 2) * C + c0, tmp);
#pragma unroll
      for (int i = 0; i < CONV_CH_PER_THREAD; ++i) h2[i] = tmp[i];
    }
    if (t_begin - 1 >= s_start) {
      Vec8<T>::load(x + (t_begin - 1) * C + c0, tmp);
#pragma unroll
      for (int i = 0; i < CONV_CH_PER_THREAD; ++i) h3[i] = tmp[i];
    }
  }
  const bool do_l2 = l2_channels > 0 && c0 < l2_channels;

  for (int64_t t = t_begin; t < t_end; ++t) {
    while (t >= s_end) {  // crossed into the next sample: reset the history
      if (cu && n + 1 < n_seqs) {
        ++n;
        s_start = s_end;
        s_end = clampi(cu[n + 1], s_start, Ttot);
      } else if (cu) {  // tokens past the last offset form one trailing region
        s_start = s_end;
        s_end = Ttot;
      } else {
        s_start = s_end;
        s_end = s_start + row_len;
      }
#pragma unroll
      for (int i = 0; i < CONV_CH_PER_THREAD; ++i) h1[i] = h2[i] = h3[i] = 0.f;
    }
    float cur[CONV_CH_PER_THREAD], out[CONV_CH_PER_THREAD];
    if (active) {
      Vec8<T>::load(x + t * C + c0, cur);
    } else {
#pragma unroll
      for (int i = 0; i < CONV_CH_PER_THREAD; ++i) cur[i] = 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < CONV_CH_PER_THREAD; ++i) {
      float z = bs[i];
      z = fmaf(wt[0][i], h1[i], z);
      z = fmaf(wt[1][i], h2[i], z);
      z = fmaf(wt[2][i], h3[i], z);
      z = fmaf(wt[3][i], cur[i], z);
      if (apply_silu) z = z / (1.f + expf(-z));
      out[i] = z;
      ss = fmaf(z, z, ss);
      h1[i] = h2[i];
      h2[i] = h3[i];
      h3[i] = cur[i];
    }
    if (l2_channels > 0) {  // uniform across the block: every lane joins the shuffles
      for (int m = 1; m < (1 << l2_lanes_log2); m <<= 1) ss += __shfl_xor(ss, m, 64);
      if (do_l2) {
        const float inv = 1.f / sqrtf(ss + l2_eps);
#pragma unroll
        for (int i = 0; i < CONV_CH_PER_THREAD; ++i) out[i] *= inv;
      }
    }
    if (active) Vec8<T>::store(y + t * C + c0, out);
  }
}

hipError_t launch_conv1d(const void* x, const void* w, const void* bias, int dt,
                         const int32_t* cu, int n_seqs, int B, int64_t T, int C, int width,
                         int apply_silu, int l2_channels, int head_dim, float l2_eps, void* y,
                         hipStream_t stream) {
  const int64_t Ttot = cu ? T : (int64_t)B * T;
  if (Ttot == 0 || C == 0) return hipSuccess;
  const int per_block = CONV_THREADS * CONV_CH_PER_THREAD;
  dim3 grid((unsigned)((C + per_block - 1) / per_block), (unsigned)((Ttot + CONV_TOK - 1) / CONV_TOK));
  int lanes_log2 = 0;
  if (l2_channels > 0)
    while ((CONV_CH_PER_THREAD << lanes_log2) < head_dim) ++lanes_log2;
  const int64_t row_len = cu ? Ttot : T;
  if (dt == 1) {
    hipLaunchKernelGGL(conv1d_kernel<uint16_t>, grid, dim3(CONV_THREADS), 0, stream,
                       (const uint16_t*)x, (const uint16_t*)w, (const uint16_t*)bias, cu, n_seqs,
                       row_len, Ttot, C, width, apply_silu, l2_channels, lanes_log2, l2_eps,
                       (uint16_t*)y);
  } else {
    hipLaunchKernelGGL(conv1d_kernel<float>, grid, dim3(CONV_THREADS), 0, stream,
                       (const float*)x, (const float*)w, (const float*)bias, cu, n_seqs, row_len,
                       Ttot, C, width, apply_silu, l2_channels, lanes_log2, l2_eps, (float*)y);
  }
  return hipGetLastError();
}

}  // namespace gdn
