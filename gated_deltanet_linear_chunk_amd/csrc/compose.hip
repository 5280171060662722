// compose.hip -- fp32 chain of segment affine maps.
//
// Given per-segment maps S_end = M_i S_start + b_i, the true start state of
// every segment follows from S_start,0 = S0 and S_start,i+1 = M_i S_start,i + b_i,
// composed in fp32 (the sglang fork PR "Qwen3.5 cp - #1" chain-reduces its
// (b, M) pairs in fp32).  Each column of the K x V state is its own affine
// chain, so the work is split over (v-head, 16-column slice): 256 threads per
// workgroup, each producing 8 entries of M_i S + b_i per step, with the
// current start state of the slice and the step's M (loaded with coalesced
// 16-byte reads, all in flight at once) held in LDS.  Segments follow one another
// inside the workgroup, which needs only the M S products (a tree over
// segments would also need M M products, K / 16 times more work per level).
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CK = 128;  // key dim
constexpr int CT = 16;   // state columns per workgroup
constexpr int CTHREADS = 256;

struct Chain {
  int n, p0, count, out0;
};

__global__ void __launch_bounds__(CTHREADS) compose_kernel(const float* __restrict__ M,
                                                           const float* __restrict__ b,
                                                           const float* __restrict__ s0,
                                                           const int32_t* __restrict__ chains,
                                                           Chain single, int Hv, int V,
                                                           float* __restrict__ out, int write_before,
                                                           float* __restrict__ final_state) {
  __shared__ float sS[2][CK][CT];
  __shared__ __attribute__((aligned(16))) float sM[CK][CK + 4];  // M of the current step
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * CT;
  const int h = blockIdx.y;
  const int ci = blockIdx.z;
  const Chain ch = chains ? Chain{chains[4 * ci], chains[4 * ci + 1], chains[4 * ci + 2], chains[4 * ci + 3]}
                          : single;
  const int d = tid >> 1;          // output row
  const int cc = (tid & 1) * 8;    // 8 output columns

  const int64_t head = (int64_t)h * CK * V;
  const int64_t row = (int64_t)Hv * CK * V;  // one [Hv, K, V] state
  for (int i = tid; i < CK * CT; i += CTHREADS) {
    const int r = i / CT, c = i % CT;
    sS[0][r][c] = (s0 && ch.n >= 0) ? s0[ch.n * row + head + (int64_t)r * V + c0 + c] : 0.f;
  }
  __syncthreads();
  int cur = 0;
  for (int j = 0; j < ch.count; ++j) {
    const int seg = ch.p0 + j;
    const int64_t seg_state = (int64_t)seg * row + head;
    float* dst = out + (int64_t)(ch.out0 + j) * row + head + (int64_t)d * V + c0 + cc;
    // M of this step into LDS with coalesced 16-byte loads (all in flight at once)
    const float* Mseg = M + ((int64_t)seg * Hv + h) * CK * CK;
    float4 mv4[CK * CK / 4 / CTHREADS];
#pragma unroll
    for (int i = 0; i < CK * CK / 4 / CTHREADS; ++i)
      mv4[i] = *reinterpret_cast<const float4*>(Mseg + 4 * (tid + CTHREADS * i));
    const float4 b0 = *reinterpret_cast<const float4*>(b + seg_state + (int64_t)d * V + c0 + cc);
    const float4 b1 = *reinterpret_cast<const float4*>(b + seg_state + (int64_t)d * V + c0 + cc + 4);
#pragma unroll
    for (int i = 0; i < CK * CK / 4 / CTHREADS; ++i) {
      const int e = 4 * (tid + CTHREADS * i);
      *reinterpret_cast<float4*>(&sM[e / CK][e % CK]) = mv4[i];
    }
    float acc[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
    if (write_before) {
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = sS[cur][d][cc + k];
    }
    __syncthreads();
#pragma unroll 4
    for (int l = 0; l < CK; l += 4) {
      const float4 m4 = *reinterpret_cast<const float4*>(&sM[d][l]);
      const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = fmaf(mv[u], sS[cur][l + u][cc + k], acc[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sS[cur ^ 1][d][cc + k] = acc[k];
      if (!write_before) dst[k] = acc[k];
    }
    cur ^= 1;
    __syncthreads();
  }
  if (final_state) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      final_state[ci * row + head + (int64_t)d * V + c0 + cc + k] = sS[cur][d][cc + k];
  }
}

}  // namespace

hipError_t launch_compose_chains(const float* M, const float* b, const float* s0,
                                 const int32_t* chains, int n_chains, int Hv, int K, int V,
                                 float* out, int write_before, float* final_state,
                                 hipStream_t stream) {
  if (n_chains == 0 || Hv == 0) return hipSuccess;
  if (K != CK || V % CT != 0) return hipErrorInvalidValue;
  dim3 grid(V / CT, Hv, n_chains);
  hipLaunchKernelGGL(compose_kernel, grid, dim3(CTHREADS), 0, stream, M, b, s0, chains, Chain{0, 0, 0, 0}, Hv, V,
                     out, write_before, final_state);
  return hipGetLastError();
}

// One chain over P segments of one sequence: starts of every segment, then
// the final state.
hipError_t launch_compose(const float* M, const float* b, const float* s0, int P, int Hv, int K,
                          int V, float* starts, float* final_state, hipStream_t stream) {
  if (P == 0 || Hv == 0) return hipSuccess;
  if (K != CK || V % CT != 0) return hipErrorInvalidValue;
  dim3 grid(V / CT, Hv, 1);
  hipLaunchKernelGGL(compose_kernel, grid, dim3(CTHREADS), 0, stream, M, b, s0, nullptr, Chain{0, 0, P, 0}, Hv, V,
                     starts, 1, final_state);
  return hipGetLastError();
}

}  // namespace gdn
