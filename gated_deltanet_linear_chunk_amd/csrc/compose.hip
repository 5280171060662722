// compose.hip -- fp32 chain of segment affine maps.
//
// Given per-segment maps S_end = M_i S_start + b_i, the true start state of
// every segment follows from S_start,0 = S0 and S_start,i+1 = M_i S_start,i + b_i,
// composed in fp32 (the sglang fork PR "Qwen3.5 cp - #1" chain-reduces its
// (b, M) pairs in fp32).  Each column of the K x V state is its own affine
// chain, so the work is split over (v-head, 16-column slice).  A step is the
// 128 x 128 by 128 x 16 product M_i S on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32, fp32 products and sums): wave w of the workgroup owns
// row tiles 2w and 2w + 1, reads its rows of M_i straight from global memory
// (16-byte loads, all in flight at once, issued one step ahead) and the state
// slice from LDS.  The k
// order of the sums is free, so lane group g (lanes 16g .. 16g + 15) takes
// k = 32 g + s at step s, which makes its M reads contiguous.  Segments follow
// one another inside the workgroup, which needs only the M S products (a tree
// over segments would also need M M products, K / 16 times more work per
// level).
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CK = 128;  // key dim
constexpr int CT = 16;   // state columns per workgroup
constexpr int CTHREADS = 256;
// State slice in LDS: row k at k * CT + 16 * (k / 32), so that the four lane
// groups of a fragment read (rows 32 apart) fall on different banks.
constexpr int SROWS = CK * CT + 16 * (CK / 32);

__device__ __forceinline__ int sidx(int k, int c) { return k * CT + c + 16 * (k >> 5); }

struct Chain {
  int n, p0, count, out0;
};

// s0 and out may be one buffer (a chain that starts from a row another launch
// wrote, and writes later rows of it): neither is restrict-qualified.
__global__ void __launch_bounds__(CTHREADS) compose_kernel(const float* __restrict__ M,
                                                           const float* __restrict__ b, const float* s0,
                                                           const int32_t* __restrict__ chains,
                                                           Chain single, int Hv, int V, float* out,
                                                           int write_before, float* __restrict__ final_state) {
  __shared__ float sS[2][SROWS];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c = lane & 15;  // lane group, column within the slice
  // 1-D grid over (slice, unit = chain * Hv + head).  Workgroups go to the
  // eight XCDs in turn by id, and every slice of a unit reads all of its M, so
  // when the units split evenly the slices of a unit get ids eight apart (one
  // XCD, one L2 copy of M); otherwise slices of a unit are consecutive.
  const int n_slices = V / CT, n_units = (int)(gridDim.x / n_slices);
  int slice, unit;
  if (n_units % 8 == 0) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    unit = x + 8 * (j / n_slices);
    slice = j % n_slices;
  } else {
    slice = blockIdx.x % n_slices;
    unit = blockIdx.x / n_slices;
  }
  const int c0 = slice * CT;
  const int h = unit % Hv;
  const int ci = unit / Hv;
  const Chain ch = chains ? Chain{chains[4 * ci], chains[4 * ci + 1], chains[4 * ci + 2], chains[4 * ci + 3]}
                          : single;

  const int64_t head = (int64_t)h * CK * V;
  const int64_t row = (int64_t)Hv * CK * V;  // one [Hv, K, V] state
  // accumulator element e of row tile t: row 16 (2 wave + t) + 4 g + e, column c
  int orow[2][4];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) orow[t][e] = 16 * (2 * wave + t) + 4 * g + e;
  // The loads of step j + 1 (rows of M and the b slice) are issued before the
  // products of step j, and those of step 0 with the start state, so a chain
  // waits on memory about once rather than once per step.  A operands: rows
  // 16 (2 wave + t) + c of M, k = 32 g .. 32 g + 31.
  // A chain from a zero state (no s0 row) has b_0 as its first result exactly
  // (M_0 0 adds only zeros), so its first step neither loads M_0 nor
  // multiplies, and M_1 is on its way at once.
  const bool zero_start = !(s0 && ch.n >= 0);
  f32x4 ma[2][8], bq[2];
  auto load_step = [&](int j, bool with_m) {
    const int seg = ch.p0 + j;
    const float* Mseg = M + ((int64_t)seg * Hv + h) * CK * CK;
    const float* bseg = b + (int64_t)seg * row + head + c0 + c;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (with_m) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          ma[t][q] =
              *reinterpret_cast<const f32x4*>(Mseg + (int64_t)(16 * (2 * wave + t) + c) * CK + 32 * g + 4 * q);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) bq[t][e] = bseg[(int64_t)orow[t][e] * V];
    }
  };
  if (ch.count > 0) load_step(0, !zero_start);
  for (int i = tid; i < CK * CT; i += CTHREADS) {
    const int r = i / CT, cc = i % CT;
    sS[0][sidx(r, cc)] = (s0 && ch.n >= 0) ? s0[ch.n * row + head + (int64_t)r * V + c0 + cc] : 0.f;
  }
  __syncthreads();
  int cur = 0;
  for (int j = 0; j < ch.count; ++j) {
    float* dst = out + (int64_t)(ch.out0 + j) * row + head + c0 + c;
    const bool product = j > 0 || !zero_start;
    f32x4 mcur[2][8], acc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t] = bq[t];
      if (product) {
#pragma unroll
        for (int q = 0; q < 8; ++q) mcur[t][q] = ma[t][q];
      }
    }
    if (j + 1 < ch.count) load_step(j + 1, true);
    if (write_before) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(int64_t)orow[t][e] * V] = sS[cur][sidx(orow[t][e], c)];
    }
    if (product) {
#pragma unroll
      for (int s = 0; s < 32; ++s) {
        const float bv = sS[cur][sidx(32 * g + s, c)];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(mcur[t][s >> 2][s & 3], bv, acc[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sS[cur ^ 1][sidx(orow[t][e], c)] = acc[t][e];
        if (!write_before) dst[(int64_t)orow[t][e] * V] = acc[t][e];
      }
    cur ^= 1;
    __syncthreads();
  }
  if (final_state) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        final_state[ci * row + head + (int64_t)orow[t][e] * V + c0 + c] = sS[cur][sidx(orow[t][e], c)];
  }
}

}  // namespace

hipError_t launch_compose_chains(const float* M, const float* b, const float* s0,
                                 const int32_t* chains, int n_chains, int Hv, int K, int V,
                                 float* out, int write_before, float* final_state,
                                 hipStream_t stream) {
  if (n_chains == 0 || Hv == 0) return hipSuccess;
  if (K != CK || V % CT != 0) return hipErrorInvalidValue;
  if ((int64_t)(V / CT) * Hv * n_chains > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((V / CT) * Hv * n_chains));
  hipLaunchKernelGGL(compose_kernel, grid, dim3(CTHREADS), 0, stream, M, b, s0, chains, Chain{0, 0, 0, 0}, Hv, V,
                     out, write_before, final_state);
  return hipGetLastError();
}

// One chain over P maps of one sequence from row 0 of s0.
hipError_t launch_compose(const float* M, const float* b, const float* s0, int P, int Hv, int K,
                          int V, float* out, int write_before, float* final_state, hipStream_t stream) {
  if (P == 0 || Hv == 0) return hipSuccess;
  if (K != CK || V % CT != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((V / CT) * Hv));
  hipLaunchKernelGGL(compose_kernel, grid, dim3(CTHREADS), 0, stream, M, b, s0, nullptr, Chain{0, 0, P, 0}, Hv, V,
                     out, write_before, final_state);
  return hipGetLastError();
}

// Index arrays travel to the device inside kernel arguments, which the launch
// itself copies: no host-to-device copy (and no pageable host read) on the
// stream.  One workgroup stores up to kPlanArgInts values.
__global__ void __launch_bounds__(256) plan_store_kernel(PlanArg p, int32_t* __restrict__ dst) {
  for (int i = threadIdx.x; i < p.n; i += 256) dst[i] = p.v[i];
}

hipError_t launch_plan_store(const int32_t* ints, int64_t n, int32_t* dst, hipStream_t stream) {
  for (int64_t i0 = 0; i0 < n; i0 += kPlanArgInts) {
    PlanArg p;
    p.n = (int)(n - i0 < kPlanArgInts ? n - i0 : kPlanArgInts);
    for (int i = 0; i < p.n; ++i) p.v[i] = ints[i0 + i];
    hipLaunchKernelGGL(plan_store_kernel, dim3(1), dim3(256), 0, stream, p, dst + i0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
