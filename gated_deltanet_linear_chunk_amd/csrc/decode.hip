// decode.hip -- the recurrent decode step: one new token per sequence.
//
// After a prefill hands over its final state (the sglang fork PR "Qwen3.5 cp -
// #1" passes the final state to the standard decode path), each new token of
// sequence n updates the K x V fp32 state of every v-head h in place:
//   S <- e^g S;  u = beta (v - S^T k);  S <- S + k u^T;  o = scale S^T q,
// the token recurrence itself.  Per (sequence, head) the step reads and
// writes the whole state (K V fp32) against O(K + V) other numbers, so it is
// bound by HBM: one pass over the state, which stays in registers between the
// two column sums over K.
//
// The state is read and written once per step, so its loads and stores are
// non-temporal (streamed past the caches: 0.222 -> 0.202 ms for 256
// sequences at H_v = 32, K = V = 128).
//
// One workgroup owns (sequence, v-head, a slice of state columns): 512
// threads over 64 columns when V % 64 == 0 (about 3 % faster on 256 sequences
// at H_v = 32, K = V = 128 than 256 threads over 32, which serve the other V).
// A thread holds four columns of the slice in K / 32 consecutive rows (its
// row group): one 16-byte load and one store per row, the column groups of a
// row covering its slice contiguously.  The column sums over the K rows
// (S^T k, then S^T q of the updated state) reduce over the row groups of a
// wave with lane exchanges and over the waves through LDS.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

// Workgroup shape: NT threads over NC state columns.  Thread t holds the
// four columns 4 (t % (NC / 4)) .. + 3 in the K / (NT / (NC / 4)) rows of row
// group t / (NC / 4).
constexpr int kWideThreads = 512, kWideCols = 64;     // V % 64 == 0
constexpr int kNarrowThreads = 256, kNarrowCols = 32; // V % 32 == 0

template <typename T>
__device__ __forceinline__ float load_f(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_f<float>(const float* p, int64_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store4(T* p, f32x4 x);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 x) {
  *reinterpret_cast<f32x4*>(p) = x;
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, f32x4 x) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}

// Sum over the row groups of the workgroup (lanes NC / 4 apart in a wave, then
// the waves through LDS); every thread gets the totals of its four columns.
template <int NT, int NC>
__device__ __forceinline__ f32x4 column_sum(f32x4 p, float (*red)[NC], int wave, int lane, int c4) {
#pragma unroll
  for (int off = NC / 4; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] += __shfl_xor(p[e], off, 64);
  if (lane < NC / 4) *reinterpret_cast<f32x4*>(&red[wave][4 * c4]) = p;
  __syncthreads();
  f32x4 t = *reinterpret_cast<const f32x4*>(&red[0][4 * c4]);
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) t += *reinterpret_cast<const f32x4*>(&red[w][4 * c4]);
  return t;
}

template <int K, int NT, int NC, typename Tin, typename Tout>
__global__ void __launch_bounds__(NT) decode_kernel(DecodeArgs a) {
  constexpr int CG = NC / 4;     // column groups of four
  constexpr int NRG = NT / CG;   // row groups
  constexpr int RPG = K / NRG;   // rows per row group
  static_assert(NT % 64 == 0 && 64 % CG == 0 && K % NRG == 0 && RPG >= 1, "workgroup shape");
  __shared__ __attribute__((aligned(16))) float red_k[NT / 64][NC];
  __shared__ __attribute__((aligned(16))) float red_q[NT / 64][NC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c4 = tid % CG, rg = tid / CG;
  const int h = blockIdx.y, n = blockIdx.z;
  const int hq = h / (a.Hv / a.Hqk);
  const int j0 = blockIdx.x * NC + 4 * c4;
  const int64_t r = a.state_indices ? (int64_t)a.state_indices[n] : (int64_t)n;
  Tout* o = reinterpret_cast<Tout*>(a.o) + ((int64_t)n * a.Hv + h) * a.V + j0;
  if (r < 0 || r >= a.n_state_rows) {  // a skipped slot (uniform over the workgroup)
    if (rg == 0) store4<Tout>(o, f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  float* S = a.state + ((r * a.Hv + h) * K + rg * RPG) * (int64_t)a.V + j0;
  f32x4 s[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(S + (int64_t)i * a.V));
  const Tin* kp = reinterpret_cast<const Tin*>(a.k) + ((int64_t)n * a.Hqk + hq) * K + rg * RPG;
  const Tin* qp = reinterpret_cast<const Tin*>(a.q) + ((int64_t)n * a.Hqk + hq) * K + rg * RPG;
  const Tin* vp = reinterpret_cast<const Tin*>(a.v) + ((int64_t)n * a.Hv + h) * a.V + j0;
  float kv[RPG], qv[RPG];
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    kv[i] = load_f<Tin>(kp, i);
    qv[i] = load_f<Tin>(qp, i);
  }
  const f32x4 vv = {load_f<Tin>(vp, 0), load_f<Tin>(vp, 1), load_f<Tin>(vp, 2), load_f<Tin>(vp, 3)};
  const float decay = expf(a.g[(int64_t)n * a.Hv + h]);
  const float bt = a.beta[(int64_t)n * a.Hv + h];

  // S <- e^g S, and this thread's rows of S^T k
  f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    s[i] *= decay;
    p += s[i] * kv[i];
  }
  const f32x4 sk = column_sum<NT, NC>(p, red_k, wave, lane, c4);
  const f32x4 u = bt * (vv - sk);
  // S <- S + k u^T, written back, and this thread's rows of S^T q
  f32x4 pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPG; ++i) {
    s[i] += kv[i] * u;
    __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4*>(S + (int64_t)i * a.V));
    pq += s[i] * qv[i];
  }
  const f32x4 sq = column_sum<NT, NC>(pq, red_q, wave, lane, c4);
  if (tid < CG) store4<Tout>(o, a.scale * sq);
}

template <int K, int NT, int NC>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.V / NC), (unsigned)a.Hv, (unsigned)a.N);
  if (a.in_dt == 1) {
    if (a.o_dt == 1)
      hipLaunchKernelGGL((decode_kernel<K, NT, NC, uint16_t, uint16_t>), grid, dim3(NT), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<K, NT, NC, uint16_t, float>), grid, dim3(NT), 0, stream, a);
  } else {
    if (a.o_dt == 1)
      hipLaunchKernelGGL((decode_kernel<K, NT, NC, float, uint16_t>), grid, dim3(NT), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_kernel<K, NT, NC, float, float>), grid, dim3(NT), 0, stream, a);
  }
  return hipGetLastError();
}

template <int K>
hipError_t launch_k(const DecodeArgs& a, hipStream_t stream) {
  return a.V % kWideCols == 0 ? launch_shape<K, kWideThreads, kWideCols>(a, stream)
                              : launch_shape<K, kNarrowThreads, kNarrowCols>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  if (a.V % kNarrowCols != 0) return hipErrorInvalidValue;
  switch (a.K) {
    case 32: return launch_k<32>(a, stream);
    case 64: return launch_k<64>(a, stream);
    case 128: return launch_k<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
