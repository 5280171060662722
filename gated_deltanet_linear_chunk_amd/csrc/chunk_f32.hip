// chunk_f32.hip -- chunked gated delta rule, fp32 vector-ALU kernel.
//
// The fp32 path (fp32 inputs, and bf16 inputs of the head sizes the MFMA
// kernel does not take): every product runs on the fp32 vector units, so
// results stay within ~1e-6 relative of exact arithmetic on the given inputs.
// One workgroup owns (sequence, v-head, 32-column slice of V; 16 columns for
// K = 128) and walks the
// sequence's 64-token chunks in order.  Per chunk, with local tokens r, s and
// G the in-chunk cumulative gate (kept in fp64 so that G_r - G_s does not
// cancel), it forms
//   A = strictly-lower(diag(beta) K K^T * e^{G_r - G_s}),  T = (I + A)^{-1},
//   W = T diag(beta e^G) K,  U0 = T diag(beta) V,
//   U = U0 - W S,  O = diag(e^G) Q S + lower(Q K^T * e^{G_r - G_s}) U,
//   S <- e^{G_last} S + (diag(e^{G_last - G}) K)^T U,
// which is the token recurrence regrouped by chunk (each column of S evolves
// independently, hence the V slices).  Rows past the end of a sequence are
// zero with g = beta = 0, which leaves S and every valid output unchanged.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CH = 64;      // chunk length
constexpr int F32_BV = 32;  // V columns per workgroup (16 for K = 128, which needs the LDS for Q, K, W)

template <int K>
constexpr int f32_bv() { return K >= 128 ? 16 : F32_BV; }
constexpr int F32_THREADS = 256;

template <typename TI>
__device__ __forceinline__ float ld(const TI* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <int K, typename TI>
__global__ void __launch_bounds__(F32_THREADS) chunk_f32_kernel(ChunkArgs a) {
  constexpr int BV = f32_bv<K>();
  __shared__ float sQ[CH][K + 1];
  __shared__ float sK[CH][K + 1];
  __shared__ float sW[CH][K + 1];
  __shared__ float sU[CH][BV + 1];
  __shared__ float sV[CH][BV + 1];
  __shared__ float sS[K][BV + 1];
  __shared__ float sA[CH][CH + 1];  // A, later P
  __shared__ float sT[CH][CH + 1];
  __shared__ double sG[CH];
  __shared__ float sBeta[CH], sGam[CH], sDec[CH];

  const int tid = threadIdx.x;
  const int v0 = blockIdx.x * BV;
  const int h = blockIdx.y;
  const int seq = blockIdx.z;
  const int hq = h / (a.Hv / a.Hqk);
  int64_t bos, eos;
  if (a.cu) {
    bos = clampi(a.cu[seq], 0, a.Ttot);
    eos = clampi(a.cu[seq + 1], bos, a.Ttot);
  } else {
    bos = (int64_t)seq * a.row_len;
    eos = bos + a.row_len;
  }
  const TI* q = (const TI*)a.q;
  const TI* k = (const TI*)a.k;
  const TI* v = (const TI*)a.v;

  // initial state
  for (int i = tid; i < K * BV; i += F32_THREADS) {
    const int d = i / BV, c = i % BV;
    float s = 0.f;
    if (a.s0_mode == 1)
      s = a.s0[((int64_t)seq * a.Hv + h) * K * a.V + (int64_t)d * a.V + v0 + c];
    else if (a.s0_mode == 2)
      s = (d == v0 + c) ? 1.f : 0.f;
    sS[d][c] = s;
  }

  for (int64_t t0 = bos; t0 < eos; t0 += CH) {
    const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);
    __syncthreads();  // previous chunk fully consumed
    for (int i = tid; i < CH * K; i += F32_THREADS) {
      const int r = i / K, d = i % K;
      float qv = 0.f, kv = 0.f;
      if (r < L) {
        kv = ld<TI>(k, (t0 + r) * a.k_stride + (int64_t)hq * K + d);
        if (a.q) qv = ld<TI>(q, (t0 + r) * a.q_stride + (int64_t)hq * K + d);
      }
      sQ[r][d] = qv;
      sK[r][d] = kv;
    }
    for (int i = tid; i < CH * BV; i += F32_THREADS) {
      const int r = i / BV, c = i % BV;
      float vv = 0.f;
      if (r < L && a.v) vv = ld<TI>(v, (t0 + r) * a.v_stride + (int64_t)h * a.V + v0 + c);
      sV[r][c] = vv;
    }
    if (tid < CH) {
      const bool ok = tid < L;
      sBeta[tid] = ok ? a.beta[(t0 + tid) * a.Hv + h] : 0.f;
    }
    if (tid == 0) {
      double G = 0.0;
      for (int r = 0; r < CH; ++r) {
        if (r < L) G += (double)a.g[(t0 + r) * a.Hv + h];
        sG[r] = G;
      }
    }
    __syncthreads();
    if (tid < CH) {
      sGam[tid] = expf((float)sG[tid]);
      sDec[tid] = expf((float)(sG[CH - 1] - sG[tid]));
    }
    // A (strictly lower)
    for (int i = tid; i < CH * CH; i += F32_THREADS) {
      const int r = i / CH, s = i % CH;
      float val = 0.f;
      if (s < r) {
        float acc = 0.f;
#pragma unroll 8
        for (int d = 0; d < K; ++d) acc = fmaf(sK[r][d], sK[s][d], acc);
        val = sBeta[r] * acc * expf((float)(sG[r] - sG[s]));
      }
      sA[r][s] = val;
    }
    __syncthreads();
    // T = (I + A)^{-1}, one column per thread, forward substitution
    if (tid < CH) {
      const int j = tid;
      for (int r = 0; r < CH; ++r) {
        float val = 0.f;
        if (r == j) {
          val = 1.f;
        } else if (r > j) {
          for (int s = j; s < r; ++s) val = fmaf(-sA[r][s], sT[s][j], val);
        }
        sT[r][j] = val;
      }
    }
    __syncthreads();
    // P (into sA), W, U0
    for (int i = tid; i < CH * CH; i += F32_THREADS) {
      const int r = i / CH, s = i % CH;
      float val = 0.f;
      if (s <= r) {
        float acc = 0.f;
#pragma unroll 8
        for (int d = 0; d < K; ++d) acc = fmaf(sQ[r][d], sK[s][d], acc);
        val = acc * expf((float)(sG[r] - sG[s]));
      }
      sA[r][s] = val;
    }
    for (int i = tid; i < CH * K; i += F32_THREADS) {
      const int r = i / K, d = i % K;
      float acc = 0.f;
      for (int s = 0; s <= r; ++s) acc = fmaf(sT[r][s] * sBeta[s] * sGam[s], sK[s][d], acc);
      sW[r][d] = acc;
    }
    for (int i = tid; i < CH * BV; i += F32_THREADS) {
      const int r = i / BV, c = i % BV;
      float acc = 0.f;
      for (int s = 0; s <= r; ++s) acc = fmaf(sT[r][s] * sBeta[s], sV[s][c], acc);
      sU[r][c] = acc;
    }
    __syncthreads();
    // U = U0 - W S
    for (int i = tid; i < CH * BV; i += F32_THREADS) {
      const int r = i / BV, c = i % BV;
      float acc = sU[r][c];
#pragma unroll 8
      for (int d = 0; d < K; ++d) acc = fmaf(-sW[r][d], sS[d][c], acc);
      sU[r][c] = acc;
    }
    __syncthreads();
    // O = diag(gamma) Q S + P U
    if (a.o) {
      for (int i = tid; i < CH * BV; i += F32_THREADS) {
        const int r = i / BV, c = i % BV;
        if (r >= L) continue;
        float qs = 0.f;
#pragma unroll 8
        for (int d = 0; d < K; ++d) qs = fmaf(sQ[r][d], sS[d][c], qs);
        float pu = 0.f;
        for (int s = 0; s <= r; ++s) pu = fmaf(sA[r][s], sU[s][c], pu);
        const float out = a.scale * fmaf(sGam[r], qs, pu);
        const int64_t off = ((t0 + r) * a.Hv + h) * (int64_t)a.V + v0 + c;
        if (a.o_dt == 1)
          ((uint16_t*)a.o)[off] = f32_to_bf16_bits(out);
        else
          ((float*)a.o)[off] = out;
      }
      __syncthreads();
    }
    // S <- gamma_last S + (diag(dec) K)^T U
    const float gl = sGam[CH - 1];
    for (int i = tid; i < K * BV; i += F32_THREADS) {
      const int d = i / BV, c = i % BV;
      float acc = 0.f;
      for (int s = 0; s < CH; ++s) acc = fmaf(sK[s][d] * sDec[s], sU[s][c], acc);
      sS[d][c] = fmaf(gl, sS[d][c], acc);
    }
  }
  __syncthreads();
  if (a.sf) {
    float* dst = a.sf + (int64_t)seq * a.sf_seq_stride + (int64_t)h * a.sf_head_stride;
    for (int i = tid; i < K * BV; i += F32_THREADS) {
      const int d = i / BV, c = i % BV;
      dst[(int64_t)d * a.sf_row_stride + v0 + c] = sS[d][c];
    }
  }
}

template <int K>
hipError_t launch_k(const ChunkArgs& a, hipStream_t stream) {
  dim3 grid(a.V / f32_bv<K>(), a.Hv, a.n_seqs);
  if (a.in_dt == 1)
    hipLaunchKernelGGL((chunk_f32_kernel<K, uint16_t>), grid, dim3(F32_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((chunk_f32_kernel<K, float>), grid, dim3(F32_THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a, hipStream_t stream) {
  if (a.n_seqs == 0 || a.Hv == 0) return hipSuccess;
  switch (a.K) {
    case 32: return launch_k<32>(a, stream);
    case 64: return launch_k<64>(a, stream);
    case 128: return launch_k<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
