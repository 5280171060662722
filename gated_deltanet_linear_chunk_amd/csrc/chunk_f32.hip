// chunk_f32.hip -- chunked gated delta rule, fp32 vector-ALU kernel.
//
// The fp32 path (fp32 inputs, and bf16 inputs of the head sizes the MFMA
// kernel does not take): every product runs on the fp32 vector units, so
// results stay within ~1e-6 relative of exact arithmetic on the given inputs.
// One workgroup of 1024 threads owns (sequence, v-head, 32-column slice of V)
// and walks the sequence's 64-token chunks in order.  Per chunk, with local
// tokens r, s and G the in-chunk cumulative gate (kept in fp64 so that
// G_r - G_s does not cancel), it forms
//   A = strictly-lower(diag(beta) K K^T * e^{G_r - G_s}),  T = (I + A)^{-1},
//   R = V - diag(e^G) K S,  U = T diag(beta) R,
//   O = diag(e^G) Q S + lower(Q K^T * e^{G_r - G_s}) U,
//   S <- e^{G_last} S + (diag(e^{G_last - G}) K)^T U,
// which is the token recurrence regrouped by chunk (the UT transform's
// U = T diag(beta) V - T diag(beta e^G) K S, grouped so that no K-wide
// product of T is formed; each column of S evolves independently, hence the
// V slices).  Rows past the end of a sequence are zero with g = beta = 0,
// which leaves S and every valid output unchanged.  The kernel is bound by
// LDS reads, so every product gives each thread a small register tile (2 x 2
// of A and P, two rows of R, U and O, K / 32 rows of S) whose operands are
// each read once and used two or more times.
//
// Fused variant (ChunkArgs::cw set): the layer's short convolution feeds the
// rule on the same token-major layout (LlamaFactory PR "[v1] support GDN
// Ulysses cp", Design), so the load stage takes the raw q | k | v channels
// instead and forms each chunk row itself: depthwise causal conv over the
// row's own sequence (x is zero before its first token), SiLU, and the L2
// norm of every q and k row over its head.  The activations stay in fp32
// registers and LDS; nothing of them is stored or rounded to in_dt.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CH = 64;      // chunk length
constexpr int TB = 16;      // block size of the triangular inverse
constexpr int BV = 32;  // V columns per workgroup
constexpr int F32_THREADS = 1024;  // 4 waves per SIMD: one workgroup fills a CU's LDS
static_assert(F32_THREADS == 1024 && CH == 64 && BV == 32, "the register tiles give one tile to every thread");

template <typename TI>
__device__ __forceinline__ float ld(const TI* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

// The thread index as a value the compiler cannot see through.  Taken anew
// in every chunk step, it keeps the LDS addresses of the phases (all indexed
// by it) from being hoisted out of the chunk loop, where they would all stay
// live across it and spill.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// SiLU(bias + sum_{j<W} w[j] x[t - W + 1 + j]) for one channel at the R
// consecutive tokens t = t_first .. t_first + R - 1: x at column col of a
// token-major buffer with `stride` elements per token, counted as zero outside
// [bos, eos); tokens from eos on give 0.  The W <= 4 taps sit in the last of
// four slots (the others hold 0, adding exact zeros first), and the R + 3
// tokens the window spans are loaded once.
template <typename TI, int R>
__device__ __forceinline__ void conv_silu_rows(const TI* x, int64_t stride, int64_t col, const TI* w, const TI* b,
                                               int W, int64_t t_first, int64_t bos, int64_t eos, float (&out)[R]) {
  float w4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) w4[j] = j >= 4 - W ? ld<TI>(w, j - (4 - W)) : 0.f;
  const float bias = b ? ld<TI>(b, 0) : 0.f;
  float xw[R + 3];
#pragma unroll
  for (int u = 0; u < R + 3; ++u) {
    const int64_t tt = t_first - 3 + u;
    xw[u] = (tt >= bos && tt < eos) ? ld<TI>(x, tt * stride + col) : 0.f;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float z = bias;
#pragma unroll
    for (int j = 0; j < 4; ++j) z = fmaf(w4[j], xw[r + j], z);
    out[r] = t_first + r < eos ? z / (1.f + expf(-z)) : 0.f;
  }
}

template <int K, typename TI, bool kConv>
__global__ void __launch_bounds__(F32_THREADS) chunk_f32_kernel(ChunkArgs a) {
  __shared__ float sQ[CH][K + 1];
  __shared__ float sK[CH][K + 1];
  __shared__ float sU[CH][BV + 1];
  __shared__ float sV[CH][BV + 1];
  __shared__ float sS[K][BV + 1];
  __shared__ float sA[CH][CH + 1];  // A, later P
  __shared__ float sT[CH][CH + 1];
  __shared__ double sG[CH];
  __shared__ float sBeta[CH], sGam[CH], sDec[CH];
  __shared__ float sInv[2 * CH];  // fused conv: 1 / L2 norm of the q rows, then the k rows

  const int tid0 = threadIdx.x;
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

  // initial state: a row of s0 or of s0_seg (picked by s0_ref when set),
  // the identity (augmented M columns), or zero
  const float* s0p = nullptr;
  if (a.s0_ref) {
    const int r = a.s0_ref[seq];
    if (r >= 0)
      s0p = a.s0_seg + ((int64_t)r * a.Hv + h) * K * a.V;
    else if (r <= -2 && a.s0)
      s0p = a.s0 + ((int64_t)(-2 - r) * a.Hv + h) * K * a.V;
  } else if (a.s0_mode == 1) {
    s0p = a.s0 + ((int64_t)seq * a.Hv + h) * K * a.V;
  }
  for (int i = tid0; i < K * BV; i += F32_THREADS) {
    const int d = i / BV, c = i % BV;
    float s = 0.f;
    if (s0p)
      s = s0p[(int64_t)d * a.V + v0 + c];
    else if (a.s0_mode == 2)
      s = (d == v0 + c) ? 1.f : 0.f;
    sS[d][c] = s;
  }

  for (int64_t t0 = bos; t0 < eos; t0 += CH) {
    const int tid = opaque(tid0);
    const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);
    __syncthreads();  // previous chunk fully consumed
    if constexpr (kConv) {
      const TI* cw = (const TI*)a.cw;
      const TI* cb = (const TI*)a.cb;
      const int W = a.conv_width;
      const int64_t kc0 = (int64_t)a.Hqk * K;  // first k channel; v's follow k's
      {  // q and k: channel d, rows rb .. rb + RQ - 1
        constexpr int RQ = CH * K / F32_THREADS;
        const int d = tid % K, rb = (tid / K) * RQ;
        const int64_t c = (int64_t)hq * K + d;
        float qv[RQ], kv[RQ];
        conv_silu_rows<TI, RQ>(k, a.k_stride, c, cw + (kc0 + c) * W, cb ? cb + kc0 + c : nullptr, W, t0 + rb, bos,
                               eos, kv);
        if (a.q) {
          conv_silu_rows<TI, RQ>(q, a.q_stride, c, cw + c * W, cb ? cb + c : nullptr, W, t0 + rb, bos, eos, qv);
        } else {
#pragma unroll
          for (int r = 0; r < RQ; ++r) qv[r] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < RQ; ++r) {
          sQ[rb + r][d] = qv[r];
          sK[rb + r][d] = kv[r];
        }
      }
      {  // v: column cc of the slice, rows rb .. rb + RV - 1
        constexpr int RV = CH * BV / F32_THREADS;
        const int cc = tid % BV, rb = (tid / BV) * RV;
        const int64_t col = (int64_t)h * a.V + v0 + cc;
        float vv[RV];
        conv_silu_rows<TI, RV>(v, a.v_stride, col, cw + (2 * kc0 + col) * W, cb ? cb + 2 * kc0 + col : nullptr, W,
                               t0 + rb, bos, eos, vv);
#pragma unroll
        for (int r = 0; r < RV; ++r) sV[rb + r][cc] = vv[r];
      }
      __syncthreads();
      if (tid < 2 * CH) {
        const int r = tid % CH;
        const float* row = tid < CH ? &sQ[r][0] : &sK[r][0];
        float ss = 0.f;
        for (int d = 0; d < K; ++d) ss = fmaf(row[d], row[d], ss);
        sInv[tid] = 1.f / sqrtf(ss + a.l2_eps);
      }
      __syncthreads();
      for (int i = tid; i < CH * K; i += F32_THREADS) {
        const int r = i / K, d = i % K;
        if (r < L) {  // rows past the end stay zero
          sQ[r][d] *= sInv[r];
          sK[r][d] *= sInv[CH + r];
        }
      }
    } else {
#pragma unroll 8
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
    }
    if (tid < CH) {  // wave 0: beta, and G as an inclusive fp64 scan across the wave's lanes
      const bool ok = tid < L;
      float gv = 0.f, bv = 0.f;
      if (ok) {
        const int64_t i = (t0 + tid) * a.Hv + h;
        if (a.ga)
          gate_values(a.ga[i], a.gb[i], a.gA_log[h], a.gdt_bias[h], gv, bv);
        else {
          gv = a.g[i];
          bv = a.beta[i];
        }
      }
      sBeta[tid] = bv;
      double G = (double)gv;
#pragma unroll
      for (int off = 1; off < CH; off <<= 1) {
        const double y = __shfl_up(G, off, CH);
        if (tid >= off) G += y;
      }
      sG[tid] = G;
    }
    __syncthreads();
    if (tid < CH) {
      sGam[tid] = expf((float)sG[tid]);
      sDec[tid] = expf((float)(sG[CH - 1] - sG[tid]));
    }
    // A (strictly lower).  Register tiles: thread (r0, c0) = (tid / 32,
    // tid % 32) forms rows r0, r0 + 32 against columns c0, c0 + 32 (the
    // block (r0, c0 + 32) is above the diagonal), so that each value read
    // from LDS feeds more than one product.
    {
      const int r0 = tid >> 5, c0 = tid & 31;
      float a00 = 0.f, a10 = 0.f, a11 = 0.f;
#pragma unroll 4
      for (int d = 0; d < K; ++d) {
        const float x0 = sK[r0][d], x1 = sK[r0 + 32][d], y0 = sK[c0][d], y1 = sK[c0 + 32][d];
        a00 = fmaf(x0, y0, a00);
        a10 = fmaf(x1, y0, a10);
        a11 = fmaf(x1, y1, a11);
      }
      const bool lo = c0 < r0;
      sA[r0][c0] = lo ? sBeta[r0] * a00 * expf((float)(sG[r0] - sG[c0])) : 0.f;
      sA[r0 + 32][c0] = sBeta[r0 + 32] * a10 * expf((float)(sG[r0 + 32] - sG[c0]));
      sA[r0 + 32][c0 + 32] = lo ? sBeta[r0 + 32] * a11 * expf((float)(sG[r0 + 32] - sG[c0 + 32])) : 0.f;
      sA[r0][c0 + 32] = 0.f;
    }
    __syncthreads();
    // T = (I + A)^{-1} by 16x16 blocks (A is strictly lower, so I + A is unit
    // lower triangular).  The diagonal blocks T_ii = (I + A_ii)^{-1} come from
    // forward substitution, one column per lane in registers; below them
    // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, which follows from (I + A) T = I
    // and needs only blocks of earlier block diagonals, so the block
    // diagonals i - j = 1, 2, 3 follow one another, each as two small
    // products over all threads (the sum into sU, free until U is formed,
    // then the product with T_ii).  Blocks above the diagonal are never read.
    if (tid < CH) {
      const int b0 = (tid / TB) * TB, j = tid % TB;
      float x[TB];
#pragma unroll
      for (int r = 0; r < TB; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < r; ++u) acc = fmaf(-sA[b0 + r][b0 + u], x[u], acc);
        x[r] = r == j ? 1.f : (r < j ? 0.f : acc);
        sT[b0 + r][b0 + j] = x[r];
      }
    }
    __syncthreads();
    for (int dd = 1; dd < CH / TB; ++dd) {
      const int nb = CH / TB - dd;  // blocks on this block diagonal
      for (int t = tid; t < nb * TB * TB; t += F32_THREADS) {
        const int jb = t / (TB * TB), r = (t / TB) % TB, c = t % TB;
        const int ib = jb + dd;
        float acc = 0.f;
        for (int kb = jb; kb < ib; ++kb) {
#pragma unroll
          for (int u = 0; u < TB; ++u) acc = fmaf(sA[ib * TB + r][kb * TB + u], sT[kb * TB + u][jb * TB + c], acc);
        }
        sU[jb * TB + r][c] = acc;
      }
      __syncthreads();
      for (int t = tid; t < nb * TB * TB; t += F32_THREADS) {
        const int jb = t / (TB * TB), r = (t / TB) % TB, c = t % TB;
        const int ib = jb + dd;
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < TB; ++u) acc = fmaf(sT[ib * TB + r][ib * TB + u], sU[jb * TB + u][c], acc);
        sT[ib * TB + r][jb * TB + c] = -acc;
      }
      __syncthreads();
    }
    // P = lower(Q K^T * D) into sA (tiles as for A), R = V - diag(gamma) K S
    // in place of V (rows r0, r0 + 32 of column c0), and T <- T diag(beta)
    {
      const int r0 = tid >> 5, c0 = tid & 31;
      float p00 = 0.f, p10 = 0.f, p11 = 0.f, k0 = 0.f, k1 = 0.f;
#pragma unroll 4
      for (int d = 0; d < K; ++d) {
        const float x0 = sQ[r0][d], x1 = sQ[r0 + 32][d], y0 = sK[c0][d], y1 = sK[c0 + 32][d];
        p00 = fmaf(x0, y0, p00);
        p10 = fmaf(x1, y0, p10);
        p11 = fmaf(x1, y1, p11);
      }
#pragma unroll 4
      for (int d = 0; d < K; ++d) {
        const float sv = sS[d][c0];
        k0 = fmaf(sK[r0][d], sv, k0);
        k1 = fmaf(sK[r0 + 32][d], sv, k1);
      }
      const bool lo = c0 <= r0;
      sA[r0][c0] = lo ? p00 * expf((float)(sG[r0] - sG[c0])) : 0.f;
      sA[r0 + 32][c0] = p10 * expf((float)(sG[r0 + 32] - sG[c0]));
      sA[r0 + 32][c0 + 32] = lo ? p11 * expf((float)(sG[r0 + 32] - sG[c0 + 32])) : 0.f;
      sA[r0][c0 + 32] = 0.f;
      sV[r0][c0] = fmaf(-sGam[r0], k0, sV[r0][c0]);
      sV[r0 + 32][c0] = fmaf(-sGam[r0 + 32], k1, sV[r0 + 32][c0]);
      sT[r0][c0] *= sBeta[c0];
      sT[r0 + 32][c0] *= sBeta[c0];
      sT[r0 + 32][c0 + 32] *= sBeta[c0 + 32];
    }
    __syncthreads();
    // U = (T diag(beta)) R, rows r0 and r0 + 32 of column c0
    {
      const int r0 = tid >> 5, c0 = tid & 31;
      float u0 = 0.f, u1 = 0.f;
      for (int s = 0; s <= r0; ++s) {
        const float rv = sV[s][c0];
        u0 = fmaf(sT[r0][s], rv, u0);
        u1 = fmaf(sT[r0 + 32][s], rv, u1);
      }
      for (int s = r0 + 1; s <= r0 + 32; ++s) u1 = fmaf(sT[r0 + 32][s], sV[s][c0], u1);
      sU[r0][c0] = u0;
      sU[r0 + 32][c0] = u1;
    }
    __syncthreads();
    // O = diag(gamma) Q S + P U
    if (a.o) {  // rows r0 and r0 + 32 of column c0
      const int r0 = tid >> 5, c0 = tid & 31;
      float q0 = 0.f, q1 = 0.f, w0 = 0.f, w1 = 0.f;
#pragma unroll 4
      for (int d = 0; d < K; ++d) {
        const float sv = sS[d][c0];
        q0 = fmaf(sQ[r0][d], sv, q0);
        q1 = fmaf(sQ[r0 + 32][d], sv, q1);
      }
      for (int s = 0; s <= r0; ++s) {
        const float uv = sU[s][c0];
        w0 = fmaf(sA[r0][s], uv, w0);
        w1 = fmaf(sA[r0 + 32][s], uv, w1);
      }
      for (int s = r0 + 1; s <= r0 + 32; ++s) w1 = fmaf(sA[r0 + 32][s], sU[s][c0], w1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = r0 + 32 * j;
        if (r >= L) continue;
        const float out = a.scale * fmaf(sGam[r], j ? q1 : q0, j ? w1 : w0);
        const int64_t off = ((t0 + r) * a.Hv + h) * (int64_t)a.V + v0 + c0;
        if (a.o_dt == 1)
          ((uint16_t*)a.o)[off] = f32_to_bf16_bits(out);
        else
          ((float*)a.o)[off] = out;
      }
      __syncthreads();
    }
    // S <- gamma_last S + (diag(dec) K)^T U: rows d0 + 32 j (j < K / 32) of
    // column c0
    {
      constexpr int NR = K / 32;
      const int d0 = tid >> 5, c0 = tid & 31;
      const float gl = sGam[CH - 1];
      float acc[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = 0.f;
#pragma unroll 4
      for (int s = 0; s < CH; ++s) {
        const float du = sDec[s] * sU[s][c0];
#pragma unroll
        for (int j = 0; j < NR; ++j) acc[j] = fmaf(sK[s][d0 + 32 * j], du, acc[j]);
      }
#pragma unroll
      for (int j = 0; j < NR; ++j) sS[d0 + 32 * j][c0] = fmaf(gl, sS[d0 + 32 * j][c0], acc[j]);
    }
  }
  __syncthreads();
  const int out_row = a.sf_map ? a.sf_map[seq] : seq;  // -1: no final state for this sequence
  if (a.sf && out_row >= 0) {
    float* dst = a.sf + (int64_t)out_row * a.sf_seq_stride + (int64_t)h * a.sf_head_stride;
    for (int i = tid0; i < K * BV; i += F32_THREADS) {
      const int d = i / BV, c = i % BV;
      dst[(int64_t)d * a.sf_row_stride + v0 + c] = sS[d][c];
    }
  }
}

template <int K>
hipError_t launch_k(const ChunkArgs& a, hipStream_t stream) {
  dim3 grid(a.V / BV, a.Hv, a.n_seqs);
  const bool conv = a.cw != nullptr;
  if (a.in_dt == 1 && conv)
    hipLaunchKernelGGL((chunk_f32_kernel<K, uint16_t, true>), grid, dim3(F32_THREADS), 0, stream, a);
  else if (a.in_dt == 1)
    hipLaunchKernelGGL((chunk_f32_kernel<K, uint16_t, false>), grid, dim3(F32_THREADS), 0, stream, a);
  else if (conv)
    hipLaunchKernelGGL((chunk_f32_kernel<K, float, true>), grid, dim3(F32_THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((chunk_f32_kernel<K, float, false>), grid, dim3(F32_THREADS), 0, stream, a);
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
