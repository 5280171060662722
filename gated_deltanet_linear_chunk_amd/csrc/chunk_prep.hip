// chunk_prep.hip -- per-chunk UT transform matrix T = (I + A)^{-1}, in parallel.
//
// For a 64-token chunk with local tokens r, s and in-chunk cumulative gate
// G (fp64), A = strictly-lower(diag(beta) K K^T * e^{G_r - G_s}) and
// T = (I + A)^{-1} is unit lower triangular.  T depends only on k, g and beta
// of its own chunk, never on the recurrent state, so it is computed here for
// every (chunk, v-head) at once, off the serial chunk scan, and stored in fp32.
//
// One wave owns one (chunk slot, v-head), so there is no cross-wave
// synchronisation and many waves share a compute unit: the K fragments come
// straight from global memory into the 16 x 16 x 32 bf16 MFMA for K K^T (exact
// products, fp32 sums); the mask is applied in registers; the four 16 x 16
// diagonal blocks are inverted by forward substitution (lane = block, column);
// the block rows follow from T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj with each
// lane producing four entries of a block row.
//
// Storage: the 10 lower 16 x 16 blocks (i >= j, index i(i+1)/2 + j), row-major
// inside a block, zeros above the diagonal of diagonal blocks:
//   tbuf[((slot * Hv + h) * 10 + blk) * 256 + 16 * r + c].
// Chunk slots: chunk j of sequence n (first token cu[n] + 64 j) has slot
// floor((cu[n] + 64 j) / 64) + n, which is unique and below
// ceil(T / 64) + n_seqs; unused slots are skipped.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CH = 64;
constexpr int KD = 128;
constexpr int BP = 17;  // fp32 pitch of a 16 x 16 block in LDS

__device__ __forceinline__ int64_t seq_begin(const ChunkArgs& a, int n) {
  return a.cu ? (int64_t)clampi(a.cu[n], 0, a.Ttot) : (int64_t)n * a.row_len;
}

__device__ __forceinline__ int blk(int i, int j) { return (i * (i + 1)) / 2 + j; }

__global__ void __launch_bounds__(64) chunk_prep_kernel(ChunkArgs a) {
  __shared__ float sA[10][16][BP];
  __shared__ float sT[10][16][BP];
  __shared__ float sY[16][BP];
  __shared__ double sG[CH];
  __shared__ float sBeta[CH];

  const int lane = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int slot = blockIdx.x;
  const int h = blockIdx.y;
  const int hq = h / (a.Hv / a.Hqk);

  // sequence n owning this slot: the largest n with floor(cu[n]/64) + n <= slot
  int lo = 0, hi = a.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((seq_begin(a, mid) >> 6) + mid <= slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int n = lo;
  const int64_t bos = seq_begin(a, n);
  const int64_t eos = a.cu ? (int64_t)clampi(a.cu[n + 1], bos, a.Ttot) : bos + a.row_len;
  const int64_t j0 = (int64_t)slot - ((bos >> 6) + n);
  if (j0 < 0) return;
  const int64_t t0 = bos + 64 * j0;
  if (t0 >= eos) return;  // unused slot
  const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);

  // ---- gates ----------------------------------------------------------------
  {
    const bool ok = lane < L;
    double G = ok ? (double)a.g[(t0 + lane) * a.Hv + h] : 0.0;
    sBeta[lane] = ok ? a.beta[(t0 + lane) * a.Hv + h] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(G, off, 64);
      if (lane >= off) G += o;
    }
    sG[lane] = G;
  }

  // ---- K fragments straight from global memory: row tile i, k-step m -------
  // (contiguous k = 32 m + 8 g4 .. +7 in both operands; rows past L are zero)
  const uint16_t* kg = (const uint16_t*)a.k + (int64_t)hq * KD + 8 * g4;
  bf16x8 kf[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * i + c16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < L) v = *reinterpret_cast<const u32x4*>(kg + (t0 + r) * a.k_stride + 32 * m);
      kf[i][m] = __builtin_bit_cast(bf16x8, v);
    }
  }
  __syncthreads();  // sG, sBeta visible to all lanes

  // ---- A = strictly-lower(diag(beta) K K^T * decay), 10 tiles ---------------
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = mfma16(kf[i][m], kf[j][m], acc);
      const int s = 16 * j + c16;
      const double Gs = sG[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 4 * g4 + e, r = 16 * i + rr;
        sA[blk(i, j)][rr][c16] = (r > s) ? sBeta[r] * acc[e] * expf((float)(sG[r] - Gs)) : 0.f;
      }
    }
  __syncthreads();

  // ---- diagonal blocks: lane = (block b, column c) ---------------------------
  {
    const int b = g4, c = c16;
    const float(*Ab)[BP] = sA[blk(b, b)];
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float val = (r == c) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < r; ++s) val = fmaf(-Ab[r][s], x[s], val);
      x[r] = val;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[blk(b, b)][r][c] = x[r];
  }
  __syncthreads();

  // ---- block rows: lane = (row rr, columns 4 c4 .. 4 c4 + 3) ----------------
  {
    const int rr = lane >> 2, c4 = (lane & 3) * 4;
    for (int i = 1; i < 4; ++i) {
      for (int jb = 0; jb < i; ++jb) {
        float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
        for (int kb = jb; kb < i; ++kb) {
          const float* Ar = sA[blk(i, kb)][rr];
          const float(*Tk)[BP] = sT[blk(kb, jb)];
#pragma unroll
          for (int s = 0; s < 16; ++s) {
            const float av = Ar[s];
            y0 = fmaf(av, Tk[s][c4], y0);
            y1 = fmaf(av, Tk[s][c4 + 1], y1);
            y2 = fmaf(av, Tk[s][c4 + 2], y2);
            y3 = fmaf(av, Tk[s][c4 + 3], y3);
          }
        }
        sY[rr][c4] = y0;
        sY[rr][c4 + 1] = y1;
        sY[rr][c4 + 2] = y2;
        sY[rr][c4 + 3] = y3;
        __syncthreads();
        const float* Ti = sT[blk(i, i)][rr];
        float t0v = 0.f, t1v = 0.f, t2v = 0.f, t3v = 0.f;
#pragma unroll
        for (int mm = 0; mm < 16; ++mm) {
          const float tv = Ti[mm];  // zero above the diagonal
          t0v = fmaf(tv, sY[mm][c4], t0v);
          t1v = fmaf(tv, sY[mm][c4 + 1], t1v);
          t2v = fmaf(tv, sY[mm][c4 + 2], t2v);
          t3v = fmaf(tv, sY[mm][c4 + 3], t3v);
        }
        float* dst = sT[blk(i, jb)][rr];
        dst[c4] = -t0v;
        dst[c4 + 1] = -t1v;
        dst[c4 + 2] = -t2v;
        dst[c4 + 3] = -t3v;
        __syncthreads();
      }
    }
  }

  // ---- write the 10 blocks: 640 float4, 10 per lane --------------------------
  float* out = a.tbuf + ((int64_t)slot * a.Hv + h) * 2560;
#pragma unroll
  for (int u = 0; u < 10; ++u) {
    const int f = lane + 64 * u;
    const int b = f >> 6, e4 = (f & 63) * 4, rr = e4 >> 4, cc = e4 & 15;
    const float* src = &sT[b][rr][cc];
    *reinterpret_cast<float4*>(out + 4 * f) = make_float4(src[0], src[1], src[2], src[3]);
  }
}

}  // namespace

int64_t chunk_slots(int64_t Ttot, int n_seqs) { return (Ttot + 63) / 64 + n_seqs; }

hipError_t launch_chunk_prep(const ChunkArgs& a, hipStream_t stream) {
  const int64_t slots = chunk_slots(a.Ttot, a.n_seqs);
  if (slots == 0 || a.Hv == 0) return hipSuccess;
  hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)slots, a.Hv), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
