// chunk_prep.hip -- everything of a chunk that does not depend on the state.
//
// For a 64-token chunk with local tokens r, s and in-chunk cumulative gate
// G (fp64):
//   A = strictly-lower(diag(beta) K K^T * e^{G_r - G_s}),  T = (I + A)^{-1},
//   P = lower(Q K^T * e^{G_r - G_s}),
//   gamma_r = e^{G_r},  dec_r = e^{G_last - G_r}.
// None of these depends on the recurrent state, so they are computed here for
// every (chunk, v-head) at once, off the serial chunk scan, which then only
// multiplies them against its state.
//
// One wave owns one (chunk slot, v-head): K and Q fragments come straight from
// global memory into the 16 x 16 x 32 bf16 MFMA (exact products, fp32 sums);
// masks are applied in registers; the four 16 x 16 diagonal blocks of T are
// inverted by forward substitution (lane = block, column) and the other
// blocks follow, one block diagonal at a time, from
// T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj on fp32 MFMAs.
//
// Record per (chunk slot, v-head), PREP_RECORD_BYTES long:
//   T diag(beta) hi, lo;  gamma[64], dec[64] (fp32);  P hi, lo
//   (each matrix: 10 lower 16 x 16 bf16 tiles, i >= j, index i(i+1)/2 + j,
//   row-major inside a tile; hi = bf16(x), lo = bf16(x - hi)), so that a
//   state-only scan reads one contiguous prefix.
// (The UT transform's other product, T diag(beta e^G) K S, is formed by the
// scan as T diag(beta) (e^G * K S), so it needs no matrix of its own.)
// Without outputs (state-only runs) the P tiles are not written.
// Chunk slots: chunk j of sequence n (first token cu[n] + 64 j) has slot
// floor((cu[n] + 64 j) / 64) + n, which is unique and below
// ceil(T / 64) + n_seqs; unused slots are skipped.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CH = 64;
constexpr int KD = 128;
constexpr int BP = 17;  // fp32 pitch of a 16 x 16 tile in LDS

__device__ __forceinline__ int64_t seq_begin(const ChunkArgs& a, int n) {
  return a.cu ? (int64_t)clampi(a.cu[n], 0, a.Ttot) : (int64_t)n * a.row_len;
}

__device__ __forceinline__ int blk(int i, int j) { return (i * (i + 1)) / 2 + j; }

// e^x for x = G_r - G_s <= 0 (an fp64 difference, so no cancellation), on the
// hardware exp2: relative error a few 2^-24, far below the bf16 pairs the
// results are stored as.
__device__ __forceinline__ float decay(double x) {
  return __builtin_amdgcn_exp2f((float)x * 1.4426950408889634f);
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// fp32 16 x 16 x 4 MFMA: lane l holds A[l % 16][l / 16], B[l / 16][l % 16];
// D rows 4 (l / 16) + e of column l % 16.
__device__ __forceinline__ f32x4_t mfma_f32_4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void tile_rc(int b, int& i, int& j) {
  i = b >= 6 ? 3 : (b >= 3 ? 2 : (b >= 1 ? 1 : 0));
  j = b - (i * (i + 1)) / 2;
}

__global__ void __launch_bounds__(64) chunk_prep_kernel(ChunkArgs a, int with_p, int heads_per_wave) {
  __shared__ float sA[10][16][BP];
  __shared__ float sT[10][16][BP];  // P staging, then T
  __shared__ float sY[3][16][BP];
  __shared__ double sG[CH];
  __shared__ float sBeta[CH];

  const int lane = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int slot = blockIdx.x;
  const int h0 = blockIdx.y * heads_per_wave;  // v-heads h0 .. h0 + heads_per_wave - 1 share q/k head hq
  const int hq = h0 / (a.Hv / a.Hqk);

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

  // ---- K and Q fragments straight from global memory, in flight first ----------
  // row tile i, k-step m: contiguous k = 32 m + 8 g4 .. +7; rows past L read
  // the last row and are zeroed (every load unconditional)
  const int64_t head_off = (int64_t)hq * KD + 8 * g4;
  bf16x8 kf[4][4], qf[4][4];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * i + c16;
      const int64_t row = t0 + (r < L ? r : L - 1);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const u32x4 v = *reinterpret_cast<const u32x4*>((const uint16_t*)a.k + row * a.k_stride + head_off + 32 * m);
        kf[i][m] = __builtin_bit_cast(bf16x8, r < L ? v : z);
      }
    }
    if (with_p) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * i + c16;
        const int64_t row = t0 + (r < L ? r : L - 1);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32x4 v = *reinterpret_cast<const u32x4*>((const uint16_t*)a.q + row * a.q_stride + head_off + 32 * m);
          qf[i][m] = __builtin_bit_cast(bf16x8, r < L ? v : z);
        }
      }
    }
  }

  for (int hh = 0; hh < heads_per_wave; ++hh) {
  const int h = h0 + hh;
  unsigned char* rec = (unsigned char*)a.tbuf + ((int64_t)slot * a.Hv + h) * PREP_RECORD_BYTES;
  uint16_t* rtb = (uint16_t*)(rec + PREP_REC_TB);  // [2][10][256]
  uint16_t* rp = (uint16_t*)(rec + PREP_REC_P);    // [2][10][256]
  float* rgam = (float*)(rec + PREP_REC_GAM);
  float* rdec = (float*)(rec + PREP_REC_DEC);
  if (hh > 0) __syncthreads();  // the previous head is done with the LDS tiles

  // ---- gates: G (fp64 prefix sum), gamma, dec ---------------------------------
  {
    const bool ok = lane < L;
    double G = ok ? (double)a.g[(t0 + lane) * a.Hv + h] : 0.0;
    const float b = ok ? a.beta[(t0 + lane) * a.Hv + h] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(G, off, 64);
      if (lane >= off) G += o;
    }
    const double Glast = __shfl(G, 63, 64);
    const float gam = expf((float)G);
    sG[lane] = G;
    sBeta[lane] = b;
    rgam[lane] = gam;
    rdec[lane] = expf((float)(Glast - G));
  }

  __syncthreads();  // gates visible to all lanes

  // ---- P = lower(Q K^T * decay) -> record (hi, lo) ----------------------------
  if (with_p) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j <= i; ++j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; ++m) acc = mfma16(qf[i][m], kf[j][m], acc);
        const int s = 16 * j + c16;
        const double Gs = sG[s];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * g4 + e, r = 16 * i + rr;
          sT[blk(i, j)][rr][c16] = (r >= s) ? acc[e] * decay(sG[r] - Gs) : 0.f;
        }
      }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 10; ++u) {
      const int f = lane + 64 * u;  // 4-element group: tile f/64, element 4 (f % 64)
      const int b = f >> 6, e4 = (f & 63) * 4, rr = e4 >> 4, cc = e4 & 15;
      const float* src = &sT[b][rr][cc];
      uint32_t h0, l0, h1, l1;
      split2(src[0], src[1], h0, l0);
      split2(src[2], src[3], h1, l1);
      *reinterpret_cast<u32x2*>(rp + (0 * 10 + b) * 256 + e4) = u32x2{h0, h1};
      *reinterpret_cast<u32x2*>(rp + (1 * 10 + b) * 256 + e4) = u32x2{l0, l1};
    }
    __syncthreads();  // sT is reused for T
  }

  // ---- A = strictly-lower(diag(beta) K K^T * decay) ---------------------------
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
        sA[blk(i, j)][rr][c16] = (r > s) ? sBeta[r] * acc[e] * decay(sG[r] - Gs) : 0.f;
      }
    }
  __syncthreads();

  // ---- T: diagonal blocks, lane = (block b, column c) -------------------------
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

  // ---- T: off-diagonal blocks, T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj -------------
  // Blocks one diagonal at a time (the blocks of a diagonal are independent);
  // each 16 x 16 x 16 product is four fp32 MFMAs with operands read from LDS.
  {
    const int ar = c16, ak = g4;  // A operand: row, k within a 4-step
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
      // Y_ij = sum_k A_ik T_kj for every block of this diagonal, kept in sY
      f32x4_t y[3];
#pragma unroll
      for (int bb = 0; bb < 4 - dist; ++bb) {
        const int i = bb + dist, j = bb;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb = j; kb < i; ++kb) {
          const float(*Aik)[BP] = sA[blk(i, kb)];
          const float(*Tkj)[BP] = sT[blk(kb, j)];
#pragma unroll
          for (int st = 0; st < 4; ++st) acc = mfma_f32_4(Aik[ar][4 * st + ak], Tkj[4 * st + ak][c16], acc);
        }
        y[bb] = acc;
      }
#pragma unroll
      for (int bb = 0; bb < 4 - dist; ++bb)
#pragma unroll
        for (int e = 0; e < 4; ++e) sY[bb][4 * g4 + e][c16] = y[bb][e];
      __syncthreads();
#pragma unroll
      for (int bb = 0; bb < 4 - dist; ++bb) {
        const int i = bb + dist, j = bb;
        const float(*Tii)[BP] = sT[blk(i, i)];
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st) acc = mfma_f32_4(Tii[ar][4 * st + ak], sY[bb][4 * st + ak][c16], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[blk(i, j)][4 * g4 + e][c16] = -acc[e];
      }
      __syncthreads();
    }
  }

  // ---- T diag(beta) as bf16 pairs -> record -----------------------------------
#pragma unroll
  for (int u = 0; u < 10; ++u) {
    const int f = lane + 64 * u;
    const int b = f >> 6, e4 = (f & 63) * 4, rr = e4 >> 4, cc = e4 & 15;
    int bi, bj;
    tile_rc(b, bi, bj);
    const int s = 16 * bj + cc;
    const float* src = &sT[b][rr][cc];
    float tb[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) tb[x] = src[x] * sBeta[s + x];
    uint32_t uh0, ul0, uh1, ul1;
    split2(tb[0], tb[1], uh0, ul0);
    split2(tb[2], tb[3], uh1, ul1);
    *reinterpret_cast<u32x2*>(rtb + (0 * 10 + b) * 256 + e4) = u32x2{uh0, uh1};
    *reinterpret_cast<u32x2*>(rtb + (1 * 10 + b) * 256 + e4) = u32x2{ul0, ul1};
  }
  }  // v-heads of this q/k head
}

}  // namespace

int64_t chunk_slots(int64_t Ttot, int n_seqs) { return (Ttot + 63) / 64 + n_seqs; }

hipError_t launch_chunk_prep(const ChunkArgs& a, int with_p, hipStream_t stream) {
  const int64_t slots = chunk_slots(a.Ttot, a.n_seqs);
  if (slots == 0 || a.Hv == 0) return hipSuccess;
  // Two v-heads that read the same q/k head share one wave (one load of the
  // q/k fragments and half the waves); otherwise one v-head per wave.
  const int per = (a.Hv / a.Hqk) % 2 == 0 ? 2 : 1;
  hipLaunchKernelGGL(chunk_prep_kernel, dim3((unsigned)slots, a.Hv / per), dim3(64), 0, stream, a, with_p, per);
  return hipGetLastError();
}

}  // namespace gdn
