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

// Three waves per SIMD (at most 168 registers; the LDS tiles take 9.5 KB):
// the kernel is a chain of dependent steps, hidden by running many waves.
// kP: also P (forward runs); a template parameter so that the loads of the
// two kinds of run need no merged wait counts.
template <bool kP>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3)))
chunk_prep_kernel(ChunkArgs a, PlanArg plan, int32_t* __restrict__ plan_dst) {
  // diagonal blocks of A (read by the forward substitution) and of T (written
  // column by column); at the end the same 8 tiles stage T diag(beta)
  __shared__ float sStage[8][16][BP];
  float(*sAd)[16][BP] = sStage;
  float(*sTd)[16][BP] = sStage + 4;
  __shared__ double sG[CH];
  __shared__ float sBeta[CH];

  const int lane = threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  // Index arrays of the scans that follow, carried in the launch's arguments
  // (see launch_plan_store): stored by workgroup 0, so they need no launch of
  // their own.
  if (blockIdx.x == 0)
    for (int i = lane; i < plan.n; i += 64) plan_dst[i] = plan.v[i];
  // 1-D grid.  Workgroup ids go to the eight XCDs in turn, so ids x and x + 8
  // share an XCD (and its L2): with an even GQA ratio they are the two v-heads
  // of one q/k head in one chunk slot, and the second reads K and Q from L2.
  int slot, h;
  {
    const int x = blockIdx.x;
    if ((a.Hv / a.Hqk) % 2 == 0) {
      const int pair = (x >> 4) * 8 + (x & 7), member = (x >> 3) & 1;
      const int pairs_per_slot = a.Hv / 2;
      slot = pair / pairs_per_slot;
      h = 2 * (pair % pairs_per_slot) + member;
    } else {
      slot = x / a.Hv;
      h = x % a.Hv;
    }
  }
  const int hq = h / (a.Hv / a.Hqk);

  // sequence n owning this slot: the largest n with floor(cu[n]/64) + n <= slot
  // (the keys grow with n).  Up to 64 sequences: every lane tests one key,
  // one load round trip; more: binary search.
  int n;
  if (a.n_seqs <= 64) {
    const int li = lane < a.n_seqs ? lane : 0;
    const bool below = lane < a.n_seqs && (seq_begin(a, li) >> 6) + li <= slot;
    const uint64_t m = __ballot(below);
    n = m ? 63 - __builtin_clzll(m) : 0;
  } else {
    int lo = 0, hi = a.n_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((seq_begin(a, mid) >> 6) + mid <= slot)
        lo = mid;
      else
        hi = mid - 1;
    }
    n = lo;
  }
  const int64_t bos = seq_begin(a, n);
  const int64_t eos = a.cu ? (int64_t)clampi(a.cu[n + 1], bos, a.Ttot) : bos + a.row_len;
  const int64_t j0 = (int64_t)slot - ((bos >> 6) + n);
  if (j0 < 0) return;
  const int64_t t0 = bos + 64 * j0;
  if (t0 >= eos) return;  // unused slot
  const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);

  // ---- the gates, then K and Q fragments straight from global memory ----------
  // The gates go first: loads complete in order, so the gate scan below waits
  // only for them while the fragments are still on their way.  Row tile i,
  // k-step m: contiguous k = 32 m + 8 g4 .. +7.  Rows past L re-read the
  // chunk's last row (every load unconditional) and are left as they are:
  // their beta is zero, so their rows of A vanish, and no row inside the
  // chunk reaches them through the lower triangles of A and P, so T and P
  // rows before L never see them (the rows past L of T and P are never used
  // for a stored output).
  const int64_t head_off = (int64_t)hq * KD + 8 * g4;
  bf16x8 kf[4][4], qf[4][4];
  float graw, braw;
  {
    const bool ok = lane < L;
    const int64_t grow = t0 + (ok ? lane : 0);
    graw = a.g[grow * a.Hv + h];
    braw = a.beta[grow * a.Hv + h];
    if (!ok) graw = braw = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * i + c16;
      const int64_t row = t0 + (r < L ? r : L - 1);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        kf[i][m] = *reinterpret_cast<const bf16x8*>((const uint16_t*)a.k + row * a.k_stride + head_off + 32 * m);
    }
    if (kP) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * i + c16;
        const int64_t row = t0 + (r < L ? r : L - 1);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          qf[i][m] = *reinterpret_cast<const bf16x8*>((const uint16_t*)a.q + row * a.q_stride + head_off + 32 * m);
      }
    }
  }

  unsigned char* rec = (unsigned char*)a.tbuf + ((int64_t)slot * a.Hv + h) * PREP_RECORD_BYTES;
  uint16_t* rtb = (uint16_t*)(rec + PREP_REC_TB);  // [2][10][256]
  uint16_t* rp = (uint16_t*)(rec + PREP_REC_P);    // [2][10][256]

  // ---- gates: G (fp64 prefix sum), gamma, dec ---------------------------------
  {
    double G = (double)graw;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(G, off, 64);
      if (lane >= off) G += o;
    }
    const double Glast = __shfl(G, 63, 64);
    sG[lane] = G;
    sBeta[lane] = braw;
    reinterpret_cast<float*>(rec + PREP_REC_GAM)[lane] = expf((float)G);
    reinterpret_cast<float*>(rec + PREP_REC_DEC)[lane] = expf((float)(Glast - G));
  }
  __syncthreads();  // gates visible to all lanes

  // ---- A and P tiles, transposed: lane (g4, c16) holds (row c16 of tile i,
  // columns 4 g4 .. 4 g4 + 3 of tile j) of
  //   A = strictly-lower(diag(beta) K K^T * decay)  (kept for T), and
  //   P = lower(Q K^T * decay)                      (4 consecutive values of a
  //                                                  row: one 8-byte store each)
  // one decay per element serves both.
  f32x4 AT[10];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = 16 * i + c16;
    const double GR = sG[R];
    const float bR = sBeta[R];
#pragma unroll
    for (int j = 0; j <= i; ++j) {
      f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) accA = mfma16(kf[j][m], kf[i][m], accA);
      if (kP) {
#pragma unroll
        for (int m = 0; m < 4; ++m) accP = mfma16(kf[j][m], qf[i][m], accP);
      }
      f32x4 av, pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int S = 16 * j + 4 * g4 + e;
        const float d = (R >= S) ? decay(GR - sG[S]) : 0.f;
        av[e] = (R > S) ? bR * accA[e] * d : 0.f;
        pv[e] = accP[e] * d;
      }
      const int b = blk(i, j);
      AT[b] = av;
      if (i == j) *reinterpret_cast<f32x4*>(&sAd[i][c16][4 * g4]) = av;
      if (kP) {
        uint32_t h0, l0, h1, l1;
        split2(pv[0], pv[1], h0, l0);
        split2(pv[2], pv[3], h1, l1);
        *reinterpret_cast<u32x2*>(rp + (0 * 10 + b) * 256 + c16 * 16 + 4 * g4) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(rp + (1 * 10 + b) * 256 + c16 * 16 + 4 * g4) = u32x2{l0, l1};
      }
    }
  }
  __syncthreads();  // diagonal blocks of A visible

  // ---- T: diagonal blocks, lane = (block b, column c) -------------------------
  {
    const int b = g4, c = c16;
    const float(*Ab)[BP] = sAd[b];
    // column c of the block's inverse: x[r] = e_c[r] - sum_{s<r} A[r][s] x[s],
    // the sums taken in order of s; once x[s] is final it updates every later
    // row, so the rows' chains run side by side
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
#pragma unroll
    for (int s = 0; s < 15; ++s)
#pragma unroll
      for (int r = s + 1; r < 16; ++r) x[r] = fmaf(-Ab[r][s], x[s], x[r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) sTd[b][r][c] = x[r];
  }
  __syncthreads();

  // ---- T: off-diagonal blocks in registers, T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  // fp32 16 x 16 x 4 MFMAs with the k index of step st at 4 g4 + st: the A
  // operand is then a transposed tile (A_ik as held above, T_ii read so), the
  // B operand a tile in the MFMA output layout (T_kj, the partial sums Y).
  f32x4 T[10], TTd[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) T[blk(b, b)][e] = sTd[b][4 * g4 + e][c16];
    TTd[b] = *reinterpret_cast<const f32x4*>(&sTd[b][c16][4 * g4]);
  }
#pragma unroll
  for (int dist = 1; dist < 4; ++dist) {
#pragma unroll
    for (int j = 0; j + dist < 4; ++j) {
      const int i = j + dist;
      f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = j; k < i; ++k)
#pragma unroll
        for (int st = 0; st < 4; ++st) y = mfma_f32_4(AT[blk(i, k)][st], T[blk(k, j)][st], y);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) acc = mfma_f32_4(TTd[i][st], y[st], acc);
      T[blk(i, j)] = f32x4{-acc[0], -acc[1], -acc[2], -acc[3]};
    }
  }

  // ---- T diag(beta) as bf16 pairs -> record, staged through LDS (eight tiles
  // at a time) so that a lane stores four consecutive values of a row
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    constexpr int kStage = 8;
    const int b0 = kStage * round, nb = round == 0 ? kStage : 10 - kStage;
    __syncthreads();  // the stage's previous contents are read
#pragma unroll
    for (int bb = 0; bb < kStage; ++bb)
      if (bb < nb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sStage[bb][4 * g4 + e][c16] = T[b0 + bb][e];
      }
    __syncthreads();
#pragma unroll
    for (int bb = 0; bb < kStage; ++bb)
      if (bb < nb) {
        const int b = b0 + bb;
        int bi, bj;
        tile_rc(b, bi, bj);
        float tb[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) tb[x] = sStage[bb][c16][4 * g4 + x] * sBeta[16 * bj + 4 * g4 + x];
        uint32_t h0, l0, h1, l1;
        split2(tb[0], tb[1], h0, l0);
        split2(tb[2], tb[3], h1, l1);
        *reinterpret_cast<u32x2*>(rtb + (0 * 10 + b) * 256 + c16 * 16 + 4 * g4) = u32x2{h0, h1};
        *reinterpret_cast<u32x2*>(rtb + (1 * 10 + b) * 256 + c16 * 16 + 4 * g4) = u32x2{l0, l1};
      }
  }
}

}  // namespace

int64_t chunk_slots(int64_t Ttot, int n_seqs) { return (Ttot + 63) / 64 + n_seqs; }

hipError_t launch_chunk_prep(const ChunkArgs& a, int with_p, hipStream_t stream, const int32_t* ints,
                             int64_t n_ints, int32_t* ints_dst) {
  const int64_t slots = chunk_slots(a.Ttot, a.n_seqs);
  if (slots == 0 || a.Hv == 0) return n_ints > 0 ? launch_plan_store(ints, n_ints, ints_dst, stream) : hipSuccess;
  PlanArg plan;
  plan.n = (int)(n_ints < kPlanArgInts ? n_ints : kPlanArgInts);
  for (int i = 0; i < plan.n; ++i) plan.v[i] = ints[i];
  if (n_ints > kPlanArgInts) {  // the rest by plan_store_kernel
    const hipError_t e = launch_plan_store(ints + kPlanArgInts, n_ints - kPlanArgInts, ints_dst + kPlanArgInts,
                                           stream);
    if (e != hipSuccess) return e;
  }
  // one wave per (chunk slot, v-head)
  // pairs of v-heads fill groups of 16 ids: pad the grid to whole groups
  int64_t n = slots * a.Hv;
  if ((a.Hv / a.Hqk) % 2 == 0) n = (n + 15) / 16 * 16;
  if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (with_p)
    hipLaunchKernelGGL(chunk_prep_kernel<true>, dim3((unsigned)n), dim3(64), 0, stream, a, plan, ints_dst);
  else
    hipLaunchKernelGGL(chunk_prep_kernel<false>, dim3((unsigned)n), dim3(64), 0, stream, a, plan, ints_dst);
  return hipGetLastError();
}

}  // namespace gdn
