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

// Sequence owning chunk slot `slot`: the largest n with floor(cu[n]/64) + n
// <= slot (the keys grow with n).  Up to 64 sequences: every lane of the wave
// tests one key, one load round trip; more: binary search.
__device__ __forceinline__ int slot_sequence(const ChunkArgs& a, int slot, int lane) {
  if (a.n_seqs <= 64) {
    const int li = lane < a.n_seqs ? lane : 0;
    const bool below = lane < a.n_seqs && (seq_begin(a, li) >> 6) + li <= slot;
    const uint64_t m = __ballot(below);
    return m ? 63 - __builtin_clzll(m) : 0;
  }
  int lo = 0, hi = a.n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((seq_begin(a, mid) >> 6) + mid <= slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// g and beta of element i (token * Hv + h): read, or formed from the raw gate
// inputs.
__device__ __forceinline__ void load_gates(const ChunkArgs& a, int64_t i, int h, float& g, float& beta) {
  if (a.ga)
    gate_values(a.ga[i], a.gb[i], a.gA_log[h], a.gdt_bias[h], g, beta);
  else {
    g = a.g[i];
    beta = a.beta[i];
  }
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

// Everything of a record once the K and Q fragments (row tile i, k-step m:
// row 16 i + c16, k = 32 m + 8 g4 .. + 7) and this lane's gate values are in
// registers: the gate scan, A and P, T = (I + A)^{-1} and the stores of
// record (slot, h).  sStage [8][16][BP], sG [64] and sBeta [64] are this
// wave's LDS; the workgroup's waves all call it once (it holds barriers).
template <bool kP>
__device__ __forceinline__ void build_record(const ChunkArgs& a, int slot, int h, const bf16x8 (&kf)[4][4],
                                             const bf16x8 (&qf)[4][4], float graw, float braw,
                                             float (*sStage)[16][BP], double* sG, float* sBeta) {
  float(*sAd)[16][BP] = sStage;
  float(*sTd)[16][BP] = sStage + 4;
  const int lane = threadIdx.x & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
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

  const int n = slot_sequence(a, slot, lane);
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
    load_gates(a, grow * a.Hv + h, h, graw, braw);
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

  build_record<kP>(a, slot, h, kf, qf, graw, braw, sStage, sG, sBeta);
}


// ---- the chunk prep with the short convolution in front ------------------------
// One workgroup per (chunk slot, q/k head) with one wave per v-head of that
// q/k head.  The waves first form the chunk's q and k rows together -- the
// depthwise conv over each token and its conv_width - 1 predecessors in its
// sequence (zero before the sequence start), SiLU, then each head row divided
// by sqrt(sum of squares + l2_eps) -- store them as bf16 to the activations
// and into two LDS tiles; each wave forms the v rows of its own head the same
// way (without the norm) and stores them; then each wave takes its K and Q
// fragments from the tiles and builds its head's record as chunk_prep_kernel
// does.  Per value the arithmetic is that of the separate conv (conv1d_kernel
// with fast rounding): the same fused multiply-adds in the same order, the
// same SiLU, the head's sum of squares over the same lanes in the same order
// and the same reciprocal square root, so the activations and everything the
// scans compute from them equal the unfused pipeline's bit for bit.
// LDS: the q and k tiles (bf16 [64][128] each, 16-byte unit u of row r at
// u ^ (r & 15), so that a fragment read's 16 rows hit different banks), then,
// once every wave holds its fragments, the waves' record stages over them.
constexpr int kQKTileBytes = CH * KD * 2;
constexpr int kWaveStageBytes = 8 * 16 * BP * 4 + CH * 8 + CH * 4;  // sStage, sG, sBeta
constexpr int kConvPrepMaxWaves = 4;

int conv_prep_lds_bytes(int waves) {
  const int stage = waves * kWaveStageBytes;
  return stage > 2 * kQKTileBytes ? stage : 2 * kQKTileBytes;
}

// Taps of channels ch .. ch + 7 aligned so that tap 3 multiplies the current
// token (leading taps zero below width 4), and their bias.
__device__ __forceinline__ void conv_taps(const ChunkArgs& a, int64_t ch, float (&wt)[4][8], float (&bs)[8]) {
  const uint16_t* w = reinterpret_cast<const uint16_t*>(a.cw);
  if (a.conv_width == 4) {  // 8 channels x 4 taps = 64 contiguous bytes
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(w + ch * 4 + 8 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // word e of vector q: channel 2q + e/2, taps 2(e%2), 2(e%2)+1
        const int c = 2 * q + (e >> 1), tap = 2 * (e & 1);
        wt[tap][c] = __uint_as_float(v[e] << 16);
        wt[tap + 1][c] = __uint_as_float(v[e] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = j - (4 - a.conv_width);
        wt[j][i] = src >= 0 ? bf16_bits_to_f32(w[(ch + i) * a.conv_width + src]) : 0.f;
      }
  }
  if (a.cb) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.cb) + ch);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bs[2 * e] = __uint_as_float(v[e] << 16);
      bs[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) bs[i] = 0.f;
  }
}

__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(v[e] << 16);
    f[2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
  }
}

// Channels ch .. ch + 7 of chunk rows r0 .. r0 + 7 (tokens t0 + r): the
// three history rows (zero before the sequence start) and the eight rows
// (rows past the chunk's end re-read its last token), as loaded.
struct ConvRows8 {
  u32x4 hist[3], rows[8];
};

__device__ __forceinline__ void conv_load8(const ChunkArgs& a, int64_t ch, int r0, int64_t t0, int64_t bos,
                                           int64_t eos, ConvRows8& in) {
  const int64_t C = a.q_stride;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.cx);
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int64_t tok = t0 + r0 - 3 + i;
    const int64_t tc = tok < eos ? tok : eos - 1;
    in.hist[i] = *reinterpret_cast<const u32x4*>(x + (tc < bos ? bos : tc) * C + ch);
  }
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int64_t tok = t0 + r0 + rr;
    in.rows[rr] = *reinterpret_cast<const u32x4*>(x + (tok < eos ? tok : eos - 1) * C + ch);
  }
}

// Conv and SiLU of the loaded rows, with kL2 the head-row norm over the 16
// aligned lanes that hold the head's 128 channels; rows below L go to the
// activations, all eight to tile row r at unit `unit` when tile is set.
template <bool kL2>
__device__ __forceinline__ void conv_rows8(const ChunkArgs& a, int64_t ch, int r0, int64_t t0, int64_t bos, int L,
                                           const ConvRows8& in, uint16_t* tile, int unit) {
  const int64_t C = a.q_stride;
  uint16_t* y = reinterpret_cast<uint16_t*>(a.cy);
  float wt[4][8], bs[8];
  conv_taps(a, ch, wt, bs);
  float h1[8], h2[8], h3[8];  // x[t-3], x[t-2], x[t-1] of row r0
  {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    unpack8(t0 + r0 - 3 >= bos ? in.hist[0] : zero, h1);
    unpack8(t0 + r0 - 2 >= bos ? in.hist[1] : zero, h2);
    unpack8(t0 + r0 - 1 >= bos ? in.hist[2] : zero, h3);
  }
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const int r = r0 + rr;
    float cur[8], out[8];
    unpack8(in.rows[rr], cur);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float z = bs[i];
      z = fmaf(wt[0][i], h1[i], z);
      z = fmaf(wt[1][i], h2[i], z);
      z = fmaf(wt[2][i], h3[i], z);
      z = fmaf(wt[3][i], cur[i], z);
      out[i] = silu_conv(z);
      if (kL2) ss = fmaf(out[i], out[i], ss);
      h1[i] = h2[i];
      h2[i] = h3[i];
      h3[i] = cur[i];
    }
    if (kL2) {
      ss = group_sum(ss, 4);
      const float inv = __builtin_amdgcn_rsqf(ss + a.l2_eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] *= inv;
    }
    const u32x4 pk = {pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]), pack_bf16x2(out[4], out[5]),
                      pack_bf16x2(out[6], out[7])};
    if (tile) *reinterpret_cast<u32x4*>(tile + r * KD + 8 * (unit ^ (r & 15))) = pk;
    if (r < L) *reinterpret_cast<u32x4*>(y + (t0 + r) * C + ch) = pk;
  }
}

template <bool kP>
__global__ void __launch_bounds__(64 * kConvPrepMaxWaves) __attribute__((amdgpu_waves_per_eu(2)))
chunk_prep_conv_kernel(ChunkArgs a, PlanArg plan, int32_t* __restrict__ plan_dst) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  if (blockIdx.x == 0)
    for (int i = tid; i < plan.n; i += nthr) plan_dst[i] = plan.v[i];
  const int slot = blockIdx.x / a.Hqk, hq = blockIdx.x % a.Hqk;
  const int h = hq * (a.Hv / a.Hqk) + wave;
  const int n = slot_sequence(a, slot, lane);
  const int64_t bos = seq_begin(a, n);
  const int64_t eos = a.cu ? (int64_t)clampi(a.cu[n + 1], bos, a.Ttot) : bos + a.row_len;
  const int64_t j0 = (int64_t)slot - ((bos >> 6) + n);
  if (j0 < 0) return;
  const int64_t t0 = bos + 64 * j0;
  if (t0 >= eos) return;  // unused slot (the whole workgroup leaves)
  const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);

  // this wave's gates first (see chunk_prep_kernel)
  float graw, braw;
  {
    const bool ok = lane < L;
    const int64_t grow = t0 + (ok ? lane : 0);
    load_gates(a, grow * a.Hv + h, h, graw, braw);
    if (!ok) graw = braw = 0.f;
  }

  // q and k rows of the chunk: 32 groups of 8 channels (16 of q, 16 of k) x 8
  // runs of 8 rows; unit u sits in lane u % 64, so a head row's 16 groups are
  // one aligned 16-lane row of a wave
  // Units are taken two at a time, both units' rows loaded before either is
  // computed, so that each pair costs one memory round trip.
  uint16_t* sQK = reinterpret_cast<uint16_t*>(smem);  // [2][64][128]
  const int64_t qk = (int64_t)a.Hqk * KD;
  auto qk_unit = [&](int u, int64_t& ch, int& r0, int& which, int& gi) {
    const int grp = u & 31;
    which = grp >> 4;  // 0 q, 1 k
    gi = grp & 15;     // group within the head
    ch = which * qk + hq * KD + 8 * gi;
    r0 = 8 * (u >> 5);
  };
  for (int u = tid; u < 256; u += 2 * nthr) {
    const int u2 = u + nthr;  // below 256 for every lane of a wave or for none (nthr is a multiple of 64)
    int64_t ch, ch2;
    int r0, r02, wh, wh2, gi, gi2;
    qk_unit(u, ch, r0, wh, gi);
    qk_unit(u2 < 256 ? u2 : u, ch2, r02, wh2, gi2);
    ConvRows8 in, in2;
    conv_load8(a, ch, r0, t0, bos, eos, in);
    if (u2 < 256) conv_load8(a, ch2, r02, t0, bos, eos, in2);
    conv_rows8<true>(a, ch, r0, t0, bos, L, in, sQK + wh * CH * KD, gi);
    if (u2 < 256) conv_rows8<true>(a, ch2, r02, t0, bos, L, in2, sQK + wh2 * CH * KD, gi2);
  }
  // v rows of this wave's head: V / 8 groups x 8 runs of 8 rows
  {
    const int ng = a.V / 8;
    const int64_t vch = 2 * qk + (int64_t)h * a.V;
    for (int u = lane; u < ng * 8; u += 128) {
      const int u2 = u + 64;  // ng * 8 is a multiple of 128
      ConvRows8 in, in2;
      conv_load8(a, vch + 8 * (u % ng), 8 * (u / ng), t0, bos, eos, in);
      conv_load8(a, vch + 8 * (u2 % ng), 8 * (u2 / ng), t0, bos, eos, in2);
      conv_rows8<false>(a, vch + 8 * (u % ng), 8 * (u / ng), t0, bos, L, in, nullptr, 0);
      conv_rows8<false>(a, vch + 8 * (u2 % ng), 8 * (u2 / ng), t0, bos, L, in2, nullptr, 0);
    }
  }
  __syncthreads();  // the q and k tiles are complete

  // fragments: row tile i, k-step m = 16-byte unit 4 m + g4 of row 16 i + c16
  bf16x8 kf[4][4], qf[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * i + c16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int off = r * KD + 8 * ((4 * m + g4) ^ c16);
      kf[i][m] = *reinterpret_cast<const bf16x8*>(sQK + CH * KD + off);
      if (kP) qf[i][m] = *reinterpret_cast<const bf16x8*>(sQK + off);
    }
  }
  __syncthreads();  // every wave holds its fragments: the tiles become the waves' stages

  unsigned char* st = smem + wave * kWaveStageBytes;
  build_record<kP>(a, slot, h, kf, qf, graw, braw, reinterpret_cast<float(*)[16][BP]>(st),
                   reinterpret_cast<double*>(st + 8 * 16 * BP * 4), reinterpret_cast<float*>(st + 8 * 16 * BP * 4 + CH * 8));
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
  if (a.cx) {
    // conv in front: one workgroup per (chunk slot, q/k head), a wave per v-head
    const int waves = a.Hv / a.Hqk;
    if (waves > kConvPrepMaxWaves || a.K != KD || a.V % 8 != 0 || !a.cy || !a.cw) return hipErrorInvalidValue;
    const int64_t nb = slots * a.Hqk;
    if (nb > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int lds = conv_prep_lds_bytes(waves);
    if (with_p)
      hipLaunchKernelGGL(chunk_prep_conv_kernel<true>, dim3((unsigned)nb), dim3(64 * waves), lds, stream, a, plan,
                         ints_dst);
    else
      hipLaunchKernelGGL(chunk_prep_conv_kernel<false>, dim3((unsigned)nb), dim3(64 * waves), lds, stream, a, plan,
                         ints_dst);
    return hipGetLastError();
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
