// chunk_bf16.hip -- serial chunk scan of the gated delta rule on gfx950 MFMA.
//
// One workgroup (NW waves) owns one (sequence or segment, q/k head, 32 NW
// state columns) and walks its 64-token chunks in order.  Its columns are
// taken from the v-heads that read that q/k head (two v-heads of 128 columns
// for NW = 8 and V = 128), so the chunk's q and k are staged once for all of
// them.  Wave w holds the K x 32 fp32 state of its 32 columns in registers,
// as sixteen 16 x 16 accumulator tiles.  What about a chunk does not depend on
// the state -- T diag(beta) (T = (I + A)^{-1}, the UT transform), the
// in-chunk cumulative gate G and the decays -- comes precomputed from the
// prep kernel (chunk_prep.hip).  Per chunk (local tokens r, s), each wave
// then does, for its own columns and without any further synchronisation:
//   R  = V - diag(e^G) K S
//   U  = T diag(beta) R                           (= U0 - W S)
//   S <- e^{G_last} S + K^T diag(e^{G_last - G}) U
//   O^T = diag(e^G) S^T Q^T + U^T P^T,  P = lower(Q K^T . e^{G_r - G_s})
// which is the token recurrence regrouped by chunk.  The masked Q K^T is
// formed by each wave from the q and k in LDS (its accumulator tiles are the
// B operand of U^T P^T as they stand).  O comes out transposed, a lane holding
// four consecutive columns of one token, and goes to global memory from the
// registers (16-byte stores), after the next chunk's first barrier.
//
// Operand order.  A pair of vertically adjacent accumulator tiles is an MFMA
// operand whose k index runs in the slot order of device_common.h
// (slot_row / row_slot).  The state's rows are kept permuted so that this
// order is the natural one on the q/k side: accumulator row p of the state
// holds key index row_slot(p), so the products against S read q and k as
// plain 16-byte runs of a token's row.  Tokens, where they are the k index
// (T diag(beta) R, U^T P^T, K^T U), run in the slot order on both sides: the
// prep record stores T diag(beta)'s columns that way, and the K^T tile its
// tokens.
//
// Precision: every fp32 quantity that meets the matrix cores is a bf16 pair
// hi + lo (~16 significant bits), multiplied against exact bf16 data (q, k)
// or against another pair (hi*hi + hi*lo + lo*hi): S against K and Q, T diag(beta)
// against R, U against P, the decayed U against K.
//
// LDS (bf16 unless noted): sQ, sK [64][136] (token rows), sKt [128][72] (row
// p: key index row_slot(p), tokens in slot order), sV [64][32 NW + 8] (v of
// the workgroup's columns), every row padded by 16 bytes, and
// two buffers of the prep records of the workgroup's v-heads, filled by direct
// global-to-LDS loads one chunk ahead.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CH = 64;
constexpr int KD = 128;
// Row pitches (bf16 elements): every row is padded by 16 bytes, so the 16
// rows of a fragment read (one 16-byte unit each, at the same unit index)
// start four banks apart and fall on distinct banks of the 64, and every
// fragment of a tile is one base address plus an immediate offset.
constexpr int QP = KD + 8;   // q, k: 128 key indices per token row
constexpr int KTP = CH + 8;  // K^T: 64 tokens per row
// Parts of a prep record (kernels.h): T diag(beta) hi and lo (the first
// TB_BYTES) and the gates G, gamma, dec (the last GX_BYTES).
constexpr int TB_BYTES = REC_G;
constexpr int GX_BYTES = PREP_RECORD_BYTES - REC_G;
static_assert(TB_BYTES % 1024 == 0 && GX_BYTES % 16 == 0 && REC_G == 12 * 1024, "record parts");

enum { kOutF32 = 0, kOutBF16 = 1, kPass1 = 2 };

template <int NW>
struct Lds {
  static constexpr int NH = NW == 8 ? 2 : 1;  // v-heads a workgroup's columns can span
  static constexpr int Q = 0;
  static constexpr int K = Q + CH * QP * 2;
  static constexpr int KT = K + CH * QP * 2;
  static constexpr int VP = 32 * NW + 8;  // v: the workgroup's 32 NW columns per token row
  static constexpr int VT = KT + KD * KTP * 2;
  // P^T operand fragments per v-head: 6 (m, tt) blocks, hi and lo, 1 KB each
  static constexpr int PF = VT + CH * VP * 2;
  static constexpr int NRM = PF + NH * 12 * 1024;  // gated norm: per-wave row sums, [2][NW][64] fp32
  static constexpr int TB = NRM + 2 * NW * 64 * 4;   // T diag(beta) of the v-heads: one buffer
  static constexpr int GX = TB + NH * TB_BYTES;      // G, gamma, dec of the v-heads: two buffers
  static constexpr int BYTES = GX + 2 * NH * GX_BYTES;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
  static_assert(TB % 1024 == 0 && GX % 16 == 0, "record buffers aligned for direct loads");
};

// Workgroups go to the eight XCDs in turn by id, each XCD with its own L2.
// The grid is 1-D over logical blocks (workgroup of a q/k head fastest, then
// q/k head, then sequence); a group of `group` consecutive logical blocks
// reads the same q/k.  When the groups split evenly over the XCDs, physical
// id L runs member (L / 8) % group of group (L % 8) + 8 (L / 8 / group), so
// every member of a group has the same L % 8 (one XCD, one L2 copy of its
// inputs) and groups still start in logical order, eight at a time.
__device__ __forceinline__ int xcd_grouped(int L, int n, int group) {
  const int groups = n / group;
  if (n % group != 0 || groups % 8 != 0) return L;
  const int x = L & 7, j = L >> 3;
  return (x + 8 * (j / group)) * group + j % group;
}

__device__ __forceinline__ void zero4(f32x4& x) { x[0] = x[1] = x[2] = x[3] = 0.f; }

// Keeps the instruction scheduler from moving work across this point: bounds
// how far LDS fragment loads are hoisted ahead of their MFMAs (and with them
// the registers in flight) to one short group of products.
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// The thread index as a value the compiler cannot see through: lane-derived
// addresses computed from it inside the chunk loop stay there (a few cheap
// integer operations per phase) instead of being hoisted out of the loop and
// held in registers across it.
__device__ __forceinline__ int fresh_id(int x) {
  asm volatile("" : "=v"(x) : "0"(x));
  return x;
}
#define LANE_IDS()                                                        \
  const int tid = fresh_id(tid0);                                         \
  const int lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;             \
  (void)lane, (void)g4, (void)c16

// Workgroup barrier that orders LDS accesses only: waits for this wave's LDS
// operations, not for its global loads and stores in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 16-byte unit of a token row of q or k: key indices 8 unit .. + 7.
__device__ __forceinline__ bf16x8 frag_row128(const uint16_t* tile, int row, int unit) {
  return *reinterpret_cast<const bf16x8*>(tile + row * QP + 8 * unit);
}
// 16-byte unit of a K^T row: operand slots 8 unit .. + 7.  The units of a
// row are swizzled by its 32-row block (u -> u ^ (row / 32)), which is uniform
// over a fragment read and keeps the stash's transposed stores, whose 16
// lanes write rows 32 apart in groups of four, on distinct banks.
__device__ __forceinline__ int kt_pos(int row, int slot) {
  return ((((slot >> 3) ^ (row >> 5)) & 7) << 3) | (slot & 7);
}
__device__ __forceinline__ bf16x8 frag_kt(const uint16_t* tile, int row, int unit) {
  return *reinterpret_cast<const bf16x8*>(tile + row * KTP + 8 * (unit ^ (row >> 5)));
}

// Columns of wave w of workgroup wgi of q/k head hq: its v-head, its first
// column, and (segment pass 1) whether they are M columns (state started at
// the identity, no values) or b columns.  In pass 1 a v-head contributes
// K + V columns, [M | b]; otherwise V.
struct WaveCols {
  int head, col;
  bool m;
};
template <bool kP1, int NW>
__device__ __forceinline__ WaveCols wave_cols(int w, int wgi, int hq, int G, int V) {
  const int gc = wgi * 32 * NW + 32 * w;
  const int per = kP1 ? KD + V : V;
  WaveCols r;
  r.head = hq * G + gc / per;
  const int within = gc % per;
  r.m = kP1 && within < KD;
  r.col = (kP1 && !r.m) ? within - KD : within;
  return r;
}

template <int kMode, int NW, bool kNorm>
__global__ void __launch_bounds__(NW * 64) chunk_scan_kernel(ChunkArgs a, float* m_out) {
  using LD = Lds<NW>;
  constexpr int NT = NW * 64;
  constexpr bool kP1 = kMode == kPass1;
  constexpr bool kOut = !kP1;
  constexpr int NPAIR = 512 / NT;  // (row pair, 8 key indices) units of q and of k per thread
  static_assert(NPAIR * NT == 512, "thread layout");
  static_assert(!kNorm || kOut, "the norm applies to outputs");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + LD::Q);
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + LD::K);
  uint16_t* sKt = reinterpret_cast<uint16_t*>(smem + LD::KT);
  uint16_t* sV = reinterpret_cast<uint16_t*>(smem + LD::VT);
  unsigned char* sPf = smem + LD::PF;
  float* sNrm = reinterpret_cast<float*>(smem + LD::NRM);
  unsigned char* sTb = smem + LD::TB;
  unsigned char* sGx = smem + LD::GX;

  const int tid0 = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);  // uniform: scalar registers

  const int G = a.Hv / a.Hqk;
  const int wpg = a.n_tiles;  // workgroups per (sequence, q/k head)
  const int lb = xcd_grouped((int)blockIdx.x, (int)gridDim.x, wpg);
  const int wgi = lb % wpg;
  const int hq = (lb / wpg) % a.Hqk;
  const int zb = lb / (wpg * a.Hqk);
  const int seq = a.seq_order ? a.seq_order[zb] : zb;
  int64_t bos, eos;
  if (a.cu) {
    bos = clampi(a.cu[seq], 0, a.Ttot);
    eos = clampi(a.cu[seq + 1], bos, a.Ttot);
  } else {
    bos = (int64_t)seq * a.row_len;
    eos = bos + a.row_len;
  }
  const WaveCols me = wave_cols<kP1, NW>(wave, wgi, hq, G, a.V);
  const int head0 = wave_cols<kP1, NW>(0, wgi, hq, G, a.V).head;
  const int nh = wave_cols<kP1, NW>(NW - 1, wgi, hq, G, a.V).head - head0 + 1;
  const int h = me.head;
  const int hslot = h - head0;

  // start state of this wave's columns: identity (M columns), zero, or rows of V
  const float* s0p = nullptr;
  if (!me.m) {
    if (a.s0_ref) {
      const int r = a.s0_ref[seq];
      if (r >= 0)
        s0p = a.s0_seg + ((int64_t)r * a.Hv + h) * (int64_t)KD * a.V;
      else if (r <= -2 && a.s0)
        s0p = a.s0 + ((int64_t)(-2 - r) * a.Hv + h) * (int64_t)KD * a.V;
    } else if (a.s0_mode == 1) {
      s0p = a.s0 + ((int64_t)seq * a.Hv + h) * (int64_t)KD * a.V;
    }
  }

  // ---- state: S[ct][pt][e] = S[row_slot(16 pt + 4 g4 + e)][col + 16 ct + c16]
  f32x4 S[2][8];
  {
  LANE_IDS();
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int pt = 0; pt < 8; ++pt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = row_slot(16 * pt + 4 * g4 + e);
        const int col = me.col + 16 * ct + c16;
        float s = 0.f;
        if (me.m)
          s = (d == col) ? 1.f : 0.f;
        else if (s0p)
          s = s0p[(int64_t)d * a.V + col];
        S[ct][pt][e] = s;
      }
  }

  // ---- prefetch of q, k and v into registers ---------------------------------
  // q/k unit u = tid + NT j covers token rows 2 (u >> 4) + {0, 1} and key
  // indices 8 (u & 15) .. + 7: 16 consecutive lanes read one token's 256
  // contiguous bytes, and a lane holds two adjacent tokens, which the K^T
  // stash packs into 4-byte words.  v unit u = tid + NT j (j = 0..3) covers
  // token row u / (4 NW) and the workgroup's columns 8 (u % (4 NW)) .. + 7.
  // Every load is unconditional: rows past the end of the sequence re-read its
  // last row (k and q are zeroed when stashed; v there meets zero columns of
  // T diag(beta)); M columns have no values and re-read k.  A load's address is a uniform base at the
  // chunk's first token plus a lane's 32-bit byte offset row * stride + column
  // (strides stay below 2^24 elements, so row * stride is one 24-bit multiply).
  const char* kbase = (const char*)((const uint16_t*)a.k + bos * a.k_stride + hq * KD);
  const char* qbase = kOut ? (const char*)((const uint16_t*)a.q + bos * a.q_stride + hq * KD) : kbase;
  const int64_t q_stride = kOut ? a.q_stride : a.k_stride;
  const uint32_t ks32 = (uint32_t)a.k_stride, qs32 = (uint32_t)q_stride;
  const char* vbase = (const char*)((const uint16_t*)a.v + bos * a.v_stride);
  const uint32_t vs32 = (uint32_t)a.v_stride;
  constexpr int NVU = 4 * NW;  // 16-byte v units per token row of the workgroup
  static_assert(NT % NVU == 0, "a thread's v units share their columns");
  // element offset of the columns of this thread's v units inside a token row
  // (every unit tid + NT j has the same columns), or -1 for M columns (no values)
  const int v_col = [&]() -> int {
    const int cg = tid0 % NVU;  // 8-column group of the workgroup
    const WaveCols wc = wave_cols<kP1, NW>(cg >> 2, wgi, hq, G, a.V);
    return wc.m ? -1 : wc.head * a.V + wc.col + 8 * (cg & 3);
  }();

  // The next chunk's loads are issued one at a time between the compute
  // phases (pf_kq: index 4 j + 2 which + row, which 0 = k, 1 = q; pf_v: index
  // 2 j + row), so that the vector memory path works through them in the
  // background instead of in one burst that stalls the issuing waves.
  u32x4 pk[NPAIR][2], pq[NPAIR][2], pv[4];
  auto pf_row = [&](int64_t T0, int r0, int row) -> uint32_t {
    const int L_ = (int)((eos - T0) < CH ? (eos - T0) : CH);
    const int r = r0 + row;
    return (uint32_t)(r < L_ ? r : L_ - 1);
  };
  // one 16-byte load at uniform base B (chunk start) + lane byte offset
  auto ld16 = [](const char* B, uint32_t row, uint32_t s32, uint32_t col) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(B + (uint32_t)(2u * (__umul24(row, s32) + col)));
  };
  auto pf_kq = [&](int64_t T0, int idx) {
    LANE_IDS();
    const int jj = idx >> 2, which = (idx >> 1) & 1, row = idx & 1;
    const int u = tid + NT * jj;
    const uint32_t d = (uint32_t)((u & 15) * 8);
    const uint32_t r = pf_row(T0, 2 * (u >> 4), row);
    if (which == 0)
      pk[jj][row] = ld16(kbase + 2 * (T0 - bos) * a.k_stride, r, ks32, d);
    else if (kOut)
      pq[jj][row] = ld16(qbase + 2 * (T0 - bos) * q_stride, r, qs32, d);
  };
  auto pf_v = [&](int64_t T0, int idx) {
    LANE_IDS();
    const int u = tid + NT * idx;
    const uint32_t r = pf_row(T0, u / NVU, 0);
    const int vc = v_col;
    if (vc < 0)
      pv[idx] = ld16(kbase + 2 * (T0 - bos) * a.k_stride, r, ks32, 0u);
    else
      pv[idx] = ld16(vbase + 2 * (T0 - bos) * a.v_stride, r, vs32, (uint32_t)vc);
  };

  // ---- prep records of the workgroup's v-heads: direct global-to-LDS loads ----
  // The records of v-heads head0 .. head0 + nh - 1 of one chunk slot are
  // adjacent in the workspace; wave w's i-th load fills 1 KB of the buffer at
  // (i NW + w) KB, lane l its 16 bytes at l * 16.
  // The records of v-heads head0 .. head0 + nh - 1 of one chunk slot are
  // adjacent in the workspace.  T diag(beta) goes to its single buffer after
  // the barrier that follows its last use in the chunk before, the gates to
  // their double buffer one chunk ahead; wave w's i-th load of a part fills
  // 1 KB at (i NW + w) KB, lane l its 16 bytes at l * 16.
  const unsigned char* recg = (const unsigned char*)a.tbuf + (int64_t)head0 * PREP_RECORD_BYTES;
  const int64_t rslot_stride = (int64_t)a.Hv * PREP_RECORD_BYTES;
  constexpr int kTbRounds = (LD::NH * TB_BYTES / 16 + NT - 1) / NT;
  auto load_tb = [&](int64_t slot, int i) {
    LANE_IDS();
    const int blk = i * NW + wave;  // 1 KB blocks: 12 per v-head
    const int u = blk * 64 + lane;
    if (blk < nh * (TB_BYTES / 1024))
      __builtin_amdgcn_global_load_lds(
          (const void*)(recg + slot * rslot_stride + (blk / 12) * PREP_RECORD_BYTES + 16 * (u - (blk / 12) * 768)),
          (__attribute__((address_space(3))) void*)(sTb + blk * 1024), 16, 0, 0);
  };
  auto load_gx = [&](int64_t slot, int buf) {
    LANE_IDS();
    const int u = wave * 64 + lane;  // 48 units per v-head
    if (wave * 64 < nh * (GX_BYTES / 16) && u < nh * (GX_BYTES / 16))
      __builtin_amdgcn_global_load_lds(
          (const void*)(recg + slot * rslot_stride + (u / 48) * PREP_RECORD_BYTES + REC_G + 16 * (u % 48)),
          (__attribute__((address_space(3))) void*)(sGx + buf * (LD::NH * GX_BYTES) + wave * 1024), 16, 0, 0);
  };

  const int64_t slot0 = (bos >> 6) + seq;  // chunk j of this sequence: slot slot0 + j
  if (bos < eos) {
#pragma unroll
    for (int i = 0; i < 4 * NPAIR; ++i) pf_kq(bos, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) pf_v(bos, i);
#pragma unroll
    for (int i = 0; i < kTbRounds; ++i) load_tb(slot0, i);
    load_gx(slot0, 0);
  }

  // O^T of a finished chunk, lane (c16, g4) of tile (ct, tt): token 16 tt + c16,
  // columns col + 16 ct + 4 g4 .. + 3; tokens at or past Lp are not stored.
  // Address: uniform element offset of (chunk start, head, columns) plus a
  // lane's 32-bit offset t * Hv * V + c (Hv * V is below 2^24: it bounds v's
  // token stride).
  f32x4 OT[2][4];
  // With the gated norm (kNorm) the stored value is, per output row (one
  // token of one v-head), y = o / sqrt(mean(o^2) + eps) * nw * silu(z) with
  // the same operations in the same order as gated_norm_kernel over a stored
  // fp32 o: the sum of squares of each run of eight columns is one fma chain
  // (held by lanes g4 = 2x and 2x + 1), and the runs are summed pairwise as an
  // xor butterfly over the run index (partner runs: the other lane pair, the
  // other column tile, then the waves of the head through sNrm).  norm_rows
  // leaves this wave's part for chunk parity `par` in sNrm; store_o combines
  // the parts of the head's waves.
  auto norm_rows = [&](int par) {
    LANE_IDS();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      float s1[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const f32x4 y = OT[ct][tt];
        float c = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) c = fmaf(y[e], y[e], c);
        const float first = __shfl_xor(c, 16, 64);  // the run's first four squares, for odd g4
        float run = first;
#pragma unroll
        for (int e = 0; e < 4; ++e) run = fmaf(y[e], y[e], run);
        const float whole = __shfl_xor(run, 16, 64);
        run = (g4 & 1) ? run : whole;  // both lanes of the pair hold the run's sum
        s1[ct] = run + __shfl_xor(run, 32, 64);
      }
      if (g4 == 0) sNrm[(par * NW + wave) * 64 + 16 * tt + c16] = s1[0] + s1[1];
    }
  };
  auto store_o = [&](int64_t tp, int Lp, int par, int tt) {
    LANE_IDS();
    const int64_t obase = (tp * a.Hv + h) * (int64_t)a.V + me.col;
    const uint32_t tok32 = (uint32_t)(a.Hv * a.V);
    const int w0 = wave - me.col / 32;  // first wave of this v-head
    {
      const int t = 16 * tt + c16;
      float inv = 0.f;
      if (kNorm) {
        const float* pr = sNrm + (par * NW + w0) * 64 + t;
        float ss = (pr[0] + pr[64]) + (pr[128] + pr[192]);
        if (a.V == 256) ss = ss + ((pr[256] + pr[320]) + (pr[384] + pr[448]));
        inv = 1.f / sqrtf(ss / (float)a.V + a.eps);
      }
      if (t < Lp) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const uint32_t lo = __umul24((uint32_t)t, tok32) + (uint32_t)(16 * ct + 4 * g4);
          f32x4 y = OT[ct][tt];  // (the scale is in O already)
          if (kNorm) {
            f32x4 zv, wv;
            if (a.z_dt == 1) {
              const u32x2 zr = *reinterpret_cast<const u32x2*>((const char*)((const uint16_t*)a.z + obase) + 2u * lo);
              zv = f32x4{__uint_as_float(zr[0] << 16), __uint_as_float(zr[0] & 0xFFFF0000u),
                         __uint_as_float(zr[1] << 16), __uint_as_float(zr[1] & 0xFFFF0000u)};
            } else {
              zv = *reinterpret_cast<const f32x4*>((const char*)((const float*)a.z + obase) + 4u * lo);
            }
            if (a.nw)
              wv = *reinterpret_cast<const f32x4*>(a.nw + me.col + 16 * ct + 4 * g4);
            else
              wv = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = y[e] * inv * wv[e] * silu_hw(zv[e]);
          }
          if (kMode == kOutBF16) {
            *reinterpret_cast<u32x2*>((char*)((uint16_t*)a.o + obase) + 2u * lo) =
                u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          } else {
            *reinterpret_cast<f32x4*>((char*)((float*)a.o + obase) + 4u * lo) = y;
          }
        }
      }
    }
  };

  int64_t j = 0;
  for (int64_t t0 = bos; t0 < eos; t0 += CH, ++j) {
    const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);
    const int buf = (int)(j & 1);
    __syncthreads();  // every wave is done with the previous chunk's tiles; this chunk's records are in

    // ---- stash q, k (row-major and transposed) and v -------------------------
    {
    LANE_IDS();
#pragma unroll
    for (int jj = 0; jj < NPAIR; ++jj) {
      const int u = tid + NT * jj;
      const int r0 = 2 * (u >> 4), d = u & 15;
      u32x4 k0 = pk[jj][0], k1 = pk[jj][1], q0 = pq[jj][0], q1 = pq[jj][1];
      if (L < CH) {  // rows past the end of a partial chunk
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (r0 >= L) k0 = q0 = z;
        if (r0 + 1 >= L) k1 = q1 = z;
      }
      *reinterpret_cast<u32x4*>(sK + r0 * QP + 8 * d) = k0;
      *reinterpret_cast<u32x4*>(sK + (r0 + 1) * QP + 8 * d) = k1;
      if (kOut) {
        *reinterpret_cast<u32x4*>(sQ + r0 * QP + 8 * d) = q0;
        *reinterpret_cast<u32x4*>(sQ + (r0 + 1) * QP + 8 * d) = q1;
      }
      // K^T: key index kk goes to row slot_row(kk) (row slot_row(kk) + 1 for
      // kk + 1), tokens r0, r0 + 1 to the adjacent slots row_slot(r0), + 1
      // (one 4-byte word)
      const int ts = row_slot(r0);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int p0 = slot_row(8 * d + 2 * x);
        const uint32_t w0 = __builtin_amdgcn_perm(k1[x], k0[x], 0x05040100u);
        const uint32_t w1 = __builtin_amdgcn_perm(k1[x], k0[x], 0x07060302u);
        const int e = kt_pos(p0, ts);  // the same position in rows p0 and p0 + 1
        *reinterpret_cast<uint32_t*>(sKt + p0 * KTP + e) = w0;
        *reinterpret_cast<uint32_t*>(sKt + (p0 + 1) * KTP + e) = w1;
      }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int u = tid + NT * jj;
      *reinterpret_cast<u32x4*>(sV + (u / NVU) * LD::VP + 8 * (u % NVU)) = pv[jj];
    }
    }
    lds_barrier();  // the chunk's tiles are in LDS
    // The previous chunk's O leaves now, after the barrier that waits for
    // outstanding memory operations, so its stores overlap this chunk's work.
    const bool more = t0 + CH < eos;
    if (kOut && j > 0) {  // the previous chunk's O (only the last chunk can be short)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) store_o(t0 - CH, CH, (int)((j - 1) & 1), tt);
    }
    if (more) load_gx(slot0 + j + 1, buf ^ 1);  // the next chunk's gates (other buffer)
    const unsigned char* gx = sGx + (buf * LD::NH + hslot) * GX_BYTES;
    const float* sG = reinterpret_cast<const float*>(gx);
    const float* sGam = reinterpret_cast<const float*>(gx + (REC_GAM - REC_G));
    const float* sDec = reinterpret_cast<const float*>(gx + (REC_DEC - REC_G));
    if (kOut) {
      LANE_IDS();
      // P^T operand fragments, shared by the waves of a v-head: fragment
      // f = (token block m, t-tile tt) holds the tiles (2 m, tt), (2 m + 1, tt)
      // of scale * P^T, (P^T)[s, t] = (K Q^T)[s, t] e^{G_t - G_s} for s <= t
      // (zero above), split into bf16 hi and lo.  Wave w < 6 forms fragment w
      // (wave w - NW / 2 ... for four waves: fragments w and w + 4) for every
      // v-head of the workgroup; a lane holds s = 16 st + 4 g4 + e, t = 16 tt + c16.
      constexpr int FM[6] = {0, 0, 0, 0, 1, 1};
      constexpr int FT[6] = {0, 1, 2, 3, 2, 3};
      constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
      for (int f0 = 0; f0 < 6; f0 += NW) {
        const int f = f0 + wave;
        if (f < 6) {
          const int m = f < 4 ? 0 : 1, tt = f < 4 ? f : f - 2;
          f32x4 acc[2];
          zero4(acc[0]);
          zero4(acc[1]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const bf16x8 fq = frag_row128(sQ, 16 * tt + c16, 4 * k + g4);
            acc[0] = mfma16(frag_row128(sK, 16 * (2 * m) + c16, 4 * k + g4), fq, acc[0]);
            if (2 * m + 1 <= tt) acc[1] = mfma16(frag_row128(sK, 16 * (2 * m + 1) + c16, 4 * k + g4), fq, acc[1]);
          }
          (void)FM, (void)FT;
          for (int hh = 0; hh < nh; ++hh) {
            const float* gh = reinterpret_cast<const float*>(sGx + (buf * LD::NH + hh) * GX_BYTES);
            const float Gt = gh[16 * tt + c16];
            f32x4 p[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
              const int st = 2 * m + x;
              const f32x4 Gs = *reinterpret_cast<const f32x4*>(gh + 16 * st + 4 * g4);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const bool keep = st <= tt && 16 * st + 4 * g4 + e <= 16 * tt + c16;
                p[x][e] = keep ? acc[x][e] * (a.scale * __builtin_amdgcn_exp2f(fminf(Gt - Gs[e], 0.f) * kLog2e)) : 0.f;
              }
            }
            bf16x8 ph, pl;
            split_frag(p[0], p[1], ph, pl);
            unsigned char* dstf = sPf + hh * (12 * 1024) + f * 2048 + lane * 16;
            *reinterpret_cast<bf16x8*>(dstf) = ph;
            *reinterpret_cast<bf16x8*>(dstf + 1024) = pl;
          }
        }
      }
    }

    const unsigned char* rec = sTb + hslot * TB_BYTES;

    // ---- K S and S^T Q^T over the split state -----------------------------------
    f32x4 KS[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        zero4(KS[ct][rt]);
        zero4(OT[ct][rt]);
      }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      LANE_IDS();
      bf16x8 sh[2], sl[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) split_frag(S[ct][2 * m], S[ct][2 * m + 1], sh[ct], sl[ct]);
      bf16x8 fk[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) fk[rt] = frag_row128(sK, 16 * rt + c16, 4 * m + g4);
#pragma unroll
      for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) KS[ct][rt] = mfma16(fk[rt], part ? sl[ct] : sh[ct], KS[ct][rt]);
      if (kOut) {
        bf16x8 fq[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) fq[tt] = frag_row128(sQ, 16 * tt + c16, 4 * m + g4);
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) OT[ct][tt] = mfma16(part ? sl[ct] : sh[ct], fq[tt], OT[ct][tt]);
      }
      SCHED_FENCE();
    }

    // ---- R = V - gamma . K S, split; U = T diag(beta) R --------------------------
    f32x4 U[2][4];
    {
      LANE_IDS();
      bf16x8 rh[2][2], rl[2][2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        f32x4 R[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const f32x4 gam = *reinterpret_cast<const f32x4*>(sGam + 16 * rt + 4 * g4);
          // v at tokens 16 rt + 4 g4 + e of this lane's column (M columns: none)
          const uint16_t* vp = sV + (16 * rt + 4 * g4) * LD::VP + 32 * wave + 16 * ct + c16;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float ve = me.m ? 0.f : __uint_as_float((uint32_t)vp[e * LD::VP] << 16);
            R[rt][e] = fmaf(-gam[e], KS[ct][rt][e], ve);
          }
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) split_frag(R[2 * m], R[2 * m + 1], rh[ct][m], rl[ct][m]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) zero4(U[ct][rt]);
      }
      constexpr int FRT[6] = {0, 1, 2, 3, 2, 3};
      constexpr int FM[6] = {0, 0, 0, 0, 1, 1};
#pragma unroll
      for (int f0 = 0; f0 < 6; f0 += 3) {
        bf16x8 th[3], tl[3];
#pragma unroll
        for (int f = 0; f < 3; ++f) {
          th[f] = *reinterpret_cast<const bf16x8*>(rec + REC_TB_HI + (f0 + f) * 1024 + lane * 16);
          tl[f] = *reinterpret_cast<const bf16x8*>(rec + REC_TB_LO + (f0 + f) * 1024 + lane * 16);
        }
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
          for (int f = 0; f < 3; ++f)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const int rt = FRT[f0 + f], m = FM[f0 + f];
              U[ct][rt] = mfma16(part == 2 ? tl[f] : th[f], part == 1 ? rl[ct][m] : rh[ct][m], U[ct][rt]);
            }
        SCHED_FENCE();
      }
    }

    // ---- U as the A operand of U^T P^T; dec . U as the B operand of K^T U -------
    bf16x8 uh[2][2], ul[2][2], dh[2][2], dl[2][2];
    {
    LANE_IDS();
    if (kOut) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int m = 0; m < 2; ++m) split_frag(U[ct][2 * m], U[ct][2 * m + 1], uh[ct][m], ul[ct][m]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const f32x4 dec = *reinterpret_cast<const f32x4*>(sDec + 16 * rt + 4 * g4);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) U[ct][rt] *= dec;
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int m = 0; m < 2; ++m) split_frag(U[ct][2 * m], U[ct][2 * m + 1], dh[ct][m], dl[ct][m]);
    }

    // Every wave is done with this chunk's T diag(beta) and (outputs) has its
    // P^T fragments in: the next chunk's T diag(beta) loads now.
    lds_barrier();
    if (more) {
#pragma unroll
      for (int i = 0; i < kTbRounds; ++i) load_tb(slot0 + j + 1, i);
    }

    // ---- S <- e^{G_last} S + K^T (dec . U) ----------------------------------
    {
      LANE_IDS();
      const float glast = sGam[CH - 1];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int pt = 0; pt < 8; ++pt) S[ct][pt] *= glast;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 fkt[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) fkt[x] = frag_kt(sKt, 16 * (4 * half + x) + c16, 4 * m + g4);
#pragma unroll
          for (int part = 0; part < 2; ++part)
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
              for (int ct = 0; ct < 2; ++ct) {
                const int pt = 4 * half + x;
                S[ct][pt] = mfma16(fkt[x], part ? dl[ct][m] : dh[ct][m], S[ct][pt]);
              }
          if (more) pf_v(t0 + CH, 2 * m + half);  // the next chunk's v
          SCHED_FENCE();
        }
    }

    if (more && (kP1 || NPAIR > 1)) {  // the next chunk's q, k not issued in the P^T steps
#pragma unroll
      for (int i = kP1 ? 0 : 4; i < 4 * NPAIR; ++i) pf_kq(t0 + CH, i);
    }
    if (kOut) {
      LANE_IDS();
      // ---- O^T = scale gamma_t . (S^T Q^T) + U^T (scale P^T) -----------------
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float gt = a.scale * sGam[16 * tt + c16];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) OT[ct][tt] *= gt;
      }
      const unsigned char* pf = sPf + hslot * (12 * 1024) + lane * 16;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (more) pf_kq(t0 + CH, tt);  // the next chunk's q, k (NPAIR = 1: four loads)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (2 * m > tt) continue;
          const int f = m == 0 ? tt : tt + 2;
          const bf16x8 ph = *reinterpret_cast<const bf16x8*>(pf + f * 2048);
          const bf16x8 pl = *reinterpret_cast<const bf16x8*>(pf + f * 2048 + 1024);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            OT[ct][tt] = mfma16(uh[ct][m], ph, OT[ct][tt]);
            OT[ct][tt] = mfma16(ul[ct][m], ph, OT[ct][tt]);
            OT[ct][tt] = mfma16(uh[ct][m], pl, OT[ct][tt]);
          }
        }
      }
      if (kNorm) norm_rows(buf);  // read after the next chunk's barriers (or the one below)
    }
  }
  if (kOut && bos < eos) {  // the last chunk's O
    const int64_t t_last = bos + CH * ((eos - bos - 1) / CH);
    if (kNorm) __syncthreads();  // every wave's row sums of the last chunk
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) store_o(t_last, (int)(eos - t_last), (int)((j - 1) & 1), tt);
  }

  // ---- final state ----------------------------------------------------------
  float* dst = nullptr;
  int64_t row_stride = 0;
  const int out_row = a.sf_map ? a.sf_map[seq] : zb;
  if (me.m) {
    dst = m_out + ((int64_t)zb * a.Hv + h) * (int64_t)KD * KD;
    row_stride = KD;
  } else if (a.sf && out_row >= 0) {
    dst = a.sf + (int64_t)out_row * a.sf_seq_stride + (int64_t)h * a.sf_head_stride;
    row_stride = a.sf_row_stride;
  }
  if (dst) {
    LANE_IDS();
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int pt = 0; pt < 8; ++pt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[(int64_t)row_slot(16 * pt + 4 * g4 + e) * row_stride + me.col + 16 * ct + c16] = S[ct][pt][e];
  }
}

// Waves per workgroup: 8 (256 columns) when the q/k head's column space splits
// into 256-column pieces, else 4 (128 columns).
int scan_waves(int cols_per_group) { return cols_per_group % 256 == 0 ? 8 : 4; }

template <int kMode, int NW, bool kNorm>
hipError_t launch_scan_nw(const ChunkArgs& a, float* m_out, int nz, int cols_per_group, hipStream_t stream) {
  const void* fn = (const void*)chunk_scan_kernel<kMode, NW, kNorm>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, Lds<NW>::BYTES);
  if (e != hipSuccess) return e;
  ChunkArgs c = a;
  c.n_tiles = cols_per_group / (32 * NW);
  const int64_t n = (int64_t)nz * a.Hqk * c.n_tiles;
  if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((chunk_scan_kernel<kMode, NW, kNorm>), dim3((unsigned)n), dim3(NW * 64), Lds<NW>::BYTES, stream,
                     c, m_out);
  return hipGetLastError();
}

template <int kMode, bool kNorm = false>
hipError_t launch_scan(const ChunkArgs& a, float* m_out, int nz, hipStream_t stream) {
  const int G = a.Hv / a.Hqk;
  const int cols = G * (kMode == kPass1 ? KD + a.V : a.V);
  return scan_waves(cols) == 8 ? launch_scan_nw<kMode, 8, kNorm>(a, m_out, nz, cols, stream)
                               : launch_scan_nw<kMode, 4, kNorm>(a, m_out, nz, cols, stream);
}

}  // namespace

bool chunk_scan_fuses_norm(int Hqk, int Hv, int V) {
  const int cols_wg = 32 * scan_waves((Hv / Hqk) * V);
  return (V == 128 || V == 256) && V <= cols_wg;
}

int chunk_scan_blocks(int Hqk, int Hv, int V, bool pass1) {
  const int cols = (Hv / Hqk) * (pass1 ? KD + V : V);
  return Hqk * (cols / (32 * scan_waves(cols)));
}

hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t stream, bool prep) {
  if (a.n_seqs == 0 || a.Hv == 0) return hipSuccess;
  if (a.K != KD || a.V % 128 != 0 || a.Hv % a.Hqk != 0 || a.tbuf == nullptr) return hipErrorInvalidValue;
  if (a.Ttot > 0 && (a.o == nullptr || a.q == nullptr)) return hipErrorInvalidValue;
  if (prep) {
    hipError_t e = launch_chunk_prep(a, stream);
    if (e != hipSuccess) return e;
  }
  const int nz = a.seq_order ? a.n_blocks_z : a.n_seqs;
  if (nz == 0) return hipSuccess;
  // (without o, as for calls with no tokens, nothing is stored but the states)
  if (a.z) {
    if (!chunk_scan_fuses_norm(a.Hqk, a.Hv, a.V)) return hipErrorInvalidValue;
    return a.o_dt == 1 ? launch_scan<kOutBF16, true>(a, nullptr, nz, stream)
                       : launch_scan<kOutF32, true>(a, nullptr, nz, stream);
  }
  return a.o_dt == 1 ? launch_scan<kOutBF16>(a, nullptr, nz, stream) : launch_scan<kOutF32>(a, nullptr, nz, stream);
}

hipError_t launch_segment_pass1(const ChunkArgs& a, float* M, float* b, hipStream_t stream, bool prep) {
  if (a.n_seqs == 0 || a.Hv == 0) return hipSuccess;
  if (a.K != KD || a.V % 128 != 0 || a.Hv % a.Hqk != 0 || a.tbuf == nullptr) return hipErrorInvalidValue;
  if (prep) {
    hipError_t e = launch_chunk_prep(a, stream);
    if (e != hipSuccess) return e;
  }
  ChunkArgs c = a;
  c.q = nullptr;
  c.o = nullptr;
  c.sf = b;
  c.sf_seq_stride = (int64_t)a.Hv * KD * a.V;
  c.sf_head_stride = (int64_t)KD * a.V;
  c.sf_row_stride = a.V;
  c.s0_mode = 0;
  c.s0_ref = nullptr;
  c.sf_map = nullptr;
  const int nz = a.seq_order ? a.n_blocks_z : a.n_seqs;
  if (nz == 0) return hipSuccess;
  return launch_scan<kPass1>(c, M, nz, stream);
}

}  // namespace gdn
