// chunk_bf16.hip -- serial chunk scan of the gated delta rule on gfx950 MFMA.
//
// One workgroup (8 waves) owns one (sequence or segment, v-head, 128-column
// slice of V) and walks its 64-token chunks in order.  The K x 128 fp32 state
// never leaves the registers: wave w holds state columns 16 w .. 16 w + 15 as
// eight 16 x 16 accumulator tiles.  Everything about a chunk that does not
// depend on the state -- T diag(beta) (T = (I + A)^{-1}, the UT transform),
// the masked Q K^T, e^G and the decays -- comes precomputed from the prep
// kernel (chunk_prep.hip).  Per chunk (local tokens r, s), each wave then
// does, for its own columns and without any further synchronisation:
//   U  = T diag(beta) (V - diag(e^G) K S)      (= U0 - W S)
//   O  = diag(e^G) Q S + P U
//   S <- e^{G_last} S + K^T diag(e^{G_last - G}) U
// which is the token recurrence regrouped by chunk.  Two barriers per chunk:
// one before the shared tiles are overwritten, one after they are filled.
// The next chunk's q, k, v and prep record are fetched into registers while
// the current chunk computes; O goes through its own LDS tile so that its
// global stores are 16-byte vectors, stored by the first half of the waves
// after the next chunk's first barrier.
//
// Precision: every fp32 quantity that meets the matrix cores is a bf16 pair
// hi + lo (~16 significant bits), multiplied against exact bf16 data (q, k)
// or against another pair (hi*hi + hi*lo + lo*hi): S against K and Q, T diag(beta)
// against V - e^G K S, P against U, the decayed U against K.
//
// LDS (bf16 unless noted).  The tiles read as MFMA operands (Q, K, K^T,
// T diag(beta), P) store each 32-wide block of their K index in fragment
// order (index 16 h + 4 g + j at 8 g + 4 h + j), so the eight values a lane
// feeds one MFMA are contiguous and come in one 16-byte read, and swizzle
// the 16-byte units of a row so that those reads meet no bank conflicts
// (tile_pos, frag16 below):
//   sQ [64][128], sK [64][128], sKt [128][64] (K^T), sP [2][64][64] (hi, lo),
//   sT2 [2][64][64] (T diag(beta) hi/lo); sVt [128][72] (V^T of this slice,
//   rows padded by 16 B), sO fp32 [64][132], gamma[64], dec[64] fp32.
#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CH = 64;
constexpr int KD = 128;
constexpr int BV = 128;

constexpr int QP = KD;      // Q, K: 128 bf16 (256 bytes) per row, no padding
constexpr int TP = CH;      // K^T, T diag(beta), P: 64 bf16 (128 bytes) per row
constexpr int VTP = CH + 8; // V^T (not an MFMA operand): padded rows
constexpr int OP = BV + 4;  // fp32 O tile pitch

constexpr int OFF_Q = 0;
constexpr int OFF_K = OFF_Q + CH * QP * 2;
constexpr int OFF_KT = OFF_K + CH * QP * 2;
constexpr int OFF_VT = OFF_KT + KD * TP * 2;
constexpr int OFF_P = OFF_VT + BV * VTP * 2;
constexpr int OFF_T2 = OFF_P + 2 * CH * TP * 2;
constexpr int OFF_O = OFF_T2 + 2 * CH * TP * 2;
constexpr int OFF_GAM = OFF_O + CH * OP * 4;
constexpr int OFF_DEC = OFF_GAM + CH * 4;
constexpr int LDS_BYTES = OFF_DEC + CH * 4;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

// 16-byte units of a prep record: T diag(beta) hi, lo (2 x 10 tiles x 32),
// gamma and dec (2 x 16), then P hi, lo (2 x 10 x 32).  Forward scans read all
// of it, state-only scans the part before P.
constexpr int REC_TB_UNITS = 2 * 10 * 32;
constexpr int REC_STATE_UNITS = REC_TB_UNITS + 2 * 16;
constexpr int REC_UNITS = REC_STATE_UNITS + 2 * 10 * 32;
static_assert(REC_UNITS * 16 == PREP_RECORD_BYTES, "record layout");
static_assert(REC_TB_UNITS * 16 == PREP_REC_GAM && REC_STATE_UNITS * 16 == PREP_REC_P, "record layout");

// Kernel modes: forward with fp32 o, forward with bf16 o, state only / pass 1.
enum { kOutF32 = 0, kOutBF16 = 1, kPass1 = 2 };

struct Pass1 {
  int m_tiles;   // leading tiles of a (segment, head) that evolve M columns (v = 0, S0 = I)
  float* m_out;  // [n_seqs, Hv, K, K]
  // Mixed launches (forward kernels with kMixed): the first n_fwd segments of
  // the launch run forward (V / 128 blocks per head), the rest form maps
  // (m_tiles + V / 128 blocks per head), M into m_out and b into b_out
  // [n_seqs - n_fwd, Hv, K, V].  The grid holds the forward blocks, then the
  // map blocks, with no idle ones: blocks are dealt to the shader engines in
  // turn, and idle blocks at fixed positions of that order would leave the
  // real ones of some engines more than their compute units.
  int n_fwd;
  float* b_out;
};

// Workgroups go to the eight XCDs in turn by id, each XCD with its own L2.
// The grid is 1-D over logical blocks (tile fastest, then v-head, then
// sequence); a group of `group` consecutive logical blocks reads the same q/k
// (the v-heads of one q/k head with all their tiles) and, within a head, the
// same records.  When the groups split evenly over the XCDs, physical id L
// runs member (L / 8) % group of group (L % 8) + 8 (L / 8 / group), so every
// member of a group has the same L % 8 (one XCD, one L2 copy of its inputs)
// and groups still start in logical order, eight at a time.
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

// tile index (0..9) -> (block row i, block column j) of the lower 4 x 4 tiles
__device__ __forceinline__ void tile_ij(int t, int& i, int& j) {
  i = t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0));
  j = t - (i * (i + 1)) / 2;
}

// Position of K index c inside its 32-wide block in the fragment order
// (c = 16 h + 4 g + j -> 8 g + 4 h + j); groups of four stay together.
__device__ __forceinline__ int frag_pos(int c) {
  return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3);
}

// The LDS serves 64 four-byte banks per cycle.  Operand tiles have unpadded
// rows (16 sixteen-byte units per 256-byte row of Q and K, 8 per 128-byte
// row of K^T, T diag(beta) and P) and store unit u of a row at u ^ swz(row).
// A fragment read puts 16 consecutive rows at one unit: the swizzle sends
// them to 16 different units of the 64 banks, so the read runs without
// conflicts (unit ^ row over 16 rows; for 128-byte rows, two rows share a
// unit index but sit in the two halves of the banks).  The extra flip by
// row bit 4 of Q and K spreads the stash's 32 even rows over 16 units.
__device__ __forceinline__ int swz16(int row) { return (row & 15) ^ ((row >> 4) & 1); }
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

// Element offset of K index c (fragment order, then swizzled) in a row of a
// 128-wide (W16) or 64-wide tile.
template <bool W16>
__device__ __forceinline__ int tile_pos(int row, int c) {
  const int p = frag_pos(c);
  return (((p >> 3) ^ (W16 ? swz16(row) : swz8(row))) << 3) | (p & 7);
}

// A or B fragment of k-step k0 (a multiple of 32) for row `row` of an
// operand tile: one 16-byte read of unit k0 / 8 + g4.
template <bool W16>
__device__ __forceinline__ bf16x8 frag16(const uint16_t* tile, int row, int k0, int g4) {
  constexpr int pitch = W16 ? QP : TP;
  const int u = ((k0 >> 3) + g4) ^ (W16 ? swz16(row) : swz8(row));
  return *reinterpret_cast<const bf16x8*>(tile + row * pitch + 8 * u);
}

// Eight consecutive K indices c .. c + 7 (c a multiple of 8) of row `row`
// of a tile, as two 8-byte stores.
template <bool W16>
__device__ __forceinline__ void store8_frag(uint16_t* tile, int row, int c, const u32x4& v) {
  uint16_t* rb = tile + row * (W16 ? QP : TP);
  *reinterpret_cast<u32x2*>(rb + tile_pos<W16>(row, c)) = u32x2{v[0], v[1]};
  *reinterpret_cast<u32x2*>(rb + tile_pos<W16>(row, c + 4)) = u32x2{v[2], v[3]};
}

template <int kMode, int NW, bool kNorm, bool kMixed>
__global__ void __launch_bounds__(NW * 64) chunk_scan_kernel(ChunkArgs a, Pass1 p1) {
  constexpr int NT = NW * 64;
  constexpr int CPW = BV / NW;     // state columns per wave
  constexpr int NCT = CPW / 16;    // 16-column tiles per wave
  constexpr int NPAIR = 512 / NT;  // (row pair, 8 columns) units per thread per matrix
  constexpr bool kOut = kMode != kPass1;
  constexpr int RUNITS = kOut ? REC_UNITS : REC_STATE_UNITS;  // record units this mode reads
  constexpr int NREC = (RUNITS + NT - 1) / NT;                 // record units per thread
  static_assert(CPW % 16 == 0 && NW * CPW == BV, "wave layout");
  static_assert(!kNorm || kOut, "the norm applies to outputs");
  static_assert(!kMixed || kOut, "mixed launches run forward kernels");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + OFF_Q);
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + OFF_K);
  uint16_t* sKt = reinterpret_cast<uint16_t*>(smem + OFF_KT);
  uint16_t* sVt = reinterpret_cast<uint16_t*>(smem + OFF_VT);
  uint16_t* sP = reinterpret_cast<uint16_t*>(smem + OFF_P);
  uint16_t* sT2 = reinterpret_cast<uint16_t*>(smem + OFF_T2);
  float* sO = reinterpret_cast<float*>(smem + OFF_O);
  float* sGam = reinterpret_cast<float*>(smem + OFF_GAM);
  float* sDec = reinterpret_cast<float*>(smem + OFF_DEC);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  bool m_mode = false;
  int n_tiles = a.n_tiles, zb0 = 0, L = (int)blockIdx.x, n_blocks = (int)gridDim.x;
  if (kMixed) {
    const int nf = p1.n_fwd * a.Hv * (a.V / BV);  // forward blocks first
    if (L < nf) {
      n_tiles = a.V / BV;
      n_blocks = nf;
    } else {
      L -= nf;
      n_blocks -= nf;
      zb0 = p1.n_fwd;
    }
  }
  const int lb = xcd_grouped(L, n_blocks, n_tiles * (a.Hv / a.Hqk));
  int tile = lb % n_tiles;
  const int h = (lb / n_tiles) % a.Hv;
  const int zb = zb0 + lb / (n_tiles * a.Hv);
  // state only: a map block of a mixed launch (from the identity for M
  // columns, zero for b columns), which skips q and O like pass 1
  bool so = false;
  if (kMode == kPass1) {
    m_mode = tile < p1.m_tiles;
    if (!m_mode) tile -= p1.m_tiles;
  }
  if (kMixed && zb >= p1.n_fwd) {
    so = true;
    m_mode = tile < p1.m_tiles;
    if (!m_mode) tile -= p1.m_tiles;
  }
  // q, O and its stores: forward kernels, except on the map blocks of a mixed launch
  const bool outb = kOut && !so;
  const int v0 = tile * BV;
  const int seq = a.seq_order ? a.seq_order[zb] : zb;
  const int hq = h / (a.Hv / a.Hqk);
  int64_t bos, eos;
  if (a.cu) {
    bos = clampi(a.cu[seq], 0, a.Ttot);
    eos = clampi(a.cu[seq + 1], bos, a.Ttot);
  } else {
    bos = (int64_t)seq * a.row_len;
    eos = bos + a.row_len;
  }
  const bool load_v = !m_mode;
  // start state of this head: identity (M columns), zero, or K x V rows of V
  const float* s0p = nullptr;
  if (!m_mode && !so) {
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
  const int col_base = v0 + wave * CPW;

  // Prefetch units: unit u = tid + NT j (j < NPAIR) covers token rows
  // 2 (u & 31) + {0, 1} and columns 8 (u >> 5) .. + 7, so all units of a
  // thread share its two rows.  Lanes run along the tokens so that the
  // transposed LDS stores (K^T, V^T) of a wave hit consecutive banks; the
  // 16-byte global loads of the column groups of a row come from neighbouring
  // waves and meet in the caches.
  const int r0_pf = 2 * (tid & 31), d8_pf = (tid >> 5) * 8;
  constexpr int kDJ = (NT / 32) * 8;  // column step between a thread's units
  // Uniform base pointers at the sequence start.  Per chunk the prefetch moves
  // them to the chunk's first token (scalar arithmetic) and adds a lane's
  // 32-bit byte offset, row * stride + column, with row clamped to the chunk's
  // last valid token; the host keeps strides below 2^24 elements, so the
  // row * stride product is one 24-bit multiply.
  const char* kbase = (const char*)((const uint16_t*)a.k + bos * a.k_stride + hq * KD);
  const char* qbase = outb ? (const char*)((const uint16_t*)a.q + bos * a.q_stride + hq * KD) : kbase;
  const int64_t q_stride = outb ? a.q_stride : a.k_stride;
  // without values (M columns) the v loads re-read k and are discarded
  const char* vbase = load_v ? (const char*)((const uint16_t*)a.v + bos * a.v_stride + (int64_t)h * a.V + v0) : kbase;
  const int64_t v_stride = load_v ? a.v_stride : a.k_stride;
  const uint32_t ks32 = (uint32_t)a.k_stride, qs32 = (uint32_t)q_stride, vs32 = (uint32_t)v_stride;
  const unsigned char* rbase = (const unsigned char*)a.tbuf + (int64_t)h * PREP_RECORD_BYTES;
  const int64_t rslot_stride = (int64_t)a.Hv * PREP_RECORD_BYTES;
  const int rec_seq = a.rec_seq ? a.rec_seq[seq] : seq;

  // ---- initial state: S[ct][dt][e] = S[16 dt + 4 g4 + e][col_base + 16 ct + c16]
  f32x4 S[NCT][8];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 16 * dt + 4 * g4 + e;
        const int col = col_base + 16 * ct + c16;
        float s = 0.f;
        if (m_mode)
          s = (d == col) ? 1.f : 0.f;
        else if (s0p)
          s = s0p[(int64_t)d * a.V + col];
        S[ct][dt][e] = s;
      }

  // Upper tiles of sP and sT2 that the triangular products read must be zero;
  // the record stash only ever writes the lower tiles.
  for (int i = tid; i < (2 + 2) * CH * TP; i += NT) sP[i] = 0;

  // ---- prefetch registers --------------------------------------------------
  // Every prefetch load is unconditional (rows past the end of the sequence
  // re-read its last row and are zeroed when stashed; record units past the
  // end re-read the last unit).  The next chunk's loads are issued in three
  // groups between the compute phases of the current one, so that the
  // vector memory pipeline works through them while the matrix cores run
  // instead of holding up a barrier.
  u32x4 pk[NPAIR][2], pq[NPAIR][2], pv[NPAIR][2], pr[NREC];
#define GDN_PF_ROWS(T0)                                                                        \
  const int64_t rel_ = (T0) - bos;                                                            \
  const int L_ = (int)((eos - (T0)) < CH ? (eos - (T0)) : CH);                                \
  const uint32_t row0_ = (uint32_t)(r0_pf < L_ ? r0_pf : L_ - 1);                             \
  const uint32_t row1_ = (uint32_t)(r0_pf + 1 < L_ ? r0_pf + 1 : L_ - 1);
// one 16-byte load at uniform base B (chunk start) + lane byte offset
#define GDN_LD16(B, ROW, S32, COL) \
  (*reinterpret_cast<const u32x4*>((B) + (uint32_t)(2u * (__umul24((ROW), (S32)) + (uint32_t)(COL)))))
#define GDN_PF_REC(T0)                                                                         \
  do {                                                                                        \
    const unsigned char* rs_ = rbase + (((T0) >> 6) + rec_seq) * rslot_stride;                \
    _Pragma("unroll") for (int u_ = 0; u_ < NREC; ++u_)                                        \
      pr[u_] = *reinterpret_cast<const u32x4*>(rs_ + 16 * min(tid + u_ * NT, RUNITS - 1));      \
  } while (0)
#define GDN_PF_KQ(T0)                                                                          \
  do {                                                                                        \
    GDN_PF_ROWS(T0)                                                                           \
    const char* kc_ = kbase + 2 * rel_ * a.k_stride;                                          \
    const char* qc_ = qbase + 2 * rel_ * q_stride;                                            \
    _Pragma("unroll") for (int j_ = 0; j_ < NPAIR; ++j_) {                                     \
      pk[j_][0] = GDN_LD16(kc_, row0_, ks32, d8_pf + kDJ * j_);                                \
      pk[j_][1] = GDN_LD16(kc_, row1_, ks32, d8_pf + kDJ * j_);                                \
      pq[j_][0] = GDN_LD16(qc_, row0_, qs32, d8_pf + kDJ * j_);                                \
      pq[j_][1] = GDN_LD16(qc_, row1_, qs32, d8_pf + kDJ * j_);                                \
    }                                                                                         \
  } while (0)
#define GDN_PF_V(T0)                                                                           \
  do {                                                                                        \
    GDN_PF_ROWS(T0)                                                                           \
    const char* vc_ = vbase + 2 * rel_ * v_stride;                                            \
    _Pragma("unroll") for (int j_ = 0; j_ < NPAIR; ++j_) {                                     \
      pv[j_][0] = GDN_LD16(vc_, row0_, vs32, d8_pf + kDJ * j_);                                \
      pv[j_][1] = GDN_LD16(vc_, row1_, vs32, d8_pf + kDJ * j_);                                \
    }                                                                                         \
  } while (0)
#define GDN_PREFETCH(T0) do { GDN_PF_REC(T0); GDN_PF_KQ(T0); GDN_PF_V(T0); } while (0)
  if (bos < eos) GDN_PREFETCH(bos);

  // O of a finished chunk from the fp32 LDS tile to 16-byte global stores, by
  // the first half of the waves: the two waves that share a SIMD finish a
  // chunk out of step, the later one (of the second half) setting the pace,
  // so the stores go to the waves that would otherwise wait at the barrier.
  // With the gated norm (kNorm) every wave stores: the norm's arithmetic
  // outweighs the slack of the first half alone.
  // Rows past the end of the chunk store a second copy of its last row
  // instead, so that every store is unconditional.  Address: uniform element
  // offset of (chunk start, head, slice) plus a lane's 32-bit offset
  // r * Hv * V + c (Hv * V is below 2^24: it bounds v's token stride).
  auto flush_o = [&](int64_t tp, int Lp) {
    constexpr int RUNS = BV / 8;  // 8-column runs per row
    constexpr int HT = kNorm ? NT : NT / 2;  // threads that store (with the norm: every wave)
    const int64_t obase = (tp * a.Hv + h) * (int64_t)a.V + v0;
    const uint32_t tok32 = (uint32_t)(a.Hv * a.V);
#pragma unroll
    for (int i = 0; i < CH * RUNS / HT; ++i) {
      const int u = tid + HT * i;
      const int r = min(u / RUNS, Lp - 1), c = 8 * (u % RUNS);
      const float* src = sO + r * OP + c;
      const float4 x0 = *reinterpret_cast<const float4*>(src);
      const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
      const uint32_t lo = __umul24((uint32_t)r, tok32) + (uint32_t)c;
      float y[8] = {a.scale * x0.x, a.scale * x0.y, a.scale * x0.z, a.scale * x0.w,
                    a.scale * x1.x, a.scale * x1.y, a.scale * x1.z, a.scale * x1.w};
      if constexpr (kNorm) {
        // gated RMS norm of the whole row (the 16 lanes of a row are adjacent
        // and aligned to 16 inside the wave): y = o rsqrt(mean o^2 + eps)
        // weight silu(z); z has o's layout, so it shares o's offsets
        float zv[8], wv[8];
        if (a.z_dt == 1) {
          const uint4 zr = *reinterpret_cast<const uint4*>((const char*)((const uint16_t*)a.z + obase) + 2u * lo);
          const uint32_t zw[4] = {zr.x, zr.y, zr.z, zr.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            zv[2 * e] = __uint_as_float(zw[e] << 16);
            zv[2 * e + 1] = __uint_as_float(zw[e] & 0xFFFF0000u);
          }
        } else {
          const float* zp = (const float*)((const char*)((const float*)a.z + obase) + 4u * lo);
          const float4 z0 = *reinterpret_cast<const float4*>(zp);
          const float4 z1 = *reinterpret_cast<const float4*>(zp + 4);
          zv[0] = z0.x, zv[1] = z0.y, zv[2] = z0.z, zv[3] = z0.w;
          zv[4] = z1.x, zv[5] = z1.y, zv[6] = z1.z, zv[7] = z1.w;
        }
        if (a.nw) {
          const float4 w0 = *reinterpret_cast<const float4*>(a.nw + v0 + c);
          const float4 w1 = *reinterpret_cast<const float4*>(a.nw + v0 + c + 4);
          wv[0] = w0.x, wv[1] = w0.y, wv[2] = w0.z, wv[3] = w0.w;
          wv[4] = w1.x, wv[5] = w1.y, wv[6] = w1.z, wv[7] = w1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) wv[e] = 1.f;
        }
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
        static_assert(RUNS == 16, "a row is one DPP row");
        ss = row16_sum(ss);
        const float inv = 1.f / sqrtf(ss / (float)BV + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = y[e] * inv * wv[e] * silu_hw(zv[e]);
      }
      if (kMode == kOutBF16) {
        uint4 w;
        w.x = pack_bf16x2(y[0], y[1]);
        w.y = pack_bf16x2(y[2], y[3]);
        w.z = pack_bf16x2(y[4], y[5]);
        w.w = pack_bf16x2(y[6], y[7]);
        *reinterpret_cast<uint4*>((char*)((uint16_t*)a.o + obase) + 2u * lo) = w;
      } else {
        float* dst = (float*)((char*)((float*)a.o + obase) + 4u * lo);
        *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(y[4], y[5], y[6], y[7]);
      }
    }
  };

  for (int64_t t0 = bos; t0 < eos; t0 += CH) {
    const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);
    __syncthreads();  // every wave is done with the previous chunk's tiles
    if (outb && t0 > bos && (kNorm || wave < NW / 2)) flush_o(t0 - CH, CH);  // a full chunk: only the last can be short

    // ---- stash q, k, v and the prep record ---------------------------------
    // Rows past the end of a partial chunk (and v of M columns) are zeroed in
    // the registers first; full chunks skip this.
    if (L < CH || !load_v) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < NPAIR; ++j) {
        if (r0_pf >= L) pk[j][0] = pq[j][0] = z;
        if (r0_pf + 1 >= L) pk[j][1] = pq[j][1] = z;
        if (!load_v || r0_pf >= L) pv[j][0] = z;
        if (!load_v || r0_pf + 1 >= L) pv[j][1] = z;
      }
    }
    // K^T words: the low halves of the two rows' words (row d0) and the high
    // halves (row d1) by byte permutes; the upper half-wave (8 rows further
    // on, the same bank half) stores row d1 first, so that each store
    // instruction covers both halves of the banks.
    const bool up_ = (lane & 32) != 0;
    const uint32_t sel_a = up_ ? 0x07060302u : 0x05040100u, sel_b = up_ ? 0x05040100u : 0x07060302u;
#pragma unroll
    for (int j = 0; j < NPAIR; ++j) {
      const int r0 = r0_pf, d8 = d8_pf + kDJ * j;
      const u32x4 k0 = pk[j][0], k1 = pk[j][1];
      const u32x4 v0v = pv[j][0], v1v = pv[j][1];
      store8_frag<true>(sK, r0, d8, k0);
      store8_frag<true>(sK, r0 + 1, d8, k1);
      if (outb) {
        store8_frag<true>(sQ, r0, d8, pq[j][0]);
        store8_frag<true>(sQ, r0 + 1, d8, pq[j][1]);
      }
#pragma unroll
      for (int jx = 0; jx < 4; ++jx) {
        const int d0 = d8 + 2 * jx, d1 = d0 + 1;
        const int da = up_ ? d1 : d0, db = up_ ? d0 : d1;
        *reinterpret_cast<uint32_t*>(sKt + da * TP + tile_pos<false>(da, r0)) =
            __builtin_amdgcn_perm(k1[jx], k0[jx], sel_a);
        *reinterpret_cast<uint32_t*>(sKt + db * TP + tile_pos<false>(db, r0)) =
            __builtin_amdgcn_perm(k1[jx], k0[jx], sel_b);
        // (zeros for M columns: their values were cleared above)
        *reinterpret_cast<uint32_t*>(sVt + d0 * VTP + r0) = (v0v[jx] & 0xFFFFu) | (v1v[jx] << 16);
        *reinterpret_cast<uint32_t*>(sVt + d1 * VTP + r0) = (v0v[jx] >> 16) | (v1v[jx] & 0xFFFF0000u);
      }
    }
    {
      // Every unit is stored (no branch around a store): a unit past the end
      // of what this mode reads holds a copy of its last unit and rewrites it
      // in place.
#pragma unroll
      for (int u = 0; u < NREC; ++u) {
        const int f = min(tid + u * NT, RUNITS - 1);
        unsigned char *dst0, *dst1;  // the unit's two 8-byte halves
        if (f < REC_TB_UNITS || f >= REC_STATE_UNITS) {
          // T diag(beta) hi, lo -> sT2; P hi, lo -> sP (two matrices each),
          // columns c .. c + 7 of row r, in fragment order
          const int fm = f < REC_TB_UNITS ? f : f - REC_STATE_UNITS;
          const int mat = fm / 320, rem = fm - 320 * mat;
          int bi, bj;
          tile_ij(rem >> 5, bi, bj);
          const int r = 16 * bi + ((rem >> 1) & 15), c = 16 * bj + 8 * (rem & 1);
          unsigned char* row = smem + (f < REC_TB_UNITS ? OFF_T2 : OFF_P) + 2 * (mat * CH * TP + r * TP);
          dst0 = row + 2 * tile_pos<false>(r, c);
          dst1 = row + 2 * tile_pos<false>(r, c + 4);
        } else {
          const int g = f - REC_TB_UNITS;  // 0..15 gamma, 16..31 dec
          dst0 = smem + OFF_GAM + 16 * g;
          dst1 = dst0 + 8;
        }
        *reinterpret_cast<u32x2*>(dst0) = u32x2{pr[u][0], pr[u][1]};
        *reinterpret_cast<u32x2*>(dst1) = u32x2{pr[u][2], pr[u][3]};
      }
    }
    // ---- fetch the next chunk while this one computes -----------------------
    __syncthreads();  // A: chunk data in LDS
    const bool more_ = t0 + CH < eos;
    if (more_) GDN_PF_REC(t0 + CH);

    // From here on each wave touches only its own state columns.
    // ---- K S and Q S over the split state (hi pass, then lo pass per k-step)
    f32x4 KS[NCT][4], O[NCT][4];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        zero4(KS[ct][rt]);
        zero4(O[ct][rt]);
      }
    auto state_products = [&](auto with_q) {
      constexpr bool WQ = decltype(with_q)::value;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        bf16x8 sp[2][NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) split_frag(S[ct][2 * m], S[ct][2 * m + 1], sp[0][ct], sp[1][ct]);
        bf16x8 fk[4], fq[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          fk[rt] = frag16<true>(sK, 16 * rt + c16, 32 * m, g4);
          if (WQ) fq[rt] = frag16<true>(sQ, 16 * rt + c16, 32 * m, g4);
        }
#pragma unroll
        for (int part = 0; part < 2; ++part)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              KS[ct][rt] = mfma16(fk[rt], sp[part][ct], KS[ct][rt]);
              if (WQ) O[ct][rt] = mfma16(fq[rt], sp[part][ct], O[ct][rt]);
            }
        SCHED_FENCE();
      }
    };
    if (outb)
      state_products(std::integral_constant<bool, kOut>{});
    else
      state_products(std::false_type{});

    if (more_) GDN_PF_KQ(t0 + CH);
    // ---- U = T diag(beta) (V - e^G K S) ------------------------------------------
    // R = V - gamma * (K S) is formed in the accumulator layout (V read from its
    // transposed tile, four consecutive tokens per lane), split into bf16
    // pairs, and multiplied by T diag(beta) as hi*hi + hi*lo + lo*hi.
    f32x4 U[NCT][4];
    {
      bf16x8 rh[NCT][2], rl[NCT][2];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 R[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          const float4 gam = *reinterpret_cast<const float4*>(sGam + 16 * rt + 4 * g4);
          R[rt][0] = -gam.x * KS[ct][rt][0];
          R[rt][1] = -gam.y * KS[ct][rt][1];
          R[rt][2] = -gam.z * KS[ct][rt][2];
          R[rt][3] = -gam.w * KS[ct][rt][3];
          const u32x2 vv =
              *reinterpret_cast<const u32x2*>(sVt + (wave * CPW + 16 * ct + c16) * VTP + 16 * rt + 4 * g4);
          R[rt][0] += __uint_as_float(vv[0] << 16);
          R[rt][1] += __uint_as_float(vv[0] & 0xFFFF0000u);
          R[rt][2] += __uint_as_float(vv[1] << 16);
          R[rt][3] += __uint_as_float(vv[1] & 0xFFFF0000u);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) split_frag(R[2 * m], R[2 * m + 1], rh[ct][m], rl[ct][m]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) zero4(U[ct][rt]);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 th[4], tl[4];
#pragma unroll
        for (int rt = 2 * m; rt < 4; ++rt) {
          th[rt] = frag16<false>(sT2, 16 * rt + c16, 32 * m, g4);
          tl[rt] = frag16<false>(sT2 + CH * TP, 16 * rt + c16, 32 * m, g4);
        }
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
          for (int rt = 2 * m; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              const bf16x8 ta = part == 2 ? tl[rt] : th[rt];
              const bf16x8 rb = part == 1 ? rl[ct][m] : rh[ct][m];
              U[ct][rt] = mfma16(ta, rb, U[ct][rt]);
            }
        SCHED_FENCE();
      }
    }
    if (more_) GDN_PF_V(t0 + CH);
    if (outb) {
      // ---- O = diag(gamma) Q S + P U  -> fp32 O tile in LDS -------------------
      bf16x8 Uhi[NCT][2], Ulo[NCT][2];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int m = 0; m < 2; ++m) split_frag(U[ct][2 * m], U[ct][2 * m + 1], Uhi[ct][m], Ulo[ct][m]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float4 gam = *reinterpret_cast<const float4*>(sGam + 16 * rt + 4 * g4);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          O[ct][rt][0] *= gam.x;
          O[ct][rt][1] *= gam.y;
          O[ct][rt][2] *= gam.z;
          O[ct][rt][3] *= gam.w;
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        bf16x8 ph[4], pl[4];
#pragma unroll
        for (int rt = 2 * m; rt < 4; ++rt) {
          ph[rt] = frag16<false>(sP, 16 * rt + c16, 32 * m, g4);
          pl[rt] = frag16<false>(sP + CH * TP, 16 * rt + c16, 32 * m, g4);
        }
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
          for (int rt = 2 * m; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
              const bf16x8 pa = part == 2 ? pl[rt] : ph[rt];
              const bf16x8 ub = part == 1 ? Ulo[ct][m] : Uhi[ct][m];
              O[ct][rt] = mfma16(pa, ub, O[ct][rt]);
            }
      }
    }
    // ---- S <- e^{G_last} S + K^T (diag(dec) U) -------------------------------
    {
      bf16x8 Uhi[NCT][2], Ulo[NCT][2];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const float4 dec = *reinterpret_cast<const float4*>(sDec + 16 * rt + 4 * g4);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          U[ct][rt][0] *= dec.x;
          U[ct][rt][1] *= dec.y;
          U[ct][rt][2] *= dec.z;
          U[ct][rt][3] *= dec.w;
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int m = 0; m < 2; ++m) split_frag(U[ct][2 * m], U[ct][2 * m + 1], Uhi[ct][m], Ulo[ct][m]);
      const float glast = sGam[CH - 1];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int e = 0; e < 4; ++e) S[ct][dt][e] *= glast;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 fk[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) fk[x] = frag16<false>(sKt, 16 * (4 * half + x) + c16, 32 * m, g4);
#pragma unroll
          for (int part = 0; part < 2; ++part)
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
              for (int ct = 0; ct < NCT; ++ct) {
                const int dt = 4 * half + x;
                S[ct][dt] = mfma16(fk[x], part ? Ulo[ct][m] : Uhi[ct][m], S[ct][dt]);
              }
          SCHED_FENCE();
        }
    }
    if (outb) {
      // O into this wave's own columns of the fp32 O tile; the first half of
      // the waves stores the whole tile after the next chunk's first barrier.
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sO[(16 * rt + 4 * g4 + e) * OP + wave * CPW + 16 * ct + c16] = O[ct][rt][e];
    }
  }
  if (outb && bos < eos) {  // the last chunk's O
    const int64_t t_last = bos + CH * ((eos - bos - 1) / CH);
    __syncthreads();
    if (kNorm || wave < NW / 2) flush_o(t_last, (int)(eos - t_last));
  }

#undef GDN_PREFETCH
#undef GDN_PF_ROWS
#undef GDN_PF_REC
#undef GDN_PF_KQ
#undef GDN_PF_V
#undef GDN_LD16
  // ---- final state ----------------------------------------------------------
  float* dst = nullptr;
  int64_t row_stride = 0;
  const int out_row = a.sf_map ? a.sf_map[seq] : zb;
  if (m_mode) {
    dst = p1.m_out + ((int64_t)(zb - (kMixed ? p1.n_fwd : 0)) * a.Hv + h) * (int64_t)KD * KD;
    row_stride = KD;
  } else if (kMixed && so) {
    dst = p1.b_out + ((int64_t)(zb - p1.n_fwd) * a.Hv + h) * (int64_t)KD * a.V;
    row_stride = a.V;
  } else if (a.sf && out_row >= 0) {
    dst = a.sf + (int64_t)out_row * a.sf_seq_stride + (int64_t)h * a.sf_head_stride;
    row_stride = a.sf_row_stride;
  }
  if (dst) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          dst[(int64_t)(16 * dt + 4 * g4 + e) * row_stride + col_base + 16 * ct + c16] = S[ct][dt][e];
  }
}

constexpr int kScanWaves = 8;  // the prefetch code assumes 512 threads

// n workgroups over blocks of n_tiles column tiles (the tile count of
// the map blocks in a mixed launch)
template <int kMode, bool kNorm = false, bool kMixed = false>
hipError_t launch_scan(const ChunkArgs& a, Pass1 p1, int n_tiles, int64_t n, hipStream_t stream) {
  // the LDS limit is raised once per device (a host call on every launch otherwise)
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
    const void* fn = (const void*)chunk_scan_kernel<kMode, kScanWaves, kNorm, kMixed>;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  // 1-D launch over (tile, v-head, sequence); the kernel decodes it
  ChunkArgs c = a;
  c.n_tiles = n_tiles;
  if (n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((chunk_scan_kernel<kMode, kScanWaves, kNorm, kMixed>), dim3((unsigned)n), dim3(kScanWaves * 64),
                     LDS_BYTES, stream, c, p1);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t stream, bool prep) {
  if (a.n_seqs == 0 || a.Hv == 0) return hipSuccess;
  if (a.K != KD || a.V % BV != 0 || a.tbuf == nullptr) return hipErrorInvalidValue;
  const bool with_o = a.o != nullptr && a.q != nullptr;
  if (prep) {
    hipError_t e = launch_chunk_prep(a, with_o ? 1 : 0, stream);
    if (e != hipSuccess) return e;
  }
  const int nz = a.seq_order ? a.n_blocks_z : a.n_seqs;
  if (nz == 0) return hipSuccess;
  const int tiles = a.V / BV;
  const int64_t n = (int64_t)tiles * a.Hv * nz;
  const Pass1 none{0, nullptr, 0, nullptr};
  if (!with_o) {
    // state only: run the scan without outputs
    return launch_scan<kPass1>(a, none, tiles, n, stream);
  }
  if (a.z) {
    // the gated norm needs a whole row of V values in one workgroup
    if (a.V != BV) return hipErrorInvalidValue;
    return a.o_dt == 1 ? launch_scan<kOutBF16, true>(a, none, tiles, n, stream)
                       : launch_scan<kOutF32, true>(a, none, tiles, n, stream);
  }
  return a.o_dt == 1 ? launch_scan<kOutBF16>(a, none, tiles, n, stream)
                     : launch_scan<kOutF32>(a, none, tiles, n, stream);
}

hipError_t launch_segment_pass1(const ChunkArgs& a, float* M, float* b, hipStream_t stream, bool prep) {
  if (a.n_seqs == 0 || a.Hv == 0) return hipSuccess;
  if (a.K != KD || a.V % BV != 0 || a.tbuf == nullptr) return hipErrorInvalidValue;
  if (prep) {
    hipError_t e = launch_chunk_prep(a, 0, stream);
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
  const int tiles = KD / BV + a.V / BV;
  return launch_scan<kPass1>(c, Pass1{KD / BV, M, 0, nullptr}, tiles, (int64_t)tiles * a.Hv * nz, stream);
}

hipError_t launch_split_pass1(const ChunkArgs& a, int n_fwd, float* M, float* b, hipStream_t stream) {
  if (a.n_seqs == 0 || a.Hv == 0 || a.n_blocks_z == 0) return hipSuccess;
  if (a.K != KD || a.V % BV != 0 || a.tbuf == nullptr) return hipErrorInvalidValue;
  if (a.o == nullptr || a.q == nullptr || n_fwd < 0 || n_fwd > a.n_blocks_z) return hipErrorInvalidValue;
  const Pass1 p1{KD / BV, M, n_fwd, b};
  const int tiles = KD / BV + a.V / BV;  // of a map block
  const int64_t n = (int64_t)n_fwd * a.Hv * (a.V / BV) + (int64_t)(a.n_blocks_z - n_fwd) * a.Hv * tiles;
  if (a.z) {
    if (a.V != BV) return hipErrorInvalidValue;
    return a.o_dt == 1 ? launch_scan<kOutBF16, true, true>(a, p1, tiles, n, stream)
                       : launch_scan<kOutF32, true, true>(a, p1, tiles, n, stream);
  }
  return a.o_dt == 1 ? launch_scan<kOutBF16, false, true>(a, p1, tiles, n, stream)
                     : launch_scan<kOutF32, false, true>(a, p1, tiles, n, stream);
}

}  // namespace gdn
