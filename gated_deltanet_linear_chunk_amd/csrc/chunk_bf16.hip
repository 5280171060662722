// chunk_bf16.hip -- chunked gated delta rule on gfx950 bf16 MFMA tiles.
//
// One workgroup of 8 waves owns one (sequence or segment, v-head, 128-column
// slice of V) and walks its 64-token chunks in order; the K x 128 fp32 state
// never leaves the registers: wave w holds columns 16w..16w+15 of it as eight
// 16 x 16 accumulator tiles (32 floats per lane).
//
// Per chunk (local tokens r, s; G = in-chunk cumulative gate, in fp64):
//  prep, independent of the state --
//    Gram products K K^T and Q K^T (bf16 inputs, exact products, fp32 sums),
//    A = strictly-lower(diag(beta) K K^T * e^{G_r - G_s}),
//    P = lower(Q K^T * e^{G_r - G_s}),
//    T = (I + A)^{-1} in fp32 (16 x 16 diagonal blocks by forward
//        substitution, then block rows),
//    W = T diag(beta e^G) K, U0 = T diag(beta) V on MFMA;
//  state step --
//    U = U0 - W S, O = diag(e^G) Q S + P U, S <- e^{G_last} S + K^T diag(e^{G_last - G}) U.
// That is the token recurrence regrouped by chunk (WY / UT form).
//
// Precision: every fp32 quantity that meets the matrix cores is split into a
// bf16 pair hi + lo (about 16 significant bits) and multiplied against exact
// bf16 data (q, k, v) or against another pair (hi*hi + hi*lo + lo*hi):
// T diag(beta e^G) and T diag(beta) against K and V, S against W and Q,
// P against U, diag(e^{G_last - G}) U against K.  W alone is a single bf16
// operand: W S is a 128-term sum whose rounding errors average out.  With
// these choices the kernel's error is set by fp32 accumulation, not by bf16.
//
// LDS (bytes, bf16 unless noted; pitches padded by 16 B):
//   sQ [64][136]            sK [64][136] (dead after the Gram products ->
//                                          reused for the fp32 T [64][68])
//   sKt [128][72] (K^T)     sVt [128][72] (V^T, this workgroup's 128 columns)
//   sP [2][64][72] (P hi, lo)
//   sT2 [4][64][72] (T diag(beta e^G) hi/lo, T diag(beta) hi/lo; also the
//                    scratch of the block-row inversion before that)
//   sA fp32 [64][68] (A; then reused for -W as bf16 [64][136])
#include "device_common.h"
#include "kernels.h"

namespace gdn {

namespace {

constexpr int CH = 64;
constexpr int KD = 128;  // key dim
constexpr int BV = 128;  // value columns per workgroup
constexpr int NWAVE = 8;
constexpr int NTHREADS = NWAVE * 64;

constexpr int QP = KD + 8;  // pitch of row-major [64][K] bf16 tiles
constexpr int TP = CH + 8;  // pitch of [*][64] bf16 tiles
constexpr int FP = CH + 4;  // pitch of fp32 [64][64] tiles

constexpr int OFF_Q = 0;
constexpr int OFF_K = OFF_Q + CH * QP * 2;      // also fp32 T
constexpr int OFF_KT = OFF_K + CH * QP * 2;
constexpr int OFF_VT = OFF_KT + KD * TP * 2;
constexpr int OFF_P = OFF_VT + BV * TP * 2;
constexpr int OFF_T2 = OFF_P + 2 * CH * TP * 2;
constexpr int OFF_A = OFF_T2 + 4 * CH * TP * 2;  // also -W
constexpr int OFF_G = OFF_A + CH * QP * 2;        // double[64]
constexpr int OFF_BETA = OFF_G + CH * 8;
constexpr int OFF_GAM = OFF_BETA + CH * 4;
constexpr int OFF_DEC = OFF_GAM + CH * 4;
constexpr int LDS_BYTES = OFF_DEC + CH * 4;
static_assert(CH * FP * 4 <= CH * QP * 2, "fp32 T must fit in the K tile");
static_assert(CH * FP * 4 <= CH * QP * 2, "fp32 A must fit in the -W tile");
static_assert(3 * 256 * 4 <= 4 * CH * TP * 2, "inversion scratch must fit in sT2");
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

struct Pass1 {
  int m_tiles;  // leading blockIdx.x values that evolve M columns (v = 0, S0 = I)
  float* m_out;  // [n_seqs, Hv, K, K]
};

__device__ __forceinline__ void zero4(f32x4& x) { x[0] = x[1] = x[2] = x[3] = 0.f; }

template <bool kHasPass1>
__global__ void __launch_bounds__(NTHREADS) chunk_bf16_kernel(ChunkArgs a, Pass1 p1) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + OFF_Q);
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + OFF_K);
  float* sTf = reinterpret_cast<float*>(smem + OFF_K);
  uint16_t* sKt = reinterpret_cast<uint16_t*>(smem + OFF_KT);
  uint16_t* sVt = reinterpret_cast<uint16_t*>(smem + OFF_VT);
  uint16_t* sP = reinterpret_cast<uint16_t*>(smem + OFF_P);
  uint16_t* sT2 = reinterpret_cast<uint16_t*>(smem + OFF_T2);
  float* sY = reinterpret_cast<float*>(smem + OFF_T2);
  float* sA = reinterpret_cast<float*>(smem + OFF_A);
  uint16_t* sWn = reinterpret_cast<uint16_t*>(smem + OFF_A);
  double* sG = reinterpret_cast<double*>(smem + OFF_G);
  float* sBeta = reinterpret_cast<float*>(smem + OFF_BETA);
  float* sGam = reinterpret_cast<float*>(smem + OFF_GAM);
  float* sDec = reinterpret_cast<float*>(smem + OFF_DEC);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  // ---- which unit this workgroup runs -------------------------------------
  bool m_mode = false;
  int tile = blockIdx.x;
  if (kHasPass1 && tile < p1.m_tiles) m_mode = true;
  if (kHasPass1 && !m_mode) tile -= p1.m_tiles;
  const int v0 = tile * BV;  // first column (of V, or of M in m_mode)
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
  const uint16_t* qg = (const uint16_t*)a.q;
  const uint16_t* kg = (const uint16_t*)a.k;
  const uint16_t* vg = m_mode ? nullptr : (const uint16_t*)a.v;
  const bool want_o = !m_mode && a.o != nullptr && qg != nullptr;
  const int s0_mode = m_mode ? 2 : a.s0_mode;
  const int col_base = v0 + wave * 16;  // this wave's first state column

  // ---- initial state: S[d][col_base + c16], d = 16*dt + 4*g4 + e ----------
  f32x4 S[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d = 16 * dt + 4 * g4 + e;
      float s = 0.f;
      if (s0_mode == 1)
        s = a.s0[((int64_t)seq * a.Hv + h) * (int64_t)KD * a.V + (int64_t)d * a.V + col_base + c16];
      else if (s0_mode == 2)
        s = (d == col_base + c16) ? 1.f : 0.f;
      S[dt][e] = s;
    }
  }

  // sP's upper tiles (0,1) and (2,3) are read as zeros by the P U product and
  // are never written afterwards.
  for (int i = tid; i < 2 * CH * TP; i += NTHREADS) sP[i] = 0;

  for (int64_t t0 = bos; t0 < eos; t0 += CH) {
    const int L = (int)((eos - t0) < CH ? (eos - t0) : CH);
    __syncthreads();  // the previous chunk is fully consumed

    // ---- load q, k (row-major + transposed), v (transposed), g, beta -------
    {
      const int rp = tid >> 4;          // row pair 0..31
      const int d8 = (tid & 15) * 8;    // 8-element column group
      const int r0 = 2 * rp, r1 = r0 + 1;
      uint4 kz0 = make_uint4(0, 0, 0, 0), kz1 = kz0, qz0 = kz0, qz1 = kz0, vz0 = kz0, vz1 = kz0;
      const int64_t head_off = (int64_t)hq * KD + d8;
      const int64_t v_off = (int64_t)h * a.V + v0 + d8;
      if (r0 < L) {
        kz0 = *reinterpret_cast<const uint4*>(kg + (t0 + r0) * a.k_stride + head_off);
        if (want_o) qz0 = *reinterpret_cast<const uint4*>(qg + (t0 + r0) * a.q_stride + head_off);
        if (vg) vz0 = *reinterpret_cast<const uint4*>(vg + (t0 + r0) * a.v_stride + v_off);
      }
      if (r1 < L) {
        kz1 = *reinterpret_cast<const uint4*>(kg + (t0 + r1) * a.k_stride + head_off);
        if (want_o) qz1 = *reinterpret_cast<const uint4*>(qg + (t0 + r1) * a.q_stride + head_off);
        if (vg) vz1 = *reinterpret_cast<const uint4*>(vg + (t0 + r1) * a.v_stride + v_off);
      }
      *reinterpret_cast<uint4*>(sK + r0 * QP + d8) = kz0;
      *reinterpret_cast<uint4*>(sK + r1 * QP + d8) = kz1;
      *reinterpret_cast<uint4*>(sQ + r0 * QP + d8) = qz0;
      *reinterpret_cast<uint4*>(sQ + r1 * QP + d8) = qz1;
      const uint32_t k0w[4] = {kz0.x, kz0.y, kz0.z, kz0.w};
      const uint32_t k1w[4] = {kz1.x, kz1.y, kz1.z, kz1.w};
      const uint32_t v0w[4] = {vz0.x, vz0.y, vz0.z, vz0.w};
      const uint32_t v1w[4] = {vz1.x, vz1.y, vz1.z, vz1.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // element 2j (low half) and 2j+1 (high half) of each row
        const uint32_t klo = (k0w[j] & 0xFFFFu) | (k1w[j] << 16);
        const uint32_t khi = (k0w[j] >> 16) | (k1w[j] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(sKt + (d8 + 2 * j) * TP + r0) = klo;
        *reinterpret_cast<uint32_t*>(sKt + (d8 + 2 * j + 1) * TP + r0) = khi;
        const uint32_t vlo = (v0w[j] & 0xFFFFu) | (v1w[j] << 16);
        const uint32_t vhi = (v0w[j] >> 16) | (v1w[j] & 0xFFFF0000u);
        *reinterpret_cast<uint32_t*>(sVt + (d8 + 2 * j) * TP + r0) = vlo;
        *reinterpret_cast<uint32_t*>(sVt + (d8 + 2 * j + 1) * TP + r0) = vhi;
      }
    }
    if (wave == 0) {
      // in-chunk inclusive cumulative gate in fp64 (padding rows add 0)
      const bool ok = lane < L;
      double G = ok ? (double)a.g[(t0 + lane) * a.Hv + h] : 0.0;
      sBeta[lane] = ok ? a.beta[(t0 + lane) * a.Hv + h] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(G, off, 64);
        if (lane >= off) G += o;
      }
      const double Glast = __shfl(G, 63, 64);
      sG[lane] = G;
      sGam[lane] = expf((float)G);
      sDec[lane] = expf((float)(Glast - G));
    }
    __syncthreads();

    // ---- Gram products: 10 lower 16x16 tiles of K K^T and of Q K^T --------
    // job 0..9: K K^T tile (i, j); job 10..19: Q K^T tile (i, j), i >= j.
    f32x4 gacc[3];
    int gjob[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int job = wave + NWAVE * u;
      gjob[u] = job;
      zero4(gacc[u]);
      if (job < 20 && (job < 10 || want_o)) {
        const int jj = job % 10;
        // tile (i, j) for jj in order (0,0),(1,0),(1,1),(2,0),(2,1),(2,2),(3,0),...
        const int i = jj >= 6 ? 3 : (jj >= 3 ? 2 : (jj >= 1 ? 1 : 0));
        const int j = jj - (i * (i + 1)) / 2;
        const uint16_t* Am = job < 10 ? sK : sQ;
#pragma unroll
        for (int m = 0; m < KD / 32; ++m) {
          const bf16x8 fa = lds_frag(Am, QP, 16 * i + c16, 32 * m, g4);
          const bf16x8 fb = lds_frag(sK, QP, 16 * j + c16, 32 * m, g4);
          gacc[u] = mfma16(fa, fb, gacc[u]);
        }
      }
    }
    __syncthreads();  // sK is about to be reused for T
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int job = gjob[u];
      if (job >= 20 || (job >= 10 && !want_o)) continue;
      const int jj = job % 10;
      const int i = jj >= 6 ? 3 : (jj >= 3 ? 2 : (jj >= 1 ? 1 : 0));
      const int j = jj - (i * (i + 1)) / 2;
      const int s = 16 * j + c16;
      const double Gs = sG[s];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * i + 4 * g4 + e;
        if (job < 10) {
          float val = 0.f;
          if (r > s) val = sBeta[r] * gacc[u][e] * expf((float)(sG[r] - Gs));
          sA[r * FP + s] = val;
        } else {
          float val = 0.f;
          if (r >= s) val = gacc[u][e] * expf((float)(sG[r] - Gs));
          uint16_t hi, lo;
          split_bf16(val, hi, lo);
          sP[r * TP + s] = hi;
          sP[CH * TP + r * TP + s] = lo;
        }
      }
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}: diagonal 16x16 blocks ----------------------------
    if (wave == 0) {
      const int b = lane >> 4;  // block
      const int j = lane & 15;  // column within the block
      const float* Ab = sA + (16 * b) * FP + 16 * b;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float val = (r == j) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < r; ++s) val = fmaf(-Ab[r * FP + s], x[s], val);
        x[r] = val;  // zero above the diagonal (r < j) by construction
      }
      float* Tb = sTf + (16 * b) * FP + 16 * b;
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[r * FP + j] = x[r];
    }
    __syncthreads();
    // ---- off-diagonal block rows: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj ----
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      for (int idx = tid; idx < 256 * i; idx += NTHREADS) {
        const int j = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        float acc = 0.f;
        for (int kb = j; kb < i; ++kb) {
          const float* Ar = sA + (16 * i + r) * FP + 16 * kb;
          const float* Tc = sTf + (16 * kb) * FP + 16 * j + c;
#pragma unroll
          for (int s = 0; s < 16; ++s) acc = fmaf(Ar[s], Tc[s * FP], acc);
        }
        sY[(j * 16 + r) * 16 + c] = acc;
      }
      __syncthreads();
      for (int idx = tid; idx < 256 * i; idx += NTHREADS) {
        const int j = idx >> 8, r = (idx >> 4) & 15, c = idx & 15;
        const float* Tr = sTf + (16 * i + r) * FP + 16 * i;
        float acc = 0.f;
        for (int m = 0; m <= r; ++m) acc = fmaf(Tr[m], sY[(j * 16 + m) * 16 + c], acc);
        sTf[(16 * i + r) * FP + 16 * j + c] = -acc;
      }
      __syncthreads();
    }

    // ---- T diag(beta e^G), T diag(beta) as bf16 pairs (full 64 x 64) -------
    for (int idx = tid; idx < CH * CH / 4; idx += NTHREADS) {
      const int r = idx >> 4, s0 = (idx & 15) * 4;
      u16x4 w_hi, w_lo, u_hi, u_lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = s0 + e;
        const float t = (s <= r) ? sTf[r * FP + s] : 0.f;
        uint16_t hi, lo;
        split_bf16(t * sBeta[s] * sGam[s], hi, lo);
        w_hi[e] = hi;
        w_lo[e] = lo;
        split_bf16(t * sBeta[s], hi, lo);
        u_hi[e] = hi;
        u_lo[e] = lo;
      }
      *reinterpret_cast<u16x4*>(sT2 + 0 * CH * TP + r * TP + s0) = w_hi;
      *reinterpret_cast<u16x4*>(sT2 + 1 * CH * TP + r * TP + s0) = w_lo;
      *reinterpret_cast<u16x4*>(sT2 + 2 * CH * TP + r * TP + s0) = u_hi;
      *reinterpret_cast<u16x4*>(sT2 + 3 * CH * TP + r * TP + s0) = u_lo;
    }
    __syncthreads();

    // ---- W^T = K^T (T diag(beta e^G))^T: wave owns key rows 16*wave.. -----
    // Stored negated as bf16 -W[r][d] (row-major), the A operand of W S.
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 acc;
      zero4(acc);
#pragma unroll
      for (int m = 0; m <= rt / 2; ++m) {
        const bf16x8 fa = lds_frag(sKt, TP, 16 * wave + c16, 32 * m, g4);
        const bf16x8 fh = lds_frag(sT2 + 0 * CH * TP, TP, 16 * rt + c16, 32 * m, g4);
        const bf16x8 fl = lds_frag(sT2 + 1 * CH * TP, TP, 16 * rt + c16, 32 * m, g4);
        acc = mfma16(fa, fh, acc);
        acc = mfma16(fa, fl, acc);
      }
      // acc[e] = W[r = 16 rt + c16][d = 16 wave + 4 g4 + e]
      u16x4 wv;
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[e] = f32_to_bf16_bits(-acc[e]);
      *reinterpret_cast<u16x4*>(sWn + (16 * rt + c16) * QP + 16 * wave + 4 * g4) = wv;
    }
    // ---- U0 = T diag(beta) V for this wave's 16 columns --------------------
    f32x4 U[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      zero4(U[rt]);
      if (vg) {
#pragma unroll
        for (int m = 0; m <= rt / 2; ++m) {
          const bf16x8 fb = lds_frag(sVt, TP, 16 * wave + c16, 32 * m, g4);
          const bf16x8 fh = lds_frag(sT2 + 2 * CH * TP, TP, 16 * rt + c16, 32 * m, g4);
          const bf16x8 fl = lds_frag(sT2 + 3 * CH * TP, TP, 16 * rt + c16, 32 * m, g4);
          U[rt] = mfma16(fh, fb, U[rt]);
          U[rt] = mfma16(fl, fb, U[rt]);
        }
      }
    }
    __syncthreads();  // -W complete

    // ---- state step ---------------------------------------------------------
    bf16x8 Shi[4], Slo[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) split_frag(S[2 * m], S[2 * m + 1], Shi[m], Slo[m]);
    // U = U0 - W S
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bf16x8 fw = lds_frag(sWn, QP, 16 * rt + c16, 32 * m, g4);
        U[rt] = mfma16(fw, Shi[m], U[rt]);
        U[rt] = mfma16(fw, Slo[m], U[rt]);
      }
    }
    bf16x8 Uhi[2], Ulo[2];
    if (want_o) {
#pragma unroll
      for (int m = 0; m < 2; ++m) split_frag(U[2 * m], U[2 * m + 1], Uhi[m], Ulo[m]);
      // O = diag(gamma) Q S + P U
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        f32x4 qs;
        zero4(qs);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8 fq = lds_frag(sQ, QP, 16 * rt + c16, 32 * m, g4);
          qs = mfma16(fq, Shi[m], qs);
          qs = mfma16(fq, Slo[m], qs);
        }
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = qs[e] * sGam[16 * rt + 4 * g4 + e];
#pragma unroll
        for (int m = 0; m <= rt / 2; ++m) {
          const bf16x8 ph = lds_frag(sP, TP, 16 * rt + c16, 32 * m, g4);
          const bf16x8 pl = lds_frag(sP + CH * TP, TP, 16 * rt + c16, 32 * m, g4);
          o = mfma16(ph, Uhi[m], o);
          o = mfma16(ph, Ulo[m], o);
          o = mfma16(pl, Uhi[m], o);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rt + 4 * g4 + e;
          if (r < L) {
            const int64_t off = ((t0 + r) * a.Hv + h) * (int64_t)a.V + col_base + c16;
            const float val = a.scale * o[e];
            if (a.o_dt == 1)
              ((uint16_t*)a.o)[off] = f32_to_bf16_bits(val);
            else
              ((float*)a.o)[off] = val;
          }
        }
      }
    }
    // S <- e^{G_last} S + K^T (diag(dec) U)
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) U[rt][e] *= sDec[16 * rt + 4 * g4 + e];
#pragma unroll
    for (int m = 0; m < 2; ++m) split_frag(U[2 * m], U[2 * m + 1], Uhi[m], Ulo[m]);
    const float glast = sGam[CH - 1];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[dt][e] *= glast;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const bf16x8 fk = lds_frag(sKt, TP, 16 * dt + c16, 32 * m, g4);
        S[dt] = mfma16(fk, Uhi[m], S[dt]);
        S[dt] = mfma16(fk, Ulo[m], S[dt]);
      }
    }
  }

  // ---- final state ----------------------------------------------------------
  float* dst = nullptr;
  int64_t row_stride = 0;
  if (m_mode) {
    dst = p1.m_out + ((int64_t)seq * a.Hv + h) * (int64_t)KD * KD;
    row_stride = KD;
  } else if (a.sf) {
    dst = a.sf + (int64_t)seq * a.sf_seq_stride + (int64_t)h * a.sf_head_stride;
    row_stride = a.sf_row_stride;
  }
  if (dst) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dst[(int64_t)(16 * dt + 4 * g4 + e) * row_stride + col_base + c16] = S[dt][e];
  }
}

}  // namespace

hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t stream) {
  if (a.n_seqs == 0 || a.Hv == 0) return hipSuccess;
  if (a.K != KD || a.V % BV != 0) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)chunk_bf16_kernel<false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  dim3 grid(a.V / BV, a.Hv, a.n_seqs);
  Pass1 p1{0, nullptr};
  hipLaunchKernelGGL(chunk_bf16_kernel<false>, grid, dim3(NTHREADS), LDS_BYTES, stream, a, p1);
  return hipGetLastError();
}

hipError_t launch_segment_pass1(const ChunkArgs& a, float* M, float* b, hipStream_t stream) {
  if (a.n_seqs == 0 || a.Hv == 0) return hipSuccess;
  if (a.K != KD || a.V % BV != 0) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)chunk_bf16_kernel<true>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  ChunkArgs c = a;
  c.q = nullptr;
  c.o = nullptr;
  c.sf = b;
  c.sf_seq_stride = (int64_t)a.Hv * KD * a.V;
  c.sf_head_stride = (int64_t)KD * a.V;
  c.sf_row_stride = a.V;
  c.s0_mode = 0;
  Pass1 p1{KD / BV, M};
  dim3 grid(KD / BV + a.V / BV, a.Hv, a.n_seqs);
  hipLaunchKernelGGL(chunk_bf16_kernel<true>, grid, dim3(NTHREADS), LDS_BYTES, stream, c, p1);
  return hipGetLastError();
}

}  // namespace gdn
