// gate_conv.hip -- gates and the causal depthwise conv1d (+ SiLU, + q/k L2 norm).
//
// Both are streaming, HBM-bound steps: no matrix work, so they use plain
// coalesced 16-byte vector loads and stores and fp32 arithmetic.
#include "device_common.h"
#include "kernels.h"

namespace gdn {

// ----------------------------------------------------------------------------
// Gates: beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias).
// ----------------------------------------------------------------------------
__global__ void __launch_bounds__(256) gate_kernel(const float* __restrict__ a,
                                                   const float* __restrict__ b,
                                                   const float* __restrict__ A_log,
                                                   const float* __restrict__ dt_bias,
                                                   int64_t n, int H, float* __restrict__ g,
                                                   float* __restrict__ beta) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int h = (int)(i % H);
    gate_values(a[i], b[i], A_log[h], dt_bias[h], g[i], beta[i]);
  }
}

hipError_t launch_gate(const float* a, const float* b, const float* A_log, const float* dt_bias,
                       int64_t n_tokens, int H, float* g, float* beta, hipStream_t stream) {
  const int64_t n = n_tokens * H;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, b, A_log,
                     dt_bias, n, H, g, beta);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// Causal depthwise conv1d.
//
// One thread owns 8 consecutive channels (one 16-byte bf16 vector); a block of
// 256 threads covers 2048 channels and walks a run of tokens in sub-tiles of
// SUB tokens.  A wave (512 channels) reads one contiguous 1 KiB row segment
// per token, so every load and store is fully coalesced.  The rows of the
// next sub-tile are loaded while the current one is computed (two register
// buffers), and the last three inputs of the thread's channels stay in
// registers as the history.  Rows before the start of the current token's
// sample count as zero: the sample of the run's first token comes from a
// binary search of cu_seqlens (or from the batch row), later boundaries from
// walking the offsets, all of it uniform across the block; sub-tiles with no
// sample start among their first three tokens skip the masking.
// A block covers either normalised (q/k) channels or the others, so every
// wave runs one kind of work.  The per-head L2 norm sums over
// head_dim / 8 adjacent lanes with DPP exchanges (xor 1, xor 2, then the
// half-row and row mirrors), which stay inside one head because heads are
// 8-channel aligned.
// Outputs are the fp32 evaluation rounded once to the output type.  On
// request (exact rounding), bf16 outputs are instead the bf16 nearest to the
// exact result: each value carries an error bound (for a normalised value,
// also from its head's sum of squares and the reciprocal square root), and the
// few whose bound straddles a bf16 rounding midpoint are queued and recomputed
// in fp64 at the end of the run (a normalised one with its whole head).
// ----------------------------------------------------------------------------
constexpr int CONV_THREADS = 256;
constexpr int CONV_CH_PER_THREAD = 8;
constexpr int CONV_QCAP = 512;  // queued doubtful roundings per wave
#ifndef GDN_CONV_BLOCKS
#define GDN_CONV_BLOCKS 512  // blocks per launch the token runs are sized for (2 per CU)
#endif

template <typename T>
struct ConvRow;

template <>
struct ConvRow<uint16_t> {  // bf16: one 16-byte vector per row
  static constexpr int SUB = 8;
  typedef u32x4 raw_t;
  static __device__ __forceinline__ raw_t load(const uint16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ void unpack(const raw_t& r, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(r[i] << 16);
      out[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* in) {
    const u32x4 w = {pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]), pack_bf16x2(in[4], in[5]),
                     pack_bf16x2(in[6], in[7])};
    *reinterpret_cast<u32x4*>(p) = w;
  }
  static __device__ __forceinline__ float scalar(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
};

template <>
struct ConvRow<float> {
  static constexpr int SUB = 4;
  struct raw_t {
    float4 a, b;
  };
  static __device__ __forceinline__ raw_t load(const float* p) {
    return raw_t{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
  }
  static __device__ __forceinline__ void unpack(const raw_t& r, float* out) {
    out[0] = r.a.x; out[1] = r.a.y; out[2] = r.a.z; out[3] = r.a.w;
    out[4] = r.b.x; out[5] = r.b.y; out[6] = r.b.z; out[7] = r.b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* in) {
    *reinterpret_cast<float4*>(p) = make_float4(in[0], in[1], in[2], in[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(in[4], in[5], in[6], in[7]);
  }
  static __device__ __forceinline__ float scalar(const float* p, int64_t i) { return p[i]; }
};

// Sample index of token t (largest n with cu[n] <= t), offsets clamped to [0, T].
__device__ __forceinline__ int find_sample(const int32_t* cu, int n_seqs, int64_t t,
                                           int64_t Ttot) {
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (clampi(cu[mid], 0, Ttot) <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// First token of the region (sample, trailing tokens past the last offset, or
// batch row) that holds token t.
__device__ __forceinline__ int64_t region_start(const int32_t* cu, int n_seqs, int64_t row_len,
                                                int64_t Ttot, int64_t t) {
  if (!cu) return (t / row_len) * row_len;
  const int64_t last = clampi(cu[n_seqs], 0, Ttot);
  if (t >= last) return last;
  return clampi(cu[find_sample(cu, n_seqs, t, Ttot)], 0, Ttot);
}

// bf16 nearest to d (ties to even), as a float.  Rounding d to fp32 first
// can only mislead when the fp32 result lands exactly on a bf16 midpoint;
// that case is decided by comparing d with the midpoint.
__device__ __forceinline__ float bf16_nearest_f64(double d) {
  const float f = (float)d;
  uint32_t b = __float_as_uint(f);
  if ((b & 0xFFFFu) == 0x8000u) {
    const double ad = fabs(d), am = fabs((double)f);
    if (ad > am) return __uint_as_float((b & 0xFFFF0000u) + 0x10000u);
    if (ad < am) return __uint_as_float(b & 0xFFFF0000u);
  }
  b = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
  return __uint_as_float(b);
}


// Whether y (fp32, from bf16 inputs) might round to another bf16 value than
// the exact conv (+ SiLU) result.  The tap products are exact and each of the
// four fused sums rounds once, by at most 2^-24 of its magnitude, which is
// below A = |bias| + sum_j |w_j| |x_j| (the output's own taps, summed in fp32
// alongside z); the SiLU evaluation adds a few ulp of y.
// E = 2^-20 |y| + 9 * 2^-24 A covers both about twice over.  The nearest
// rounding midpoint to y is the one above its bf16 truncation.
// Ab = 9 * 2^-24 * A.
__device__ __forceinline__ bool rounding_in_doubt(float y, float Ab) {
  const float E = fmaf(0x1p-20f, fabsf(y), Ab);
  const float mid = __uint_as_float((__float_as_uint(y) & 0xFFFF0000u) | 0x8000u);
  return fabsf(y - mid) <= E;
}

// One conv (+ SiLU) output in fp64 (the products of bf16 values and their sum
// are exact there), stored as its nearest bf16.  hist: how many rows before t
// lie in t's sample (at most 3 matter).
__device__ __noinline__ void settle_value(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                          const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                          int64_t C, int width, int apply_silu, int64_t t, int64_t c, int hist) {
  double z = bias ? (double)bf16_bits_to_f32(bias[c]) : 0.0;
  for (int j = 0; j < width; ++j) {
    const int back = width - 1 - j;  // tap j multiplies x[t - back]
    if (back <= hist)
      z += (double)bf16_bits_to_f32(w[c * width + j]) * (double)bf16_bits_to_f32(x[(t - back) * C + c]);
  }
  const double v = apply_silu ? z / (1.0 + exp(-z)) : z;
  y[t * C + c] = f32_to_bf16_bits(bf16_nearest_f64(v));
}

// One L2-normalised output in fp64: the conv (+ SiLU) of every channel of
// c's head, their sum of squares S, and y_c / sqrt(S + eps) stored as its
// nearest bf16.  hist as for settle_value.
__device__ __noinline__ void settle_l2_value(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                             const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t C,
                                             int width, int apply_silu, int head_dim, double eps, int64_t t,
                                             int64_t c, int hist) {
  const int64_t h0 = c - c % head_dim;
  double S = 0.0, yc = 0.0;
  for (int jc = 0; jc < head_dim; ++jc) {
    const int64_t cj = h0 + jc;
    double z = bias ? (double)bf16_bits_to_f32(bias[cj]) : 0.0;
    for (int j = 0; j < width; ++j) {
      const int back = width - 1 - j;
      if (back <= hist)
        z += (double)bf16_bits_to_f32(w[cj * width + j]) * (double)bf16_bits_to_f32(x[(t - back) * C + cj]);
    }
    const double v = apply_silu ? z / (1.0 + exp(-z)) : z;
    S += v * v;
    if (cj == c) yc = v;
  }
  y[t * C + c] = f32_to_bf16_bits(bf16_nearest_f64(yc / sqrt(S + eps)));
}

struct ConvParams {
  const int32_t* cu;
  int n_seqs;
  int64_t row_len, Ttot;
  int C;            // channels of the whole row (the row pitch)
  int c_begin, c_end;  // channel range of this launch
  int l2_end;          // channels below are L2-normalised per head
  int width, apply_silu;
  int l2_lanes_log2;
  float l2_eps;
  int tile_tokens;  // tokens per block (a multiple of SUB)
};

// One sub-tile of SUB tokens for this thread's 8 channels.  kMode: 0 plain,
// 1 plain with the rounding check (bf16 output), 2 L2-normalised, 3
// L2-normalised with the rounding check (bf16 output).  kMasked:
// the sub-tile reaches past the run or starts a sample within its first
// three tokens, so history rows are masked per token (hist_code: 2 bits per
// token, the count of its history rows inside its sample).
template <typename T, int kMode, bool kMasked, bool kSilu>
__device__ __forceinline__ void conv_sub(const typename ConvRow<T>::raw_t (&buf)[ConvRow<T>::SUB],
                                         float (&h1)[CONV_CH_PER_THREAD], float (&h2)[CONV_CH_PER_THREAD],
                                         float (&h3)[CONV_CH_PER_THREAD],
                                         const float (&wt)[4][CONV_CH_PER_THREAD],
                                         const float (&bs)[CONV_CH_PER_THREAD],
                                         const float (&wa)[4][CONV_CH_PER_THREAD],
                                         const float (&ba)[CONV_CH_PER_THREAD],
                                         int n_valid,
                                         uint32_t hist_code, const ConvParams& p, bool active,
                                         T* __restrict__ yrow, uint32_t* queue, uint32_t* qcount,
                                         int64_t ts, int64_t tw0, int c0, bool& overflow) {
  using Row = ConvRow<T>;
  constexpr int SUB = Row::SUB;
  constexpr int NCH = CONV_CH_PER_THREAD;
  constexpr bool kCheck = (kMode == 1 || kMode == 3) && sizeof(T) == 2;
  constexpr bool kL2 = kMode >= 2;
#pragma unroll
  for (int tt = 0; tt < SUB; ++tt) {
    if (kMasked && tt >= n_valid) break;
    const int hist = kMasked ? (int)((hist_code >> (2 * tt)) & 3u) : 3;
    float cur[NCH], out[NCH];
    Row::unpack(buf[tt], cur);
    float ss = 0.f, es = 0.f, eb[NCH];
    uint32_t dbits = 0;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const float x1 = (!kMasked || hist >= 3) ? h1[i] : 0.f;
      const float x2 = (!kMasked || hist >= 2) ? h2[i] : 0.f;
      const float x3 = (!kMasked || hist >= 1) ? h3[i] : 0.f;
      float z = bs[i];
      z = fmaf(wt[0][i], x1, z);
      z = fmaf(wt[1][i], x2, z);
      z = fmaf(wt[2][i], x3, z);
      z = fmaf(wt[3][i], cur[i], z);
      const float v = kSilu ? silu_conv(z) : z;
      out[i] = v;
      if (kL2) ss = fmaf(v, v, ss);
      if (kCheck) {
        // Ab = 9 * 2^-24 * (|bias| + sum_j |w_j| |x_j|) from taps scaled by
        // 9 * 2^-24 beforehand (exact for bf16 taps)
        float Ab = ba[i];
        Ab = fmaf(wa[0][i], fabsf(x1), Ab);
        Ab = fmaf(wa[1][i], fabsf(x2), Ab);
        Ab = fmaf(wa[2][i], fabsf(x3), Ab);
        Ab = fmaf(wa[3][i], fabsf(cur[i]), Ab);
        if (kMode == 1) {
          dbits |= (rounding_in_doubt(v, Ab) ? 1u : 0u) << i;
        } else {
          // bound of |v - exact| as for unnormalised outputs; 2 |v| E bounds
          // this value's share of the error of the head's sum of squares
          eb[i] = fmaf(0x1p-20f, fabsf(v), Ab);
          es = fmaf(2.f * fabsf(v), eb[i], es);
        }
      }
      h1[i] = h2[i];
      h2[i] = h3[i];
      h3[i] = cur[i];
    }
    if (kL2) {  // every lane of the wave joins the exchanges
      ss = group_sum(ss, p.l2_lanes_log2);
      const float inv = __builtin_amdgcn_rsqf(ss + p.l2_eps);
#pragma unroll
      for (int i = 0; i < NCH; ++i) out[i] *= inv;
      if (kMode == 3) {
        // n = y / sqrt(S + eps): its relative error is that of y, half that
        // of S + eps (es from the values, 16 roundings of the positive sum),
        // the reciprocal square root (1 ulp) and the product, taken twice
        es = group_sum(es, p.l2_lanes_log2);
        const float rel = fmaf(0.5f, (es + 16.f * 0x1p-24f * ss) * __builtin_amdgcn_rcpf(ss + p.l2_eps), 0x1p-22f);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const float bound = 2.f * fmaf(eb[i], inv, fabsf(out[i]) * rel);
          const float mid = __uint_as_float((__float_as_uint(out[i]) & 0xFFFF0000u) | 0x8000u);
          dbits |= (fabsf(out[i] - mid) <= bound ? 1u : 0u) << i;
        }
      }
    }
    if (active) Row::store(yrow + (int64_t)tt * p.C, out);
    if constexpr (kCheck) {
      if (active && dbits) {  // rare: queue (token, channel) for the fp64 pass
        // entry = channel within the launch << 10 | history rows << 8 | token within the run
        const uint32_t nq = (uint32_t)__popc(dbits);
        uint32_t pos = atomicAdd(qcount, nq);
        const uint32_t tag = ((uint32_t)hist << 8) | (uint32_t)(ts + tt - tw0);
        while (dbits) {
          const int i = __builtin_ctz(dbits);
          dbits &= dbits - 1;
          if (pos < CONV_QCAP)
            queue[pos] = ((uint32_t)(c0 + i - p.c_begin) << 10) | tag;
          else  // queue full: this lane settles its whole run at the end
            overflow = true;
          ++pos;
        }
      }
    }
    // one token at a time: keeps the scheduler from interleaving tokens,
    // which would unpack every row at once and run out of registers
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T, int kMode, bool kSilu>
__device__ __forceinline__ void conv1d_run(const T* __restrict__ x, const T* __restrict__ w,
                                           const T* __restrict__ bias, T* __restrict__ y, const ConvParams& p) {
  using Row = ConvRow<T>;
  constexpr int SUB = Row::SUB;
  constexpr int NCH = CONV_CH_PER_THREAD;
  __shared__ uint32_t s_queue[CONV_THREADS / 64][CONV_QCAP];
  __shared__ uint32_t s_qcount[CONV_THREADS / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c0 = p.c_begin + (blockIdx.x * CONV_THREADS + threadIdx.x) * NCH;
  const bool active = c0 < p.c_end;
  const int cl = active ? c0 : p.c_begin;  // an inactive lane reads a valid segment
  const int64_t tw0 = (int64_t)blockIdx.y * p.tile_tokens;
  const int64_t tw1 = tw0 + p.tile_tokens < p.Ttot ? tw0 + p.tile_tokens : p.Ttot;
  const int64_t C = p.C;
  if (lane == 0) s_qcount[wave] = 0;

  // ---- history rows and the first sub-tile, in flight before anything else --------
  typename Row::raw_t hraw[3], bufA[SUB], bufB[SUB];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int64_t r = tw0 - 3 + i;
    hraw[i] = Row::load(x + (r < 0 ? 0 : r) * C + cl);
  }
  auto load_sub = [&](typename Row::raw_t(&buf)[SUB], int64_t ts) {
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
      // rows past the run re-read its last row (a cache hit), not the next run's
      const int64_t r = ts + i < tw1 ? ts + i : tw1 - 1;
      buf[i] = Row::load(x + r * C + cl);
    }
  };
  load_sub(bufA, tw0);

  // ---- taps aligned so that tap 3 multiplies the current token --------------------
  float wt[4][NCH], bs[NCH];
  if (sizeof(T) == 2 && p.width == 4) {  // 8 channels x 4 taps = 64 contiguous bytes
    const uint16_t* wp = reinterpret_cast<const uint16_t*>(w) + (int64_t)cl * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(wp + 8 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // word e of vector q: channel 2q + e/2, taps 2(e%2), 2(e%2)+1
        const int ch = 2 * q + (e >> 1), tap = 2 * (e & 1);
        wt[tap][ch] = __uint_as_float(v[e] << 16);
        wt[tap + 1][ch] = __uint_as_float(v[e] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src = j - (4 - p.width);
        wt[j][i] = src >= 0 ? Row::scalar(w, (int64_t)(cl + i) * p.width + src) : 0.f;
      }
  }
  if (sizeof(T) == 2 && bias) {
    float tmp[NCH];
    ConvRow<uint16_t>::unpack(*reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(bias) + cl), tmp);
#pragma unroll
    for (int i = 0; i < NCH; ++i) bs[i] = tmp[i];
  } else {
#pragma unroll
    for (int i = 0; i < NCH; ++i) bs[i] = bias ? Row::scalar(bias, cl + i) : 0.f;
  }

  // |taps| and |bias| scaled by 9 * 2^-24 for the rounding check's bound
  float wa[4][NCH], ba[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    ba[i] = fabsf(bs[i]) * (9.f * 0x1p-24f);
#pragma unroll
    for (int j = 0; j < 4; ++j) wa[j][i] = fabsf(wt[j][i]) * (9.f * 0x1p-24f);
  }

  // ---- region (sample / batch row) of the first token ----------------------------
  int n = 0;
  int64_t s_start, s_end;
  if (p.cu && p.n_seqs < 64) {
    // one load of every offset across the wave instead of a chain of
    // dependent loads: the sample is the last n with cu[n] <= tw0
    const int li = lane < p.n_seqs ? lane : p.n_seqs;
    const int cl_ = (int)clampi(p.cu[li], 0, p.Ttot);
    const uint64_t m = __ballot(lane < p.n_seqs && cl_ <= tw0);
    n = m ? 63 - __builtin_clzll(m) : 0;
    s_start = __builtin_amdgcn_readfirstlane(__shfl(cl_, n, 64));
    const int64_t e_ = __builtin_amdgcn_readfirstlane(__shfl(cl_, n + 1, 64));
    s_end = e_ > s_start ? e_ : s_start;
  } else if (p.cu) {
    n = find_sample(p.cu, p.n_seqs, tw0, p.Ttot);
    s_start = clampi(p.cu[n], 0, p.Ttot);
    s_end = clampi(p.cu[n + 1], s_start, p.Ttot);
  } else {
    s_start = (tw0 / p.row_len) * p.row_len;
    s_end = s_start + p.row_len;
  }
  float h1[NCH], h2[NCH], h3[NCH];  // x[t-3], x[t-2], x[t-1]
  Row::unpack(hraw[0], h1);
  Row::unpack(hraw[1], h2);
  Row::unpack(hraw[2], h3);

  // Uniform walk over the sub-tile at ts: 2-bit history counts per token, and
  // whether anything needs masking.
  auto walk = [&](int64_t ts, uint32_t& code) -> bool {
    const int64_t te = ts + SUB < tw1 ? ts + SUB : tw1;
    if (te == ts + SUB && te <= s_end && ts - s_start >= 3) {
      code = 0xFFFFFFFFu;
      return false;
    }
    code = 0;
    for (int64_t t = ts; t < te; ++t) {
      while (t >= s_end) {  // the next region starts at or before t
        if (p.cu && n + 1 < p.n_seqs) {
          ++n;
          s_start = s_end;
          s_end = clampi(p.cu[n + 1], s_start, p.Ttot);
        } else if (p.cu) {  // tokens past the last offset form one trailing region
          s_start = s_end;
          s_end = p.Ttot;
        } else {
          s_start = s_end;
          s_end = s_start + p.row_len;
        }
      }
      const int64_t back = t - s_start;
      code |= (uint32_t)(back < 3 ? back : 3) << (2 * (t - ts));
    }
    return true;
  };

  uint32_t* queue = s_queue[wave];
  uint32_t* qcount = &s_qcount[wave];
  bool overflow = false;
#define GDN_CONV_SUB(BUF, TS)                                                                          \
  do {                                                                                                 \
    uint32_t code_;                                                                                    \
    const bool masked_ = walk((TS), code_);                                                            \
    const int nv_ = (int)((TS) + SUB < tw1 ? SUB : tw1 - (TS));                                        \
    T* yrow_ = y + (TS) * C + c0;                                                                      \
    if (masked_)                                                                                       \
      conv_sub<T, kMode, true, kSilu>(BUF, h1, h2, h3, wt, bs, wa, ba, nv_, code_, p, active, yrow_, queue,   \
                               qcount, (TS), tw0, c0, overflow);                                       \
    else                                                                                               \
      conv_sub<T, kMode, false, kSilu>(BUF, h1, h2, h3, wt, bs, wa, ba, nv_, code_, p, active, yrow_, queue,  \
                                qcount, (TS), tw0, c0, overflow);                                      \
  } while (0)
  for (int64_t ts = tw0; ts < tw1; ts += 2 * SUB) {
    load_sub(bufB, ts + SUB);
    GDN_CONV_SUB(bufA, ts);
    if (ts + SUB >= tw1) break;
    load_sub(bufA, ts + 2 * SUB);
    GDN_CONV_SUB(bufB, ts + SUB);
  }
#undef GDN_CONV_SUB

  // ---- settle the queued roundings in fp64 -----------------------------------------
  if constexpr (kMode == 3 && sizeof(T) == 2) {
    // normalised outputs: each queued value is recomputed with its whole head
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const uint32_t nq = min(*qcount, (uint32_t)CONV_QCAP);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    const uint16_t* wb = reinterpret_cast<const uint16_t*>(w);
    const uint16_t* bb = reinterpret_cast<const uint16_t*>(bias);
    uint16_t* yb = reinterpret_cast<uint16_t*>(y);
    const int head_dim = CONV_CH_PER_THREAD << p.l2_lanes_log2;
    for (uint32_t e = lane; e < nq; e += 64) {
      const uint32_t v = queue[e];
      const int64_t t = tw0 + (int64_t)(v & 0xFFu);
      const int64_t c = p.c_begin + (int64_t)(v >> 10);
      if (t < tw1 && c < p.c_end)
        settle_l2_value(xb, wb, bb, yb, C, p.width, kSilu ? 1 : 0, head_dim, (double)p.l2_eps, t, c,
                        (int)((v >> 8) & 3u));
    }
    if (overflow && active) {  // more doubtful values than the queue holds: redo the run in fp64
      for (int64_t t = tw0; t < tw1; ++t) {
        const int64_t back = t - region_start(p.cu, p.n_seqs, p.row_len, p.Ttot, t);
        for (int i = 0; i < NCH; ++i)
          settle_l2_value(xb, wb, bb, yb, C, p.width, kSilu ? 1 : 0, head_dim, (double)p.l2_eps, t, c0 + i,
                          back < 3 ? (int)back : 3);
      }
    }
  }
  if constexpr (kMode == 1 && sizeof(T) == 2) {
    // the queue and this wave's stores above are complete before any lane
    // reads the queue or overwrites a value another lane stored
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // A lane takes entries lane, lane + 64, ...: every load of all of them is
    // issued first (one memory round trip; unused slots read a valid
    // address), then each value is recomputed in fp64 and stored.
    const uint32_t nq = min(*qcount, (uint32_t)CONV_QCAP);
    constexpr int SE = CONV_QCAP / 64;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    const uint16_t* wb = reinterpret_cast<const uint16_t*>(w);
    const uint16_t* bb = reinterpret_cast<const uint16_t*>(bias);
    bool eok[SE];
    int64_t et[SE], ec[SE];
    int eh[SE];
    uint16_t xv[SE][4], wv[SE][4], bv[SE];
#pragma unroll
    for (int k = 0; k < SE; ++k) {
      const uint32_t e = lane + 64u * k;
      const uint32_t v = queue[e < nq ? e : 0];
      const int64_t t = tw0 + (int64_t)(v & 0xFFu);
      const int64_t c = p.c_begin + (int64_t)(v >> 10);
      eok[k] = e < nq && t < tw1 && c < p.c_end;  // entries come from active lanes only
      et[k] = eok[k] ? t : tw0;
      ec[k] = eok[k] ? c : p.c_begin;
      eh[k] = (int)((v >> 8) & 3u);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int jj = j < p.width ? j : p.width - 1;
        const int64_t r = et[k] - (p.width - 1 - jj);  // tap jj multiplies x[t - (width - 1 - jj)]
        xv[k][j] = xb[(r < 0 ? 0 : r) * C + ec[k]];
        wv[k][j] = wb[ec[k] * p.width + jj];
      }
      bv[k] = bb ? bb[ec[k]] : (uint16_t)0;
    }
#pragma unroll
    for (int k = 0; k < SE; ++k) {
      if (!eok[k]) continue;
      double z = (double)bf16_bits_to_f32(bv[k]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < p.width && p.width - 1 - j <= eh[k])
          z += (double)bf16_bits_to_f32(wv[k][j]) * (double)bf16_bits_to_f32(xv[k][j]);
      const double val = p.apply_silu ? z / (1.0 + exp(-z)) : z;
      reinterpret_cast<uint16_t*>(y)[et[k] * C + ec[k]] = f32_to_bf16_bits(bf16_nearest_f64(val));
    }
    if (overflow && active) {  // more doubtful values than the queue holds: redo the run in fp64
      for (int64_t t = tw0; t < tw1; ++t) {
        const int64_t back = t - region_start(p.cu, p.n_seqs, p.row_len, p.Ttot, t);
        for (int i = 0; i < NCH; ++i)
          settle_value(reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(w),
                       reinterpret_cast<const uint16_t*>(bias), reinterpret_cast<uint16_t*>(y), C, p.width,
                       p.apply_silu, t, c0 + i, back < 3 ? (int)back : 3);
      }
    }
  }
}

// Blocks below l2_end run the normalised channels, the others the plain ones
// (with the rounding check for bf16 when kExact); every block lies on one side.
template <typename T, bool kExact>
__global__ void __launch_bounds__(CONV_THREADS) conv1d_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                              const T* __restrict__ bias, T* __restrict__ y,
                                                              ConvParams p) {
  constexpr int kPlain = (kExact && sizeof(T) == 2) ? 1 : 0;
  constexpr int kNorm = (kExact && sizeof(T) == 2) ? 3 : 2;
  const bool l2 = p.c_begin + (int)blockIdx.x * CONV_THREADS * CONV_CH_PER_THREAD < p.l2_end;
  if (p.apply_silu) {
    if (l2)
      conv1d_run<T, kNorm, true>(x, w, bias, y, p);
    else
      conv1d_run<T, kPlain, true>(x, w, bias, y, p);
  } else {
    if (l2)
      conv1d_run<T, kNorm, false>(x, w, bias, y, p);
    else
      conv1d_run<T, kPlain, false>(x, w, bias, y, p);
  }
}

hipError_t launch_conv1d(const void* x, const void* w, const void* bias, int dt,
                         const int32_t* cu, int n_seqs, int B, int64_t T, int C, int width,
                         int apply_silu, int l2_channels, int head_dim, float l2_eps, int exact, void* y,
                         hipStream_t stream) {
  const int64_t Ttot = cu ? T : (int64_t)B * T;
  if (Ttot == 0 || C == 0) return hipSuccess;
  const int per_block = CONV_THREADS * CONV_CH_PER_THREAD;
  int lanes_log2 = 0;
  if (l2_channels > 0)
    while ((CONV_CH_PER_THREAD << lanes_log2) < head_dim) ++lanes_log2;
  ConvParams p;
  p.cu = cu;
  p.n_seqs = n_seqs;
  p.row_len = cu ? Ttot : T;
  p.Ttot = Ttot;
  p.C = C;
  p.width = width;
  p.apply_silu = apply_silu;
  p.l2_lanes_log2 = lanes_log2;
  p.l2_eps = l2_eps;
  const int sub = dt == 1 ? ConvRow<uint16_t>::SUB : ConvRow<float>::SUB;
  p.l2_end = l2_channels;
  // One launch when the normalised channels end on a block boundary,
  // otherwise one launch on each side of that boundary.
  const bool split = l2_channels % per_block != 0;
  for (int part = 0; part < (split ? 2 : 1); ++part) {
    p.c_begin = split && part == 1 ? l2_channels : 0;
    p.c_end = split && part == 0 ? l2_channels : C;
    if (p.c_end <= p.c_begin) continue;
    const int cblocks = (p.c_end - p.c_begin + per_block - 1) / per_block;
    // runs of 2-8 sub-tiles per block, aiming at about GDN_CONV_BLOCKS blocks;
    // a run of 8 bf16 sub-tiles gives a wave 32K values, about 120 of which
    // (well below CONV_QCAP) are queued for fp64 on data like the layer's
    const int64_t subs = (Ttot + sub - 1) / sub;
    int64_t per = (subs * cblocks + GDN_CONV_BLOCKS - 1) / GDN_CONV_BLOCKS;
    per = per < 2 ? 2 : (per > 8 ? 8 : per);
    const int64_t per_min = (subs + 65534) / 65535;  // grid y stays within 65535
    if (per < per_min) per = per_min;
    p.tile_tokens = (int)(per * sub);
    // queued bf16 roundings name their token within the run in 8 bits and
    // their channel within the launch in 22
    if (dt == 1 && (p.tile_tokens > 256 || p.c_end - p.c_begin > (1 << 22))) return hipErrorInvalidValue;
    const dim3 grid((unsigned)cblocks, (unsigned)((Ttot + p.tile_tokens - 1) / p.tile_tokens));
    if (dt == 1 && exact)
      hipLaunchKernelGGL((conv1d_kernel<uint16_t, true>), grid, dim3(CONV_THREADS), 0, stream, (const uint16_t*)x,
                         (const uint16_t*)w, (const uint16_t*)bias, (uint16_t*)y, p);
    else if (dt == 1)
      hipLaunchKernelGGL((conv1d_kernel<uint16_t, false>), grid, dim3(CONV_THREADS), 0, stream, (const uint16_t*)x,
                         (const uint16_t*)w, (const uint16_t*)bias, (uint16_t*)y, p);
    else
      hipLaunchKernelGGL((conv1d_kernel<float, false>), grid, dim3(CONV_THREADS), 0, stream, (const float*)x,
                         (const float*)w, (const float*)bias, (float*)y, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
