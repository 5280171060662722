// device_common.h -- small device helpers shared by the gfx950 kernels.
//
// bf16 <-> fp32 conversion (round to nearest even), split of an fp32 value into
// a bf16 pair (hi + lo), and the MFMA fragment conventions used by the chunk
// kernels.
//
// MFMA v_mfma_f32_16x16x32_bf16 (wave64): lane l, c16 = l % 16, g4 = l / 16.
//   A (16 x 32, M x K): lane holds 8 values of row c16,
//   B (32 x 16, K x N): lane holds 8 values of column c16,
//   C/D (16 x 16):      lane holds rows 4*g4 + e (e = 0..3) of column c16.
// The K index carried by (g4, j) only has to agree between A and B.  These
// kernels use the "accumulator-compatible" assignment
//   j = 0..3 -> k = 4*g4 + j,   j = 4..7 -> k = 16 + 4*g4 + (j - 4),
// so that the accumulator tiles of one product (rows 4*g4+e of two vertically
// adjacent 16 x 16 tiles) are, register for register, the B operand of the
// next product along that row index -- no trip through LDS.  An operand read
// from a row-major LDS matrix under this assignment is two 8-byte reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// x ~= hi + lo with both in bf16; |x - hi - lo| <= 2^-16 |x| (about).
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (element 0 in the low half), round to nearest even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1) {
  const f32x2 v = {x0, x1};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Split two fp32 values into packed bf16 hi and lo words: x ~= hi + lo.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(x0, x1);
  const float r0 = x0 - __uint_as_float(hi << 16);
  const float r1 = x1 - __uint_as_float(hi & 0xFFFF0000u);
  lo = pack_bf16x2(r0, r1);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 as_bf16x8(u16x8 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// A/B fragment from a row-major bf16 LDS matrix (pitch in elements):
// row `row`, K columns k0 + {4*g4..4*g4+3} and k0 + 16 + {4*g4..4*g4+3}.
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base, int pitch, int row, int k0,
                                           int g4) {
  const uint16_t* p = base + row * pitch + k0 + 4 * g4;
  u16x4 a = *reinterpret_cast<const u16x4*>(p);
  u16x4 b = *reinterpret_cast<const u16x4*>(p + 16);
  u16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return as_bf16x8(r);
}

// Pack two accumulator tiles (4 floats each, rows 4*g4+e of tiles t0 and t1)
// into hi and lo B fragments.
__device__ __forceinline__ void split_frag(const f32x4& t0, const f32x4& t1, bf16x8& hi,
                                           bf16x8& lo) {
  uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
  split2(t0[0], t0[1], h0, l0);
  split2(t0[2], t0[3], h1, l1);
  split2(t1[0], t1[1], h2, l2);
  split2(t1[2], t1[3], h3, l3);
  const u32x4 h = {h0, h1, h2, h3};
  const u32x4 l = {l0, l1, l2, l3};
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// Sum over the 16 lanes of a DPP row (lanes 16j .. 16j + 15), the result in
// every lane: partners at distance 1 and 2 (quad permutes), then the two quads
// of each half-row (half-row mirror) and the two halves (row mirror).  Both
// partners of a step add the same two values, so the sum has the same bits as
// a butterfly over lane distances 1, 2, 4, 8.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false));  // row mirror
  return x;
}

// SiLU, z * sigmoid(z) = z / (1 + 2^(-z log2 e)), with the hardware base-2
// exponential and reciprocal (about 1 ulp each); infinities give 0 and z.
__device__ __forceinline__ float silu_hw(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// The short convolution's SiLU, z / (1 + e^-z) with the hardware reciprocal;
// the separate conv and the conv fused into the chunk prep share it, so that
// both store the same activations.
__device__ __forceinline__ float silu_conv(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// The gates of one (token, v-head): g = -e^{A_log} softplus(a + dt_bias),
// beta = sigmoid(b); the gate kernel and the kernels that form the gates
// from the raw inputs themselves share it, so both give the same values.
__device__ __forceinline__ void gate_values(float a, float b, float A_log, float dt_bias, float& g, float& beta) {
  const float x = a + dt_bias;
  const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
  g = -expf(A_log) * sp;
  beta = 1.f / (1.f + expf(-b));
}

template <int kCtrl>
__device__ __forceinline__ float dpp_add(float v) {
  const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false);
  return v + __int_as_float(o);
}

// Sum over aligned groups of 2^lanes_log2 lanes (uniform lanes_log2 <= 6).
__device__ __forceinline__ float group_sum(float v, int lanes_log2) {
  if (lanes_log2 >= 1) v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]: xor 1
  if (lanes_log2 >= 2) v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]: xor 2
  if (lanes_log2 >= 3) v = dpp_add<0x141>(v);  // half-row mirror: the other quad of 8
  if (lanes_log2 >= 4) v = dpp_add<0x140>(v);  // row mirror: the other half of 16
  if (lanes_log2 >= 5) v += __shfl_xor(v, 16, 64);
  if (lanes_log2 >= 6) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ int clampi(int64_t x, int64_t lo, int64_t hi) {
  return (int)(x < lo ? lo : (x > hi ? hi : x));
}

}  // namespace gdn
