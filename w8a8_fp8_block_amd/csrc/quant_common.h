// Per-group FP8 e4m3 quantization (one scale per 128 bf16 values, the codes
// of x / scale) and the dense FFN's SiLU * up, shared by the activation
// quantizer (quant.hip), the FFN intermediate quantizer (ffn.hip) and the
// fused gate/up GEMM epilogue (gemm.hip), so that every path takes the same
// decisions in the same arithmetic.  The method and the exactness argument
// of the division are described in quant.hip.
#pragma once

#include "fp8q_internal.h"

namespace fp8q {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t dpp_row_max_u32(uint32_t v) {
  // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror:
  // after the four steps every lane of the 16-lane row holds the row max.
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return v;
}

// The same over the 8-lane halves of each row: quad_perm [1,0,3,2],
// quad_perm [2,3,0,1], row_half_mirror.
__device__ __forceinline__ uint32_t dpp_half_row_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ u16x2 as_u16x2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }

// bf16 pair in one dword -> two floats (exact)
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// q[i] = fl32(x[i] / s), the correctly rounded quotient, for N values that
// share the scale s (see quant.hip for why the reciprocal form is exact when
// s >= 2^-100); a zero scale (all-zero group) keeps the signed zeros.  The
// choice of method is uniform over the wave, and both give the same result.
template <int N>
__device__ __forceinline__ void quotients(const float* x, float s, float* q) {
  const bool slow = !(s >= 0x1p-100f);  // zero or tiny scale
  if (__builtin_amdgcn_ballot_w64(slow) == 0) {
    // r = fl32(1/s): the hardware reciprocal (within 1 ulp) and one
    // Newton-Raphson step with fmas, r = r0 + r0*(1 - s*r0).  From any start
    // within one ulp of the correctly rounded reciprocal the step lands on
    // it, for every scale >= 2^-100 that a bf16 group maximum can produce.
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      // en = q0*s - x is the negated residual; q1 = q0 - en*r.  Written this
      // way round, x = -0 gives en = +0 and q1 = -0 + -0 = -0, keeping the sign
      // (the residual x - q0*s would be +0 and turn q1 into +0).
      const float q0 = x[i] * r;
      const float en = __builtin_fmaf(q0, s, -x[i]);
      q[i] = __builtin_fmaf(-en, r, q0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) q[i] = (s == 0.0f) ? x[i] : x[i] / s;
  }
}

// Four quotients -> four e4m3 codes (little-endian bytes in element order):
// the hardware conversion, round to nearest even.  No clamp is needed: with
// |x| <= amax and s = fl32(amax/448), |x/s| is at most 448 plus one fp32 ulp,
// which the conversion rounds to 448 (every (x, amax) pair is checked on the
// device against the oracle's clamp-then-round).
__device__ __forceinline__ uint32_t encode4(const float* q) {
  int c = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false);
  c = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], c, true);
  return (uint32_t)c;
}

// Scale of a group from the bit pattern of its bf16 magnitude maximum.
// fl32(a/448) without a divide: q0 = a*k with k = fl32(1/448), then one
// fma correction, q0 - (q0*448 - a)*k.  Equal to the correctly rounded
// quotient for every finite bf16 magnitude a, subnormal results included
// (all 32640 of them checked); a non-finite maximum keeps a/448 = a.
__device__ __forceinline__ float group_scale(uint32_t amax_bits) {
  const float a = __uint_as_float(amax_bits << 16);
  constexpr float k = 1.0f / 448.0f;
  const float q0 = a * k;
  const float s = __builtin_fmaf(-__builtin_fmaf(q0, 448.0f, -a), k, q0);
  return amax_bits >= 0x7F80u ? a : s;
}

// Quantize the group held by this lane's 16-lane row.  v = this lane's 8 bf16;
// returns the 8 codes (little-endian bytes in element order) and the scale.
__device__ __forceinline__ u32x2 quant_group(u32x4 v, float& scale_out) {
  const uint32_t mag = 0x7FFF7FFFu;
  u16x2 m01 = __builtin_elementwise_max(as_u16x2(v.x & mag), as_u16x2(v.y & mag));
  u16x2 m23 = __builtin_elementwise_max(as_u16x2(v.z & mag), as_u16x2(v.w & mag));
  u16x2 mm = __builtin_elementwise_max(m01, m23);
  uint32_t amax_bits = max((uint32_t)mm.x, (uint32_t)mm.y);
  amax_bits = dpp_row_max_u32(amax_bits);
  const float s = group_scale(amax_bits);
  scale_out = s;

  float x[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
  float q[8];
  quotients<8>(x, s, q);
  return u32x2{encode4(q), encode4(q + 4)};
}

// ---- the dense FFN's intermediate h = bf16(silu(gate) * up) ----
// e^x = 2^(x log2 e) for -110 <= x <= 64: the hardware exp2 (1 ulp) of the rounded
// product x*L, times 2^r for the product's rounding residual r (exact by an
// fma, plus the tail of log2 e), 2^r ~ 1 + r ln 2 with |r| < 2^-17: about
// 2 ulps in all, where the exp2 of the rounded product alone would be off by
// up to |x| * 2^-24 relative.  Results below 2^-126 may be flushed; they
// only arise for silu values far below the smallest bf16.
__device__ __forceinline__ float exp_f32(float x) {
  const float L = 1.44269502e+00f, Ltail = 1.92596299e-08f;  // log2(e) = L + Ltail
  const float ph = x * L;
  const float r = __builtin_fmaf(x, Ltail, __builtin_fmaf(x, L, -ph));
  const float e = __builtin_amdgcn_exp2f(ph);
  return __builtin_fmaf(e, r * 0.693147182f, e);
}

// silu(g) = g / (1 + e^-g) in binary32: silu = g * rcp(1 + e^-g), times up,
// a few ulps of binary32 in all.  Below g = -64 the form g * e^(g+64) * e^-64
// keeps every intermediate finite (e^-g overflows binary32 below about
// -88.7); g + 64 is exact there.  The exponent is clamped at -110, where e^x
// is already below the smallest binary32 (so huge |g| cannot overflow x*L).
__device__ __forceinline__ float silu_mul_f32(float g, float u) {
  const bool deep = g < -64.0f;
  const float t = exp_f32(fmaxf(deep ? g + 64.0f : -g, -110.0f));  // one exp per element
  const float s = deep ? (g * t) * 1.60381089e-28f /* e^-64 */ : g * __builtin_amdgcn_rcpf(1.0f + t);
  return s * u;
}

// fp32 -> bf16 bit pattern, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace
}  // namespace fp8q
