// The dense FFN's intermediate on gfx950: h = bf16(silu(gate) * up), then the
// per-(token, 128-group) FP8 quantization of h for the down projection, its
// scales written straight into the K-major layout the GEMM reads.
//
// Page "dispatch_proj.rs", doc of cublas_fp8_proj_prequant: the gate and up
// projections of the dense FFN read one quantized input, and the post-SiLU
// intermediate is quantized once for down.  silu(g) = g / (1 + e^-g); gate
// and up are the bf16 outputs of their projections, and h is rounded to
// bf16 before it is quantized (the quantizer's input format), so each stage
// keeps the format it has between separate kernels.
//
// SiLU * up and the quantization are the shared helpers of quant_common.h.
#include "quant_common.h"

namespace fp8q {
namespace {

// 8 (gate, up) bf16 pairs -> 8 bf16 h, packed like the inputs
__device__ __forceinline__ u32x4 silu_mul_8(u32x4 g, u32x4 u) {
  uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w}, hw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = silu_mul_f32(__uint_as_float(gw[i] << 16), __uint_as_float(uw[i] << 16));
    const float hi = silu_mul_f32(__uint_as_float(gw[i] & 0xFFFF0000u),
                                  __uint_as_float(uw[i] & 0xFFFF0000u));
    hw[i] = bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
  }
  return u32x4{hw[0], hw[1], hw[2], hw[3]};
}

// Eight lanes per group of 128 (gate, up) pairs, 16 pairs per lane:
// elements 8l..8l+7 and 64+8l..64+8l+7 of the group, as in the activation
// quantizer's flat variant (each 128-bit load covers 128 contiguous bytes
// across the 8 lanes).  Gate and up are read once (non-temporal); the codes
// and scales are left in the caches for the down projection that reads them
// next.  The K-major scale slot takes a 32-bit divide (M * I/128 < 2^32);
// the pad slots M..Mp-1 are written by the last row's groups.
constexpr uint32_t kSiluWaves = 4;
constexpr uint32_t kSiluGroupsPerWg = 8 * kSiluWaves;

__global__ __launch_bounds__(64 * kSiluWaves) void silu_mul_quant_kernel(
    const u32x4* __restrict__ g, const u32x4* __restrict__ u, u32x2* __restrict__ q,
    float* __restrict__ skm, uint32_t ngroups, uint32_t M, uint32_t G, uint32_t Mp) {
  const uint32_t gi = blockIdx.x * kSiluGroupsPerWg + (threadIdx.x >> 3);
  const uint32_t l = threadIdx.x & 7;
  if (gi >= ngroups) return;  // uniform over the group's 8 lanes
  const uint64_t base = (uint64_t)gi * 16;
  const u32x4 g0 = __builtin_nontemporal_load(&g[base + l]);
  const u32x4 g1 = __builtin_nontemporal_load(&g[base + 8 + l]);
  const u32x4 u0 = __builtin_nontemporal_load(&u[base + l]);
  const u32x4 u1 = __builtin_nontemporal_load(&u[base + 8 + l]);
  const u32x4 h0 = silu_mul_8(g0, u0), h1 = silu_mul_8(g1, u1);
  const uint32_t mag = 0x7FFF7FFFu;
  const u16x2 m0 = __builtin_elementwise_max(as_u16x2(h0.x & mag), as_u16x2(h0.y & mag));
  const u16x2 m1 = __builtin_elementwise_max(as_u16x2(h0.z & mag), as_u16x2(h0.w & mag));
  const u16x2 m2 = __builtin_elementwise_max(as_u16x2(h1.x & mag), as_u16x2(h1.y & mag));
  const u16x2 m3 = __builtin_elementwise_max(as_u16x2(h1.z & mag), as_u16x2(h1.w & mag));
  const u16x2 mm = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                             __builtin_elementwise_max(m2, m3));
  const uint32_t amax = dpp_half_row_max_u32(max((uint32_t)mm.x, (uint32_t)mm.y));
  const float sc = group_scale(amax);
  const float xv[16] = {bf_lo(h0.x), bf_hi(h0.x), bf_lo(h0.y), bf_hi(h0.y), bf_lo(h0.z),
                        bf_hi(h0.z), bf_lo(h0.w), bf_hi(h0.w), bf_lo(h1.x), bf_hi(h1.x),
                        bf_lo(h1.y), bf_hi(h1.y), bf_lo(h1.z), bf_hi(h1.z), bf_lo(h1.w),
                        bf_hi(h1.w)};
  float qv[16];
  quotients<16>(xv, sc, qv);
  q[base + l] = u32x2{encode4(qv), encode4(qv + 4)};
  q[base + 8 + l] = u32x2{encode4(qv + 8), encode4(qv + 12)};
  if (l == 0) {
    // the last token row's groups also clear their column's pad slots
    float* col = skm + (uint64_t)(gi % G) * Mp;
    const uint32_t m = gi / G;
    col[m] = sc;
    if (m + 1 == M)
      for (uint32_t p = M; p < Mp; ++p) col[p] = 0.0f;
  }
}

}  // namespace

hipError_t launch_silu_mul_quant(const uint16_t* gate, const uint16_t* up, uint8_t* q,
                                 float* scale_km, uint32_t M, uint32_t I, hipStream_t s) {
  const uint32_t G = I / kGroup;
  const uint32_t ngroups = M * G;  // M * I < 2^32 (checked by the caller)
  const uint32_t grid = (ngroups + kSiluGroupsPerWg - 1) / kSiluGroupsPerWg;
  silu_mul_quant_kernel<<<dim3(grid), dim3(64 * kSiluWaves), 0, s>>>(
      reinterpret_cast<const u32x4*>(gate), reinterpret_cast<const u32x4*>(up),
      reinterpret_cast<u32x2*>(q), scale_km, ngroups, M, G, m_pad16(M));
  return hipGetLastError();
}

}  // namespace fp8q
