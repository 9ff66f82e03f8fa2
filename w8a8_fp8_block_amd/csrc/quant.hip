// Per-(token, 128-group) FP8 e4m3 activation quantizer for gfx950.
//
// Method (page "dispatch_proj.rs", doc of cublas_fp8_proj; page
// "fp8_act_quant_floor.rs" for the two launch shapes): for every group of 128
// consecutive K elements of a token row, scale = fl32(amax / 448) and each
// element becomes the OCP e4m3fn code of x / scale (round to nearest even,
// saturating at +-448).  The input is a flat sequence of M*(K/128) groups of
// 128 bf16, so group i lives at x + 128*i, its codes at q + 128*i and its
// row-major scale at scale_rm[i].
//
// Work split: variant A gives each group 8 lanes of a wave, 16 values per
// lane (two 128-bit loads, two 64-bit stores), variant B one 16-lane DPP row,
// 8 values per lane.  The group maximum is an integer max over bf16
// magnitudes (packed u16 max, then a DPP butterfly inside the 8 or 16
// lanes), which is exact and needs no float canonicalization.  The scale
// amax/448 and its reciprocal take no divide (quant_common.h), so the vector
// ALU work per value is the unpack, three fp32 operations and half a packed
// conversion: at prefill sizes the kernel then runs close to a pure stream
// with the same access pattern.
//
// Exactness of q = fl32(x / scale) without a divide per element: with
// r = fl32(1 / scale) (correctly rounded, once per group),
//   q0 = x * r,  en = fma(q0, scale, -x),  q1 = fma(-en, r, q0)
// is the correctly rounded quotient, signed zeros included, for every bf16
// pair (x, amax) whose scale is at least 2^-100; groups with a smaller (or
// zero) scale take an exact per-element divide instead.  The e4m3 code is
// the hardware conversion of q1, which rounds the largest quotients (448 and
// at most one fp32 ulp above) to 448 just as the pages' clamp to +-448 does.
// The exhaustive (x, amax) test checks the whole map on the device.
#include "quant_common.h"

namespace fp8q {
namespace {

// Scale of group g in the row-major layout and/or the K-major one; the
// groups of the last token row also clear their K-major column's pad slots
// M..Mp-1, so the K-major layout needs no separate pad pass.
__device__ __forceinline__ void write_scales(float s, uint64_t g, float* __restrict__ srm,
                                             float* __restrict__ skm, uint32_t M, uint32_t G,
                                             uint32_t Mp) {
  if (srm) srm[g] = s;
  if (skm) {
    // g < M*K/128 < 2^25 (Mp*K < 2^32 is checked on the host): 32-bit divide
    const uint32_t g32 = (uint32_t)g, m = g32 / G, gg = g32 % G;
    float* col = skm + (uint64_t)gg * Mp;
    col[m] = s;
    if (m + 1 == M)
      for (uint32_t p = M; p < Mp; ++p) col[p] = 0.0f;
  }
}

// Variant A (fine-grained): 8 lanes per group, lane l holding elements
// 8l..8l+7 and 64+8l..64+8l+7 (each of the two loads covers the group's 256
// bytes contiguously across its 8 lanes).  Against 16 lanes of 8 values this
// halves the per-group work per value (butterfly, scale, reciprocal,
// addresses) at the same bytes in flight per lane.  The codes, which nothing
// reads back soon, are stored non-temporally.  Quantizes group g (this
// lane's share) and returns its scale.
__device__ __forceinline__ float quant_group_a(const u32x4* __restrict__ x, u32x2* __restrict__ q,
                                               uint64_t g, uint32_t l) {
  const u32x4 v0 = __builtin_nontemporal_load(&x[g * 16 + l]);
  const u32x4 v1 = __builtin_nontemporal_load(&x[g * 16 + 8 + l]);
  const uint32_t mag = 0x7FFF7FFFu;
  const u16x2 m0 = __builtin_elementwise_max(as_u16x2(v0.x & mag), as_u16x2(v0.y & mag));
  const u16x2 m1 = __builtin_elementwise_max(as_u16x2(v0.z & mag), as_u16x2(v0.w & mag));
  const u16x2 m2 = __builtin_elementwise_max(as_u16x2(v1.x & mag), as_u16x2(v1.y & mag));
  const u16x2 m3 = __builtin_elementwise_max(as_u16x2(v1.z & mag), as_u16x2(v1.w & mag));
  const u16x2 mm = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                             __builtin_elementwise_max(m2, m3));
  const uint32_t amax = dpp_half_row_max_u32(max((uint32_t)mm.x, (uint32_t)mm.y));
  const float s = group_scale(amax);
  const float xv[16] = {bf_lo(v0.x), bf_hi(v0.x), bf_lo(v0.y), bf_hi(v0.y), bf_lo(v0.z),
                        bf_hi(v0.z), bf_lo(v0.w), bf_hi(v0.w), bf_lo(v1.x), bf_hi(v1.x),
                        bf_lo(v1.y), bf_hi(v1.y), bf_lo(v1.z), bf_hi(v1.z), bf_lo(v1.w),
                        bf_hi(v1.w)};
  float qv[16];
  quotients<16>(xv, s, qv);
  __builtin_nontemporal_store(u32x2{encode4(qv), encode4(qv + 4)}, &q[g * 16 + l]);
  __builtin_nontemporal_store(u32x2{encode4(qv + 8), encode4(qv + 12)}, &q[g * 16 + 8 + l]);
  return s;
}

// Flat over the M*(K/128) groups, kQuantAGroupsPerWg consecutive groups per
// workgroup; the K-major scales too where skm is given (4-byte stores
// strided by Mp, cheap up to kQuantTileMinGroups groups).
__global__ __launch_bounds__(64 * kQuantAWaves) void quant_a_kernel(
    const u32x4* __restrict__ x, u32x2* __restrict__ q, float* __restrict__ srm,
    float* __restrict__ skm, uint64_t ngroups, uint32_t M, uint32_t G, uint32_t Mp) {
  const uint64_t g = (uint64_t)blockIdx.x * kQuantAGroupsPerWg + (threadIdx.x >> 3);
  const uint32_t l = threadIdx.x & 7;
  if (g >= ngroups) return;  // uniform over the group's 8 lanes
  const float s = quant_group_a(x, q, g, l);
  if (l == 0) write_scales(s, g, srm, skm, M, G, Mp);
}

// With the K-major scales beyond kQuantTileMinGroups groups: the same
// per-group work, the groups dealt in
// tiles of kQuantTileRows token rows x kQuantTileGroups groups, one tile per
// workgroup, wave v taking row m0 + v (8 consecutive groups: 2 KB of
// contiguous input, as in the flat order).  The tile's 64 scales meet in
// LDS, and two waves store them: row-major as 8 runs of 8 and K-major as 8
// runs of 8, each run one whole 32-byte sector.  (Tiles without the
// staging, each wave taking one group column of the 8 rows, wrote the
// row-major scales 4 bytes at a time from different waves: 6-9% slower
// than the row-major quantizer plus the separate relayout from M = 4576,
// K = 17408 on.)  The row tiles run to Mp = ceil16(M), so that
// the K-major pad slots M .. Mp-1 are written (+0.0) by the same stores.
__global__ __launch_bounds__(64 * kQuantTileRows) void quant_a_tile_kernel(
    const u32x4* __restrict__ x, u32x2* __restrict__ q, float* __restrict__ srm,
    float* __restrict__ skm, uint32_t M, uint32_t G, uint32_t Mp, uint32_t gtiles) {
  __shared__ float ts[kQuantTileRows][kQuantTileGroups];
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l = lane & 7;
  const uint32_t m0 = (blockIdx.x / gtiles) * kQuantTileRows;
  const uint32_t g0 = (blockIdx.x % gtiles) * kQuantTileGroups;
  {
    const uint32_t m = m0 + wave, gg = g0 + (lane >> 3);
    if (m < M && gg < G) {  // uniform over the group's 8 lanes
      const float s = quant_group_a(x, q, (uint64_t)m * G + gg, l);
      if (l == 0) ts[wave][lane >> 3] = s;
    }
  }
  __syncthreads();
  if (wave == 0 && srm) {
    const uint32_t r = lane >> 3, c = lane & 7, m = m0 + r, gg = g0 + c;
    if (m < M && gg < G) srm[(uint64_t)m * G + gg] = ts[r][c];
  } else if (wave == 1) {
    const uint32_t c = lane >> 3, r = lane & 7, m = m0 + r, gg = g0 + c;
    if (m < Mp && gg < G) skm[(uint64_t)gg * Mp + m] = m < M ? ts[r][c] : 0.0f;
  }
}

// Variant B (K-grouped): workgroup (m, by) covers groups
// [by*kQuantBGroupsPerWg, ...) of token row m; each 16-lane row takes
// kQuantBRounds groups, all loads issued before any is consumed.
__global__ __launch_bounds__(64 * kQuantBWaves) void quant_b_kernel(
    const u32x4* __restrict__ x, u32x2* __restrict__ q, float* __restrict__ srm,
    float* __restrict__ skm, uint32_t M, uint32_t G, uint32_t Mp) {
  const uint32_t m = blockIdx.x;
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t g0 = blockIdx.y * kQuantBGroupsPerWg + wave * 4 * kQuantBRounds + (lane >> 4);
  u32x4 v[kQuantBRounds];
#pragma unroll
  for (uint32_t r = 0; r < kQuantBRounds; ++r) {
    const uint32_t gg = g0 + 4 * r;
    if (gg < G) v[r] = __builtin_nontemporal_load(&x[((uint64_t)m * G + gg) * 16 + (lane & 15)]);
  }
#pragma unroll
  for (uint32_t r = 0; r < kQuantBRounds; ++r) {
    const uint32_t gg = g0 + 4 * r;
    if (gg < G) {
      float s;
      const uint64_t g = (uint64_t)m * G + gg;
      const u32x2 c = quant_group(v[r], s);
      q[g * 16 + (lane & 15)] = c;
      if ((lane & 15) == 0) write_scales(s, g, srm, skm, M, G, Mp);
    }
  }
}

}  // namespace

hipError_t launch_quant_a(const uint16_t* x, uint8_t* q, float* scale_rm, float* scale_km,
                          uint32_t M, uint32_t K, hipStream_t s) {
  const uint32_t G = K / kGroup;
  const uint64_t ngroups = (uint64_t)M * G;
  if (scale_km && ngroups > kQuantTileMinGroups) {
    const uint32_t gtiles = (G + kQuantTileGroups - 1) / kQuantTileGroups;
    const uint64_t grid = (uint64_t)((m_pad16(M) + kQuantTileRows - 1) / kQuantTileRows) * gtiles;
    quant_a_tile_kernel<<<dim3((uint32_t)grid), dim3(64 * kQuantTileRows), 0, s>>>(
        reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x2*>(q), scale_rm, scale_km, M, G,
        m_pad16(M), gtiles);
    return hipGetLastError();
  }
  const uint64_t grid = (ngroups + kQuantAGroupsPerWg - 1) / kQuantAGroupsPerWg;
  quant_a_kernel<<<dim3((uint32_t)grid), dim3(64 * kQuantAWaves), 0, s>>>(
      reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x2*>(q), scale_rm, scale_km,
      ngroups, M, G, m_pad16(M));
  return hipGetLastError();
}

hipError_t launch_quant_b(const uint16_t* x, uint8_t* q, float* scale_rm, float* scale_km,
                          uint32_t M, uint32_t K, hipStream_t s) {
  const uint32_t G = K / kGroup;
  const uint32_t gy = (G + kQuantBGroupsPerWg - 1) / kQuantBGroupsPerWg;
  quant_b_kernel<<<dim3(M, gy), dim3(64 * kQuantBWaves), 0, s>>>(
      reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x2*>(q), scale_rm, scale_km, M, G,
      m_pad16(M));
  return hipGetLastError();
}

}  // namespace fp8q
