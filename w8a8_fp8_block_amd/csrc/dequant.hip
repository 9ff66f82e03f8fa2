// FP8 e4m3 weights [N,K] -> bf16 [N,K] for gfx950 (page "dispatch_proj.rs",
// doc of dequant_fp8_bf16_into): dst[n,k] = bf16(fl32(dec(w[n,k]) * s)),
// s = scale[(n/block_n)*sk + k/block_k], one formula for both weight
// formats: (128, 128, K/128) for 128x128 block scales, (1, K, 1) per row.
//
// HBM-bound stream (1 byte read, 2 written per element): each thread takes
// 16 consecutive codes of one row (one 16-byte load, 16 codes inside one
// 128-wide scale block since 16 divides 128), decodes them with the
// hardware OCP e4m3 -> fp32 conversion (exact), multiplies by the fp32
// scale (one IEEE rounding) and rounds to bf16 (nearest even), two 16-byte
// stores.  Grid-stride over the N*K/16 chunks.
#include "fp8q_internal.h"

namespace fp8q {
namespace {

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// four codes (one dword) -> two dwords of bf16 pairs, scaled
__device__ __forceinline__ u32x2 dequant4(uint32_t c, float s) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false);  // bytes 0, 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c, true);   // bytes 2, 3
  return u32x2{bf16_bits(lo[0] * s) | (bf16_bits(lo[1] * s) << 16),
               bf16_bits(hi[0] * s) | (bf16_bits(hi[1] * s) << 16)};
}

__global__ __launch_bounds__(256) void dequant_kernel(const u32x4* __restrict__ w,
                                                      const float* __restrict__ scale,
                                                      u32x4* __restrict__ dst, uint64_t chunks,
                                                      uint32_t cpr, uint32_t K, uint32_t per_row) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks; i += stride) {
    const uint32_t n = (uint32_t)(i / cpr), k0 = (uint32_t)(i % cpr) * 16;
    const float s = per_row ? scale[n] : scale[(uint64_t)(n / kGroup) * (K / kGroup) + k0 / kGroup];
    const u32x4 c = __builtin_nontemporal_load(&w[i]);
    const u32x2 a = dequant4(c.x, s), b = dequant4(c.y, s), d = dequant4(c.z, s), e = dequant4(c.w, s);
    dst[2 * i] = u32x4{a.x, a.y, b.x, b.y};
    dst[2 * i + 1] = u32x4{d.x, d.y, e.x, e.y};
  }
}

}  // namespace

hipError_t launch_dequant(const uint8_t* w, const float* scale, uint16_t* dst, uint32_t N,
                          uint32_t K, bool per_row, hipStream_t s) {
  const uint64_t chunks = (uint64_t)N * K / 16;
  const uint64_t want = (chunks + 255) / 256;
  const uint32_t grid = (uint32_t)(want < 8192 ? want : 8192);
  dequant_kernel<<<dim3(grid), dim3(256), 0, s>>>(
      reinterpret_cast<const u32x4*>(w), scale, reinterpret_cast<u32x4*>(dst), chunks, K / 16, K,
      per_row ? 1u : 0u);
  return hipGetLastError();
}

}  // namespace fp8q
