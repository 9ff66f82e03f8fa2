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

// One 16-lane row per group of 128 (gate, up) pairs, kSiluRounds groups per
// row with all loads issued first.  Gate and up are read once
// (non-temporal); the codes and scales are left in the caches for the down
// projection that reads them next.
constexpr uint32_t kSiluWaves = 4, kSiluRounds = 2;
constexpr uint32_t kSiluGroupsPerWg = 4 * kSiluWaves * kSiluRounds;

__global__ __launch_bounds__(64 * kSiluWaves) void silu_mul_quant_kernel(
    const u32x4* __restrict__ g, const u32x4* __restrict__ u, u32x2* __restrict__ q,
    float* __restrict__ skm, uint64_t ngroups, uint32_t G, uint32_t Mp) {
  const uint64_t g0 =
      ((uint64_t)blockIdx.x * (kSiluGroupsPerWg / kSiluRounds) + (threadIdx.x >> 4)) * kSiluRounds;
  const uint32_t l = threadIdx.x & 15;
  u32x4 gv[kSiluRounds], uv[kSiluRounds];
#pragma unroll
  for (uint32_t r = 0; r < kSiluRounds; ++r) {
    if (g0 + r < ngroups) {
      gv[r] = __builtin_nontemporal_load(&g[(g0 + r) * 16 + l]);
      uv[r] = __builtin_nontemporal_load(&u[(g0 + r) * 16 + l]);
    }
  }
#pragma unroll
  for (uint32_t r = 0; r < kSiluRounds; ++r) {
    if (g0 + r < ngroups) {  // uniform over the 16-lane row
      float s;
      const u32x2 c = quant_group(silu_mul_8(gv[r], uv[r]), s);
      q[(g0 + r) * 16 + l] = c;
      if (l == 0) {
        const uint64_t gi = g0 + r;
        skm[(gi % G) * Mp + gi / G] = s;
      }
    }
  }
}

}  // namespace

hipError_t launch_silu_mul_quant(const uint16_t* gate, const uint16_t* up, uint8_t* q,
                                 float* scale_km, uint32_t M, uint32_t I, hipStream_t s) {
  const uint32_t G = I / kGroup;
  const uint64_t ngroups = (uint64_t)M * G;
  const uint64_t grid = (ngroups + kSiluGroupsPerWg - 1) / kSiluGroupsPerWg;
  silu_mul_quant_kernel<<<dim3((uint32_t)grid), dim3(64 * kSiluWaves), 0, s>>>(
      reinterpret_cast<const u32x4*>(gate), reinterpret_cast<const u32x4*>(up),
      reinterpret_cast<u32x2*>(q), scale_km, ngroups, G, m_pad16(M));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_kmajor_pad(scale_km, M, I, s);
}

}  // namespace fp8q
