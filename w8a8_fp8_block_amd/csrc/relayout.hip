// Activation-scale relayout [M, K/128] -> [K/128, Mp], Mp = ceil16(M), pad
// slots m in [M, Mp) set to +0.0 (page "dispatch_proj.rs",
// fp8_act_scale_to_kmajor and the scale-layout note on cublas_fp8_proj_prequant).
//
// A 64-token x 16-group tile is staged through LDS so that both the read
// (16 consecutive groups of a row) and the write (64 consecutive tokens of a
// group column) are contiguous.  Every output slot, pad included, is written
// by exactly one thread.
#include "fp8q_internal.h"

namespace fp8q {
namespace {

constexpr uint32_t kTm = 64, kTg = 16;

__global__ __launch_bounds__(256) void relayout_kernel(const float* __restrict__ rm,
                                                       float* __restrict__ km, uint32_t M,
                                                       uint32_t Mp, uint32_t G) {
  __shared__ float tile[kTg][kTm + 1];
  const uint32_t m0 = blockIdx.x * kTm, g0 = blockIdx.y * kTg;
  const uint32_t t = threadIdx.x;
  // read: 16 rows per pass, 16 groups per row
#pragma unroll
  for (uint32_t p = 0; p < kTm / 16; ++p) {
    const uint32_t mm = p * 16 + (t >> 4), gg = t & 15;
    const uint32_t m = m0 + mm, g = g0 + gg;
    float v = 0.0f;
    if (m < M && g < G) v = rm[(uint64_t)m * G + g];
    tile[gg][mm] = v;
  }
  __syncthreads();
  // write: 4 group columns per pass, 64 tokens per column
#pragma unroll
  for (uint32_t p = 0; p < kTg / 4; ++p) {
    const uint32_t gg = p * 4 + (t >> 6), mm = t & 63;
    const uint32_t m = m0 + mm, g = g0 + gg;
    if (m < Mp && g < G) km[(uint64_t)g * Mp + m] = tile[gg][mm];
  }
}

}  // namespace

hipError_t launch_relayout(const float* scale_rm, float* scale_km, uint32_t M, uint32_t K,
                           hipStream_t s) {
  const uint32_t G = K / kGroup, Mp = m_pad16(M);
  const dim3 grid((Mp + kTm - 1) / kTm, (G + kTg - 1) / kTg);
  relayout_kernel<<<grid, dim3(256), 0, s>>>(scale_rm, scale_km, M, Mp, G);
  return hipGetLastError();
}

}  // namespace fp8q
