// Clock stamps: the sustained shader clock over a timed region of the
// stream (measurement support for the benchmark, not part of the
// projection).  Each of `n` one-wave workgroups records, from its first
// lane, the id of the XCD it runs on (hardware register XCC_ID), the
// hardware id of its wave slot (HW_ID: CU, shader array and engine in bits
// 8-15), the shader clock counter (s_memtime) and the constant 100 MHz
// counter (s_memrealtime).  The shader clock counters of different CUs are
// not aligned with each other, so two stamps around a region are paired by
// (XCD, CU): each pair gives that XCD's average clock, d(memtime) /
// d(memrealtime) * 100 MHz.  With n = 1024 the two stamps share most CUs.
#include "fp8q_internal.h"

namespace fp8q {
namespace {

// XCC_ID: hardware register 20, bits [3:0]; HW_ID: hardware register 4
constexpr int kHwRegXccId = 20 | (0 << 6) | ((4 - 1) << 11);
constexpr int kHwRegHwId = 4 | (0 << 6) | ((32 - 1) << 11);

__global__ __launch_bounds__(64) void clock_stamp_kernel(unsigned long long* __restrict__ dst) {
  if (threadIdx.x == 0) {
    const unsigned long long t = __builtin_amdgcn_s_memtime();
    const unsigned long long r = __builtin_amdgcn_s_memrealtime();
    const unsigned xcc = (unsigned)__builtin_amdgcn_s_getreg(kHwRegXccId) & 15u;
    const unsigned hw = (unsigned)__builtin_amdgcn_s_getreg(kHwRegHwId);
    dst[4 * blockIdx.x + 0] = xcc;
    dst[4 * blockIdx.x + 1] = hw;
    dst[4 * blockIdx.x + 2] = t;
    dst[4 * blockIdx.x + 3] = r;
  }
}

}  // namespace

hipError_t launch_clock_stamp(unsigned long long* dst, uint32_t n, hipStream_t s) {
  clock_stamp_kernel<<<dim3(n), dim3(64), 0, s>>>(dst);
  return hipGetLastError();
}

}  // namespace fp8q
