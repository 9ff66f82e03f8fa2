// Building blocks shared by the MFMA GEMM kernels (gemm.hip, gemm_bf16.hip):
// operand vector types, bf16 rounding of the epilogue, buffer-resource
// loads straight into LDS, the LDS chunk swizzle, wait/barrier/scheduling
// helpers and the XCD-aware tile order.  Everything is internal (anonymous
// namespace): each kernel source includes its own copy.
#pragma once

#include <utility>

#include "fp8q_internal.h"

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint2 pack_bf16x4(const v4f& v) {
  return make_uint2(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16));
}

__device__ __forceinline__ v8i join(u32x4 a, u32x4 b) {
  v8i r = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return r;
}

// Direct global->LDS loads through a buffer resource: every lane of the wave
// copies `bytes` (4 or 16) from base + voff (per lane, VGPR) + soff (uniform,
// SGPR); lane i's data lands at lds + i * bytes, and lds must be the same for
// the whole wave (it goes to M0).  With the per-K-block advance in soff the
// loop spends no vector instructions on addresses.  (Kept out of lambdas: HIP
// lambdas are host+device, and a device-only builtin inside one called from
// a kernel template makes the host pass drop that kernel's stub.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0): bound = bytes; word 3 = 0x00020000 for gfx9-family
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff,
                                           soff, 0, 0);
}

// The same with the LDS destination as a byte address in the workgroup's
// LDS (for addresses formed at run time; no generic-pointer null check).
__device__ __forceinline__ void dma16_at(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                         uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(size_t)lds,
                                           16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4_at(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                        uint32_t lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(size_t)lds,
                                           4, voff, soff, 0, 0);
}
// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ uint32_t swz(uint32_t r) { return (r & 7u) ^ ((r >> 3) & 1u); }

// s_waitcnt vmcnt(n) leaving expcnt/lgkmcnt unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// wait until at most ahead*L of this wave's vector loads are outstanding
template <int L, int A>
__device__ __forceinline__ void wait_ahead(uint32_t ahead) {
  if constexpr (A <= 0) {
    wait_vmcnt<0>();
  } else {
    if (ahead >= (uint32_t)A) wait_vmcnt<A * L>();
    else wait_ahead<L, A - 1>(ahead);
  }
}

template <class F, int... Is>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}

// Tile t of the grouped order: tile ids walk blocks of GROUP_M tile rows, N
// fastest inside a block, so that the tiles that run together share their
// activation rows and weight columns.
__device__ __forceinline__ void grouped_tile(uint32_t t, uint32_t tiles_m, uint32_t tiles_n,
                                             uint32_t& tmi, uint32_t& tni) {
  constexpr uint32_t GROUP_M = 8;
  const uint32_t per_group = GROUP_M * tiles_n;
  const uint32_t group = t / per_group, first_m = group * GROUP_M;
  const uint32_t gm = min(tiles_m - first_m, GROUP_M);
  tmi = first_m + (t % per_group) % gm;
  tni = (t % per_group) / gm;
}

// Tile of a workgroup in an XCD-aware, grouped order.  Workgroup ids are
// dealt round-robin to the 8 XCDs; each XCD gets a contiguous run of tile
// ids so that the tiles it runs together share its L2, and tile ids follow
// the grouped order above.
__device__ __forceinline__ void tile_coords(uint32_t tiles_m, uint32_t tiles_n, uint32_t& tmi,
                                            uint32_t& tni) {
  const uint32_t ntiles = tiles_m * tiles_n;
  const uint32_t bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const uint32_t q = ntiles >> 3, r8 = ntiles & 7;
  const uint32_t t = (xcd < r8) ? xcd * (q + 1) + slot : r8 * (q + 1) + (xcd - r8) * q + slot;
  grouped_tile(t, tiles_m, tiles_n, tmi, tni);
}

// Split-K form: the grid holds splits workgroups per tile.  Workgroup ids
// are dealt to the XCDs as above over tiles_m * tiles_n * splits slots; the
// slot picks the tile (grouped order) and the split.
__device__ __forceinline__ void tile_split_coords(uint32_t tiles_m, uint32_t tiles_n,
                                                  uint32_t splits, uint32_t& tmi, uint32_t& tni,
                                                  uint32_t& split) {
  const uint32_t nslots = tiles_m * tiles_n * splits;
  const uint32_t bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const uint32_t q = nslots >> 3, r8 = nslots & 7;
  const uint32_t v = (xcd < r8) ? xcd * (q + 1) + slot : r8 * (q + 1) + (xcd - r8) * q + slot;
  split = v % splits;
  grouped_tile(v / splits, tiles_m, tiles_n, tmi, tni);
}

}  // namespace
}  // namespace fp8q
