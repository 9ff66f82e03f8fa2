// Internal launch interface between the C-ABI layer (fp8q_api.hip) and the
// kernel translation units.  Launchers assume validated arguments: shapes
// checked, pointers non-NULL and aligned, M > 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr uint32_t kGroup = 128;  // K elements per scale group / weight block edge

// native 128-/64-bit vectors (usable with the nontemporal builtins)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- quantizer geometry (shared with the selector) ----
// Variant A: flat over all M*(K/128) groups, 8 lanes per group,
// kQuantAWaves waves per workgroup.
constexpr uint32_t kQuantAWaves = 4;
constexpr uint32_t kQuantAGroupsPerWg = 8 * kQuantAWaves;
// Variant B: K-grouped; a workgroup covers kQuantBGroupsPerWg consecutive
// groups of one token row, kQuantBRounds groups per 16-lane row.
constexpr uint32_t kQuantBWaves = 4;
constexpr uint32_t kQuantBRounds = 2;
constexpr uint32_t kQuantBGroupsPerWg = 4 * kQuantBWaves * kQuantBRounds;
// Floor of the selection rule on gfx950 (workgroups per CU).
constexpr uint32_t kQuantMinWgPerCu = 2;
// Target default of the lever that lets variant B run at all.  Off on
// gfx950: timed with a cache flush before every launch over the token/K
// sweep (M in 16..16384, K in 5120/6144/17408), B was never faster than A by
// more than 0.1 us and was 3-15% slower wherever its grid fills the device.
constexpr bool kQuantBRequestedByDefault = false;

hipError_t launch_quant_a(const uint16_t* x, uint8_t* q, float* scale_rm,
                          float* scale_km, uint32_t M, uint32_t K, hipStream_t s);
hipError_t launch_quant_b(const uint16_t* x, uint8_t* q, float* scale_rm,
                          float* scale_km, uint32_t M, uint32_t K, hipStream_t s);
// K-major pad slots m in [M, ceil16(M)) of scale_km are written by this
// launcher when the quantizer writes scale_km directly.

hipError_t launch_relayout(const float* scale_rm, float* scale_km, uint32_t M,
                           uint32_t K, hipStream_t s);

// GEMM kernels: LDS-tiled MFMA (tile configuration cfg: 0/1 = 128x128
// tiles, 4 waves, 2 LDS stages so that two workgroups share a CU; 2 =
// 256x128 with 8 waves; 3 = 256x128 with 4 waves; 4 = 256x128 with two
// ping-pong groups of 4 waves) and skinny (M <= 64).
constexpr uint32_t kSkinnyMaxM = 65535u * 64u;  // skinny kernel: row tiles of 64 (grid y <= 65535)
// row_scaled: w_s is one fp32 scale per weight row [N] (applied to the
// finished accumulator) instead of [N/128, K/128] block scales.
hipError_t launch_gemm_tiled(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                             const float* w_s, uint16_t* out, uint32_t M, uint32_t N,
                             uint32_t K, int cfg, bool row_scaled, hipStream_t s);
// Split-K form of the 128x128 tiled kernel (block-scaled weights): splits
// workgroups per tile, each over a contiguous range of K blocks, write fp32
// partial tiles to part [splits, M, N]; a reduction adds them in split order
// into out.  2 <= splits <= K/128.
hipError_t launch_splitk_128(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                             const float* w_s, uint16_t* out, float* part, uint32_t M,
                             uint32_t N, uint32_t K, uint32_t splits, hipStream_t s);
hipError_t launch_gemm_skinny(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                              const float* w_s, uint16_t* out, uint32_t M, uint32_t N,
                              uint32_t K, uint32_t cu_count, bool row_scaled, hipStream_t s);

// bf16 comparator GEMM: out[M,N] = bf16(x[M,K] . w[N,K]^T), N % 128 == 0,
// K % 64 == 0.
hipError_t launch_gemm_bf16(const uint16_t* x, const uint16_t* w, uint16_t* out, uint32_t M,
                            uint32_t N, uint32_t K, hipStream_t s);

// FP8 weights [N,K] -> bf16 [N,K]: dst = bf16(fl32(dec(w) * scale[(n/bn)*sk + k/bk]))
// with (bn, bk, sk) = (128, 128, K/128) or, per_row, (1, K, 1).
hipError_t launch_dequant(const uint8_t* w, const float* scale, uint16_t* dst, uint32_t N,
                          uint32_t K, bool per_row, hipStream_t s);

// FFN intermediate: h = bf16(silu(gate) * up) for bf16 gate/up [M,I], then
// quantized per (token, 128-group): codes [M,I] and K-major scales
// [I/128, ceil16(M)] with the pad slots zeroed.
hipError_t launch_silu_mul_quant(const uint16_t* gate, const uint16_t* up, uint8_t* q,
                                 float* scale_km, uint32_t M, uint32_t I, hipStream_t s);

// Fused gate/up projection of the dense FFN: x codes [M,H] with K-major
// scales [H/128, ceil16(M)], gate and up weights [I,H] with block scales
// [I/128, H/128] -> the intermediate's codes [M,I] and K-major scales
// [I/128, ceil16(M)] (pad slots zeroed), equal to launch_silu_mul_quant of
// the two bf16 projections.  I % 128 == 0, H % 128 == 0.
hipError_t launch_ffn_gate_up(const uint8_t* x, const float* x_s_km, const uint8_t* w_gate,
                              const float* ws_gate, const uint8_t* w_up, const float* ws_up,
                              uint8_t* hq, float* hs_km, uint32_t M, uint32_t H, uint32_t I,
                              hipStream_t s);

inline uint32_t m_pad16(uint32_t m) { return (m + 15u) / 16u * 16u; }

}  // namespace fp8q
