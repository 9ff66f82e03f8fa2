// Block-scaled FP8 GEMM for gfx950:
//   out[m,n] = bf16( sum_kb a_s[kb][m] * w_s[n/128][kb] * P(m,n,kb) ),
//   P(m,n,kb) = sum_{j<128} a[m,128kb+j] * w[n,128kb+j]   (e4m3 x e4m3 -> fp32)
// (page "dispatch_proj.rs": cublas_fp8_proj_prequant computes act . W^T with
// VEC128 activation scales in the K-major layout and 128x128 weight-block
// scales; weight-scale index (n/128)*(K/128) + k/128 per dequant_fp8_bf16_into).
//
// One v_mfma_f32_16x16x128_f8f6f4 consumes exactly one 128-deep scale block,
// so each MFMA starts from zero and its 16x16 partial is folded into the fp32
// accumulator with one fma per element: acc += P * (a_s * w_s).  The weight
// tile is the MFMA's first operand and the activation tile its second, so
// lane l of the 16x16 result holds out[m = l%16][n = 4*(l/16) .. +3]: one
// activation scale per lane per M-subtile, four contiguous output columns.
//
// Operand fragments: lane l supplies row (l % 16) of its 16-row tile and the
// 32 bytes [32*(l/16), 32*(l/16)+32) of the 128-byte K block, for both
// operands, so both see the same K permutation and the dot product is the
// full 128-term sum whatever order the hardware assigns to those bytes.
#include <atomic>
#include <chrono>
#include "mfma_common.h"
#include "quant_common.h"

namespace fp8q {
namespace {

// Promotion distance: the fp32 promotion of MFMA i is issued in the slot of
// MFMA i + kPromoteDist.  A VALU read of an MFMA result waits until the
// matrix pipe has written it; measured with one wave per SIMD issuing
// 16x16x128 FP8 MFMAs and four promotion fmas per MFMA from registers, the
// matrix pipe is busy 51% / 75% / 91% of the time at distance 1 / 2 / 3
// (99% without the fmas).  The results rotate through four register sets,
// so the distance is at most 3, and the last kPromoteDist MFMAs of a K block
// (promoted in the next block, with that block's scale) lie in one row.
constexpr int kPromoteDist = 3;

__device__ __forceinline__ v4f mfma_e4m3_128(const v8i& w, const v8i& a) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // cbsz = blgp = 0: both operands OCP e4m3; zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, zero, 0, 0, 0, 0, 0, 0);
}

// ------------------------------------------------------------------------
// LDS-tiled kernel.  Workgroup tile BM x BN, K step 128 (one scale block),
// WGM x WGN waves, each owning a WM x WN = (BM/WGM) x (BN/WGN) sub-tile made
// of TM x TN MFMA tiles of 16 x 16.
//
// Operands reach LDS through direct buffer->LDS loads (64 lanes x 16 B land in
// 1 KB of consecutive LDS), so the ring of STAGES LDS buffers is filled
// without staging registers.  A stage holds [BM rows][128 B] of activations,
// [BN rows][128 B] of weights and, per wave, the activation scales of its WM
// rows (read from the K-major scale layout, where they are contiguous) and 64
// copies of the block's weight scale.  16-byte chunk c of row r sits at chunk
// position c ^ f(r), f(r) = (r & 7) ^ ((r >> 3) & 1), so the 16 lanes that
// read one chunk column of 16 consecutive rows hit 16 different (row parity,
// chunk) bank groups; f depends on r mod 16 only, so every fragment address is
// a per-lane constant plus a compile-time offset.  The direct load realises
// the swizzle by choosing, per lane, which global chunk lands in its fixed
// LDS slot.
//
// Register pipeline, per K block: the MFMAs of block kb run from registers
// while the fragments of block kb+1 are read from LDS into a second register
// set (activation fragments in place, as soon as the last MFMA of their row
// has been issued).  The fp32 promotion of MFMA i is issued after MFMA
// i + kPromoteDist, by which time the matrix pipe has written its result; the
// promotions of a block's last kPromoteDist MFMAs run in the next block.
// Each MFMA slot (the MFMA, the four fmas, one or two LDS reads) is fenced
// off from the next with a scheduling barrier: left to itself the compiler hoists all MFMAs of a block and then
// has to serialise the next one on a single result register.
// ------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int STAGES, bool ROW = false>
struct TileCfg {
  static constexpr int NW = WGM * WGN, NT = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN, TM = WM / 16, TN = WN / 16, NP = TM * TN;
  static constexpr int A_BYTES = BM * 128, W_BYTES = BN * 128;
  static constexpr int SA = (WM + 63) / 64;        // activation-scale loads per wave and stage
  static constexpr int SCW_BYTES = SA * 256 + 256;  // per wave: its scales + 64 weight-scale copies
  static constexpr int STAGE_BYTES = A_BYTES + W_BYTES + NW * SCW_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int DA = BM * 8 / 64 / NW;  // 1 KB direct loads per wave: activations
  static constexpr int DW = BN * 8 / 64 / NW;  //                              weights
  static constexpr int LOADS = DA + DW + SA + (ROW ? 0 : 1);  // direct loads per wave and stage
  // LDS reads of the next block per MFMA slot: slot TN*tm + TN-1 (after the
  // last MFMA of row tm) reads activation fragment tm; the other slots take,
  // in order, the 2*TN weight-fragment halves, TM/2 activation-scale pairs
  // and the weight scale.
  static constexpr int FREE_OPS = 2 * TN + TM / 2 + (ROW ? 0 : 1);
  static_assert(WM % 16 == 0 && WN % 16 == 0 && TN >= 2 && TM % 2 == 0 && NP % 4 == 0, "wave tile");
  static_assert(NP - TM >= FREE_OPS, "too few MFMA slots for the LDS reads");
  static_assert(kPromoteDist >= 1 && kPromoteDist <= 3 && kPromoteDist <= TN && NP % 4 == 0,
                "pending promotions lie in the last row; four result registers");
  static_assert(BM * 8 % (64 * NW) == 0 && BN * 8 % (64 * NW) == 0, "tile/wave mismatch");
  static_assert(128 % WN == 0, "a wave's columns lie in one weight-scale block");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(STAGES >= 2 && (STAGES - 2) * LOADS < 64, "vmcnt range");
  static_assert(STAGE_BYTES % 256 == 0, "stage alignment");
};

// ROW: per-row weight scales Ws[N] (one multiplier per output column,
// applied to the finished accumulator) instead of 128x128 block scales
// applied per K block.
//
// SPLIT: split-K.  The grid holds `splits` workgroups per tile; split s takes
// the K blocks [s*G/splits, (s+1)*G/splits) and stores its fp32 partial tile
// to part[s][M][N]; a second kernel (splitk_reduce_kernel) adds the splits'
// partials in split order and rounds to bf16.  Block-scaled weights only.
template <int BM, int BN, int WGM, int WGN, int STAGES, bool ROW, bool SPLIT = false>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_tiled_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp, uint32_t tiles_m, uint32_t tiles_n, uint32_t splits = 1,
    float* __restrict__ part = nullptr) {
  using C = TileCfg<BM, BN, WGM, WGN, STAGES, ROW>;
  constexpr int TM = C::TM, TN = C::TN, NP = C::NP;
  static_assert(!(SPLIT && ROW), "split-K for block-scaled weights only");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const uint32_t wm = wave / WGN, wn = wave % WGN;

  uint32_t tmi, tni, split = 0;  // this workgroup's tile (XCD-aware, grouped order)
  if constexpr (SPLIT)
    tile_split_coords(tiles_m, tiles_n, splits, tmi, tni, split);
  else
    tile_coords(tiles_m, tiles_n, tmi, tni);
  const uint32_t m0 = tmi * BM, n0 = tni * BN;
  const uint32_t GK = K / kGroup;  // K blocks in all
  // this workgroup's K blocks: kbeg .. kbeg + G - 1
  const uint32_t kbeg = SPLIT ? split * GK / splits : 0;
  const uint32_t G = SPLIT ? (split + 1) * GK / splits - kbeg : GK;
  const uint32_t nb = (n0 + wn * C::WN) / kGroup;  // this wave's weight-scale block row

  // ---- buffer resources and per-lane source offsets (K block 0) ----
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A, M * K);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(W, N * K);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(As, GK * Mp * 4);
  const __amdgpu_buffer_rsrc_t rWs = make_rsrc(Ws, ROW ? N * 4 : (N / kGroup) * GK * 4);
  uint32_t a_off[C::DA], w_off[C::DW], s_off[C::SA];
#pragma unroll
  for (int j = 0; j < C::DA; ++j) {
    const uint32_t c = (wave * C::DA + j) * 64 + lane, row = c >> 3;
    a_off[j] = min(m0 + row, M - 1) * K + ((c & 7) ^ swz(row)) * 16;
  }
#pragma unroll
  for (int j = 0; j < C::DW; ++j) {
    const uint32_t c = (wave * C::DW + j) * 64 + lane, row = c >> 3;
    w_off[j] = (n0 + row) * K + ((c & 7) ^ swz(row)) * 16;
  }
  // activation scales of this wave's rows (rows past Mp are clamped in
  // bounds and never used; rows in [M, Mp) hold the layout's zero pad)
#pragma unroll
  for (int j = 0; j < C::SA; ++j) s_off[j] = min(m0 + wm * C::WM + j * 64 + lane, Mp - 1) * 4;
  const uint32_t ws_off = nb * GK * 4;  // every lane loads the same weight scale
  const uint32_t sc_base = C::A_BYTES + C::W_BYTES + wave * C::SCW_BYTES;
  const uint32_t ws_base = sc_base + C::SA * 256;

  // K block kbeg + kl (kl counted from this workgroup's first block)
  auto issue_stage = [&](uint32_t kl, uint32_t stage) {
    const uint32_t kb = kbeg + kl;
    uint8_t* base = smem + stage * C::STAGE_BYTES;
#pragma unroll
    for (int j = 0; j < C::DA; ++j) dma16(rA, a_off[j], kb * kGroup, base + (wave * C::DA + j) * 1024);
#pragma unroll
    for (int j = 0; j < C::DW; ++j)
      dma16(rW, w_off[j], kb * kGroup, base + C::A_BYTES + (wave * C::DW + j) * 1024);
#pragma unroll
    for (int j = 0; j < C::SA; ++j) dma4(rS, s_off[j], kb * Mp * 4, base + sc_base + j * 256);
    if constexpr (!ROW) dma4(rWs, ws_off, kb * 4, base + ws_base);
  };

  // Per-lane byte offsets of a fragment inside a 16-row slab: this lane's row
  // (lane % 16) and its two chunks 2*(lane/16) and 2*(lane/16)+1, swizzled.
  const uint32_t l16 = lane & 15, c0 = 2 * (lane >> 4);
  const uint32_t lo0 = l16 * 128 + ((c0 ^ swz(l16)) * 16);
  const uint32_t lo1 = l16 * 128 + (((c0 + 1) ^ swz(l16)) * 16);
  auto ld16 = [](const uint8_t* p) -> v4i { return *reinterpret_cast<const v4i*>(p); };
  auto ldf = [](const uint8_t* p) -> float { return *reinterpret_cast<const float*>(p); };
  const uint32_t a_row0 = wm * C::WM * 128, w_row0 = C::A_BYTES + wn * C::WN * 128;

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // ---- prologue: the first STAGES stages, then block 0 into registers ----
  // Stages past the last K block reload the last block (in bounds, never
  // read), so that every iteration issues the same loads and waits for the
  // same count, and the loop body stays one basic block per K block.
#pragma unroll
  for (int s = 0; s < STAGES; ++s) issue_stage(min((uint32_t)s, G - 1), s);
  wait_vmcnt<(STAGES - 1) * C::LOADS>();
  wg_barrier();

  v8i af[TM], bf0[TN], bf1[TN];
  float as0[TM], as1[TM], ws0, ws1;
  {
    const uint8_t* s0 = smem;  // slot 0
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      af[tm].lo = ld16(s0 + a_row0 + tm * 2048 + lo0);
      af[tm].hi = ld16(s0 + a_row0 + tm * 2048 + lo1);
      as0[tm] = ldf(s0 + sc_base + (tm * 16 + l16) * 4);
    }
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      bf0[tn].lo = ld16(s0 + w_row0 + tn * 2048 + lo0);
      bf0[tn].hi = ld16(s0 + w_row0 + tn * 2048 + lo1);
    }
    ws0 = ROW ? 1.0f : ldf(s0 + ws_base);
  }
  ws1 = 1.0f;

  // MFMA results rotate through 4 register sets; the promotions of the last
  // kPromoteDist MFMAs of a block are pending when the next block starts
  // (zero before the first block).
  v4f p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float sc[TM], sc_tail = 0.0f;

  // one K block; S = kb % STAGES, a compile-time constant (the loop below is
  // unrolled by a multiple of STAGES), so that the LDS addresses of the next
  // block's fragments are loop-invariant registers plus immediate offsets
  auto step = [&](uint32_t kb, auto slot_c, const v8i(&bf)[TN], const float(&as)[TM], float ws,
                  v8i(&bfn)[TN], float(&asn)[TM], float& wsn) {
    constexpr int S = decltype(slot_c)::value;
    wait_lgkm0();  // fragments and scales of block kb are in registers
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) sc[tm] = as[tm] * ws;
    wait_vmcnt<(STAGES - 2) * C::LOADS>();
    wg_barrier();  // stage kb+1 is in LDS; slot kb % STAGES is free
    issue_stage(min(kb + STAGES, G - 1), S);
    // (on the last block the reads below fetch a slot holding a reloaded
    // copy of the last block, never used; its load has completed)
    const uint8_t* nx = smem + ((S + 1) % STAGES) * C::STAGE_BYTES;
    unroll_seq(
        [&](auto ic) {
          constexpr int I = decltype(ic)::value;
          constexpr int tm = I / TN, tn = I % TN;
          p[I & 3] = mfma_e4m3_128(bf[tn], af[tm]);
          if constexpr (I < kPromoteDist) {
            constexpr int J = NP - kPromoteDist + I;
            acc[J / TN][J % TN] += p[J & 3] * sc_tail;
          } else {
            constexpr int J = I - kPromoteDist;
            acc[J / TN][J % TN] += p[J & 3] * sc[J / TN];
          }
          if constexpr (tn == TN - 1) {
            af[tm].lo = ld16(nx + a_row0 + tm * 2048 + lo0);
            af[tm].hi = ld16(nx + a_row0 + tm * 2048 + lo1);
          } else {
            constexpr int Q = I - I / TN;
            if constexpr (Q < 2 * TN) {
              if constexpr (Q & 1) bfn[Q / 2].hi = ld16(nx + w_row0 + (Q / 2) * 2048 + lo1);
              else bfn[Q / 2].lo = ld16(nx + w_row0 + (Q / 2) * 2048 + lo0);
            } else if constexpr (Q < 2 * TN + TM / 2) {
              constexpr int T2 = 2 * (Q - 2 * TN);
              asn[T2] = ldf(nx + sc_base + (T2 * 16 + l16) * 4);
              asn[T2 + 1] = ldf(nx + sc_base + ((T2 + 1) * 16 + l16) * 4);
            } else if constexpr (!ROW && Q == 2 * TN + TM / 2) {
              wsn = ldf(nx + ws_base);
            }
          }
          sched_fence();
        },
        std::make_integer_sequence<int, NP>{});
    sc_tail = sc[TM - 1];
  };
  // block kb0 + I: register set I % 2, LDS slot I % STAGES
  auto step_i = [&](uint32_t kb0, auto ic) {
    constexpr int I = decltype(ic)::value;
    using Slot = std::integral_constant<int, I % STAGES>;
    if constexpr (I % 2 == 0)
      step(kb0 + I, Slot{}, bf0, as0, ws0, bf1, as1, ws1);
    else
      step(kb0 + I, Slot{}, bf1, as1, ws1, bf0, as0, ws0);
  };
  constexpr int U = STAGES % 2 == 0 ? STAGES : 2 * STAGES;  // blocks per loop iteration
  uint32_t kb = 0;
  for (; kb + U <= G; kb += U)
    unroll_seq([&](auto ic) { step_i(kb, ic); }, std::make_integer_sequence<int, U>{});
  unroll_seq(
      [&](auto ic) {
        if (kb + decltype(ic)::value < G) step_i(kb, ic);
      },
      std::make_integer_sequence<int, U - 1>{});
  wait_vmcnt<0>();  // no direct load may still be writing LDS when the workgroup ends
  // promotions of the last block's last kPromoteDist MFMAs (all in its last row)
#pragma unroll
  for (int j = NP - kPromoteDist; j < NP; ++j) acc[j / TN][j % TN] += p[j & 3] * sc_tail;

  if constexpr (ROW) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const float4 r = *reinterpret_cast<const float4*>(Ws + n0 + wn * C::WN + tn * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc[tm][tn] *= v4f{r.x, r.y, r.z, r.w};
    }
  }
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const uint32_t m = m0 + wm * C::WM + tm * 16 + (lane & 15);
    if (m < M) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const uint32_t n = n0 + wn * C::WN + tn * 16 + 4 * (lane >> 4);
        if constexpr (SPLIT)
          *reinterpret_cast<v4f*>(part + ((uint64_t)split * M + m) * N + n) = acc[tm][tn];
        else
          *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(acc[tm][tn]);
      }
    }
  }
}

// out[m, n] = bf16(sum over s < splits, in order, of part[s][m][n]); four
// columns per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const v4f* __restrict__ part,
                                                            uint2* __restrict__ out,
                                                            uint64_t quads, uint32_t splits) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < quads;
       i += (uint64_t)gridDim.x * 256) {
    v4f s = __builtin_nontemporal_load(&part[i]);
    for (uint32_t k = 1; k < splits; ++k) s += __builtin_nontemporal_load(&part[k * quads + i]);
    out[i] = pack_bf16x4(s);
  }
}

template <int BM, int BN, int WGM, int WGN, int STAGES, bool ROW>
hipError_t launch_tiled_cfg(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                            const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                            hipStream_t s) {
  using C = TileCfg<BM, BN, WGM, WGN, STAGES, ROW>;
  if (N % BN != 0) return hipErrorInvalidValue;
  static std::atomic<bool> attr_set{false};  // the call is idempotent: racing threads repeat it
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_tiled_kernel<BM, BN, WGM, WGN, STAGES, ROW>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  const uint32_t tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  gemm_tiled_kernel<BM, BN, WGM, WGN, STAGES, ROW><<<dim3(tiles_m * tiles_n), dim3(C::NT), C::LDS_BYTES, s>>>(
      a, a_s_km, w, w_s, out, M, N, K, m_pad16(M), tiles_m, tiles_n);
  return hipGetLastError();
}

// split-K launch of the 128x128 tiled kernel and the reduction
template <int STAGES>
hipError_t launch_splitk_cfg(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                             const float* w_s, float* part, uint32_t M, uint32_t N, uint32_t K,
                             uint32_t splits, hipStream_t s) {
  constexpr int BM = 128, BN = 128, WGM = 2, WGN = 2;
  using C = TileCfg<BM, BN, WGM, WGN, STAGES, false>;
  static std::atomic<bool> attr_set{false};  // the call is idempotent: racing threads repeat it
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_tiled_kernel<BM, BN, WGM, WGN, STAGES, false, true>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  const uint32_t tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  gemm_tiled_kernel<BM, BN, WGM, WGN, STAGES, false, true>
      <<<dim3(tiles_m * tiles_n * splits), dim3(C::NT), C::LDS_BYTES, s>>>(
          a, a_s_km, w, w_s, nullptr, M, N, K, m_pad16(M), tiles_m, tiles_n, splits, part);
  return hipGetLastError();
}

// Split grids that fit one workgroup per CU take three LDS stages (99 KB:
// one workgroup per CU, two blocks of loads in flight); larger ones two (two
// workgroups per CU).  Measured with cold caches at N = 5120, K = 17408 on
// 256 CUs: 44.2 / 47.8 / 56.5 us against 46.0 / 50.9 / 64.5 us at M = 65 /
// 128 / 256; at N = 6144, K = 5120: 22.2 / 25.4 / 32.3 against 23.2 / 27.5 /
// 36.3 us.
hipError_t launch_splitk_128_t(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                               const float* w_s, uint16_t* out, float* part, uint32_t M,
                               uint32_t N, uint32_t K, uint32_t splits, uint32_t cus,
                               hipStream_t s) {
  if (N % 128 != 0 || splits < 2 || splits > K / kGroup) return hipErrorInvalidValue;
  // up to 64 rows: the skinny kernel's split form (its weight loads go to
  // registers, and its ranges of columns hold the rows' activations once)
  hipError_t serr = hipSuccess;
  if (launch_skinny_split(a, a_s_km, w, w_s, out, part, M, N, K, splits, cus, s, serr)) return serr;
  const uint64_t wgs = (uint64_t)((M + 127) / 128) * (N / 128) * splits;
  hipError_t e = wgs <= cus
                     ? launch_splitk_cfg<3>(a, a_s_km, w, w_s, part, M, N, K, splits, s)
                     : launch_splitk_cfg<2>(a, a_s_km, w, w_s, part, M, N, K, splits, s);
  if (e != hipSuccess) return e;
  const uint64_t quads = (uint64_t)M * N / 4;
  const uint64_t blocks = (quads + 255) / 256;
  const uint32_t grid = (uint32_t)(blocks < 4096 ? blocks : 4096);
  splitk_reduce_kernel<<<dim3(grid), dim3(256), 0, s>>>(reinterpret_cast<const v4f*>(part),
                                                          reinterpret_cast<uint2*>(out), quads,
                                                          splits);
  return hipGetLastError();
}
// ------------------------------------------------------------------------
// Ping-pong kernel: 256x128 workgroup tile, 8 waves of 64x64 in two groups.
// Group 0 (waves 0-3, tile rows 0-127) and group 1 (waves 4-7, rows
// 128-255) put one wave on each SIMD and take turns: while one group runs
// the MFMAs and promotions of a K block from registers, the other reads its
// fragments of the block from LDS, so each SIMD's matrix pipe is fed by one
// wave at a time instead of two waves that leave every barrier together and
// compete.  Per K block kb:
//   phase A: group 0 computes block kb; group 1 reads block kb
//   phase B: group 1 computes block kb; group 0 reads block kb+1
// with a workgroup barrier after each phase.  A wave holds one fragment set
// (loaded in its read phase, consumed in its compute phase).
//
// Direct loads: a stage is 48 1-KB operand chunks (chunk c at LDS offset
// c*1024: activation rows 8c..8c+7 for c < 32, weight rows 8(c-32).. after)
// plus every wave's scales.  Each wave issues 8 loads per block at the end
// of its read phase (group 0: 8 operand chunks; group 1: 4 chunks and the
// scales of two waves), so the texture unit gets 32 or 16 KB per phase and
// the compute phases hold nothing but MFMAs and promotions.  Stage s
// (block min(s, G-1): stages past the last block reload it, in bounds and
// never read) goes to slot s % STAGES.  Before the phase-A barrier of block
// kb each wave waits for its own part of stage kb+1.
//
// FFN mode (the dense FFN's fused gate/up projection): the workgroup tile is
// 128 token rows by 256 weight rows, the 128 gate rows n0.. and the 128 up
// rows n0.. of one intermediate column block; group 0 computes gate and group
// 1 up, wave for wave on the same 64x64 output positions, and the epilogue
// forms h = bf16(silu(bf16 gate) * bf16 up), quantizes it per (token,
// 128-group) and writes the codes and the K-major scales (see
// ffn_epilogue).  The main loop is the same code with the weight chunks
// read from two sources.
// ------------------------------------------------------------------------
template <int STAGES, bool ROW = false, bool FFN = false>
struct PpCfg {
  static constexpr int BM = FFN ? 128 : 256, BN = FFN ? 256 : 128, NW = 8, NT = 512;
  static constexpr int WM = 64, WN = 64, TM = 4, TN = 4, NP = 16;
  static constexpr int A_BYTES = BM * 128, W_BYTES = BN * 128;
  static constexpr int SCW_BYTES = 512;  // per wave: 64 activation scales + 64 weight-scale copies
  static constexpr int STAGE_BYTES = A_BYTES + W_BYTES + NW * SCW_BYTES;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int CHUNKS = (A_BYTES + W_BYTES) / 1024;  // 48
  // loads per wave and stage: group 0 eight operand chunks; group 1 four
  // operand chunks and the scales of itself and of its group-0 partner
  static constexpr int CH0 = 8, CH1 = 4;
  static constexpr int LW0 = CH0, LW1 = CH1 + 2 * (ROW ? 1 : 2);
  static_assert(4 * (CH0 + CH1) == CHUNKS && 2 * LW1 < 64, "chunk split, vmcnt range");
  static_assert(LDS_BYTES <= 160 * 1024 && STAGES == 3, "config");
  static_assert(kPromoteDist >= 1 && kPromoteDist <= 3 && kPromoteDist <= TN && NP % 4 == 0,
                "pending promotions lie in the last row; four result registers");
};

// Second weight operand and outputs of the FFN mode: W/Ws are the gate
// weights and their block scales, these the up weights and scales, the
// intermediate's codes [M,N] and its K-major scales [N/128, Mp].
struct FfnArgs {
  const uint8_t* w_up;
  const float* ws_up;
  uint8_t* hq;
  float* hs;
};

// FFN-mode epilogue, after the main loop (all direct loads of this wave
// complete).  Gate wave gw (group 0) and up wave gw (group 1, wave gw + 4)
// hold the same 64x64 output positions in the same registers; they split
// the rows: the gate wave finishes rows tm = 0, 1 of its band, the up wave
// rows tm = 2, 3.
//   1. each wave rounds its accumulators to bf16 (the projections' output
//      format) and parks the half its partner finishes in LDS;
//   2. each wave forms h = bf16(silu(g) * u) for its rows (silu_mul_f32, the
//      same code as the standalone intermediate kernel) and the maximum |h|
//      of each row over its 64 columns (integer max of bf16 magnitudes:
//      within a lane, then across the 4 lanes of a row);
//   3. the two waves of a group covering columns 0-63 and 64-127 of the
//      128-column group combine their row maxima through LDS; scale =
//      amax/448 and the codes of h / scale follow the activation quantizer's
//      exact steps (quotients, encode4).  Codes of rows < M are stored; the
//      wave on columns 0-63 stores the K-major scales of its rows < M and
//      zeros for pad rows M .. Mp-1.
// Every wave passes the same three workgroup barriers, each after its own LDS
// writes have completed (s_barrier alone does not wait for them).
template <int TM, int TN>
__device__ __forceinline__ void ffn_epilogue(const v4f (&acc)[TM][TN], uint8_t* smem,
                                             const FfnArgs& ffn, uint32_t wave, uint32_t lane,
                                             uint32_t mrow0, uint32_t ncol0, uint32_t nb,
                                             uint32_t M, uint32_t N, uint32_t Mp) {
  static_assert(TM == 4 && TN == 4, "64x64 wave tile");
  uint32_t* park = reinterpret_cast<uint32_t*>(smem);                // [8][4][64][4] u32: 32 KB
  uint32_t* rmax = reinterpret_cast<uint32_t*>(smem + 32 * 1024);    // [8][2][16] u32
  const uint32_t l16 = lane & 15, q4 = lane >> 4;
  const bool up = wave >= 4;
  auto lds_barrier = [] {
    wait_lgkm0();
    wg_barrier();
  };
  lds_barrier();  // every wave is done with the operand ring
  // 1. park the partner's half: tiles of rows tm = 0, 1 (up waves) or 2, 3
  //    (gate waves), two 16x16 tiles per 16-byte slot
#pragma unroll
  for (int t2 = 0; t2 < 4; ++t2) {
    const int t = 2 * t2;  // tile index within the half
    const uint2 a = up ? pack_bf16x4(acc[t / TN][t % TN]) : pack_bf16x4(acc[2 + t / TN][t % TN]);
    const uint2 b = up ? pack_bf16x4(acc[(t + 1) / TN][(t + 1) % TN])
                       : pack_bf16x4(acc[2 + (t + 1) / TN][(t + 1) % TN]);
    *reinterpret_cast<uint4*>(park + ((wave * 4 + t2) * 64 + lane) * 4) = make_uint4(a.x, a.y, b.x, b.y);
  }
  lds_barrier();
  // 2. h for this wave's rows
  const uint32_t partner = wave ^ 4;
  uint32_t hb[2][TN][2];  // h as packed bf16 pairs: rows i = 0, 1 of this wave's half
  uint32_t amax[2];
#pragma unroll
  for (int t2 = 0; t2 < 4; ++t2) {
    const uint4 pp = *reinterpret_cast<const uint4*>(park + ((partner * 4 + t2) * 64 + lane) * 4);
    const uint32_t pw[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 2 * t2 + h, i = t / TN, tn = t % TN;
      const uint2 own = up ? pack_bf16x4(acc[2 + i][tn]) : pack_bf16x4(acc[i][tn]);
      const uint32_t ow[2] = {own.x, own.y};
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint32_t g2 = up ? pw[2 * h + d] : ow[d], u2 = up ? ow[d] : pw[2 * h + d];
        const float lo = silu_mul_f32(__uint_as_float(g2 << 16), __uint_as_float(u2 << 16));
        const float hi = silu_mul_f32(__uint_as_float(g2 & 0xFFFF0000u), __uint_as_float(u2 & 0xFFFF0000u));
        hb[i][tn][d] = bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t mx = 0;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const uint32_t a = hb[i][tn][0] & 0x7FFF7FFFu, b = hb[i][tn][1] & 0x7FFF7FFFu;
      mx = max(mx, max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16)));
    }
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 16));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, 32));
    amax[i] = mx;
    if (q4 == 0) rmax[(wave * 2 + i) * 16 + l16] = mx;
  }
  lds_barrier();
  // 3. scales and codes
  const uint32_t mate = wave ^ 1;  // the other 64 columns of the 128-column group
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t a = max(amax[i], rmax[(mate * 2 + i) * 16 + l16]);
    const float sc = group_scale(a);
    float x[16], q[16];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      x[4 * tn + 0] = __uint_as_float(hb[i][tn][0] << 16);
      x[4 * tn + 1] = __uint_as_float(hb[i][tn][0] & 0xFFFF0000u);
      x[4 * tn + 2] = __uint_as_float(hb[i][tn][1] << 16);
      x[4 * tn + 3] = __uint_as_float(hb[i][tn][1] & 0xFFFF0000u);
    }
    quotients<16>(x, sc, q);
    const uint32_t m = mrow0 + ((up ? 2 : 0) + i) * 16 + l16;
    if (m < M) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        *reinterpret_cast<uint32_t*>(ffn.hq + (uint64_t)m * N + ncol0 + tn * 16 + 4 * q4) =
            encode4(q + 4 * tn);
    }
    if ((wave & 1) == 0 && q4 == 0 && m < Mp) ffn.hs[(uint64_t)nb * Mp + m] = (m < M) ? sc : 0.0f;
  }
}

template <int STAGES, bool ROW, bool FFN>
__global__ __launch_bounds__(512) void gemm_pp_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp, uint32_t tiles_m, uint32_t tiles_n, FfnArgs ffn) {
  using C = PpCfg<STAGES, ROW, FFN>;
  constexpr int TM = C::TM, TN = C::TN, NP = C::NP, BM = C::BM, BN = C::BN;
  constexpr int CH0 = C::CH0, CH1 = C::CH1, LW0 = C::LW0, LW1 = C::LW1;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t grp = wave >> 2, gw = wave & 3;
  const uint32_t wm = FFN ? gw >> 1 : 2 * grp + (gw >> 1);
  const uint32_t wn = FFN ? 2 * grp + (gw & 1) : gw & 1;

  uint32_t tmi, tni;  // this workgroup's tile (XCD-aware, grouped order)
  tile_coords(tiles_m, tiles_n, tmi, tni);
  const uint32_t m0 = tmi * BM, n0 = tni * (FFN ? kGroup : BN);
  const uint32_t G = K / kGroup;
  const uint32_t nb = n0 / kGroup;

  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A, M * K);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(W, N * K);
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(As, G * Mp * 4);
  const __amdgpu_buffer_rsrc_t rWs = make_rsrc(Ws, ROW ? N * 4 : (N / kGroup) * G * 4);
  // FFN mode: the up weights and their scales
  const __amdgpu_buffer_rsrc_t rW2 = FFN ? make_rsrc(ffn.w_up, N * K) : rW;
  const __amdgpu_buffer_rsrc_t rWs2 = FFN ? make_rsrc(ffn.ws_up, (N / kGroup) * G * 4) : rWs;

  // Operand chunks of this wave (LDS chunk c covers 8 rows of 128 bytes:
  // activations first, then weights; FFN mode: activations 0-15, gate
  // 16-31, up 32-47).  A wave may only overwrite, in its read phase, LDS
  // rows that no other wave of its own group reads:
  //   group 1 (loads in phase A, right after its own reads of block kb):
  //     four chunks that only group 0 reads -- activation rows 0-127 (plain)
  //     or the gate rows (FFN) -- and the scales of itself and of its
  //     group-0 partner wave gw, which only their owners read;
  //   group 0 (loads in phase B, after the phase-A barrier, when both groups
  //     are done with block kb): the other 32 chunks, eight per wave.
  uint32_t c_off[CH0], c_lds[CH0];
  const bool g0_act = !FFN && gw < 2;  // plain group 0: activation rows 128-255 (gw 0, 1) or weights
#pragma unroll
  for (int j = 0; j < CH0; ++j) {
    uint32_t c, ch;  // LDS chunk, chunk within its operand
    bool act;
    if (grp) {
      c = (FFN ? 16 : 0) + 4 * gw + (j & 3);
      ch = 4 * gw + (j & 3);
      act = !FFN;
    } else if constexpr (FFN) {
      c = (j < 4) ? 4 * gw + j : 32 + 4 * gw + (j - 4);
      ch = 4 * gw + (j & 3);
      act = j < 4;
    } else {
      c = 16 + 8 * gw + j;
      ch = g0_act ? c : c - 32;
      act = g0_act;
    }
    const uint32_t row = ch * 8 + (lane >> 3), col = lane & 7;  // row within the operand
    c_lds[j] = c;
    c_off[j] = act ? min(m0 + row, M - 1) * K + (col ^ swz(row)) * 16
                   : (n0 + row) * K + (col ^ swz(row)) * 16;  // swz: low 4 bits of the LDS row
  }
  const uint32_t s_off = min(m0 + wm * C::WM + lane, Mp - 1) * 4;       // own activation scales
  const uint32_t s_off_p = min(m0 + (gw >> 1) * C::WM + lane, Mp - 1) * 4;  // partner's (group 1)
  const uint32_t ws_off = nb * G * 4;
  const uint32_t my_sc = C::A_BYTES + C::W_BYTES + wave * C::SCW_BYTES;
  const uint32_t p_sc = C::A_BYTES + C::W_BYTES + gw * C::SCW_BYTES;

  auto issue_g0 = [&](uint32_t kb, uint32_t stage) {
    uint8_t* base = smem + stage * C::STAGE_BYTES;
    unroll_seq(
        [&](auto jc) {
          constexpr int J = decltype(jc)::value;
          if constexpr (FFN)
            dma16(J < 4 ? rA : rW2, c_off[J], kb * kGroup, base + c_lds[J] * 1024);
          else
            dma16(g0_act ? rA : rW, c_off[J], kb * kGroup, base + c_lds[J] * 1024);
        },
        std::make_integer_sequence<int, CH0>{});
  };
  auto issue_g1 = [&](uint32_t kb, uint32_t stage) {
    uint8_t* base = smem + stage * C::STAGE_BYTES;
    unroll_seq(
        [&](auto jc) {
          constexpr int J = decltype(jc)::value;
          dma16(FFN ? rW : rA, c_off[J], kb * kGroup, base + c_lds[J] * 1024);
        },
        std::make_integer_sequence<int, CH1>{});
    dma4(rS, s_off, kb * Mp * 4, base + my_sc);
    dma4(rS, s_off_p, kb * Mp * 4, base + p_sc);
    if constexpr (!ROW) {
      dma4(FFN ? rWs2 : rWs, ws_off, kb * 4, base + my_sc + 256);  // up scales in FFN mode
      dma4(rWs, ws_off, kb * 4, base + p_sc + 256);
    }
  };

  const uint32_t l16 = lane & 15, c0 = 2 * (lane >> 4);
  const uint32_t lo0 = l16 * 128 + ((c0 ^ swz(l16)) * 16);
  const uint32_t lo1 = l16 * 128 + (((c0 + 1) ^ swz(l16)) * 16);
  auto ld16 = [](const uint8_t* p) -> v4i { return *reinterpret_cast<const v4i*>(p); };
  auto ldf = [](const uint8_t* p) -> float { return *reinterpret_cast<const float*>(p); };
  const uint32_t a_row0 = wm * C::WM * 128, w_row0 = C::A_BYTES + wn * C::WN * 128;

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  v8i af[TM], bf[TN];
  float as[TM], ws = 0.0f, sc[TM], sc_tail = 0.0f;
  v4f p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // read this wave's fragments and scales from LDS slot S (18 LDS reads);
  // the slot is a compile-time constant, so every address is a loop-invariant
  // register plus an immediate offset
  // 16-row sub-tiles of this wave's band that hold rows below M (all TM
  // but in a last row tile that M ends inside; uniform over the wave)
  const uint32_t band0 = m0 + wm * C::WM;
  const uint32_t vt = FFN ? TM : (M <= band0 ? 0u : min((uint32_t)TM, (M - band0 + 15) / 16));
  // read this wave's fragments and scales from LDS slot S (18 LDS reads);
  // the slot is a compile-time constant, so every address is a loop-invariant
  // register plus an immediate offset.  Partial bands (FULL false) skip the
  // activation fragments of sub-tiles past M.
  auto read_block = [&](auto slot_c, auto full_c) {
    const uint8_t* sb = smem + decltype(slot_c)::value * C::STAGE_BYTES;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      bf[tn].lo = ld16(sb + w_row0 + tn * 2048 + lo0);
      bf[tn].hi = ld16(sb + w_row0 + tn * 2048 + lo1);
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      if (decltype(full_c)::value || (uint32_t)tm < vt) {
        af[tm].lo = ld16(sb + a_row0 + tm * 2048 + lo0);
        af[tm].hi = ld16(sb + a_row0 + tm * 2048 + lo1);
        as[tm] = ldf(sb + my_sc + (tm * 16 + l16) * 4);
      }
    }
    ws = ROW ? 1.0f : ldf(sb + my_sc + 256);
  };
  // MFMAs and promotions of the block in registers; the promotions of its
  // last kPromoteDist MFMAs are left pending for the next block's compute
  // phase.  A partial band runs only the MFMAs of its sub-tiles below M
  // (the others' accumulators hold rows that are never stored): in a last
  // row tile that M ends inside, the group's compute phase shrinks and the
  // matrix pipe spends no power on rows past M.
  auto compute_block = [&](auto full_c) {
    constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) sc[tm] = as[tm] * ws;
    unroll_seq(
        [&](auto ic) {
          constexpr int I = decltype(ic)::value;
          constexpr int tm = I / TN, tn = I % TN;
          if (FULL || (uint32_t)tm < vt) p[I & 3] = mfma_e4m3_128(bf[tn], af[tm]);
          if constexpr (I < kPromoteDist) {
            constexpr int J = NP - kPromoteDist + I;
            if (FULL || (uint32_t)(J / TN) < vt) acc[J / TN][J % TN] += p[J & 3] * sc_tail;
          } else {
            constexpr int J = I - kPromoteDist;
            if (FULL || (uint32_t)(J / TN) < vt) acc[J / TN][J % TN] += p[J & 3] * sc[J / TN];
          }
          sched_fence();
        },
        std::make_integer_sequence<int, NP>{});
    sc_tail = sc[TM - 1];
  };
  using FullT = std::true_type;
  using PartT = std::false_type;

  // Each group runs its own loop (its own body, so no value is live across
  // a merge of the two roles); both execute the same
  // sequence of workgroup barriers.  Every wave issues its part of stages
  // 0 .. STAGES-1 up front and its part of stage kb+STAGES (slot kb %
  // STAGES) in its read phase of iteration kb: group 1 in phase A, after its
  // own reads of block kb, only rows that group 0 alone reads (group 0 read
  // them one phase earlier); group 0 in phase B, after the phase-A barrier,
  // when both groups are done with block kb.  (A group-1 load of rows that
  // another group-1 wave reads could overwrite them before that wave has
  // read them: the direct loads land within a few hundred cycles when the
  // operands sit in L2.)
  // The K loop is unrolled by STAGES so that each copy's slot (kb % STAGES)
  // is a compile-time constant.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  static_assert(STAGES == 3, "the unrolled loop below assumes three slots");
  if (grp == 0) {
    // iteration kb: phase A computes block kb, phase B reads block kb+1
    // (block G: a reloaded copy of the last block, unused) and refills slot
    // kb % STAGES with block kb+STAGES
    auto run = [&](auto full_c) {
      auto step = [&](uint32_t kb, auto slot_c) {
        constexpr int S = decltype(slot_c)::value;
        compute_block(full_c);  // phase A
        wait_vmcnt<LW0>();      // own part of stage kb+1 (that of kb+2 may be in flight)
        wg_barrier();
        read_block(std::integral_constant<int, (S + 1) % STAGES>{}, full_c);  // phase B
        wait_lgkm0();
        issue_g0(min(kb + STAGES, G - 1), S);
        wg_barrier();
      };
#pragma unroll
      for (int s = 0; s < STAGES; ++s) issue_g0(min((uint32_t)s, G - 1), s);
      wait_vmcnt<(STAGES - 1) * LW0>();  // own part of stage 0
      wg_barrier();
      read_block(S0{}, full_c);
      wait_lgkm0();
      wg_barrier();
      uint32_t kb = 0;
      for (; kb + 3 <= G; kb += 3) {
        step(kb, S0{});
        step(kb + 1, S1{});
        step(kb + 2, S2{});
      }
      if (kb < G) step(kb, S0{});
      if (kb + 1 < G) step(kb + 1, S1{});
    };
    if (vt == (uint32_t)TM)
      run(FullT{});
    else
      run(PartT{});
  } else {
    // iteration kb: phase A reads block kb and refills its slot, phase B
    // computes it
    auto run = [&](auto full_c) {
      auto step = [&](uint32_t kb, auto slot_c) {
        constexpr int S = decltype(slot_c)::value;
        read_block(slot_c, full_c);  // phase A
        wait_lgkm0();
        issue_g1(min(kb + STAGES, G - 1), S);
        wait_vmcnt<2 * LW1>();  // own part of stage kb+1 (kb+2, kb+3 may be in flight)
        wg_barrier();
        compute_block(full_c);  // phase B
        wg_barrier();
      };
#pragma unroll
      for (int s = 0; s < STAGES; ++s) issue_g1(min((uint32_t)s, G - 1), s);
      wait_vmcnt<(STAGES - 1) * LW1>();  // own part of stage 0
      wg_barrier();
      wg_barrier();
      uint32_t kb = 0;
      for (; kb + 3 <= G; kb += 3) {
        step(kb, S0{});
        step(kb + 1, S1{});
        step(kb + 2, S2{});
      }
      if (kb < G) step(kb, S0{});
      if (kb + 1 < G) step(kb + 1, S1{});
    };
    if (vt == (uint32_t)TM)
      run(FullT{});
    else
      run(PartT{});
  }
  wait_vmcnt<0>();  // no direct load may still be writing LDS at exit
#pragma unroll
  for (int j = NP - kPromoteDist; j < NP; ++j) acc[j / TN][j % TN] += p[j & 3] * sc_tail;
  if constexpr (FFN) {
    ffn_epilogue<TM, TN>(acc, smem, ffn, wave, lane, m0 + wm * C::WM, n0 + (wn & 1) * C::WN, nb,
                         M, N, Mp);
    return;
  }
  if constexpr (ROW) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const float4 r = *reinterpret_cast<const float4*>(Ws + n0 + wn * C::WN + tn * 16 + 4 * (lane >> 4));
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) acc[tm][tn] *= v4f{r.x, r.y, r.z, r.w};
    }
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const uint32_t m = m0 + wm * C::WM + tm * 16 + l16;
    if (m < M) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const uint32_t n = n0 + wn * C::WN + tn * 16 + 4 * (lane >> 4);
        *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(acc[tm][tn]);
      }
    }
  }
}

template <int STAGES, bool ROW, bool FFN = false>
hipError_t launch_pp_cfg(const uint8_t* a, const float* a_s_km, const uint8_t* w, const float* w_s,
                         uint16_t* out, uint32_t M, uint32_t N, uint32_t K, hipStream_t s,
                         FfnArgs ffn = FfnArgs{nullptr, nullptr, nullptr, nullptr}) {
  using C = PpCfg<STAGES, ROW, FFN>;
  constexpr uint32_t BNO = FFN ? kGroup : C::BN;  // output columns per tile
  if (N % BNO != 0) return hipErrorInvalidValue;
  static std::atomic<bool> attr_set{false};  // the call is idempotent: racing threads repeat it
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_pp_kernel<STAGES, ROW, FFN>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  const uint32_t tiles_m = (M + C::BM - 1) / C::BM, tiles_n = N / BNO;
  gemm_pp_kernel<STAGES, ROW, FFN><<<dim3(tiles_m * tiles_n), dim3(C::NT), C::LDS_BYTES, s>>>(
      a, a_s_km, w, w_s, out, M, N, K, m_pad16(M), tiles_m, tiles_n, ffn);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// Stream-K form of the ping-pong kernel (block-scaled weights).  The grid
// holds C persistent workgroups, one per CU.  With T tiles of 256x128 and
// G = K/128 blocks each, workgroup q first computes whole tiles r*C + q for
// r < R = floor(T/C) (the data-parallel rounds).  The Tt = T - R*C tail
// tiles are cut along K into P pieces at block boundaries 0 = b_0 < b_1 <
// ... < b_P = G: workgroup q < Tt (a primary) computes piece 0 of tail tile
// q; the other S = C - Tt workgroups (secondaries) share the (P-1)*Tt later
// pieces, unit u = (p-1)*Tt + t (piece p of tail tile t) going to secondary
// u mod S in round u / S.  This keeps what makes the data-parallel rounds
// fast: at any moment the primaries run the same K block of consecutive
// tiles, and so do the secondaries, so the workgroups of one XCD read the
// same activation and weight panels and share them in its L2.  (Cutting the
// tail's iterations into one contiguous range per workgroup instead puts
// neighbouring workgroups at unrelated K offsets; the tail then runs at the
// rate of the memory behind the L2, slower than the data-parallel kernel's
// partly idle last wave.)  P and b_1 balance the two sides (sk_make_plan).
//
// All of a workgroup's segments run as one LDS pipeline: the loads of
// iteration i + STAGES may belong to the next segment, so a segment boundary
// costs no refill.  q numbers the workgroups XCD by XCD (workgroup ids are
// dealt round robin to the 8 XCDs), so consecutive tiles sit on one XCD.
//
// A secondary writes each piece's fp32 partial tile to the piece's slot of
// the workspace (slot t*(P-1) + p-1: a tile's partials are contiguous) (each wave its 64x64 part, in register order, with
// device-coherent stores), waits for the stores to complete, then writes the
// slot's per-wave flag with the call's generation number.  The primary, once
// its own piece is done, waits for the flags of pieces 1 .. P-1, reads those
// partials with device-coherent loads, adds them in piece order and stores
// the bf16 tile.  A wave gives up waiting after kSkSpinLimit polls and writes
// NaN, so every wave ends even if a partner never ran.  The sum differs from
// the single-pass kernels only in the fp32 association of the K blocks, and
// is the same run to run.
// ------------------------------------------------------------------------
struct SkPlan {
  uint32_t C;          // persistent workgroups (the grid)
  uint32_t rounds;     // data-parallel rounds R
  uint32_t tail_base;  // first tail tile = R * C
  uint32_t tail;       // tail tiles Tt, 0 < Tt < C
  uint32_t pieces;     // pieces per tail tile P >= 2; (P-1) * Tt <= C - Tt
  uint32_t b1;         // end of piece 0; pieces 1 .. P-1 split blocks [b1, G) evenly
};
struct SkArgs {
  float* part;                // [C][8 waves][16 MFMA tiles][64 lanes] x 4 fp32
  unsigned long long* flags;  // [C][8 waves]
  unsigned long long gen;     // generation number of this call
};
constexpr uint32_t kSkSpinLimit = 1u << 22;
// at most this many pieces per tail tile: a piece's partial costs its
// primary a 128 KB read, and one lane polls each piece's flags
constexpr uint32_t kSkMaxPieces = 16;
// minimum by value (a min returning a reference to its argument keeps the
// cursor fields in private memory, and loads from there count as per-lane)
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
// Cache policy of the partials' buffer stores and loads: sc1, the
// device-coherent form (coherent across the XCDs' L2 caches without an L2
// write-back or invalidate, which would stall every wave of the XCD).
constexpr int kCoherent = 16;

template <int STAGES>
__global__ __launch_bounds__(512) void gemm_pp_sk_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp, uint32_t tiles_m, uint32_t tiles_n, SkPlan plan, SkArgs sk) {
  using C = PpCfg<STAGES, false, false>;
  constexpr int TM = C::TM, TN = C::TN, NP = C::NP, BM = C::BM, BN = C::BN;
  constexpr int CH0 = C::CH0, CH1 = C::CH1, LW0 = C::LW0, LW1 = C::LW1;
  static_assert(STAGES == 3, "the unrolled loop below assumes three slots");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t G = K / kGroup;
  const uint32_t w = blockIdx.x;
  const uint32_t q = (plan.C % 8 == 0) ? (w % 8) * (plan.C / 8) + w / 8 : w;
  const uint32_t R = plan.rounds, Tt = plan.tail, S = plan.C - Tt;
  const uint32_t units = Tt * (plan.pieces - 1);
  const bool primary = q < Tt;
  // segments of this workgroup: R data-parallel tiles, then its tail work
  const uint32_t n_seg =
      R + (primary ? 1u : (q - Tt < units ? (units - (q - Tt) + S - 1) / S : 0u));
  if (n_seg == 0) return;  // uniform over the workgroup
  // first block of piece p >= 1
  auto bound = [&](uint32_t p) __attribute__((always_inline)) -> uint32_t {
    return plan.b1 + ((p - 1) * (G - plan.b1)) / (plan.pieces - 1);
  };
  // unit of segment k >= R of a secondary
  auto unit_of = [&](uint32_t k) __attribute__((always_inline)) -> uint32_t {
    return (q - Tt) + (k - R) * S;
  };
  // segment k: tile and K blocks kb0 .. kb1-1
  auto segment = [&](uint32_t k, uint32_t& tile, uint32_t& kb0, uint32_t& kb1)
      __attribute__((always_inline)) {
    if (k < R) {
      tile = q + k * plan.C;
      kb0 = 0;
      kb1 = G;
    } else if (primary) {
      tile = plan.tail_base + q;
      kb0 = 0;
      kb1 = plan.b1;
    } else {
      const uint32_t u = unit_of(k), p = 1 + u / Tt;
      tile = plan.tail_base + u % Tt;
      kb0 = bound(p);
      kb1 = bound(p + 1);
    }
  };

  // ---- iteration cursors (the load side runs STAGES iterations ahead) ----
  // Plain scalars, so that they stay in scalar registers.  Past the last
  // segment the load cursor stays on the last block, which the load side
  // then reloads (in bounds, unused).
  uint32_t l_seg = 0, l_tile, l_kb, l_kb1;  // load cursor
  segment(0, l_tile, l_kb, l_kb1);
  uint32_t c_seg = 0, c_tile = l_tile, c_kb0 = l_kb, c_kb1 = l_kb1;  // compute cursor
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(sk.part, plan.C * 8 * NP * 64 * 16);

  // The two wave groups run different halves of each step; each is compiled
  // for its group (grp a constant), so that every choice below that
  // depends on it folds away.
  auto body = [&](auto grp_c) __attribute__((always_inline)) {
    constexpr uint32_t grp = decltype(grp_c)::value;
    const uint32_t gw = wave & 3;
    const uint32_t wm = 2 * grp + (gw >> 1), wn = gw & 1;
    // Operand chunks of this wave, as in gemm_pp_kernel: group 1 loads
    // activation rows 0-127 (chunks 4*gw .. 4*gw+3) and the scales of itself
    // and of its group-0 partner; in group 0, waves 0 and 1 load activation
    // rows 128-255 (chunks 16 + 8*gw + j), waves 2 and 3 weight rows
    // (chunks 32 .. 47).  Each chunk is 8 rows of 128 bytes, row + lane/8 per
    // lane.  The per-lane offsets are relative to the tile's first row and
    // the same for every tile; the tile's origin is in the buffer resource
    // (rebuilt when the load cursor moves to another tile), whose bound ends
    // at row M: activation rows past M fall outside it and load as zeros
    // (without a memory access), and their outputs are not stored.
    constexpr int CH = grp ? CH1 : CH0;
    const bool act = grp || gw < 2;
    auto chunk = [&](int j) __attribute__((always_inline)) -> uint32_t {
      return grp ? 4 * gw + j : 16 + 8 * gw + j;
    };
    uint32_t c_off[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const uint32_t row = (act ? chunk(j) : chunk(j) - 32) * 8 + (lane >> 3), col = lane & 7;
      c_off[j] = row * K + (col ^ swz(row)) * 16;
    }
    const uint32_t my_sc = C::A_BYTES + C::W_BYTES + wave * C::SCW_BYTES;
    const uint32_t p_sc = C::A_BYTES + C::W_BYTES + gw * C::SCW_BYTES;
    __amdgpu_buffer_rsrc_t rOp;  // this wave's operand from the tile's origin
    uint32_t s_off = 0, s_off_p = 0, ws_off = 0;
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(As, G * Mp * 4);
    const __amdgpu_buffer_rsrc_t rWs = make_rsrc(Ws, (N / kGroup) * G * 4);
    auto load_offsets = [&](uint32_t tile) __attribute__((always_inline)) {
      uint32_t tmi, tni;
      grouped_tile(tile, tiles_m, tiles_n, tmi, tni);
      const uint32_t m0 = tmi * BM, n0 = tni * BN;
      rOp = act ? make_rsrc(A + (uint64_t)m0 * K, (M - m0) * K)
                : make_rsrc(W + (uint64_t)n0 * K, BN * K);
      if constexpr (grp == 1) {
        s_off = min(m0 + wm * C::WM + lane, Mp - 1) * 4;
        s_off_p = min(m0 + (gw >> 1) * C::WM + lane, Mp - 1) * 4;
        ws_off = (n0 / kGroup) * G * 4;
      }
    };
    load_offsets(l_tile);
    // after each issue: the next block, or the first of the next segment
    // (with the origin of its tile)
    auto load_next = [&]() __attribute__((always_inline)) {
      if (l_kb + 1 < l_kb1) {
        ++l_kb;
      } else if (l_seg + 1 < n_seg) {
        segment(++l_seg, l_tile, l_kb, l_kb1);
        load_offsets(l_tile);
      }
    };
    auto issue = [&](uint32_t stage) __attribute__((always_inline)) {
      // the LDS address of each chunk is formed here, from a base the
      // compiler cannot hoist (hoisted, the 3 x 8 chunk addresses would hold
      // 24 scalar registers through the loop)
      uint32_t lds = lds_addr(smem) + stage * C::STAGE_BYTES;
      asm volatile("" : "+s"(lds));
      const uint32_t kb = l_kb;
      unroll_seq(
          [&](auto jc) {
            constexpr int J = decltype(jc)::value;
            dma16_at(rOp, c_off[J], kb * kGroup, lds + chunk(J) * 1024);
          },
          std::make_integer_sequence<int, CH>{});
      if constexpr (grp == 1) {
        dma4_at(rS, s_off, kb * Mp * 4, lds + my_sc);
        dma4_at(rS, s_off_p, kb * Mp * 4, lds + p_sc);
        dma4_at(rWs, 0, ws_off + kb * 4, lds + my_sc + 256);
        dma4_at(rWs, 0, ws_off + kb * 4, lds + p_sc + 256);
      }
      load_next();
    };

    const uint32_t l16 = lane & 15, c0 = 2 * (lane >> 4);
    const uint32_t lo0 = l16 * 128 + ((c0 ^ swz(l16)) * 16);
    const uint32_t lo1 = l16 * 128 + (((c0 + 1) ^ swz(l16)) * 16);
    auto ld16 = [](const uint8_t* p) __attribute__((always_inline)) -> v4i { return *reinterpret_cast<const v4i*>(p); };
    auto ldf = [](const uint8_t* p) __attribute__((always_inline)) -> float { return *reinterpret_cast<const float*>(p); };
    const uint32_t a_row0 = wm * C::WM * 128, w_row0 = C::A_BYTES + wn * C::WN * 128;

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    v8i af[TM], bf[TN];
    float as[TM], ws = 0.0f, sc[TM], sc_tail = 0.0f;
    v4f p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto read_block = [&](auto slot_c) __attribute__((always_inline)) {
      const uint8_t* sb = smem + decltype(slot_c)::value * C::STAGE_BYTES;
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        bf[tn].lo = ld16(sb + w_row0 + tn * 2048 + lo0);
        bf[tn].hi = ld16(sb + w_row0 + tn * 2048 + lo1);
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        af[tm].lo = ld16(sb + a_row0 + tm * 2048 + lo0);
        af[tm].hi = ld16(sb + a_row0 + tm * 2048 + lo1);
        as[tm] = ldf(sb + my_sc + (tm * 16 + l16) * 4);
      }
      ws = ldf(sb + my_sc + 256);
    };
    auto compute_block = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) sc[tm] = as[tm] * ws;
      unroll_seq(
          [&](auto ic) {
            constexpr int I = decltype(ic)::value;
            constexpr int tm = I / TN, tn = I % TN;
            p[I & 3] = mfma_e4m3_128(bf[tn], af[tm]);
            // each promotion is pinned to its slot: with the segment-end
            // branches after the block the compiler would otherwise sink them
            // past the barrier (and keep every MFMA result live until then)
            if constexpr (I < kPromoteDist) {
              constexpr int J = NP - kPromoteDist + I;
              acc[J / TN][J % TN] += p[J & 3] * sc_tail;
              asm volatile("" : "+v"(acc[J / TN][J % TN]));
            } else {
              constexpr int J = I - kPromoteDist;
              acc[J / TN][J % TN] += p[J & 3] * sc[J / TN];
              asm volatile("" : "+v"(acc[J / TN][J % TN]));
            }
            sched_fence();
          },
          std::make_integer_sequence<int, NP>{});
      sc_tail = sc[TM - 1];
    };
    // the promotions still pending after a tile's last block; the next
    // block's pending slots then add zero
    auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = NP - kPromoteDist; j < NP; ++j) acc[j / TN][j % TN] += p[j & 3] * sc_tail;
      sc_tail = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    };
    // end of the compute cursor's segment: store, publish or finalize the
    // tile, then clear the accumulators
    auto epilogue = [&]() __attribute__((always_inline)) {
      flush();
      if (c_kb0 > 0) {
        // a later piece of a split tile: publish the partial (device-coherent
        // stores, complete before the flag is written)
        const uint32_t u = unit_of(c_seg);
        const uint32_t slot = (u % Tt) * (plan.pieces - 1) + u / Tt;
        const uint32_t voff = ((slot * 8 + wave) * NP * 64 + lane) * 16;
#pragma unroll
        for (int i = 0; i < NP; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i / TN][i % TN]),
                                                 rP, voff, i * 1024, kCoherent);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (lane == 0)
          __hip_atomic_store(&sk.flags[slot * 8 + wave], sk.gen, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      } else {
        if (c_kb1 < G) {
          // piece 0 of a tail tile: add the later pieces' partials.  Lane j
          // polls the flag of piece j + 1 (all pieces at once); the partials
          // are then read and added in piece order.  A
          // flag is cleared once its partial has been read, so that a replay
          // of the same launch (same generation number) waits afresh.
          const uint32_t np = plan.pieces - 1, slot0 = (c_tile - plan.tail_base) * np;
          unsigned long long* flag = &sk.flags[(slot0 + lane) * 8 + wave];
          uint32_t ok = 1;
          if (lane < np) {
            uint32_t n = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != sk.gen) {
              if (++n >= kSkSpinLimit) {
                ok = 0;
                break;
              }
              __builtin_amdgcn_s_sleep(2);
            }
          }
          const float bad = __builtin_amdgcn_ballot_w64(ok == 0) == 0 ? 0.0f : __builtin_nanf("");
          asm volatile("" ::: "memory");
          // device-coherent loads of the partials
          constexpr uint32_t vstride = 8 * NP * 64 * 16;  // from piece p to piece p + 1
          uint32_t voff = ((slot0 * 8 + wave) * NP * 64 + lane) * 16;
          for (uint32_t j = 0; j < np; ++j, voff += vstride) {
#pragma unroll
            for (int i = 0; i < NP; ++i)
              acc[i / TN][i % TN] += __builtin_bit_cast(
                                         v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rP, voff, i * 1024, kCoherent)) +
                                     bad;
          }
          if (lane < np && ok)
            __hip_atomic_store(flag, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        uint32_t tmi, tni;
        grouped_tile(c_tile, tiles_m, tiles_n, tmi, tni);
        const uint32_t m0 = tmi * BM, n0 = tni * BN;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const uint32_t m = m0 + wm * C::WM + tm * 16 + l16;
          if (m < M) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
              const uint32_t n = n0 + wn * C::WN + tn * 16 + 4 * (lane >> 4);
              *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(acc[tm][tn]);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    };

    // One pipeline step on LDS slot S, in two halves split by a barrier.
    // Group 0: compute the block read in the previous step | read the next
    // slot, issue the loads of iteration i + 3.  Group 1: read slot S, issue
    // | compute.  A segment's epilogue goes where the group holds nothing
    // but its accumulators: for group 0 between the halves of the segment's
    // last step (before it reads the next segment's first block), for
    // group 1 after it.
    auto half0 = [&](auto slot_c) __attribute__((always_inline)) {
      constexpr int S = decltype(slot_c)::value;
      if constexpr (grp == 0) {
        compute_block();
        wait_vmcnt<LW0>();
        wg_barrier();
      } else {
        read_block(slot_c);
        wait_lgkm0();
        issue(S);
        wait_vmcnt<2 * LW1>();
        wg_barrier();
      }
    };
    auto half1 = [&](auto slot_c) __attribute__((always_inline)) {
      constexpr int S = decltype(slot_c)::value;
      if constexpr (grp == 0) {
        read_block(std::integral_constant<int, (S + 1) % STAGES>{});
        wait_lgkm0();
        issue(S);
        wg_barrier();
      } else {
        compute_block();
        wg_barrier();
      }
    };
    auto step = [&](auto slot_c) __attribute__((always_inline)) {
      half0(slot_c);
      half1(slot_c);
    };
    // a half step on the slot known at run time
    auto dispatch = [&](uint32_t sl, auto&& half) __attribute__((always_inline)) {
      if (sl == 0)
        half(std::integral_constant<int, 0>{});
      else if (sl == 1)
        half(std::integral_constant<int, 1>{});
      else
        half(std::integral_constant<int, 2>{});
    };
    // The last step of a segment, with its epilogue.  In the workgroup's
    // final segment group 0 has no next block to hold, and runs its epilogue
    // after the second half, at the same time as group 1 (a tail tile's
    // final sum then costs one epilogue, not two in turn).
    auto last_step = [&](uint32_t sl) __attribute__((always_inline)) {
      const bool final_seg = c_seg + 1 >= n_seg;
      dispatch(sl, half0);
      if constexpr (grp == 0) {
        if (!final_seg) epilogue();
      }
      dispatch(sl, half1);
      if (grp == 1 || final_seg) epilogue();
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;

    // prologue: the first STAGES loads; group 0 reads slot 0
#pragma unroll
    for (int st = 0; st < STAGES; ++st) issue(st);
    if constexpr (grp == 0) {
      wait_vmcnt<(STAGES - 1) * LW0>();
      wg_barrier();
      read_block(S0{});
      wait_lgkm0();
      wg_barrier();
    } else {
      wait_vmcnt<(STAGES - 1) * LW1>();
      wg_barrier();
      wg_barrier();
    }
    // Iterations of each compute segment, i counting over the workgroup's
    // iterations (slot i % 3): all but the segment's last through the loop
    // unrolled by the three slots, the last one with the epilogue.
    uint32_t i = 0;
    while (true) {
      const uint32_t last = i + (c_kb1 - c_kb0) - 1;
      const uint32_t ph = i % 3;
      if (ph == 1 && i < last) {
        step(S1{});
        ++i;
      }
      if (i % 3 == 2 && i < last) {
        step(S2{});
        ++i;
      }
      for (; i + 3 <= last; i += 3) {
        step(S0{});
        step(S1{});
        step(S2{});
      }
      if (i < last) {
        step(S0{});
        ++i;
      }
      if (i < last) {
        step(S1{});
        ++i;
      }
      last_step(i % 3);
      ++i;
      if (c_seg + 1 >= n_seg) break;
      segment(++c_seg, c_tile, c_kb0, c_kb1);
    }
    wait_vmcnt<0>();  // no direct load may still be writing LDS at exit
  };
  if (wave >> 2)
    body(std::integral_constant<uint32_t, 1>{});
  else
    body(std::integral_constant<uint32_t, 0>{});
}

hipError_t launch_pp_sk_cfg(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                            const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                            const SkPlan& plan, const SkArgs& args, hipStream_t s) {
  using C = PpCfg<3, false, false>;
  static std::atomic<bool> attr_set{false};  // the call is idempotent: racing threads repeat it
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_pp_sk_kernel<3>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  const uint32_t tiles_m = (M + C::BM - 1) / C::BM, tiles_n = N / C::BN;
  gemm_pp_sk_kernel<3><<<dim3(plan.C), dim3(C::NT), C::LDS_BYTES, s>>>(
      a, a_s_km, w, w_s, out, M, N, K, m_pad16(M), tiles_m, tiles_n, plan, args);
  return hipGetLastError();
}

// ------------------------------------------------------------------------
// Skinny kernel for decode and small-batch widths.  Rows come in tiles of
// 16*TM <= 64 (grid dimension y; beyond 64 rows every row tile streams the
// weights again, mostly from the last-level cache).  The projection is then
// bound by streaming the weight matrix once, and the weight bytes must be
// spread evenly over the CUs: with one workgroup per 16 output columns
// (384 workgroups at N = 6144 on 256 CUs) half the CUs stream twice as much
// as the others.  So the grid has one workgroup per CU and workgroup w owns
// the contiguous column range [c0, c0 + cw), cw = N/grid rounded to 4
// columns, covered by ceil(cw/16) MFMA tiles of 16 columns (the last one
// partial: its missing weight rows are zero fragments, its missing columns
// are not stored).  The NWV waves take interleaved K blocks (wave w: blocks
// w, w+NWV, ...) for all of the workgroup's tiles; each wave issues the loads
// of U blocks before consuming any, the activation fragments of a block are
// loaded once for all tiles, and the NWV partial tiles are summed through
// LDS in wave order.
// ------------------------------------------------------------------------
// SPLIT: the K blocks are cut into gridDim.z contiguous ranges; workgroup
// (w, y, z) sums range z and stores its fp32 partial tile to part[z][M][N],
// which splitk_reduce_kernel adds in split order (block-scaled weights only).
template <int TM, int TN, int NWV, int U, bool ROW, bool SPLIT = false>
__global__ __launch_bounds__(64 * NWV) void gemm_skinny_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp, uint32_t units_base, uint32_t units_rem, float* __restrict__ part = nullptr) {
  static_assert(!(SPLIT && ROW), "split form for block-scaled weights only");
  // partial sums of the waves (dynamic LDS: NWV*TN*TM KB)
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  v4f(*red)[TN][TM][64] = reinterpret_cast<v4f(*)[TN][TM][64]>(smem);
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6, w = blockIdx.x;
  // this workgroup's columns, in units of 4
  const uint32_t c0 = 4 * (w * units_base + min(w, units_rem));
  const uint32_t c1 = c0 + 4 * (units_base + (w < units_rem ? 1u : 0u));
  const uint32_t nt = (c1 - c0 + 15) / 16;
  const uint32_t G = K / kGroup;
  const uint32_t l16 = lane & 15, kq = 32 * (lane >> 4);  // this lane's byte offset in a K block
  // operand rows: weight row c0 + 16t + l16 (zero beyond c1), activation row 16tm + l16
  const uint8_t* wrow[TN];
  bool wok[TN];
  uint32_t wsi[TN];  // weight-scale row of this lane's four output columns
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const uint32_t r = c0 + 16 * t + l16;
    wok[t] = r < c1;
    wrow[t] = W + (uint64_t)min(r, N - 1) * K + kq;
    wsi[t] = min(c0 + 16 * t + 4 * (lane >> 4), N - 1) / kGroup * G;
  }
  const uint32_t m0 = blockIdx.y * (16 * TM);  // this workgroup's rows
  const uint8_t* arow[TM];
  uint32_t srow[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const uint32_t m = m0 + tm * 16 + l16;
    arow[tm] = A + (uint64_t)min(m, M - 1) * K + kq;
    srow[tm] = min(m, Mp - 1);
  }

  v4f acc[TN][TM];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) acc[t][tm] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // this workgroup's K blocks [kbeg, kend): all of them, or split z's range
  const uint32_t kbeg = SPLIT ? blockIdx.z * G / gridDim.z : 0;
  const uint32_t kend = SPLIT ? (blockIdx.z + 1) * G / gridDim.z : G;
  for (uint32_t kb0 = kbeg + wave; kb0 < kend; kb0 += NWV * U) {
    v8i wf[U][TN], af[U][TM];
    float as[U][TM], ws[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = kb0 + u * NWV;
      if (k < kend) {
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          if ((uint32_t)t < nt) {
            if (wok[t]) {
              const u32x4* wp = reinterpret_cast<const u32x4*>(wrow[t] + (uint64_t)k * kGroup);
              wf[u][t] = join(__builtin_nontemporal_load(wp), __builtin_nontemporal_load(wp + 1));
            } else {
              wf[u][t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            }
            ws[u][t] = ROW ? 1.0f : Ws[wsi[t] + k];
          }
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const u32x4* ap = reinterpret_cast<const u32x4*>(arow[tm] + (uint64_t)k * kGroup);
          af[u][tm] = join(ap[0], ap[1]);
          as[u][tm] = As[(uint64_t)k * Mp + srow[tm]];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb0 + u * NWV < kend) {
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          if ((uint32_t)t < nt) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) {
              const v4f p = mfma_e4m3_128(wf[u][t], af[u][tm]);
              acc[t][tm] += p * (as[u][tm] * ws[u][t]);
            }
          }
        }
      }
    }
  }

#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) red[wave][t][tm][lane] = acc[t][tm];
  __syncthreads();
  // waves share the final sums: wave v sums and stores tiles (t, tm) with
  // t*TM + tm = v (mod NWV)
#pragma unroll
  for (int j = 0; j < TN * TM; ++j) {
    const int t = j / TM, tm = j % TM;
    if ((uint32_t)(j % NWV) == wave && (uint32_t)t < nt) {
      v4f s = red[0][t][tm][lane];
#pragma unroll
      for (int v = 1; v < NWV; ++v) s += red[v][t][tm][lane];
      const uint32_t m = m0 + tm * 16 + l16;
      const uint32_t n = c0 + 16 * t + 4 * (lane >> 4);
      if constexpr (ROW) {
        if (n < c1) {
          const float4 r = *reinterpret_cast<const float4*>(Ws + n);
          s *= v4f{r.x, r.y, r.z, r.w};
        }
      }
      if (m < M && n < c1) {
        if constexpr (SPLIT)
          *reinterpret_cast<v4f*>(part + ((uint64_t)blockIdx.z * M + m) * N + n) = s;
        else
          *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(s);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Decode-width kernel for the shapes whose per-workgroup weight slice fits
// in LDS (up to 32 rows, 16*TM <= 32 activation rows, at most 8*GW K
// blocks).  The projection streams the weight matrix once from HBM, and how
// the weight bytes are read decides its speed: fragment-layout loads (lane
// l: 32 bytes of row l%16, gemm_skinny_kernel) touch 16 rows K bytes apart
// with every instruction, while direct-to-LDS loads of whole 1 KB row pieces,
// all in flight at once, stream the same bytes about 1.6x faster (N = 6144,
// K = 5120 on 256 CUs, the weight read alone from HBM: 6.8 us against 10.7
// us).  Workgroup w owns the contiguous column range [c0, c0 + R) as in
// gemm_skinny_kernel; it loads the R weight rows into LDS (each row's K bytes
// contiguous and followed by a 16-byte pad, so that the 16 rows of an MFMA
// fragment read fall in 16 different bank quads), and, into registers, the
// activation fragments and the scales of the K blocks its waves take (wave
// v: blocks v, v+8, ..., every row tile, as gemm_skinny_kernel), all before
// the first wait.  Then the waves compute their blocks and add the 8 partial
// tiles in wave order through LDS: the same products as gemm_skinny_kernel,
// each wave's blocks added in an order rotated by the workgroup index.
// Measured at N = 6144, K = 5120 (weights from HBM, graph-timed back-to-back
// launches): 9.5 / 11.0 / 11.7 us at M = 16 / 17 / 25 against 12.6 / 14.0 /
// 14.8 us for gemm_skinny_kernel.  What remains above the bare weight stream
// is the activation reads (every workgroup reads all M x K activation bytes
// through its vector memory unit ahead of its weight loads: 0.7 us at M = 16,
// 2 us at M = 25) and the products, the reduction and the store after the
// single wait (about 1.8 us).  Waiting for the weight loads stage by stage,
// one K slot at a time, was slower: the barriers cost more than the overlap
// gains.
// ------------------------------------------------------------------------
constexpr uint32_t kDecodeMaxRows = 32, kDecodeLds = 150 * 1024;

template <int TM, int GW, bool ROW>
__global__ __launch_bounds__(512) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp, uint32_t units_base, uint32_t units_rem) {
  constexpr int NT = 2;  // 16-column MFMA tiles of the range (R <= 32)
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t w = blockIdx.x;
  const uint32_t c0 = 4 * (w * units_base + min(w, units_rem));
  const uint32_t R = 4 * (units_base + (w < units_rem ? 1u : 0u));  // columns = weight rows
  const uint32_t G = K / kGroup, rowb = K + 16;
  const uint32_t l16 = lane & 15, q = lane >> 4;

  // this wave's activation fragments and scales (L2-resident: every
  // workgroup reads them), and weight scales: issued first, ahead of the
  // weight stream.  Slot j holds
  // block wave + 8*((j + w) mod GW): the workgroups start their activation
  // reads at different blocks, so that the 32 CUs of an XCD do not all ask
  // its L2 for the same lines at once.
  const uint32_t nb_last = N / kGroup - 1, rot = w % GW;
  auto blk = [&](int j) __attribute__((always_inline)) -> uint32_t {
    const uint32_t jr = (uint32_t)j + rot;
    return wave + 8 * (jr >= (uint32_t)GW ? jr - GW : jr);
  };
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(A, M * K);  // M * K < 2^31 here
  v8i af[GW][TM];
  float as[GW][TM], ws[GW][NT];
#pragma unroll
  for (int j = 0; j < GW; ++j) {
    const uint32_t b = min(blk(j), G - 1);  // blocks past G: loaded, not used
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      // rows past M read at an offset beyond the buffer's range, which gives
      // zeros without a memory request (not a load under a branch: that
      // load would be waited for inside the branch, one L2 round trip per
      // fragment)
      const uint32_t m = 16 * tm + l16;
      const uint32_t off = m < M ? m * K + b * kGroup + 32 * q : 0x80000000u;
      af[j][tm] = join(__builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0),
                       __builtin_amdgcn_raw_buffer_load_b128(rA, off + 16, 0, 0));
      as[j][tm] = As[(uint64_t)b * Mp + min(m, Mp - 1)];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      ws[j][t] = ROW ? 1.0f : Ws[min((c0 + 16 * t + 4 * q) / kGroup, nb_last) * G + b];
  }
  // the weight rows: piece p of row r is bytes [1024 p, 1024 p + 1024) (the
  // last piece of a row may be shorter); loads dealt round robin to the waves
  const __amdgpu_buffer_rsrc_t rW = make_rsrc(W + (uint64_t)c0 * K, R * K);
  const uint32_t pieces = (K + 1023) / 1024, lds0 = lds_addr(smem);
#pragma unroll 1
  for (uint32_t i = wave; i < R * pieces; i += 8) {
    const uint32_t r = i / pieces, p = i % pieces;
    if (1024 * p + 16 * lane < K) dma16_at(rW, r * K + 1024 * p + 16 * lane, 0, lds0 + r * rowb + 1024 * p);
  }
  // the loaded registers are pinned here, before the wait: the compiler
  // would otherwise sink loads into the compute branches below, after the
  // barrier, and pay a second memory round trip there
#pragma unroll
  for (int j = 0; j < GW; ++j) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)  // (16-byte operands: valid on the host pass too)
      asm volatile("" ::"v"(af[j][tm].lo), "v"(af[j][tm].hi), "v"(as[j][tm]));
#pragma unroll
    for (int t = 0; t < NT; ++t) asm volatile("" ::"v"(ws[j][t]));
  }
  wait_vmcnt<0>();
  wg_barrier();

  // all weight fragments of this wave's blocks, then the products, then the
  // promotions (no LDS or MFMA latency between dependent steps); blocks past
  // G and rows past R give zero fragments
  v8i wf[GW][NT];
#pragma unroll
  for (int j = 0; j < GW; ++j)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t r = 16 * t + l16, b = min(blk(j), G - 1);
      const uint8_t* wr = smem + min(r, R - 1) * rowb + b * kGroup + 32 * q;
      wf[j][t] = join(*reinterpret_cast<const u32x4*>(wr), *reinterpret_cast<const u32x4*>(wr + 16));
      if (r >= R || blk(j) >= G) wf[j][t] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  v4f acc[NT][TM];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      v4f p[GW];
#pragma unroll
      for (int j = 0; j < GW; ++j) p[j] = mfma_e4m3_128(wf[j][t], af[j][tm]);
      acc[t][tm] = p[0] * (as[0][tm] * ws[0][t]);
#pragma unroll
      for (int j = 1; j < GW; ++j) acc[t][tm] += p[j] * (as[j][tm] * ws[j][t]);
    }
  wg_barrier();  // every wave done with the weight rows: LDS takes the partial tiles
  v4f* red = reinterpret_cast<v4f*>(smem);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) red[((wave * NT + t) * TM + tm) * 64 + lane] = acc[t][tm];
  wg_barrier();
  // waves share the final sums: wave v adds and stores tiles (t, tm) with
  // t*TM + tm = v (mod 8), the partials in wave order
  for (uint32_t jt = wave; jt < (uint32_t)(NT * TM); jt += 8) {
    const uint32_t t = jt / TM, tm = jt % TM;
    if (16 * t >= R) continue;
    v4f sum = red[(t * TM + tm) * 64 + lane];
    for (uint32_t v = 1; v < 8; ++v) sum += red[((v * NT + t) * TM + tm) * 64 + lane];
    const uint32_t m = 16 * tm + l16, n = c0 + 16 * t + 4 * q;
    if constexpr (ROW) {
      if (n < c0 + R) {
        const float4 rs = *reinterpret_cast<const float4*>(Ws + n);
        sum *= v4f{rs.x, rs.y, rs.z, rs.w};
      }
    }
    if (m < M && n < c0 + R) *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(sum);
  }
}

template <int TM, int GW, bool ROW>
hipError_t launch_decode_cfg(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                             const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                             uint32_t grid, uint32_t base, uint32_t rem, uint32_t lds,
                             hipStream_t s) {
  static std::atomic<bool> attr_set{false};  // idempotent: racing threads repeat it
  if (!attr_set.load(std::memory_order_acquire)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_decode_kernel<TM, GW, ROW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kDecodeLds);
    if (e != hipSuccess) return e;
    attr_set.store(true, std::memory_order_release);
  }
  gemm_decode_kernel<TM, GW, ROW><<<dim3(grid), dim3(512), lds, s>>>(
      a, a_s_km, w, w_s, out, M, N, K, m_pad16(M), base, rem);
  return hipGetLastError();
}

// Whether the decode kernel takes the shape (its limits: at most 32 rows and
// kDecodeMaxRows columns a workgroup, 48 K blocks, the slice within
// kDecodeLds), and then its template arguments and LDS bytes.
bool decode_plan(uint32_t M, uint32_t K, uint32_t base, uint32_t rem, uint32_t& tm, uint32_t& gw,
                 uint32_t& lds) {
  const uint32_t rmax = 4 * (base + (rem ? 1 : 0)), g = (K / kGroup + 7) / 8;
  const uint64_t l = std::max<uint64_t>((uint64_t)rmax * (K + 16), 8 * 2 * 2 * 64 * 16);
  if (M > 32 || rmax > kDecodeMaxRows || g > 6 || l > kDecodeLds) return false;
  tm = M <= 16 ? 1 : 2;
  gw = g <= 2 ? 2 : g <= 4 ? 4 : g == 5 ? 5 : 6;
  lds = (uint32_t)l;
  return true;
}

// the decode kernel where its shape limits hold (else false)
template <bool ROW>
bool launch_decode(const uint8_t* a, const float* a_s_km, const uint8_t* w, const float* w_s,
                   uint16_t* out, uint32_t M, uint32_t N, uint32_t K, uint32_t grid,
                   uint32_t base, uint32_t rem, hipStream_t s, hipError_t& err) {
  uint32_t tm = 0, gw = 0, l = 0;
  if (!decode_plan(M, K, base, rem, tm, gw, l)) return false;
#define FP8Q_DECODE(TM_, GW_) \
  err = launch_decode_cfg<TM_, GW_, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, l, s)
  if (tm == 1) {
    if (gw == 2) FP8Q_DECODE(1, 2);
    else if (gw == 4) FP8Q_DECODE(1, 4);
    else if (gw == 5) FP8Q_DECODE(1, 5);
    else FP8Q_DECODE(1, 6);
  } else {
    if (gw == 2) FP8Q_DECODE(2, 2);
    else if (gw == 4) FP8Q_DECODE(2, 4);
    else if (gw == 5) FP8Q_DECODE(2, 5);
    else FP8Q_DECODE(2, 6);
  }
#undef FP8Q_DECODE
  return true;
}

// Registers of a skinny wave: about 4*TN*TM accumulators + 4*TN + 3*TM + 20
// fixed, 9*TN + 9*TM per K block in flight.
constexpr int skinny_fixed_regs(int tm, int tn) { return 4 * tn * tm + 4 * tn + 3 * tm + 20; }
constexpr int skinny_block_regs(int tm, int tn) { return 9 * tn + 9 * tm; }
// Two waves per SIMD wherever the partial sums of eight fit in 128 KB of LDS,
// with the K blocks in flight that ~242 registers a wave leave (at least
// one).  Measured against one wave per SIMD with more blocks in flight (cold
// caches): TM = 2, TN = 6 (17-32 rows, N = 17408, K = 5120; two blocks
// against four): 28.9 / 30.1 / 30.8 against 31.4 / 32.5 / 33.2 us at M = 17
// / 25 / 32; TM = 4, TN = 4 (65-128 rows in 64-row tiles, 64 columns a
// workgroup; one block against four): 78.4-80.3 against 87.1-90.0 us at
// N = 5120, K = 17408 and 28.4-30.5 against 32.0-34.2 at N = 6144, K = 5120.
constexpr bool skinny_two_per_simd(int tm, int tn) { return 8 * tn * tm <= 128; }
// waves per workgroup: 8 where the rule above holds, else 4 where the
// partial sums of 4 fit in 128 KB (one wave per SIMD), else 2
constexpr int skinny_waves(int tm, int tn) {
  return skinny_two_per_simd(tm, tn) ? 8 : (128 / (tn * tm) >= 4) ? 4 : 2;
}
// K blocks in flight per wave: what the register budget leaves (~200 a wave
// at two waves per SIMD where eight waves' partial sums fit in 64 KB, as
// first tuned; 242 for the wider configurations; ~440 at one wave per SIMD)
constexpr int skinny_unroll(int tm, int tn) {
  const int budget = skinny_waves(tm, tn) != 8 ? 440 : (64 / (tn * tm) >= 8) ? 200 : 242;
  const int uf = (budget - skinny_fixed_regs(tm, tn)) / skinny_block_regs(tm, tn);
  return uf > 8 ? 8 : uf < 1 ? 1 : uf;
}
// the template arguments the skinny dispatch picks: row tiles TM of 16 rows,
// column tiles TN of 16 columns.  TM = 3 for 33-48 rows: against TM = 4 it
// leaves the registers for two K blocks in flight at TN = 4 (one at TM =
// 4) and loads a quarter fewer activation fragments; back to back over
// rotating weights, M = 33 / 48: single pass 41.1 / 46.4 -> 36.7 / 42.9 us
// at N = 5120, K = 17408 (3 splits 33.0 / 35.0 -> 30.3 / 32.8), 34.6 / 35.9
// -> 31.8 / 33.4 at N = 17408, K = 5120, 16.3 / 17.8 -> 15.2 / 16.9 at
// N = 6144, K = 5120.
uint32_t skinny_tm(uint32_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : M <= 48 ? 3 : 4; }
uint32_t skinny_tn(uint32_t tn) { return tn <= 2 ? 2 : tn <= 4 ? 4 : tn <= 6 ? 6 : 8; }

template <int TM, int TN, bool ROW, bool SPLIT = false>
hipError_t launch_skinny_tn(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                            const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                            uint32_t grid, uint32_t base, uint32_t rem, hipStream_t s,
                            uint32_t splits = 1, float* part = nullptr) {
  // LDS for the partial sums: NWV*TN*TM KB <= 128 KB; registers as above.
  constexpr int NWV = skinny_waves(TM, TN);
  constexpr int U = skinny_unroll(TM, TN);
  constexpr uint32_t LDS = NWV * TN * TM * 1024;
  static_assert(LDS <= 128 * 1024, "LDS for the partial sums");
  if constexpr (LDS > 64 * 1024) {
    static std::atomic<bool> attr_set{false};  // idempotent: racing threads repeat it
    if (!attr_set.load(std::memory_order_acquire)) {
      hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void*>(&gemm_skinny_kernel<TM, TN, NWV, U, ROW, SPLIT>),
          hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
      if (e != hipSuccess) return e;
      attr_set.store(true, std::memory_order_release);
    }
  }
  const uint32_t row_tiles = (M + 16 * TM - 1) / (16 * TM);
  gemm_skinny_kernel<TM, TN, NWV, U, ROW, SPLIT>
      <<<dim3(grid, row_tiles, splits), dim3(64 * NWV), LDS, s>>>(a, a_s_km, w, w_s, out, M, N, K,
                                                                  m_pad16(M), base, rem, part);
  return hipGetLastError();
}

template <int TM, bool ROW, bool SPLIT = false>
hipError_t launch_skinny_tm(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                            const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                            uint32_t grid, uint32_t base, uint32_t rem, uint32_t tn, hipStream_t s,
                            uint32_t splits = 1, float* part = nullptr) {
#define FP8Q_SKINNY(TN_) \
  launch_skinny_tn<TM, TN_, ROW, SPLIT>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, s, splits, part)
  if (tn <= 2) return FP8Q_SKINNY(2);
  if (tn <= 4) return FP8Q_SKINNY(4);
  if (tn <= 6) return FP8Q_SKINNY(6);
  return FP8Q_SKINNY(8);
#undef FP8Q_SKINNY
}

}  // namespace

namespace {
template <bool ROW>
hipError_t launch_gemm_tiled_t(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                               const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                               int cfg, hipStream_t s) {
  switch (cfg) {
    case 0:
    case 1: return launch_tiled_cfg<128, 128, 2, 2, 2, ROW>(a, a_s_km, w, w_s, out, M, N, K, s);
    case 2: return launch_tiled_cfg<256, 128, 4, 2, 3, ROW>(a, a_s_km, w, w_s, out, M, N, K, s);
    case 3: return launch_tiled_cfg<256, 128, 2, 2, 3, ROW>(a, a_s_km, w, w_s, out, M, N, K, s);
    case 4: return launch_pp_cfg<3, ROW>(a, a_s_km, w, w_s, out, M, N, K, s);
    default: return hipErrorInvalidValue;
  }
}

// The skinny path's grid.  Up to 64 rows (one row tile): one workgroup per
// CU, at most 128 columns each, at least 16.  Beyond (several row tiles,
// each streaming the weights again): workgroups of 64 columns, so that a row
// tile re-reads the activations once per 64 columns rather than once per CU
// (measured at M = 128, N = 5120, K = 17408: 90 us with 64-column
// workgroups, 108 us with one per CU, 117 us for the ping-pong kernel).
// Workgroup w owns 4*(base + (w < rem)) columns; tn 16-column tiles at most.
void skinny_grid(uint32_t M, uint32_t N, uint32_t cu_count, uint32_t& grid, uint32_t& base,
                 uint32_t& rem, uint32_t& tn) {
  const uint32_t units = N / 4;
  grid = max(cu_count, (N + 127) / 128);
  grid = max(1u, min(grid, N / 16));
  if (M > 64) grid = N / 64;
  base = units / grid;
  rem = units % grid;
  tn = (4 * (base + (rem ? 1 : 0)) + 15) / 16;
}

template <bool ROW>
hipError_t launch_gemm_skinny_t(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                                const float* w_s, uint16_t* out, uint32_t M, uint32_t N,
                                uint32_t K, uint32_t cu_count, hipStream_t s) {
  uint32_t grid = 0, base = 0, rem = 0, tn = 0;
  skinny_grid(M, N, cu_count, grid, base, rem, tn);
  hipError_t err = hipSuccess;
  if (launch_decode<ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, s, err)) return err;
  switch ((M + 15) / 16) {
    case 1: return launch_skinny_tm<1, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, tn, s);
    case 2: return launch_skinny_tm<2, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, tn, s);
    case 3: return launch_skinny_tm<3, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, tn, s);
    default: return launch_skinny_tm<4, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, tn, s);
  }
}
}  // namespace

hipError_t launch_gemm_tiled(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                             const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                             int cfg, bool row_scaled, hipStream_t s) {
  return row_scaled ? launch_gemm_tiled_t<true>(a, a_s_km, w, w_s, out, M, N, K, cfg, s)
                    : launch_gemm_tiled_t<false>(a, a_s_km, w, w_s, out, M, N, K, cfg, s);
}

bool decode_takes(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count) {
  uint32_t grid = 0, base = 0, rem = 0, tn = 0, tm = 0, gw = 0, lds = 0;
  skinny_grid(M, N, cu_count, grid, base, rem, tn);
  return decode_plan(M, K, base, rem, tm, gw, lds);
}

uint32_t skinny_split_grid(uint32_t N, uint32_t splits, uint32_t cus) {
  return max(1u, min(max(cus / max(splits, 1u), 1u), N / 16));
}

uint32_t skinny_split_columns(uint32_t N, uint32_t splits, uint32_t cus) {
  const uint32_t units = N / 4, grid = skinny_split_grid(N, splits, cus);
  return 4 * ((units + grid - 1) / grid);
}

hipError_t launch_gemm_skinny(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                              const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                              uint32_t cu_count, bool row_scaled, hipStream_t s) {
  return row_scaled ? launch_gemm_skinny_t<true>(a, a_s_km, w, w_s, out, M, N, K, cu_count, s)
                    : launch_gemm_skinny_t<false>(a, a_s_km, w, w_s, out, M, N, K, cu_count, s);
}

// Split-K form of the skinny kernel (up to 64 rows, block-scaled weights):
// splits * W workgroups, W = cus / splits column ranges (at least 16 columns
// each, at most 128), each summing its split's K range into part[split];
// then the reduction.  False (nothing launched) where the ranges would be
// wider than 128 columns.
bool launch_skinny_split(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                         const float* w_s, uint16_t* out, float* part, uint32_t M, uint32_t N,
                         uint32_t K, uint32_t splits, uint32_t cus, hipStream_t s,
                         hipError_t& err) {
  if (M == 0 || M > 64 || splits < 2) return false;
  const uint32_t units = N / 4;
  const uint32_t grid = skinny_split_grid(N, splits, cus);
  const uint32_t base = units / grid, rem = units % grid;
  const uint32_t cols = skinny_split_columns(N, splits, cus);
  if (cols > 128) return false;
  const uint32_t tn = (cols + 15) / 16;
  switch ((M + 15) / 16) {
    case 1: err = launch_skinny_tm<1, false, true>(a, a_s_km, w, w_s, nullptr, M, N, K, grid, base, rem, tn, s, splits, part); break;
    case 2: err = launch_skinny_tm<2, false, true>(a, a_s_km, w, w_s, nullptr, M, N, K, grid, base, rem, tn, s, splits, part); break;
    case 3: err = launch_skinny_tm<3, false, true>(a, a_s_km, w, w_s, nullptr, M, N, K, grid, base, rem, tn, s, splits, part); break;
    default: err = launch_skinny_tm<4, false, true>(a, a_s_km, w, w_s, nullptr, M, N, K, grid, base, rem, tn, s, splits, part); break;
  }
  if (err != hipSuccess) return true;
  const uint64_t quads = (uint64_t)M * N / 4;
  const uint64_t blocks = (quads + 255) / 256;
  const uint32_t rgrid = (uint32_t)(blocks < 4096 ? blocks : 4096);
  splitk_reduce_kernel<<<dim3(rgrid), dim3(256), 0, s>>>(reinterpret_cast<const v4f*>(part),
                                                         reinterpret_cast<uint2*>(out), quads, splits);
  err = hipGetLastError();
  return true;
}

void gemm_skinny_kernel_name(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count,
                             bool row_scaled, char* buf, size_t len) {
  uint32_t grid = 0, base = 0, rem = 0, tn = 0, tm = 0, gw = 0, lds = 0;
  skinny_grid(M, N, cu_count, grid, base, rem, tn);
  const char* row = row_scaled ? "true" : "false";
  if (decode_plan(M, K, base, rem, tm, gw, lds)) {
    snprintf(buf, len, "gemm_decode_kernel<%u, %u, %s>", tm, gw, row);
  } else {
    const int t = (int)skinny_tm(M), n = (int)skinny_tn(tn);
    snprintf(buf, len, "gemm_skinny_kernel<%d, %d, %d, %d, %s>", t, n, skinny_waves(t, n),
             skinny_unroll(t, n), row);
  }
}

hipError_t launch_ffn_gate_up(const uint8_t* x, const float* x_s_km, const uint8_t* w_gate,
                              const float* ws_gate, const uint8_t* w_up, const float* ws_up,
                              uint8_t* hq, float* hs_km, uint32_t M, uint32_t H, uint32_t I,
                              hipStream_t s) {
  return launch_pp_cfg<3, false, true>(x, x_s_km, w_gate, ws_gate, nullptr, M, I, H, s,
                                       FfnArgs{w_up, ws_up, hq, hs_km});
}

hipError_t launch_splitk_128(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                             const float* w_s, uint16_t* out, float* part, uint32_t M,
                             uint32_t N, uint32_t K, uint32_t splits, uint32_t cus,
                             hipStream_t s) {
  return launch_splitk_128_t(a, a_s_km, w, w_s, out, part, M, N, K, splits, cus, s);
}

namespace {
// Stream-K plan on `cus` CUs, or false where the data-parallel kernel is as
// good: no tail (the tiles fill whole rounds), fewer tiles than CUs, a tail
// round more than 90% full, or fewer than 4 tail iterations a workgroup.
// The stream-K plan for M x N x K on cus workgroups, or false where the
// data-parallel kernels are expected to be as fast (unless forced: then
// wherever the structure allows one).  In units of one K
// block's time: the longest workgroup runs R*G + crit + (P-1)*kSkPartialCost
// + kSkPollCost (its own blocks, then reading P-1 partials and waiting on
// their flags, measured at about 4.5 and 8 block times), against R*G +
// G*max(Tt/cus, kSkLastWave) for the data-parallel kernel, whose last wave
// of Tt tiles runs at a higher clock while the other CUs idle (the chip is
// power-limited: 24 tiles alone took 0.73 of a full wave's time).  The plan
// is kept where it is at least 10% shorter.  With more than cus/2 tail
// tiles, P = 2: the S secondaries take the tiles' second pieces in r =
// ceil(Tt/S) rounds, and b1 minimizes crit = max(b1, r*(G - b1)).  With
// fewer, near-equal pieces, P in [2, min(cus/Tt, G, kSkMaxPieces)] chosen
// for the least crit + (P-1)*kSkPartialCost, at most one unit per secondary.
constexpr uint64_t kSkPartialCost = 5, kSkPollCost = 8;
constexpr double kSkLastWave = 0.73;
bool sk_make_plan(uint32_t M, uint32_t N, uint32_t K, uint32_t cus, bool forced, SkPlan& p) {
  const uint64_t T = (uint64_t)((M + 255) / 256) * (N / 128), G = K / kGroup;
  if (cus < 8 || cus % 8 != 0 || N % 128 != 0 || G < 2 || T <= cus || T % cus == 0)
    return false;
  const uint64_t R = T / cus, Tt = T % cus, S = cus - Tt;
  uint64_t P = 2, b1, crit;
  if (2 * Tt > cus) {
    const uint64_t r = (Tt + S - 1) / S;
    auto cost = [&](uint64_t b) { return std::max(b, r * (G - b)); };
    b1 = std::min<uint64_t>(std::max<uint64_t>((r * G) / (r + 1), 1), G - 1);
    if (b1 + 1 < G && cost(b1 + 1) < cost(b1)) ++b1;
    crit = cost(b1);
  } else {
    const uint64_t pmax = std::min<uint64_t>(std::min<uint64_t>(cus / Tt, G), kSkMaxPieces);
    auto cost = [&](uint64_t q) { return std::max(G / q, (G - G / q + q - 2) / (q - 1)); };
    for (uint64_t q = 3; q <= pmax; ++q)
      if (cost(q) + (q - 1) * kSkPartialCost < cost(P) + (P - 1) * kSkPartialCost) P = q;
    b1 = G / P;
    crit = cost(P);
  }
  const double sk = (double)(R * G + crit + (P - 1) * kSkPartialCost + kSkPollCost);
  const double dp = (double)(R * G) + (double)G * std::max((double)Tt / cus, kSkLastWave);
  if (!forced && sk > 0.9 * dp) return false;
  p.C = cus;
  p.rounds = (uint32_t)R;
  p.tail_base = (uint32_t)(R * cus);
  p.tail = (uint32_t)Tt;
  p.pieces = (uint32_t)P;
  p.b1 = (uint32_t)b1;
  return true;
}

// generation numbers: a per-process random start, then one per call
std::atomic<unsigned long long> g_sk_gen{0};
unsigned long long sk_next_gen() {
  static const unsigned long long base = [] {
    unsigned long long v = (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    v ^= (unsigned long long)(uintptr_t)&g_sk_gen;
    return v * 0x9E3779B97F4A7C15ull;
  }();
  return base + 0xD1B54A32D192ED03ull * (g_sk_gen.fetch_add(1, std::memory_order_relaxed) + 1);
}

uint64_t sk_flag_bytes(uint32_t cus) { return ((uint64_t)cus * 8 * 8 + 255) / 256 * 256; }
}  // namespace

bool gemm_streamk_applies(uint32_t M, uint32_t N, uint32_t K, uint32_t cus, bool forced) {
  SkPlan p;
  return sk_make_plan(M, N, K, cus, forced, p);
}

uint64_t gemm_streamk_workspace_bytes(uint32_t cus) {
  return sk_flag_bytes(cus) + (uint64_t)cus * 8 * 16 * 64 * 16;
}

hipError_t launch_gemm_streamk(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                               const float* w_s, uint16_t* out, void* workspace, uint32_t M,
                               uint32_t N, uint32_t K, uint32_t cus, bool forced, hipStream_t s) {
  SkPlan plan;
  if (!sk_make_plan(M, N, K, cus, forced, plan)) return hipErrorInvalidValue;
  SkArgs args;
  args.flags = static_cast<unsigned long long*>(workspace);
  args.part = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + sk_flag_bytes(cus));
  args.gen = sk_next_gen();
  return launch_pp_sk_cfg(a, a_s_km, w, w_s, out, M, N, K, plan, args, s);
}

}  // namespace fp8q
