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
#include "mfma_common.h"
#include "quant_common.h"

namespace fp8q {
namespace {

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
// has been issued).  The fp32 promotion of MFMA i is issued after MFMA i+2, so
// the vector ALU never waits for the matrix pipe; the promotions of a block's
// last two MFMAs run in the next block.  Each MFMA slot (the MFMA, the four
// fmas, one or two LDS reads) is fenced off from the next with a scheduling
// barrier: left to itself the compiler hoists all MFMAs of a block and then
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
  // two MFMAs of a block are pending when the next block starts (zero before
  // the first block).
  v4f p[4];
  p[(NP - 2) & 3] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  p[(NP - 1) & 3] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
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
          if constexpr (I < 2) {
            constexpr int J = NP - 2 + I;
            acc[J / TN][J % TN] += p[J & 3] * sc_tail;
          } else {
            constexpr int J = I - 2;
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
  // promotions of the last block's last two MFMAs (both in its last row)
  acc[(NP - 2) / TN][(NP - 2) % TN] += p[(NP - 2) & 3] * sc_tail;
  acc[(NP - 1) / TN][(NP - 1) % TN] += p[(NP - 1) & 3] * sc_tail;

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

// Split grids that fit one workgroup per CU (kSplitOneRoundWgs) take three
// LDS stages (99 KB: one workgroup per CU, two blocks of loads in flight);
// larger ones two (two workgroups per CU).  Measured with cold caches at
// N = 5120, K = 17408: 44.2 / 47.8 / 56.5 us against 46.0 / 50.9 / 64.5 us
// at M = 65 / 128 / 256; at N = 6144, K = 5120: 22.2 / 25.4 / 32.3 against
// 23.2 / 27.5 / 36.3 us.
constexpr uint32_t kSplitOneRoundWgs = 256;

hipError_t launch_splitk_128_t(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                               const float* w_s, uint16_t* out, float* part, uint32_t M,
                               uint32_t N, uint32_t K, uint32_t splits, hipStream_t s) {
  if (N % 128 != 0 || splits < 2 || splits > K / kGroup) return hipErrorInvalidValue;
  const uint64_t wgs = (uint64_t)((M + 127) / 128) * (N / 128) * splits;
  hipError_t e = wgs <= kSplitOneRoundWgs
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
  p[(NP - 2) & 3] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  p[(NP - 1) & 3] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // read this wave's fragments and scales from LDS slot S (18 LDS reads);
  // the slot is a compile-time constant, so every address is a loop-invariant
  // register plus an immediate offset
  auto read_block = [&](auto slot_c) {
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
    ws = ROW ? 1.0f : ldf(sb + my_sc + 256);
  };
  // MFMAs and promotions of the block in registers; the promotions of its
  // last two MFMAs are left pending for the next block's compute phase.
  auto compute_block = [&]() {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) sc[tm] = as[tm] * ws;
    unroll_seq(
        [&](auto ic) {
          constexpr int I = decltype(ic)::value;
          constexpr int tm = I / TN, tn = I % TN;
          p[I & 3] = mfma_e4m3_128(bf[tn], af[tm]);
          if constexpr (I < 2) {
            constexpr int J = NP - 2 + I;
            acc[J / TN][J % TN] += p[J & 3] * sc_tail;
          } else {
            constexpr int J = I - 2;
            acc[J / TN][J % TN] += p[J & 3] * sc[J / TN];
          }
          sched_fence();
        },
        std::make_integer_sequence<int, NP>{});
    sc_tail = sc[TM - 1];
  };

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
    auto step = [&](uint32_t kb, auto slot_c) {
      constexpr int S = decltype(slot_c)::value;
      compute_block();    // phase A
      wait_vmcnt<LW0>();  // own part of stage kb+1 (that of kb+2 may be in flight)
      wg_barrier();
      read_block(std::integral_constant<int, (S + 1) % STAGES>{});  // phase B
      wait_lgkm0();
      issue_g0(min(kb + STAGES, G - 1), S);
      wg_barrier();
    };
#pragma unroll
    for (int s = 0; s < STAGES; ++s) issue_g0(min((uint32_t)s, G - 1), s);
    wait_vmcnt<(STAGES - 1) * LW0>();  // own part of stage 0
    wg_barrier();
    read_block(S0{});
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
  } else {
    // iteration kb: phase A reads block kb and refills its slot, phase B
    // computes it
    auto step = [&](uint32_t kb, auto slot_c) {
      constexpr int S = decltype(slot_c)::value;
      read_block(slot_c);  // phase A
      wait_lgkm0();
      issue_g1(min(kb + STAGES, G - 1), S);
      wait_vmcnt<2 * LW1>();  // own part of stage kb+1 (kb+2, kb+3 may be in flight)
      wg_barrier();
      compute_block();  // phase B
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
  }
  wait_vmcnt<0>();  // no direct load may still be writing LDS at exit
  acc[(NP - 2) / TN][(NP - 2) % TN] += p[(NP - 2) & 3] * sc_tail;
  acc[(NP - 1) / TN][(NP - 1) % TN] += p[(NP - 1) & 3] * sc_tail;
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
template <int TM, int TN, int NWV, int U, bool ROW>
__global__ __launch_bounds__(64 * NWV) void gemm_skinny_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp, uint32_t units_base, uint32_t units_rem) {
  __shared__ v4f red[NWV][TN][TM][64];
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

  for (uint32_t kb0 = wave; kb0 < G; kb0 += NWV * U) {
    v8i wf[U][TN], af[U][TM];
    float as[U][TM], ws[U][TN];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = kb0 + u * NWV;
      if (k < G) {
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
      if (kb0 + u * NWV < G) {
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
      if (m < M && n < c1) *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(s);
    }
  }
}

template <int TM, int TN, bool ROW>
hipError_t launch_skinny_tn(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                            const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                            uint32_t grid, uint32_t base, uint32_t rem, hipStream_t s) {
  // static LDS for the partial sums: NWV*TN*TM KB <= 64 KB.  Registers: about
  // 4*TN*TM accumulators + 4*TN + 3*TM + 20 fixed, 9*TN + 9*TM per K block in
  // flight, within ~200 (two waves per SIMD, NWV = 8) or ~440 (one wave).
  constexpr int NWV = (64 / (TN * TM) >= 8) ? 8 : (64 / (TN * TM) >= 4) ? 4 : 2;
  constexpr int FIXED = 4 * TN * TM + 4 * TN + 3 * TM + 20;
  constexpr int PER = 9 * TN + 9 * TM;
  constexpr int BUDGET = NWV == 8 ? 200 : 440;
  constexpr int UF = (BUDGET - FIXED) / PER;
  constexpr int U = UF > 8 ? 8 : UF < 1 ? 1 : UF;
  static_assert(NWV * TN * TM <= 64, "LDS for the partial sums");
  const uint32_t row_tiles = (M + 16 * TM - 1) / (16 * TM);
  gemm_skinny_kernel<TM, TN, NWV, U, ROW><<<dim3(grid, row_tiles), dim3(64 * NWV), 0, s>>>(
      a, a_s_km, w, w_s, out, M, N, K, m_pad16(M), base, rem);
  return hipGetLastError();
}

template <int TM, bool ROW>
hipError_t launch_skinny_tm(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                            const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                            uint32_t grid, uint32_t base, uint32_t rem, uint32_t tn, hipStream_t s) {
  if (tn <= 2) return launch_skinny_tn<TM, 2, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, s);
  if (tn <= 4) return launch_skinny_tn<TM, 4, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, s);
  if (tn <= 6) return launch_skinny_tn<TM, 6, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, s);
  return launch_skinny_tn<TM, 8, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, s);
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

template <bool ROW>
hipError_t launch_gemm_skinny_t(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                                const float* w_s, uint16_t* out, uint32_t M, uint32_t N,
                                uint32_t K, uint32_t cu_count, hipStream_t s) {
  // Up to 64 rows (one row tile): one workgroup per CU, at most 128 columns
  // each, at least 16.  Beyond (several row tiles, each streaming the
  // weights again): workgroups of 64 columns, so that a row tile re-reads
  // the activations once per 64 columns rather than once per CU (measured
  // at M = 128, N = 5120, K = 17408: 90 us with 64-column workgroups, 108 us
  // with one per CU, 117 us for the ping-pong kernel).
  const uint32_t units = N / 4;
  uint32_t grid = max(cu_count, (N + 127) / 128);
  grid = max(1u, min(grid, N / 16));
  if (M > 64) grid = N / 64;
  const uint32_t base = units / grid, rem = units % grid;
  const uint32_t tn = (4 * (base + (rem ? 1 : 0)) + 15) / 16;
  switch ((M + 15) / 16) {
    case 1: return launch_skinny_tm<1, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, tn, s);
    case 2: return launch_skinny_tm<2, ROW>(a, a_s_km, w, w_s, out, M, N, K, grid, base, rem, tn, s);
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

hipError_t launch_gemm_skinny(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                              const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                              uint32_t cu_count, bool row_scaled, hipStream_t s) {
  return row_scaled ? launch_gemm_skinny_t<true>(a, a_s_km, w, w_s, out, M, N, K, cu_count, s)
                    : launch_gemm_skinny_t<false>(a, a_s_km, w, w_s, out, M, N, K, cu_count, s);
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
                             uint32_t N, uint32_t K, uint32_t splits, hipStream_t s) {
  return launch_splitk_128_t(a, a_s_km, w, w_s, out, part, M, N, K, splits, s);
}

}  // namespace fp8q
