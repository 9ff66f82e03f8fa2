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
#include "fp8q_internal.h"

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_e4m3_128(const v8i& w, const v8i& a) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // cbsz = blgp = 0: both operands OCP e4m3; zero scale operands select the
  // unscaled instruction.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, zero, 0, 0, 0, 0, 0, 0);
}

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

// ------------------------------------------------------------------------
// LDS-tiled kernel.  Workgroup tile BM x BN, K step 128 (one scale block),
// WAVES_M x WAVES_N waves, each owning a (BM/WAVES_M) x (BN/WAVES_N) sub-tile.
// LDS holds two stages of [BM + BN rows][128 B]; 16-byte chunk c of row r is
// stored at chunk position c ^ (r & 7) so that the 16 lanes reading the same
// chunk column of 16 consecutive rows spread over the banks.
// ------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_tiled_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp, uint32_t tiles_m, uint32_t tiles_n) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int CA = BM * 8 / NT, CW = BN * 8 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must sit in one 128-block");
  __shared__ u32x4 lds[2][(BM + BN) * 8];

  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t wm = wave / WAVES_N, wn = wave % WAVES_N;

  // Tile order: consecutive workgroup ids walk down M inside a column strip
  // of tiles so that concurrently running workgroups share weight tiles.
  const uint32_t tile = blockIdx.x;
  const uint32_t tmi = tile % tiles_m, tni = tile / tiles_m;
  const uint32_t m0 = tmi * BM, n0 = tni * BN;
  const uint32_t G = K / kGroup;
  const uint32_t nb = (n0 + wn * WN) / kGroup;

  u32x4 ra[CA], rw[CW];
  auto gload = [&](uint32_t kb) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const uint32_t q = tid + i * NT, row = q >> 3, c = q & 7;
      const uint32_t grow = min(m0 + row, M - 1);
      ra[i] = *reinterpret_cast<const u32x4*>(A + (uint64_t)grow * K + kb * kGroup + c * 16);
    }
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const uint32_t q = tid + i * NT, row = q >> 3, c = q & 7;
      rw[i] = *reinterpret_cast<const u32x4*>(W + (uint64_t)(n0 + row) * K + kb * kGroup + c * 16);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const uint32_t q = tid + i * NT, row = q >> 3, c = q & 7;
      lds[buf][row * 8 + (c ^ (row & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const uint32_t q = tid + i * NT, row = q >> 3, c = q & 7;
      lds[buf][(BM + row) * 8 + (c ^ (row & 7))] = rw[i];
    }
  };
  auto frag = [&](int buf, uint32_t row) -> v8i {
    const uint32_t c0 = 2 * (lane >> 4), sw = row & 7;
    return join(lds[buf][row * 8 + (c0 ^ sw)], lds[buf][row * 8 + ((c0 + 1) ^ sw)]);
  };

  // activation-scale rows of this lane (clamped into the Mp-wide buffer;
  // rows >= M are computed but never stored)
  uint32_t srow[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) srow[tm] = min(m0 + wm * WM + tm * 16 + (lane & 15), Mp - 1);

  v4f acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  float as_next[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) as_next[tm] = As[srow[tm]];
  float ws_next = Ws[(uint64_t)nb * G];

  gload(0);
  lstore(0);
  __syncthreads();

  for (uint32_t kb = 0; kb < G; ++kb) {
    const int cur = kb & 1;
    float sc[TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) sc[tm] = as_next[tm] * ws_next;
    if (kb + 1 < G) {
      gload(kb + 1);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) as_next[tm] = As[(uint64_t)(kb + 1) * Mp + srow[tm]];
      ws_next = Ws[(uint64_t)nb * G + kb + 1];
    }
    v8i bf[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) bf[tn] = frag(cur, BM + wn * WN + tn * 16 + (lane & 15));
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const v8i af = frag(cur, wm * WM + tm * 16 + (lane & 15));
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const v4f p = mfma_e4m3_128(bf[tn], af);
        acc[tm][tn] += p * sc[tm];
      }
    }
    if (kb + 1 < G) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const uint32_t m = m0 + wm * WM + tm * 16 + (lane & 15);
    if (m < M) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const uint32_t n = n0 + wn * WN + tn * 16 + 4 * (lane >> 4);
        *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(acc[tm][tn]);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Skinny kernel for decode widths (M <= 16*TM <= 64).  The projection is then
// bound by streaming the weight matrix once, so each workgroup owns 16 output
// columns for all M rows and its 4 waves split the K blocks; fragments come
// straight from global memory (no reuse to stage) with kUnroll blocks of
// loads in flight per wave, and the 4 partial tiles are summed through LDS.
// ------------------------------------------------------------------------
constexpr int kSkinnyWaves = 4;
constexpr int kSkinnyUnroll = 4;

template <int TM>
__global__ __launch_bounds__(64 * kSkinnyWaves) void gemm_skinny_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ W,
    const float* __restrict__ Ws, uint16_t* __restrict__ out, uint32_t M, uint32_t N, uint32_t K,
    uint32_t Mp) {
  __shared__ v4f red[kSkinnyWaves][TM][64];
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t n0 = blockIdx.x * 16;
  const uint32_t G = K / kGroup, nb = n0 / kGroup;
  const uint32_t kq = 32 * (lane >> 4);  // this lane's byte offset in a K block
  const uint8_t* wrow = W + (uint64_t)(n0 + (lane & 15)) * K + kq;
  const uint8_t* arow[TM];
  uint32_t srow[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const uint32_t m = tm * 16 + (lane & 15);
    arow[tm] = A + (uint64_t)min(m, M - 1) * K + kq;
    srow[tm] = min(m, Mp - 1);
  }

  v4f acc[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) acc[tm] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // contiguous K-block range of this wave
  const uint32_t per = (G + kSkinnyWaves - 1) / kSkinnyWaves;
  const uint32_t kb_lo = min(wave * per, G), kb_hi = min(kb_lo + per, G);
  for (uint32_t kb = kb_lo; kb < kb_hi; kb += kSkinnyUnroll) {
    v8i wf[kSkinnyUnroll], af[kSkinnyUnroll][TM];
    float as[kSkinnyUnroll][TM], ws[kSkinnyUnroll];
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      const uint32_t k = kb + u;
      if (k < kb_hi) {
        const u32x4* wp = reinterpret_cast<const u32x4*>(wrow + (uint64_t)k * kGroup);
        wf[u] = join(__builtin_nontemporal_load(wp), __builtin_nontemporal_load(wp + 1));
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const u32x4* ap = reinterpret_cast<const u32x4*>(arow[tm] + (uint64_t)k * kGroup);
          af[u][tm] = join(ap[0], ap[1]);
          as[u][tm] = As[(uint64_t)k * Mp + srow[tm]];
        }
        ws[u] = Ws[(uint64_t)nb * G + k];
      }
    }
#pragma unroll
    for (int u = 0; u < kSkinnyUnroll; ++u) {
      if (kb + u < kb_hi) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          const v4f p = mfma_e4m3_128(wf[u], af[u][tm]);
          acc[tm] += p * (as[u][tm] * ws[u]);
        }
      }
    }
  }

#pragma unroll
  for (int tm = 0; tm < TM; ++tm) red[wave][tm][lane] = acc[tm];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      v4f s = red[0][tm][lane];
#pragma unroll
      for (int w = 1; w < kSkinnyWaves; ++w) s += red[w][tm][lane];
      const uint32_t m = tm * 16 + (lane & 15);
      if (m < M) {
        const uint32_t n = n0 + 4 * (lane >> 4);
        *reinterpret_cast<uint2*>(out + (uint64_t)m * N + n) = pack_bf16x4(s);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_tiled(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                             const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                             hipStream_t s) {
  constexpr int BM = 128, BN = 128;
  const uint32_t tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  gemm_tiled_kernel<BM, BN, 2, 2><<<dim3(tiles_m * tiles_n), dim3(256), 0, s>>>(
      a, a_s_km, w, w_s, out, M, N, K, m_pad16(M), tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const uint8_t* a, const float* a_s_km, const uint8_t* w,
                              const float* w_s, uint16_t* out, uint32_t M, uint32_t N, uint32_t K,
                              hipStream_t s) {
  const dim3 grid(N / 16), block(64 * kSkinnyWaves);
  const uint32_t Mp = m_pad16(M);
  switch ((M + 15) / 16) {
    case 1: gemm_skinny_kernel<1><<<grid, block, 0, s>>>(a, a_s_km, w, w_s, out, M, N, K, Mp); break;
    case 2: gemm_skinny_kernel<2><<<grid, block, 0, s>>>(a, a_s_km, w, w_s, out, M, N, K, Mp); break;
    case 3: gemm_skinny_kernel<3><<<grid, block, 0, s>>>(a, a_s_km, w, w_s, out, M, N, K, Mp); break;
    case 4: gemm_skinny_kernel<4><<<grid, block, 0, s>>>(a, a_s_km, w, w_s, out, M, N, K, Mp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fp8q
