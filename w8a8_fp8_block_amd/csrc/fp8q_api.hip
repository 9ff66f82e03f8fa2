// C-ABI entry points of libfp8q.so: argument validation, the quantizer
// variant selection rule, once-per-branch logging and kernel dispatch.
// Declarations and the contract of every function: include/fp8q.h.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/fp8q.h"
#include "fp8q_internal.h"

using namespace fp8q;

// Device memory of fp8q_gemm_blockscaled_splitk_noalloc's split-K partials,
// for callers that cannot allocate.  Every GPU the library runs on holds its
// own copy (until the process ends); in host code the name is a host-side
// stand-in, and the device address comes from hipGetSymbolAddress.
static_assert(FP8Q_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[FP8Q_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[256] = "";

fp8q_status fail(fp8q_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

fp8q_status ok() {
  g_err[0] = '\0';
  return FP8Q_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                              \
  do {                                                                              \
    if ((p) == nullptr) return fail(FP8Q_ERR_NULL, "%s: " #p " is NULL", fn);       \
    if (!aligned16(p)) return fail(FP8Q_ERR_ALIGN, "%s: " #p " is not 16-byte aligned", fn); \
  } while (0)

constexpr uint64_t kMaxElems = 0xFFFFFFFFull;

fp8q_status check_k(const char* fn, uint32_t K) {
  if (K == 0 || K % kGroup != 0) return fail(FP8Q_ERR_SHAPE, "%s: K=%u is not a positive multiple of 128", fn, K);
  return FP8Q_OK;
}

fp8q_status check_mk(const char* fn, uint32_t M, uint32_t K) {
  fp8q_status st = check_k(fn, K);
  if (st != FP8Q_OK) return st;
  if ((uint64_t)M * K > kMaxElems) return fail(FP8Q_ERR_SHAPE, "%s: M*K=%llu exceeds 2^32-1", fn, (unsigned long long)M * K);
  return FP8Q_OK;
}

fp8q_status check_n(const char* fn, uint32_t M, uint32_t N, uint32_t K) {
  if (N == 0 || N % kGroup != 0) return fail(FP8Q_ERR_SHAPE, "%s: N=%u is not a positive multiple of 128", fn, N);
  if ((uint64_t)N * K > kMaxElems || (uint64_t)M * N > kMaxElems)
    return fail(FP8Q_ERR_SHAPE, "%s: N*K or M*N exceeds 2^32-1", fn);
  return FP8Q_OK;
}

// ---- device check: the current device must be gfx950; cached per device ----
constexpr int kMaxDev = 64;
std::atomic<int> g_dev_state[kMaxDev];  // 0 unknown, 1 gfx950, 2 other
std::atomic<uint32_t> g_dev_cus[kMaxDev];

// State of device dev (0 <= dev < kMaxDev): 1 gfx950, 2 other, 0 when its
// properties cannot be read; the first query caches the state and the CU
// count.
int probe_device(int dev) {
  int st = g_dev_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_cus[dev].store((uint32_t)prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_state[dev].store(st, std::memory_order_release);
  }
  return st;
}

fp8q_status check_device(const char* fn, uint32_t* cu_count = nullptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(FP8Q_ERR_DEVICE, "%s: no current HIP device", fn);
  if (dev >= kMaxDev) return fail(FP8Q_ERR_DEVICE, "%s: device index %d unsupported", fn, dev);
  const int st = probe_device(dev);
  if (st == 0) return fail(FP8Q_ERR_DEVICE, "%s: hipGetDeviceProperties failed", fn);
  if (st != 1) return fail(FP8Q_ERR_DEVICE, "%s: current device %d is not gfx950", fn, dev);
  if (cu_count) *cu_count = g_dev_cus[dev].load(std::memory_order_relaxed);
  return FP8Q_OK;
}

// CU count the selector queries without a device argument assume when no
// HIP device can be queried: a full MI355X.
constexpr uint32_t kDefaultCus = 256;

// CU count of the current device (what the launching entry points use), or
// kDefaultCus when there is none.
uint32_t current_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return kDefaultCus;
  if (probe_device(dev) == 0) return kDefaultCus;
  const uint32_t c = g_dev_cus[dev].load(std::memory_order_relaxed);
  return c ? c : kDefaultCus;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::atomic<void*> g_scratch[kMaxDev];
std::mutex g_scratch_mu;

fp8q_status scratch_address(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
    return fail(FP8Q_ERR_DEVICE, "%s: no current HIP device", fn);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(FP8Q_ERR_DEVICE, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn,
                    dev, hipGetErrorString(e));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP8Q_OK;
}

fp8q_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(FP8Q_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  return ok();
}

// ---- selector lever and log ----
// FP8Q_QUANT_VARIANT: "a" = variant B not requested, "b" = force B,
// "floor" = B requested (it runs when its grid reaches the floor), anything
// else / unset = the target default (kQuantBRequestedByDefault).  Read once
// per process.
int env_variant() {
  static const int v = [] {
    const char* e = getenv("FP8Q_QUANT_VARIANT");
    if (e && (e[0] == 'a' || e[0] == 'A') && e[1] == '\0') return 1;
    if (e && (e[0] == 'b' || e[0] == 'B') && e[1] == '\0') return 2;
    if (e && strcmp(e, "floor") == 0) return 3;
    return 0;
  }();
  return v;
}

bool log_enabled() {
  static const bool on = [] {
    const char* e = getenv("FP8Q_LOG");
    return e && e[0] == '1';
  }();
  return on;
}

const char* const kRejects[3] = {
    "variant B not requested",
    "variant B absent",
    "too few workgroups for variant B to fill the device",
};

std::once_flag g_log_once[4];

void log_pick(int variant, const char* reject, int requested, uint32_t M, uint32_t K,
              const uint32_t grid[3]) {
  if (!log_enabled()) return;
  const int slot = fp8q_quant_log_slot(variant, reject, requested);
  if (slot < 0) return;
  std::call_once(g_log_once[slot], [&] {
    if (reject)
      fprintf(stderr, "fp8q: act-quant variant B not used at M=%u K=%u: %s (FP8Q_QUANT_VARIANT)\n",
              M, K, reject);
    else
      fprintf(stderr, "fp8q: act-quant variant B (K-grouped) at M=%u K=%u grid=(%u,%u,1) block=%u\n",
              M, K, grid[0], grid[1], 64 * kQuantBWaves);
  });
}

uint32_t ceil_div(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

fp8q_status run_quant(const char* fn, const uint16_t* x, uint8_t* q, float* srm, float* skm,
                      uint32_t M, uint32_t K, int variant, hipStream_t s) {
  uint32_t cus = 0;
  fp8q_status st = check_device(fn, &cus);
  if (st != FP8Q_OK) return st;
  if (variant == 0) {
    const int env = env_variant();
    if (env == 2) {
      variant = 2;
    } else {
      uint32_t grid[3];
      const char* reject = nullptr;
      fp8q_select_params p = fp8q_default_select_params(cus);
      variant = fp8q_quant_select_with(M, K, &p, grid, &reject);
      log_pick(variant, reject, p.requested, M, K, grid);
    }
  }
  // (with skm, the quantizer also writes the K-major pad slots)
  const hipError_t e = (variant == 2) ? launch_quant_b(x, q, srm, skm, M, K, s)
                                      : launch_quant_a(x, q, srm, skm, M, K, s);
  return launched(fn, e);
}

// GEMM kernel choice: the skinny kernel up to kSkinnyAutoMaxM rows (at M = 64
// it streams the weights in half the tiled kernel's time), and up to
// kSkinnyWideMaxM rows when N <= kSkinnyWideMaxN (few 128-column tiles:
// with the last-level cache flushed before each call, at K = 17408,
// N = 5120: 88 / 90 / 92 us at M = 80 / 128 / 192 against 112-134 /
// 117-146 / 134 us for the tiled kernels; at N = 6144, K = 5120: 32-34 us
// against 41-52 us up to M = 128, no gain beyond); 128 x 128 tiles (two
// workgroups per CU) below kRoundRuleMinM rows.  From there on the choice
// between them and the ping-pong 256 x 128 kernel (one workgroup per CU, a
// few percent faster per full round) follows the last, partial round of
// workgroups on the device's CUs: a ping-pong round costs one unit whether
// full or not, a 128 x 128 round one unit when more than one workgroup per
// CU remains and about half a unit when at most one per CU does (a lone
// workgroup has its CU to itself).  The kernel with fewer units wins; ties
// go to the ping-pong kernel.  Back-to-back launches on one box at N = 17408
// and 6144 (K = 5120) and N = 5120 (K = 17408), M = 640 .. 4576: the rule
// picks the faster kernel at all 22 shapes, by 3-12% (M = 1168, N = 5120:
// 108 vs 124 us; N = 6144, M = 4576: 128 x 128 tiles, 159 vs 164 us).  From
// 129 rows to 511 (same method, M = 129 / 192 / 256 / 320 / 384 / 448 /
// 511) it picks the faster one at all 7 at N = 17408 (the ping-pong kernel
// to 256 rows, one round of 136 tiles: 39.2 / 45.2 / 51.7 against 46.5 /
// 52.2 / 60.3 us), and the 128 x 128 kernel, as before, at N = 5120 and
// 6144, where the ping-pong kernel was 4-12% faster at M = 129, 320 and 384
// (a half-full ping-pong round against a light 128 x 128 one); those shapes
// take split-K where a workspace is at hand.
constexpr uint32_t kSkinnyAutoMaxM = 64;
constexpr uint32_t kSkinnyWideMaxM = 128;
constexpr uint32_t kSkinnyWideMaxN = 8192;
// fp8q_proj writes the K-major scales from the quantizer itself (its tiled
// form, one launch fewer) up to this many scale groups.  Back to back over
// rotating inputs, quantizer + relayout -> tiled quantizer: 7.7 -> 5.9 us at
// M = 1168, K = 5120; 15.2 -> 13.0 at M = 1168, K = 17408; 16.4 -> 14.6 /
// 18.6 -> 16.7 at M = 4576, K = 5120 / 6144.  Beyond it the two are within
// 1% (42.1 / 41.7 us at M = 4576, K = 17408; 138.8 / 138.9 at M = 16384,
// K = 17408) and the row-major quantizer alone runs 8% faster than the
// tiled one there (38.6 against 41.7 us), so the separate relayout stays.
constexpr uint64_t kFusedKmajorMaxGroups = 1u << 19;
constexpr uint32_t kTailRuleMinM = 512;  // the stream-K form from here
constexpr uint32_t kRoundRuleMinM = 129;

int gemm_auto_kernel(uint32_t M, uint32_t N, uint32_t cus) {
  if (M <= kSkinnyAutoMaxM || (M <= kSkinnyWideMaxM && N <= kSkinnyWideMaxN)) return 2;
  if (M < kRoundRuleMinM) return 1;
  const uint64_t c = cus ? cus : 1;
  const uint64_t nt = N / kGroup;
  const uint64_t t_pp = (M + 255) / 256 * nt, t_128 = (M + 127) / 128 * nt;
  // costs in half rounds
  const uint64_t c_pp = 2 * ((t_pp + c - 1) / c);
  const uint64_t tail = t_128 % (2 * c);
  const uint64_t c_128 = 2 * (t_128 / (2 * c)) + (tail == 0 ? 0 : tail > c ? 2 : 1);
  return c_pp <= c_128 ? 5 : 1;
}

// Split-K (fp8q_gemm_blockscaled_splitk).  Above kSplitMinM rows, wherever
// the single-pass choice is not the 256 x 128 kernel: the 128x128 tiled
// kernel's split form with splits = floor(CUs / tiles) when that is at least
// 2 (the split grid fits one workgroup per CU and runs the three-stage form),
// else floor(2 CUs / tiles) (one round of two workgroups per CU, two
// stages), at most K/1280 (10 K blocks a split) and 6.  Cold caches
// (bench.py --gemm-sweep, 256 CUs), us single-pass -> split-K: N=5120,
// K=17408: 87 -> 46 at M=65, 135 -> 55 at M=192, 143 -> 73 at M=384, 143 ->
// 87 at M=512, 144 -> 109 at M=768; N=6144, K=5120: 32 -> 23 at M=65, 47 ->
// 32 at M=192, 51 -> 39 at M=384; N=17408, K=5120: 55 -> 47 at M=65.  A
// count past one round (M=512, N=5120: 4 splits, 640 workgroups) was up to
// 30% slower than the one below it; beyond 512 tiles no count helped.
// Up to kSplitMinM rows, where the decode kernel does not take the shape and
// from kSplitSkinnyMinM rows: the skinny kernel's split form
// (launch_skinny_split) with the most splits, at most K/1280 and 6, whose
// column ranges stay within 96 columns a workgroup up to kSplitMidM rows and
// 64 beyond; where no count fits (wide N), from kSplitTiledMinM rows the
// tiled split form with the count of the rule above.  Fixed on back-to-back
// launches over rotating weight copies (bench.py --gemm-sweep-b2b, 256 CUs,
// us single-pass -> split): N = 5120, K = 17408: 24.7 -> 24.5 (4 splits) at
// M = 8, 27.4 -> 25.2 at 16, 35.4 -> 27.3 at 32, 36.7 -> 30.3 (3 splits) at
// 33 (48-row tiles), 51.4 -> 36.2 at 64, while at M <= 4 the single pass was 0.5-1.2 us
// ahead and 6 splits (124 columns) 1-2 us behind 4; N = 17408, K = 5120
// (tiled, 3 splits): 26.5 -> 24.8 at M = 24, 34.6 -> 26.4 at 33, 37.1 ->
// 29.8 at 64, 0.2-1.4 us behind at M <= 16; N = 6144, K = 5120: 2 splits
// 16.4-18.0 against 16.3-19.4 at M = 33-64.  With a 512 MiB write before
// each call (bench.py --gemm-sweep) the form that streams the weights
// fastest loses the most (N = 17408, M = 32: the tiled split 43.4 against
// the skinny kernel's 31.1 us; N = 6144, M = 16: the decode kernel 17.0
// against 4 splits' 16.0), probably because the write leaves the
// last-level cache full of dirty lines whose write-back shares HBM with the
// weight stream.  Layers run back to back in a model, so the back-to-back
// figures decide.
constexpr uint32_t kSplitMinBlocks = 10;
constexpr uint32_t kSplitMax = 6;
constexpr uint32_t kSplitMinM = 64;
constexpr uint32_t kSplitMidM = 32;
constexpr uint32_t kSplitSkinnyMinM = 8;
constexpr uint32_t kSplitTiledMinM = 24;
constexpr uint32_t kSplitMaxUser = 64;  // bound of an explicit split count

uint32_t splitk_auto(uint32_t M, uint32_t N, uint32_t K, uint32_t cus) {
  if (M == 0 || gemm_auto_kernel(M, N, cus) == 5) return 1;
  const uint64_t cap = std::min<uint64_t>(K / kGroup / kSplitMinBlocks, kSplitMax);
  if (M <= kSplitMinM) {
    if (M < kSplitSkinnyMinM || decode_takes(M, N, K, cus)) return 1;
    const uint32_t colmax = M <= kSplitMidM ? 96 : 64;
    uint64_t sk = std::min<uint64_t>((uint64_t)cus * colmax / N, cap);
    while (sk >= 2 && skinny_split_columns(N, (uint32_t)sk, cus) > colmax) --sk;
    if (sk >= 2) return (uint32_t)sk;
    if (M < kSplitTiledMinM) return 1;
  }
  const uint64_t tiles = (uint64_t)((M + 127) / 128) * (N / 128);
  // prefer a count whose grid fits one workgroup per CU (the three-stage
  // form), else one round of two per CU
  const uint64_t s1 = std::min<uint64_t>(cus / tiles, cap);
  if (s1 >= 2) return (uint32_t)s1;
  const uint64_t s2 = std::min<uint64_t>(2ull * cus / tiles, cap);
  return s2 < 2 ? 1 : (uint32_t)s2;
}

uint64_t splitk_workspace(uint32_t M, uint32_t N, uint32_t splits) {
  return splits < 2 ? 0 : (uint64_t)splits * M * N * 4;
}

// The automatic GEMM where a caller workspace is at hand: the stream-K form
// of the 256 x 128 ping-pong kernel where its plan applies (sk_make_plan: a
// last round of data-parallel tiles small enough that the balanced split is
// predicted 10% shorter), from kTailRuleMinM rows, else split-K where
// splitk_auto splits, else the single-pass kernel.  Measured, graph-timed
// back-to-back launches on 256 CUs, single-pass -> stream-K: M = 1792,
// N = 5120, K = 17408 (280 tiles, 24 in the last round) 215 -> 203 us with 10
// pieces a tail tile, before the partial-read cost entered the plan.  Where
// most CUs have a tile in the last round (the prefill shapes: M = 4576,
// N = 5120, K = 17408, 720 tiles; M = 1168, N = 17408, K = 5120, 680) the
// stream-K form was 4-7% slower than the data-parallel kernel: on this
// power-limited chip a partial last round clocks higher, and the split
// tiles' partial reads cost more than the balance gains.
bool streamk_auto(uint32_t M, uint32_t N, uint32_t K, uint32_t cus) {
  return M >= kTailRuleMinM && gemm_streamk_applies(M, N, K, cus, false);
}

uint64_t auto_workspace(uint32_t M, uint32_t N, uint32_t K, uint32_t cus) {
  if (streamk_auto(M, N, K, cus)) return gemm_streamk_workspace_bytes(cus);
  return splitk_workspace(M, N, splitk_auto(M, N, K, cus));
}

fp8q_status run_gemm(const char* fn, const uint8_t* a, const float* as, const uint8_t* w,
                     const float* ws, uint16_t* out, uint32_t M, uint32_t N, uint32_t K, int kernel,
                     bool row_scaled, hipStream_t s) {
  uint32_t cus = 0;
  const fp8q_status st = check_device(fn, &cus);
  if (st != FP8Q_OK) return st;
  if (kernel == 0) kernel = gemm_auto_kernel(M, N, cus);
  if (kernel == 2 && M > kSkinnyMaxM)
    return fail(FP8Q_ERR_VARIANT, "%s: skinny kernel needs M <= %u (M=%u)", fn, kSkinnyMaxM, M);
  const hipError_t e =
      (kernel == 2) ? launch_gemm_skinny(a, as, w, ws, out, M, N, K, cus, row_scaled, s)
                    : launch_gemm_tiled(a, as, w, ws, out, M, N, K, kernel == 1 ? 1 : kernel - 1,
                                        row_scaled, s);
  return launched(fn, e);
}

// The automatic block-scaled GEMM where a workspace is at hand (part, of
// auto_workspace bytes): stream-K or split-K where auto_workspace says so,
// else the automatic single-pass kernel.
fp8q_status run_gemm_ws(const char* fn, const uint8_t* a, const float* as, const uint8_t* w,
                        const float* ws, uint16_t* out, float* part, uint32_t M, uint32_t N,
                        uint32_t K, hipStream_t s) {
  uint32_t cus = 0;
  const fp8q_status st = check_device(fn, &cus);
  if (st != FP8Q_OK) return st;
  if (streamk_auto(M, N, K, cus))
    return launched(fn, launch_gemm_streamk(a, as, w, ws, out, part, M, N, K, cus, false, s));
  const uint32_t splits = splitk_auto(M, N, K, cus);
  if (splits < 2) return run_gemm(fn, a, as, w, ws, out, M, N, K, 0, false, s);
  return launched(fn, launch_splitk_128(a, as, w, ws, out, part, M, N, K, splits, cus, s));
}

// Shared argument checks of the GEMM entry points.
fp8q_status check_gemm_args(const char* fn, const uint8_t* a_e4m3, const float* a_scale_km,
                            const uint8_t* w_e4m3, const float* w_scale, const char* w_scale_name,
                            uint16_t* out_bf16, uint32_t M, uint32_t N, uint32_t K, int kernel) {
  if (kernel < 0 || kernel > 5) return fail(FP8Q_ERR_VARIANT, "%s: kernel %d out of range", fn, kernel);
  fp8q_status st = check_mk(fn, M, K);
  if (st != FP8Q_OK) return st;
  st = check_n(fn, M, N, K);
  if (st != FP8Q_OK) return st;
  if ((uint64_t)m_pad16(M) * K > kMaxElems) return fail(FP8Q_ERR_SHAPE, "%s: Mp*K exceeds 2^32-1", fn);
  REQUIRE_PTR(a_e4m3);
  REQUIRE_PTR(a_scale_km);
  REQUIRE_PTR(w_e4m3);
  if (w_scale == nullptr) return fail(FP8Q_ERR_NULL, "%s: %s is NULL", fn, w_scale_name);
  if (!aligned16(w_scale)) return fail(FP8Q_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, w_scale_name);
  REQUIRE_PTR(out_bf16);
  return FP8Q_OK;
}

// split_k: fp8q_proj_splitk (the GEMM takes the automatic split count and
// split_ws, a caller workspace of split_ws_bytes, holds the partials); the
// other projections run the single-pass automatic kernel.
fp8q_status run_proj(const char* fn, const uint16_t* x_bf16, const uint8_t* w_e4m3,
                     const float* w_scale, uint16_t* out_bf16, uint8_t* act_q_scratch,
                     float* act_scale_scratch, float* act_scale_km_scratch, uint32_t M, uint32_t N,
                     uint32_t K, bool row_scaled, hipStream_t stream, bool split_k = false,
                     void* split_ws = nullptr, size_t split_ws_bytes = 0);

fp8q_status run_proj(const char* fn, const uint16_t* x_bf16, const uint8_t* w_e4m3,
                     const float* w_scale, uint16_t* out_bf16, uint8_t* act_q_scratch,
                     float* act_scale_scratch, float* act_scale_km_scratch, uint32_t M, uint32_t N,
                     uint32_t K, bool row_scaled, hipStream_t stream, bool split_k,
                     void* split_ws, size_t split_ws_bytes) {
  fp8q_status st = check_mk(fn, M, K);
  if (st != FP8Q_OK) return st;
  st = check_n(fn, M, N, K);
  if (st != FP8Q_OK) return st;
  if ((uint64_t)m_pad16(M) * K > kMaxElems) return fail(FP8Q_ERR_SHAPE, "%s: Mp*K exceeds 2^32-1", fn);
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(w_e4m3);
  REQUIRE_PTR(w_scale);
  REQUIRE_PTR(out_bf16);
  REQUIRE_PTR(act_q_scratch);
  REQUIRE_PTR(act_scale_scratch);
  REQUIRE_PTR(act_scale_km_scratch);
  if (M == 0) return ok();
  // the workspace is sized for the current device (as the size query is);
  // the device itself is checked once the arguments are
  const uint32_t cus = current_cus();
  const bool streamk = split_k && streamk_auto(M, N, K, cus);
  const uint32_t splits = split_k && !streamk ? splitk_auto(M, N, K, cus) : 1;
  if (splits >= 2 || streamk) {
    const uint64_t need = streamk ? gemm_streamk_workspace_bytes(cus) : splitk_workspace(M, N, splits);
    void* workspace = split_ws;
    REQUIRE_PTR(workspace);
    if (split_ws_bytes < need)
      return fail(FP8Q_ERR_SHAPE, "%s: workspace of %llu bytes, %llu needed", fn,
                  (unsigned long long)split_ws_bytes, (unsigned long long)need);
  }
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  if ((uint64_t)M * (K / kGroup) <= kFusedKmajorMaxGroups) {
    // one kernel writes both scale layouts (saves a launch)
    st = run_quant(fn, x_bf16, act_q_scratch, act_scale_scratch, act_scale_km_scratch, M, K, 0,
                   stream);
    if (st != FP8Q_OK) return st;
  } else {
    st = run_quant(fn, x_bf16, act_q_scratch, act_scale_scratch, nullptr, M, K, 0, stream);
    if (st != FP8Q_OK) return st;
    st = launched(fn, launch_relayout(act_scale_scratch, act_scale_km_scratch, M, K, stream));
    if (st != FP8Q_OK) return st;
  }
  if (streamk)
    return launched(fn, launch_gemm_streamk(act_q_scratch, act_scale_km_scratch, w_e4m3, w_scale,
                                            out_bf16, split_ws, M, N, K, cus, false, stream));
  if (splits >= 2)
    return launched(fn, launch_splitk_128(act_q_scratch, act_scale_km_scratch, w_e4m3, w_scale,
                                          out_bf16, static_cast<float*>(split_ws), M, N, K, splits,
                                          cus, stream));
  return run_gemm(fn, act_q_scratch, act_scale_km_scratch, w_e4m3, w_scale, out_bf16, M, N, K, 0,
                  row_scaled, stream);
}

// ---- dense FFN ----
// fp8q_ffn's automatic choice: the fused gate/up kernel (one pass over both
// weight matrices, no bf16 gate/up round trip through HBM) from 65 rows on;
// up to 64, the separate path, whose skinny GEMMs (16-, 32-, 48- and
// 64-row tiles) stream the weights with one workgroup per CU.  Measured on the
// whole call at H=5120, I=17408 with the last-level cache flushed before
// each call (the weights of one layer are not resident in serving):
// separate 89.5 vs fused 114.9 us at M=16, 106.6 vs 121.0 at M=32, 119.4
// vs 126.4 at M=33, 126.5 vs 129.0 at M=64; fused 129.3 vs 156.6 at M=80,
// 446 vs 458 at M=1168, 1328 vs 1374 at M=4576.
constexpr uint32_t kFfnFusedMinM = 65;

int ffn_auto_variant(uint32_t M) { return M >= kFfnFusedMinM ? 1 : 2; }

// Workspace carve-up of fp8q_ffn: regions in this order, each starting on a
// 256-byte boundary.
struct FfnWorkspace {
  uint64_t xq, xs_rm, xs_km, hq, hs_km, g, u, part, total;
};

uint64_t align256(uint64_t v) { return (v + 255u) & ~uint64_t(255); }

FfnWorkspace ffn_workspace(uint32_t M, uint32_t H, uint32_t I, int variant, uint32_t cus) {
  const uint64_t Mp = m_pad16(M);
  FfnWorkspace w;
  uint64_t o = 0;
  w.xq = o;    o = align256(o + (uint64_t)M * H);
  w.xs_rm = o; o = align256(o + (uint64_t)M * (H / kGroup) * 4);
  w.xs_km = o; o = align256(o + Mp * (H / kGroup) * 4);
  w.hq = o;    o = align256(o + (uint64_t)M * I);
  w.hs_km = o; o = align256(o + Mp * (I / kGroup) * 4);
  w.g = w.u = 0;
  if (variant == 2) {
    w.g = o; o = align256(o + (uint64_t)M * I * 2);
    w.u = o; o = align256(o + (uint64_t)M * I * 2);
  }
  // stream-K or split-K workspace of the down projection (empty when it runs
  // single-pass; gate and up never split, so that the variants stay
  // bit-identical)
  const uint64_t part = auto_workspace(M, H, I, cus);
  w.part = part ? o : 0;
  o = align256(o + part);
  w.total = o;
  return w;
}

fp8q_status check_ffn_shape(const char* fn, uint32_t M, uint32_t H, uint32_t I) {
  if (H == 0 || H % kGroup != 0) return fail(FP8Q_ERR_SHAPE, "%s: H=%u is not a positive multiple of 128", fn, H);
  if (I == 0 || I % kGroup != 0) return fail(FP8Q_ERR_SHAPE, "%s: I=%u is not a positive multiple of 128", fn, I);
  const uint64_t Mp = m_pad16(M);
  if (Mp * H > kMaxElems || Mp * I > kMaxElems || (uint64_t)I * H > kMaxElems)
    return fail(FP8Q_ERR_SHAPE, "%s: ceil16(M)*H, ceil16(M)*I or I*H exceeds 2^32-1", fn);
  return FP8Q_OK;
}

}  // namespace

extern "C" {

uint32_t fp8q_m_pad(uint32_t m) { return m_pad16(m); }

const char* fp8q_last_error(void) { return g_err; }

const char* fp8q_version(void) { return "fp8q 0.1.0 gfx950"; }

fp8q_select_params fp8q_default_select_params(uint32_t cu_count) {
  fp8q_select_params p;
  p.cu_count = cu_count;
  p.min_wg_per_cu = kQuantMinWgPerCu;
  p.b_groups_per_wg = kQuantBGroupsPerWg;
  p.a_groups_per_wg = kQuantAGroupsPerWg;
  const int env = env_variant();
  p.requested = env == 3 || env == 2 || (env == 0 && kQuantBRequestedByDefault);
  p.b_present = 1;
  p.a_present = 1;
  return p;
}

int fp8q_quant_select_with(uint32_t M, uint32_t K, const fp8q_select_params* p,
                           uint32_t grid_out[3], const char** reject) {
  const char* fn = "fp8q_quant_select";
  if (p == nullptr) {
    fail(FP8Q_ERR_NULL, "%s: params is NULL", fn);
    return -1;
  }
  if (K == 0 || K % kGroup != 0 || p->b_groups_per_wg == 0 || p->a_groups_per_wg == 0 ||
      (!p->a_present && !p->b_present)) {
    fail(FP8Q_ERR_SHAPE, "%s: K=%u invalid or no variant present", fn, K);
    return -1;
  }
  const uint32_t G = K / kGroup;
  const uint32_t gx_b = ceil_div(G, p->b_groups_per_wg);
  const uint64_t wg_b = (uint64_t)gx_b * M;
  const uint64_t floor_wg = (uint64_t)p->min_wg_per_cu * (p->cu_count ? p->cu_count : 1);
  const char* why = nullptr;
  if (!p->b_present)
    why = kRejects[1];
  else if (!p->a_present)
    why = nullptr;
  else if (!p->requested)
    why = kRejects[0];
  else if (wg_b < floor_wg)
    why = kRejects[2];
  const int variant = why ? 1 : 2;
  if (grid_out) {
    if (variant == 2) {
      grid_out[0] = M;
      grid_out[1] = gx_b;
    } else {
      grid_out[0] = ceil_div((uint64_t)M * G, p->a_groups_per_wg);
      grid_out[1] = 1;
    }
    grid_out[2] = 1;
  }
  if (reject) *reject = why;
  return variant;
}

int fp8q_quant_select(uint32_t M, uint32_t K, uint32_t cu_count, uint32_t grid_out[3],
                      const char** reject) {
  const fp8q_select_params p = fp8q_default_select_params(cu_count);
  return fp8q_quant_select_with(M, K, &p, grid_out, reject);
}

uint32_t fp8q_quant_b_min_m(uint32_t K, const fp8q_select_params* p) {
  if (p == nullptr || K == 0 || K % kGroup != 0 || p->b_groups_per_wg == 0) return 0;
  const uint32_t gx_b = ceil_div(K / kGroup, p->b_groups_per_wg);
  const uint64_t floor_wg = (uint64_t)p->min_wg_per_cu * (p->cu_count ? p->cu_count : 1);
  return ceil_div(floor_wg, gx_b);
}

int fp8q_quant_log_slot(int variant, const char* reject, int requested) {
  if (variant == 2 && reject == nullptr) return 3;
  if (!requested) return -1;
  for (int i = 0; i < 3; ++i)
    if (reject && strcmp(reject, kRejects[i]) == 0) return i;
  return -1;
}

fp8q_status fp8q_quant_act_ex(const uint16_t* x_bf16, uint8_t* q_e4m3, float* scale_rm,
                              uint32_t M, uint32_t K, int variant, hipStream_t stream) {
  const char* fn = "fp8q_quant_act";
  if (variant < 0 || variant > 2) return fail(FP8Q_ERR_VARIANT, "%s: variant %d out of range", fn, variant);
  fp8q_status st = check_mk(fn, M, K);
  if (st != FP8Q_OK) return st;
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(q_e4m3);
  REQUIRE_PTR(scale_rm);
  if (M == 0) return ok();
  return run_quant(fn, x_bf16, q_e4m3, scale_rm, nullptr, M, K, variant, stream);
}

fp8q_status fp8q_quant_act(const uint16_t* x_bf16, uint8_t* q_e4m3, float* scale_rm, uint32_t M,
                           uint32_t K, hipStream_t stream) {
  return fp8q_quant_act_ex(x_bf16, q_e4m3, scale_rm, M, K, 0, stream);
}

fp8q_status fp8q_quant_act_kmajor(const uint16_t* x_bf16, uint8_t* q_e4m3, float* scale_rm,
                                  float* scale_km, uint32_t M, uint32_t K, hipStream_t stream) {
  return fp8q_quant_act_kmajor_ex(x_bf16, q_e4m3, scale_rm, scale_km, M, K, 0, stream);
}

fp8q_status fp8q_quant_act_kmajor_ex(const uint16_t* x_bf16, uint8_t* q_e4m3, float* scale_rm,
                                     float* scale_km, uint32_t M, uint32_t K, int variant,
                                     hipStream_t stream) {
  const char* fn = "fp8q_quant_act_kmajor";
  if (variant < 0 || variant > 2) return fail(FP8Q_ERR_VARIANT, "%s: variant %d out of range", fn, variant);
  fp8q_status st = check_mk(fn, M, K);
  if (st != FP8Q_OK) return st;
  if ((uint64_t)m_pad16(M) * K > kMaxElems) return fail(FP8Q_ERR_SHAPE, "%s: Mp*K exceeds 2^32-1", fn);
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(q_e4m3);
  REQUIRE_PTR(scale_km);
  if (scale_rm != nullptr && !aligned16(scale_rm))
    return fail(FP8Q_ERR_ALIGN, "%s: scale_rm is not 16-byte aligned", fn);
  if (M == 0) return ok();
  return run_quant(fn, x_bf16, q_e4m3, scale_rm, scale_km, M, K, variant, stream);
}

fp8q_status fp8q_scale_to_kmajor(const float* scale_rm, float* scale_km, uint32_t M, uint32_t K,
                                 hipStream_t stream) {
  const char* fn = "fp8q_scale_to_kmajor";
  fp8q_status st = check_mk(fn, M, K);
  if (st != FP8Q_OK) return st;
  if ((uint64_t)m_pad16(M) * K > kMaxElems) return fail(FP8Q_ERR_SHAPE, "%s: Mp*K exceeds 2^32-1", fn);
  REQUIRE_PTR(scale_rm);
  REQUIRE_PTR(scale_km);
  if (M == 0) return ok();
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fn, launch_relayout(scale_rm, scale_km, M, K, stream));
}

fp8q_status fp8q_gemm_blockscaled_ex(const uint8_t* a_e4m3, const float* a_scale_km,
                                     const uint8_t* w_e4m3, const float* w_scale,
                                     uint16_t* out_bf16, uint32_t M, uint32_t N, uint32_t K,
                                     int kernel, hipStream_t stream) {
  const char* fn = "fp8q_gemm_blockscaled";
  fp8q_status st =
      check_gemm_args(fn, a_e4m3, a_scale_km, w_e4m3, w_scale, "w_scale", out_bf16, M, N, K, kernel);
  if (st != FP8Q_OK) return st;
  if (M == 0) return ok();
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return run_gemm(fn, a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16, M, N, K, kernel, false, stream);
}

fp8q_status fp8q_gemm_rowscaled(const uint8_t* a_e4m3, const float* a_scale_km,
                                const uint8_t* w_e4m3, const float* w_scale_row, uint16_t* out_bf16,
                                uint32_t M, uint32_t N, uint32_t K, hipStream_t stream) {
  return fp8q_gemm_rowscaled_ex(a_e4m3, a_scale_km, w_e4m3, w_scale_row, out_bf16, M, N, K, 0,
                                stream);
}

fp8q_status fp8q_gemm_rowscaled_ex(const uint8_t* a_e4m3, const float* a_scale_km,
                                   const uint8_t* w_e4m3, const float* w_scale_row,
                                   uint16_t* out_bf16, uint32_t M, uint32_t N, uint32_t K,
                                   int kernel, hipStream_t stream) {
  const char* fn = "fp8q_gemm_rowscaled";
  fp8q_status st =
      check_gemm_args(fn, a_e4m3, a_scale_km, w_e4m3, w_scale_row, "w_scale_row", out_bf16, M, N,
                      K, kernel);
  if (st != FP8Q_OK) return st;
  if (M == 0) return ok();
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return run_gemm(fn, a_e4m3, a_scale_km, w_e4m3, w_scale_row, out_bf16, M, N, K, kernel, true,
                  stream);
}

fp8q_status fp8q_gemm_bf16(const uint16_t* x_bf16, const uint16_t* w_bf16, uint16_t* out_bf16,
                           uint32_t M, uint32_t N, uint32_t K, hipStream_t stream) {
  const char* fn = "fp8q_gemm_bf16";
  if (K == 0 || K % 64 != 0) return fail(FP8Q_ERR_SHAPE, "%s: K=%u is not a positive multiple of 64", fn, K);
  if (N == 0 || N % kGroup != 0) return fail(FP8Q_ERR_SHAPE, "%s: N=%u is not a positive multiple of 128", fn, N);
  if ((uint64_t)M * K * 2 > kMaxElems || (uint64_t)N * K * 2 > kMaxElems || (uint64_t)M * N > kMaxElems)
    return fail(FP8Q_ERR_SHAPE, "%s: M*K*2, N*K*2 or M*N exceeds 2^32-1", fn);
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(w_bf16);
  REQUIRE_PTR(out_bf16);
  if (M == 0) return ok();
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fn, launch_gemm_bf16(x_bf16, w_bf16, out_bf16, M, N, K, stream));
}

fp8q_status fp8q_dequant_fp8_bf16(const uint8_t* w_e4m3, const float* scale, uint16_t* dst_bf16,
                                  uint32_t N, uint32_t K, int per_row, hipStream_t stream) {
  const char* fn = "fp8q_dequant_fp8_bf16";
  if (per_row != 0 && per_row != 1)
    return fail(FP8Q_ERR_VARIANT, "%s: per_row must be 0 or 1 (got %d)", fn, per_row);
  if (K == 0 || K % (per_row ? 16u : kGroup) != 0)
    return fail(FP8Q_ERR_SHAPE, "%s: K=%u is not a positive multiple of %u", fn, K,
                per_row ? 16u : kGroup);
  if ((uint64_t)N * K > kMaxElems) return fail(FP8Q_ERR_SHAPE, "%s: N*K exceeds 2^32-1", fn);
  REQUIRE_PTR(w_e4m3);
  REQUIRE_PTR(scale);
  REQUIRE_PTR(dst_bf16);
  if (N == 0) return ok();
  fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fn, launch_dequant(w_e4m3, scale, dst_bf16, N, K, per_row != 0, stream));
}

uint32_t fp8q_gemm_splitk_select_cus(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count) {
  if (N == 0 || N % kGroup != 0 || K == 0 || K % kGroup != 0 || cu_count == 0) return 0;
  return splitk_auto(M, N, K, cu_count);
}

uint32_t fp8q_gemm_splitk_select(uint32_t M, uint32_t N, uint32_t K) {
  return fp8q_gemm_splitk_select_cus(M, N, K, current_cus());
}

size_t fp8q_gemm_splitk_workspace_bytes(uint32_t M, uint32_t N, uint32_t K, uint32_t splits) {
  if (N % kGroup != 0 || K == 0 || K % kGroup != 0 || splits > K / kGroup) return 0;
  if (splits == 0) return (size_t)auto_workspace(M, N, K, current_cus());
  return (size_t)splitk_workspace(M, N, splits);
}

int fp8q_gemm_streamk_select_cus(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count) {
  if (N == 0 || N % kGroup != 0 || K == 0 || K % kGroup != 0 || cu_count == 0) return -1;
  return streamk_auto(M, N, K, cu_count) ? 1 : 0;
}

int fp8q_gemm_streamk_select(uint32_t M, uint32_t N, uint32_t K) {
  return fp8q_gemm_streamk_select_cus(M, N, K, current_cus());
}

size_t fp8q_gemm_streamk_workspace_bytes(uint32_t workgroups) {
  if (workgroups == 0) workgroups = current_cus();
  if (workgroups % 8 != 0) return 0;
  return gemm_streamk_workspace_bytes(workgroups);
}

fp8q_status fp8q_gemm_blockscaled_streamk(const uint8_t* a_e4m3, const float* a_scale_km,
                                          const uint8_t* w_e4m3, const float* w_scale,
                                          uint16_t* out_bf16, void* workspace,
                                          size_t workspace_bytes, uint32_t M, uint32_t N,
                                          uint32_t K, uint32_t workgroups, hipStream_t stream) {
  const char* fn = "fp8q_gemm_blockscaled_streamk";
  fp8q_status st =
      check_gemm_args(fn, a_e4m3, a_scale_km, w_e4m3, w_scale, "w_scale", out_bf16, M, N, K, 0);
  if (st != FP8Q_OK) return st;
  if (workgroups % 8 != 0)
    return fail(FP8Q_ERR_VARIANT, "%s: workgroups=%u (0 = the CU count, else a multiple of 8)",
                fn, workgroups);
  if (M == 0) return ok();
  const uint32_t wg = workgroups ? workgroups : current_cus();
  if (!gemm_streamk_applies(M, N, K, wg, true))
    return fail(FP8Q_ERR_SHAPE,
                "%s: no stream-K plan for M=%u N=%u K=%u on %u workgroups (needs more 256x128 "
                "tiles than workgroups, not a multiple of them, and K >= 256)",
                fn, M, N, K, wg);
  REQUIRE_PTR(workspace);
  const uint64_t need = gemm_streamk_workspace_bytes(wg);
  if (workspace_bytes < need)
    return fail(FP8Q_ERR_SHAPE, "%s: workspace of %llu bytes, %llu needed", fn,
                (unsigned long long)workspace_bytes, (unsigned long long)need);
  uint32_t cus = 0;
  st = check_device(fn, &cus);
  if (st != FP8Q_OK) return st;
  // every workgroup must be resident at once (they wait on one another)
  if (wg > cus)
    return fail(FP8Q_ERR_VARIANT, "%s: workgroups=%u exceeds the device's %u compute units", fn,
                wg, cus);
  return launched(fn, launch_gemm_streamk(a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16,
                                          workspace, M, N, K, wg, true, stream));
}

fp8q_status fp8q_gemm_blockscaled_splitk(const uint8_t* a_e4m3, const float* a_scale_km,
                                         const uint8_t* w_e4m3, const float* w_scale,
                                         uint16_t* out_bf16, void* workspace,
                                         size_t workspace_bytes, uint32_t M, uint32_t N,
                                         uint32_t K, uint32_t splits, hipStream_t stream) {
  const char* fn = "fp8q_gemm_blockscaled_splitk";
  fp8q_status st =
      check_gemm_args(fn, a_e4m3, a_scale_km, w_e4m3, w_scale, "w_scale", out_bf16, M, N, K, 0);
  if (st != FP8Q_OK) return st;
  if (splits == 1 || splits > std::min(K / kGroup, kSplitMaxUser))
    return fail(FP8Q_ERR_VARIANT, "%s: splits=%u (0 = auto, else 2..min(K/128, %u))", fn, splits,
                kSplitMaxUser);
  if (M == 0) return ok();
  const uint32_t cus = current_cus();  // as fp8q_gemm_splitk_workspace_bytes sizes it
  if (splits == 0 && streamk_auto(M, N, K, cus)) {
    const uint64_t need = gemm_streamk_workspace_bytes(cus);
    REQUIRE_PTR(workspace);
    if (workspace_bytes < need)
      return fail(FP8Q_ERR_SHAPE, "%s: workspace of %llu bytes, %llu needed", fn,
                  (unsigned long long)workspace_bytes, (unsigned long long)need);
    st = check_device(fn);
    if (st != FP8Q_OK) return st;
    return launched(fn, launch_gemm_streamk(a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16,
                                            workspace, M, N, K, cus, false, stream));
  }
  if (splits == 0) splits = splitk_auto(M, N, K, cus);
  if (splits >= 2) {
    const uint64_t need = splitk_workspace(M, N, splits);
    REQUIRE_PTR(workspace);
    if (workspace_bytes < need)
      return fail(FP8Q_ERR_SHAPE, "%s: workspace of %llu bytes, %llu needed", fn,
                  (unsigned long long)workspace_bytes, (unsigned long long)need);
  }
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  if (splits < 2)
    return run_gemm(fn, a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16, M, N, K, 0, false, stream);
  return launched(fn, launch_splitk_128(a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16,
                                        static_cast<float*>(workspace), M, N, K, splits, cus,
                                        stream));
}

fp8q_status fp8q_clock_stamp(unsigned long long* stamps, uint32_t n, hipStream_t stream) {
  const char* fn = "fp8q_clock_stamp";
  REQUIRE_PTR(stamps);
  if (n == 0 || n > 1024) return fail(FP8Q_ERR_SHAPE, "%s: n=%u (1..1024 workgroups)", fn, n);
  const fp8q_status st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fn, launch_clock_stamp(stamps, n, stream));
}

fp8q_status fp8q_gemm_blockscaled_splitk_noalloc(const uint8_t* a_e4m3, const float* a_scale_km,
                                                 const uint8_t* w_e4m3, const float* w_scale,
                                                 uint16_t* out_bf16, uint32_t M, uint32_t N,
                                                 uint32_t K, uint32_t splits, hipStream_t stream) {
  const char* fn = "fp8q_gemm_blockscaled_splitk_noalloc";
  fp8q_status st =
      check_gemm_args(fn, a_e4m3, a_scale_km, w_e4m3, w_scale, "w_scale", out_bf16, M, N, K, 0);
  if (st != FP8Q_OK) return st;
  if (splits == 1 || splits > std::min(K / kGroup, kSplitMaxUser))
    return fail(FP8Q_ERR_VARIANT, "%s: splits=%u (0 = auto, else 2..min(K/128, %u))", fn, splits,
                kSplitMaxUser);
  if (M == 0) return ok();
  const uint32_t cus = current_cus();
  if (splits == 0) splits = splitk_auto(M, N, K, cus);
  if (splits >= 2) {
    const uint64_t need = splitk_workspace(M, N, splits);
    if (need > FP8Q_NOALLOC_SCRATCH_BYTES)
      return fail(FP8Q_ERR_SHAPE,
                  "%s: %u splits of M=%u x N=%u need %llu bytes of partials, more than the %llu "
                  "bytes of static scratch",
                  fn, splits, M, N, (unsigned long long)need,
                  (unsigned long long)FP8Q_NOALLOC_SCRATCH_BYTES);
  }
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  if (splits < 2)
    return run_gemm(fn, a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16, M, N, K, 0, false, stream);
  // every partial slot the reduction reads is written by the split kernel of
  // the same call: nothing in the scratch has to start at zero
  void* part = nullptr;
  st = scratch_address(fn, &part);
  if (st != FP8Q_OK) return st;
  return launched(fn, launch_splitk_128(a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16,
                                        static_cast<float*>(part), M, N, K, splits, cus, stream));
}

int fp8q_gemm_select_cus(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count) {
  if (N == 0 || N % kGroup != 0 || K == 0 || K % kGroup != 0 || cu_count == 0) return -1;
  return gemm_auto_kernel(M, N, cu_count);
}

int fp8q_gemm_select(uint32_t M, uint32_t N, uint32_t K) {
  return fp8q_gemm_select_cus(M, N, K, current_cus());
}

const char* fp8q_gemm_kernel_name(uint32_t M, uint32_t N, uint32_t K, int kernel) {
  static thread_local char buf[96];
  const uint32_t cus = current_cus();
  if (N == 0 || N % kGroup != 0 || K == 0 || K % kGroup != 0 || kernel < 0 || kernel > 5)
    return "";
  if (kernel == 0) kernel = gemm_auto_kernel(M, N, cus);
  switch (kernel) {
    case 1: return "gemm_tiled_kernel<128, 128, 2, 2, 2, false, false>";
    case 3: return "gemm_tiled_kernel<256, 128, 4, 2, 3, false, false>";
    case 4: return "gemm_tiled_kernel<256, 128, 2, 2, 3, false, false>";
    case 5: return "gemm_pp_kernel<3, false, false>";
    default:
      gemm_skinny_kernel_name(M, N, K, cus, false, buf, sizeof buf);
      return buf;
  }
}

fp8q_status fp8q_gemm_blockscaled(const uint8_t* a_e4m3, const float* a_scale_km,
                                  const uint8_t* w_e4m3, const float* w_scale, uint16_t* out_bf16,
                                  uint32_t M, uint32_t N, uint32_t K, hipStream_t stream) {
  return fp8q_gemm_blockscaled_ex(a_e4m3, a_scale_km, w_e4m3, w_scale, out_bf16, M, N, K, 0, stream);
}

int fp8q_proj_quant_fused(uint32_t M, uint32_t K) {
  return (uint64_t)M * (K / kGroup) <= kFusedKmajorMaxGroups ? 1 : 0;
}

fp8q_status fp8q_proj(const uint16_t* x_bf16, const uint8_t* w_e4m3, const float* w_scale,
                      uint16_t* out_bf16, uint8_t* act_q_scratch, float* act_scale_scratch,
                      float* act_scale_km_scratch, uint32_t M, uint32_t N, uint32_t K,
                      hipStream_t stream) {
  return run_proj("fp8q_proj", x_bf16, w_e4m3, w_scale, out_bf16, act_q_scratch,
                  act_scale_scratch, act_scale_km_scratch, M, N, K, false, stream);
}

fp8q_status fp8q_proj_splitk(const uint16_t* x_bf16, const uint8_t* w_e4m3, const float* w_scale,
                             uint16_t* out_bf16, uint8_t* act_q_scratch, float* act_scale_scratch,
                             float* act_scale_km_scratch, void* workspace, size_t workspace_bytes,
                             uint32_t M, uint32_t N, uint32_t K, hipStream_t stream) {
  return run_proj("fp8q_proj_splitk", x_bf16, w_e4m3, w_scale, out_bf16, act_q_scratch,
                  act_scale_scratch, act_scale_km_scratch, M, N, K, false, stream, true, workspace,
                  workspace_bytes);
}

fp8q_status fp8q_proj_rowscaled(const uint16_t* x_bf16, const uint8_t* w_e4m3,
                                const float* w_scale_row, uint16_t* out_bf16,
                                uint8_t* act_q_scratch, float* act_scale_scratch,
                                float* act_scale_km_scratch, uint32_t M, uint32_t N, uint32_t K,
                                hipStream_t stream) {
  return run_proj("fp8q_proj_rowscaled", x_bf16, w_e4m3, w_scale_row, out_bf16, act_q_scratch,
                  act_scale_scratch, act_scale_km_scratch, M, N, K, true, stream);
}

fp8q_status fp8q_silu_mul_quant(const uint16_t* gate_bf16, const uint16_t* up_bf16,
                                uint8_t* h_e4m3, float* h_scale_km, uint32_t M, uint32_t I,
                                hipStream_t stream) {
  const char* fn = "fp8q_silu_mul_quant";
  fp8q_status st = check_mk(fn, M, I);
  if (st != FP8Q_OK) return st;
  if ((uint64_t)m_pad16(M) * I > kMaxElems) return fail(FP8Q_ERR_SHAPE, "%s: Mp*I exceeds 2^32-1", fn);
  REQUIRE_PTR(gate_bf16);
  REQUIRE_PTR(up_bf16);
  REQUIRE_PTR(h_e4m3);
  REQUIRE_PTR(h_scale_km);
  if (M == 0) return ok();
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fn, launch_silu_mul_quant(gate_bf16, up_bf16, h_e4m3, h_scale_km, M, I, stream));
}

fp8q_status fp8q_ffn_gate_up(const uint8_t* x_e4m3, const float* x_scale_km,
                             const uint8_t* w_gate, const float* w_gate_scale,
                             const uint8_t* w_up, const float* w_up_scale, uint8_t* h_e4m3,
                             float* h_scale_km, uint32_t M, uint32_t H, uint32_t I,
                             hipStream_t stream) {
  const char* fn = "fp8q_ffn_gate_up";
  fp8q_status st = check_ffn_shape(fn, M, H, I);
  if (st != FP8Q_OK) return st;
  REQUIRE_PTR(x_e4m3);
  REQUIRE_PTR(x_scale_km);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(w_gate_scale);
  REQUIRE_PTR(w_up);
  REQUIRE_PTR(w_up_scale);
  REQUIRE_PTR(h_e4m3);
  REQUIRE_PTR(h_scale_km);
  if (M == 0) return ok();
  st = check_device(fn);
  if (st != FP8Q_OK) return st;
  return launched(fn, launch_ffn_gate_up(x_e4m3, x_scale_km, w_gate, w_gate_scale, w_up, w_up_scale,
                                         h_e4m3, h_scale_km, M, H, I, stream));
}

int fp8q_ffn_select(uint32_t M, uint32_t H, uint32_t I) {
  if (H == 0 || H % kGroup != 0 || I == 0 || I % kGroup != 0) return -1;
  return ffn_auto_variant(M);
}

size_t fp8q_ffn_workspace_bytes(uint32_t M, uint32_t H, uint32_t I, int variant) {
  if (variant < 0 || variant > 2 || H % kGroup != 0 || I % kGroup != 0) return 0;
  if (variant == 0) variant = ffn_auto_variant(M);
  return (size_t)ffn_workspace(M, H, I, variant, current_cus()).total;
}

fp8q_status fp8q_ffn(const uint16_t* x_bf16, const uint8_t* w_gate, const float* w_gate_scale,
                     const uint8_t* w_up, const float* w_up_scale, const uint8_t* w_down,
                     const float* w_down_scale, uint16_t* out_bf16, void* workspace,
                     size_t workspace_bytes, uint32_t M, uint32_t H, uint32_t I, int variant,
                     hipStream_t stream) {
  const char* fn = "fp8q_ffn";
  if (variant < 0 || variant > 2) return fail(FP8Q_ERR_VARIANT, "%s: variant %d out of range", fn, variant);
  fp8q_status st = check_ffn_shape(fn, M, H, I);
  if (st != FP8Q_OK) return st;
  REQUIRE_PTR(x_bf16);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(w_gate_scale);
  REQUIRE_PTR(w_up);
  REQUIRE_PTR(w_up_scale);
  REQUIRE_PTR(w_down);
  REQUIRE_PTR(w_down_scale);
  REQUIRE_PTR(out_bf16);
  if (M == 0) return ok();
  REQUIRE_PTR(workspace);
  if (variant == 0) variant = ffn_auto_variant(M);
  // sized for the current device, as fp8q_ffn_workspace_bytes sizes it
  const FfnWorkspace w = ffn_workspace(M, H, I, variant, current_cus());
  if (workspace_bytes < w.total)
    return fail(FP8Q_ERR_SHAPE, "%s: workspace of %llu bytes, %llu needed", fn,
                (unsigned long long)workspace_bytes, (unsigned long long)w.total);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* xq = ws + w.xq;
  float* xs_rm = reinterpret_cast<float*>(ws + w.xs_rm);
  float* xs_km = reinterpret_cast<float*>(ws + w.xs_km);
  uint8_t* hq = ws + w.hq;
  float* hs_km = reinterpret_cast<float*>(ws + w.hs_km);
  float* part = reinterpret_cast<float*>(ws + w.part);

  // x is quantized once for both gate and up
  if ((uint64_t)M * (H / kGroup) <= kFusedKmajorMaxGroups) {
    st = run_quant(fn, x_bf16, xq, xs_rm, xs_km, M, H, 0, stream);
  } else {
    st = run_quant(fn, x_bf16, xq, xs_rm, nullptr, M, H, 0, stream);
    if (st == FP8Q_OK) st = launched(fn, launch_relayout(xs_rm, xs_km, M, H, stream));
  }
  if (st != FP8Q_OK) return st;
  if (variant == 1) {
    st = launched(fn, launch_ffn_gate_up(xq, xs_km, w_gate, w_gate_scale, w_up, w_up_scale, hq,
                                         hs_km, M, H, I, stream));
  } else {
    uint16_t* g = reinterpret_cast<uint16_t*>(ws + w.g);
    uint16_t* u = reinterpret_cast<uint16_t*>(ws + w.u);
    st = run_gemm(fn, xq, xs_km, w_gate, w_gate_scale, g, M, I, H, 0, false, stream);
    if (st == FP8Q_OK) st = run_gemm(fn, xq, xs_km, w_up, w_up_scale, u, M, I, H, 0, false, stream);
    if (st == FP8Q_OK) st = launched(fn, launch_silu_mul_quant(g, u, hq, hs_km, M, I, stream));
  }
  if (st != FP8Q_OK) return st;
  return run_gemm_ws(fn, hq, hs_km, w_down, w_down_scale, out_bf16, part, M, H, I, stream);
}

}  // extern "C"
