/*
 * fp8q -- W8A8 block-scaled FP8 projection for AMD MI355X (gfx950).
 *
 * C ABI of libfp8q.so.  The projection it implements is the one routed by
 * the page "dispatch_proj.rs" (spark_model/layers/ops), functions
 * cublas_fp8_proj and cublas_fp8_proj_prequant:
 *
 *   1. quantize bf16 activations [M,K] to OCP FP8 e4m3 with one fp32 scale
 *      per (token, 128-wide K group), scale = amax/448      (fp8q_quant_act)
 *   2. rewrite those scales from row-major [M,K/128] to the K-major
 *      [K/128, ceil16(M)] layout, pad slots zero       (fp8q_scale_to_kmajor)
 *   3. out[M,N] = act . W^T with FP8 weights [N,K] carrying one fp32 scale
 *      per 128x128 block, applied per 128-deep K block  (fp8q_gemm_blockscaled)
 *
 * and fp8q_proj runs all three.  The choice between the two quantizer
 * variants follows the workgroup-count floor of the page
 * "fp8_act_quant_floor.rs" (fp8q_quant_select).
 *
 * Conventions shared by every entry point:
 *
 *  - Memory.  Every array argument is DEVICE memory owned by the caller, on
 *    the current HIP device, 16-byte aligned, densely packed row-major.  The
 *    library allocates nothing and frees nothing; scratch buffers are the
 *    caller's (as the pages' arena buffers are).
 *  - Streams.  Work is enqueued on `stream` (0 = the null stream) and is
 *    ordered with the caller's other work on that stream.  No entry point
 *    synchronizes the host.
 *  - Errors.  Arguments are validated before anything is enqueued; on
 *    failure nothing is launched and a status != FP8Q_OK is returned, with a
 *    message naming the failed check in fp8q_last_error().  A launch failure
 *    returns FP8Q_ERR_LAUNCH (earlier kernels of a composite call may have
 *    been enqueued).
 *  - Empty batch.  M == 0 is a successful no-op.
 *  - Aliasing.  Outputs must not overlap inputs or each other.
 *  - Inputs must be finite; NaN/Inf activations give unspecified codes.
 *  - Concurrency.  Entry points are thread-safe; calls on different streams
 *    may run concurrently as long as their buffers are disjoint.
 *  - Logging.  With FP8Q_LOG=1 in the environment, the quantizer variant
 *    choice prints one line to stderr per selector branch per process.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8q_status {
  FP8Q_OK = 0,
  FP8Q_ERR_NULL = 1,    /* a required pointer is NULL                        */
  FP8Q_ERR_SHAPE = 2,   /* K == 0, K % 128 != 0, N == 0, N % 128 != 0, or a
                           size whose element count does not fit 2^32 - 1     */
  FP8Q_ERR_ALIGN = 3,   /* an array pointer is not 16-byte aligned           */
  FP8Q_ERR_DEVICE = 4,  /* the current HIP device is not gfx950, or the HIP
                           runtime could not be queried                      */
  FP8Q_ERR_LAUNCH = 5,  /* a kernel launch reported an error                  */
  FP8Q_ERR_VARIANT = 6  /* a forced variant / kernel id is out of range       */
} fp8q_status;

/* ------------------------------------------------------------ utilities */

/* ceil16(m) = the padded token count of the K-major scale layout
 * (dispatch_proj.rs, cublas_fp8_m_pad: M rounded up to a multiple of 16).
 * Pure; never fails. */
uint32_t fp8q_m_pad(uint32_t m);

/* Message of the last failed check on the calling thread ("" if none).  The
 * pointer stays valid until the thread's next fp8q call. */
const char *fp8q_last_error(void);

/* Library version string, e.g. "fp8q 0.1.0 gfx950". */
const char *fp8q_version(void);

/* ----------------------------------------------------------- quantizer */

/* Per-(token, 128-group) activation quantizer (dispatch_proj.rs, doc of
 * cublas_fp8_proj; the kernel is called per_token_group_quant_fp8 there).
 *
 *   x_bf16    [M,K] bf16 bit patterns, read only
 *   q_e4m3    [M,K] out: OCP e4m3fn codes; q = e4m3_rne_sat(x / scale), the
 *             sign of zero kept; codes 0x7F/0xFF (NaN) are never written
 *   scale_rm  [M,K/128] out: fp32 scale[m,g] = fl32(amax/448), amax the
 *             largest |x| of the 128 elements x[m, 128g .. 128g+127];
 *             an all-zero group gets scale +0.0 and codes 0x00/0x80
 *   K % 128 == 0.  Results are bit-identical for every variant.
 *
 * The variant (fine-grained A or K-grouped B) is picked by fp8q_quant_select
 * for the current device. */
fp8q_status fp8q_quant_act(const uint16_t *x_bf16, uint8_t *q_e4m3,
                           float *scale_rm, uint32_t M, uint32_t K,
                           hipStream_t stream);

/* As fp8q_quant_act with the variant forced: 0 = auto (selector),
 * 1 = A (fine-grained), 2 = B (K-grouped).  Forcing an arm is how the
 * pages' microtest measures each one (fp8_act_quant_floor.rs, doc of
 * fp8_act_quant_hopper_reject).  Other values -> FP8Q_ERR_VARIANT. */
fp8q_status fp8q_quant_act_ex(const uint16_t *x_bf16, uint8_t *q_e4m3,
                              float *scale_rm, uint32_t M, uint32_t K,
                              int variant, hipStream_t stream);

/* Quantizer + relayout in one kernel: the outputs of fp8q_quant_act plus
 * the K-major copy of the scales that fp8q_scale_to_kmajor would write
 * (scale_km [K/128, ceil16(M)], pad slots +0.0).  scale_rm may be NULL when
 * only the K-major copy is wanted.  Bit-identical to the two-call path. */
fp8q_status fp8q_quant_act_kmajor(const uint16_t *x_bf16, uint8_t *q_e4m3,
                                  float *scale_rm, float *scale_km,
                                  uint32_t M, uint32_t K, hipStream_t stream);

/* As fp8q_quant_act_kmajor with the variant forced (0 = auto, 1 = A,
 * 2 = B), as fp8q_quant_act_ex forces it for the row-major form; the pad
 * slots of scale_km are written by either variant.  Other values ->
 * FP8Q_ERR_VARIANT. */
fp8q_status fp8q_quant_act_kmajor_ex(const uint16_t *x_bf16, uint8_t *q_e4m3,
                                     float *scale_rm, float *scale_km,
                                     uint32_t M, uint32_t K, int variant,
                                     hipStream_t stream);

/* Parameters of the quantizer variant selection rule
 * (fp8_act_quant_floor.rs, module header "The rule" and
 * fp8_act_quant_hopper_reject).  The K-grouped variant B runs only when its
 * own grid has at least min_wg_per_cu * cu_count workgroups. */
typedef struct fp8q_select_params {
  uint32_t cu_count;       /* compute units of the device (>= 1 assumed)     */
  uint32_t min_wg_per_cu;  /* floor multiplier (workgroups per CU)           */
  uint32_t b_groups_per_wg;/* K-groups one workgroup of variant B covers;
                              its grid is M x ceil((K/128)/b_groups_per_wg)  */
  uint32_t a_groups_per_wg;/* groups one workgroup of variant A covers; its
                              grid is ceil(M*(K/128)/a_groups_per_wg)        */
  int requested;           /* lever: 0 = never pick B                        */
  int b_present;           /* 0 = variant B unavailable                      */
  int a_present;           /* 0 = variant A unavailable                      */
} fp8q_select_params;

/* The parameters fp8q_quant_select uses on this library's gfx950 kernels
 * for a device with cu_count compute units.  `requested` comes from the
 * FP8Q_QUANT_VARIANT environment variable: "floor" or "b" -> 1, "a" -> 0,
 * unset/other -> the gfx950 target default, 0 (variant B measured no faster
 * than A at any swept shape on gfx950).  With "b" the automatic entry points
 * run B unconditionally (measurement). */
fp8q_select_params fp8q_default_select_params(uint32_t cu_count);

/* Pure selection rule.  Returns 2 when variant B runs and 1 when A runs,
 * and writes that variant's launch grid to grid_out[3] (variant and grid are
 * decided together, as the page's Fp8QuantPick carries both).  *reject is
 * set to NULL when B runs, else to the named reason A runs instead:
 *   "variant B not requested", "variant B absent", or
 *   "too few workgroups for variant B to fill the device".
 * Reasons are tested in the page's order: B absent -> A absent (B runs) ->
 * not requested -> grid below the floor.  Returns -1 (FP8Q_ERR_SHAPE in
 * fp8q_last_error) when K is 0 or not a multiple of 128, or when neither
 * variant is present.  grid_out and reject may be NULL. */
int fp8q_quant_select_with(uint32_t M, uint32_t K, const fp8q_select_params *p,
                           uint32_t grid_out[3], const char **reject);

/* fp8q_quant_select_with(M, K, fp8q_default_select_params(cu_count), ...) */
int fp8q_quant_select(uint32_t M, uint32_t K, uint32_t cu_count,
                      uint32_t grid_out[3], const char **reject);

/* Smallest M at which variant B's grid reaches the floor for this K
 * (fp8_act_quant_floor.rs, fp8_quant_hopper_min_m).  0 if K invalid. */
uint32_t fp8q_quant_b_min_m(uint32_t K, const fp8q_select_params *p);

/* Log slot of a verdict (fp8_act_quant_floor.rs, fp8_quant_log_slot): -1 =
 * silent (B did not run and B was not requested), 0..2 = the index of the
 * reject reason in the order listed above, 3 = B ran.  Pure. */
int fp8q_quant_log_slot(int variant, const char *reject, int requested);

/* ------------------------------------------------------------- relayout */

/* Scale relayout (dispatch_proj.rs, fp8_act_scale_to_kmajor):
 *   scale_km[g * Mp + m] = m < M ? scale_rm[m * (K/128) + g] : +0.0f
 * for g < K/128, m < Mp = fp8q_m_pad(M).  Every slot is written.
 *   scale_rm  [M, K/128] fp32, read only
 *   scale_km  [K/128, Mp] fp32 out */
fp8q_status fp8q_scale_to_kmajor(const float *scale_rm, float *scale_km,
                                 uint32_t M, uint32_t K, hipStream_t stream);

/* ----------------------------------------------------------------- GEMM */

/* Block-scaled FP8 GEMM (dispatch_proj.rs, cublas_fp8_proj_prequant):
 *
 *   out[m,n] = bf16_rne( sum_kb a_scale_km[kb*Mp + m] * w_scale[(n/128)*(K/128) + kb]
 *                               * sum_{j<128} dec(a[m,128kb+j]) * dec(w[n,128kb+j]) )
 *
 *   a_e4m3      [M,K] e4m3fn codes (activations), read only
 *   a_scale_km  [K/128, Mp] fp32, Mp = fp8q_m_pad(M) (K-major, as written by
 *               fp8q_scale_to_kmajor); pad slots m >= M may be read but never
 *               reach the output
 *   w_e4m3      [N,K] e4m3fn codes (weights), read only
 *   w_scale     [N/128, K/128] fp32, one scale per 128x128 weight block
 *   out_bf16    [M,N] bf16 out; exactly the M*N real rows are written
 *               (activation rows >= M are neither read nor written)
 *   N % 128 == 0, K % 128 == 0.  Accumulation is fp32 with each 128-deep
 *   block's partial product scaled before it is added; the summation order
 *   is not specified, so outputs are reproducible run to run but not
 *   bit-defined. */
fp8q_status fp8q_gemm_blockscaled(const uint8_t *a_e4m3, const float *a_scale_km,
                                  const uint8_t *w_e4m3, const float *w_scale,
                                  uint16_t *out_bf16, uint32_t M, uint32_t N,
                                  uint32_t K, hipStream_t stream);

/* The kernel fp8q_gemm_blockscaled runs for this shape on a device with
 * cu_count compute units (the ids of fp8q_gemm_blockscaled_ex below), or -1
 * if N or K is not a positive multiple of 128 or cu_count is 0.  Pure host
 * function, thread-safe. */
int fp8q_gemm_select_cus(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count);

/* fp8q_gemm_select_cus with the compute-unit count of the current HIP
 * device (256, a full MI355X, when no device can be queried): the choice
 * the launching entry points make on that device. */
int fp8q_gemm_select(uint32_t M, uint32_t N, uint32_t K);

/* The name, with its template arguments as a kernel trace shows it, of the
 * kernel fp8q_gemm_blockscaled_ex launches for this shape with this kernel
 * id (0 = the automatic choice) on the current device; for id 2 the decode
 * kernel (gemm_decode_kernel, where a workgroup's weight slice fits in LDS)
 * or the fragment-layout skinny kernel.  "" for a bad N, K or id.  Host
 * function; the string is valid until the calling thread's next call. */
const char *fp8q_gemm_kernel_name(uint32_t M, uint32_t N, uint32_t K, int kernel);

/* As fp8q_gemm_blockscaled with the kernel forced: 0 = auto (2 for
 * M <= 64 and for M <= 128 when N <= 8192, 1 below 129 rows; from 129 rows
 * on 5 or 1, whichever needs fewer rounds of workgroups on the device's CUs
 * when a last round of at most one 128x128 workgroup per CU counts as half a
 * round; 5 on a tie), 1 =
 * the LDS-tiled MFMA kernel with 128x128 tiles and two workgroups per CU,
 * 2 = the skinny kernel (decode and small-batch widths; rows in
 * tiles of up to 64, up to 64 rows one workgroup per CU, each streaming an
 * equal column range of the weights, beyond that workgroups of 64 columns
 * per row tile), 3 = the LDS-tiled kernel with 256x128 tiles
 * and 8 waves, 4 = 256x128 tiles with 4 waves (kept for measurement), 5 =
 * 256x128 tiles with two groups of 4 waves taking turns between MFMAs and
 * LDS reads.  Kernels 1, 3, 4 and 5 add the blocks' scaled partial products
 * in the same order and give bit-identical outputs; the skinny kernel keeps
 * one partial sum per wave (interleaved K blocks) and adds them in wave
 * order.  Other values -> FP8Q_ERR_VARIANT. */
fp8q_status fp8q_gemm_blockscaled_ex(const uint8_t *a_e4m3, const float *a_scale_km,
                                     const uint8_t *w_e4m3, const float *w_scale,
                                     uint16_t *out_bf16, uint32_t M, uint32_t N,
                                     uint32_t K, int kernel, hipStream_t stream);

/* fp8q_gemm_blockscaled with the K blocks shared out over more workgroups
 * than the output tiles give (the same operation, same argument conventions
 * and errors), with a caller workspace:
 *  - split-K, for row counts whose 128x128 tiles are too few to fill the
 *    device: the K blocks are cut into `splits` contiguous ranges, block
 *    range s covering [s*(K/128)/splits, (s+1)*(K/128)/splits); each tile's
 *    range sums are written in fp32 to the workspace as part[s][M][N], then a
 *    second kernel forms out = bf16_rne(part[0] + part[1] + ... +
 *    part[splits-1]), added in that order.  Up to 64 rows, where W =
 *    min(max(floor(C/splits), 1), N/16) workgroups a split (C compute units)
 *    own at most 128 columns each (4*ceil(N/(4W))), the skinny kernel's split
 *    form computes the range sums, else the 128x128 tiled kernel's;
 *  - stream-K (splits = 0 where fp8q_gemm_streamk_select says 1): the form
 *    of fp8q_gemm_blockscaled_streamk below on one workgroup per CU.
 * Results are reproducible run to run; they differ from the single-pass
 * kernels by the fp32 summation order only.
 *   workspace        device memory, 16-byte aligned, at least
 *                    fp8q_gemm_splitk_workspace_bytes(M, N, K, splits) bytes
 *                    (may be NULL when that is 0); contents on entry are
 *                    ignored, on return undefined; owned by the caller, who
 *                    must not let two calls in flight share it
 *   splits           0 = automatic (fp8q_gemm_splitk_select; when it gives
 *                    1, fp8q_gemm_blockscaled's automatic kernel runs and the
 *                    workspace is not touched), else 2 <= splits <=
 *                    min(K/128, 64); 1 or a larger count -> FP8Q_ERR_VARIANT
 *   workspace_bytes  smaller than needed -> FP8Q_ERR_SHAPE */
fp8q_status fp8q_gemm_blockscaled_splitk(const uint8_t *a_e4m3, const float *a_scale_km,
                                         const uint8_t *w_e4m3, const float *w_scale,
                                         uint16_t *out_bf16, void *workspace,
                                         size_t workspace_bytes, uint32_t M, uint32_t N,
                                         uint32_t K, uint32_t splits, hipStream_t stream);

/* The split count fp8q_gemm_blockscaled_splitk takes for splits = 0 on a
 * device with C = cu_count compute units, with T = ceil(M/128) * (N/128)
 * tiles of 128x128 and c = min(floor(K/1280), 6) (at least 10 K blocks a
 * split), when fp8q_gemm_select_cus does not pick the 256x128 kernel (id 5):
 *  - M > 64: the tiled count, min(floor(C / T), c) if that is at least 2
 *    (one workgroup per CU), else min(floor(2C / T), c) (two per CU);
 *  - 8 <= M <= 64 where the automatic kernel is not the decode kernel
 *    (fp8q_gemm_kernel_name): the largest s <= min(floor(C*L/N), c) whose
 *    skinny split ranges (4*ceil(N/(4W)) columns, W as above) are at most
 *    L = 96 columns (M <= 32) or 64 (M > 32) if s >= 2; where no such s
 *    exists, from M = 24 the tiled count;
 * 1 (no split) otherwise (M < 8 among them) or when the count is below 2.
 * 0 if N or K is not a positive multiple of 128 or cu_count is 0.  Pure
 * host function. */
uint32_t fp8q_gemm_splitk_select_cus(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count);

/* fp8q_gemm_splitk_select_cus for the current HIP device (256 compute
 * units when no device can be queried). */
uint32_t fp8q_gemm_splitk_select(uint32_t M, uint32_t N, uint32_t K);

/* Workspace bytes of fp8q_gemm_blockscaled_splitk: splits * M * N * 4 for
 * splits >= 2; for splits = 0 the automatic choice on the current device
 * (stream-K: 64 * CUs rounded up to 256, plus 128 KiB per CU; split-K as
 * above; 0 for the single-pass kernel); 0 for an invalid shape or count.
 * Host function. */
size_t fp8q_gemm_splitk_workspace_bytes(uint32_t M, uint32_t N, uint32_t K, uint32_t splits);

/* 1 if fp8q_gemm_blockscaled_splitk with splits = 0 (and fp8q_proj_splitk)
 * runs the stream-K form on a device with cu_count compute units: M >= 512
 * and a stream-K plan exists whose longest workgroup is predicted at least
 * 10% shorter than the 256x128 kernel's last round (see
 * fp8q_gemm_blockscaled_streamk; in K-block times, with each partial read
 * costed at 5 and the flag wait at 8, and a partial last round of Tt tiles
 * at max(Tt/cu_count, 0.73) of a full one); 0 otherwise; -1 for a bad N, K
 * or cu_count.  In practice: a last round of few tiles and a long K (M =
 * 1792, N = 5120, K = 17408 on 256 CUs), not where most CUs have a tile in
 * the last round.  Pure host function.  fp8q_gemm_streamk_select: for the
 * current device (256 CUs when none can be queried). */
int fp8q_gemm_streamk_select_cus(uint32_t M, uint32_t N, uint32_t K, uint32_t cu_count);
int fp8q_gemm_streamk_select(uint32_t M, uint32_t N, uint32_t K);

/* The block-scaled GEMM (fp8q_gemm_blockscaled: same operation, operand
 * conventions and errors) in its stream-K form, run wherever a plan exists
 * (the automatic choice above takes it only where it is predicted to pay).
 * With T = ceil(M/256) * (N/128) tiles of 256x128, G = K/128 blocks, C =
 * `workgroups` persistent workgroups (all resident at once, one per CU):
 * workgroup q computes the whole tiles q, q + C, ... of R = floor(T/C)
 * rounds; the Tt = T mod C remaining tiles are cut along K into P pieces at
 * blocks 0 < b_1 < ... < G, workgroup q < Tt computing piece 0 of tail tile
 * q, the other C - Tt workgroups the later pieces (piece p of tail tile t is
 * unit (p-1)*Tt + t, taken by the workgroup Tt + (unit mod (C - Tt)) in round
 * unit / (C - Tt)).  With Tt > C/2, P = 2 and b_1 balances piece 0 against
 * the rounds of second pieces; else P <= min(C/Tt, G, 16) near-equal pieces.
 * Each later piece's fp32 partial goes to the workspace with a flag holding
 * the call's generation number; the piece-0 workgroup waits for the flags,
 * adds the partials in piece order and stores the bf16 tile, then clears
 * the flags (so a captured launch replays correctly).  A wait gives up after
 * a bounded number of polls and stores NaN.  Results are reproducible run
 * to run and differ from fp8q_gemm_blockscaled only in the fp32 summation
 * order of the K blocks.
 *   workspace        device memory, 16-byte aligned, at least
 *                    fp8q_gemm_streamk_workspace_bytes(workgroups) bytes;
 *                    contents on entry ignored, on return undefined; owned
 *                    by the caller, who must not let two calls in flight
 *                    share it
 *   workgroups       0 = the current device's CU count, else a multiple of
 *                    8 no larger than it -> else FP8Q_ERR_VARIANT
 *   no plan (T <= C, T a multiple of C, or K < 256) or a short workspace ->
 *   FP8Q_ERR_SHAPE; M = 0 -> nothing launched. */
fp8q_status fp8q_gemm_blockscaled_streamk(const uint8_t *a_e4m3, const float *a_scale_km,
                                          const uint8_t *w_e4m3, const float *w_scale,
                                          uint16_t *out_bf16, void *workspace,
                                          size_t workspace_bytes, uint32_t M, uint32_t N,
                                          uint32_t K, uint32_t workgroups, hipStream_t stream);

/* Workspace bytes of fp8q_gemm_blockscaled_streamk on `workgroups` (0 = the
 * current device's CU count): 64 per workgroup rounded up to 256, plus 128
 * KiB per workgroup; 0 if workgroups is not a multiple of 8.  Host
 * function. */
size_t fp8q_gemm_streamk_workspace_bytes(uint32_t workgroups);

/* Bytes of static device scratch behind fp8q_gemm_blockscaled_splitk_noalloc
 * (per GPU, held until the process ends): 32 MiB. */
#define FP8Q_NOALLOC_SCRATCH_BYTES (32u << 20)

/* fp8q_gemm_blockscaled_splitk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same operation, kernels, split choice, results
 * (bit-identical to fp8q_gemm_blockscaled_splitk with the same splits) and
 * errors, with the split-K partials kept in a static device array of
 * FP8Q_NOALLOC_SCRATCH_BYTES instead of a caller workspace.  No entry
 * point allocates; this one takes no workspace either.
 *   splits  0 = automatic split count (fp8q_gemm_splitk_select; when it
 *           gives 1 the single-pass automatic kernel runs and the scratch
 *           is not touched; the stream-K form is not used here), else
 *           2 <= splits <= min(K/128, 64)
 * splits * M * N * 4 > FP8Q_NOALLOC_SCRATCH_BYTES -> FP8Q_ERR_SHAPE, before
 * anything is enqueued.  The first call on a device looks the array's
 * device address up (hipGetSymbolAddress) and keeps it.  All calls on one
 * GPU share its array: calls that may overlap on one GPU (different
 * streams, or graphs replayed concurrently) race and give undefined
 * results; calls in order on one stream are safe.  No scratch contents
 * need to start at zero (every partial read is written first). */
fp8q_status fp8q_gemm_blockscaled_splitk_noalloc(const uint8_t *a_e4m3,
                                                 const float *a_scale_km,
                                                 const uint8_t *w_e4m3,
                                                 const float *w_scale, uint16_t *out_bf16,
                                                 uint32_t M, uint32_t N, uint32_t K,
                                                 uint32_t splits, hipStream_t stream);

/* Per-row FP8 weights (the pages' other weight format, dispatch_proj.rs,
 * dequant_fp8_bf16_into: WeightQuantFormat::Fp8PerRow; the scale index
 * formula scale[(n/block_n)*sk + k/block_k] with block_n = 1, block_k = K,
 * sk = 1 gives one multiplier per weight row):
 *
 *   out[m,n] = bf16_rne( w_scale_row[n] * sum_kb a_scale_km[kb*Mp + m]
 *                               * sum_{j<128} dec(a[m,128kb+j]) * dec(w[n,128kb+j]) )
 *
 *   w_scale_row  [N] fp32, one scale per weight row (= output column), applied
 *                to the fp32 accumulator before the bf16 rounding
 *   all other arguments, conventions, kernels and errors as for
 *   fp8q_gemm_blockscaled / fp8q_gemm_blockscaled_ex (same kernel ids and
 *   automatic choice). */
fp8q_status fp8q_gemm_rowscaled(const uint8_t *a_e4m3, const float *a_scale_km,
                                const uint8_t *w_e4m3, const float *w_scale_row,
                                uint16_t *out_bf16, uint32_t M, uint32_t N,
                                uint32_t K, hipStream_t stream);
fp8q_status fp8q_gemm_rowscaled_ex(const uint8_t *a_e4m3, const float *a_scale_km,
                                   const uint8_t *w_e4m3, const float *w_scale_row,
                                   uint16_t *out_bf16, uint32_t M, uint32_t N,
                                   uint32_t K, int kernel, hipStream_t stream);

/* FP8 weights -> bf16 into a caller-owned buffer (dispatch_proj.rs,
 * dequant_fp8_bf16_into):
 *   dst_bf16[n,k] = bf16_rne( fl32( dec(w_e4m3[n,k]) * scale[i] ) ),
 *   i = (n/128)*(K/128) + k/128   (per_row = 0: 128x128 block scales,
 *                                  scale [ceil(N/128), K/128], K % 128 == 0)
 *   i = n                         (per_row = 1: one scale per row, scale [N],
 *                                  K % 16 == 0)
 * Any N.  The e4m3 value itself is exact in bf16, so with power-of-two
 * scales the expansion is lossless.  Codes 0x7F/0xFF (NaN) give unspecified
 * output.  Errors: FP8Q_ERR_SHAPE (K), FP8Q_ERR_VARIANT (per_row not 0/1),
 * FP8Q_ERR_NULL / FP8Q_ERR_ALIGN, FP8Q_ERR_DEVICE, FP8Q_ERR_LAUNCH. */
fp8q_status fp8q_dequant_fp8_bf16(const uint8_t *w_e4m3, const float *scale,
                                  uint16_t *dst_bf16, uint32_t N, uint32_t K,
                                  int per_row, hipStream_t stream);

/* bf16 GEMM, the same-box comparator of the FP8 path (dispatch_proj.rs:
 * the bf16 projection over the dequantized weight, against which the page
 * quotes the FP8 path's speedup):
 *   out_bf16[m,n] = bf16_rne( sum_k x_bf16[m,k] * w_bf16[n,k] )   (fp32 sum)
 *   x_bf16 [M,K], w_bf16 [N,K] (e.g. from fp8q_dequant_fp8_bf16), out [M,N].
 * N % 128 == 0, K % 64 == 0, M*K*2 and N*K*2 below 2^32 bytes.  Same
 * conventions and errors as fp8q_gemm_blockscaled. */
fp8q_status fp8q_gemm_bf16(const uint16_t *x_bf16, const uint16_t *w_bf16,
                           uint16_t *out_bf16, uint32_t M, uint32_t N, uint32_t K,
                           hipStream_t stream);

/* ----------------------------------------------------------- projection */

/* 1 if fp8q_proj quantizes with the fused kernel that writes both scale
 * layouts (M*(K/128) <= 2^19 scale groups), 0 if it runs the quantizer and
 * the relayout separately.  Pure host function. */
int fp8q_proj_quant_fused(uint32_t M, uint32_t K);

/* Whole W8A8 projection (dispatch_proj.rs, cublas_fp8_proj): quantize x,
 * relayout the scales (fused into the quantizer for small batches, see
 * fp8q_proj_quant_fused), run the GEMM with the automatic kernel choice.
 *   x_bf16               [M,K] bf16 activations, read only
 *   w_e4m3, w_scale      as for fp8q_gemm_blockscaled
 *   out_bf16             [M,N] bf16 out
 *   act_q_scratch        >= M*K bytes       (receives the codes)
 *   act_scale_scratch    >= M*(K/128) fp32  (receives the row-major scales)
 *   act_scale_km_scratch >= Mp*(K/128) fp32 (receives the K-major scales)
 * The scratch buffers hold the intermediate results afterwards. */
fp8q_status fp8q_proj(const uint16_t *x_bf16, const uint8_t *w_e4m3,
                      const float *w_scale, uint16_t *out_bf16,
                      uint8_t *act_q_scratch, float *act_scale_scratch,
                      float *act_scale_km_scratch, uint32_t M, uint32_t N,
                      uint32_t K, hipStream_t stream);

/* As fp8q_proj, with the GEMM run as fp8q_gemm_blockscaled_splitk with
 * splits = 0 (stream-K or split-K where that takes them; elsewhere
 * fp8q_gemm_blockscaled's automatic kernel, and the workspace is not
 * touched):
 *   workspace        device memory, 16-byte aligned, at least
 *                    fp8q_gemm_splitk_workspace_bytes(M, N, K, 0) bytes (may
 *                    be NULL when that is 0); contents undefined on return;
 *                    calls in flight must not share it
 *   workspace_bytes  smaller than needed -> FP8Q_ERR_SHAPE (before any launch)
 * The codes and scales written to the scratch buffers are those of
 * fp8q_proj; the output is fp8q_gemm_blockscaled_splitk's on them. */
fp8q_status fp8q_proj_splitk(const uint16_t *x_bf16, const uint8_t *w_e4m3,
                             const float *w_scale, uint16_t *out_bf16,
                             uint8_t *act_q_scratch, float *act_scale_scratch,
                             float *act_scale_km_scratch, void *workspace,
                             size_t workspace_bytes, uint32_t M, uint32_t N, uint32_t K,
                             hipStream_t stream);

/* As fp8q_proj with per-row weight scales w_scale_row [N] (see
 * fp8q_gemm_rowscaled). */
fp8q_status fp8q_proj_rowscaled(const uint16_t *x_bf16, const uint8_t *w_e4m3,
                                const float *w_scale_row, uint16_t *out_bf16,
                                uint8_t *act_q_scratch, float *act_scale_scratch,
                                float *act_scale_km_scratch, uint32_t M, uint32_t N,
                                uint32_t K, hipStream_t stream);

/* ------------------------------------------------------------ dense FFN */

/* The dense FFN on FP8 weights (dispatch_proj.rs, doc of
 * cublas_fp8_proj_prequant: the gate and up projections read the same
 * [M,H] input, so it is quantized once for both; the post-SiLU intermediate
 * is quantized once for down):
 *   out = down( quant( h ) ),  h = bf16( silu(gate) * up ),
 *   gate = bf16(quant(x) . Wg^T), up = bf16(quant(x) . Wu^T),
 *   silu(g) = g / (1 + e^-g), evaluated in binary32.
 * Weights are FP8 e4m3 with 128x128 block scales: w_gate and w_up [I,H]
 * with scales [I/128, H/128], w_down [H,I] with scales [H/128, I/128].
 * H % 128 == 0 and I % 128 == 0. */

/* The intermediate from bf16 gate/up projections:
 *   gate_bf16, up_bf16  [M,I] bf16, read only
 *   h_e4m3              [M,I] out: codes of h quantized per (token,
 *                       128-group) exactly as fp8q_quant_act quantizes
 *   h_scale_km          [I/128, ceil16(M)] fp32 out: K-major scales, pad
 *                       slots written 0 (as fp8q_scale_to_kmajor)
 * Same conventions and errors as fp8q_quant_act. */
fp8q_status fp8q_silu_mul_quant(const uint16_t *gate_bf16, const uint16_t *up_bf16,
                                uint8_t *h_e4m3, float *h_scale_km, uint32_t M,
                                uint32_t I, hipStream_t stream);

/* Fused gate/up projection: one kernel computes both projections of the
 * quantized input and writes the quantized intermediate; gate, up and h
 * never reach memory in bf16.
 *   x_e4m3, x_scale_km   [M,H] codes and [H/128, ceil16(M)] K-major scales
 *                        (as from fp8q_quant_act_kmajor), read only
 *   w_gate, w_gate_scale, w_up, w_up_scale   as above, read only
 *   h_e4m3, h_scale_km   as for fp8q_silu_mul_quant
 * The result is bit-identical to fp8q_gemm_blockscaled for gate and for up
 * followed by fp8q_silu_mul_quant.  Errors as fp8q_gemm_blockscaled. */
fp8q_status fp8q_ffn_gate_up(const uint8_t *x_e4m3, const float *x_scale_km,
                             const uint8_t *w_gate, const float *w_gate_scale,
                             const uint8_t *w_up, const float *w_up_scale,
                             uint8_t *h_e4m3, float *h_scale_km, uint32_t M,
                             uint32_t H, uint32_t I, hipStream_t stream);

/* Variant fp8q_ffn takes with variant 0: 1 (fused gate/up kernel) for
 * M >= 65, 2 (separate gate and up GEMMs, then fp8q_silu_mul_quant) below;
 * -1 if H or I is not a positive multiple of 128.  Pure host function. */
int fp8q_ffn_select(uint32_t M, uint32_t H, uint32_t I);

/* Bytes of device workspace fp8q_ffn needs for (M, H, I, variant) on the
 * current HIP device; 0 for an invalid variant or shape.  Variant 2 also
 * holds the bf16 gate and up outputs (4*M*I bytes more); where
 * fp8q_gemm_splitk_select(M, H, I) splits the down projection, its partials
 * add splits*M*H*4 bytes. */
size_t fp8q_ffn_workspace_bytes(uint32_t M, uint32_t H, uint32_t I, int variant);

/* The whole FFN:
 *   x_bf16           [M,H] bf16, read only
 *   weights          as above, read only
 *   out_bf16         [M,H] bf16 out
 *   workspace        device memory of >= fp8q_ffn_workspace_bytes(M,H,I,
 *                    variant) bytes, 16-byte aligned; holds the x codes and
 *                    scales, the intermediate's codes and scales (and for
 *                    variant 2 gate and up) afterwards
 *   variant          0 auto (fp8q_ffn_select), 1 fused gate/up, 2 separate;
 *                    both give bit-identical results
 * Launches: the quantizer (and the scale relayout beyond 2^19 scale groups,
 * as fp8q_proj), the gate/up stage, the down GEMM (split-K, as
 * fp8q_gemm_blockscaled_splitk with splits = 0, where that splits); all on
 * `stream`.
 * Errors: FP8Q_ERR_SHAPE also for a short workspace; FP8Q_ERR_VARIANT for a
 * variant outside 0..2; otherwise as fp8q_proj. */
fp8q_status fp8q_ffn(const uint16_t *x_bf16, const uint8_t *w_gate,
                     const float *w_gate_scale, const uint8_t *w_up,
                     const float *w_up_scale, const uint8_t *w_down,
                     const float *w_down_scale, uint16_t *out_bf16, void *workspace,
                     size_t workspace_bytes, uint32_t M, uint32_t H, uint32_t I,
                     int variant, hipStream_t stream);

/* ------------------------------------------------- measurement support */

/* Clock stamp, for measuring the sustained shader clock over a region of a
 * stream (not part of the projection): n one-wave workgroups (1 <= n <=
 * 1024, dealt round robin to the XCDs) each write four values to
 * stamps[4*i .. 4*i+3]: the id of the XCD the workgroup ran on, the
 * hardware id of its wave slot (HW_ID; bits 8-15 name the CU), the shader
 * clock counter of that CU (s_memtime) and the constant 100 MHz counter
 * (s_memrealtime).  The shader clock counters of different CUs are not
 * aligned, so two stamps around a region are paired by (XCD, CU): each pair
 * gives that XCD's average shader clock d(memtime) / d(memrealtime) *
 * 100 MHz over the region.
 *   stamps   device memory of 4*n uint64, 16-byte aligned, written */
fp8q_status fp8q_clock_stamp(unsigned long long *stamps, uint32_t n, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
