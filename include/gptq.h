/*
 * gptq.h - C ABI of the MI355X (gfx950) GPTQ-family layer-quantisation library (libgptq_hip.so).
 *
 * The library implements the hot path of one linear layer's post-training quantisation:
 *   1. gptq_accumulate_hessian  H += 2 X^T X over calibration batches              ([T] section 1)
 *                               [A += 2 (X~ - X)^T X for asymmetric calibration]     ([R] item 3, [A])
 *   2. gptq_prepare             dead coordinates, damping, U with H_d^{-1} = U^T U   ([T] sections 4, 6)
 *      gptq_prepare_groups      the same on the per-group Hessians of [G], all groups in each launch
 *   3. gptq_asym_correction     P1 = [(A U^T) masked strictly upper] U               ([R] item 3)
 *   4. gptq_quantize_layer      shared-order column loop with lazy block updates     ([T] sections 3-5)
 *      gptq_quantize_layer_groups  the same for output-channel groups with a Hessian each ([G])
 *
 * Sources, cited by page title and section:
 *   [T] GPTQ tutorial page "GPTQ：量化一个权重之后怎样补偿输出误差" (charlestar.github.io, 2026-10-15); its
 *       sections in order: 1 calibration objective and Hessian, 2 two-weight example, 3 one constrained
 *       compensation, 4 Cholesky factor vs inverse, 5 shared order, layout and lazy blocks, 6 damping, dead
 *       coordinates and grouping parameters, 7-8 worked checks, 9 grid values vs stored codes.
 *   [R] "Rethinking Residual Errors in Compensation-based LLM Quantization" notes (ICLR 2026), "关键设计" 1-3.
 *   [A] "GPTAQ: Efficient Finetuning-Free Quantization for Asymmetric Calibration" notes (ICML 2025).
 *   [G] "G²PTQ: Improving LLM Post-Training Quantization with Generalized Gradient Compensation" digest
 *       (output-channel groups that each own a Hessian; symmetric per-channel weight grids).
 *
 * Conventions shared by every call
 *   - Layout follows [T]: X is M x K (tokens x input features), W is K x N (input features x output
 *     channels).  Matrices are row-major with an explicit leading dimension unless strides are given.
 *   - Every pointer named as "device" must point to device memory (hipMalloc / a torch CUDA tensor) of the
 *     current HIP device.  The caller owns every buffer; the library never allocates or frees device memory
 *     and keeps no state between calls (the optional kernel timer below aside).  Scratch memory is passed in as `workspace` (device, 256-byte aligned,
 *     size from gptq_workspace_bytes); its contents need not be initialised and are clobbered.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on it in order and every call
 *     returns after enqueueing, so a caller can queue the layers of a model back to back on one stream.  The
 *     one exception is gptq_prepare(_groups) asked for its host-side outputs (damp_out, n_dead_out), which
 *     synchronises `stream` to fill them.
 *   - Errors found on the device (a non-finite input, a non-positive pivot) are latched in a status word at
 *     the head of `workspace`: gptq_prepare(_groups) and gptq_quantize_layer(_groups) clear it when their work
 *     starts on the stream and set bits in it as their kernels find problems; the kernels of the same call
 *     skip their remaining work once it is set.  gptq_device_status reads it (after synchronising `stream`).
 *     This follows the refusal convention of the worked 2-D check of [T] section 7: non-finite values and
 *     non-positive pivots are reported as errors, never repaired.
 *   - Arguments are validated on the host before any HIP call; an invalid call returns GPTQ_ERR_ARG and
 *     enqueues nothing.  No input is ever silently repaired, except by the two documented rules of [T]
 *     section 6: dead coordinates and damping.
 *   - Results are deterministic: no floating-point atomics are used, so two identical calls give
 *     bit-identical outputs.
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GPTQ_OK = 0,
    GPTQ_ERR_ARG = 1,        /* invalid argument: shape, leading dimension, bits, blocksize, NULL pointer */
    GPTQ_ERR_NONFINITE = 2,  /* NaN or Inf found in an input (H diagonal, pivot, weights) */
    GPTQ_ERR_NOT_PD = 3,     /* damped Hessian is not positive definite (a pivot <= 0) */
    GPTQ_ERR_WORKSPACE = 4,  /* workspace NULL, misaligned or smaller than gptq_workspace_bytes */
    GPTQ_ERR_HIP = 5         /* a HIP runtime call failed (launch, synchronisation, copy) */
} gptq_status_t;

typedef enum {
    GPTQ_DTYPE_F32 = 0,      /* IEEE binary32 */
    GPTQ_DTYPE_BF16 = 1      /* bfloat16 (top half of binary32) */
} gptq_dtype_t;

typedef enum {
    GPTQ_CALL_ACCUMULATE_HESSIAN = 0,
    GPTQ_CALL_PREPARE = 1,
    GPTQ_CALL_ASYM_CORRECTION = 2,
    GPTQ_CALL_QUANTIZE_LAYER = 3,
    GPTQ_CALL_ACT_ORDER = 4
} gptq_call_t;

/* Flags of gptq_quantize_layer. */
#define GPTQ_FLAG_SCALES_GIVEN 1u  /* `scales` is an input (e.g. the fixed teaching grid of [T] section 2) */
#define GPTQ_FLAG_CAE 4u           /* add the compensation-aware error term of [R] items 2-3 (gptq_quantize_layer) */
#define GPTQ_FLAG_STATIC_GROUPS 8u /* group scales fixed from W before the loop ([T] section 6 "static groups") */
#define GPTQ_FLAG_MSE 16u          /* weight-MSE clipping of scales taken from W before the loop ([G]) */

/*
 * gptq_workspace_bytes - bytes of `workspace` a call needs for the given sizes.
 *   call: which entry point; K, N, M: sizes as in that call (unused ones are ignored; for
 *   GPTQ_CALL_QUANTIZE_LAYER, M is the number of output-channel groups of gptq_quantize_layer_groups, 0 or 1 for
 *   gptq_quantize_layer); flags: for
 *   gptq_accumulate_hessian 1 if X_float will be given | 2 if row_scale will be given; for
 *   gptq_quantize_layer its flags (GPTQ_FLAG_CAE matters) | 2 if P1 will be given; else 0.
 * Returns 0 for an unknown call.  Never fails otherwise.
 */
size_t gptq_workspace_bytes(gptq_call_t call, int64_t K, int64_t N, int64_t M, unsigned flags);

/*
 * gptq_accumulate_hessian - H += 2 Xs^T Xs for one calibration batch ([T] section 1: the K x K statistic
 * shared by all output channels is accumulated batch by batch; the unnormalised 2 X^T X is used).
 *
 *   H          device, K x K fp32 row-major (ld = K), read-modify-written; both triangles are updated and
 *              stay symmetric.  Zero it before the first batch.
 *   K          input features, >= 1.
 *   X          device, M x K, dtype x_dtype, row-major with leading dimension ldx >= K (elements).
 *   M          tokens in this batch, >= 0 (M == 0 enqueues nothing).
 *   row_scale  NULL, or device fp32[M]: output-channel-group weights ([G]); then Xs = bf16(row_scale_t * x_t)
 *              (fp32 product, rounded to nearest-even bf16).  Requires x_dtype == GPTQ_DTYPE_BF16.
 *              Without it Xs = X.
 *   X_float    NULL, or device M x K, same dtype, leading dimension ldxf >= K: the float stream X~ of
 *              asymmetric calibration ([A], [R] item 3).  Then also A += 2 (X~ - X)^T X with the mismatch
 *              formed in fp32 and rounded to bf16 (exact for bf16 streams whose difference is
 *              bf16-representable).  Requires x_dtype == GPTQ_DTYPE_BF16 and row_scale == NULL.
 *   A          device, K x K fp32 row-major, read-modify-written; required iff X_float != NULL.  Not
 *              symmetric.
 *   workspace  device scratch of gptq_workspace_bytes(GPTQ_CALL_ACCUMULATE_HESSIAN, K, 0, M, flags) with flags
 *              (X_float != 0) | 2 (row_scale != 0).  It holds the per-token-range partial sums of the
 *              256 x 256 tiles (up to 64 ranges for small K; 8 once there are >= 1024 tiles, i.e. K > 11264, or
 *              K > 7936 for the cross term: about 16 K^2 bytes, 13 GB at K = 28672).  With a transformed
 *              operand (row_scale or X_float), K a multiple of 256 and M a multiple of 32 it includes M x K
 *              bf16 of staging for that operand.
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP.  Asynchronous.
 */
gptq_status_t gptq_accumulate_hessian(float* H, int64_t K,
                                      const void* X, gptq_dtype_t x_dtype, int64_t M, int64_t ldx,
                                      const float* row_scale,
                                      const void* X_float, int64_t ldxf, float* A,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_gram_plan - how gptq_accumulate_hessian splits its work for K features and M tokens (host-side query; no
 * device work).  out[0] = 256-column blocks nb, out[1] = 256 x 256 tiles (nb (nb + 1) / 2 upper tiles, or nb^2 for
 * the cross term), out[2] = token splits, out[3] = tokens per split (a multiple of 32), out[4] = floats of split
 * partials the launch writes (splits x tiles x 65536), out[5] = bf16 elements of staging for a transformed
 * operand (0 if the operand is not staged).  cross: 0 symmetric, 1 cross term; transformed: 1 if row_scale or
 * X_float is given.  Errors: GPTQ_ERR_ARG (K < 1, M < 0, out NULL).
 */
gptq_status_t gptq_gram_plan(int64_t K, int64_t M, int cross, int transformed, int64_t* out);

/*
 * gptq_prepare - in place H -> U ([T] sections 4 and 6).
 *   1. dead coordinates: every k with H_kk == 0 gets H_kk := 1 and dead[k] = 1 (else 0);
 *   2. damping: damp = percdamp * mean_k(H_kk) (after step 1), H_d = H + damp * I;
 *   3. U: the upper-triangular matrix with H_d^{-1} = U^T U (so that U_qq^2 is the inverse of the Hessian
 *      left when q is the first free coordinate), computed as H_d = R R^T with R upper then U = R^{-1}.
 *
 *   H_to_U     device, K x K fp32 row-major, symmetric on entry (only the upper triangle is read); on
 *              return holds U with the strictly lower triangle set to zero.
 *   K          >= 1.
 *   percdamp   >= 0 and finite (0 disables damping).
 *   dead       device uint8[K], written.
 *   damp_out   NULL or host float*: receives damp.   n_dead_out: NULL or host int64_t*: number of dead.
 *   workspace  device scratch of gptq_workspace_bytes(GPTQ_CALL_PREPARE, K, 0, 0, 0) (N counts the Hessians of
 *              gptq_prepare_groups; 0 or 1 here).
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP on return.  The device-side errors GPTQ_ERR_NONFINITE
 * (non-finite diagonal or pivot) and GPTQ_ERR_NOT_PD (a pivot <= 0; the contents of H_to_U are then unspecified)
 * are latched in the workspace status word.  If damp_out or n_dead_out is given, the call synchronises `stream`,
 * fills them and returns the latched status as well; with both NULL it returns after enqueueing, and the status
 * is read with gptq_device_status(workspace, stream).
 */
gptq_status_t gptq_prepare(float* H_to_U, int64_t K, float percdamp,
                           uint8_t* dead, float* damp_out, int64_t* n_dead_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_prepare_groups - gptq_prepare on `groups` independent Hessians at once (the output-channel groups of
 * [G], each with its own Hessian): every step of the factorisation runs as one launch over all groups,
 * so the latency-bound small products and diagonal blocks of the recursion fill the GPU `groups` times better.
 * Results are those of gptq_prepare on each Hessian.
 *
 *   H_to_U        device, groups K x K fp32 row-major matrices, Hessian g at H_to_U + g * group_stride.
 *   K             >= 1.
 *   groups        1 .. 65535.
 *   group_stride  floats between consecutive Hessians, >= K * K (a multiple of 4 keeps the vector loads).
 *   percdamp      as for gptq_prepare (the same for every group).
 *   dead          device uint8[groups * K], dead[g * K + k] for coordinate k of group g.
 *   damp_out      NULL or host float[groups].   n_dead_out: NULL or host int64_t[groups].
 *   workspace     device scratch of gptq_workspace_bytes(GPTQ_CALL_PREPARE, K, groups, 0, 0).
 * Errors: as gptq_prepare; GPTQ_ERR_NONFINITE or GPTQ_ERR_NOT_PD if any group fails (damp_out and n_dead_out
 * are still written for every group).  Synchronises `stream` only if damp_out or n_dead_out is given; the
 * latched status of all groups together is read with gptq_device_status.
 */
gptq_status_t gptq_prepare_groups(float* H_to_U, int64_t K, int64_t groups, int64_t group_stride, float percdamp,
                                  uint8_t* dead, float* damp_out, int64_t* n_dead_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_asym_correction - GPTAQ correction matrix ([R] item 3; [A] closed form with channel
 * parallelisation):  P1 = [(A U^T) (.) M] U, with M the strictly upper-triangular mask and U from
 * gptq_prepare on the quantised-stream Hessian.  Row q of P1 is the ridge least-squares response of the
 * coordinates after q to coordinate q's input mismatch.
 *
 *   U          device, K x K fp32 upper-triangular (strictly lower part zero), from gptq_prepare.
 *   A          device, K x K fp32, from gptq_accumulate_hessian (same scaling as H).
 *   P1         device, K x K fp32, written (strictly upper; lower triangle and diagonal written as 0).
 *   workspace  device scratch of gptq_workspace_bytes(GPTQ_CALL_ASYM_CORRECTION, K, 0, 0, 0).
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP.  Asynchronous.
 */
gptq_status_t gptq_asym_correction(const float* U, const float* A, float* P1, int64_t K,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_act_order - act-order ([T] section 6): a processing order of the input coordinates by descending Hessian
 * diagonal, a heuristic of the official implementation.  Reading: the dead fix comes first (a zero diagonal counts
 * as 1), the order is stable (equal diagonals keep their natural order).
 *
 *   H      device, K x K fp32 from gptq_accumulate_hessian; permuted in place: H <- H[perm][:, perm].
 *   A      NULL, or the cross Gram of asymmetric calibration, permuted the same way.
 *   perm   device int32[K], written: processing position j handles original coordinate perm[j].
 *   Then gptq_prepare (and gptq_asym_correction) on the permuted matrices, and gptq_quantize_layer with perm and
 *   the returned dead mask (which is in processing order).
 *   workspace  device scratch of gptq_workspace_bytes(GPTQ_CALL_ACT_ORDER, K, 0, 0, 0) (a K x K copy).
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP.  Asynchronous.
 */
gptq_status_t gptq_act_order(float* H, float* A, int64_t K, int32_t* perm, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * gptq_quantize_layer - quantise every output channel of W in the natural (shared) input-coordinate order
 * ([T] sections 3-5; symmetric per-channel grid of [G]).
 *
 *   Grid: zero point z = 2^(bits-1), codes c in [0, 2^bits - 1], value s_n (c - z).  Unless
 *   GPTQ_FLAG_SCALES_GIVEN, s_n = fp32(2 * max_k |W_kn| / (2^bits - 1)), taken from W before dead rows
 *   are zeroed, and 1 for an all-zero channel.
 *   Loop, coordinate j = 0..K-1 for all channels at once (w = working copy, dead rows zeroed):
 *     c = clamp(round_half_even(w_j / s) + z, 0, 2^bits - 1);  q = s (c - z);  E_j = (w_j - q) / U_jj
 *     w_k -= U_jk E_j for the remaining k of the current block;  [P1: w_k += P1_jk * w_j(before rounding)]
 *     after each block of `blocksize` coordinates the same updates are applied to all later coordinates
 *     at once (lazy batch, [T] section 5).
 *   Group-wise scales (groupsize 32, 64 or 128; [T] section 6: the group size changes the representation, the
 *     block size only the computation): one scale per channel and group.  Default, re-estimated during the
 *     loop: groups of `groupsize` consecutive processing positions, the scale taken from the current
 *     (compensated) weights, s = fp32(2 max|w| / (2^bits - 1)) over the group, when the loop reaches the
 *     group's first coordinate.  GPTQ_FLAG_STATIC_GROUPS: groups of consecutive original coordinates whose
 *     scales come from W before the loop.  scales is then ceil(K / groupsize) x N (row g: group g).
 *   GPTQ_FLAG_MSE: scales taken from W before the loop (per channel, or static groups) are clipped: among
 *     fp32(fp32(2 max|w| a) / (2^bits - 1)) for a = 1.00, 0.99, .., 0.80 the one with the least sum of squared
 *     rounding errors over the channel (group) is used.
 *   perm (act-order): from gptq_act_order; U, dead and P1 then belong to the permuted Hessian; W, codes, W_hat
 *     and g_idx stay in the original coordinate order (pre_round is in processing order).
 *   GPTQ_FLAG_CAE ([R] items 2-3): every step also aligns to the original float output, adding
 *     w_k += P2_jk (w0_j - w_j(before rounding)) with w0 the original weights (dead rows zeroed) and
 *     P2 = [((H + A) U^T) masked strictly upper] U (A = 0 without P1).  Because H_d U^T is upper triangular
 *     with diagonal 1/U_jj, and damping and the dead fix are diagonal, P2 = P1 + I - diag(U)^-1 U, so the
 *     step becomes w_k -= (U_jk / U_jj)(w0_j - q) [+ P1_jk w0_j]: no extra input is needed.  Works with or
 *     without P1; losses still report the step errors E_j above.
 *
 *   W          device, K x N weights, dtype w_dtype, element (k, n) at W[k * w_rs + n * w_cs]
 *              (row-major K x N: w_rs = ldw, w_cs = 1; an N x K nn.Linear weight: w_rs = 1, w_cs = K).
 *   U          device, K x K fp32 from gptq_prepare.        dead: device uint8[K] from gptq_prepare or NULL.
 *   P1         NULL, or device K x K fp32 from gptq_asym_correction (asymmetric calibration).
 *   bits       2..6 (7 and 8 are rejected with GPTQ_ERR_ARG: with |w / s| up to 2^(bits-1) the fp32 working weights
 *              drift past a 1e-4 s band around the rounding midpoints over a few thousand coordinates, so the codes
 *              would no longer be those of an exact-arithmetic loop; measured 2.6e-4 s at 8 bits and 3.4e-5 s at
 *              6 bits for K = 4096).
 *   blocksize  128 (the lazy-batch width; other values are rejected with GPTQ_ERR_ARG).
 *   perm       NULL, or device int32[K] from gptq_act_order.
 *   groupsize  0 (one scale per channel), 32, 64 or 128.
 *   g_idx      NULL, or device int32[K]: the group of every original coordinate (0 without groups).
 *   codes      device uint8, code of (k, n) written at codes[k * c_rs + n * c_cs].
 *   scales     device fp32[N] (groups: [ceil(K/groupsize) * N]): written, or read with GPTQ_FLAG_SCALES_GIVEN
 *              (per channel only; then each > 0 and finite).
 *   W_hat      NULL, or device, dtype w_dtype, s (c - z) evaluated in fp32 then converted, written at
 *              W_hat[k * w_rs + n * w_cs] (same strides as W; may alias W).
 *   losses     NULL, or device fp32[N]: per channel sum_j 1/2 E_j^2 ([T] section 3: the added objective).
 *   pre_round  NULL, or device fp32, K x N row-major (ld = N): w_j / s just before rounding (diagnostic).
 *   flags      GPTQ_FLAG_SCALES_GIVEN | GPTQ_FLAG_CAE | GPTQ_FLAG_STATIC_GROUPS | GPTQ_FLAG_MSE (others rejected;
 *              SCALES_GIVEN excludes groups and MSE, STATIC_GROUPS needs groupsize, MSE needs no groups or static
 *              groups).
 *   workspace  device scratch of gptq_workspace_bytes(GPTQ_CALL_QUANTIZE_LAYER, K, N, 0, flags | (P1?2:0))
 *              (with GPTQ_FLAG_CAE it also holds a copy of the original weights, N x K fp32).
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP on return (asynchronous: the call returns after
 * enqueueing).  A NaN/Inf weight or given scale latches GPTQ_ERR_NONFINITE in the workspace status word (the
 * loop is then skipped and the outputs are unspecified); read it with gptq_device_status.
 */
gptq_status_t gptq_quantize_layer(const void* W, gptq_dtype_t w_dtype, int64_t K, int64_t N,
                                  int64_t w_rs, int64_t w_cs,
                                  const float* U, const uint8_t* dead, const float* P1,
                                  int bits, int blocksize, unsigned flags,
                                  uint8_t* codes, int64_t c_rs, int64_t c_cs,
                                  float* scales, void* W_hat, float* losses, float* pre_round,
                                  const int32_t* perm, int64_t groupsize, int32_t* g_idx,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_quantize_layer_noalloc - gptq_quantize_layer for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  It takes no workspace: its scratch is a static
 * device array of the library, 64 MiB (67,108,864 bytes), one per GPU, held from the first call on that GPU until the
 * process ends.  It calls no hipMalloc, hipFree or other allocating routine (the kernel timer records nothing
 * during it).
 *
 *   Arguments, results and errors: as gptq_quantize_layer (same kernels, same outputs), without workspace.
 *   The layer must fit the array: gptq_workspace_bytes(GPTQ_CALL_QUANTIZE_LAYER, K, N, 0, flags | (P1 ? 2 : 0))
 *   <= 67,108,864 (e.g. K = 4096 with up to 2448 channels), else GPTQ_ERR_WORKSPACE and nothing is enqueued; wider
 *   layers can be quantised in channel slices (W, codes, scales and the other outputs offset by the slice).
 *   Every call on a GPU uses that GPU's one array, which keeps the previous call's contents (each call clears what
 *   must start at zero): calls that overlap on one GPU (other streams, other threads) race and must be ordered by
 *   the caller.  Device-side errors are latched in the array's status word: gptq_device_status(NULL, stream) reads
 *   it for the current device.
 */
gptq_status_t gptq_quantize_layer_noalloc(const void* W, gptq_dtype_t w_dtype, int64_t K, int64_t N,
                                          int64_t w_rs, int64_t w_cs,
                                          const float* U, const uint8_t* dead, const float* P1,
                                          int bits, int blocksize, unsigned flags,
                                          uint8_t* codes, int64_t c_rs, int64_t c_cs,
                                          float* scales, void* W_hat, float* losses, float* pre_round,
                                          const int32_t* perm, int64_t groupsize, int32_t* g_idx, void* stream);

/*
 * gptq_quantize_layer_groups - gptq_quantize_layer on a layer whose N output channels form `groups` equal
 * contiguous groups, each quantised against its own Hessian ([G]: output-channel groups with a Hessian each).
 * Channel n belongs to group g = n / (N / groups) and uses U + g * u_stride, P1 + g * u_stride (if given),
 * dead + g * K and perm + g * K (if given), and its act-order rows go to g_idx + g * K.  Every launch covers
 * all groups (the column loop of every channel at once, the trailing products batched over the groups), so a
 * layer with small groups fills the GPU like one large layer.  Codes, scales, W_hat, losses and pre_round are
 * per channel as for gptq_quantize_layer, whose results this equals group by group.
 *
 *   groups     >= 1, dividing N; with groups > 1, N / groups must be a multiple of 16.
 *   U, P1      device, groups K x K fp32 matrices, u_stride floats apart (u_stride >= K * K when groups > 1;
 *              a multiple of 4 keeps the trailing products' vector loads).
 *   dead       NULL or device uint8[groups * K].   perm: NULL or device int32[groups * K], one act-order
 *              permutation per group (from gptq_act_order on that group's Hessian).
 *   g_idx      NULL or device int32[groups * K] (written).
 *   workspace  device scratch of gptq_workspace_bytes(GPTQ_CALL_QUANTIZE_LAYER, K, N, groups, flags | (P1?2:0))
 *              (one call over all N channels, plus per group the split diagonal blocks of its U).
 *   All other arguments as for gptq_quantize_layer.
 * Errors: as gptq_quantize_layer (asynchronous; device-side errors through gptq_device_status).
 */
gptq_status_t gptq_quantize_layer_groups(const void* W, gptq_dtype_t w_dtype, int64_t K, int64_t N,
                                         int64_t w_rs, int64_t w_cs, int64_t groups,
                                         const float* U, int64_t u_stride, const uint8_t* dead, const float* P1,
                                         int bits, int blocksize, unsigned flags,
                                         uint8_t* codes, int64_t c_rs, int64_t c_cs,
                                         float* scales, void* W_hat, float* losses, float* pre_round,
                                         const int32_t* perm, int64_t groupsize, int32_t* g_idx,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptq_hadamard_rotate - randomised Hadamard rotation of rows, the step before quantisation in [G] (setup
 * paragraph): out_r = (in_r * signs) H_K / sqrt(K) for every row r, H_K the Sylvester Hadamard matrix.  Rotating
 * the activation rows (M x K) and the weight rows in the nn.Linear layout (N x K) with the same signs keeps
 * X W^T unchanged.
 *
 *   in, out   device, rows x K, dtype (F32 or BF16), row r at in + r * ld_in (out + r * ld_out); in == out with
 *             ld_in == ld_out rotates in place.  Arithmetic in fp32; BF16 output is rounded to nearest even.
 *   K         a power of two, 16 <= K <= 16384.     signs: NULL (all +1) or device int8[K] of +-1.
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_HIP.  Asynchronous.
 */
gptq_status_t gptq_hadamard_rotate(const void* in, int64_t ld_in, void* out, int64_t ld_out, gptq_dtype_t dtype,
                                   int64_t rows, int64_t K, const int8_t* signs, void* stream);

/*
 * gptq_pack_codes - store codes in 32-bit words ([T] section 9: the integer codes, not the grid values, are what
 * a quantised layer stores, packed into a wider integer container with scale, zero point and layout kept
 * alongside; the pages fix no bit layout, the one below is this library's).
 *
 *   Layout: each channel's K codes form one little-endian bitstream, code k in stream bits
 *   [bits * k, bits * k + bits), stream bit i being bit i % 32 of word i / 32.  Word w of channel n is written
 *   at packed[w * ldp + n], w < gptq_packed_words(K, bits) = ceil(K * bits / 32).
 *   codes   device uint8, code (k, n) at codes[k * c_rs + n * c_cs]; each < 2^bits (higher bits are dropped).
 *   bits    1..8.   packed: device uint32, ldp >= N.
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_HIP.  Asynchronous.
 */
gptq_status_t gptq_pack_codes(const uint8_t* codes, int64_t c_rs, int64_t c_cs, int64_t K, int64_t N, int bits,
                              uint32_t* packed, int64_t ldp, void* stream);

/* Number of 32-bit words per channel that gptq_pack_codes writes: ceil(K * bits / 32). */
int64_t gptq_packed_words(int64_t K, int bits);

/*
 * gptq_unpack_codes - read packed codes back (layout of gptq_pack_codes) and optionally dequantise them.
 *   codes   NULL, or device uint8: code (k, n) written at codes[k * c_rs + n * c_cs].
 *   W_hat   NULL, or device, dtype w_dtype: s_n (c - z), z = 2^(bits-1), evaluated in fp32 then converted
 *           (the values gptq_quantize_layer writes), at W_hat[k * w_rs + n * w_cs]; needs `scales` (fp32[N]).
 * Errors: GPTQ_ERR_ARG, GPTQ_ERR_HIP.  Asynchronous.
 */
gptq_status_t gptq_unpack_codes(const uint32_t* packed, int64_t ldp, int64_t K, int64_t N, int bits,
                                const float* scales, uint8_t* codes, int64_t c_rs, int64_t c_cs,
                                void* W_hat, gptq_dtype_t w_dtype, int64_t w_rs, int64_t w_cs, void* stream);

/*
 * gptq_device_status - the error latched on the device by the latest gptq_prepare, gptq_prepare_groups,
 * gptq_quantize_layer or gptq_quantize_layer_groups call that used `workspace` (the refusal convention of [T]
 * section 7: a non-finite input or a non-positive pivot is an error, reported and not repaired).
 *
 *   workspace  the device workspace given to that call (its 256-byte head holds the status word), or NULL for
 *              the static scratch of gptq_quantize_layer_noalloc on the current device.
 *   stream     the stream that call was enqueued on; it is synchronised before the word is read.
 * Returns GPTQ_OK, GPTQ_ERR_NONFINITE or GPTQ_ERR_NOT_PD (the latter two as latched), GPTQ_ERR_ARG for a
 * misaligned workspace (or NULL before any gptq_quantize_layer_noalloc call on the current device), GPTQ_ERR_HIP if
 * the synchronisation or the read fails.  Does not clear the word:
 * the next latching call on the same workspace does.  Read it before reusing the workspace for such a call
 * if both calls' errors matter.
 */
gptq_status_t gptq_device_status(const void* workspace, void* stream);

/*
 * Kernel timer: a measurement aid, off by default.  While it is on, every kernel launch of the library is
 * bracketed by two HIP events on its stream and attributed to one class; gptq_timer_read synchronises the
 * recorded events and returns the summed GPU time per class.  The timer is process-wide state of the library
 * (events are created on first use and kept); enabling or disabling it drops unread records.  Event records
 * add a few microseconds per launch, so timed runs leave it off.
 */
typedef enum {
    GPTQ_TIMER_GRAM = 0,          /* Gram kernels (including the staging of a transformed operand) */
    GPTQ_TIMER_GRAM_REDUCE = 1,   /* fixed-order sum of the token-split partials into H (or A) */
    GPTQ_TIMER_FACTOR_DIAG = 2,   /* 128 x 128 diagonal blocks of the factorisation */
    GPTQ_TIMER_FACTOR_GEMM = 3,   /* matrix products of the factorisation and of gptq_asym_correction */
    GPTQ_TIMER_LOOP = 4,          /* the column-loop kernel (quantise and compensate inside a block) */
    GPTQ_TIMER_TRAILING = 5,      /* lazy trailing products of the column loop */
    GPTQ_TIMER_OTHER = 6,         /* everything else (conversions, scales, dead/damp, outputs, ...) */
    GPTQ_TIMER_CLASSES = 7
} gptq_timer_class_t;

/* on != 0 turns the timer on, 0 off; either way unread records are dropped.  Errors: GPTQ_ERR_HIP. */
gptq_status_t gptq_timer_enable(int on);

/* ms[c] = summed GPU milliseconds and launches[c] (nullable) = launches of class c recorded since the last
 * enable or read, for c < GPTQ_TIMER_CLASSES; clears the records.  Synchronises the recorded events.
 * Errors: GPTQ_ERR_ARG (ms NULL), GPTQ_ERR_HIP. */
gptq_status_t gptq_timer_read(double* ms, int64_t* launches);

/* Human-readable name of a status code (static string, never NULL). */
const char* gptq_status_string(gptq_status_t status);

/* Library version as "major.minor.patch" (static string). */
const char* gptq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H */
