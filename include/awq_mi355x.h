/*
 * awq_mi355x.h -- C ABI of the AWQ W4A16 group-quantized linear layer on
 * MI355X (gfx950).
 *
 * The method (activation-aware weight quantization, AWQ) as the source pages
 * describe it:
 *   - jsqmd.com "从Java转行大模型应用，大模型量化实现，AWQ 与 GPTQ 算法",
 *     section 二.1 (2) weight importance via the per-channel mean |activation|,
 *     section 二.1 (3) channel scaling: salient input channels of W are
 *     multiplied by s, the activation is divided by s, and s minimises the
 *     output error of the quantized layer; section 五.3 asks for a clip
 *     against scale overflow;
 *   - CSDN "LLM-AWQ学术影响力…", section "量化流程优化": a scale search whose
 *     result is dumped, then real 4-bit, group-128 quantization into packed
 *     weights;
 *   - bjdmk.com.cn "大模型量化技术极速优化…", section "量化参数配置": 4-bit
 *     weights, group size 128, zero point on, GEMV mode for batch 1 and GEMM
 *     mode for long inputs;
 *   - zeeklog.com "LLM-AWQ多模态基准…": W4A16 = 4-bit weights, 16-bit
 *     activations.
 * Where the pages leave a step open, the reading used is stated at the entry
 * point that implements it.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (HIP device memory) owned by the
 *     caller.  fp16 tensors are passed as uint16_t bit patterns.  Matrices are
 *     row-major with K (input features) contiguous: W is [N out][K in], X is
 *     [M tokens][K].
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous and ordered on that stream; nothing is synchronised.
 *   - Argument errors are detected on the host before any launch and nothing
 *     is written; the status code says which check failed and
 *     awq_last_error() returns a message (thread-local).
 *   - Launch failures return AWQ_ERR_HIP.
 *   - Results are bitwise deterministic run to run: every reduction has a
 *     fixed order.
 *   - Outputs must not alias inputs.
 *   - Non-finite data cannot be seen on the host without a synchronisation;
 *     it is reported through device-side values as stated per entry point
 *     (AWQ_ERR_NONFINITE is reserved for that condition and is never
 *     returned: no entry point waits for the device).
 *   - The library allocates no device memory and keeps no device state.
 *     Device scratch comes from the caller as a workspace whose size a query
 *     function returns; the query runs the call's own launch plan without
 *     launching, so the size is exactly what that call uses (0 when its
 *     kernels need none, and then the workspace may be NULL).  Calls that
 *     run at the same time, on any streams, need workspaces that do not
 *     overlap; a workspace may be reused by calls ordered on one stream.
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AWQ_OK = 0,
  AWQ_ERR_NULL = 1,        /* a required pointer is NULL                          */
  AWQ_ERR_SHAPE = 2,       /* a size or group size is out of range                */
  AWQ_ERR_ALIGN = 3,       /* a pointer is not aligned as required                 */
  AWQ_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required           */
  AWQ_ERR_NONFINITE = 5,   /* reserved: non-finite data is reported on the device  */
  AWQ_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed           */
  AWQ_ERR_UNSUPPORTED = 7  /* not supported on this device                         */
} awq_status;

/* Version of this ABI and of the packed layout ("layout v1" below). */
int32_t awq_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* awq_last_error(void);

/* ---------------------------------------------------------------------------
 * awq_calib_stats -- per-input-channel mean absolute activation.
 * Passage: jsqmd.com page, section 二.1 (2): the importance of input channel j
 * comes from E[|X_j|], the mean absolute activation over calibration data
 * (the pseudocode of section 二.2 takes mean(|activation|) over tokens).
 *
 *   x        [m][k] fp16 calibration tokens, 16-byte aligned.
 *   mean_abs [k] float64 out: a_j = (sum_t |x_tj|) / m.  The sum is exact
 *            (|fp16| * 2^24 is an integer; the kernel sums integers), and
 *            a_j is the exact mean rounded once.
 *   Limits: 1 <= m <= 8192, 1 <= k, k % 8 == 0.
 *   Non-finite x: an inf gives a_j = inf, a NaN gives a_j = NaN.
 * ------------------------------------------------------------------------- */
awq_status awq_calib_stats(const uint16_t* x, int64_t m, int64_t k,
                           double* mean_abs, void* stream);

/* ---------------------------------------------------------------------------
 * awq_search_scale -- grid search of the per-channel scale s = a^alpha.
 * Passage: jsqmd.com page, section 二.1 (3): scale salient input channels of W
 * by s, divide the activation by s, and pick s to minimise the output error
 * of the quantized layer.  Readings (the pages give no parametrisation):
 *   alpha_i = i / n_grid, i = 0 .. n_grid-1;
 *   s_ik    = fp16_rn(max(a_k^alpha_i, 2^-14))  (lower clamp = the clip the
 *             page asks for; a NaN power stays NaN);
 *   W'      = fp16_rn(W * s_i) per element;
 *   per (row, group of g along K): D = fp16_rn(max(max W' - min W', 2^-16)/15),
 *             z = clamp(RNE(-min W' / D), 0, 15),
 *             q = clamp(RNE(W' / D) + z, 0, 15)   (RNE = round half to even);
 *   loss    L_i = sum_{t,n} (sum_k ((q - z) D / s_ik - W_nk) X_tk)^2;
 *   best    = first index of the minimum over finite L_i (-1 if none).
 * The kernels evaluate L_i with fp32 MFMA accumulation of an fp16 hi+lo split
 * of the weight error, and reduce squares in float64 (relative error of L_i
 * about 1e-7; the index is exact whenever the best-vs-second gap is larger).
 *
 *   w        [n][k] fp16 weights;  x [m][k] fp16 calibration tokens
 *            (both 16-byte aligned);  mean_abs [k] float64 (awq_calib_stats).
 *   best_idx [1] int32 out;  s16 [k] fp16 out = s at the best alpha;
 *   inv_s16  [k] fp16 out = fp16_rn(1 / s16) (float64 quotient);
 *   losses   [n_grid] float64 out (may be NULL);
 *   When no loss is finite: best_idx = -1 and s16 = inv_s16 = 1.0.
 *   workspace/ws_bytes: device scratch of at least
 *            awq_search_workspace_size(n, k, m, g, n_grid) bytes, 256-byte
 *            aligned; contents on entry are ignored.
 *   Limits: g in {32, 64, 128}; k % g == 0; 1 <= n; 1 <= m <= 8192;
 *           1 <= n_grid <= 64.
 * ------------------------------------------------------------------------- */
size_t awq_search_workspace_size(int64_t n, int64_t k, int64_t m, int32_t g,
                                 int32_t n_grid);
awq_status awq_search_scale(const uint16_t* w, const uint16_t* x,
                            const double* mean_abs, int64_t n, int64_t k,
                            int64_t m, int32_t g, int32_t n_grid,
                            int32_t* best_idx, uint16_t* s16, uint16_t* inv_s16,
                            double* losses, void* workspace, size_t ws_bytes,
                            void* stream);

/* ---------------------------------------------------------------------------
 * awq_pack_int4 -- real quantization and nibble packing (layout v1).
 * Passage: CSDN page, section "量化流程优化" (real 4-bit, group-128
 * quantization of the scaled weights into a packed dump) and bjdmk.com.cn
 * page, section "量化参数配置" (4 bit, group 128, zero point on).  The
 * arithmetic is the per-group rule of awq_search_scale at s = s16.
 *
 *   w        [n][k] fp16, 16-byte aligned.
 *   s16      [k] fp16 channel scale, or NULL for s = 1 (plain RTN).
 *   qweight  [n][k/8] uint32 out: bits 4*(k%8)..+3 of word k/8 hold q_nk.
 *   scales   [n][k/g] fp16 out: D_nj.
 *   qzeros   [n][ceil(k/(8g))] uint32 out: bits 4*(j%8)..+3 of word j/8 hold
 *            z_nj; unused nibbles of the last word are 0.
 *   nonfinite_groups: optional device int32 out (may be NULL): number of
 *            groups whose W' holds inf or NaN (fp16 overflow of W * s or a
 *            non-finite W).  Such a group gets q = 0, z = 0 and scale =
 *            fp16 NaN (0x7E00).
 *   Limits: g in {32, 64, 128}; k % g == 0; n >= 1; k >= g; qweight 16-byte
 *           aligned.
 * ------------------------------------------------------------------------- */
awq_status awq_pack_int4(const uint16_t* w, const uint16_t* s16, int64_t n,
                         int64_t k, int32_t g, uint32_t* qweight,
                         uint16_t* scales, uint32_t* qzeros,
                         int32_t* nonfinite_groups, void* stream);

/* ---------------------------------------------------------------------------
 * awq_fold_inv_scale -- fold a linear's division by s into the per-channel
 * weight of the elementwise operation that produces its input (for example
 * a normalisation weight), so that the linear runs with inv_s16 = NULL.
 * Passage: jsqmd.com page, section 二.1 (3) (the activation is divided by s
 * at inference so the product is unchanged) and bjdmk.com.cn page, section
 * "融合模块优化" (merging computation steps into one operation).  Projections
 * that read one input (q, k, v; gate, up) share one s when awq_search_scale
 * runs on their weights stacked along N (its loss then sums over all their
 * output rows) and awq_pack_int4 packs the stack as one linear.
 *
 *   out_k = fp16_rn(v_k / s16_k): the exact quotient rounded once to fp16.
 *   v, s16   [k] fp16 (device); out [k] fp16 (device, may alias v).
 *   Errors: NULL pointers, k < 1, pointers not 2-byte aligned.  s16_k = 0
 *   gives +-inf (NaN for v_k = 0), as the division does.
 * ------------------------------------------------------------------------- */
awq_status awq_fold_inv_scale(const uint16_t* v, const uint16_t* s16, int64_t k,
                              uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * awq_fold_inv_scale_rows -- the fold of awq_fold_inv_scale when the input of
 * the linear is produced by another linear whose output channel j is its
 * input channel j (in a decoder block the up projection, whose output,
 * multiplied by the activated gate output, is the down projection's input):
 * row j of that linear's fp16 weight is divided by s_j.
 * Passage: as awq_fold_inv_scale.  The producing linear is then searched and
 * packed from the folded weight, and the consuming linear runs with
 * inv_s16 = NULL.  (Under grouped-query attention an output channel of the v
 * projection feeds several channels of the o projection's input, which would
 * need equal s on them; that fold is not offered.)
 *
 *   out[j][c] = fp16_rn(w[j][c] / s16[j]): the exact quotient rounded once.
 *   w, out [n][k] fp16 (device; out may alias w); s16 [n] fp16 (device).
 *   Errors: NULL pointers, n < 1 or k < 1, pointers not 2-byte aligned.
 * ------------------------------------------------------------------------- */
awq_status awq_fold_inv_scale_rows(const uint16_t* w, const uint16_t* s16, int64_t n,
                                   int64_t k, uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Mixed-precision baseline: awq_salient_channels, awq_channel_mask,
 * awq_gather_channels, awq_mixed_loss, awq_linear_mixed.
 * Passage: jsqmd.com page, section 二.1 (1) (a small share, 0.1 - 1 %, of the
 * weights, on the input channels with large activations, decides the accuracy
 * and suffers most from direct quantization) and section 五.1 (protection
 * ratio 0.1 - 1 % by default); CSDN page (mixed-precision optimisation beside
 * the scaling).  The contrasting approach to the search: keep the protected
 * channels' weights in fp16, quantize the rest with plain RTN (awq_pack_int4
 * with s16 = NULL; groups over all channels).
 *
 * awq_salient_channels: idx[count] (device int32, ascending) = the channels of
 *   the `count` largest mean_abs[k] (device float64), ties to the lower index,
 *   NaN above +inf.  count = round(frac * k) for a protection ratio frac.
 *   Limits: 0 <= count <= min(k, 1024).
 * awq_channel_mask: keep16[k] (device fp16) = 1.0, and 0.0 on idx[count].
 * awq_gather_channels: w_s[count][n] (device fp16) = w[:, idx] of w[n][k],
 *   channel-major (w_s[j][r] = w[r][idx[j]]).
 * awq_mixed_loss: *loss (device float64) = sum_{t,n} (sum_k (Wm - W)_nk x_tk)^2
 *   for the mixed weight Wm (RTN with the columns where keep16 = 0 restored
 *   to W): the alpha = 0 loss of awq_search_scale on x with those channels
 *   zeroed.  w [n][k], x [m][k] fp16 (16-byte aligned); workspace of
 *   awq_mixed_loss_workspace_size(n, k, m, g) bytes, 256-byte aligned.
 *   Limits: those of awq_search_scale.
 * awq_linear_mixed: y[m][n] = x Wm^T: awq_linear_w4a16 with inv_s16 = keep16
 *   (the protected channels leave the quantized product), then
 *   y = fp16_rn(y + sum_j x[:, idx_j] w_s[j, :]) (fp32 accumulation in eight
 *   interleaved slices of j, added in slice order; the quantized part is
 *   rounded to fp16 first).  Within 5e-3 *
 *   max(|y_ref|, rms of the row of y_ref) of the float64 value.  qweight,
 *   scales, qzeros: the RTN pack of W (layout v1).  keep16 16-byte aligned.
 *   Workspace: awq_linear_workspace_size(m, n, k, g) bytes (the quantized
 *   part is awq_linear_w4a16).  Limits: those of awq_linear_w4a16;
 *   0 <= count <= min(k, 1024); m <= 1048560.
 * Errors: NULL pointers, shapes and alignment as stated, before any launch.
 * ------------------------------------------------------------------------- */
awq_status awq_salient_channels(const double* mean_abs, int64_t k, int32_t count,
                                int32_t* idx, void* stream);
awq_status awq_channel_mask(const int32_t* idx, int32_t count, int64_t k,
                            uint16_t* keep16, void* stream);
awq_status awq_gather_channels(const uint16_t* w, int64_t n, int64_t k,
                               const int32_t* idx, int32_t count, uint16_t* w_s,
                               void* stream);
size_t awq_mixed_loss_workspace_size(int64_t n, int64_t k, int64_t m, int32_t g);
awq_status awq_mixed_loss(const uint16_t* w, const uint16_t* x, const uint16_t* keep16,
                          int64_t n, int64_t k, int64_t m, int32_t g, double* loss,
                          void* workspace, size_t ws_bytes, void* stream);
awq_status awq_linear_mixed(const uint16_t* x, const uint32_t* qweight,
                            const uint16_t* scales, const uint32_t* qzeros,
                            const uint16_t* keep16, const uint16_t* w_s,
                            const int32_t* idx, int32_t count, int64_t m, int64_t n,
                            int64_t k, int32_t g, uint16_t* y, void* workspace,
                            size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * awq_search_scale_wbit -- awq_search_scale for 3-, 4- or 8-bit codes.
 * Passage: CSDN page, section "量化流程优化" (the weight bit width is a
 * parameter of the search and of the real quantization); jsqmd.com page,
 * section 六 (AWQ for 3- and 4-bit weights); zeeklog.com page (INT3 weights
 * with activation-aware scaling); bjdmk.com.cn page (INT4 and INT8 weights).
 * The per-group rule of awq_search_scale with max_int = 2^w_bit - 1 in place
 * of 15: D = fp16_rn(max(max W' - min W', 2^-16) / max_int),
 * z = clamp(RNE(-min W' / D), 0, max_int), q = clamp(RNE(W' / D) + z, 0,
 * max_int).  Arguments, outputs, workspace and limits as awq_search_scale
 * (w_bit = 4 gives its exact results); w_bit must be 3, 4 or 8.
 * ------------------------------------------------------------------------- */
awq_status awq_search_scale_wbit(const uint16_t* w, const uint16_t* x,
                                 const double* mean_abs, int64_t n, int64_t k,
                                 int64_t m, int32_t g, int32_t n_grid, int32_t w_bit,
                                 int32_t* best_idx, uint16_t* s16, uint16_t* inv_s16,
                                 double* losses, void* workspace, size_t ws_bytes,
                                 void* stream);

/* ---------------------------------------------------------------------------
 * awq_pack_wbit -- real quantization and packing for 3-, 4- or 8-bit codes.
 * Passage: as awq_search_scale_wbit.  The codes and zero points are those of
 * awq_search_scale_wbit's rule at s = s16; w_bit = 4 is awq_pack_int4.
 *
 *   w, s16, scales, nonfinite_groups: as awq_pack_int4.
 *   w_bit 8: qweight [n][k/4] uint32, code k at bits 8*(k%4)..+7 of word
 *            k/4; qzeros [n][ceil(k/(4g))] uint32, z_nj at bits 8*(j%4)..+7
 *            of word j/4.
 *   w_bit 3: qweight [n][3k/32] uint32: codes 32p .. 32p+31 of a row fill
 *            the 96-bit little-endian value of words 3p, 3p+1, 3p+2, code
 *            32p+i at bits 3i..3i+2 (codes 10 and 21 straddle two words);
 *            qzeros [n][ceil(k/(8g))] uint32 with 4-bit fields as layout v1.
 *   Unused fields of the last qzeros word are 0.
 *   Limits: those of awq_pack_int4; w_bit in {3, 4, 8}.
 * ------------------------------------------------------------------------- */
awq_status awq_pack_wbit(const uint16_t* w, const uint16_t* s16, int64_t n,
                         int64_t k, int32_t g, int32_t w_bit, uint32_t* qweight,
                         uint16_t* scales, uint32_t* qzeros,
                         int32_t* nonfinite_groups, void* stream);

/* ---------------------------------------------------------------------------
 * awq_linear_wbit -- y = x_tilde W_deq^T for the layouts of awq_pack_wbit.
 * Passage: as awq_search_scale_wbit, and the W4A16 contract of
 * awq_linear_w4a16 (16-bit activations, dequantization in the kernel).
 *
 *   y[t][n] = fp16_rn( sum_k x_tilde_tk (q_nk - z_nj) D_nj ), as
 *   awq_linear_w4a16, within the same 5e-3 bound.  w_bit = 4 runs
 *   awq_linear_w4a16 (and takes its limits).  w_bit 3 and 8: up to 16
 *   tokens one MFMA kernel that streams the weights per 16-token chunk; from
 *   17 tokens a tiled GEMM (x * inv_s16 staged in the workspace, and fp32
 *   partial tiles there where the linear is split along K).
 *   x [m][k] fp16, qweight and inv_s16 [k] fp16 (or NULL) 16-byte aligned;
 *   scales and qzeros 4-byte aligned; y [m][n] fp16 out.
 *   workspace: awq_linear_wbit_workspace_size(m, n, k, g, w_bit,
 *            inv_s16 != NULL) bytes, 256-byte aligned (NULL if that is 0).
 *   Limits: g in {32, 64, 128}; k % g == 0; k % 64 == 0; 1 <= m, n
 *           <= 2^31 - 1; w_bit in {3, 4, 8}.
 * ------------------------------------------------------------------------- */
size_t awq_linear_wbit_workspace_size(int64_t m, int64_t n, int64_t k, int32_t g,
                                      int32_t w_bit, int32_t has_inv_s16);
awq_status awq_linear_wbit(const uint16_t* x, const uint32_t* qweight,
                           const uint16_t* scales, const uint32_t* qzeros,
                           const uint16_t* inv_s16, int64_t m, int64_t n,
                           int64_t k, int32_t g, int32_t w_bit, uint16_t* y,
                           void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * awq_linear_w4a16 -- y = x_tilde W_deq^T with 4-bit weights and fp16
 * activations.
 * Passage: bjdmk.com.cn page, section "量化参数配置" / "技术选型决策树"
 * (GEMV mode for batch-1 decode, GEMM mode for long inputs); zeeklog.com page
 * (W4A16 kernels); jsqmd.com page, section 二.1 (3) (the activation is
 * divided by s at inference, here x_tilde = x * inv_s16).
 *
 *   y[t][n] = fp16_rn( sum_k x_tilde_tk (q_nk - z_nj) D_nj ),  j = k / g,
 *   x_tilde = x * inv_s16 (per channel) or x when inv_s16 is NULL.
 *   Accumulation is fp32; against the float64 value the result is within
 *   5e-3 * max(|y_ref|, rms of the row of y_ref) per output.
 *   x        [m][k] fp16, 16-byte aligned;  inv_s16 [k] fp16 or NULL,
 *            16-byte aligned;  qweight/scales/qzeros in layout v1
 *            (awq_pack_int4), qweight 16-byte aligned, scales and qzeros
 *            4-byte aligned;  y [m][n] fp16 out.
 *   workspace: device scratch of awq_linear_workspace_size(m, n, k, g)
 *            bytes, 256-byte aligned, owned by the caller (NULL when the
 *            size is 0); contents on entry are ignored.
 *   m = 1 runs the decode GEMV and 2 <= m <= 16 one fused skinny kernel,
 *   both without scratch; 17 <= m <= 32 a group-major kernel with two
 *   token chunks, or for linears above 16 MiB of packed weights with more
 *   than 512 column blocks or k > 8192 the tiled GEMM (GEMV mode); m > 32
 *   the prefill GEMM (x * inv_s16 staged in the
 *   workspace, and fp32 partial tiles there where the linear is split along
 *   K).  Shapes whose activations or scale rows do not fit LDS for these take
 *   a staged two-kernel decode path (activations staged in the workspace).
 *   Every path dequantizes in-kernel.
 *   Limits: g in {32, 64, 128}; k % g == 0; k % 64 == 0 (the kernels step
 *           through K in 64-channel steps); m >= 1; n >= 1; n * k / 2 below
 *           4 GiB.  |x_tilde| must stay within the fp16 range (larger values
 *           give a non-finite y).
 * ------------------------------------------------------------------------- */
size_t awq_linear_workspace_size(int64_t m, int64_t n, int64_t k, int32_t g);
awq_status awq_linear_w4a16(const uint16_t* x, const uint32_t* qweight,
                            const uint16_t* scales, const uint32_t* qzeros,
                            const uint16_t* inv_s16, int64_t m, int64_t n,
                            int64_t k, int32_t g, uint16_t* y, void* workspace,
                            size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * awq_linear_w4a16_group -- independent linears of one decode step in one
 * launch.
 * Passage: as awq_linear_w4a16 (bjdmk.com.cn page, section "量化参数配置":
 * GEMV mode for batch-1 decode).  In a decoder layer the q, k and v
 * projections read the same input and do not depend on one another, and so
 * do gate and up; one launch for such a group saves the fixed launch and
 * ramp time of the others.
 *
 *   items    host array of `count` (1..4) linears with the same m, k and g:
 *            x [m][k] fp16 (16-byte aligned), inv_s16 [k] fp16 or NULL,
 *            qweight [n][k/8] (16-byte aligned), scales [n][k/g],
 *            qzeros [n][ceil(k/(8g))] in layout v1, y [m][n] fp16 out, n.
 *            The linears may share x; no y may overlap an x, a packed
 *            tensor, an inv_s16 or another y of the group.
 *   Every y holds exactly the bits awq_linear_w4a16 writes for that linear
 *   alone (the arithmetic of a column block does not depend on the launch).
 *   m = 1 and 2 <= m <= 16 run the whole group in one launch of the decode
 *   GEMV (with the tokens as MFMA rows for m <= 8) or of the fused skinny
 *   kernel when their shared-memory plans fit the k and every linear of the
 *   group plans alike; 17 <= m <= 32 one tiled-GEMM launch for the linears
 *   above 16 MiB of packed weights with more than 512 column blocks or
 *   k > 8192 and one launch of the two-chunk group-major kernel for the
 *   others; m > 32 one activation-prep launch and one GEMM launch over the
 *   tiles of every linear; otherwise the linears run one after another on
 *   the stream, reusing the workspace in stream order.
 *   workspace: awq_linear_group_workspace_size(n, count, m, k, g) bytes for
 *            the outputs' widths n[0..count-1], 256-byte aligned (NULL if
 *            that is 0).
 *   Limits: those of awq_linear_w4a16 for every linear; 1 <= count <= 4.
 * ------------------------------------------------------------------------- */
typedef struct {
  const uint16_t* x;
  const uint16_t* inv_s16;
  const uint32_t* qweight;
  const uint16_t* scales;
  const uint32_t* qzeros;
  uint16_t* y;
  int64_t n;
} awq_linear_item;

size_t awq_linear_group_workspace_size(const int64_t* n, int32_t count, int64_t m,
                                       int64_t k, int32_t g);
awq_status awq_linear_w4a16_group(const awq_linear_item* items, int32_t count,
                                  int64_t m, int64_t k, int32_t g, void* workspace,
                                  size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * awq_linear_w4a16_group_noalloc -- awq_linear_w4a16_group without a
 * workspace and without any allocation, for callers that cannot allocate
 * device memory: code under graph capture, tight serving loops, harnesses that
 * forbid allocation.
 *
 *   Arguments, results (bit for bit), limits and errors: those of
 *   awq_linear_w4a16_group, with the scratch taken from a device array of the
 *   library, awq_linear_noalloc_scratch_bytes() = 64 MiB per GPU, held by each
 *   GPU the library runs on until the process ends.  A call whose plan needs
 *   more (awq_linear_group_workspace_size) returns AWQ_ERR_WORKSPACE before
 *   any launch: decode calls (m <= 32) need little or none, prefill of the
 *   Llama-3-8B-shaped groups fits; larger prefill calls take the workspace
 *   form.  The first call on a device takes the array's device address
 *   (hipGetSymbolAddress), which allocates nothing.
 *   Every call on one GPU uses the same array and leaves its contents behind
 *   (nothing in it needs to start at zero): calls that overlap on one GPU
 *   (concurrent streams, or host threads) race on it and must be serialised
 *   by the caller.
 * ------------------------------------------------------------------------- */
size_t awq_linear_noalloc_scratch_bytes(void);
awq_status awq_linear_w4a16_group_noalloc(const awq_linear_item* items, int32_t count,
                                          int64_t m, int64_t k, int32_t g, void* stream);

/* ---------------------------------------------------------------------------
 * awq_linear_w4a16_bf16, awq_linear_w4a16_group_bf16 -- the 4-bit linear and
 * its group call with bf16 activations: x and y hold bf16 bit patterns.
 * Passage: jsqmd.com page, section 二.1 (3) and bjdmk.com.cn page, section
 * "量化参数配置", as awq_linear_w4a16 (16-bit activations; the pages pair the
 * 4-bit weights with 16-bit activations without fixing the 16-bit format).
 *
 *   Each x is rounded once to fp16 (exact for |x| in [2^-14, 65504]; smaller
 *   values lose the bits below 2^-24, larger ones become +-inf) and the call
 *   then computes what awq_linear_w4a16 computes for that fp16 x; each output
 *   is rounded once from the fp32 accumulation to bf16 (nearest, ties to even)
 *   instead of fp16.  Within 5e-3 * max(|y_ref|, rms of the row of y_ref) of
 *   the float64 value for x in that range.  inv_s16, qweight, scales, qzeros:
 *   as awq_linear_w4a16 (fp16 scales and inv_s16).  Arguments, limits,
 *   workspace sizes and errors: those of awq_linear_w4a16 and
 *   awq_linear_w4a16_group.
 * ------------------------------------------------------------------------- */
awq_status awq_linear_w4a16_bf16(const uint16_t* x, const uint32_t* qweight,
                                 const uint16_t* scales, const uint32_t* qzeros,
                                 const uint16_t* inv_s16, int64_t m, int64_t n,
                                 int64_t k, int32_t g, uint16_t* y, void* workspace,
                                 size_t ws_bytes, void* stream);
awq_status awq_linear_w4a16_group_bf16(const awq_linear_item* items, int32_t count,
                                       int64_t m, int64_t k, int32_t g, void* workspace,
                                       size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_H */
