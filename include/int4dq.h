/*
 * int4dq.h -- C ABI of the MI355X (gfx950) INT4 group-quantization library:
 * block-wise symmetric INT4 weight quantization with two's-complement nibble
 * packing, unpacking, and the fused dequantizing matmul; also dequantization,
 * the bias/ReLU epilogue, affine (zero-point) codes and a linear-layer call
 * with binary16 output.
 *
 * The three operations are the ones stated on the drill page "Implement INT4
 * group quantization, nibble packing and a dequantizing matmul"
 * (inferenceinterviews.com), section "statement": quantize_int4,
 * unpack_int4 and int4_matmul, with the same argument order (x, packed,
 * scales, K, group) and the same layouts.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers (hipMalloc'd or equivalent) to
 *    dense row-major arrays. The caller owns every buffer; the library never
 *    allocates, frees, or synchronises, and never keeps a pointer after the
 *    call returns.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *    default stream) and the call returns without waiting for it. A kernel
 *    fault therefore surfaces at the caller's next synchronisation.
 *  - Arguments are validated before anything is enqueued. On a non-OK return
 *    nothing has been written to any output. int4_last_error() then returns a
 *    description (thread-local; valid until the next call on this thread).
 *  - Inputs are never modified; outputs are overwritten in full, including
 *    the zero pad nibble of an odd K.
 *  - There is no alignment requirement. Internally, 16-byte aligned bases with
 *    suitable strides select the vectorised kernels; anything else runs a
 *    general kernel with the same results.
 *  - Calls hold no global state besides the thread-local error text, so they
 *    may be issued concurrently from several threads and streams.
 *  - Preconditions not checked: weights and activations are finite, and
 *    |w| <= 7 * 65504 (so every scale is finite in binary16).
 */
#ifndef INT4DQ_H
#define INT4DQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by the entry points. */
#define INT4DQ_OK           0  /* enqueued */
#define INT4DQ_EINVAL       1  /* bad argument: size, null pointer, dtype, overflow */
#define INT4DQ_EUNSUPPORTED 2  /* a forced kernel path that cannot take this shape/layout */
#define INT4DQ_EHIP         3  /* the HIP runtime refused the launch */

/* Element type of the activations x in int4_matmul. */
#define INT4DQ_X_F32 0         /* IEEE binary32 */
#define INT4DQ_X_F16 1         /* IEEE binary16 */

/* Element type of the output of int4_dequantize. */
#define INT4DQ_OUT_F32 0       /* IEEE binary32 */
#define INT4DQ_OUT_F16 1       /* IEEE binary16 */

/* Element type of y in int4_linear (the other matmul calls write binary32). */
#define INT4DQ_Y_F32 0         /* IEEE binary32 */
#define INT4DQ_Y_F16 1         /* IEEE binary16: the binary32 result rounded to nearest even */

/* Output activation of int4_matmul_ex / int4_matmul_path. */
#define INT4DQ_ACT_NONE 0      /* y = v */
#define INT4DQ_ACT_RELU 1      /* y = v > 0 ? v : +0 */

/* Kernel selection for int4_matmul_path (int4_matmul always uses AUTO). */
#define INT4DQ_PATH_AUTO    0  /* choose by M, dtype and alignment */
#define INT4DQ_PATH_GENERIC 1  /* VALU kernel, any shape, any group, fp32 or fp16 x */
#define INT4DQ_PATH_SKINNY  2  /* M <= 64, fp16 x, N < 2^25: weight-streaming MFMA kernel */
#define INT4DQ_PATH_TILED   3  /* any M, fp16 x, M and N < 2^31 and fewer than 2^24 output
                                   tiles (128 x 256 for large M): LDS-tiled MFMA kernel */
#define INT4DQ_PATH_GEMV    4  /* fp16 x, N < 2^25, group and K multiples of 32, M = 1; or M <= 4
                                   with K <= 12288 and group = 32 * 2^p: weight-streaming kernels */

/*
 * Number of scale groups per row, G = ceil(K / group) (drill page,
 * statement: scales [N, G]). Returns -1 if K < 1 or group < 1.
 */
int64_t int4_num_groups(int64_t K, int64_t group);

/*
 * Bytes of the packed weight array, N * ceil(K / 2) (drill page, statement:
 * packed [N, ceil(K / 2)] uint8). Returns -1 on N < 1, K < 1 or overflow.
 * The scale array takes a further 2 * N * G bytes.
 */
int64_t int4_packed_bytes(int64_t N, int64_t K);

/*
 * quantize_int4 (drill page, statement).
 *   w       in : [N, K] binary32 weights.
 *   packed  out: [N, ceil(K/2)] bytes. Byte j of row n holds element 2j in its
 *                low nibble and element 2j+1 in its high nibble, each the 4-bit
 *                two's complement code q = clip(round(w / scale), -8, 7); an odd
 *                K leaves a zero high nibble in the row's last byte.
 *   scales  out: [N, G] binary16 bit patterns, G = ceil(K / group). Group gi of
 *                row n covers k in [gi*group, min((gi+1)*group, K)); its scale is
 *                binary16(absmax / 7), the division done in binary32 and both
 *                roundings to nearest even; a group of zeros gets scale 0 and
 *                codes 0.
 *   Rounding of w / scale: the divisor is the stored binary16 scale widened to
 *   binary32, the division is correctly rounded binary32, and ties round to
 *   even (NumPy's round). Bit-exact with a CPU reference computing the same.
 *   Errors: EINVAL if N, K or group < 1, a pointer is NULL, or sizes overflow.
 */
int int4_quantize(const float *w, int64_t N, int64_t K, int64_t group,
                  uint8_t *packed, uint16_t *scales, void *stream);

/*
 * unpack_int4 (drill page, statement): int8 [N, K], sign-extended.
 *   packed in : [N, ceil(K/2)] bytes in the layout written by int4_quantize.
 *   out    out: [N, K] int8, out[n, k] = the sign-extended nibble of element k
 *               (the pad nibble of an odd K is not emitted).
 *   Errors: EINVAL if N or K < 1, a pointer is NULL, or sizes overflow.
 */
int int4_unpack(const uint8_t *packed, int64_t N, int64_t K, int8_t *out, void *stream);

/*
 * Dequantize (drill page, statement: the reconstruction w_hat = q * scale;
 * "Build a Blockwise INT4 Inference Engine": the materialised weights of the
 * unfused dequantize-then-GEMM baseline that the fused matmul avoids).
 *   packed  in : [N, ceil(K/2)] bytes, scales in: [N, G] binary16, as written
 *                by int4_quantize with the same K and group.
 *   out     out: [N, K] of out_dtype. INT4DQ_OUT_F32: q * scale exactly (q has
 *                4 significant bits and the scale 11). INT4DQ_OUT_F16: that
 *                exact product rounded to the nearest binary16, ties to even
 *                (magnitudes from 65520 up become infinities).
 *   Errors: EINVAL if N, K or group < 1, a pointer is NULL, out_dtype is
 *   unknown, or sizes overflow.
 */
int int4_dequantize(const uint8_t *packed, const uint16_t *scales, int64_t N, int64_t K,
                    int64_t group, int out_dtype, void *out, void *stream);

/*
 * int4_matmul (drill page, statement):
 *   y = x @ dequantize(W).T, the statement's sum over groups of the group's
 *   scale times x dotted with the group's integer weights, without writing
 *   full-precision weights to memory.
 *   x       in : [M, K], element type x_dtype (INT4DQ_X_F32 or INT4DQ_X_F16).
 *   packed  in : [N, ceil(K/2)] bytes, scales in: [N, G] binary16, as written
 *                by int4_quantize with the same K and group.
 *   y       out: [M, N] binary32.
 *   Arithmetic: sums in binary32. The kernels for a few rows of x form each
 *   group's integer dot product (fp16 x times the exact integer codes) and
 *   multiply it by the group's scale; the kernel for many rows multiplies each
 *   code by its scale in binary16 first (q * scale rounded once, at most 2^-11
 *   relative) and accumulates x times that. Either way each output is within
 *   2e-3 * sum_k |x[m,k] * q[n,k] * scale| of the exactly rounded result.
 *   A group whose scale is zero (+0 or -0) contributes nothing, whatever its
 *   codes. M = 0 is a valid no-op. The pad nibble of an odd K is never used
 *   and x[:, K] is never read. Every shape that passes the checks below is
 *   computed: where the fast kernels' limits (INT4DQ_PATH_*) exclude it, the
 *   generic kernel takes it.
 *   Errors: EINVAL if M < 0, N, K or group < 1, a pointer is NULL (when M > 0),
 *   x_dtype is unknown, or sizes overflow.
 */
int int4_matmul(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                const uint16_t *scales, int64_t N, int64_t K, int64_t group,
                float *y, void *stream);

/*
 * int4_matmul with the output step of the engine page's fused kernel and
 * layer forward ("Build a Blockwise INT4 Inference Engine"):
 *   y = act(x @ dequantize(W).T + bias)
 *   bias in : [N] binary32 added to every row, or NULL for none.
 *   act     : INT4DQ_ACT_NONE or INT4DQ_ACT_RELU (v > 0 ? v : +0).
 * The matmul part is int4_matmul's; the bias is one binary32 add after it.
 * Each output is within 2e-3 * sum_k |x[m,k] * q[n,k] * scale| + 2^-22 * |y|
 * of act applied to the exact sum plus bias rounded once.
 * Errors: those of int4_matmul, and EINVAL for an unknown act.
 */
int int4_matmul_ex(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                   const uint16_t *scales, int64_t N, int64_t K, int64_t group,
                   const float *bias, int act, float *y, void *stream);

/*
 * int4_matmul_ex with an explicit kernel choice (INT4DQ_PATH_*), for testing
 * one kernel against another on the same shapes. Same arguments, results
 * and errors as int4_matmul_ex, plus EUNSUPPORTED when the forced kernel
 * cannot take this dtype, shape, group or alignment (the reason is in
 * int4_last_error()).
 */
int int4_matmul_path(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                     const uint16_t *scales, int64_t N, int64_t K, int64_t group,
                     const float *bias, int act, float *y, int path, void *stream);

/*
 * Affine (asymmetric) variant of the codes ("Build a Blockwise INT4 Inference
 * Engine", step 2: per-group scale and zero point, codes in [0, 15], value
 * (q - zp) * scale; "Quantizing a Language Model From Scratch", affine
 * quantization: the zero point makes 0.0 exact).
 *
 * int4_quantize_affine:
 *   w       in : [N, K] binary32 weights.
 *   packed  out: [N, ceil(K/2)] bytes, the same nibble layout as int4_quantize
 *                but each nibble an UNSIGNED code u in [0, 15]; an odd K leaves
 *                a zero high nibble in the row's last byte.
 *   scales  out: [N, G] binary16 bit patterns, zeros out: [N, G] bytes.
 *   For group gi of row n, with lo = min(min w, 0) and hi = max(max w, 0)
 *   over the group (the range always contains zero):
 *     scale = binary16((hi - lo) / 15)   subtraction and division in binary32
 *     zp    = clip(round(-lo / scale), 0, 15)
 *     u     = clip(round(w / scale + zp), 0, 15)
 *   where every division uses the stored scale widened to binary32 and is a
 *   correctly rounded binary32 division, w / scale + zp is formed exactly,
 *   and round() is ties-to-even. A group whose scale is 0 gets zp = 0 and
 *   codes 0. Bit-exact with a CPU reference computing the same.
 *   Errors: EINVAL if N, K or group < 1, a pointer is NULL, or sizes overflow.
 */
int int4_quantize_affine(const float *w, int64_t N, int64_t K, int64_t group,
                         uint8_t *packed, uint16_t *scales, uint8_t *zeros, void *stream);

/*
 * int4_dequantize for affine codes: out[n, k] = (u[n, k] - zp) * scale of
 * element k's group, in out_dtype (binary32: exact; binary16: the exact value
 * rounded to nearest even). zeros: [N, G] bytes, values in [0, 15], as written
 * by int4_quantize_affine with the same K and group.
 * Errors: those of int4_dequantize, and EINVAL if zeros is NULL.
 */
int int4_dequantize_affine(const uint8_t *packed, const uint16_t *scales, const uint8_t *zeros,
                           int64_t N, int64_t K, int64_t group, int out_dtype, void *out,
                           void *stream);

/*
 * int4_matmul_path for affine codes:
 *   y = act(x @ dequantize_affine(W).T + bias), one group at a time: x times
 *   the group's integer weights u - zp first, then the group's scale.
 * Same arguments, layouts, arithmetic and errors as int4_matmul_path, plus
 * zeros ([N, G] bytes in [0, 15], as written by int4_quantize_affine; EINVAL if
 * NULL). Each output is within 2e-3 * sum_k |x[m,k] * (u[n,k] - zp) * scale|
 * (+ 2^-22 * |y| with a bias) of act applied to the exact result. Every
 * kernel path (INT4DQ_PATH_*) takes affine codes under the same conditions as
 * symmetric ones.
 */
int int4_matmul_affine(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                       const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                       int64_t group, const float *bias, int act, float *y, int path,
                       void *stream);

/*
 * One quantized linear layer, the engine page's layer forward ("Build a
 * Blockwise INT4 Inference Engine": y = act(x @ W_dq.T + b)), in the output
 * precision the next layer takes:
 *   y = act(x @ dequantize(W).T + bias), written as y_dtype.
 *   zeros   in : NULL for symmetric codes (int4_quantize), else the [N, G] zero
 *                points of affine codes (int4_quantize_affine).
 *   y       out: [M, N] of y_dtype. INT4DQ_Y_F32 as int4_matmul_ex /
 *                int4_matmul_affine; INT4DQ_Y_F16 rounds that binary32 result to
 *                nearest even (overflowing to infinity past 65504), so a chain
 *                of layers passes fp16 activations with no conversion pass.
 * The kernel is chosen as int4_matmul does. Other arguments, layouts and
 * errors as int4_matmul_affine (zeros may be NULL), plus EINVAL for an
 * unknown y_dtype.
 */
int int4_linear(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                int64_t group, const float *bias, int act, void *y, int y_dtype, void *stream);

/*
 * int4_linear with a caller-owned device workspace, which lets a kernel cut K
 * into shares when its grid is too small to fill the GPU: the kernel for many
 * rows of x when its output tiles are few (a few hundred rows against a few
 * thousand weight rows), and the kernel for 5 to 64 rows when the weight
 * matrix has fewer than 2048 rows and long rows (a small transformer's MLP
 * down projection at 16 or more rows, 64 rows against 1024 weight rows of
 * 8192 codes). Each share's partial tile goes to the workspace and a second
 * kernel adds the partials in share order and applies bias, activation and
 * the output precision, so results do not depend on timing and stay within
 * the tolerance of int4_matmul. Engine page ("Build a Blockwise INT4 Inference
 * Engine"), layer forward, as int4_linear.
 *   workspace       : device memory, 256-byte aligned, any contents, or NULL
 *                     with workspace_bytes = 0.
 *   workspace_bytes : its size. A call whose shape wants more than this (see
 *                     int4_linear_workspace_bytes) runs without the split, as
 *                     int4_linear does.
 * Calls that share a workspace must not overlap (same stream, or ordered by
 * events): they use it as their scratch. Other arguments, results and errors
 * as int4_linear, plus EINVAL for a negative size, a NULL workspace with a
 * positive size or a workspace that is not 256-byte aligned.
 */
int int4_linear_ws(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                   const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                   int64_t group, const float *bias, int act, void *y, int y_dtype,
                   void *workspace, int64_t workspace_bytes, void *stream);

/*
 * int4_linear_ws for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same call with the library's own scratch as the workspace. The library
 * holds one 16 MiB scratch array per GPU from module load to the end of the
 * process (the split plans need at most that); this call allocates and frees
 * nothing. The device of the call's stream must be the current device.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (several streams or threads at once) race, so they must be ordered.
 * Arguments, results and errors as int4_linear, plus EINVAL when a shape would
 * need more scratch than the library holds, EUNSUPPORTED for a device ordinal
 * of 64 or more, and EHIP if the scratch's device address cannot be obtained.
 */
int int4_linear_noalloc(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                        const uint16_t *scales, const uint8_t *zeros, int64_t N, int64_t K,
                        int64_t group, const float *bias, int act, void *y, int y_dtype,
                        void *stream);

/*
 * Workspace bytes int4_linear_ws uses for M rows of x_dtype activations, an
 * [N, K] weight matrix and this group size, with 16-byte aligned x and packed
 * codes (0: the call does not split K). -1 on invalid sizes or dtype.
 */
int64_t int4_linear_workspace_bytes(int x_dtype, int64_t M, int64_t N, int64_t K, int64_t group);

/*
 * Kernel that int4_matmul would run for these arguments (an INT4DQ_PATH_*
 * other than AUTO), or -1 if the arguments are invalid. Enqueues nothing.
 */
int int4_matmul_select(const void *x, int x_dtype, int64_t M, const uint8_t *packed,
                       const uint16_t *scales, int64_t N, int64_t K, int64_t group,
                       const float *y);

/* Text describing the last non-OK status on the calling thread ("" if none). */
const char *int4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* INT4DQ_H */
