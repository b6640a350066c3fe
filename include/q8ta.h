/*
 * libq8ta -- int8 quantized-activation ("q8ta") operations for AMD Instinct
 * MI355X (gfx950), C ABI.
 *
 * The operations follow three ExecuTorch WebGPU pull-request pages:
 *   [QPT]  "Add quantize_per_tensor op (int8 buffer path)" (#21187)
 *   [LIN]  "Add q8ta_linear op (int8 quantized linear)"     (#21197)
 *   [DCV]  "Add q8ta_conv2d_transposed op (int8 transposed conv)" (#21205)
 *
 * Common rules for every entry point:
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *     allocated and owned by the caller; the library never frees or retains
 *     it.  Tensors are dense and contiguous in the stated layout.  int8
 *     tensors are plain byte arrays (element i at byte i).
 *   - Workspace: some paths need device scratch memory: the fused
 *     quantize entry points take an int8 copy of their input
 *     (q8ta_quantize_linear(_dq) with M > 4 or a shape the M <= 4 kernel
 *     refuses: M * K bytes; q8ta_quantize_conv2d_transposed:
 *     N * IC * H_in * W_in bytes); q8ta_conv2d_transposed(_acc) and
 *     q8ta_conv2d(_acc) take, on their implicit-GEMM path, an NHWC copy of
 *     the input inside a zero-point border plus 4 * stride_h * stride_w * OC
 *     bytes of weight sums, and on the transposed conv's tiled path a
 *     channel-blocked copy of the input (N * H_in * ceil(IC/16) * W_in * 16
 *     bytes).  The default matrix-core kernels of q8ta_linear and
 *     q8ta_conv2d_transposed take none.  The library keeps up to 4 such
 *     buffers per device and holds them until the process ends.  Taking one
 *     never blocks the host: a buffer last used on another stream is ordered
 *     after that use with hipStreamWaitEvent, and one that is too small is
 *     replaced in stream order (hipFreeAsync / hipMallocAsync on `stream`).
 *     When all 4 are in use, under graph capture and above 256 MiB a call
 *     takes its own stream-ordered allocation instead.  A failed allocation
 *     returns Q8TA_ERR_HIP.
 *   - Sizes: element counts up to 2^40 per tensor (the kernels address in
 *     64 bits; a row length K of the linear below 2^31).
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns after the launch; results are visible to later work on that
 *     stream.  Calls are reentrant (several host threads may call at once)
 *     and keep no state between calls except the cached workspaces and the
 *     kernel choice of q8ta_select_kernel.
 *   - Scales are passed as double.  The library forms every reciprocal as
 *     (float)(1.0 / scale) in double on the host ([QPT] commit message) and
 *     uses (float)scale for a scale that multiplies.
 *   - Rounding is round-half-to-even; the dequant/requant epilogue is
 *     evaluated in float, left to right, one rounding per operation, with no
 *     fused multiply-add:  v = ((float)acc * (float)input_scale) *
 *     weight_scales[c] + bias[c];  q = clamp(rint(v * inv_output_scale) +
 *     output_zero_point, -128, 127)  ([LIN]/[DCV] Solution).
 *   - Accumulators are int32 ([LIN] Solution: an i32 GEMM).  Inputs whose
 *     exact sums leave the int32 range are outside the contract.
 *   - Errors are loud: on any invalid argument the call returns a non-zero
 *     q8ta_status, launches nothing, and q8ta_last_error() describes the
 *     problem.  Argument checks run before any HIP runtime call.
 *     Q8TA_ERR_HIP reports a failed launch (for example, no GPU present).
 *     NaN inputs are outside the contract.
 */
#ifndef Q8TA_H
#define Q8TA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum q8ta_status {
  Q8TA_OK = 0,
  Q8TA_ERR_NULL = 1,        /* a required pointer is NULL */
  Q8TA_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  Q8TA_ERR_QPARAM = 3,      /* a scale is not finite and > 0, or a zero point is outside [-128, 127] */
  Q8TA_ERR_UNSUPPORTED = 4, /* an argument value the op does not implement (an activation other than "none" / "relu") */
  Q8TA_ERR_HIP = 5          /* the HIP runtime reported an error */
} q8ta_status;

/* Message for the last non-OK status returned on the calling thread
 * (a static or thread-local string; never NULL). */
const char* q8ta_last_error(void);

/* Kernel-family choice, for testing and tuning; callers of the ops never need
 * it.  Forces one kernel family of an op where the shape allows it (shapes
 * that family cannot take keep the default choice); results are bit-identical
 * whichever kernel runs.  Process-wide: applies to calls made after it returns.
 *   op "linear":            kernel "default" | "mfma32" | "mfma32_8w" |
 *                           "generic"
 *                           (mfma32: the 32x32x32 matrix-core GEMM with two
 *                           four-wave workgroups per CU for every shape the
 *                           matrix-core path takes; mfma32_8w: the
 *                           eight-wave 256 x 256-tile form where K is a
 *                           multiple of 64; generic: the shape-general
 *                           kernel instead of the GEMV / matrix-core GEMM)
 *   op "conv2d_transposed": "default" | "fixed" | "mfma32" | "mfma" | "igemm" |
 *                           "tiled" | "generic"
 *   op "conv2d":            "default" | "fixed" | "mfma32" | "mfma" | "igemm" |
 *                           "generic"
 * Returns Q8TA_ERR_NULL for a NULL name and Q8TA_ERR_UNSUPPORTED for an unknown
 * op or kernel name (the choice is then unchanged).  Host-only, no HIP call. */
q8ta_status q8ta_select_kernel(const char* op, const char* kernel);

/* ---------------------------------------------------------------------------
 * [QPT] commit message (Solution / Implementation):
 *   out[i] = clamp(rint(x[i] * (float)(1.0 / scale)) + zero_point, -128, 127)
 * x: fp32 [numel]; out: int8 [numel]; numel >= 0 (0 is a no-op).
 * scale finite and > 0; zero_point in [-128, 127].
 * The page's numel % 4 requirement (a WebGPU word-binding artifact) does not
 * apply: any numel and any byte alignment of out is accepted.
 */
q8ta_status q8ta_quantize_per_tensor(const float* x, int8_t* out, int64_t numel,
                                     double scale, int64_t zero_point,
                                     hipStream_t stream);

/* ---------------------------------------------------------------------------
 * dequantize_per_tensor, the op named beside the q8ta ops in the
 * quantize -> q8ta_* -> dequantize subgraph ([LIN]/[DCV] Problem); the pages
 * do not print it, and the decomposed definition is used:
 *   out[i] = (float)(x[i] - zero_point) * (float)scale
 * x: int8 [numel]; out: fp32 [numel]; numel >= 0.  Same checks as quantize.
 */
q8ta_status q8ta_dequantize_per_tensor(const int8_t* x, float* out, int64_t numel,
                                       double scale, int64_t zero_point,
                                       hipStream_t stream);

/* ---------------------------------------------------------------------------
 * q8ta_linear ([LIN] Solution and Constraints (2)):
 *   acc[m,n] = sum_k (x[m,k] - input_zero_point) * weight[n,k]      (int32)
 *   out[m,n] = epilogue(acc[m,n]) with channel c = n
 * x: int8 [M, K] row-major; weight: int8 [N, K] row-major (symmetric, no
 * weight zero point); weight_scales: fp32, at least N entries (only [0, N)
 * is read); bias: fp32, at least N entries, or NULL for no bias;
 * out: int8 [M, N] row-major.  M, K, N >= 1.
 * weight_sums: accepted and ignored, as on the page (the zero-point term is
 * computed from the weights on every call); may be NULL.
 * activation: "none", or "relu" for the relu-fused variant that [LIN]
 * Implementation names as a follow-up: the epilogue then requantizes
 * max(v, 0), so every code is at least output_zero_point.  Anything else
 * (including NULL) returns Q8TA_ERR_UNSUPPORTED.
 * The page's N % 4 and M*K % 4 requirements do not apply.
 */
q8ta_status q8ta_linear(const int8_t* x, int64_t M, int64_t K,
                        double input_scale, int64_t input_zero_point,
                        const int8_t* weight, int64_t N,
                        const int32_t* weight_sums,
                        const float* weight_scales, const float* bias,
                        double output_scale, int64_t output_zero_point,
                        const char* activation, int8_t* out,
                        hipStream_t stream);

/* q8ta_linear_gemv ([LIN] Solution: identical schema, the M == 1 case, served
 * by the same handler).  Same arguments and results as q8ta_linear; returns
 * Q8TA_ERR_SHAPE unless M == 1. */
q8ta_status q8ta_linear_gemv(const int8_t* x, int64_t M, int64_t K,
                             double input_scale, int64_t input_zero_point,
                             const int8_t* weight, int64_t N,
                             const int32_t* weight_sums,
                             const float* weight_scales, const float* bias,
                             double output_scale, int64_t output_zero_point,
                             const char* activation, int8_t* out,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * q8ta_linear followed by dequantize_per_tensor of its output, in one call
 * (the q8ta_linear -> dequantize chain the [LIN] Problem section describes,
 * with the dequantize folded into the epilogue):
 *   out[m, n] = (float)(q[m, n] - output_zero_point) * (float)output_scale,
 *   q = the int8 result q8ta_linear would produce for the same arguments.
 * Bit-identical to the two calls; the int8 tensor is never written.
 * out: fp32 [M, N] row-major.  Other arguments as for q8ta_linear.
 */
q8ta_status q8ta_linear_dq(const int8_t* x, int64_t M, int64_t K,
                           double input_scale, int64_t input_zero_point,
                           const int8_t* weight, int64_t N,
                           const int32_t* weight_sums,
                           const float* weight_scales, const float* bias,
                           double output_scale, int64_t output_zero_point,
                           const char* activation, float* out,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * quantize_per_tensor of fp32 activations followed by q8ta_linear (and, for
 * the _dq form, by dequantize_per_tensor of its output), in one call: the
 * whole quantize -> q8ta_linear -> dequantize chain of the [LIN] Problem
 * section.
 *   xq[m, k] = clamp(rint(x[m, k] * (float)(1/input_scale)) + input_zero_point,
 *                    -128, 127)   (the q8ta_quantize_per_tensor formula)
 *   q8ta_quantize_linear:    out = q8ta_linear(xq, ...)            int8 [M, N]
 *   q8ta_quantize_linear_dq: out = q8ta_linear_dq(xq, ...)          fp32 [M, N]
 * Bit-identical to the two (three) separate calls with the same scales and
 * zero points.  x: fp32 [M, K] row-major, device.  For M <= 4 with K % 16 == 0
 * and 16-byte aligned x and weight the activations are quantized inside the
 * weight-streaming kernel and xq is never stored; otherwise the library
 * quantizes into its own stream-ordered workspace (M * K bytes) and runs the
 * q8ta_linear path.  Other arguments, requirements and errors as for
 * q8ta_linear / q8ta_linear_dq (x NULL -> Q8TA_ERR_NULL).
 */
q8ta_status q8ta_quantize_linear(const float* x, int64_t M, int64_t K,
                                 double input_scale, int64_t input_zero_point,
                                 const int8_t* weight, int64_t N,
                                 const int32_t* weight_sums,
                                 const float* weight_scales, const float* bias,
                                 double output_scale, int64_t output_zero_point,
                                 const char* activation, int8_t* out,
                                 hipStream_t stream);
q8ta_status q8ta_quantize_linear_dq(const float* x, int64_t M, int64_t K,
                                    double input_scale, int64_t input_zero_point,
                                    const int8_t* weight, int64_t N,
                                    const int32_t* weight_sums,
                                    const float* weight_scales, const float* bias,
                                    double output_scale, int64_t output_zero_point,
                                    const char* activation, float* out,
                                    hipStream_t stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation as q8ta_quantize_linear, bit-identical results, but the call never
 * allocates.  Shapes the M <= 4 kernel takes need no staging; every other
 * shape stages its quantized activations (M * K bytes) in a static device
 * array of 16 MiB (16,777,216 bytes) that the library holds on each GPU it runs
 * on until the process ends, and a call with M * K above that size returns
 * Q8TA_ERR_SHAPE before any HIP call.  All calls on one GPU share that array
 * and it keeps the last call's contents (every call writes the bytes it reads
 * first): calls that overlap in time on one GPU -- on different streams or
 * from different threads -- race, and the caller must order them.  The array's
 * device address is looked up once per device on the first call.  Arguments,
 * requirements and other errors as for q8ta_quantize_linear.
 */
q8ta_status q8ta_quantize_linear_noalloc(const float* x, int64_t M, int64_t K,
                                         double input_scale, int64_t input_zero_point,
                                         const int8_t* weight, int64_t N,
                                         const int32_t* weight_sums,
                                         const float* weight_scales, const float* bias,
                                         double output_scale, int64_t output_zero_point,
                                         const char* activation, int8_t* out,
                                         hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Precomputed weight sums (opt-in).  [LIN] Constraints (1): the zero-point
 * term needs sum_k weight[n, k]; the pages' op ignores its weight_sums
 * argument and folds the term per call, while the Vulkan op it mirrors takes
 * the sums precomputed.  These entry points offer the latter for weights that
 * are reused across calls:
 *   q8ta_weight_sums:  sums[n] = sum_{k<K} weight[n*K + k] (int32 [N]; exact
 *     for K < 2^24).  weight: int8 [N, K] row-major.  Any K and alignment.
 *   q8ta_linear_presummed / q8ta_linear_dq_presummed: q8ta_linear /
 *     q8ta_linear_dq with weight_sums REQUIRED (NULL -> Q8TA_ERR_NULL) and
 *     TRUSTED: the kernels subtract input_zero_point * weight_sums[n] instead of
 *     forming the sums themselves.  With the sums q8ta_weight_sums returns the
 *     results are bit-identical to q8ta_linear / q8ta_linear_dq; other sums
 *     give other results (the library cannot check them).  All other
 *     arguments, requirements and errors as for q8ta_linear / q8ta_linear_dq.
 */
q8ta_status q8ta_weight_sums(const int8_t* weight, int64_t N, int64_t K, int32_t* sums,
                             hipStream_t stream);

q8ta_status q8ta_linear_presummed(const int8_t* x, int64_t M, int64_t K,
                                  double input_scale, int64_t input_zero_point,
                                  const int8_t* weight, int64_t N,
                                  const int32_t* weight_sums,
                                  const float* weight_scales, const float* bias,
                                  double output_scale, int64_t output_zero_point,
                                  const char* activation, int8_t* out,
                                  hipStream_t stream);

q8ta_status q8ta_linear_dq_presummed(const int8_t* x, int64_t M, int64_t K,
                                     double input_scale, int64_t input_zero_point,
                                     const int8_t* weight, int64_t N,
                                     const int32_t* weight_sums,
                                     const float* weight_scales, const float* bias,
                                     double output_scale, int64_t output_zero_point,
                                     const char* activation, float* out,
                                     hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Prepacked weights (opt-in; the prepacked-layout half of the weight
 * preparation the Vulkan op behind [LIN] does ahead of time, Constraints
 * (1)/(2)).  A weight reused across calls is rearranged once into the operand
 * order of the int8 matrix-core instruction, so the GEMM streams it without
 * staging:
 *   packed layout: fragments of 32 rows x 32 K bytes; byte 16*l + j of
 *     fragment (nb, s) is weight[32*nb + l % 32][32*s + 16*(l / 32) + j]
 *     (l = 0..63, j = 0..15), zero past N or K; fragment (nb, s) starts at
 *     byte (nb * KS + s) * 1024 with KS = 2 * ceil(K / 64).
 *   q8ta_weight_prepacked_bytes: size of that buffer,
 *     ceil(N/32)*32 * ceil(K/64)*64 bytes; -1 for N < 1, K < 1 or sizes past
 *     2^31 elements.  Host-only, no HIP call.
 *   q8ta_weight_prepack: weight int8 [N, K] row-major -> packed (device,
 *     caller-allocated, q8ta_weight_prepacked_bytes(N, K) bytes).  Needs
 *     K % 16 == 0 and 16-byte aligned weight and packed
 *     (else Q8TA_ERR_UNSUPPORTED).
 *   q8ta_linear_prepacked / q8ta_linear_dq_prepacked: q8ta_linear_presummed /
 *     q8ta_linear_dq_presummed with packed_weight in place of weight (N is the
 *     weight's row count, K its row length).  weight_sums is REQUIRED and
 *     TRUSTED (sum over the unpacked rows, as q8ta_weight_sums returns).
 *     Needs K % 16 == 0 and 16-byte aligned x and packed_weight
 *     (else Q8TA_ERR_UNSUPPORTED).  With the weight's own sums the results are
 *     bit-identical to q8ta_linear / q8ta_linear_dq.  Other arguments and
 *     errors as for q8ta_linear / q8ta_linear_dq.
 */
int64_t q8ta_weight_prepacked_bytes(int64_t N, int64_t K);

q8ta_status q8ta_weight_prepack(const int8_t* weight, int64_t N, int64_t K, int8_t* packed,
                                hipStream_t stream);

q8ta_status q8ta_linear_prepacked(const int8_t* x, int64_t M, int64_t K,
                                  double input_scale, int64_t input_zero_point,
                                  const int8_t* packed_weight, int64_t N,
                                  const int32_t* weight_sums,
                                  const float* weight_scales, const float* bias,
                                  double output_scale, int64_t output_zero_point,
                                  const char* activation, int8_t* out,
                                  hipStream_t stream);

q8ta_status q8ta_linear_dq_prepacked(const int8_t* x, int64_t M, int64_t K,
                                     double input_scale, int64_t input_zero_point,
                                     const int8_t* packed_weight, int64_t N,
                                     const int32_t* weight_sums,
                                     const float* weight_scales, const float* bias,
                                     double output_scale, int64_t output_zero_point,
                                     const char* activation, float* out,
                                     hipStream_t stream);

/* ---------------------------------------------------------------------------
 * q8ta_conv2d_transposed ([DCV] Solution, Implementation, Constraints):
 *   acc[n,oc,oh,ow] = sum over (ic, kh, kw) of
 *       (x[n,ic,ih,iw] - input_zero_point) * weight[oc, (kh*Kw + kw)*IC + ic]
 *   where ih = (oh + pad_h - kh*dilation_h) / stride_h is used only when the
 *   numerator is >= 0, divisible by stride_h and ih < H_in (iw likewise);
 *   out[n,oc,oh,ow] = epilogue(acc) with channel c = oc.
 * x: int8 NCHW [N, IC, H_in, W_in]; weight: int8 [OC, weight_row_stride],
 * weight_row_stride >= Kh*Kw*IC (row padding is tolerated, only the first
 * Kh*Kw*IC bytes of a row are read); weight_scales / bias: fp32 with at least
 * OC entries (bias may be NULL); out: int8 NCHW [N, OC, H_out, W_out].
 * H_out and W_out are given explicitly (the page takes them from the
 * serialized output dims); output_padding_h/_w are accepted and unused.
 * Requirements: all sizes >= 1, stride >= 1, padding >= 0, dilation in
 * [1, 4096], groups dividing IC and OC; activation "none" or "relu" (as for
 * q8ta_linear).  weight_sums is ignored.
 * Dilation, groups and relu are the follow-ups the page keeps fail-loud.
 * Dilation enters the gather's numerator as printed.  Groups (not on the
 * page): output channel oc of group g = oc / (OC/groups) sums only over input
 * channels g*(IC/groups) + icg, with weight[oc, (kh*Kw + kw)*(IC/groups) + icg]
 * (weight_row_stride >= Kh*Kw*IC/groups) -- the page's reshape of the
 * original [IC, OC, Kh, Kw] weight applied to each group's block.
 * Kernels: the 3x3 / 4x4 stride-2 shapes with at least 256 tiles take a
 * compile-time-pattern matrix-core kernel; other groups-1 shapes a tiled
 * matrix-core kernel, an implicit GEMM or a tiled direct kernel; grouped
 * shapes a one-output-per-thread kernel.
 */
q8ta_status q8ta_conv2d_transposed(const int8_t* x, int64_t N, int64_t IC,
                                   int64_t H_in, int64_t W_in,
                                   double input_scale, int64_t input_zero_point,
                                   const int8_t* weight, int64_t OC,
                                   int64_t Kh, int64_t Kw,
                                   int64_t weight_row_stride,
                                   const int32_t* weight_sums,
                                   const float* weight_scales, const float* bias,
                                   double output_scale, int64_t output_zero_point,
                                   int64_t stride_h, int64_t stride_w,
                                   int64_t pad_h, int64_t pad_w,
                                   int64_t output_padding_h, int64_t output_padding_w,
                                   int64_t dilation_h, int64_t dilation_w,
                                   int64_t groups, const char* activation,
                                   int8_t* out, int64_t H_out, int64_t W_out,
                                   hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Prepacked transposed-conv weight (opt-in; the prepacked-layout half of the
 * weight preparation [DCV] Constraints (1) leaves to the caller, as for the
 * GEMM above).  A weight reused across calls is rearranged once so that every
 * matrix-core operand fragment the compile-time-pattern kernel reads is one
 * contiguous KiB:
 *   packed layout: byte 16*l + j of fragment (ob, kh, kw, kc) is
 *     weight[32*ob + l % 32][(kh*Kw + kw)*IC + 32*kc + 16*(l / 32) + j]
 *     (l = 0..63, j = 0..15), zero for rows past OC; the fragment starts at
 *     byte (((ob*Kh + kh)*Kw + kw)*(IC/32) + kc) * 1024.
 *   q8ta_conv2d_transposed_weight_prepacked_bytes: size of that buffer,
 *     ceil(OC/32)*32 * Kh*Kw*IC bytes; -1 for sizes < 1, IC % 64 != 0 or sizes
 *     past 2^40 elements.  Host-only, no HIP call.
 *   q8ta_conv2d_transposed_weight_prepack: weight int8 [OC, weight_row_stride]
 *     (as for q8ta_conv2d_transposed) -> packed (device, caller-allocated,
 *     q8ta_conv2d_transposed_weight_prepacked_bytes(OC, IC, Kh, Kw) bytes).
 *     Needs IC % 64 == 0, weight_row_stride % 16 == 0 and 16-byte aligned
 *     weight and packed (else Q8TA_ERR_UNSUPPORTED).
 *   q8ta_conv2d_transposed_prepacked: q8ta_conv2d_transposed with
 *     packed_weight in place of weight and no weight_row_stride.  Takes only
 *     the shapes of the compile-time-pattern kernel: Kh == Kw in {3, 4},
 *     stride 2 x 2, pad_h % 2 == pad_w % 2, groups 1, dilation 1,
 *     IC % 64 == 0 with the input halo of a tile within LDS (IC <= 256),
 *     W_in % 4 == 0, 4-byte aligned x, 16-byte aligned packed_weight; other
 *     shapes return Q8TA_ERR_UNSUPPORTED (use q8ta_conv2d_transposed).  The
 *     results are bit-identical to q8ta_conv2d_transposed on the unpacked
 *     weight.  Other arguments and errors as for q8ta_conv2d_transposed.
 *   q8ta_quantize_conv2d_transposed_prepacked: q8ta_quantize_conv2d_transposed
 *     (fp32 input, quantized in the same call) on the packed weight; the same
 *     shapes, with a 16-byte aligned x (else Q8TA_ERR_UNSUPPORTED: use
 *     q8ta_quantize_conv2d_transposed).
 */
int64_t q8ta_conv2d_transposed_weight_prepacked_bytes(int64_t OC, int64_t IC, int64_t Kh,
                                                      int64_t Kw);

q8ta_status q8ta_conv2d_transposed_weight_prepack(const int8_t* weight, int64_t OC, int64_t IC,
                                                  int64_t Kh, int64_t Kw,
                                                  int64_t weight_row_stride, int8_t* packed,
                                                  hipStream_t stream);

q8ta_status q8ta_quantize_conv2d_transposed_prepacked(
    const float* x, int64_t N, int64_t IC, int64_t H_in, int64_t W_in, double input_scale,
    int64_t input_zero_point, const int8_t* packed_weight, int64_t OC, int64_t Kh, int64_t Kw,
    const int32_t* weight_sums, const float* weight_scales, const float* bias,
    double output_scale, int64_t output_zero_point, int64_t stride_h, int64_t stride_w,
    int64_t pad_h, int64_t pad_w, int64_t output_padding_h, int64_t output_padding_w,
    int64_t dilation_h, int64_t dilation_w, int64_t groups, const char* activation,
    int8_t* out, int64_t H_out, int64_t W_out, hipStream_t stream);

q8ta_status q8ta_conv2d_transposed_prepacked(const int8_t* x, int64_t N, int64_t IC,
                                             int64_t H_in, int64_t W_in,
                                             double input_scale, int64_t input_zero_point,
                                             const int8_t* packed_weight, int64_t OC,
                                             int64_t Kh, int64_t Kw,
                                             const int32_t* weight_sums,
                                             const float* weight_scales, const float* bias,
                                             double output_scale, int64_t output_zero_point,
                                             int64_t stride_h, int64_t stride_w,
                                             int64_t pad_h, int64_t pad_w,
                                             int64_t output_padding_h, int64_t output_padding_w,
                                             int64_t dilation_h, int64_t dilation_w,
                                             int64_t groups, const char* activation,
                                             int8_t* out, int64_t H_out, int64_t W_out,
                                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * quantize_per_tensor followed by q8ta_conv2d_transposed, in one call (the
 * chain the [DCV] Problem section describes, with the quantize folded into
 * the transposed conv's input read): x is fp32 NCHW [N, IC, H_in, W_in] and is
 * quantized with input_scale / input_zero_point exactly as
 * q8ta_quantize_per_tensor would; the result is bit-identical to the two
 * calls.  Other arguments, requirements and workspaces as for
 * q8ta_conv2d_transposed (plus, off the implicit-GEMM path, an int8 copy of
 * the quantized input).
 */
q8ta_status q8ta_quantize_conv2d_transposed(const float* x, int64_t N, int64_t IC,
                                            int64_t H_in, int64_t W_in,
                                            double input_scale, int64_t input_zero_point,
                                            const int8_t* weight, int64_t OC,
                                            int64_t Kh, int64_t Kw,
                                            int64_t weight_row_stride,
                                            const int32_t* weight_sums,
                                            const float* weight_scales, const float* bias,
                                            double output_scale, int64_t output_zero_point,
                                            int64_t stride_h, int64_t stride_w,
                                            int64_t pad_h, int64_t pad_w,
                                            int64_t output_padding_h, int64_t output_padding_w,
                                            int64_t dilation_h, int64_t dilation_w,
                                            int64_t groups, const char* activation,
                                            int8_t* out, int64_t H_out, int64_t W_out,
                                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * q8ta_conv2d: the forward int8 convolution whose scaffold and weight layout
 * the transposed op reuses ([DCV] Solution).  The pages print only the
 * transposed index relation; the forward one is the standard convolution's:
 *   acc[n,oc,oh,ow] = sum over (ic, kh, kw) of
 *       (x[n,ic,ih,iw] - input_zero_point) * weight[oc, (kh*Kw + kw)*IC + ic]
 *   with ih = oh*stride_h - pad_h + kh*dilation_h used only when
 *   0 <= ih < H_in (iw likewise);  out[n,oc,oh,ow] = epilogue(acc), c = oc.
 * Groups (not on the pages; the usual grouped convolution on the same
 * layout): groups must divide IC and OC; output channel oc belongs to group
 * g = oc / (OC/groups) and sums only over input channels g*(IC/groups) + icg,
 * with weight[oc, (kh*Kw + kw)*(IC/groups) + icg] (weight_row_stride >=
 * Kh*Kw*IC/groups).  groups == IC == OC is the depthwise convolution.
 * Layouts, scales, bias, weight_row_stride and the epilogue as for
 * q8ta_conv2d_transposed; H_out / W_out are given explicitly (any sizes >= 1).
 * Requirements: all sizes >= 1, stride >= 1, padding >= 0, dilation in
 * [1, 4096]; activation "none" or "relu".  weight_sums is ignored.  Workspace
 * on the implicit-GEMM path (groups 1, IC % 64 == 0): an NHWC copy of the
 * input inside a zero-point border plus 4 * OC bytes; none otherwise.
 */
q8ta_status q8ta_conv2d(const int8_t* x, int64_t N, int64_t IC,
                        int64_t H_in, int64_t W_in,
                        double input_scale, int64_t input_zero_point,
                        const int8_t* weight, int64_t OC,
                        int64_t Kh, int64_t Kw, int64_t weight_row_stride,
                        const int32_t* weight_sums,
                        const float* weight_scales, const float* bias,
                        double output_scale, int64_t output_zero_point,
                        int64_t stride_h, int64_t stride_w,
                        int64_t pad_h, int64_t pad_w,
                        int64_t dilation_h, int64_t dilation_w,
                        int64_t groups, const char* activation,
                        int8_t* out, int64_t H_out, int64_t W_out,
                        hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Accumulator outputs (for verification).  These run the same contraction
 * kernels as q8ta_linear / q8ta_conv2d_transposed / q8ta_conv2d but store the int32
 * accumulator (the sum above, zero-point term included) instead of the
 * requantized int8 value.  acc: int32 [M, N] row-major, or NCHW
 * [N, OC, H_out, W_out].  Argument checks as for the parent op.
 */
q8ta_status q8ta_linear_acc(const int8_t* x, int64_t M, int64_t K,
                            int64_t input_zero_point,
                            const int8_t* weight, int64_t N,
                            int32_t* acc, hipStream_t stream);

q8ta_status q8ta_conv2d_transposed_acc(const int8_t* x, int64_t N, int64_t IC,
                                       int64_t H_in, int64_t W_in,
                                       int64_t input_zero_point,
                                       const int8_t* weight, int64_t OC,
                                       int64_t Kh, int64_t Kw,
                                       int64_t weight_row_stride,
                                       int64_t stride_h, int64_t stride_w,
                                       int64_t pad_h, int64_t pad_w,
                                       int64_t dilation_h, int64_t dilation_w,
                                       int64_t groups,
                                       int32_t* acc, int64_t H_out, int64_t W_out,
                                       hipStream_t stream);

q8ta_status q8ta_conv2d_acc(const int8_t* x, int64_t N, int64_t IC,
                            int64_t H_in, int64_t W_in,
                            int64_t input_zero_point,
                            const int8_t* weight, int64_t OC,
                            int64_t Kh, int64_t Kw, int64_t weight_row_stride,
                            int64_t stride_h, int64_t stride_w,
                            int64_t pad_h, int64_t pad_w,
                            int64_t dilation_h, int64_t dilation_w, int64_t groups,
                            int32_t* acc, int64_t H_out, int64_t W_out,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8TA_H */
