/*
 * q8ta CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct C definitions of the int8 quantized-activation
 * ("q8ta") operations described by three ExecuTorch WebGPU pull-request pages:
 *   - "[WebGPU] Add quantize_per_tensor op (int8 buffer path)" (#21187),
 *     commit message / Solution + Implementation sections;
 *   - "[WebGPU] Add q8ta_linear op (int8 quantized linear)" (#21197),
 *     Solution and Constraints sections;
 *   - "[WebGPU] Add q8ta_conv2d_transposed op (int8 transposed conv)" (#21205),
 *     Solution, Implementation and Constraints sections (and the forward
 *     q8ta_conv2d whose scaffold that page says the transposed op reuses).
 *
 * Only tests, the smoke check and the benchmark's CPU-baseline leg load this
 * library.  It shares no code, header or constant with the GPU library.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -shared -fPIC
 * (no FMA contraction; x86-64 SSE float arithmetic, round-to-nearest-even).
 *
 * Conventions fixed here where the pages leave a step open:
 *   - "round" is round-half-to-even (nearbyintf under the default rounding mode);
 *   - every scale crosses the interface as a double; the quantize reciprocal is
 *     taken in double and cast once to float; the input scale used by the
 *     epilogue is the double cast once to float;
 *   - the dequant/requant epilogue is evaluated left to right in float, one
 *     rounding per operation: ((float(acc) * s_in) * w_scale[c]) + bias[c],
 *     then * inv_out, round, + zero_point, clamp to [-128, 127];
 *   - a NULL bias means no bias term;
 *   - the relu-fused activation (a follow-up the pages keep fail-loud) is
 *     max(v, 0) on the real-valued output v, before it is requantized;
 *   - dequantize is float(q - zp) * float(scale).
 * Integer sums are formed in int64 and each result is checked to fit int32;
 * the functions return a non-zero code if not (or on a bad argument).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_OVERFLOW 2

/* ---- quantize_per_tensor (#21187, Solution / Implementation) -------------
 * q = clamp(round(x * inv_scale) + zero_point, -128, 127) with
 * inv_scale = float(1.0 / scale) computed in double. */
int oracle_quantize_per_tensor(const float* x, int8_t* out, int64_t numel,
                               double scale, int64_t zero_point) {
  if (numel < 0 || (numel > 0 && (!x || !out))) return ORACLE_BAD_ARG;
  const float inv_scale = (float)(1.0 / scale);
  const float zp = (float)zero_point;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < numel; ++i) {
    float t = x[i] * inv_scale;
    float r = nearbyintf(t);
    float u = r + zp;
    if (u < -128.0f) u = -128.0f;
    if (u > 127.0f) u = 127.0f;
    out[i] = (int8_t)u;
  }
  return ORACLE_OK;
}

/* ---- dequantize_per_tensor (the "landed C0 op" named by #21197/#21205,
 * Problem section; the pages do not print it, this is the decomposed
 * definition (q - zp) * scale evaluated in float). */
int oracle_dequantize_per_tensor(const int8_t* q, float* out, int64_t numel,
                                 double scale, int64_t zero_point) {
  if (numel < 0 || (numel > 0 && (!q || !out))) return ORACLE_BAD_ARG;
  const float s = (float)scale;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < numel; ++i) {
    int d = (int)q[i] - (int)zero_point;
    out[i] = (float)d * s;
  }
  return ORACLE_OK;
}

/* ---- per-channel dequant + requant epilogue (#21197 and #21205, Solution):
 * v = acc * input_scale * weight_scales[c] + bias[c];
 * q = clamp(round(v * inv_output_scale) + output_zero_point, -128, 127).
 * The element at flat index e belongs to channel (e / inner) % channels.
 * pre (optional) receives v, the value just before the requantize multiply.
 * relu != 0 is the relu-fused activation, which the pages leave as a fail-loud
 * follow-up (#21197 Implementation and Constraints, #21205 Constraints): the
 * rectifier acts on the real-valued output, v = max(v, 0), before it is
 * requantized. */
int oracle_epilogue(const int32_t* acc, int64_t numel, int64_t channels,
                    int64_t inner, double input_scale,
                    const float* weight_scales, const float* bias,
                    double output_scale, int64_t output_zero_point,
                    int64_t relu, int8_t* out, float* pre) {
  if (numel < 0 || channels <= 0 || inner <= 0) return ORACLE_BAD_ARG;
  if (numel > 0 && (!acc || !out || !weight_scales)) return ORACLE_BAD_ARG;
  const float s_in = (float)input_scale;
  const float inv_out = (float)(1.0 / output_scale);
  const float ozp = (float)output_zero_point;
#pragma omp parallel for schedule(static)
  for (int64_t e = 0; e < numel; ++e) {
    int64_t c = (e / inner) % channels;
    float v = (float)acc[e];
    v = v * s_in;
    v = v * weight_scales[c];
    if (bias) v = v + bias[c];
    if (pre) pre[e] = v;
    if (relu && v < 0.0f) v = 0.0f;
    float t = v * inv_out;
    float r = nearbyintf(t);
    float u = r + ozp;
    if (u < -128.0f) u = -128.0f;
    if (u > 127.0f) u = 127.0f;
    out[e] = (int8_t)u;
  }
  return ORACLE_OK;
}

/* ---- q8ta_linear contraction (#21197, Solution):
 * acc[m, n] = sum_k (x[m, k] - input_zero_point) * w[n, k],
 * x row-major [M, K], w row-major [N, ldw] with ldw >= K (#21197 Constraints). */
int oracle_linear_acc(const int8_t* x, int64_t M, int64_t K,
                      int64_t input_zero_point, const int8_t* w, int64_t N,
                      int64_t ldw, int32_t* acc) {
  if (M < 0 || N < 0 || K < 0 || ldw < K) return ORACLE_BAD_ARG;
  int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      int64_t s = 0;
      for (int64_t k = 0; k < K; ++k)
        s += ((int64_t)x[m * K + k] - input_zero_point) * (int64_t)w[n * ldw + k];
      if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
      acc[m * N + n] = (int32_t)s;
    }
  }
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* Folded form of the same sum (#21197 and #21205, Constraints (1)):
 * sum_k x*w - zp * sum_k w.  Used only to check the identity. */
int oracle_linear_acc_folded(const int8_t* x, int64_t M, int64_t K,
                             int64_t input_zero_point, const int8_t* w,
                             int64_t N, int64_t ldw, int32_t* acc) {
  if (M < 0 || N < 0 || K < 0 || ldw < K) return ORACLE_BAD_ARG;
  int overflow = 0;
#pragma omp parallel for schedule(static) reduction(| : overflow)
  for (int64_t m = 0; m < M; ++m) {
    for (int64_t n = 0; n < N; ++n) {
      int64_t xw = 0, ws = 0;
      for (int64_t k = 0; k < K; ++k) {
        xw += (int64_t)x[m * K + k] * (int64_t)w[n * ldw + k];
        ws += (int64_t)w[n * ldw + k];
      }
      int64_t s = xw - input_zero_point * ws;
      if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
      acc[m * N + n] = (int32_t)s;
    }
  }
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* Full q8ta_linear: contraction then epilogue, channel = n. */
int oracle_linear(const int8_t* x, int64_t M, int64_t K, double input_scale,
                  int64_t input_zero_point, const int8_t* w, int64_t N,
                  int64_t ldw, const float* weight_scales, const float* bias,
                  double output_scale, int64_t output_zero_point, int64_t relu,
                  int8_t* out, int32_t* acc_out) {
  if (M < 0 || N <= 0 || K < 0) return ORACLE_BAD_ARG;
  int32_t* acc = acc_out ? acc_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * N + 1));
  if (!acc) return ORACLE_BAD_ARG;
  int rc = oracle_linear_acc(x, M, K, input_zero_point, w, N, ldw, acc);
  if (rc == ORACLE_OK)
    rc = oracle_epilogue(acc, M * N, N, 1, input_scale, weight_scales, bias,
                         output_scale, output_zero_point, relu, out, NULL);
  if (!acc_out) free(acc);
  return rc;
}

/* ---- q8ta_conv2d_transposed gather (#21205, Solution):
 * acc[n, oc, oh, ow] = sum over (ic, kh, kw) of
 *     (x[n, ic, ih, iw] - input_zero_point) * w[oc, (kh*Kw + kw)*IC + ic]
 * where ih = (oh + pad_h - kh*dil_h) / stride_h is used only when that
 * numerator is >= 0, divisible by stride_h and ih < H_in (iw likewise).
 * x is NCHW [N, IC, H_in, W_in]; w is [OC, ldw], ldw >= Kh*Kw*IC
 * (#21205 Implementation: the row stride tolerates padding); acc is NCHW
 * [N, OC, H_out, W_out] with H_out/W_out given by the caller.
 * Dilation and groups are the pages' fail-loud follow-ups (#21205
 * Implementation and Constraints); dil_h enters the numerator as printed.
 * Groups (not on the pages) split IC and OC into `groups` equal groups as in
 * the forward conv below: output channel oc of group g = oc / (OC/groups) sums
 * over ic = g*(IC/groups) + icg only, with w[oc, (kh*Kw + kw)*(IC/groups) + icg]
 * (the reshape of #21205 Constraints (2) applied to each group's
 * [IC/groups, OC/groups, Kh, Kw] block of the original weight). */
static int tap_index(int64_t o, int64_t pad, int64_t k, int64_t dil,
                     int64_t stride, int64_t in_size, int64_t* i_out) {
  int64_t num = o + pad - k * dil;
  if (num < 0) return 0;            /* checked before dividing */
  if (num % stride != 0) return 0;
  int64_t i = num / stride;
  if (i >= in_size) return 0;
  *i_out = i;
  return 1;
}

static int groups_ok(int64_t IC, int64_t OC, int64_t groups) {
  return groups >= 1 && IC > 0 && OC > 0 && IC % groups == 0 && OC % groups == 0;
}

int oracle_deconv_acc_gather(const int8_t* x, int64_t N, int64_t IC,
                             int64_t H_in, int64_t W_in,
                             int64_t input_zero_point, const int8_t* w,
                             int64_t OC, int64_t Kh, int64_t Kw, int64_t ldw,
                             int64_t stride_h, int64_t stride_w, int64_t pad_h,
                             int64_t pad_w, int64_t dil_h, int64_t dil_w,
                             int64_t groups, int64_t H_out, int64_t W_out,
                             int32_t* acc) {
  if (!groups_ok(IC, OC, groups)) return ORACLE_BAD_ARG;
  const int64_t ICg = IC / groups, OCg = OC / groups;
  if (N < 0 || Kh <= 0 || Kw <= 0 || ldw < Kh * Kw * ICg ||
      stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || H_out < 0 || W_out < 0)
    return ORACLE_BAD_ARG;
  int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t oc = 0; oc < OC; ++oc) {
      for (int64_t oh = 0; oh < H_out; ++oh) {
        for (int64_t ow = 0; ow < W_out; ++ow) {
          int64_t s = 0;
          const int64_t g = oc / OCg;
          for (int64_t icg = 0; icg < ICg; ++icg) {
            const int64_t ic = g * ICg + icg;
            for (int64_t kh = 0; kh < Kh; ++kh) {
              int64_t ih;
              if (!tap_index(oh, pad_h, kh, dil_h, stride_h, H_in, &ih)) continue;
              for (int64_t kw = 0; kw < Kw; ++kw) {
                int64_t iw;
                if (!tap_index(ow, pad_w, kw, dil_w, stride_w, W_in, &iw)) continue;
                int64_t xv = x[((n * IC + ic) * H_in + ih) * W_in + iw];
                int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];
                s += (xv - input_zero_point) * wv;
              }
            }
          }
          if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
          acc[((n * OC + oc) * H_out + oh) * W_out + ow] = (int32_t)s;
        }
      }
    }
  }
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* Scatter formulation of the same sum, used only as a self-check: every input
 * pixel (ih, iw) and tap (kh, kw) contributes to oh = ih*stride_h - pad_h +
 * kh*dil_h (ow likewise) when that lands inside the output. */
int oracle_deconv_acc_scatter(const int8_t* x, int64_t N, int64_t IC,
                              int64_t H_in, int64_t W_in,
                              int64_t input_zero_point, const int8_t* w,
                              int64_t OC, int64_t Kh, int64_t Kw, int64_t ldw,
                              int64_t stride_h, int64_t stride_w, int64_t pad_h,
                              int64_t pad_w, int64_t dil_h, int64_t dil_w,
                              int64_t groups, int64_t H_out, int64_t W_out,
                              int32_t* acc) {
  if (!groups_ok(IC, OC, groups)) return ORACLE_BAD_ARG;
  const int64_t ICg = IC / groups, OCg = OC / groups;
  if (N < 0 || Kh <= 0 || Kw <= 0 || ldw < Kh * Kw * ICg ||
      stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || H_out < 0 || W_out < 0)
    return ORACLE_BAD_ARG;
  int64_t plane = H_out * W_out;
  int64_t total = N * OC * plane;
  int64_t* s = (int64_t*)calloc((size_t)(total + 1), sizeof(int64_t));
  if (!s) return ORACLE_BAD_ARG;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t ic = 0; ic < IC; ++ic)
      for (int64_t ih = 0; ih < H_in; ++ih)
        for (int64_t iw = 0; iw < W_in; ++iw) {
          int64_t xv = (int64_t)x[((n * IC + ic) * H_in + ih) * W_in + iw] - input_zero_point;
          for (int64_t kh = 0; kh < Kh; ++kh) {
            int64_t oh = ih * stride_h - pad_h + kh * dil_h;
            if (oh < 0 || oh >= H_out) continue;
            for (int64_t kw = 0; kw < Kw; ++kw) {
              int64_t ow = iw * stride_w - pad_w + kw * dil_w;
              if (ow < 0 || ow >= W_out) continue;
              const int64_t g = ic / ICg, icg = ic % ICg;
              for (int64_t oc = g * OCg; oc < (g + 1) * OCg; ++oc)
                s[((n * OC + oc) * H_out + oh) * W_out + ow] +=
                    xv * (int64_t)w[oc * ldw + (kh * Kw + kw) * ICg + icg];
            }
          }
        }
  int overflow = 0;
  for (int64_t e = 0; e < total; ++e) {
    if (s[e] > INT32_MAX || s[e] < INT32_MIN) overflow = 1;
    acc[e] = (int32_t)s[e];
  }
  free(s);
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* Zero-point-fill formulation (#21205, Constraints (1)): every tap whose
 * numerator is divisible by the stride is summed; a tap that falls outside the
 * input reads the zero point, and sum(x*w) - zp*sum(w) runs over all those
 * taps.  Used only to check that it equals the gather. */
static int tap_divisible(int64_t o, int64_t pad, int64_t k, int64_t dil,
                         int64_t stride, int64_t* i_out) {
  int64_t num = o + pad - k * dil;
  int64_t r = num % stride;
  if (r != 0) return 0;             /* C remainder is 0 exactly when divisible */
  *i_out = num / stride;            /* exact, also for negative multiples */
  return 1;
}

int oracle_deconv_acc_zpfill(const int8_t* x, int64_t N, int64_t IC,
                             int64_t H_in, int64_t W_in,
                             int64_t input_zero_point, const int8_t* w,
                             int64_t OC, int64_t Kh, int64_t Kw, int64_t ldw,
                             int64_t stride_h, int64_t stride_w, int64_t pad_h,
                             int64_t pad_w, int64_t dil_h, int64_t dil_w,
                             int64_t groups, int64_t H_out, int64_t W_out,
                             int32_t* acc) {
  if (!groups_ok(IC, OC, groups)) return ORACLE_BAD_ARG;
  const int64_t ICg = IC / groups, OCg = OC / groups;
  if (N < 0 || Kh <= 0 || Kw <= 0 || ldw < Kh * Kw * ICg ||
      stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || H_out < 0 || W_out < 0)
    return ORACLE_BAD_ARG;
  int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t oc = 0; oc < OC; ++oc) {
      for (int64_t oh = 0; oh < H_out; ++oh) {
        for (int64_t ow = 0; ow < W_out; ++ow) {
          int64_t xw = 0, ws = 0;
          const int64_t g = oc / OCg;
          for (int64_t kh = 0; kh < Kh; ++kh) {
            int64_t ih;
            if (!tap_divisible(oh, pad_h, kh, dil_h, stride_h, &ih)) continue;
            for (int64_t kw = 0; kw < Kw; ++kw) {
              int64_t iw;
              if (!tap_divisible(ow, pad_w, kw, dil_w, stride_w, &iw)) continue;
              for (int64_t icg = 0; icg < ICg; ++icg) {
                const int64_t ic = g * ICg + icg;
                int64_t xv = input_zero_point;
                if (ih >= 0 && ih < H_in && iw >= 0 && iw < W_in)
                  xv = x[((n * IC + ic) * H_in + ih) * W_in + iw];
                int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];
                xw += xv * wv;
                ws += wv;
              }
            }
          }
          int64_t s = xw - input_zero_point * ws;
          if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
          acc[((n * OC + oc) * H_out + oh) * W_out + ow] = (int32_t)s;
        }
      }
    }
  }
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* Full q8ta_conv2d_transposed: gather contraction then epilogue, channel = oc. */
int oracle_conv2d_transposed(const int8_t* x, int64_t N, int64_t IC,
                             int64_t H_in, int64_t W_in, double input_scale,
                             int64_t input_zero_point, const int8_t* w,
                             int64_t OC, int64_t Kh, int64_t Kw, int64_t ldw,
                             const float* weight_scales, const float* bias,
                             double output_scale, int64_t output_zero_point,
                             int64_t stride_h, int64_t stride_w, int64_t pad_h,
                             int64_t pad_w, int64_t dil_h, int64_t dil_w,
                             int64_t groups, int64_t H_out, int64_t W_out,
                             int64_t relu, int8_t* out, int32_t* acc_out) {
  if (N < 0 || OC <= 0 || H_out < 0 || W_out < 0) return ORACLE_BAD_ARG;
  int64_t total = N * OC * H_out * W_out;
  int32_t* acc = acc_out ? acc_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)(total + 1));
  if (!acc) return ORACLE_BAD_ARG;
  int rc = oracle_deconv_acc_gather(x, N, IC, H_in, W_in, input_zero_point, w, OC,
                                    Kh, Kw, ldw, stride_h, stride_w, pad_h, pad_w,
                                    dil_h, dil_w, groups, H_out, W_out, acc);
  if (rc == ORACLE_OK && total > 0)
    rc = oracle_epilogue(acc, total, OC, H_out * W_out, input_scale, weight_scales,
                         bias, output_scale, output_zero_point, relu, out, NULL);
  if (!acc_out) free(acc);
  return rc;
}

/* ---- forward q8ta_conv2d (the general int8 conv whose scaffold and
 * [OC, Kh*Kw*IC] weight layout the transposed op reuses, #21205 Solution; the
 * pages print only the transposed index relation, so the forward one is the
 * standard convolution index):
 * acc[n, oc, oh, ow] = sum over (ic, kh, kw) of
 *     (x[n, ic, ih, iw] - input_zero_point) * w[oc, (kh*Kw + kw)*IC + ic]
 * with ih = oh*stride_h - pad_h + kh*dil_h, used only when 0 <= ih < H_in
 * (iw likewise).  x is NCHW [N, IC, H_in, W_in]; w is [OC, ldw]; acc is NCHW
 * [N, OC, H_out, W_out] int32.
 * Groups (not on the pages; the usual grouped convolution on the same layout):
 * the channels split into `groups` equal groups, output channel oc belongs to
 * group g = oc / (OC/groups) and sums only over the IC/groups input channels
 * ic = g*(IC/groups) + icg, with w[oc, (kh*Kw + kw)*(IC/groups) + icg].
 * groups == IC == OC is the depthwise convolution. */
int oracle_conv2d_acc(const int8_t* x, int64_t N, int64_t IC, int64_t H_in,
                      int64_t W_in, int64_t input_zero_point, const int8_t* w,
                      int64_t OC, int64_t Kh, int64_t Kw, int64_t ldw,
                      int64_t stride_h, int64_t stride_w, int64_t pad_h,
                      int64_t pad_w, int64_t dil_h, int64_t dil_w, int64_t groups,
                      int64_t H_out, int64_t W_out, int32_t* acc) {
  if (groups < 1 || IC % groups != 0 || OC % groups != 0) return ORACLE_BAD_ARG;
  const int64_t ICg = IC / groups, OCg = OC / groups;
  if (N < 0 || IC <= 0 || OC <= 0 || Kh <= 0 || Kw <= 0 || ldw < Kh * Kw * ICg ||
      stride_h < 1 || stride_w < 1 || dil_h < 1 || dil_w < 1 || H_out < 0 || W_out < 0)
    return ORACLE_BAD_ARG;
  int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t oc = 0; oc < OC; ++oc) {
      for (int64_t oh = 0; oh < H_out; ++oh) {
        for (int64_t ow = 0; ow < W_out; ++ow) {
          int64_t s = 0;
          const int64_t g = oc / OCg;
          for (int64_t icg = 0; icg < ICg; ++icg) {
            const int64_t ic = g * ICg + icg;
            for (int64_t kh = 0; kh < Kh; ++kh) {
              const int64_t ih = oh * stride_h - pad_h + kh * dil_h;
              if (ih < 0 || ih >= H_in) continue;
              for (int64_t kw = 0; kw < Kw; ++kw) {
                const int64_t iw = ow * stride_w - pad_w + kw * dil_w;
                if (iw < 0 || iw >= W_in) continue;
                int64_t xv = x[((n * IC + ic) * H_in + ih) * W_in + iw];
                int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];
                s += (xv - input_zero_point) * wv;
              }
            }
          }
          if (s > INT32_MAX || s < INT32_MIN) overflow = 1;
          acc[((n * OC + oc) * H_out + oh) * W_out + ow] = (int32_t)s;
        }
      }
    }
  }
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* Full q8ta_conv2d: contraction then the per-channel epilogue, channel = oc. */
int oracle_conv2d(const int8_t* x, int64_t N, int64_t IC, int64_t H_in,
                  int64_t W_in, double input_scale, int64_t input_zero_point,
                  const int8_t* w, int64_t OC, int64_t Kh, int64_t Kw, int64_t ldw,
                  const float* weight_scales, const float* bias, double output_scale,
                  int64_t output_zero_point, int64_t stride_h, int64_t stride_w,
                  int64_t pad_h, int64_t pad_w, int64_t dil_h, int64_t dil_w,
                  int64_t groups, int64_t H_out, int64_t W_out, int64_t relu,
                  int8_t* out, int32_t* acc_out) {
  if (N < 0 || OC <= 0 || H_out < 0 || W_out < 0) return ORACLE_BAD_ARG;
  int64_t total = N * OC * H_out * W_out;
  int32_t* acc = acc_out ? acc_out : (int32_t*)malloc(sizeof(int32_t) * (size_t)(total + 1));
  if (!acc) return ORACLE_BAD_ARG;
  int rc = oracle_conv2d_acc(x, N, IC, H_in, W_in, input_zero_point, w, OC, Kh, Kw, ldw,
                             stride_h, stride_w, pad_h, pad_w, dil_h, dil_w, groups, H_out,
                             W_out, acc);
  if (rc == ORACLE_OK && total > 0)
    rc = oracle_epilogue(acc, total, OC, H_out * W_out, input_scale, weight_scales, bias,
                         output_scale, output_zero_point, relu, out, NULL);
  if (!acc_out) free(acc);
  return rc;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
