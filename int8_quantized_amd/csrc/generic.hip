// Shape-general kernels: any sizes, any alignment.  They serve the shapes the
// tiled kernels do not take (reduction lengths that are not a multiple of 16
// bytes, unaligned pointers, tap sets that do not fit the staged tile) and
// evaluate the definitions directly, one output element per thread.
#include "q8ta_internal.h"

namespace q8ta {
namespace {

constexpr int kThreads = 256;

// "Add q8ta_linear op", Solution: acc = sum_k (x[m,k] - izp) * w[n,k].
__global__ __launch_bounds__(kThreads) void k_linear_generic(LinearArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= a.M * a.N) return;
  const int64_t m = idx / a.N, n = idx % a.N;
  const int8_t* xr = a.x + m * a.K;
  const int8_t* wr = a.w + n * a.K;
  int32_t acc = 0;
  for (int64_t k = 0; k < a.K; ++k) acc += ((int32_t)xr[k] - a.izp) * (int32_t)wr[k];
  if (a.acc) {
    a.acc[idx] = acc;
  } else {
    float b = a.bias ? a.bias[n] : 0.0f;
    const int q = requant(acc, a.wscale[n], b, a.rq);
    if (a.outf)
      a.outf[idx] = dequant1(q, a.dq_zp, a.dq_scale);
    else
      a.out[idx] = (int8_t)q;
  }
}

// "Add q8ta_conv2d_transposed op", Solution: the gather
//   ih = (oh + pad_h - kh*dil_h) / stride_h, used only when the numerator is
//   >= 0, divisible and ih < H_in (iw likewise).  With groups, output channel
//   oc sums over the IC/groups input channels of its group, weight row
//   w[oc, (kh*Kw + kw)*(IC/groups) + icg].
__global__ __launch_bounds__(kThreads) void k_deconv_generic(DeconvArgs a) {
  const int64_t total = a.N * a.OC * a.H_out * a.W_out;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total) return;
  const int64_t ow = idx % a.W_out;
  const int64_t oh = (idx / a.W_out) % a.H_out;
  const int64_t oc = (idx / (a.W_out * a.H_out)) % a.OC;
  const int64_t n = idx / (a.W_out * a.H_out * a.OC);
  const int64_t ICg = a.IC / a.groups, OCg = a.OC / a.groups;
  const int64_t ic0 = (oc / OCg) * ICg;  // first input channel of oc's group
  const int64_t plane = a.H_in * a.W_in;
  int32_t acc = 0;
  for (int64_t kh = 0; kh < a.Kh; ++kh) {
    const int64_t nh = oh + a.ph - kh * a.dil_h;
    if (nh < 0 || nh % a.sh != 0) continue;
    const int64_t ih = nh / a.sh;
    if (ih >= a.H_in) continue;
    for (int64_t kw = 0; kw < a.Kw; ++kw) {
      const int64_t nw = ow + a.pw - kw * a.dil_w;
      if (nw < 0 || nw % a.sw != 0) continue;
      const int64_t iw = nw / a.sw;
      if (iw >= a.W_in) continue;
      const int8_t* xp = a.x + ((n * a.IC + ic0) * a.H_in + ih) * a.W_in + iw;
      const int8_t* wp = a.w + oc * a.ldw + (kh * a.Kw + kw) * ICg;
      for (int64_t icg = 0; icg < ICg; ++icg)
        acc += ((int32_t)xp[icg * plane] - a.izp) * (int32_t)wp[icg];
    }
  }
  if (a.acc) {
    a.acc[idx] = acc;
  } else {
    float b = a.bias ? a.bias[oc] : 0.0f;
    a.out[idx] = (int8_t)requant(acc, a.wscale[oc], b, a.rq);
  }
}

// Forward q8ta_conv2d, one output per thread: ih = oh*stride_h - pad_h +
// kh*dil_h, taps outside the input skipped; with groups, output channel oc
// sums over the IC/groups input channels of its group.
__global__ __launch_bounds__(kThreads) void k_conv2d_generic(DeconvArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = a.N * a.OC * a.H_out * a.W_out;
  if (idx >= total) return;
  const int64_t ow = idx % a.W_out;
  int64_t r = idx / a.W_out;
  const int64_t oh = r % a.H_out;
  r /= a.H_out;
  const int64_t oc = r % a.OC;
  const int64_t n = r / a.OC;
  const int64_t plane = a.H_in * a.W_in;
  const int64_t ICg = a.IC / a.groups, OCg = a.OC / a.groups;
  const int64_t ic0 = (oc / OCg) * ICg;  // first input channel of oc's group
  int32_t acc = 0;
  for (int64_t kh = 0; kh < a.Kh; ++kh) {
    const int64_t ih = oh * a.sh - a.ph + kh * a.dil_h;
    if (ih < 0 || ih >= a.H_in) continue;
    for (int64_t kw = 0; kw < a.Kw; ++kw) {
      const int64_t iw = ow * a.sw - a.pw + kw * a.dil_w;
      if (iw < 0 || iw >= a.W_in) continue;
      const int8_t* xp = a.x + ((n * a.IC + ic0) * a.H_in + ih) * a.W_in + iw;
      const int8_t* wp = a.w + oc * a.ldw + (kh * a.Kw + kw) * ICg;
      for (int64_t ic = 0; ic < ICg; ++ic)
        acc += ((int32_t)xp[ic * plane] - a.izp) * (int32_t)wp[ic];
    }
  }
  if (a.acc) {
    a.acc[idx] = acc;
  } else {
    float b = a.bias ? a.bias[oc] : 0.0f;
    a.out[idx] = (int8_t)requant(acc, a.wscale[oc], b, a.rq);
  }
}

}  // namespace

hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t s) {
  int64_t total = a.M * a.N;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_linear_generic, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// sum_k w[n, k] for any K and alignment: one thread per row.
__global__ __launch_bounds__(kThreads) void k_row_sums_generic(const int8_t* w, int64_t N, int64_t K,
                                                               int64_t ldw, int32_t* out) {
  const int64_t n = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (n >= N) return;
  const int8_t* r = w + n * ldw;
  int32_t s = 0;
  for (int64_t k = 0; k < K; ++k) s += r[k];
  out[n] = s;
}

hipError_t launch_row_sums_generic(const int8_t* w, int64_t N, int64_t K, int64_t ldw, int32_t* out,
                                   hipStream_t s) {
  hipLaunchKernelGGL(k_row_sums_generic, dim3((unsigned)((N + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, w, N, K, ldw, out);
  return hipGetLastError();
}

hipError_t launch_deconv_generic(const DeconvArgs& a, hipStream_t s) {
  int64_t total = a.N * a.OC * a.H_out * a.W_out;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_deconv_generic, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_conv2d_generic(const DeconvArgs& a, hipStream_t s) {
  int64_t total = a.N * a.OC * a.H_out * a.W_out;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_conv2d_generic, dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace q8ta
