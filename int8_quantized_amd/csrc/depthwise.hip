// Depthwise q8ta_conv2d (groups == IC == OC): output channel c convolves only
// its own input plane, acc[n,c,oh,ow] = sum over (kh, kw) of
// (x[n,c,ih,iw] - izp) * w[c, kh*Kw + kw], ih = oh*stride_h - pad_h +
// kh*dil_h used only inside the input (iw likewise) -- the forward conv of the
// transposed-conv page's scaffold with one input channel per group.
//
// A reduction over Kh*Kw taps only: the op moves each input and output byte
// about once and is bound by HBM.  Blocks work on one (n, c) plane
// (blockIdx.y), so the channel's weights, scale and bias are wave-uniform and
// come through the scalar unit.  For square K x K kernels with K in {3, 5},
// stride 1 or 2 and no dilation, a thread computes a 4 x 4 patch of outputs
// from the input window it needs ((4-1)*S + K rows and columns, loaded once
// into registers with the zero point subtracted and out-of-range pixels set to
// 0), so each input byte is loaded about (1 + (K-S)/4)^2 times instead of K*K.
// Other shapes take a thread per 4 consecutive outputs of one row.
#include "q8ta_internal.h"

namespace q8ta {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxTaps = 64;   // Kh*Kw taken by this kernel

typedef const __attribute__((address_space(4))) int8_t* cbptr;

__global__ __launch_bounds__(kThreads) void k_depthwise(DeconvArgs a) {
  const int64_t plane_id = blockIdx.y;  // n * C + c
  const int64_t c = plane_id % a.OC;
  const int QW = (int)((a.W_out + 3) / 4);
  const int64_t item = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (item >= a.H_out * QW) return;
  const int64_t oh = item / QW;
  const int64_t ow0 = (item % QW) * 4;
  const int8_t* xp = a.x + plane_id * a.H_in * a.W_in;
  const cbptr wc = (cbptr)(a.w + c * a.ldw);  // wave-uniform weights
  int32_t acc[4] = {0, 0, 0, 0};
  for (int kh = 0; kh < (int)a.Kh; ++kh) {
    const int64_t ih = oh * a.sh - a.ph + kh * a.dil_h;
    if (ih < 0 || ih >= a.H_in) continue;
    const int8_t* row = xp + ih * a.W_in;
    for (int kw = 0; kw < (int)a.Kw; ++kw) {
      const int32_t wv = wc[kh * a.Kw + kw];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t iw = (ow0 + q) * a.sw - a.pw + kw * a.dil_w;
        if (iw >= 0 && iw < a.W_in && ow0 + q < a.W_out)
          acc[q] += ((int32_t)row[iw] - a.izp) * wv;
      }
    }
  }
  const int64_t o = (plane_id * a.H_out + oh) * a.W_out + ow0;
  if (a.acc) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ow0 + q < a.W_out) a.acc[o + q] = acc[q];
    return;
  }
  const float sc = a.wscale[c];
  const float bv = a.bias ? a.bias[c] : 0.0f;
  int r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) r[q] = requant(acc[q], sc, bv, a.rq);
  int8_t* op = a.out + o;
  if (ow0 + 3 < a.W_out && ((uintptr_t)op & 3) == 0) {
    *reinterpret_cast<uint32_t*>(op) = pack4(r[0], r[1], r[2], r[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (ow0 + q < a.W_out) op[q] = (int8_t)r[q];
  }
}

// DW: rows are read as 32-bit words (W_in % 4 == 0 and 4-byte aligned input).
template <int K, int S, bool DW>
__global__ __launch_bounds__(kThreads) void k_depthwise_patch(DeconvArgs a) {
  constexpr int P = 4;                   // outputs per patch side
  constexpr int WN = (P - 1) * S + K;    // input window side
  const int64_t plane_id = blockIdx.y;   // n * C + c
  const int64_t c = (int)blockIdx.y % (int)a.OC;
  const int H_in = (int)a.H_in, W_in = (int)a.W_in, H_out = (int)a.H_out, W_out = (int)a.W_out;
  const int QW = (W_out + P - 1) / P, QH = (H_out + P - 1) / P;
  const int item = blockIdx.x * kThreads + threadIdx.x;
  if (item >= QH * QW) return;
  const int oh0 = (item / QW) * P, ow0 = (item % QW) * P;
  const int ih0 = oh0 * S - (int)a.ph, iw0 = ow0 * S - (int)a.pw;
  const int8_t* xp = a.x + plane_id * (int64_t)H_in * W_in;
  const int izp = a.izp;
  int win[WN][WN];  // x - izp inside the input, 0 outside
  bool cok[WN];
#pragma unroll
  for (int q = 0; q < WN; ++q) cok[q] = iw0 + q >= 0 && iw0 + q < W_in;
  if constexpr (DW) {
    // Rows as 32-bit words (W_in % 4 == 0, 4-byte aligned planes): the window
    // starts `shift` bytes into word dq0 (shift is the same for every thread:
    // iw0 = ow0*S - pad_w with ow0*S a multiple of 4); ND clamped word loads
    // per row, realigned with v_alignbyte, then one signed byte per column.
    constexpr int ND = (WN + 3) / 4 + 1;
    const int shift = (4 - ((int)a.pw & 3)) & 3;
    const int dq0 = (iw0 - shift) / 4;
    const int nwords = W_in / 4;
#pragma unroll
    for (int r = 0; r < WN; ++r) {
      const int ih = ih0 + r;
      const bool rok = ih >= 0 && ih < H_in;
      const uint32_t* row = reinterpret_cast<const uint32_t*>(
          xp + (int64_t)(ih < 0 ? 0 : (ih >= H_in ? H_in - 1 : ih)) * W_in);
      uint32_t d[ND];
#pragma unroll
      for (int k = 0; k < ND; ++k) {
        const int dk = dq0 + k;
        d[k] = row[dk < 0 ? 0 : (dk >= nwords ? nwords - 1 : dk)];
        asm volatile("" : "+v"(d[k]));  // unconditional load (no branch around it)
      }
      uint32_t e[ND - 1];
#pragma unroll
      for (int k = 0; k < ND - 1; ++k) e[k] = __builtin_amdgcn_alignbyte(d[k + 1], d[k], shift);
#pragma unroll
      for (int q = 0; q < WN; ++q) {
        const int v = (int)(int8_t)(e[q / 4] >> (8 * (q % 4))) - izp;
        win[r][q] = v & -(int)(rok && cok[q]);  // arithmetic select, no branch
      }
    }
  } else {
    // Byte loads from clamped, in-range addresses (no branch around them); the
    // select afterwards zeroes the pixels outside the input.
    int iwc[WN];
#pragma unroll
    for (int q = 0; q < WN; ++q) {
      const int iw = iw0 + q;
      iwc[q] = iw < 0 ? 0 : (iw >= W_in ? W_in - 1 : iw);
    }
#pragma unroll
    for (int r = 0; r < WN; ++r) {
      const int ih = ih0 + r;
      const bool rok = ih >= 0 && ih < H_in;
      const int8_t* row = xp + (int64_t)(ih < 0 ? 0 : (ih >= H_in ? H_in - 1 : ih)) * W_in;
#pragma unroll
      for (int q = 0; q < WN; ++q) {
        int v = (int)row[iwc[q]] - izp;
        asm volatile("" : "+v"(v));  // keep the load unconditional (no branch around it)
        win[r][q] = (rok && cok[q]) ? v : 0;
      }
    }
  }
  const cbptr wc = (cbptr)(a.w + c * a.ldw);
  int wv[K * K];
#pragma unroll
  for (int t = 0; t < K * K; ++t) wv[t] = wc[t];
  int32_t acc[P][P];
#pragma unroll
  for (int r = 0; r < P; ++r)
#pragma unroll
    for (int q = 0; q < P; ++q) {
      int32_t s = 0;
#pragma unroll
      for (int kh = 0; kh < K; ++kh)
#pragma unroll
        for (int kw = 0; kw < K; ++kw)  // |x - izp| <= 255, |w| <= 128: a 24-bit product
          s += __mul24(win[r * S + kh][q * S + kw], wv[kh * K + kw]);
      acc[r][q] = s;
    }
  const float sc = a.acc ? 0.0f : a.wscale[c];
  const float bv = (!a.acc && a.bias) ? a.bias[c] : 0.0f;
#pragma unroll
  for (int r = 0; r < P; ++r) {
    const int oh = oh0 + r;
    if (oh >= H_out) break;
    const int64_t o = (plane_id * H_out + oh) * (int64_t)W_out + ow0;
    if (a.acc) {
#pragma unroll
      for (int q = 0; q < P; ++q)
        if (ow0 + q < W_out) a.acc[o + q] = acc[r][q];
      continue;
    }
    int v[P];
#pragma unroll
    for (int q = 0; q < P; ++q) v[q] = requant(acc[r][q], sc, bv, a.rq);
    int8_t* op = a.out + o;
    if (ow0 + 3 < W_out && ((uintptr_t)op & 3) == 0) {
      *reinterpret_cast<uint32_t*>(op) = pack4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int q = 0; q < P; ++q)
        if (ow0 + q < W_out) op[q] = (int8_t)v[q];
    }
  }
}

template <int K, int S>
hipError_t launch_patch(const DeconvArgs& a, hipStream_t s) {
  const int64_t items = ((a.H_out + 3) / 4) * ((a.W_out + 3) / 4);
  const dim3 grid((unsigned)((items + kThreads - 1) / kThreads), (unsigned)(a.N * a.OC));
  const bool dw = a.W_in % 4 == 0 && ((uintptr_t)a.x & 3) == 0;
  if (dw)
    hipLaunchKernelGGL((k_depthwise_patch<K, S, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_depthwise_patch<K, S, false>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool depthwise_supported(const DeconvArgs& a) {
  const int64_t QW = (a.W_out + 3) / 4;
  return a.groups == a.IC && a.IC == a.OC && a.Kh * a.Kw <= kMaxTaps &&
         (a.H_out * QW + kThreads - 1) / kThreads < ((int64_t)1 << 31) &&
         a.N * a.OC < 65536;
}

hipError_t launch_depthwise(const DeconvArgs& a, hipStream_t s) {
  if (a.Kh == a.Kw && a.sh == a.sw && a.dil_h == 1 && a.dil_w == 1 && a.H_in < (1 << 24) &&
      a.W_in < (1 << 24) && a.H_out < (1 << 14) && a.W_out < (1 << 14)) {
    if (a.Kh == 3 && a.sh == 1) return launch_patch<3, 1>(a, s);
    if (a.Kh == 3 && a.sh == 2) return launch_patch<3, 2>(a, s);
    if (a.Kh == 5 && a.sh == 1) return launch_patch<5, 1>(a, s);
    if (a.Kh == 5 && a.sh == 2) return launch_patch<5, 2>(a, s);
  }
  const int64_t QW = (a.W_out + 3) / 4;
  const dim3 grid((unsigned)((a.H_out * QW + kThreads - 1) / kThreads), (unsigned)(a.N * a.OC));
  hipLaunchKernelGGL(k_depthwise, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace q8ta
