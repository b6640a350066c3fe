// q8ta_conv2d_transposed on the vector ALU ("Add q8ta_conv2d_transposed op",
// Solution: acc[n,oc,oh,ow] = sum over (ic, kh, kw) of (x[n,ic,ih,iw] - izp) *
// w[oc, (kh*Kw + kw)*IC + ic], with ih = (oh + pad_h - kh) / stride_h used only
// when the numerator is >= 0, divisible and ih < H_in; iw likewise).
//
// Stride phases: which taps qualify depends only on rh = oh mod s_h and
// rw = ow mod s_w.  For oh = rh + s_h*i a qualifying tap kh reads row
// ih = i + dh with dh = (rh + pad_h - kh) / s_h (exact), and likewise for
// columns, so a fixed (rh, rw) is a dense stride-1 correlation with its own
// sub-kernel and no product with a non-qualifying tap is ever formed.
//
// A wave owns one image, one row residue rh with RQ consecutive phase rows
// (output rows oh = rh + s_h*i), one column residue rw, 64 phase columns j
// (one per lane: ow = rw + s_w*j) and OCB output channels; all its lanes share
// the same taps.  The input is first relaid out into blocks of 16 channels per
// pixel (k_nchw_to_blocked16); per tap and 16 input channels a lane then loads,
// for each of its RQ rows, the 16 bytes x[n, ic..ic+15, ih, iw] in one 16-byte
// load and accumulates v_dot4 against the weights w[oc, tap, ic..ic+15], which are the
// same for all lanes, come through the scalar unit and are reused RQ times.  A tap that falls outside the input
// reads the zero point, so with sum w taken over all of the phase's taps the
// result sum x*w - izp * sum w equals the gather (the zero-point-filled form of
// the page's Constraints (1)).  sum w per output channel is formed once per
// wave, the lanes splitting the (tap, channel) range, then reduced across the
// wave.  The epilogue requantizes in registers and stores bytes.
#include <cstdlib>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

constexpr int kThreads = 256;

// Weights are only read by these kernels: reading them through the constant
// address space lets the compiler fetch wave-uniform words with scalar loads.
typedef const __attribute__((address_space(4))) int32_t* cwptr;

// Input relayout for the blocked path: x NCHW -> xb[n][h][g][w][16] with
// g = ic / 16 (channels past IC are zero).  One thread per (n, h, g, w): it
// reads the 16 channel bytes of its pixel (each load instruction reads 64
// consecutive columns of one channel plane) and writes them as one 16-byte
// chunk (consecutive threads write consecutive chunks).
__global__ __launch_bounds__(kThreads) void k_nchw_to_blocked16(const int8_t* __restrict__ x,
                                                               int8_t* __restrict__ xb,
                                                               int64_t N, int IC, int H, int W,
                                                               int G) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = N * H * G * (int64_t)W;
  if (t >= total) return;
  const int w = (int)(t % W);
  int64_t r = t / W;
  const int g = (int)(r % G);
  r /= G;
  const int h = (int)(r % H);
  const int64_t n = r / H;
  const int64_t plane = (int64_t)H * W;
  const int8_t* src = x + (n * IC + 16 * g) * plane + (int64_t)h * W + w;
  uint32_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t d = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * g + 4 * q + e;
      const uint32_t by = c < IC ? (uint32_t)(uint8_t)src[(int64_t)(4 * q + e) * plane] : 0u;
      d |= by << (8 * e);
    }
    v[q] = d;
  }
  typedef int v4i __attribute__((ext_vector_type(4)));
  *reinterpret_cast<v4i*>(xb + t * 16) = v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
}

// Main kernel: the wave layout above with RQ phase rows per wave; the 16
// channels of a pixel come in one 16-byte load from xb (lanes read
// consecutive 16-byte chunks).  The inner loop is
// branch-free: weight rows past OC are clamped to OC - 1 (their results are
// never stored), the OCB weight quads of a 16-channel group are requested
// together through the scalar unit, and the next group's activations are
// loaded while the current one is multiplied.  ICF: IC is a multiple of 16,
// so no weight needs masking.
template <int OCB, bool ICF, int RQ>
__global__ __launch_bounds__(kThreads) void k_deconv_dot4_blocked(DeconvArgs a, Phases p,
                                                                 const int8_t* __restrict__ xb) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + wave;
  const int ob = (int)(wid % p.ocb);  wid /= p.ocb;
  const int jb = (int)(wid % p.jb);   wid /= p.jb;
  const int sw = (int)a.sw, sh = (int)a.sh;
  const int rw = (int)(wid % sw);     wid /= sw;
  const int ib = (int)(wid % p.ib);   wid /= p.ib;
  const int rh = (int)(wid % sh);     wid /= sh;
  const int64_t n = wid;
  if (n >= a.N) return;
  const int i0 = ib * RQ;               // phase rows i0 .. i0+RQ-1: output rows rh + sh*i
  const int j = jb * 64 + lane;
  const int ow = rw + sw * j;
  const int oc0 = ob * OCB;
  const int IC = (int)a.IC, H_in = (int)a.H_in, W_in = (int)a.W_in;
  const int G = (IC + 15) / 16;
  const int zp4 = (int)(0x01010101u * ((uint32_t)a.izp & 0xffu));
  const int nth = p.nth[rh], ntw = p.ntw[rw];
  const int64_t ldw4 = a.ldw / 4;
  int64_t wrow4[OCB];  // dword offset of each (clamped) weight row
#pragma unroll
  for (int o = 0; o < OCB; ++o) {
    const int oc = oc0 + o < a.OC ? oc0 + o : (int)a.OC - 1;
    wrow4[o] = (int64_t)oc * ldw4;
  }

  int32_t wsum[OCB];
#pragma unroll
  for (int o = 0; o < OCB; ++o) wsum[o] = 0;
  for (int th = 0; th < nth; ++th) {
    for (int tw = 0; tw < ntw; ++tw) {
      const int64_t tapoff = (int64_t)(p.thk[rh][th] * a.Kw + p.twk[rw][tw]) * IC;
      for (int ic = lane * 4; ic < IC; ic += 256) {
#pragma unroll
        for (int o = 0; o < OCB; ++o) {
          const int32_t wv = *reinterpret_cast<const int32_t*>(a.w + wrow4[o] * 4 + tapoff + ic);
          wsum[o] = __builtin_amdgcn_sdot4(wv, 0x01010101, wsum[o], false);
        }
      }
    }
  }
#pragma unroll
  for (int o = 0; o < OCB; ++o) wsum[o] = wave_total(wsum[o]);

  int32_t acc[RQ][OCB];
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int o = 0; o < OCB; ++o) acc[q][o] = 0;
  const int64_t gstride = (int64_t)W_in * 16;  // bytes between channel groups of a pixel row
  for (int th = 0; th < nth; ++th) {
    const int kh = p.thk[rh][th];
    const int dh = p.thd[rh][th];
    for (int tw = 0; tw < ntw; ++tw) {
      const int kw = p.twk[rw][tw];
      const int iw = j + p.twd[rw][tw];
      const bool col_ok = iw >= 0 && iw < W_in;
      const int8_t* xp[RQ];
      bool ok[RQ];
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        const int ih = i0 + q + dh;
        ok[q] = col_ok && ih >= 0 && ih < H_in;
        xp[q] = xb + (((n * H_in + (ok[q] ? ih : 0)) * G) * (int64_t)W_in + (ok[q] ? iw : 0)) * 16;
      }
      const cwptr wt = (cwptr)(a.w + (int64_t)(kh * a.Kw + kw) * IC);
      v4i xn[RQ];
#pragma unroll
      for (int q = 0; q < RQ; ++q) xn[q] = *reinterpret_cast<const v4i*>(xp[q]);
      for (int g = 0; g < G; ++g) {
        v4i xv[RQ];
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
          xv[q] = xn[q];
          if (g + 1 < G) xn[q] = *reinterpret_cast<const v4i*>(xp[q] + (int64_t)(g + 1) * gstride);
        }
        const int ic = 16 * g;
        int32_t wq[OCB][4];
#pragma unroll
        for (int o = 0; o < OCB; ++o)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            if constexpr (ICF) {
              wq[o][d] = wt[wrow4[o] + ic / 4 + d];
            } else {
              const bool in = ic + 4 * d < IC;
              const int32_t v = wt[wrow4[o] + (in ? ic / 4 + d : 0)];
              wq[o][d] = in ? v : 0;
            }
          }
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
          if (!ok[q]) {
            // zero-point fill of an out-of-image tap (channels past IC stay 0)
#pragma unroll
            for (int d = 0; d < 4; ++d) xv[q][d] = (ICF || ic + 4 * d < IC) ? zp4 : 0;
          }
        }
#pragma unroll
        for (int o = 0; o < OCB; ++o)
#pragma unroll
          for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int q = 0; q < RQ; ++q)
              acc[q][o] = __builtin_amdgcn_sdot4(xv[q][d], wq[o][d], acc[q][o], false);
      }
    }
  }
  if (ow >= a.W_out) return;
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const int oh = rh + sh * (i0 + q);
    if (oh >= a.H_out) break;
#pragma unroll
    for (int o = 0; o < OCB; ++o) {
      const int oc = oc0 + o;
      if (oc >= a.OC) break;
      const int32_t c = acc[q][o] - a.izp * wsum[o];
      const int64_t idx = (((int64_t)n * a.OC + oc) * a.H_out + oh) * a.W_out + ow;
      if (a.acc) {
        a.acc[idx] = c;
      } else {
        const float b = a.bias ? a.bias[oc] : 0.0f;
        a.out[idx] = (int8_t)requant(c, a.wscale[oc], b, a.rq);
      }
    }
  }
}

int floordiv(int x, int y) { return x >= 0 ? x / y : -((-x + y - 1) / y); }

}  // namespace

bool make_phases(const DeconvArgs& a, Phases& p) {
  if (a.sh > kMaxS || a.sw > kMaxS || a.ph > (1 << 20) || a.pw > (1 << 20) || a.dil_h > 4096 ||
      a.dil_w > 4096 || a.Kh > 4096 || a.Kw > 4096)
    return false;
  p = Phases{};
  for (int r = 0; r < (int)a.sh; ++r) {
    int cnt = 0;
    for (int k = 0; k < (int)a.Kh; ++k) {
      const int num = r + (int)a.ph - k * (int)a.dil_h;
      if (((num % (int)a.sh) + (int)a.sh) % (int)a.sh != 0) continue;
      if (cnt >= kMaxT) return false;
      p.thk[r][cnt] = k;
      p.thd[r][cnt] = floordiv(num, (int)a.sh);
      ++cnt;
    }
    p.nth[r] = cnt;
  }
  for (int r = 0; r < (int)a.sw; ++r) {
    int cnt = 0;
    for (int k = 0; k < (int)a.Kw; ++k) {
      const int num = r + (int)a.pw - k * (int)a.dil_w;
      if (((num % (int)a.sw) + (int)a.sw) % (int)a.sw != 0) continue;
      if (cnt >= kMaxT) return false;
      p.twk[r][cnt] = k;
      p.twd[r][cnt] = floordiv(num, (int)a.sw);
      ++cnt;
    }
    p.ntw[r] = cnt;
  }
  const int64_t Wp = (a.W_out + a.sw - 1) / a.sw;
  p.jb = (int)((Wp + 63) / 64);
  return true;
}

namespace {

template <int OCB, int RQ>
hipError_t launch_blocked(const DeconvArgs& a, Phases p, hipStream_t s) {
  p.ocb = (int)((a.OC + OCB - 1) / OCB);
  const int64_t Hp = (a.H_out + a.sh - 1) / a.sh;
  p.ib = (int)((Hp + RQ - 1) / RQ);
  const int G = (int)((a.IC + 15) / 16);
  const size_t bytes = (size_t)a.N * a.H_in * a.W_in * G * 16;
  void* ws = nullptr;
  hipError_t e = workspace_acquire(&ws, bytes, s);
  if (e != hipSuccess) return e;
  const int64_t t = (int64_t)a.N * a.H_in * G * a.W_in;
  hipLaunchKernelGGL(k_nchw_to_blocked16, dim3((unsigned)((t + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, a.x, (int8_t*)ws, a.N, (int)a.IC, (int)a.H_in,
                     (int)a.W_in, G);
  e = hipGetLastError();
  if (e == hipSuccess) {
    const int64_t waves = (int64_t)p.ocb * p.jb * a.sw * p.ib * a.sh * a.N;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (a.IC % 16 == 0)
      hipLaunchKernelGGL((k_deconv_dot4_blocked<OCB, true, RQ>), grid, dim3(kThreads), 0, s, a, p,
                         (const int8_t*)ws);
    else
      hipLaunchKernelGGL((k_deconv_dot4_blocked<OCB, false, RQ>), grid, dim3(kThreads), 0, s, a, p,
                         (const int8_t*)ws);
    e = hipGetLastError();
  }
  hipError_t f = workspace_release(ws, s);
  return e != hipSuccess ? e : f;
}

}  // namespace

bool deconv_dot4_supported(const DeconvArgs& a) {
  Phases p;
  if (a.groups != 1 || a.IC % 4 != 0 || a.ldw % 4 != 0 || ((uintptr_t)a.w & 3) != 0) return false;
  if (a.H_out > (1 << 24) || a.W_out > (1 << 24) || a.H_in > (1 << 24) || a.W_in > (1 << 24) ||
      a.IC > (1 << 24) || a.OC > (1 << 24))
    return false;
  if (!make_phases(a, p)) return false;
  const int64_t waves = ((a.OC + 7) / 8) * (int64_t)p.jb * a.sw * (a.H_out + 1) * a.N;
  return (waves + 3) / 4 < ((int64_t)1 << 31);
}

// The blocked path: the input relaid out into channel blocks of 16 in a
// stream-ordered workspace, then 8 output channels x 1 phase row per wave.
// (The direct NCHW path without a workspace and tiles of 16 channels or 2-4
// phase rows per wave measured no faster and were removed.)
hipError_t launch_deconv_dot4(const DeconvArgs& a, hipStream_t s) {
  Phases p;
  if (!make_phases(a, p)) return hipErrorInvalidValue;
  return launch_blocked<8, 1>(a, p, s);
}

}  // namespace q8ta
