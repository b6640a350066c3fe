// q8ta_conv2d_transposed (and the stride-1 forward q8ta_conv2d) as an
// implicit GEMM on v_mfma_i32_32x32x32_i8.
//
// The gather of "Add q8ta_conv2d_transposed op" (Solution) sums, for output
// (oh, ow), the taps (kh, kw) whose numerators oh + pad_h - kh*dil_h and
// ow + pad_w - kw*dil_w are non-negative multiples of the stride and land
// inside the input.  Which taps qualify depends only on the residues
// rh = oh mod s_h and rw = ow mod s_w, so for strides up to 2 the output
// splits into at most four phases; in phase (rh, rw) output
// (s_h*i + rh, s_w*j + rw) reads input (i + dh, j + dw) for every qualifying
// tap, a dense correlation of the input with the phase's sub-kernel.  Taps
// that fall outside the input read the zero point, so with the weight sum
// taken over all of the phase's taps, sum x*w - zp * sum w is the gather (the
// zero-point-filled form of the page's Constraints (1)).
//
// Workgroup: one image n, one phase row i, 64 phase columns j0 .. j0 + 63 and
// 32 * WO output channels (WO <= 4 waves of 32 channels).
//  1. The input halo -- rows i + dh_min .. i + dh_max, columns
//     j0 + dw_min .. j0 + 63 + dw_max, all IC channels -- is staged once in
//     LDS in the operand's K-contiguous order: block q of 16 channels of
//     pixel (r, c) is 16 bytes at ((r * IC/16 + q) * HC + pos(c)) * 16, so
//     the 32 lanes of a half-wave that read 32 consecutive pixels of one
//     channel block read 512 contiguous bytes.  A thread loads one 32-bit
//     word (4 columns) from each of 16 channel planes, transposes the 16 x 4
//     bytes in registers and writes four 16-byte chunks; words outside the
//     image hold the zero point.
//  2. Each wave runs every phase with its accumulators live together
//     (2 fragments of 32 pixels per phase): for each tap of the phase and
//     each 32 channels, two pixel fragments come from LDS (the A operand,
//     lane l: pixel l % 32, channels 16 * (l / 32) .. +15) and one weight
//     fragment straight from global memory / L2 (the B operand, lane l: row
//     oc = l % 32 of the [OC, ldw] weight, the same 16 channels).  The weight
//     fragments of the next tap block are requested before the current one
//     is multiplied.  v_dot4 against 0x01010101 over the weight fragments
//     gives the phase's weight sums.
//  3. Accumulator register r of lane l holds pixel 8 * (r / 4) + 4 * (l / 32)
//     + r % 4 of its fragment and channel l % 32.  With s_w = 2 the two column
//     phases of a row give each lane 8 consecutive output columns
//     (4 pixels x 2 residues) of one channel: the epilogue requantizes them
//     in registers and stores 8 bytes (4 with s_w = 1).
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kTJ = 64;                // phase columns per workgroup
constexpr int kThreads = 256;          // 4 waves
constexpr int kMaxHalo = 64 * 1024;    // LDS bytes of the halo (two workgroups per CU)
constexpr int kMaxTaps = 8;            // qualifying taps per residue

template <int B, int E>
struct Static {
  template <class F>
  __device__ __forceinline__ static void each(F&& f) {
    if constexpr (B < E) {
      f(std::integral_constant<int, B>{});
      Static<B + 1, E>::each(f);
    }
  }
};

// Tap plan.  The qualifying taps of residue r form arithmetic progressions
// in the kernel index and in the input offset (solutions of one linear
// congruence): tap t of row residue r is kernel row hk0[r] + t*hks[r] with
// input row offset hd0[r] + t*hds[r]; likewise for columns.
struct MxPlan {
  int nth[2], hk0[2], hks[2], hd0[2], hds[2];
  int ntw[2], wk0[2], wks[2], wd0[2], wds[2];
  int dhmin, dwmin, coff;     // halo origin: row i + dhmin, column j0 + dwmin - coff (a multiple of 4)
  int HR, HC, NQ;             // halo rows, columns (multiple of 8), channel blocks of 16
  int Hp, Wp;                 // phase rows and columns
  int tiles_j, tiles_oc, WO;  // column tiles, channel tiles, waves per workgroup
  int nib;                    // channel blocks of 32*KB per tap
  int out_vec;                // whole 8- (4-) byte stores are aligned
  int xcd;                    // remap workgroups so each XCD walks consecutive rows
};

// LDS column slot: chunk c of a 16-byte-per-pixel row at c ^ 4 when bit 4 of
// c is set, so that the lanes one ds_read_b128 cycle serves (lane quads of
// even, resp. odd, index in a half-wave) reach distinct bank groups for
// aligned runs of 32 pixels.  Rows are padded to a multiple of 8 chunks, so
// the slot stays inside the row.
__device__ __forceinline__ int pos(int c) { return c ^ (((c >> 4) & 1) << 2); }

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int e) { return (w >> (8 * e)) & 0xffu; }

template <int SH, int SW, int KB>
__global__ __launch_bounds__(kThreads, 2) void k_deconv_mx(DeconvArgs a, MxPlan p) {
  extern __shared__ __attribute__((aligned(16))) v4i xs4[];
  int8_t* xs = reinterpret_cast<int8_t*>(xs4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lo = lane & 31;
  const int hi = lane >> 5;

  // Workgroups go round-robin to the 8 XCDs; with p.xcd the block index is
  // remapped so that each XCD walks a contiguous run of tiles (neighbouring
  // phase rows share halo rows in that XCD's L2).
  int b = blockIdx.x;
  if (p.xcd) {
    const int per = (int)(gridDim.x >> 3);
    b = (b & 7) * per + (b >> 3);
  }
  const int tj = b % p.tiles_j;  b /= p.tiles_j;
  const int i = b % p.Hp;        b /= p.Hp;
  const int toc = b % p.tiles_oc; b /= p.tiles_oc;
  const int n = b;
  const int j0 = tj * kTJ;

  const int H_in = (int)a.H_in, W_in = (int)a.W_in, IC = (int)a.IC, OC = (int)a.OC;
  const int NQ = p.NQ, HC = p.HC;

  // ---- 1. input halo -> LDS ----------------------------------------------
  {
    const int row0 = i + p.dhmin;
    const int col0 = j0 + p.dwmin - p.coff;
    const int CG = HC >> 2;
    const int units = p.HR * NQ * CG;
    const uint32_t zp4 = 0x01010101u * ((uint32_t)a.izp & 0xffu);
    const int64_t plane = (int64_t)H_in * W_in;
    const int8_t* xn = a.x + (int64_t)n * IC * plane;
    for (int u = tid; u < units; u += kThreads) {
      const int cg = u % CG;
      const int rq = u / CG;
      const int q = rq % NQ;
      const int r = rq / NQ;
      const int ih = row0 + r;
      const int iw = col0 + 4 * cg;
      // W_in % 4 == 0 and iw % 4 == 0: a word is wholly inside or outside.
      // The loads are unconditional, from addresses clamped into the image.
      const bool in_img = ih >= 0 && ih < H_in && iw >= 0 && iw < W_in;
      const int ihc = ih < 0 ? 0 : (ih >= H_in ? H_in - 1 : ih);
      const int iwc = iw < 0 ? 0 : (iw > W_in - 4 ? W_in - 4 : iw);
      const int8_t* src = xn + (int64_t)(16 * q) * plane + (int64_t)ihc * W_in + iwc;
      uint32_t d[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) d[t] = *reinterpret_cast<const uint32_t*>(src + t * plane);
#pragma unroll
      for (int t = 0; t < 16; ++t) d[t] = in_img ? d[t] : zp4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v4i chunk;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          chunk[g] = (int)(byte_of(d[4 * g], e) | (byte_of(d[4 * g + 1], e) << 8) |
                           (byte_of(d[4 * g + 2], e) << 16) | (byte_of(d[4 * g + 3], e) << 24));
        xs4[(r * NQ + q) * HC + pos(4 * cg + e)] = chunk;
      }
    }
  }
  __syncthreads();
  if (wave >= p.WO) return;

  // ---- 2. phases -----------------------------------------------------------
  const int ocw = toc * (32 * p.WO) + 32 * wave;
  const int oc = ocw + lo;
  const int occ = oc < OC ? oc : OC - 1;   // rows past OC read row OC - 1 (never stored)
  const int8_t* wrow = a.w + (int64_t)occ * a.ldw + 16 * hi;
  const int Kw = (int)a.Kw;

  v16i acc[SH * SW][2];
  int32_t wsum[SH * SW];
#pragma unroll
  for (int ph = 0; ph < SH * SW; ++ph) {
    wsum[ph] = 0;
    acc[ph][0] = v16i{};
    acc[ph][1] = v16i{};
  }

  // Load cursor: one tap block (KB steps of 32 channels) ahead of the
  // compute, across phases; past the last block it re-reads block 0.
  int lrh = 0, lrw = 0, lth = 0, ltw = 0, lib = 0;
  bool ldone = false;
  auto nth_of = [&](int r) { return r ? p.nth[1] : p.nth[0]; };
  auto ntw_of = [&](int r) { return r ? p.ntw[1] : p.ntw[0]; };
  auto skip_empty = [&]() {
    while (lrh < SH && nth_of(lrh) * ntw_of(lrw) == 0) {
      if (++lrw == SW) { lrw = 0; ++lrh; }
    }
    if (lrh >= SH) ldone = true;
  };
  skip_empty();
  auto load_blk = [&](v4i (&dst)[KB]) {
    int off = 0;
    if (!ldone) {
      const int kh = (lrh ? p.hk0[1] : p.hk0[0]) + lth * (lrh ? p.hks[1] : p.hks[0]);
      const int kw = (lrw ? p.wk0[1] : p.wk0[0]) + ltw * (lrw ? p.wks[1] : p.wks[0]);
      off = (kh * Kw + kw) * IC + lib * (32 * KB);
    }
    const int8_t* src = wrow + off;
#pragma unroll
    for (int k = 0; k < KB; ++k) dst[k] = *reinterpret_cast<const v4i*>(src + 32 * k);
    if (ldone) return;
    if (++lib < p.nib) return;
    lib = 0;
    if (++ltw < ntw_of(lrw)) return;
    ltw = 0;
    if (++lth < nth_of(lrh)) return;
    lth = 0;
    if (++lrw == SW) { lrw = 0; ++lrh; }
    skip_empty();
  };

  v4i bcur[KB], bnext[KB];
  load_blk(bcur);

  Static<0, SH>::each([&](auto RH) {
    constexpr int rh = decltype(RH)::value;
    Static<0, SW>::each([&](auto RW) {
      constexpr int rw = decltype(RW)::value;
      constexpr int ph = rh * SW + rw;
      const int nth = p.nth[rh], ntw = p.ntw[rw];
      for (int th = 0; th < nth; ++th) {
        const int r = p.hd0[rh] + th * p.hds[rh] - p.dhmin;
        for (int tw = 0; tw < ntw; ++tw) {
          const int cs = p.wd0[rw] + tw * p.wds[rw] - p.dwmin + p.coff;
          const int c0 = pos(lo + cs), c1 = pos(32 + lo + cs);
          for (int ib = 0; ib < p.nib; ++ib) {
            load_blk(bnext);
#pragma unroll
            for (int k = 0; k < KB; ++k) {
              const int q = 2 * (ib * KB + k) + hi;
              const int base = (r * NQ + q) * HC;
              const v4i a0 = xs4[base + c0];
              const v4i a1 = xs4[base + c1];
              acc[ph][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, bcur[k], acc[ph][0], 0, 0, 0);
              acc[ph][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, bcur[k], acc[ph][1], 0, 0, 0);
              int32_t t = __builtin_amdgcn_sdot4(bcur[k][0], 0x01010101, 0, false);
              t = __builtin_amdgcn_sdot4(bcur[k][1], 0x01010101, t, false);
              t = __builtin_amdgcn_sdot4(bcur[k][2], 0x01010101, t, false);
              t = __builtin_amdgcn_sdot4(bcur[k][3], 0x01010101, t, false);
              wsum[ph] += t;
            }
#pragma unroll
            for (int k = 0; k < KB; ++k) bcur[k] = bnext[k];
          }
        }
      }
    });
  });

  // ---- 3. epilogue ---------------------------------------------------------
  // lanes l and l + 32 hold the two 16-channel halves of each weight
  // fragment; wsum becomes the zero-point term izp * sum w, once per phase
#pragma unroll
  for (int ph = 0; ph < SH * SW; ++ph) wsum[ph] = a.izp * (wsum[ph] + __shfl_xor(wsum[ph], 32, 64));
  if (oc >= OC) return;
  float sc = 0.0f, bi = 0.0f;
  if (!a.acc) {
    sc = a.wscale[oc];
    bi = a.bias ? a.bias[oc] : 0.0f;
  }
  const int H_out = (int)a.H_out, W_out = (int)a.W_out;
  Static<0, SH>::each([&](auto RH) {
    constexpr int rh = decltype(RH)::value;
    const int oh = SH * i + rh;
    if (oh >= H_out) return;
    const int64_t orow = (((int64_t)n * OC + oc) * H_out + oh) * W_out;
#pragma unroll
    for (int jf = 0; jf < 2; ++jf) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int jb = j0 + jf * 32 + 8 * g + 4 * hi;   // phase column of register 4g
        const int ow0 = SW * jb;
        int32_t c[4 * SW];                                // output columns ow0 .. ow0 + 4*SW - 1
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int rw = 0; rw < SW; ++rw)
            c[SW * e + rw] = acc[rh * SW + rw][jf][4 * g + e] - wsum[rh * SW + rw];
        if (a.acc) {
#pragma unroll
          for (int k = 0; k < 4 * SW; ++k)
            if (ow0 + k < W_out) a.acc[orow + ow0 + k] = c[k];
          continue;
        }
        int qv[4 * SW];
#pragma unroll
        for (int k = 0; k < 4 * SW; ++k) qv[k] = requant(c[k], sc, bi, a.rq);
        if (p.out_vec && ow0 + 4 * SW <= W_out) {
          if constexpr (SW == 2) {
            typedef uint32_t v2u __attribute__((ext_vector_type(2)));
            *reinterpret_cast<v2u*>(a.out + orow + ow0) =
                v2u{pack4(qv[0], qv[1], qv[2], qv[3]), pack4(qv[4], qv[5], qv[6], qv[7])};
          } else {
            *reinterpret_cast<uint32_t*>(a.out + orow + ow0) = pack4(qv[0], qv[1], qv[2], qv[3]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4 * SW; ++k)
            if (ow0 + k < W_out) a.out[orow + ow0 + k] = (int8_t)qv[k];
        }
      }
    }
  });
}

int floordiv(int x, int y) { return x >= 0 ? x / y : -((-x + y - 1) / y); }

// Builds the tap plan; false when this kernel cannot take the shape.
bool make_mx_plan(const DeconvArgs& a, MxPlan& p, int& KB, bool forward) {
  if (a.groups != 1) return false;
  if (forward ? (a.sh != 1 || a.sw != 1) : (a.sh < 1 || a.sh > 2 || a.sw < 1 || a.sw > 2))
    return false;
  if (a.IC % 32 != 0 || a.IC > 4096 || a.ldw % 16 != 0 || ((uintptr_t)a.w & 15) != 0) return false;
  if (a.W_in % 4 != 0 || ((uintptr_t)a.x & 3) != 0) return false;
  if (a.OC > (1 << 20) || a.H_out > (1 << 20) || a.W_out > (1 << 20) || a.H_in > (1 << 20) ||
      a.W_in > (1 << 20) || a.N > (1 << 20) || a.ph > 4096 || a.pw > 4096 || a.dil_h > 4096 ||
      a.dil_w > 4096 || a.Kh > 4096 || a.Kw > 4096)
    return false;
  KB = a.IC % 256 == 0 ? 8 : a.IC % 128 == 0 ? 4 : a.IC % 64 == 0 ? 2 : 1;
  const int sh = (int)a.sh, sw = (int)a.sw;
  p = MxPlan{};
  int dhmin = 1 << 30, dhmax = -(1 << 30), dwmin = 1 << 30, dwmax = -(1 << 30);
  // residue tables of one axis: (kernel index, input offset) of each qualifying tap
  auto axis = [&](int s, int K, int pad, int dil, int* nt, int* k0, int* ks, int* d0, int* ds,
                  int& dmin, int& dmax) {
    for (int r = 0; r < s; ++r) {
      int tk[kMaxTaps], td[kMaxTaps], cnt = 0;
      for (int k = 0; k < K; ++k) {
        const int num = r + pad - k * dil;
        if (!forward && ((num % s) + s) % s != 0) continue;
        if (cnt >= kMaxTaps) return false;
        tk[cnt] = k;
        td[cnt] = forward ? k * dil - pad : floordiv(num, s);
        ++cnt;
      }
      nt[r] = cnt;
      k0[r] = cnt ? tk[0] : 0;
      d0[r] = cnt ? td[0] : 0;
      ks[r] = cnt > 1 ? tk[1] - tk[0] : 0;
      ds[r] = cnt > 1 ? td[1] - td[0] : 0;
      for (int t = 0; t < cnt; ++t) {
        if (tk[t] != k0[r] + t * ks[r] || td[t] != d0[r] + t * ds[r]) return false;
        dmin = td[t] < dmin ? td[t] : dmin;
        dmax = td[t] > dmax ? td[t] : dmax;
      }
    }
    return true;
  };
  if (!axis(sh, (int)a.Kh, (int)a.ph, (int)a.dil_h, p.nth, p.hk0, p.hks, p.hd0, p.hds, dhmin,
            dhmax))
    return false;
  if (!axis(sw, (int)a.Kw, (int)a.pw, (int)a.dil_w, p.ntw, p.wk0, p.wks, p.wd0, p.wds, dwmin,
            dwmax))
    return false;
  if (dhmin > dhmax) dhmin = dhmax = 0;   // no taps on that axis at all
  if (dwmin > dwmax) dwmin = dwmax = 0;
  p.dhmin = dhmin;
  p.dwmin = dwmin;
  p.coff = ((dwmin % 4) + 4) % 4;
  p.HR = dhmax - dhmin + 1;
  p.HC = (p.coff + kTJ + dwmax - dwmin + 7) / 8 * 8;
  p.NQ = (int)(a.IC / 16);
  if ((int64_t)p.HR * p.NQ * p.HC * 16 > kMaxHalo) return false;
  p.Hp = (int)((a.H_out + sh - 1) / sh);
  p.Wp = (int)((a.W_out + sw - 1) / sw);
  p.tiles_j = (p.Wp + kTJ - 1) / kTJ;
  p.WO = (int)(a.OC >= 128 ? 4 : (a.OC + 31) / 32);
  p.tiles_oc = (int)((a.OC + 32 * p.WO - 1) / (32 * p.WO));
  p.nib = (int)(a.IC / (32 * KB));
  const int step = 4 * sw;   // bytes per lane store
  p.out_vec = (a.W_out % step == 0) && (((uintptr_t)a.out % step) == 0);
  const int64_t blocks = (int64_t)a.N * p.Hp * p.tiles_j * p.tiles_oc;
  p.xcd = blocks % 8 == 0;
  return blocks < ((int64_t)1 << 31);
}

template <int SH, int SW, int KB>
hipError_t launch_mx_t(const DeconvArgs& a, const MxPlan& p, hipStream_t s) {
  const int64_t blocks = (int64_t)a.N * p.Hp * p.tiles_j * p.tiles_oc;
  const size_t lds = (size_t)p.HR * p.NQ * p.HC * 16;
  hipLaunchKernelGGL((k_deconv_mx<SH, SW, KB>), dim3((unsigned)blocks), dim3(kThreads), lds, s, a,
                     p);
  return hipGetLastError();
}

template <int SH, int SW>
hipError_t launch_mx_kb(const DeconvArgs& a, const MxPlan& p, int KB, hipStream_t s) {
  switch (KB) {
    case 8: return launch_mx_t<SH, SW, 8>(a, p, s);
    case 4: return launch_mx_t<SH, SW, 4>(a, p, s);
    case 2: return launch_mx_t<SH, SW, 2>(a, p, s);
    default: return launch_mx_t<SH, SW, 1>(a, p, s);
  }
}

hipError_t launch_mx(const DeconvArgs& a, hipStream_t s, bool forward) {
  MxPlan p;
  int KB = 1;
  if (!make_mx_plan(a, p, KB, forward)) return hipErrorInvalidValue;
  const int sh = forward ? 1 : (int)a.sh, sw = forward ? 1 : (int)a.sw;
  if (sh == 2 && sw == 2) return launch_mx_kb<2, 2>(a, p, KB, s);
  if (sh == 2) return launch_mx_kb<2, 1>(a, p, KB, s);
  if (sw == 2) return launch_mx_kb<1, 2>(a, p, KB, s);
  return launch_mx_kb<1, 1>(a, p, KB, s);
}

}  // namespace

bool deconv_mx_supported(const DeconvArgs& a) {
  MxPlan p;
  int KB;
  return make_mx_plan(a, p, KB, false);
}

bool conv_mx_supported(const DeconvArgs& a) {
  MxPlan p;
  int KB;
  return make_mx_plan(a, p, KB, true);
}

// Default for stride-1 forward convs with at least 256 workgroups.
bool conv_mx_preferred(const DeconvArgs& a) {
  MxPlan p;
  int KB;
  if (!make_mx_plan(a, p, KB, true)) return false;
  return (int64_t)a.N * p.Hp * p.tiles_j * p.tiles_oc >= 256;
}

hipError_t launch_deconv_mx(const DeconvArgs& a, hipStream_t s) { return launch_mx(a, s, false); }
hipError_t launch_conv_mx(const DeconvArgs& a, hipStream_t s) { return launch_mx(a, s, true); }

}  // namespace q8ta
