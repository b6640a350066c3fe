// q8ta_conv2d_transposed as an implicit GEMM on CDNA4 int8 matrix cores.
//
// The gather of "Add q8ta_conv2d_transposed op" (Solution) sums, for output
// (oh, ow), the taps (kh, kw) whose numerators oh + pad_h - kh and
// ow + pad_w - kw are non-negative multiples of the stride and land inside the
// input.  Which taps qualify depends only on the residues rh = oh mod s_h and
// rw = ow mod s_w, so the output splits into s_h * s_w phases.  Writing
// oh = rh + s_h*i, each qualifying tap kh of residue rh reads input row
// ih = i + dh with dh = (rh + pad_h - kh) / s_h (an exact division), and the
// same for columns.  Every phase is a dense stride-1 correlation of the input
// with its own sub-kernel: no product with a non-qualifying tap is issued.
//
// Borders: a qualifying tap whose (ih, iw) falls outside the input reads the
// zero point, so that (zp - zp) * w adds nothing, and the kernel forms
// sum x*w - zp * sum w over the phase's taps (the zero-point-filled
// formulation the page cites in its Constraints (1); equal to the gather).
//
// Workgroup tile: one image n, WI consecutive phase rows i, TJ = 16*FJ phase
// columns j, OCB = WO*16*FO output channels, all s_h*s_w phases.  Steps:
//  1. Stage the input halo (rows i0+dh_min .. i0+WI-1+dh_max, columns
//     j0+dw_min .. j0+TJ-1+dw_max, all IC channels) from NCHW global memory
//     into LDS in pixel-major order (each pixel's channels contiguous), which
//     is the K-contiguous layout the MFMA operand wants.  A thread loads one
//     32-bit word (4 columns) from each of 16 channel planes -- coalesced
//     along the row -- transposes the 16x4 bytes in registers and writes four
//     16-byte pixel chunks.  Out-of-image words hold the zero point.
//  2. Each wave owns one phase row i and FO output-channel fragments and runs
//     its phases one after another (all of them, or every PS-th when PS waves
//     split them): for every tap of the phase and every 64
//     channels, FJ activation fragments come from LDS and FO weight fragments
//     (16 channels x 64 input channels, K-contiguous rows of the [OC, ldw]
//     weight) come straight from global memory / L2; v_mfma_i32_16x16x64_i8
//     accumulates D[16 pixels][16 oc].  The weight fragments are also summed
//     with v_dot4 against 0x01010101 for the zero-point term.
//  3. The epilogue requantizes in registers and writes bytes into an LDS copy
//     of the workgroup's NCHW output block (phases interleaved there), which
//     is then written to global memory in whole rows.
#include <cstdlib>
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMaxS = 4;   // largest stride the tiled kernel takes
constexpr int kMaxT = 8;   // largest number of taps per residue
constexpr int kMaxLds = 160 * 1024;
constexpr int kDepth = 2;  // weight-fragment prefetch distance (iterations)

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

struct Plan {
  int nth[kMaxS], thk[kMaxS][kMaxT], thd[kMaxS][kMaxT];
  int ntw[kMaxS], twk[kMaxS][kMaxT], twd[kMaxS][kMaxT];
  // The qualifying taps of a residue form an arithmetic progression in both
  // the kernel index and the input offset (solutions of one linear
  // congruence): tap t of row residue r is kernel row hk0[r] + t*hks[r],
  // input row offset hd0[r] + t*hds[r]; likewise for columns.  The kernel
  // uses these (scalar arithmetic) instead of indexing the tables.
  int hk0[kMaxS], hks[kMaxS], hd0[kMaxS], hds[kMaxS];
  int wk0[kMaxS], wks[kMaxS], wd0[kMaxS], wds[kMaxS];
  int dhmin, dwmin;
  int Hp, Wp;                 // phase rows / columns: ceil(H_out/s_h), ceil(W_out/s_w)
  int WI, WO, TJ, OCB;        // workgroup tile
  int PS;                     // waves splitting the phases (1: a wave runs them all)
  int HR, HC, ICP;            // staged input tile: rows, columns (multiple of 4), channels (x64)
  int ORows, OCols, OPlane;   // staged output tile
  int tiles_i, tiles_j, tiles_oc;
  int x_dword;                // 32-bit input loads are safe (W_in % 4 == 0, aligned x)
  int out_vec;                // 16-byte output stores are safe
  int x_bytes;                // LDS bytes of the input tile
};

// Chunk position of 16-byte channel chunk q of LDS pixel column c: the 16
// lanes that read 16 consecutive pixels at one chunk hit distinct banks.
__device__ __forceinline__ int xswz(int c, int q, int icp) {
  return (icp & 127) == 0 ? (q ^ (c & 7)) : (q ^ ((c >> 1) & 3));
}

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int p) { return (w >> (8 * p)) & 0xffu; }

template <int FJ, int FO>
__global__ __launch_bounds__(512) void k_deconv(DeconvArgs a, Plan p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  int8_t* xs = smem;
  int8_t* os = smem + p.x_bytes;

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;

  int b = blockIdx.x;
  const int tj = b % p.tiles_j;  b /= p.tiles_j;
  const int ti = b % p.tiles_i;  b /= p.tiles_i;
  const int toc = b % p.tiles_oc; b /= p.tiles_oc;
  const int n = b;
  const int i0 = ti * p.WI;
  const int j0 = tj * p.TJ;
  const int oc0 = toc * p.OCB;

  const int H_in = (int)a.H_in, W_in = (int)a.W_in, IC = (int)a.IC;
  const int row0 = i0 + p.dhmin;                 // input row of LDS row 0
  const int col0 = ((j0 + p.dwmin) >> 2) * 4;   // input column of LDS column 0 (floor to 4)

  // Wave roles: phase row wi of the tile, output-channel group wo, and phase
  // group ps (the wave runs phases ps, ps + PS, ... of the s_h * s_w).
  const int waves_used = p.WI * p.WO * p.PS;
  const bool active = wave < waves_used;
  const int wi = wave % p.WI;
  const int wo = (wave / p.WI) % p.WO;
  const int ps = wave / (p.WI * p.WO);
  const int i = i0 + wi;
  const int ocw = oc0 + wo * 16 * FO;
  const int sh = (int)a.sh, sw = (int)a.sw;
  const int S = sh * sw;
  const int NQ64 = p.ICP >> 6;
  // first phase s' >= s of this wave whose output row exists
  auto next_phase = [&](int s) {
    while (s < S && s / sw + sh * i >= (int)a.H_out) s += p.PS;
    return s;
  };

  // Per-phase iteration state.  A phase's (tap row, tap column, 64-channel
  // slice) iterations run as one flat sequence; the weight fragments of
  // iteration it + kDepth are requested while iteration it computes (ring of
  // kDepth + 1 register buffers), so their global/L2 latency overlaps the
  // MFMAs.  The first phase's first fragments are requested before the input
  // staging, so that latency overlaps the staging's.
  constexpr int R = kDepth + 1;
  v4i bb[R][FO];
  int rh = 0, rw = 0, nth = 0, ntw = 0, nit = 0;
  int hk0 = 0, hks = 0, hd0 = 0, hds = 0, wk0 = 0, wks = 0, wd0 = 0, wds = 0;
  int pth = 0, ptw = 0, pc = 0;   // prefetch cursor
  int cth = 0, ctw = 0, cc = 0;   // compute cursor
  // The loads are unconditional (an exec-masked load would make the
  // compiler wait for every outstanding load before the next MFMA):
  // rows past OC read row OC - 1 (their accumulators are never
  // stored) and channel chunks past IC read the row's last chunk
  // (their activations are zero in LDS; their weight sums are dropped
  // in `compute`).  tapoff + icb + 16 <= Kh*Kw*IC <= ldw.
  auto load_b = [&](v4i (&dst)[FO]) {
    const int64_t tapoff = (int64_t)((hk0 + pth * hks) * (int)a.Kw + wk0 + ptw * wks) * IC;
    const int icb = (pc * 4 + lgrp) * 16;
    const int icc = icb < IC ? icb : IC - 16;
#pragma unroll
    for (int f = 0; f < FO; ++f) {
      const int oc = ocw + f * 16 + lrow;
      const int occ = oc < a.OC ? oc : (int)a.OC - 1;
      dst[f] = *reinterpret_cast<const v4i*>(a.w + (int64_t)occ * a.ldw + tapoff + icc);
    }
    // advance, saturating at the phase's last iteration (prefetches
    // past the end re-read it and are never consumed)
    if (++pc == NQ64) {
      pc = 0;
      if (++ptw == ntw) { ptw = 0; ++pth; }
    }
    if (pth >= nth) { pth = nth - 1; ptw = ntw - 1; pc = NQ64 - 1; }
  };
  auto setup = [&](int s) {
    rh = s / sw;
    rw = s - rh * sw;
    nth = p.nth[rh];
    ntw = p.ntw[rw];
    nit = nth * ntw * NQ64;
    hk0 = p.hk0[rh]; hks = p.hks[rh]; hd0 = p.hd0[rh] - p.dhmin; hds = p.hds[rh];
    wk0 = p.wk0[rw]; wks = p.wks[rw]; wd0 = p.wd0[rw]; wds = p.wds[rw];
    pth = ptw = pc = 0;
    cth = ctw = cc = 0;
    if (nit > 0) Static<0, kDepth>::each([&](auto U) { load_b(bb[decltype(U)::value]); });
  };
  int s = active ? next_phase(ps) : S;
  if (s < S) setup(s);

  // ---- 1. stage the input halo tile -------------------------------------
  {
    const int CG = p.HC >> 2;
    const int NQ = p.ICP >> 4;
    const int units = CG * p.HR * NQ;
    const uint32_t zp4 = 0x01010101u * ((uint32_t)a.izp & 0xffu);
    const int64_t plane = (int64_t)H_in * W_in;
    const int8_t* xn = a.x + (int64_t)n * IC * plane;
    for (int u = tid; u < units; u += nthreads) {
      const int cg = u % CG;
      const int r = (u / CG) % p.HR;
      const int q = u / (CG * p.HR);
      const int ih = row0 + r;
      const int iw = col0 + 4 * cg;
      const bool row_ok = ih >= 0 && ih < H_in;
      uint32_t d[16];
      if (p.x_dword) {
        // All 16 loads are unconditional, from addresses clamped into the
        // image (an exec-masked load per channel would make the compiler
        // wait for each one before the next); out-of-image words and
        // channels past IC are then replaced.  W_in % 4 == 0 and iw is a
        // multiple of 4, so the clamped column stays word-aligned.
        const bool in_img = row_ok && iw >= 0 && iw < W_in;
        const int ihc = ih < 0 ? 0 : (ih >= H_in ? H_in - 1 : ih);
        const int iwc = iw < 0 ? 0 : (iw > W_in - 4 ? W_in - 4 : iw);
        const int8_t* src0 = xn + (int64_t)ihc * W_in + iwc;
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int ic = q * 16 + t;
          const int icc = ic < IC ? ic : IC - 1;
          d[t] = *reinterpret_cast<const uint32_t*>(src0 + (int64_t)icc * plane);
        }
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int ic = q * 16 + t;
          d[t] = ic >= IC ? 0u : (in_img ? d[t] : zp4);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int ic = q * 16 + t;
          uint32_t v;
          if (ic >= IC) {
            v = 0u;
          } else if (!row_ok) {
            v = zp4;
          } else {
            const int8_t* src = xn + (int64_t)ic * plane + (int64_t)ih * W_in;
            v = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c = iw + e;
              const uint32_t by = (c >= 0 && c < W_in) ? (uint32_t)(uint8_t)src[c]
                                                       : ((uint32_t)a.izp & 0xffu);
              v |= by << (8 * e);
            }
          }
          d[t] = v;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {   // pixel 4*cg + e of this row
        v4i chunk;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          chunk[g] = (int)(byte_of(d[4 * g], e) | (byte_of(d[4 * g + 1], e) << 8) |
                           (byte_of(d[4 * g + 2], e) << 16) | (byte_of(d[4 * g + 3], e) << 24));
        const int c = 4 * cg + e;
        *reinterpret_cast<v4i*>(xs + ((int64_t)(r * p.HC + c) * p.ICP) +
                                16 * xswz(c, q, p.ICP)) = chunk;
      }
    }
  }
  __syncthreads();

  // ---- 2. per-wave phase loop --------------------------------------------
  if (active) {
    // Scales and bias only for the requantizing call (the accumulator entry
    // point passes no weight_scales).
    float sc[FO], bi[FO];
#pragma unroll
    for (int f = 0; f < FO; ++f) {
      const int oc = ocw + f * 16 + lrow;
      const bool ok = oc < a.OC && !a.acc;
      sc[f] = ok ? a.wscale[oc] : 0.0f;
      bi[f] = (ok && a.bias) ? a.bias[oc] : 0.0f;
    }

    while (s < S) {
      const int oh = rh + sh * i;
      v4i acc[FJ][FO];
      int32_t wsum[FO];
#pragma unroll
      for (int f = 0; f < FO; ++f) {
        wsum[f] = 0;
#pragma unroll
        for (int g = 0; g < FJ; ++g) acc[g][f] = v4i{0, 0, 0, 0};
      }
      auto compute = [&](const v4i (&bf)[FO]) {
        const int lr = wi + hd0 + cth * hds;
        const int dw = wd0 + ctw * wds;
        const int q = cc * 4 + lgrp;
        v4i af[FJ];
#pragma unroll
        for (int g = 0; g < FJ; ++g) {
          const int c = j0 + g * 16 + lrow + dw - col0;
          af[g] = *reinterpret_cast<const v4i*>(xs + ((int64_t)(lr * p.HC + c) * p.ICP) +
                                                16 * xswz(c, q, p.ICP));
        }
        const bool in_ic = q * 16 < IC;
#pragma unroll
        for (int f = 0; f < FO; ++f) {
          int32_t t = __builtin_amdgcn_sdot4(bf[f][0], 0x01010101, 0, false);
          t = __builtin_amdgcn_sdot4(bf[f][1], 0x01010101, t, false);
          t = __builtin_amdgcn_sdot4(bf[f][2], 0x01010101, t, false);
          t = __builtin_amdgcn_sdot4(bf[f][3], 0x01010101, t, false);
          wsum[f] += in_ic ? t : 0;
        }
#pragma unroll
        for (int g = 0; g < FJ; ++g)
#pragma unroll
          for (int f = 0; f < FO; ++f)
            acc[g][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[g], bf[f], acc[g][f], 0, 0, 0);
        if (++cc == NQ64) {
          cc = 0;
          if (++ctw == ntw) { ctw = 0; ++cth; }
        }
      };
      // Whole groups of R iterations run without guards, so the compiler
      // sees every load of the ring and waits only for the oldest; the
      // remaining nit % R iterations follow.  The ring's first kDepth
      // fragments were requested by `setup`.
      if (nit > 0) {
        const int nfull = nit - nit % R;
        for (int base = 0; base < nfull; base += R) {
          Static<0, R>::each([&](auto U) {
            constexpr int u = decltype(U)::value;
            load_b(bb[(u + kDepth) % R]);
            compute(bb[u]);
          });
        }
        Static<0, R - 1>::each([&](auto U) {
          constexpr int u = decltype(U)::value;
          if (nfull + u < nit) {
            load_b(bb[(u + kDepth) % R]);
            compute(bb[u]);
          }
        });
      }
      // epilogue of phase (rh, rw): lane holds pixels j = j0+16g+4*lgrp+e of
      // output channel ocw + 16f + lrow.
#pragma unroll
      for (int f = 0; f < FO; ++f) {
        int32_t v = wsum[f];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        const int oc = ocw + f * 16 + lrow;
        const int ocl = oc - oc0;
#pragma unroll
        for (int g = 0; g < FJ; ++g) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jl = g * 16 + 4 * lgrp + e;       // phase column within the tile
            const int ow = rw + sw * (j0 + jl);
            const int32_t c = acc[g][f][e] - a.izp * v;
            if (a.acc) {
              if (oc < a.OC && ow < a.W_out)
                a.acc[(((int64_t)n * a.OC + oc) * a.H_out + oh) * a.W_out + ow] = c;
            } else {
              const int qv = requant(c, sc[f], bi[f], a.rq);
              os[ocl * p.OPlane + (rh + sh * wi) * p.OCols + rw + sw * jl] = (int8_t)qv;
            }
          }
        }
      }
      s = next_phase(s + p.PS);
      if (s < S) setup(s);
    }
  }
  if (a.acc) return;
  __syncthreads();

  // ---- 3. write the output block -----------------------------------------
  {
    const int oh0 = (int)a.sh * i0;
    const int ow0 = (int)a.sw * j0;
    const int rows = p.OCB * p.ORows;
    if (p.out_vec) {
      const int chunks = p.OCols >> 4;
      for (int u = tid; u < rows * chunks; u += nthreads) {
        const int ch = u % chunks;
        const int rr = u / chunks;
        const int orow = rr % p.ORows;
        const int ocl = rr / p.ORows;
        const int oc = oc0 + ocl;
        const int oh = oh0 + orow;
        const int ow = ow0 + ch * 16;
        if (oc < a.OC && oh < a.H_out && ow < a.W_out) {
          const v4i v = *reinterpret_cast<const v4i*>(os + ocl * p.OPlane + orow * p.OCols + ch * 16);
          *reinterpret_cast<v4i*>(a.out + (((int64_t)n * a.OC + oc) * a.H_out + oh) * a.W_out + ow) = v;
        }
      }
    } else {
      for (int u = tid; u < rows * p.OCols; u += nthreads) {
        const int col = u % p.OCols;
        const int rr = u / p.OCols;
        const int orow = rr % p.ORows;
        const int ocl = rr / p.ORows;
        const int oc = oc0 + ocl;
        const int oh = oh0 + orow;
        const int ow = ow0 + col;
        if (oc < a.OC && oh < a.H_out && ow < a.W_out)
          a.out[(((int64_t)n * a.OC + oc) * a.H_out + oh) * a.W_out + ow] =
              os[ocl * p.OPlane + orow * p.OCols + col];
      }
    }
  }
}

int floordiv(int a, int b) { return (a >= 0) ? a / b : -((-a + b - 1) / b); }

// Builds the phase/tap tables and the tile geometry; returns false when the
// tiled kernel cannot take the shape.  forward: the stride-1 forward conv,
// one phase whose taps kh read input rows oh + kh*dil_h - pad_h (a dense
// correlation like every phase of the transposed conv).
bool make_plan(const DeconvArgs& a, Plan& p, int& FJ, int& FO, bool forward = false) {
  if (a.sh > kMaxS || a.sw > kMaxS) return false;
  if (forward && (a.sh != 1 || a.sw != 1)) return false;
  if (a.groups != 1 || a.dil_h < 1 || a.dil_w < 1 || a.dil_h > 4096 || a.dil_w > 4096 ||
      a.Kh > 4096 || a.Kw > 4096)
    return false;
  if (a.IC % 16 != 0 || a.ldw % 16 != 0 || ((uintptr_t)a.w & 15) != 0) return false;
  if (a.IC > 4096 || a.OC > (1 << 20) || a.H_out > (1 << 20) || a.W_out > (1 << 20) ||
      a.H_in > (1 << 20) || a.W_in > (1 << 20) || a.N > (1 << 20) || a.ph > 4096 || a.pw > 4096)
    return false;
  const int sh = (int)a.sh, sw = (int)a.sw, ph = (int)a.ph, pw = (int)a.pw;
  p = Plan{};
  int dhmin = 1 << 30, dhmax = -(1 << 30), dwmin = 1 << 30, dwmax = -(1 << 30);
  for (int r = 0; r < sh; ++r) {
    int cnt = 0;
    for (int k = 0; k < (int)a.Kh; ++k) {
      const int num = r + ph - k * (int)a.dil_h;
      if (!forward && ((num % sh) + sh) % sh != 0) continue;
      if (cnt >= kMaxT) return false;
      p.thk[r][cnt] = k;
      p.thd[r][cnt] = forward ? k * (int)a.dil_h - ph : floordiv(num, sh);
      dhmin = p.thd[r][cnt] < dhmin ? p.thd[r][cnt] : dhmin;
      dhmax = p.thd[r][cnt] > dhmax ? p.thd[r][cnt] : dhmax;
      ++cnt;
    }
    p.nth[r] = cnt;
  }
  for (int r = 0; r < sw; ++r) {
    int cnt = 0;
    for (int k = 0; k < (int)a.Kw; ++k) {
      const int num = r + pw - k * (int)a.dil_w;
      if (!forward && ((num % sw) + sw) % sw != 0) continue;
      if (cnt >= kMaxT) return false;
      p.twk[r][cnt] = k;
      p.twd[r][cnt] = forward ? k * (int)a.dil_w - pw : floordiv(num, sw);
      dwmin = p.twd[r][cnt] < dwmin ? p.twd[r][cnt] : dwmin;
      dwmax = p.twd[r][cnt] > dwmax ? p.twd[r][cnt] : dwmax;
      ++cnt;
    }
    p.ntw[r] = cnt;
  }
  // progressions (checked against the scanned tables)
  for (int r = 0; r < sh; ++r) {
    const int n = p.nth[r];
    p.hk0[r] = n ? p.thk[r][0] : 0;
    p.hd0[r] = n ? p.thd[r][0] : 0;
    p.hks[r] = n > 1 ? p.thk[r][1] - p.thk[r][0] : 0;
    p.hds[r] = n > 1 ? p.thd[r][1] - p.thd[r][0] : 0;
    for (int t = 0; t < n; ++t)
      if (p.thk[r][t] != p.hk0[r] + t * p.hks[r] || p.thd[r][t] != p.hd0[r] + t * p.hds[r])
        return false;
  }
  for (int r = 0; r < sw; ++r) {
    const int n = p.ntw[r];
    p.wk0[r] = n ? p.twk[r][0] : 0;
    p.wd0[r] = n ? p.twd[r][0] : 0;
    p.wks[r] = n > 1 ? p.twk[r][1] - p.twk[r][0] : 0;
    p.wds[r] = n > 1 ? p.twd[r][1] - p.twd[r][0] : 0;
    for (int t = 0; t < n; ++t)
      if (p.twk[r][t] != p.wk0[r] + t * p.wks[r] || p.twd[r][t] != p.wd0[r] + t * p.wds[r])
        return false;
  }
  if (dhmin > dhmax) { dhmin = dhmax = 0; }   // no row taps at all
  if (dwmin > dwmax) { dwmin = dwmax = 0; }
  p.dhmin = dhmin;
  p.dwmin = dwmin;
  p.Hp = (int)((a.H_out + sh - 1) / sh);
  p.Wp = (int)((a.W_out + sw - 1) / sw);

  // Two 16-channel fragments per wave and up to four phase rows per
  // workgroup: 8 waves (two per SIMD) where the LDS tiles allow, which
  // measured faster than four fragments per wave with one wave per SIMD
  // ([8,256,64,64] K3 s2: 45.6 -> 36.7 us; forward K3 s1: 30.5 -> 29.2 us).
  FJ = p.Wp >= 64 ? 4 : p.Wp >= 32 ? 2 : 1;
  FO = a.OC >= 32 ? 2 : 1;
  bool small = false;
  {
    // Small problems are latency-bound: when the default tile leaves the chip
    // mostly idle (fewer than 256 workgroups), take one 16-channel fragment
    // and one 16-column phase fragment per wave and one phase row per
    // workgroup, for as many workgroups as the problem allows (measured on
    // [1,64,32,32] K4 s2: 18.3 -> 12.7 us with one channel fragment, 10.8 ->
    // 9.3 us with one column fragment and one row: 16 -> 64 workgroups).
    const int64_t ocb = 2 * 16 * FO;
    const int64_t est = a.N * ((p.Hp + 3) / 4) * ((p.Wp + 16 * FJ - 1) / (16 * FJ)) *
                        ((a.OC + ocb - 1) / ocb);
    small = est < 256;
    if (small) {
      FO = 1;
      FJ = 1;
    }
  }
  p.TJ = 16 * FJ;
  const int ocf = 16 * FO;
  p.WO = (int)((a.OC + ocf - 1) / ocf);
  if (p.WO > 2) p.WO = 2;
  p.OCB = p.WO * ocf;
  p.ICP = (int)((a.IC + 63) / 64 * 64);
  const int c_lo = (dwmin >> 2) * 4;   // relative to j0, j0 is a multiple of 16
  const int c_hi = p.TJ - 1 + dwmax + 1;
  p.HC = ((c_hi - c_lo) + 3) / 4 * 4;
  p.OCols = sw * p.TJ;
  int wi_pref = small ? 1 : 4;   // small problems: more, smaller workgroups
  if (wi_pref * p.WO > 8) wi_pref = 8 / p.WO;
  for (int WI = wi_pref; WI >= 1; --WI) {
    p.WI = WI;
    p.HR = WI + dhmax - dhmin;
    p.ORows = sh * WI;
    p.OPlane = p.ORows * p.OCols + 16;
    const int64_t xb = (int64_t)p.HR * p.HC * p.ICP;
    const int64_t ob = a.acc ? 0 : (int64_t)p.OCB * p.OPlane;
    if (xb + ob <= kMaxLds) {
      p.x_bytes = (int)xb;
      p.tiles_i = (p.Hp + WI - 1) / WI;
      p.tiles_j = (p.Wp + p.TJ - 1) / p.TJ;
      p.tiles_oc = (int)((a.OC + p.OCB - 1) / p.OCB);
      // Small problems also split the phases over up to 8 waves, so a wave's
      // serial chain of weight-fetch latencies is shorter.
      p.PS = 1;
      if (small) {
        const int S = sh * sw;
        const int room = 8 / (p.WI * p.WO);
        p.PS = S < room ? S : room;
        if (p.PS < 1) p.PS = 1;
      }
      p.x_dword = (a.W_in % 4 == 0) && (((uintptr_t)a.x & 3) == 0);
      p.out_vec = (a.W_out % 16 == 0) && (((uintptr_t)a.out & 15) == 0) && (p.OCols % 16 == 0);
      const int64_t blocks = (int64_t)p.tiles_j * p.tiles_i * p.tiles_oc * a.N;
      return blocks < (int64_t)1 << 31;
    }
  }
  return false;
}

template <int FJ, int FO>
hipError_t launch_t(const DeconvArgs& a, const Plan& p, hipStream_t s) {
  const size_t lds = (size_t)p.x_bytes + (a.acc ? 0 : (size_t)p.OCB * p.OPlane);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_deconv<FJ, FO>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t blocks = (int64_t)p.tiles_j * p.tiles_i * p.tiles_oc * a.N;
  const int threads = 64 * p.WI * p.WO * p.PS;
  hipLaunchKernelGGL((k_deconv<FJ, FO>), dim3((unsigned)blocks), dim3(threads), lds, s, a, p);
  return hipGetLastError();
}

}  // namespace

// Scales and bias are read only by requantizing calls (the accumulator entry
// point passes no weight_scales); the same NULL read once faulted the
// matrix-core GEMM.
constexpr bool kMfmaDeconvEnabled = true;

bool deconv_mfma_supported(const DeconvArgs& a) {
  if (!kMfmaDeconvEnabled) return false;
  Plan p;
  int FJ, FO;
  return make_plan(a, p, FJ, FO);
}

bool conv_mfma_supported(const DeconvArgs& a) {
  if (!kMfmaDeconvEnabled) return false;
  Plan p;
  int FJ, FO;
  return make_plan(a, p, FJ, FO, true);
}

namespace {
hipError_t launch_mfma(const DeconvArgs& a, hipStream_t s, bool forward) {
  Plan p;
  int FJ, FO;
  if (!make_plan(a, p, FJ, FO, forward)) return hipErrorInvalidValue;
#define Q8TA_DC(fj, fo) \
  if (FJ == fj && FO == fo) return launch_t<fj, fo>(a, p, s);
  Q8TA_DC(1, 1) Q8TA_DC(1, 2)
  Q8TA_DC(2, 1) Q8TA_DC(2, 2)
  Q8TA_DC(4, 1) Q8TA_DC(4, 2)
#undef Q8TA_DC
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_deconv_mfma(const DeconvArgs& a, hipStream_t s) { return launch_mfma(a, s, false); }
hipError_t launch_conv_mfma(const DeconvArgs& a, hipStream_t s) { return launch_mfma(a, s, true); }

}  // namespace q8ta
