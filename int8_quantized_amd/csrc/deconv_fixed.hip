// q8ta_conv2d_transposed for a kernel size and stride known at compile time
// (the 3x3 and 4x4 stride-2 convolutions, and the 3x3 stride-1 forward conv),
// as an implicit GEMM on v_mfma_i32_32x32x32_i8.
//
// The gather of "Add q8ta_conv2d_transposed op" (Solution) sums, for output
// (oh, ow), the taps (kh, kw) whose numerators oh + pad_h - kh and
// ow + pad_w - kw are non-negative multiples of the stride and land inside the
// input.  With oh = s*i + rh the qualifying kernel rows of residue rh are the
// kh with kh = rh + pad_h (mod s), and each reads input row i + dh(rh, kh),
// dh = (rh + pad_h - kh) / s; columns likewise.  So phase (rh, rw) is a dense
// correlation of the input with its sub-kernel, and every (phase, tap) pair
// reads the input at one of a few shifts (dh, dw): for 3x3 stride 2 the 9
// taps of the 4 phases use only 4 shifts, for 4x4 the 16 taps 9 shifts.  All
// of this is fixed by (K, s, pad mod s) and is built at compile time.  Taps
// that fall outside the input read the zero point, so with the weight sum
// taken over the phase's taps, sum x*w - zp * sum w is the gather (the page's
// Constraints (1), zero-point-filled form).
//
// Workgroup: one image, two phase rows, 64 phase columns and 128 output
// channels.  With stride 2 the taps fall into two groups by output-row
// residue (the phases (rh, 0) and (rh, 1) of each rh); eight waves, two per
// SIMD: wave w takes channels 32 (w % 4) .. +31 of group w / 4, so the two
// waves of a SIMD share its matrix cores and one wave's requantize (vector
// ALU) runs beside the other's products.  (Within one wave a 32x32x32
// product hides only about four independent vector instructions.)  A wave's
// accumulators: 2 phases x 4 fragments of 32 pixels (2 rows x 2 column
// halves).  With stride 1 (one phase) four waves take all taps.
// Steps:
//  * the whole input halo of the tile (all channels) is staged in LDS once,
//    in the operand's K-contiguous order: 32-bit words of 16 channel planes,
//    transposed in registers with byte permutes; out-of-image words hold the
//    zero point;
//  * then, per 32 channels and per shift, the wave reads its 4 pixel
//    fragments from LDS once (the A operand; the next shift's fragments are
//    requested before the current shift's products) and multiplies them with the
//    weight fragment of every tap of its group that reads that shift (the B
//    operand, lane l: row l % 32 of the [OC, ldw] weight, K bytes
//    16 * (l / 32) .. +15, straight from global memory / L2); each tap's
//    register is refilled right after its products, two steps ahead from
//    two register sets where registers allow;
//  * v_dot4 against 0x01010101 over the weight fragments gives the phase
//    weight sums.
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// Threads per workgroup: 8 waves (two per SIMD) for stride 2, whose taps
// split into two groups; 4 waves for stride 1.
template <int S>
constexpr int threads_of() { return S == 2 ? 512 : 256; }
constexpr int kTR = 2;          // phase rows per workgroup
constexpr int kTJ = 64;         // phase columns per workgroup
constexpr int kOCB = 128;       // output channels per workgroup
constexpr int kStageUnits = 1024;  // halo staging units per workgroup (the host checks the count)

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

constexpr int fdiv(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
constexpr int fmod_(int a, int b) { return ((a % b) + b) % b; }

// Compile-time tap table of a (K, stride, pad mod stride) pattern.  Tap t:
// phase ph = rh*S + rw, kernel position (kh, kw), and input shift index.
// Shift (dh, dw) is relative: the input row of phase row i is
// i + dh + base_h, base_h = (pad_h - PM) / S for the transposed conv
// (-pad_h for the forward one), so only PM = pad mod S enters the table.
template <int S, int K, int PM, bool FWD>
struct Pattern {
  int T = 0;                 // taps
  int ph[64] = {}, kh[64] = {}, kw[64] = {}, sh[64] = {};
  int NS = 0;                // distinct shifts
  int sdh[64] = {}, sdw[64] = {};
  int dhmin = 0, dhmax = 0, dwmin = 0, dwmax = 0;
  constexpr Pattern() {
    int rk[8][8] = {}, rd[8][8] = {}, rn[8] = {};
    for (int r = 0; r < S; ++r)
      for (int k = 0; k < K; ++k) {
        if (!FWD && fmod_(r + PM - k, S) != 0) continue;
        rk[r][rn[r]] = k;
        rd[r][rn[r]] = FWD ? k : fdiv(r + PM - k, S);
        ++rn[r];
      }
    dhmin = dwmin = 1 << 20;
    dhmax = dwmax = -(1 << 20);
    for (int rh = 0; rh < S; ++rh)
      for (int rw = 0; rw < S; ++rw)
        for (int a = 0; a < rn[rh]; ++a)
          for (int b = 0; b < rn[rw]; ++b) {
            const int dh = rd[rh][a], dw = rd[rw][b];
            int s = 0;
            while (s < NS && !(sdh[s] == dh && sdw[s] == dw)) ++s;
            if (s == NS) {
              sdh[NS] = dh;
              sdw[NS] = dw;
              ++NS;
            }
            ph[T] = rh * S + rw;
            kh[T] = rk[rh][a];
            kw[T] = rk[rw][b];
            sh[T] = s;
            ++T;
            dhmin = dh < dhmin ? dh : dhmin;
            dhmax = dh > dhmax ? dh : dhmax;
            dwmin = dw < dwmin ? dw : dwmin;
            dwmax = dw > dwmax ? dw : dwmax;
          }
  }
};

// Taps of one group: output-row residue g of the stride phases (-1: every
// tap), in the order the K loop visits them (shift by shift, then by tap).
struct ShiftList {
  int n = 0;
  int s[64] = {};
};

template <int S, int K, int PM, bool FWD>
constexpr bool in_group(int t, int g) {
  constexpr Pattern<S, K, PM, FWD> P{};
  return g < 0 || P.ph[t] / S == g;
}

template <int S, int K, int PM, bool FWD>
constexpr int group_taps(int g) {
  constexpr Pattern<S, K, PM, FWD> P{};
  int n = 0;
  for (int t = 0; t < P.T; ++t) n += in_group<S, K, PM, FWD>(t, g) ? 1 : 0;
  return n;
}

// distinct input shifts read by group g, in increasing shift index
template <int S, int K, int PM, bool FWD>
constexpr ShiftList group_shifts(int g) {
  constexpr Pattern<S, K, PM, FWD> P{};
  ShiftList L{};
  for (int s = 0; s < P.NS; ++s) {
    bool used = false;
    for (int t = 0; t < P.T; ++t) used = used || (P.sh[t] == s && in_group<S, K, PM, FWD>(t, g));
    if (used) L.s[L.n++] = s;
  }
  return L;
}

// position of tap t in group g's visiting order
template <int S, int K, int PM, bool FWD>
constexpr int tap_ord(int g, int t) {
  constexpr Pattern<S, K, PM, FWD> P{};
  const ShiftList L = group_shifts<S, K, PM, FWD>(g);
  int o = 0;
  for (int i = 0; i < L.n; ++i)
    for (int u = 0; u < P.T; ++u)
      if (P.sh[u] == L.s[i] && in_group<S, K, PM, FWD>(u, g)) {
        if (u == t) return o;
        ++o;
      }
  return -1;
}

// The output block in LDS: row (channel o, output row) at OPITCH bytes.
// With stride 2 the 16-byte chunk c of a row sits at slot c ^ out_swz(o) and
// its two 8-byte halves are exchanged when bit 4 of o is set: then the
// requantize's 64-bit stores (32 channels of one row position per cycle) and
// the copy-out's 16-byte reads (two channels' rows per cycle) each cover all
// 64 LDS banks once.
template <int S>
constexpr int out_pitch() { return S == 2 ? 160 : kTJ * S + 16; }
template <int S>
__device__ __forceinline__ int out_swz(int o) {
  return S == 2 ? (((o >> 2) & 1) | (((o >> 3) & 1) << 1) | (((o >> 1) & 1) << 2)) : 0;
}
template <int S>
__device__ __forceinline__ int out_half(int o) { return S == 2 ? ((o >> 4) & 1) : 0; }

// Runtime geometry (host-built).
struct FxPlan {
  int base_h, base_w;    // input row / column of phase (0, 0) shift (0, 0)
  int HR, HC, coff;      // halo rows, columns (multiple of 8), column offset in the first word
  int Hp, Wp, tiles_i, tiles_j, tiles_oc;
  int xcd;
  int out_vec;           // 16-byte output stores allowed
};

// LDS column slot (see the 32-pixel fragment reads): chunk c at c ^ 4 when
// bit 4 of c is set; rows are padded to a multiple of 8 chunks.
__device__ __forceinline__ int pos(int c) { return c ^ (((c >> 4) & 1) << 2); }

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int e) { return (w >> (8 * e)) & 0xffu; }

// XF: the input is fp32 (a.xf; the fused quantize -> transposed conv) and is
// quantized with the quantize_per_tensor formula as the halo is staged, so
// the int8 input never goes to memory.
// RELU: the relu-fused epilogue (lower clamp at the output zero point).
// PKW: the weight is prepacked (a.wpk): fragment (channel block ob, kh, kw,
// 32-channel step kc) is one contiguous KiB, lane l's 16 bytes at 16 l.
template <int S, int K, int PM, bool FWD, bool XF, bool RELU, bool PKW = false>
__global__ __launch_bounds__(threads_of<S>(), 1) void k_deconv_fixed(DeconvArgs a, FxPlan p) {
  constexpr int kThreads = threads_of<S>();
  constexpr int kStageSlots = kStageUnits / kThreads;
  constexpr bool SPLIT = S == 2;
  constexpr Pattern<S, K, PM, FWD> P{};
  constexpr int NPH = S * S;
  constexpr int OROWS = kTR * S;                // output rows of the tile
  constexpr int OCOLS = kTJ * S;                // output columns of the tile
  constexpr int OPITCH = out_pitch<S>();        // LDS bytes per (channel, row) of the output copy

  extern __shared__ __attribute__((aligned(16))) v4i smem[];
  const int HR = p.HR, HC = p.HC;
  const int NQ = (int)a.IC / 16;               // 16-channel blocks
  v4i* xs = smem;                               // the halo: HR x NQ x HC chunks
  int8_t* os = reinterpret_cast<int8_t*>(smem + HR * NQ * HC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lo = lane & 31;
  const int hi = lane >> 5;

  int b = blockIdx.x;
  if (p.xcd) {
    const int per = (int)(gridDim.x >> 3);
    b = (b & 7) * per + (b >> 3);
  }
  const int tj = b % p.tiles_j;   b /= p.tiles_j;
  const int ti = b % p.tiles_i;   b /= p.tiles_i;
  const int toc = b % p.tiles_oc; b /= p.tiles_oc;
  const int n = b;
  const int i0 = ti * kTR, j0 = tj * kTJ, oc0 = toc * kOCB;

  const int H_in = (int)a.H_in, W_in = (int)a.W_in, IC = (int)a.IC, OC = (int)a.OC;
  const int64_t plane = (int64_t)H_in * W_in;
  const uint32_t zp4 = 0x01010101u * ((uint32_t)a.izp & 0xffu);
  const int row0 = i0 + P.dhmin + p.base_h;        // input row of halo row 0
  const int col0 = j0 + P.dwmin + p.base_w - p.coff;   // input column of halo column 0 (multiple of 4)

  // ---- halo staging: unit u = (halo row, 16-channel block, 4 columns) ----
  // All units are loaded before any is transposed and stored, at most
  // kStageSlots per thread (the host checks the count); from fp32 input two
  // at a time (16-byte loads of 4 pixels per channel, quantized in registers).
  {
    const int CG = HC >> 2;
    const int units = HR * NQ * CG;
    auto unit_src = [&](int uu, int& ih, int& iw) {
      const int cg = uu % CG;
      const int q = (uu / CG) % NQ;
      const int r = uu / (CG * NQ);
      ih = row0 + r;
      iw = col0 + 4 * cg;
      const int ihc = ih < 0 ? 0 : (ih >= H_in ? H_in - 1 : ih);
      const int iwc = iw < 0 ? 0 : (iw > W_in - 4 ? W_in - 4 : iw);
      return (int64_t)(16 * q) * plane + (int64_t)ihc * W_in + iwc;
    };
    // 4x4 byte transposes (chunk e, dword g = byte e of channels 4g .. 4g+3)
    // and the LDS store of one unit
    auto put = [&](int u, const uint32_t (&d)[16]) {
      const int cg = u % CG;
      const int q = (u / CG) % NQ;
      const int r = u / (CG * NQ);
      v4i chunk[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t t0 = __builtin_amdgcn_perm(d[4 * g + 1], d[4 * g], 0x05010400u);
        const uint32_t t1 = __builtin_amdgcn_perm(d[4 * g + 1], d[4 * g], 0x07030602u);
        const uint32_t t2 = __builtin_amdgcn_perm(d[4 * g + 3], d[4 * g + 2], 0x05010400u);
        const uint32_t t3 = __builtin_amdgcn_perm(d[4 * g + 3], d[4 * g + 2], 0x07030602u);
        chunk[0][g] = (int)__builtin_amdgcn_perm(t2, t0, 0x05040100u);
        chunk[1][g] = (int)__builtin_amdgcn_perm(t2, t0, 0x07060302u);
        chunk[2][g] = (int)__builtin_amdgcn_perm(t3, t1, 0x05040100u);
        chunk[3][g] = (int)__builtin_amdgcn_perm(t3, t1, 0x07060302u);
      }
      v4i* dst = xs + (r * NQ + q) * HC;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[pos(4 * cg + e)] = chunk[e];
    };
    if constexpr (!XF) {
      const int8_t* xn = a.x + (int64_t)n * IC * plane;
      uint32_t stg[kStageSlots][16];
#pragma unroll
      for (int sl = 0; sl < kStageSlots; ++sl) {
        if (sl * kThreads >= units) break;   // wave-uniform
        const int u = tid + sl * kThreads;
        int ih, iw;
        const int8_t* src = xn + unit_src(u < units ? u : units - 1, ih, iw);
#pragma unroll
        for (int t = 0; t < 16; ++t) stg[sl][t] = *reinterpret_cast<const uint32_t*>(src + t * plane);
      }
#pragma unroll
      for (int sl = 0; sl < kStageSlots; ++sl) {
        if (sl * kThreads >= units) break;
        const int u = tid + sl * kThreads;
        if (u < units) {
          int ih, iw;
          unit_src(u, ih, iw);
          // W_in % 4 == 0, iw % 4 == 0: a word is wholly inside or outside
          const bool in_img = ih >= 0 && ih < H_in && iw >= 0 && iw < W_in;
          uint32_t d[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) d[t] = in_img ? stg[sl][t] : zp4;
          put(u, d);
        }
      }
    } else {
      typedef float v4f __attribute__((ext_vector_type(4)));
      const float* xn = a.xf + (int64_t)n * IC * plane;
      const float zpf = (float)a.izp;
      constexpr int PAIR = 2;
      static_assert(kStageSlots % PAIR == 0, "slot pairs");
#pragma unroll
      for (int sl0 = 0; sl0 < kStageSlots; sl0 += PAIR) {
        if (sl0 * kThreads >= units) break;   // wave-uniform
        v4f raw[PAIR][16];
#pragma unroll
        for (int h = 0; h < PAIR; ++h) {
          const int u = tid + (sl0 + h) * kThreads;
          int ih, iw;
          const float* src = xn + unit_src(u < units ? u : units - 1, ih, iw);
#pragma unroll
          for (int t = 0; t < 16; ++t) raw[h][t] = *reinterpret_cast<const v4f*>(src + t * plane);
        }
#pragma unroll
        for (int h = 0; h < PAIR; ++h) {
          const int u = tid + (sl0 + h) * kThreads;
          if (u < units) {
            int ih, iw;
            unit_src(u, ih, iw);
            const bool in_img = ih >= 0 && ih < H_in && iw >= 0 && iw < W_in;
            uint32_t d[16];
#pragma unroll
            for (int t = 0; t < 16; ++t)
              d[t] = in_img ? pack4(quantize1(raw[h][t][0], a.inv_in, zpf),
                                    quantize1(raw[h][t][1], a.inv_in, zpf),
                                    quantize1(raw[h][t][2], a.inv_in, zpf),
                                    quantize1(raw[h][t][3], a.inv_in, zpf))
                            : zp4;
            put(u, d);
          }
        }
      }
    }
  }

  // ---- per wave: 32 output channels of one tap group ------------------------
  // With stride 2 the taps split by output-row residue rh: waves 0-3 take
  // the phases of one residue, waves 4-7 (which share the SIMDs of 0-3) the
  // other, so one wave's requantize (vector ALU) runs beside the other's
  // products (matrix cores).  A wave owns whole output rows: it requantizes
  // them into LDS and copies them out itself.
  constexpr int NF = 2 * kTR;                   // pixel fragments: kTR rows x 2 column halves
  constexpr int NG = SPLIT ? S : 1;             // phases per group
  const int og = wave & 3;                      // 32-channel block
  const int oc = oc0 + 32 * og + lo;
  const int occ = oc < OC ? oc : OC - 1;    // rows past OC read row OC - 1 (never stored)
  const int8_t* wrow = a.w + (int64_t)occ * a.ldw + 16 * hi;
  const int Kw = __builtin_amdgcn_readfirstlane((int)a.Kw);
  const int nk = IC / 32;   // even: IC % 64 == 0
  // prepacked: blocks past the last one (OC not a multiple of 128) read the
  // last block (outputs never stored)
  const int nob = (OC + 31) / 32;
  const int ob = (oc0 >> 5) + og < nob ? (oc0 >> 5) + og : nob - 1;
  const int8_t* wpkw = PKW ? a.wpk + (int64_t)ob * (K * K * nk * 1024) + 16 * lane : nullptr;
  // tap offsets are wave-uniform (scalar); only wrow differs between lanes
  auto wfrag = [&](int t, int off) {
    if constexpr (PKW)
      return *reinterpret_cast<const v4i*>(wpkw + ((P.kh[t] * K + P.kw[t]) * nk + (off >> 5)) * 1024);
    else
      return *reinterpret_cast<const v4i*>(wrow + ((P.kh[t] * Kw + P.kw[t]) * IC + off));
  };
  // The 32-channel steps run in a rotated order, a different rotation for
  // neighbouring workgroups of one XCD: all workgroups start together and
  // would otherwise request the same weight lines from L2 at the same moment
  // (the integer sums do not depend on the order).
  const int rot = (int)(blockIdx.x >> 3) % nk;
  auto kidx = [&](int k) { return k + rot < nk ? k + rot : k + rot - nk; };

  const int ocl = 32 * og + lo;
  const bool oc_ok = oc < OC;
  float sc = 0.0f, bi = 0.0f;
  if (oc_ok && !a.acc) {
    sc = a.wscale[oc];
    bi = a.bias ? a.bias[oc] : 0.0f;
  }
  const int H_out = (int)a.H_out, W_out = (int)a.W_out;
  const float ozp128 = a.rq.ozp + 128.0f, qmin128 = a.rq.qmin + 128.0f;
  constexpr int PIECES = OCOLS / 16;
  const int oh0 = S * i0, ow0 = S * j0;

  auto run = [&](auto gtag) {
    constexpr int G = decltype(gtag)::value;        // row residue of the group, -1: every tap
    constexpr int RH = G < 0 ? 0 : G;
    constexpr ShiftList L = group_shifts<S, K, PM, FWD>(G);
    // Groups of up to 6 taps request each weight fragment two steps ahead,
    // into two alternating register sets; the 8-tap groups of 4x4 (longer
    // steps, no registers to spare) and stride 1 one step ahead.
    constexpr bool TWO = SPLIT && group_taps<S, K, PM, FWD>(G) <= 6;
    v16i acc[NG][NF];
    int32_t wsum[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      wsum[g] = 0;
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[g][f] = v16i{};
    }
    // first fragments, in the order the loop refills them (set 0, then set
    // 1, each shift by shift): the compiler's wait counts at the loop head
    // are then those of the steady state
    v4i bw[P.T], bw1[P.T];
    Static<0, TWO ? 2 : 1>::each([&](auto RI) {
      constexpr int set = decltype(RI)::value;
      Static<0, L.n>::each([&](auto SI) {
        constexpr int s = L.s[decltype(SI)::value];
        Static<0, P.T>::each([&](auto TI) {
          constexpr int t = decltype(TI)::value;
          if constexpr (P.sh[t] == s && in_group<S, K, PM, FWD>(t, G)) {
            if constexpr (set == 0) bw[t] = wfrag(t, 32 * kidx(0));
            else bw1[t] = wfrag(t, 32 * kidx(1));
          }
        });
      });
    });
    __syncthreads();   // the halo is staged

    // A fragments of input shift (s_dh, s_dw), step k
    // chunk (r * NQ + 2k + hi) * HC + pos(c): the lane's part (hi, column c)
    // is fixed for the whole loop, one offset per column half and column
    // shift, so a step adds only the wave-uniform (r * NQ + 2k) * HC
    constexpr int NDW = P.dwmax - P.dwmin + 1;
    int loff[2][NDW];
#pragma unroll
    for (int fx = 0; fx < 2; ++fx)
#pragma unroll
      for (int j = 0; j < NDW; ++j) loff[fx][j] = hi * HC + pos(fx * 32 + lo + j + p.coff);
    auto aload = [&](v4i (&dst)[NF], int s_dh, int s_dw, int k) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int r = (f >> 1) + s_dh - P.dhmin;
        dst[f] = xs[(r * NQ + 2 * k) * HC + loff[f & 1][s_dw - P.dwmin]];
      }
    };
    v4i acur[NF], anext[NF];
    // Step k: the products of the group's taps, shift by shift (the next
    // shift's fragments requested before the current shift's products;
    // after the last shift, the first shift of step k + 1).  Tap t's register
    // is refilled with step kref's fragment right after its products.
    auto step = [&](int k, int kref, v4i (&cur)[P.T]) {
      const int kc = kidx(k);
      const int kr = kidx(kref);
      const int knext = k + 1 < nk ? kidx(k + 1) : kc;   // past the end: re-read (unused)
      Static<0, L.n>::each([&](auto SI) {
        constexpr int si = decltype(SI)::value;
        constexpr int s = L.s[si];
        if constexpr (si + 1 < L.n) aload(anext, P.sdh[L.s[si + 1]], P.sdw[L.s[si + 1]], kc);
        else aload(anext, P.sdh[L.s[0]], P.sdw[L.s[0]], knext);
        Static<0, P.T>::each([&](auto TI) {
          constexpr int t = decltype(TI)::value;
          if constexpr (P.sh[t] == s && in_group<S, K, PM, FWD>(t, G)) {
            constexpr int g = P.ph[t] % NG;
#pragma unroll
            for (int f = 0; f < NF; ++f)
              acc[g][f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(acur[f], cur[t], acc[g][f], 0, 0, 0);
            int32_t w4 = __builtin_amdgcn_sdot4(cur[t][0], 0x01010101, 0, false);
            w4 = __builtin_amdgcn_sdot4(cur[t][1], 0x01010101, w4, false);
            w4 = __builtin_amdgcn_sdot4(cur[t][2], 0x01010101, w4, false);
            w4 = __builtin_amdgcn_sdot4(cur[t][3], 0x01010101, w4, false);
            wsum[g] += w4;
            cur[t] = wfrag(t, 32 * kr);
            // keep the refill here: left to itself the compiler sinks every
            // refill to the end of the step, and the next step then starts
            // with a wait for all of them
            __builtin_amdgcn_sched_barrier(0);
          }
        });
#pragma unroll
        for (int f = 0; f < NF; ++f) acur[f] = anext[f];
      });
    };
    aload(acur, P.sdh[L.s[0]], P.sdw[L.s[0]], kidx(0));
    if constexpr (TWO) {
      for (int k = 0; k < nk; k += 2) {
        step(k, k + 2 < nk ? k + 2 : k, bw);
        step(k + 1, k + 3 < nk ? k + 3 : k + 1, bw1);
      }
    } else {
      for (int k = 0; k < nk; ++k) step(k, k + 1 < nk ? k + 1 : k, bw);
    }
    // The group with fewer taps waits here for the other's products: its
    // requantize (a long run of vector instructions) would otherwise win
    // the SIMD's issue and slow them down; the two requantize together.
    if constexpr (SPLIT) __syncthreads();
    // zw = input zero point x the phase's weight sum (lanes l and l + 32 hold
    // the two 16-channel halves of each weight fragment)
    int32_t zw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) zw[g] = a.izp * (wsum[g] + __shfl_xor(wsum[g], 32, 64));

    if (a.acc) {
      // accumulator output (verification entry point): direct int32 stores
      if (oc_ok) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int ii = i0 + (f >> 1);
              const int j = j0 + (f & 1) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              const int oh = S * ii + RH, ow = S * j + g;
              if (oh < H_out && ow < W_out)
                a.acc[(((int64_t)n * OC + oc) * H_out + oh) * W_out + ow] = acc[g][f][r] - zw[g];
            }
      }
      return;
    }
    // Requantize the group's rows into LDS.  Word (f, gr, h): 4 codes of one
    // output row, packed in offset form (code + 128) by the conversion
    // itself: fragment f, register group gr, and with S == 2 phase columns
    // e = 2h, 2h + 1 at both column residues.
    // With S == 2 the two words of (f, gr) are one 8-byte store: half hi of
    // chunk 4 (f & 1) + gr.
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const int swz = out_swz<S>(ocl), hsw = out_half<S>(ocl);
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int gr = 0; gr < 4; ++gr) {
        uint32_t wd[S];
#pragma unroll
        for (int h = 0; h < S; ++h) {
          wd[h] = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int e = S == 2 ? 2 * h + (b >> 1) : b;
            const int g = S == 2 ? (b & 1) : 0;
            wd[h] = requant_u8<RELU>(acc[g][f][4 * gr + e] - zw[g], sc, bi, a.rq, ozp128, qmin128,
                                     b, wd[h]);
          }
          wd[h] ^= 0x80808080u;
        }
        int8_t* rowp = os + (ocl * OROWS + (f >> 1) * S + RH) * OPITCH;
        if constexpr (S == 2) {
          *reinterpret_cast<v2u*>(rowp + 16 * ((4 * (f & 1) + gr) ^ swz) + 8 * (hi ^ hsw)) =
              v2u{wd[0], wd[1]};
        } else {
          *reinterpret_cast<uint32_t*>(rowp + (f & 1) * 32 + 8 * gr + 4 * hi) = wd[0];
        }
      }
    // The wave reads back only rows it wrote: its LDS operations run in
    // order, so no workgroup barrier is needed.
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // copy the wave's rows out: 16-byte pieces of whole rows (piece, then
    // channel, then row)
    for (int u = lane; u < 32 * kTR * PIECES; u += 64) {
      const int pc = u % PIECES;
      const int ocq = 32 * og + (u / PIECES) % 32;
      const int orow = (u / (PIECES * 32)) * S + RH;
      const int occ2 = oc0 + ocq, oh = oh0 + orow, ow = ow0 + 16 * pc;
      if (occ2 >= OC || oh >= H_out || ow >= W_out) continue;
      v4i v = *reinterpret_cast<const v4i*>(os + (ocq * OROWS + orow) * OPITCH +
                                            16 * (pc ^ out_swz<S>(ocq)));
      if (out_half<S>(ocq)) v = v4i{v[2], v[3], v[0], v[1]};
      int8_t* g_ = a.out + (((int64_t)n * OC + occ2) * H_out + oh) * W_out + ow;
      if (p.out_vec && ow + 16 <= W_out) {
        *reinterpret_cast<v4i*>(g_) = v;
      } else {
        for (int e = 0; e < 16 && ow + e < W_out; ++e) g_[e] = (int8_t)(v[e >> 2] >> (8 * (e & 3)));
      }
    }
  };
  if constexpr (SPLIT) {
    if (wave < 4) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, -1>{});
  }
}

template <int S, int K, int PM, bool FWD>
bool plan_t(const DeconvArgs& a, FxPlan& p, size_t& lds) {
  constexpr Pattern<S, K, PM, FWD> P{};
  p = FxPlan{};
  p.base_h = FWD ? -(int)a.ph : (int)(a.ph - PM) / S;
  p.base_w = FWD ? -(int)a.pw : (int)(a.pw - PM) / S;
  const int dwmin = P.dwmin + p.base_w;
  p.coff = ((dwmin % 4) + 4) % 4;
  p.HR = P.dhmax - P.dhmin + kTR;
  p.HC = (p.coff + kTJ + P.dwmax - P.dwmin + 7) / 8 * 8;
  const int64_t NQ = a.IC / 16;
  if (p.HR * NQ * (p.HC / 4) > (int64_t)kStageUnits) return false;
  p.Hp = (int)((a.H_out + S - 1) / S);
  p.Wp = (int)((a.W_out + S - 1) / S);
  p.tiles_i = (p.Hp + kTR - 1) / kTR;
  p.tiles_j = (p.Wp + kTJ - 1) / kTJ;
  p.tiles_oc = (int)((a.OC + kOCB - 1) / kOCB);
  p.out_vec = (a.W_out % 16 == 0) && (((uintptr_t)a.out & 15) == 0);
  const int64_t blocks = (int64_t)a.N * p.tiles_i * p.tiles_j * p.tiles_oc;
  p.xcd = blocks % 8 == 0;
  lds = (size_t)p.HR * NQ * p.HC * 16 + (size_t)kOCB * kTR * S * out_pitch<S>();
  return blocks < ((int64_t)1 << 31) && lds <= 160 * 1024;
}

template <int S, int K, int PM, bool FWD, bool XF, bool PKW = false>
hipError_t launch_x(const DeconvArgs& a, const FxPlan& p, size_t lds, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    for (const void* f : {(const void*)k_deconv_fixed<S, K, PM, FWD, XF, false, PKW>,
                          (const void*)k_deconv_fixed<S, K, PM, FWD, XF, true, PKW>}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
    }
    attr = true;
  }
  const int64_t blocks = (int64_t)a.N * p.tiles_i * p.tiles_j * p.tiles_oc;
  if (a.rq.qmin > -128.0f)
    hipLaunchKernelGGL((k_deconv_fixed<S, K, PM, FWD, XF, true, PKW>), dim3((unsigned)blocks),
                       dim3(threads_of<S>()), lds, s, a, p);
  else
    hipLaunchKernelGGL((k_deconv_fixed<S, K, PM, FWD, XF, false, PKW>), dim3((unsigned)blocks),
                       dim3(threads_of<S>()), lds, s, a, p);
  return hipGetLastError();
}

template <int S, int K, int PM, bool FWD>
hipError_t launch_t(const DeconvArgs& a, hipStream_t s) {
  FxPlan p;
  size_t lds = 0;
  if (!plan_t<S, K, PM, FWD>(a, p, lds)) return hipErrorInvalidValue;
  if constexpr (!FWD) {
    if (a.wpk)
      return a.xf ? launch_x<S, K, PM, FWD, true, true>(a, p, lds, s)
                  : launch_x<S, K, PM, FWD, false, true>(a, p, lds, s);
    if (a.xf) return launch_x<S, K, PM, FWD, true>(a, p, lds, s);
  }
  return launch_x<S, K, PM, FWD, false>(a, p, lds, s);
}

// Which instance takes a shape: 0 = none.
int pick(const DeconvArgs& a, bool fwd) {
  if (a.groups != 1 || a.dil_h != 1 || a.dil_w != 1 || a.Kh != a.Kw) return 0;
  if (a.IC % 64 != 0 || a.IC > 4096 || a.ldw % 16 != 0 || ((uintptr_t)a.w & 15) != 0) return 0;
  // int8 input: 4-byte words of 4 pixels; fp32 input (fused quantize, the
  // transposed conv only): 16-byte loads of 4 pixels
  if (a.W_in % 4 != 0) return 0;
  if (a.xf ? (fwd || ((uintptr_t)a.xf & 15) != 0) : ((uintptr_t)a.x & 3) != 0) return 0;
  if (a.OC > (1 << 20) || a.H_out > (1 << 20) || a.W_out > (1 << 20) || a.H_in > (1 << 20) ||
      a.W_in > (1 << 20) || a.N > (1 << 20) || a.ph > 4096 || a.pw > 4096)
    return 0;
  if (fwd) {
    if (a.sh != 1 || a.sw != 1 || a.Kh != 3) return 0;
    return 1;
  }
  if (a.sh != 2 || a.sw != 2 || (a.ph % 2) != (a.pw % 2)) return 0;
  if (a.Kh == 3) return a.ph % 2 ? 2 : 3;
  if (a.Kh == 4) return a.ph % 2 ? 4 : 5;
  return 0;
}

hipError_t launch_pick(const DeconvArgs& a, int k, hipStream_t s) {
  switch (k) {
    case 1: return launch_t<1, 3, 0, true>(a, s);
    case 2: return launch_t<2, 3, 1, false>(a, s);
    case 3: return launch_t<2, 3, 0, false>(a, s);
    case 4: return launch_t<2, 4, 1, false>(a, s);
    case 5: return launch_t<2, 4, 0, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

bool fits(const DeconvArgs& a, int k) {
  FxPlan p;
  size_t lds;
  switch (k) {
    case 1: return plan_t<1, 3, 0, true>(a, p, lds);
    case 2: return plan_t<2, 3, 1, false>(a, p, lds);
    case 3: return plan_t<2, 3, 0, false>(a, p, lds);
    case 4: return plan_t<2, 4, 1, false>(a, p, lds);
    case 5: return plan_t<2, 4, 0, false>(a, p, lds);
    default: return false;
  }
}

}  // namespace

namespace {

// The prepacked transposed-conv weight: one 16-byte piece per thread;
// fragment ((ob * Kh + kh) * Kw + kw) * (IC / 32) + kc, lane l: row
// 32 ob + l % 32, bytes (kh * Kw + kw) * IC + 32 kc + 16 (l / 32) .. +15 of
// that row; rows past OC are zero.
__global__ __launch_bounds__(256) void k_deconv_wprepack(const int8_t* __restrict__ w, int64_t ldw,
                                                         int OC, int IC, int taps, int64_t total,
                                                         int8_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int nk = IC / 32;
  const int l = (int)(t & 63);
  const int64_t fi = t >> 6;
  const int kc = (int)(fi % nk);
  const int tap = (int)((fi / nk) % taps);
  const int64_t row = 32 * (fi / ((int64_t)nk * taps)) + (l & 31);
  v4i v = {0, 0, 0, 0};
  if (row < OC)
    v = *reinterpret_cast<const v4i*>(w + row * ldw + (int64_t)tap * IC + 32 * kc + 16 * (l >> 5));
  *reinterpret_cast<v4i*>(out + 16 * t) = v;
}

}  // namespace

int64_t deconv_prepacked_bytes(int64_t OC, int64_t IC, int64_t Kh, int64_t Kw) {
  return (OC + 31) / 32 * 32 * Kh * Kw * IC;
}

hipError_t launch_deconv_wprepack(const int8_t* w, int64_t OC, int64_t IC, int64_t Kh, int64_t Kw,
                                  int64_t ldw, int8_t* packed, hipStream_t s) {
  const int64_t total = deconv_prepacked_bytes(OC, IC, Kh, Kw) / 16;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(k_deconv_wprepack, dim3((unsigned)blocks), dim3(256), 0, s, w, ldw, (int)OC,
                     (int)IC, (int)(Kh * Kw), total, packed);
  return hipGetLastError();
}

bool deconv_fixed_supported(const DeconvArgs& a) {
  const int k = pick(a, false);
  return k && fits(a, k);
}

// The default choice for shapes with at least one workgroup per CU (256 tiles
// of two phase rows x 64 columns x 128 channels); smaller problems are
// latency-bound and run faster on the tiled 16x16x64 kernel.
bool deconv_fixed_preferred(const DeconvArgs& a) {
  if (!deconv_fixed_supported(a)) return false;
  const int64_t Hp = (a.H_out + 1) / 2, Wp = (a.W_out + 1) / 2;
  const int64_t tiles = a.N * ((Hp + kTR - 1) / kTR) * ((Wp + kTJ - 1) / kTJ) * ((a.OC + kOCB - 1) / kOCB);
  return tiles >= 256;
}

bool conv_fixed_supported(const DeconvArgs& a) {
  const int k = pick(a, true);
  return k && fits(a, k);
}

hipError_t launch_deconv_fixed(const DeconvArgs& a, hipStream_t s) {
  return launch_pick(a, pick(a, false), s);
}

hipError_t launch_conv_fixed(const DeconvArgs& a, hipStream_t s) {
  return launch_pick(a, pick(a, true), s);
}

}  // namespace q8ta
