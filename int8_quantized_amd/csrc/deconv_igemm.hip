// q8ta_conv2d_transposed as an implicit GEMM on the vector ALU ("Add
// q8ta_conv2d_transposed op", Solution: acc[n,oc,oh,ow] = sum over (ic, kh,
// kw) of (x[n,ic,ih,iw] - izp) * w[oc, (kh*Kw + kw)*IC + ic], with ih = (oh +
// pad_h - kh) / stride_h used only when the numerator is >= 0, divisible and
// ih < H_in; iw likewise), for IC a multiple of 64.
//
// Stride phases: for output rows oh = rh + s_h*i and columns ow = rw + s_w*j,
// the qualifying taps (kh, kw) depend only on (rh, rw) and read input pixel
// (i + dh, j + dw) with fixed offsets (dh, dw).  Each phase is therefore a
// GEMM: rows = the phase's output pixels, columns = output channels, K = the
// phase's taps x IC, where the K-vector of pixel (i, j) at tap (kh, kw) is the
// channel vector of input pixel (i + dh, j + dw).  The input is first copied
// to NHWC (channels innermost) in a stream-ordered workspace, with a border of
// pixels whose every byte is the input zero point wide enough for every
// (i + dh, j + dw) a tile can form: so every load is unconditional and in
// bounds, and a tap that falls outside the input reads the zero point
// (zero-point fill).  The weights are already [OC, (kh*Kw + kw)*IC + ic],
// contiguous in ic per tap.
//
// Register tiling as in the linear's grouped kernel: groups of LPG = 4 lanes
// (inside one DPP row) own an 8 x 8 tile (8 pixels of one phase row, 8 output
// channels) and split each 64-byte K slice (lane l reads bytes 16 l .. 16 l +
// 15); 16 groups, 4 along the pixels and 4 along the channels, make a wave tile
// of 32 consecutive phase columns of one phase row by 32 output channels.  The
// weight-row pointers of a tap are wave-uniform (scalar registers); pixel rows
// use one wave-uniform pointer and a 32-bit lane offset per row.  With sum w
// taken over all of the phase's taps, sum x'*w - izp * sum w (x' = x with the
// zero-point border) equals the gather over the qualifying in-range taps (the
// pages' Constraints (1) fold).  A pre-pass forms sum w per (phase,
// output channel).  After the K loop a two-step DPP butterfly leaves each lane
// with 2 pixels x 8 channels, which it requantizes and stores (NCHW bytes).
//
// Blocks are 2 x 2 waves (2 phase rows x 64 output channels); the grid lists
// every phase's blocks one after the other (phase offsets in `off`).
#include <cstdlib>
#include <cstring>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

constexpr int kThreads = 256;
constexpr int kSlice = 64;         // largest K slice (4 lanes x 16 bytes): IC % kSlice == 0
constexpr int kMaxPhases = kMaxS * kMaxS;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) v4i* vptr;

struct Plan {
  int off[kMaxPhases + 1];  // first block of each phase; off[nph] = grid size
  int nph;
  int pt, pl;               // zero-point border above / left of the input
  int Hpad, Wpad;           // padded NHWC height / width
  // Geometry: phase (rh, rw) holds output pixels (rh + osh*i, rw + osw*j), and
  // tap t of its row list reads input row i*ish + thd[rh][t] (columns
  // likewise).  Transposed conv: osh/osw = stride, ish/isw = 1; forward conv:
  // one phase, osh/osw = 1, ish/isw = stride.
  int osh, osw, ish, isw;
};

// x NCHW -> xp, NHWC inside a zero-point border: xp[n][hp][wp][c] =
// x[n][c][hp - pt][wp - pl] inside the input, the zero-point byte outside (with
// xf set, the fp32 input quantized on the way: quantize_per_tensor fused).  16
// channels per thread: 16 byte loads (each load instruction reads 64
// consecutive columns of one channel plane) packed into one 16-byte store.  t
// enumerates (n, hp, g, wp) with wp fastest.
__device__ __forceinline__ void relayout_one(const int8_t* __restrict__ x,
                                             const float* __restrict__ xf, float inv_in,
                                             int8_t* __restrict__ xp, int64_t N, int C, int H,
                                             int W, const Plan& plan, int zp, int64_t t) {
  const int G = C / 16;
  if (t >= N * plan.Hpad * G * plan.Wpad) return;
  const int wp = (int)(t % plan.Wpad);
  int64_t r = t / plan.Wpad;
  const int g = (int)(r % G);
  r /= G;
  const int hp = (int)(r % plan.Hpad);
  const int64_t n = r / plan.Hpad;
  const int h = hp - plan.pt, w = wp - plan.pl;
  uint32_t d[4];
  if (h >= 0 && h < H && w >= 0 && w < W) {
    const int64_t plane = (int64_t)H * W;
    const int64_t off = (n * C + g * 16) * plane + (int64_t)h * W + w;
    if (xf) {  // fused quantize of the fp32 input
      const float* src = xf + off;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b)
          v |= (uint32_t)(quantize1(src[(q * 4 + b) * plane], inv_in, (float)zp) & 0xff) << (8 * b);
        d[q] = v;
      }
    } else {
      const int8_t* src = x + off;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= (uint32_t)(uint8_t)src[(q * 4 + b) * plane] << (8 * b);
        d[q] = v;
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = 0x01010101u * ((uint32_t)zp & 0xffu);
  }
  *reinterpret_cast<v4i*>(xp + ((n * plan.Hpad + hp) * plan.Wpad + wp) * C + g * 16) =
      v4i{(int)d[0], (int)d[1], (int)d[2], (int)d[3]};
}

// wsum[ph * OC + oc] = sum over the phase's taps and all ic of w[oc, tap, ic]:
// one wave per (phase, channel), lanes split the (tap, ic) words.
__device__ __forceinline__ void phase_wsum_one(const DeconvArgs& a, const Phases& p,
                                               const Plan& plan, int32_t* __restrict__ wsum,
                                               int64_t id) {
  const int lane = threadIdx.x & 63;
  if (id >= (int64_t)plan.nph * a.OC) return;
  const int ph = (int)(id / a.OC);
  const int64_t oc = id % a.OC;
  const int rh = ph / plan.osw, rw = ph % plan.osw;
  const int IC = (int)a.IC;
  int32_t s = 0;
  for (int th = 0; th < p.nth[rh]; ++th)
    for (int tw = 0; tw < p.ntw[rw]; ++tw) {
      const int8_t* row = a.w + oc * a.ldw + (int64_t)(p.thk[rh][th] * a.Kw + p.twk[rw][tw]) * IC;
      for (int c = lane * 4; c < IC; c += 256)
        s = __builtin_amdgcn_sdot4(*reinterpret_cast<const int32_t*>(row + c), 0x01010101, s,
                                   false);
    }
  s = wave_total(s);
  if (lane == 0) wsum[id] = s;
}

// One launch for both preparations: blocks below `relayout_blocks` copy the
// input, the others form the weight sums (one wave per (phase, channel)).
__global__ __launch_bounds__(kThreads) void k_prep(DeconvArgs a, Phases p, Plan plan,
                                                   int8_t* __restrict__ xp,
                                                   int32_t* __restrict__ wsum,
                                                   int64_t relayout_blocks) {
  const int64_t b = blockIdx.x;
  if (b < relayout_blocks) {
    relayout_one(a.x, a.xf, a.inv_in, xp, a.N, (int)a.IC, (int)a.H_in, (int)a.W_in, plan,
                 (int)a.izp, b * kThreads + threadIdx.x);
  } else {
    const int64_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    phase_wsum_one(a, p, plan, wsum, (b - relayout_blocks) * (kThreads / 64) + wave);
  }
}

// Groups of LPG lanes (LPG = 4: 64-byte K slices, two butterfly steps; the
// code also holds LPG = 1: 16-byte slices, no butterfly), GM groups along the
// pixels and 64/LPG/GM along the channels.  FULL_OC: OC is a multiple of the wave's
// channel count, so every weight row a running wave reads exists and no load
// is masked.
template <bool FULL_OC, int LPG, int GM>
__global__ __launch_bounds__(kThreads) void k_deconv_igemm(DeconvArgs a, Phases p, Plan plan,
                                                           const int8_t* __restrict__ xp,
                                                           const int32_t* __restrict__ wsum) {
  constexpr int GN = 64 / LPG / GM;
  constexpr int WJ = 8 * GM, WO = 8 * GN;  // wave tile: WJ phase columns x WO channels
  constexpr int V = 64 / LPG;              // values per lane after the butterfly
  constexpr int SL = LPG * 16;             // K bytes per slice
  static_assert(GM * GN * LPG == 64, "group layout");
  const int lane = threadIdx.x & 63;
  const int lg = lane % LPG;
  const int grp = lane / LPG;
  const int gm = grp % GM, gn = grp / GM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // block -> phase, then (ob fastest, jb, ib, n) inside the phase
  const int b = (int)blockIdx.x;
  int ph = 0;
  while (ph + 1 < plan.nph && plan.off[ph + 1] <= b) ++ph;
  const int osh = plan.osh, osw = plan.osw;
  const int rh = ph / osw, rw = ph % osw;
  const int Hp = ((int)a.H_out - rh + osh - 1) / osh;
  const int Wp = ((int)a.W_out - rw + osw - 1) / osw;
  const int OB = ((int)a.OC + 2 * WO - 1) / (2 * WO);
  const int JB = (Wp + WJ - 1) / WJ;
  const int IB = (Hp + 1) / 2;
  int local = b - plan.off[ph];
  const int ob = local % OB;
  local /= OB;
  const int jb = local % JB;
  local /= JB;
  const int ib = local % IB;
  const int64_t n = local / IB;
  const int i = ib * 2 + (wave & 1);
  const int oc0w = ob * 2 * WO + WO * (wave >> 1);
  const int j0w = jb * WJ;
  if (i >= Hp || oc0w >= a.OC) return;  // wave-uniform

  const int IC = (int)a.IC;
  const int jg = j0w + 8 * gm;              // first pixel column of this lane's group
  const int oc0 = oc0w + 8 * gn;            // first channel of this lane's group
  const int nrem = (int)a.OC - oc0;         // channel rows r < nrem exist
  // lane offset of pixel row r inside the tap's window of WJ pixels
  uint32_t xoff[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) xoff[r] = (uint32_t)((8 * gm + r) * plan.isw * IC + 16 * lg);
  const uint32_t woff = (uint32_t)(8 * gn) * (uint32_t)a.ldw + (uint32_t)(16 * lg);

  int32_t acc[64];
#pragma unroll
  for (int q = 0; q < 64; ++q) acc[q] = 0;

  for (int th = 0; th < p.nth[rh]; ++th) {
    const int kh = p.thk[rh][th];
    const int64_t hp = (int64_t)i * plan.ish + p.thd[rh][th] + plan.pt;  // padded row, in range
    for (int tw = 0; tw < p.ntw[rw]; ++tw) {
      const int kw = p.twk[rw][tw];
      const int64_t wp0 = (int64_t)j0w * plan.isw + p.twd[rw][tw] + plan.pl;  // of pixel j0w
      const gptr xr = uniform_ptr(xp + ((n * plan.Hpad + hp) * plan.Wpad + wp0) * IC);
      const int8_t* wu = a.w + (int64_t)oc0w * a.ldw + (int64_t)(kh * a.Kw + kw) * IC;
      gptr wr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        wr[r] = uniform_ptr(wu + (int64_t)r * a.ldw);
        asm volatile("" : "+s"(wr[r]));
      }
      for (int c0 = 0; c0 < IC; c0 += SL) {
        const uint32_t ku = __builtin_amdgcn_readfirstlane((uint32_t)c0);
        const uint32_t wo = woff + ku;
        v4i xs[8], ws[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
          ws[r] = (FULL_OC || r < nrem) ? *reinterpret_cast<vptr>(wr[r] + wo) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 8; ++r) xs[r] = *reinterpret_cast<vptr>(xr + (xoff[r] + ku));
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int m = 0; m < 8; ++m) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
              acc[m * 8 + c] = __builtin_amdgcn_sdot4(xs[m][d], ws[c][d], acc[m * 8 + c], false);
          }
        }
      }
    }
  }
  if constexpr (LPG > 1) reduce_group<LPG>(acc, lg);

  // acc[q] = tile element e = V*lg + q (pixel row e / 8, channel e % 8): R rows
  // of C consecutive channels, starting at row m0l and channel c0l.
  constexpr int R = V >= 8 ? V / 8 : 1;
  constexpr int C = V >= 8 ? 8 : V;
  const int m0l = (V * lg) >> 3, c0l = (V * lg) & 7;
  const int64_t plane = a.H_out * a.W_out;
  const int64_t oh = rh + (int64_t)osh * i;
  const int32_t* wsp = wsum + (int64_t)ph * a.OC;
#pragma unroll
  for (int h = 0; h < R; ++h) {
    const int j = jg + m0l + h;
    if (j >= Wp) continue;
    // output index of (n, channel, oh, ow); the next channel is one plane further
    int64_t o = ((n * a.OC + oc0 + c0l) * a.H_out + oh) * a.W_out + rw + (int64_t)osw * j;
#pragma unroll
    for (int t = 0; t < C; ++t, o += plane) {
      const int oc = oc0 + c0l + t;
      if (!FULL_OC && oc >= a.OC) break;
      const int32_t c = acc[h * C + t] - a.izp * wsp[oc];
      if (a.acc) {
        a.acc[o] = c;
      } else {
        const float bv = a.bias ? a.bias[oc] : 0.0f;
        a.out[o] = (int8_t)requant(c, a.wscale[oc], bv, a.rq);
      }
    }
  }
}

// Tile counts per phase, block offsets and the zero-point border, for the
// geometry (osh, osw, ish, isw) described at Plan.
bool make_plan(const DeconvArgs& a, const Phases& p, int osh, int osw, int ish, int isw, int WJ,
               int WO, Plan& plan, int64_t& blocks) {
  plan = Plan{};
  plan.osh = osh;
  plan.osw = osw;
  plan.ish = ish;
  plan.isw = isw;
  plan.nph = osh * osw;
  if (plan.nph > kMaxPhases) return false;
  blocks = 0;
  int64_t lo_h = 0, hi_h = a.H_in - 1, lo_w = 0, hi_w = a.W_in - 1;
  for (int ph = 0; ph < plan.nph; ++ph) {
    const int rh = ph / osw, rw = ph % osw;
    const int64_t Hp = (a.H_out - rh + osh - 1) / osh, Wp = (a.W_out - rw + osw - 1) / osw;
    const int64_t JB = (Wp + WJ - 1) / WJ;
    plan.off[ph] = (int)blocks;
    blocks += a.N * ((Hp + 1) / 2) * JB * ((a.OC + 2 * WO - 1) / (2 * WO));
    if (blocks >= ((int64_t)1 << 31) - 1) return false;
    if (Hp > 0)
      for (int th = 0; th < p.nth[rh]; ++th) {
        const int64_t d = p.thd[rh][th], last = (Hp - 1) * ish + d;
        lo_h = lo_h < d ? lo_h : d;
        hi_h = hi_h > last ? hi_h : last;
      }
    if (Wp > 0)
      for (int tw = 0; tw < p.ntw[rw]; ++tw) {
        const int64_t d = p.twd[rw][tw], last = (JB * WJ - 1) * isw + d;
        lo_w = lo_w < d ? lo_w : d;
        hi_w = hi_w > last ? hi_w : last;
      }
  }
  plan.off[plan.nph] = (int)blocks;
  if (hi_h - lo_h + 1 >= (1 << 30) || hi_w - lo_w + 1 >= (1 << 30)) return false;
  plan.pt = (int)-lo_h;
  plan.pl = (int)-lo_w;
  plan.Hpad = (int)(hi_h - lo_h + 1);
  plan.Wpad = (int)(hi_w - lo_w + 1);
  // the bordered copy stays within a few times the input (large padding or
  // dilation takes the other kernels)
  if ((double)plan.Hpad * plan.Wpad > 4.0 * ((double)a.H_in + 64) * ((double)a.W_in + 64))
    return false;
  // 32-bit lane offsets: pixel rows reach (WJ - 1) * isw * IC + IC bytes
  if ((double)WJ * isw * a.IC >= (double)((int64_t)1 << 31)) return false;
  return true;
}

// Forward conv as one phase: every tap qualifies; tap kh reads input row
// oh*stride_h + kh*dil_h - pad_h.
bool make_conv_phases(const DeconvArgs& a, Phases& p) {
  if (a.Kh > kMaxT || a.Kw > kMaxT) return false;
  p = Phases{};
  p.nth[0] = (int)a.Kh;
  for (int k = 0; k < (int)a.Kh; ++k) {
    p.thk[0][k] = k;
    p.thd[0][k] = (int)(k * a.dil_h - a.ph);
  }
  p.ntw[0] = (int)a.Kw;
  for (int k = 0; k < (int)a.Kw; ++k) {
    p.twk[0][k] = k;
    p.twd[0][k] = (int)(k * a.dil_w - a.pw);
  }
  return true;
}

bool igemm_shape_ok(const DeconvArgs& a) {
  if (a.IC % kSlice != 0 || a.ldw % 16 != 0 || ((uintptr_t)a.w & 15) != 0) return false;
  // 32-bit lane offsets (< 32 * ldw) and 32-bit tile counters
  return a.IC < (1 << 25) && a.ldw < (1 << 25) && a.H_out < (1 << 30) && a.W_out < (1 << 30) &&
         a.H_in < (1 << 30) && a.W_in < (1 << 30) && a.OC < (1 << 30);
}

}  // namespace

bool deconv_igemm_supported(const DeconvArgs& a) {
  Phases p;
  Plan plan;
  int64_t blocks;
  const int sh = (int)a.sh, sw = (int)a.sw;
  return a.groups == 1 && igemm_shape_ok(a) && make_phases(a, p) &&
         make_plan(a, p, sh, sw, 1, 1, 32, 32, plan, blocks) &&
         make_plan(a, p, sh, sw, 1, 1, 64, 16, plan, blocks);
}

bool conv_igemm_supported(const DeconvArgs& a) {
  Phases p;
  Plan plan;
  int64_t blocks;
  if (a.groups != 1 || a.sh > 4096 || a.sw > 4096 || a.dil_h > 4096 || a.dil_w > 4096) return false;
  const int sh = (int)a.sh, sw = (int)a.sw;
  return igemm_shape_ok(a) && make_conv_phases(a, p) &&
         make_plan(a, p, 1, 1, sh, sw, 32, 32, plan, blocks) &&
         make_plan(a, p, 1, 1, sh, sw, 64, 16, plan, blocks);
}

namespace {

template <int LPG, int GM>
hipError_t launch_igemm_t(const DeconvArgs& a, const Phases& p, int osh, int osw, int ish,
                          int isw, hipStream_t s) {
  constexpr int GN = 64 / LPG / GM;
  constexpr int WJ = 8 * GM, WO = 8 * GN;
  Plan plan;
  int64_t blocks;
  if (!make_plan(a, p, osh, osw, ish, isw, WJ, WO, plan, blocks)) return hipErrorInvalidValue;
  const size_t xbytes = (size_t)a.N * plan.Hpad * plan.Wpad * a.IC;
  const size_t xpad = (xbytes + 255) / 256 * 256;
  const size_t wsbytes = (size_t)plan.nph * (size_t)a.OC * sizeof(int32_t);
  void* ws = nullptr;
  hipError_t e = workspace_acquire(&ws, xpad + wsbytes, s);
  if (e != hipSuccess) return e;
  int8_t* xp = (int8_t*)ws;
  int32_t* wsum = (int32_t*)((char*)ws + xpad);
  const int64_t t = a.N * plan.Hpad * (a.IC / 16) * plan.Wpad;
  const int64_t rblocks = (t + kThreads - 1) / kThreads;
  const int64_t wblocks = ((int64_t)plan.nph * a.OC + kThreads / 64 - 1) / (kThreads / 64);
  hipLaunchKernelGGL(k_prep, dim3((unsigned)(rblocks + wblocks)), dim3(kThreads), 0, s, a, p,
                     plan, xp, wsum, rblocks);
  e = hipGetLastError();
  if (e == hipSuccess && blocks > 0) {
    if (a.OC % WO == 0)
      hipLaunchKernelGGL((k_deconv_igemm<true, LPG, GM>), dim3((unsigned)blocks), dim3(kThreads),
                         0, s, a, p, plan, (const int8_t*)xp, (const int32_t*)wsum);
    else
      hipLaunchKernelGGL((k_deconv_igemm<false, LPG, GM>), dim3((unsigned)blocks), dim3(kThreads),
                         0, s, a, p, plan, (const int8_t*)xp, (const int32_t*)wsum);
    e = hipGetLastError();
  }
  hipError_t f = workspace_release(ws, s);
  return e != hipSuccess ? e : f;
}

}  // namespace

// NHWC copy of the input inside its zero-point border and sum w per (phase,
// channel) in one stream-ordered workspace, then the implicit GEMM over every
// phase (4 x 4 groups of 4 lanes: a 32 x 32 wave tile).
hipError_t launch_deconv_igemm(const DeconvArgs& a, hipStream_t s) {
  Phases p;
  if (!make_phases(a, p)) return hipErrorInvalidValue;
  const int sh = (int)a.sh, sw = (int)a.sw;
  return launch_igemm_t<4, 4>(a, p, sh, sw, 1, 1, s);
}

// The forward conv through the same kernels: one phase, every tap.
hipError_t launch_conv_igemm(const DeconvArgs& a, hipStream_t s) {
  Phases p;
  if (!make_conv_phases(a, p)) return hipErrorInvalidValue;
  const int sh = (int)a.sh, sw = (int)a.sw;
  return launch_igemm_t<4, 4>(a, p, 1, 1, sh, sw, s);
}

}  // namespace q8ta
