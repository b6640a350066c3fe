// q8ta_linear for M > 4 on the vector ALU: a register-tiled int8 GEMM built
// on the packed dot-product instruction v_dot4 ("Add q8ta_linear op",
// Solution: acc[m,n] = sum_k (x[m,k] - izp) * w[n,k] in int32, then the
// per-channel epilogue).
//
// The 64 lanes of a wave form 64/LPG groups of LPG lanes (LPG = 16, 8 or 4,
// each group inside one DPP row).  A group owns an 8 x 8 output tile (8
// activation rows, 8 weight rows); the groups of a wave are arranged GM along
// M by 64/LPG/GM along N.  The LPG lanes of a group split K: in one slice lane
// l reads 4*LW bytes at byte 4*LW*l of an LPG*4*LW-byte stretch of each of its
// 16 rows and accumulates the 64 partial dot products of the tile with v_dot4.
// All row pointers are wave-uniform (scalar registers); each load adds one
// 32-bit lane offset, so a slice costs 16 load instructions, 2 vector adds and
// 64*LW v_dot4.
//
// At the end the 64 partials of a lane are summed over the LPG lanes of its
// group with a transposing butterfly: at each step a lane keeps half of its
// values, receives its partner's copy of that half through a DPP lane move
// inside the row (mirror of 16, mirror of 8, quad reverse, quad swap: lane
// masks 15, 7, 3, 1, which span the group) and adds it.  After log2(LPG) steps
// lane l holds tile elements 64/LPG*l .. +64/LPG-1 (row-major 8 x 8), i.e.
// consecutive output channels of one or two activation rows, which it
// requantizes and stores as whole 32-bit words.
//
// The zero-point term is folded as sum x*w - izp*sum w, with the row sums of
// W formed by a small pass over W before the GEMM (one wave per row, v_dot4
// against 0x01010101) into a stream-ordered workspace.
//
// The 4 waves of a block cover a 2 x 2 group of wave tiles (rows shared by two
// waves are served from the CU's cache).  Blocks are dispatched round-robin to
// the 8 XCDs; with XCD strips, block b is mapped so that XCD b % 8 owns a
// contiguous strip of block-columns (each weight row is fetched into one L2),
// and block-rows are walked in groups of GROUP so that the blocks resident at
// a time touch a compact set of activation rows.
#include <cstdlib>
#include <cstring>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

constexpr int kThreads = 256;

template <int LW>
struct Vec;
template <>
struct Vec<2> {
  typedef int type __attribute__((ext_vector_type(2)));
};
template <>
struct Vec<4> {
  typedef int type __attribute__((ext_vector_type(4)));
};

// One slice of a group's 8 weight rows and 8 activation rows.
template <int LW>
struct Slice {
  typename Vec<LW>::type w[8], x[8];
};

// sum_k w[n, k] for every weight row: one wave per row, lanes split K, v_dot4
// against 0x01010101, then a reduction across the wave.
__global__ __launch_bounds__(kThreads) void k_row_sums(const int8_t* __restrict__ w, int64_t N,
                                                       int64_t K, int32_t* __restrict__ out) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (n >= N) return;
  int32_t s = 0;
  for (int64_t k = (int64_t)lane * 16; k < K; k += 1024) {
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(w + n * K + k));
#pragma unroll
    for (int d = 0; d < 4; ++d) s = __builtin_amdgcn_sdot4(v[d], 0x01010101, s, false);
  }
  s = wave_total(s);
  if (lane == 0) out[n] = s;
}

// ---------------------------------------------------------------------------
// Loads one slice for a group: row r of the weights is read at
// p.w[r] + (woff + k) and row m of the activations at p.x[m] + (xoff + k):
// the row pointers are wave-uniform (scalar registers) and the
// 32-bit lane offset holds the group's row offset, the lane's byte offset in
// the slice and the slice start k, so every load is one scalar-base plus
// 32-bit-offset instruction.  k passes through readfirstlane so that the
// loop does not turn the offsets into per-row 64-bit induction variables.
// Unless FULL, rows at or past nrem / mrem (counted from the group's first
// row) and lanes with `kin` false read zeros.
// Row pointers of a wave's 8 weight rows and 8 activation rows (wave-uniform,
// kept in scalar registers; the empty asm makes each one opaque so that the
// compiler does not fold the lane offset into a per-row 64-bit vector add).
struct RowPtrs {
  gptr w[8], x[8];
};

__device__ __forceinline__ void row_ptrs(RowPtrs& p, gptr wu, gptr xu, int64_t K) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    p.w[r] = wu + r * K;
    p.x[r] = xu + r * K;
    asm volatile("" : "+s"(p.w[r]));
    asm volatile("" : "+s"(p.x[r]));
  }
}

template <bool FULL, int LW>
__device__ __forceinline__ void load_slice_g(Slice<LW>& s, const RowPtrs& p, uint32_t woff,
                                             uint32_t xoff, int64_t k, bool kin, int64_t nrem,
                                             int64_t mrem) {
  typedef typename Vec<LW>::type V;
  typedef const __attribute__((address_space(1))) V* vptr;
  const uint32_t ku = __builtin_amdgcn_readfirstlane((uint32_t)k);
  const uint32_t wo = woff + ku, xo = xoff + ku;
#pragma unroll
  for (int r = 0; r < 8; ++r)
    s.w[r] = (FULL || (kin && r < nrem)) ? *reinterpret_cast<vptr>(p.w[r] + wo) : V{};
#pragma unroll
  for (int m = 0; m < 8; ++m)
    s.x[m] = (FULL || (kin && m < mrem)) ? *reinterpret_cast<vptr>(p.x[m] + xo) : V{};
}

// acc[m * 8 + n] += x row m . w row n over one slice (m, n < 8).
template <int LW>
__device__ __forceinline__ void dot_slice_mn(const Slice<LW>& s, int32_t (&acc)[64]) {
#pragma unroll
  for (int d = 0; d < LW; ++d) {
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int n = 0; n < 8; ++n)
        acc[m * 8 + n] = __builtin_amdgcn_sdot4(s.x[m][d], s.w[n][d], acc[m * 8 + n], false);
    }
  }
}

// Block b covers a (2*8*GM) x (2*8*GN) output tile (4 waves, 2 x 2).
template <int LW, bool PIPE, int LPG, int GM>
__global__ __launch_bounds__(kThreads) void k_dot4_gemm(LinearArgs a, uint32_t BMb, uint32_t BNb,
                                                        uint32_t group, int xcd_strips,
                                                        const int32_t* __restrict__ wsum) {
  constexpr int GN = 64 / LPG / GM;
  constexpr int WM = 8 * GM, WN = 8 * GN;  // wave tile
  constexpr int V = 64 / LPG;               // values per lane after the butterfly
  constexpr int64_t SL = LPG * 4 * LW;      // bytes of one row covered by one slice
  static_assert(GM >= 1 && GN >= 1 && GM * GN * LPG == 64, "group layout");
  const int lane = threadIdx.x & 63;
  const int lg = lane % LPG;
  const int grp = lane / LPG;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t width = xcd_strips ? (BNb + 7) / 8 : BNb;
  const uint32_t b = xcd_strips ? blockIdx.x / 8 : blockIdx.x;
  const uint32_t strip0 = xcd_strips ? (blockIdx.x % 8) * width : 0;
  const uint32_t per_group = group * width;
  const uint32_t g = b / per_group;
  const uint32_t rows_here = (g * group + group <= BMb) ? group : BMb - g * group;
  const uint32_t in_g = b - g * per_group;
  const uint32_t bm_i = g * group + in_g % rows_here;
  const uint32_t bn_i = strip0 + in_g / rows_here;
  if (bn_i >= BNb) return;
  const int64_t m0w = (int64_t)bm_i * (2 * WM) + WM * (wave & 1);
  const int64_t n0w = (int64_t)bn_i * (2 * WN) + WN * (wave >> 1);
  if (m0w >= a.M || n0w >= a.N) return;  // wave-uniform
  const int gm = grp % GM, gn = grp / GM;
  const int64_t m0 = m0w + 8 * gm;
  const int64_t n0 = n0w + 8 * gn;
  const int64_t nrem = a.N - n0, mrem = a.M - m0;
  const uint32_t kl = (uint32_t)(lg * 4 * LW);
  const uint32_t woff = (uint32_t)(8 * gn) * (uint32_t)a.K + kl;
  const uint32_t xoff = (uint32_t)(8 * gm) * (uint32_t)a.K + kl;
  RowPtrs rp;
  row_ptrs(rp, uniform_ptr(a.w + n0w * a.K), uniform_ptr(a.x + m0w * a.K), a.K);

  int32_t acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0;

  const int64_t Kf = a.K - a.K % SL;  // whole slices; the rest is one masked slice
  const bool full = (m0w + WM <= a.M) && (n0w + WN <= a.N);
  if constexpr (PIPE) {
    if (Kf > 0) {
      Slice<LW> s0, s1;
      load_slice_g<false>(s0, rp, woff, xoff, 0, true, nrem, mrem);
      for (int64_t k0 = 0; k0 < Kf; k0 += 2 * SL) {
        if (k0 + SL < Kf) load_slice_g<false>(s1, rp, woff, xoff, k0 + SL, true, nrem, mrem);
        dot_slice_mn(s0, acc);
        if (k0 + SL >= Kf) break;
        if (k0 + 2 * SL < Kf)
          load_slice_g<false>(s0, rp, woff, xoff, k0 + 2 * SL, true, nrem, mrem);
        dot_slice_mn(s1, acc);
      }
    }
  } else if (full) {
    for (int64_t k0 = 0; k0 < Kf; k0 += SL) {
      Slice<LW> s0;
      load_slice_g<true>(s0, rp, woff, xoff, k0, true, nrem, mrem);
      dot_slice_mn(s0, acc);
    }
  } else {
    for (int64_t k0 = 0; k0 < Kf; k0 += SL) {
      Slice<LW> s0;
      load_slice_g<false>(s0, rp, woff, xoff, k0, true, nrem, mrem);
      dot_slice_mn(s0, acc);
    }
  }
  if (Kf < a.K) {
    Slice<LW> s0;
    load_slice_g<false>(s0, rp, woff, xoff, Kf, Kf + kl < a.K, nrem, mrem);
    dot_slice_mn(s0, acc);
  }
  reduce_group<LPG>(acc, lg);

  // acc[t] = tile element e = V*lg + t (row e / 8, channel e % 8), in chunks of
  // C consecutive channels of one row.
  constexpr int C = V < 8 ? V : 8;
#pragma unroll
  for (int c = 0; c < V / C; ++c) {
    const int e = V * lg + C * c;
    const int64_t mm = m0 + (e >> 3);
    const int64_t nb = n0 + (e & 7);
    if (mm >= a.M) continue;
    int32_t cv[C];
#pragma unroll
    for (int t = 0; t < C; ++t) cv[t] = (nb + t < a.N) ? acc[C * c + t] - a.izp * wsum[nb + t] : 0;
    if (a.acc) {
#pragma unroll
      for (int t = 0; t < C; ++t)
        if (nb + t < a.N) a.acc[mm * a.N + nb + t] = cv[t];
      continue;
    }
    int q[C];
#pragma unroll
    for (int t = 0; t < C; ++t) {
      const bool ok = nb + t < a.N;
      const float sc = ok ? a.wscale[nb + t] : 0.0f;
      const float bv = (ok && a.bias) ? a.bias[nb + t] : 0.0f;
      q[t] = requant(cv[t], sc, bv, a.rq);
    }
    if (a.outf) {
      float* of = a.outf + mm * a.N + nb;
      if (nb + C <= a.N && ((uintptr_t)of & 15) == 0) {
        typedef float v4f __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int t = 0; t < C; t += 4)
          *reinterpret_cast<v4f*>(of + t) =
              v4f{dequant1(q[t], a.dq_zp, a.dq_scale), dequant1(q[t + 1], a.dq_zp, a.dq_scale),
                  dequant1(q[t + 2], a.dq_zp, a.dq_scale), dequant1(q[t + 3], a.dq_zp, a.dq_scale)};
      } else {
#pragma unroll
        for (int t = 0; t < C; ++t)
          if (nb + t < a.N) of[t] = dequant1(q[t], a.dq_zp, a.dq_scale);
      }
      continue;
    }
    int8_t* o = a.out + mm * a.N + nb;
    if (nb + C <= a.N && ((uintptr_t)o & 3) == 0) {
#pragma unroll
      for (int t = 0; t < C; t += 4)
        *reinterpret_cast<uint32_t*>(o + t) = pack4(q[t], q[t + 1], q[t + 2], q[t + 3]);
    } else {
#pragma unroll
      for (int t = 0; t < C; ++t)
        if (nb + t < a.N) o[t] = (int8_t)q[t];
    }
  }
}

// Row sums of W into a stream-ordered workspace, then the GEMM.
template <int LW, bool PIPE, int LPG, int GM>
hipError_t launch_t(const LinearArgs& a, hipStream_t s, int64_t group, int xcd) {
  constexpr int GN = 64 / LPG / GM;
  constexpr int BTM = 16 * GM, BTN = 16 * GN;
  const uint32_t BMb = (uint32_t)((a.M + BTM - 1) / BTM), BNb = (uint32_t)((a.N + BTN - 1) / BTN);
  const int64_t blocks = (int64_t)BMb * (xcd ? ((int64_t)BNb + 7) / 8 * 8 : BNb);
  if (group < 1) group = 1;
  if (group > BMb) group = BMb;
  if (a.wsum_pre) {   // the caller's row sums: no pre-pass, no workspace
    hipLaunchKernelGGL((k_dot4_gemm<LW, PIPE, LPG, GM>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, a, BMb, BNb, (uint32_t)group, xcd, a.wsum_pre);
    return hipGetLastError();
  }
  void* ws = nullptr;
  hipError_t e = workspace_acquire(&ws, (size_t)a.N * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_row_sums, dim3((unsigned)((a.N + 3) / 4)), dim3(kThreads), 0, s, a.w, a.N,
                     a.K, (int32_t*)ws);
  e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL((k_dot4_gemm<LW, PIPE, LPG, GM>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, a, BMb, BNb, (uint32_t)group, xcd, (const int32_t*)ws);
    e = hipGetLastError();
  }
  hipError_t f = workspace_release(ws, s);
  return e != hipSuccess ? e : f;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

hipError_t launch_row_sums(const int8_t* w, int64_t N, int64_t K, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_row_sums, dim3((unsigned)((N + 3) / 4)), dim3(kThreads), 0, s, w, N, K, out);
  return hipGetLastError();
}

bool gemm_dot4_supported(const LinearArgs& a) {
  // The smallest block tile is 32 x 32; the grid must stay below 2^31 blocks.
  const int64_t blocks = ((a.M + 31) / 32) * (((a.N + 31) / 32 + 7) / 8 * 8);
  // K < 2^25 keeps the 32-bit lane offsets (< 8 * (64 / LPG / GM) * K + 2 K) in range.
  return (a.K % 16) == 0 && a.K < ((int64_t)1 << 25) && aligned16(a.x) && aligned16(a.w) &&
         blocks < ((int64_t)1 << 31);
}

// Variant: Q8TA_DOT4_CFG = "<LW><P|S>.<LPG>x<GM>[:group[:x]]": LW = 2 or 4
// dwords per lane per row; P = two-slice pipeline, S = single slice; LPG x GM
// = lanes per group x groups along M (built: 16x2, 8x2, 8x4, 4x4 with 4S;
// 16x2, 8x2 with 2P and 2S); group = block-rows walked together; x = one
// weight strip per XCD.  Default: "4S.4x4:8" (32 x 32 wave tile, 8 block-rows
// of 64 activation rows walked together), with XCD strips when N >= 1024;
// on 2048 x 4096 x 11008 this fetches about 0.27 GB from HBM per call, against
// 0.25 to 1.5 GB for the other orders measured, at the same speed.
hipError_t launch_gemm_dot4(const LinearArgs& a, hipStream_t s) {
  int lw = 4, lpg = 4, gm = 4;
  bool pipe = false;
  int64_t group = 8;
  int xcd = a.N >= 1024;
  if (const char* e = getenv("Q8TA_DOT4_CFG")) {
    if (e[0] == '2') lw = 2;
    if (e[0] && e[1] == 'P') pipe = true;
    if (const char* d = strchr(e, '.')) {
      lpg = atoi(d + 1);
      if (const char* xx = strchr(d, 'x')) gm = atoi(xx + 1);
    }
    if (const char* c = strchr(e, ':')) {
      group = atoll(c + 1);
      xcd = strchr(c + 1, 'x') != nullptr;
    }
  }
  if (lw == 2) {
    if (lpg == 8) return pipe ? launch_t<2, true, 8, 2>(a, s, group, xcd)
                              : launch_t<2, false, 8, 2>(a, s, group, xcd);
    return pipe ? launch_t<2, true, 16, 2>(a, s, group, xcd)
                : launch_t<2, false, 16, 2>(a, s, group, xcd);
  }
  if (lpg == 8 && gm == 4) return launch_t<4, false, 8, 4>(a, s, group, xcd);
  if (lpg == 8) return launch_t<4, false, 8, 2>(a, s, group, xcd);
  if (lpg == 4) return launch_t<4, false, 4, 4>(a, s, group, xcd);
  return launch_t<4, false, 16, 2>(a, s, group, xcd);
}

}  // namespace q8ta
