// q8ta_linear for M > 4 on the vector ALU: a register-tiled int8 GEMM built
// on the packed dot-product instruction v_dot4 ("Add q8ta_linear op",
// Solution: acc[m,n] = sum_k (x[m,k] - izp) * w[n,k] in int32, then the
// per-channel epilogue).
//
// Each wave owns an RN x RM tile (RN weight rows, RM activation rows).  The
// 64 lanes split K: in one pass lane l reads LW dwords at byte 4*LW*l of a
// 256*LW-byte slice of every one of the RN + RM rows (each load instruction
// moves 256*LW contiguous bytes), and accumulates RN*RM partial dot products
// in registers.  The zero-point term is folded as sum x*w - izp*sum w, with
// the row sums of W formed by a small pass over W before the GEMM (one wave
// per row, v_dot4 against 0x01010101) into a stream-ordered workspace.  At the
// end the RN*RM partials are summed over the 64 lanes with a transposing
// butterfly: at each of the 6 steps a lane keeps half of its values, sends the
// other half to its partner and adds what it receives, so after 63 exchanges
// lane l holds the complete sum of tile element l (RN*RM == 64).  Lane l then
// requantizes that element.
//
// With PIPE the K loop keeps two register slices, so the loads of the next
// slice are in flight while the current one is multiplied.  The 4 waves of a
// block cover a 2 x 2 group of tiles (each weight and each activation row is
// fetched once per block and served to two waves from the CU's cache), and
// blocks are ordered in groups of GROUP block-rows along M so that the blocks
// resident on the GPU at a time touch a compact set of rows that L2 holds.
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

template <int RN, int RM, int LW>
struct Slice {
  typename Vec<LW>::type w[RN], x[RM];
};

// Loads LW dwords at byte k of every row of the tile (zeros past M, N, K).
// FULL: the whole tile lies inside M and N and k < K, so no bound is tested.
template <bool FULL, int RN, int RM, int LW>
__device__ __forceinline__ void load_slice(Slice<RN, RM, LW>& s, const LinearArgs& a,
                                           const int8_t* wb, const int8_t* xb, int64_t n0,
                                           int64_t m0, int64_t k) {
  typedef typename Vec<LW>::type V;
  if constexpr (FULL) {
#pragma unroll
    for (int r = 0; r < RN; ++r) s.w[r] = *reinterpret_cast<const V*>(wb + r * a.K + k);
#pragma unroll
    for (int m = 0; m < RM; ++m) s.x[m] = *reinterpret_cast<const V*>(xb + m * a.K + k);
    return;
  }
  const bool ok = k < a.K;
#pragma unroll
  for (int r = 0; r < RN; ++r)
    s.w[r] = (ok && n0 + r < a.N) ? *reinterpret_cast<const V*>(wb + r * a.K + k) : V{};
#pragma unroll
  for (int m = 0; m < RM; ++m)
    s.x[m] = (ok && m0 + m < a.M) ? *reinterpret_cast<const V*>(xb + m * a.K + k) : V{};
}

template <int RN, int RM, int LW>
__device__ __forceinline__ void dot_slice(const Slice<RN, RM, LW>& s, int32_t (&acc)[RN * RM]) {
#pragma unroll
  for (int d = 0; d < LW; ++d) {
#pragma unroll
    for (int r = 0; r < RN; ++r) {
#pragma unroll
      for (int m = 0; m < RM; ++m)
        acc[r * RM + m] = __builtin_amdgcn_sdot4(s.x[m][d], s.w[r][d], acc[r * RM + m], false);
    }
  }
}

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
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) out[n] = s;
}

template <int RN, int RM, int LW, bool PIPE>
__global__ __launch_bounds__(kThreads) void k_dot4_gemm(LinearArgs a, int64_t tiles_m,
                                                        int64_t tiles_n, int64_t group,
                                                        int xcd_strips,
                                                        const int32_t* __restrict__ wsum) {
  static_assert(RN * RM == 64, "one tile element per lane after the reduction");
  constexpr int64_t SL = 256 * LW;  // bytes of one row covered by one slice
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  // block -> (block-row bm_i along M, block-column bn_i along N), grouped:
  // `group` block-rows are walked together before moving to the next columns.
  const int64_t BM = (tiles_m + 1) / 2, BN = (tiles_n + 1) / 2;
  // With xcd_strips, block b runs on XCD b % 8 (round-robin dispatch) and each
  // XCD owns a contiguous strip of `width` block-columns, so the weight rows
  // of a strip are fetched into one L2 only; the grid is padded to 8 strips.
  const int64_t width = xcd_strips ? (BN + 7) / 8 : BN;
  const int64_t b = xcd_strips ? (int64_t)blockIdx.x / 8 : (int64_t)blockIdx.x;
  const int64_t strip0 = xcd_strips ? (int64_t)(blockIdx.x % 8) * width : 0;
  const int64_t per_group = group * width;
  const int64_t g = b / per_group;
  const int64_t rows_here = (g * group + group <= BM) ? group : BM - g * group;
  const int64_t in_g = b - g * per_group;
  const int64_t bm_i = g * group + in_g % rows_here;
  const int64_t bn_i = strip0 + in_g / rows_here;
  if (bn_i >= BN) return;
  const int64_t tm = bm_i * 2 + (wave & 1);
  const int64_t tn = bn_i * 2 + (wave >> 1);
  if (tm >= tiles_m || tn >= tiles_n) return;
  const int64_t m0 = tm * RM;
  const int64_t n0 = tn * RN;
  const int8_t* wb = a.w + n0 * a.K;
  const int8_t* xb = a.x + m0 * a.K;

  int32_t acc[RN * RM];
#pragma unroll
  for (int i = 0; i < RN * RM; ++i) acc[i] = 0;

  const int64_t kl = (int64_t)lane * 4 * LW;
  const bool full = (n0 + RN <= a.N) && (m0 + RM <= a.M) && (a.K % SL == 0);
  if constexpr (PIPE) {
    Slice<RN, RM, LW> s0, s1;
    load_slice<false>(s0, a, wb, xb, n0, m0, kl);
    for (int64_t k0 = 0; k0 < a.K; k0 += 2 * SL) {
      load_slice<false>(s1, a, wb, xb, n0, m0, k0 + SL + kl);
      dot_slice(s0, acc);
      if (k0 + 2 * SL >= a.K) {
        dot_slice(s1, acc);
        break;
      }
      load_slice<false>(s0, a, wb, xb, n0, m0, k0 + 2 * SL + kl);
      dot_slice(s1, acc);
    }
  } else if (full) {
    for (int64_t k0 = 0; k0 < a.K; k0 += SL) {
      Slice<RN, RM, LW> s0;
      load_slice<true>(s0, a, wb, xb, n0, m0, k0 + kl);
      dot_slice(s0, acc);
    }
  } else {
    for (int64_t k0 = 0; k0 < a.K; k0 += SL) {
      Slice<RN, RM, LW> s0;
      load_slice<false>(s0, a, wb, xb, n0, m0, k0 + kl);
      dot_slice(s0, acc);
    }
  }
  // Transposing butterfly over the 64 lanes (element index bit b <- lane bit b).
#pragma unroll
  for (int half = 32; half >= 1; half >>= 1) {
    const bool upper = (lane & half) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const int32_t lo = acc[i], hi = acc[i + half];
      const int32_t keep = upper ? hi : lo;
      const int32_t send = upper ? lo : hi;
      acc[i] = keep + __shfl_xor(send, half, 64);
    }
  }
  const int r = lane / RM, m = lane % RM;
  const int64_t n = n0 + r, mm = m0 + m;
  if (n < a.N && mm < a.M) {
    const int32_t c = acc[0] - a.izp * wsum[n];
    if (a.acc) {
      a.acc[mm * a.N + n] = c;
    } else {
      const float bv = a.bias ? a.bias[n] : 0.0f;
      a.out[mm * a.N + n] = (int8_t)requant(c, a.wscale[n], bv, a.rq);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped variant: the 64 lanes of a wave form 4 groups of 16 (one DPP row
// each).  Group g owns an 8 x 8 tile (8 activation rows, 8 weight rows) of the
// wave's 16 x 16 tile; its 16 lanes split K, lane l reading 4*LW bytes at byte
// 4*LW*l of a 64*LW-byte slice of each of its 16 rows.  The 64 partial sums of
// a lane are reduced over its 16-lane row only, with a transposing butterfly
// whose exchanges are DPP lane moves inside the row (mirror of 16, mirror of 8,
// quad reverse, quad swap: lane masks 15, 7, 3, 1, which span all 16 lanes), so
// the reduction costs one exchange per four outputs and no LDS traffic.
// Afterwards lane l of a group holds four consecutive output channels of one
// activation row: row (l >> 1) & 7, channels 4 * (l & 1) .. +3 of the tile.

// Lane moves inside a row of 16 lanes (DPP controls of the gfx9 encoding).
constexpr int kDppSwap1 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppRev4 = 0x1B;      // quad_perm [3,2,1,0]: lane ^ 3
constexpr int kDppMirror8 = 0x141;  // row_half_mirror:     lane ^ 7
constexpr int kDppMirror16 = 0x140; // row_mirror:          lane ^ 15

template <int CTRL>
__device__ __forceinline__ int32_t row_move(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// One butterfly step over HALF value pairs: keep the upper or lower half by
// `upper`, receive the partner's copy of the kept half and add it.
template <int HALF, int CTRL>
__device__ __forceinline__ void fold(int32_t (&acc)[64], bool upper) {
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const int32_t lo = acc[i], hi = acc[i + HALF];
    const int32_t keep = upper ? hi : lo;
    const int32_t send = upper ? lo : hi;
    acc[i] = keep + row_move<CTRL>(send);
  }
}

// Loads one slice for a group: row r of the weights is read at
// p.w[r] + (woff + k) and row m of the activations at p.x[m] + (xoff + k):
// the row pointers are wave-uniform (scalar registers) and the
// 32-bit lane offset holds the group's row offset, the lane's byte offset in
// the slice and the slice start k, so every load is one scalar-base plus
// 32-bit-offset instruction.  k passes through readfirstlane so that the
// loop does not turn the offsets into per-row 64-bit induction variables.
// Unless FULL, rows at or past nrem / mrem (counted from the group's first
// row) and lanes with `kin` false read zeros.
typedef const __attribute__((address_space(1))) int8_t* gptr;

__device__ __forceinline__ gptr uniform_ptr(const int8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (gptr)(((uint64_t)hi << 32) | lo);
}

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
__device__ __forceinline__ void load_slice_g(Slice<8, 8, LW>& s, const RowPtrs& p, uint32_t woff,
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
__device__ __forceinline__ void dot_slice_mn(const Slice<8, 8, LW>& s, int32_t (&acc)[64]) {
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

// Block b covers a 32 x 32 output tile (4 waves, 2 x 2).  Block order as in
// k_dot4_gemm: `group` block-rows walked together, optionally one strip of
// block-columns per XCD.
template <int LW, bool PIPE>
__global__ __launch_bounds__(kThreads) void k_dot4_gemm_g(LinearArgs a, uint32_t BMb, uint32_t BNb,
                                                          uint32_t group, int xcd_strips,
                                                          const int32_t* __restrict__ wsum) {
  constexpr int64_t SL = 64 * LW;  // bytes of one row covered by one slice of a group
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
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
  const int64_t m0w = (int64_t)bm_i * 32 + 16 * (wave & 1);
  const int64_t n0w = (int64_t)bn_i * 32 + 16 * (wave >> 1);
  if (m0w >= a.M || n0w >= a.N) return;  // wave-uniform
  const int64_t m0 = m0w + 8 * (grp & 1);
  const int64_t n0 = n0w + 8 * (grp >> 1);
  const int64_t nrem = a.N - n0, mrem = a.M - m0;
  const uint32_t kl = (uint32_t)(l16 * 4 * LW);
  const uint32_t woff = (uint32_t)(8 * (grp >> 1)) * (uint32_t)a.K + kl;
  const uint32_t xoff = (uint32_t)(8 * (grp & 1)) * (uint32_t)a.K + kl;
  const gptr wu = uniform_ptr(a.w + n0w * a.K);
  const gptr xu = uniform_ptr(a.x + m0w * a.K);
  RowPtrs rp;
  row_ptrs(rp, wu, xu, a.K);

  int32_t acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0;

  const int64_t Kf = a.K - a.K % SL;  // whole slices; the rest is one masked slice
  const bool full = (m0w + 16 <= a.M) && (n0w + 16 <= a.N);
  if constexpr (PIPE) {
    if (Kf > 0) {
      Slice<8, 8, LW> s0, s1;
      load_slice_g<false>(s0, rp, woff, xoff, 0, true, nrem, mrem);
      for (int64_t k0 = 0; k0 < Kf; k0 += 2 * SL) {
        if (k0 + SL < Kf)
          load_slice_g<false>(s1, rp, woff, xoff, k0 + SL, true, nrem, mrem);
        dot_slice_mn(s0, acc);
        if (k0 + SL >= Kf) break;
        if (k0 + 2 * SL < Kf)
          load_slice_g<false>(s0, rp, woff, xoff, k0 + 2 * SL, true, nrem,
                              mrem);
        dot_slice_mn(s1, acc);
      }
    }
  } else if (full) {
    for (int64_t k0 = 0; k0 < Kf; k0 += SL) {
      Slice<8, 8, LW> s0;
      load_slice_g<true>(s0, rp, woff, xoff, k0, true, nrem, mrem);
      dot_slice_mn(s0, acc);
    }
  } else {
    for (int64_t k0 = 0; k0 < Kf; k0 += SL) {
      Slice<8, 8, LW> s0;
      load_slice_g<false>(s0, rp, woff, xoff, k0, true, nrem, mrem);
      dot_slice_mn(s0, acc);
    }
  }
  if (Kf < a.K) {
    Slice<8, 8, LW> s0;
    load_slice_g<false>(s0, rp, woff, xoff, Kf, Kf + kl < a.K, nrem, mrem);
    dot_slice_mn(s0, acc);
  }
  fold<32, kDppMirror16>(acc, (l16 & 8) != 0);
  fold<16, kDppMirror8>(acc, (l16 & 4) != 0);
  fold<8, kDppRev4>(acc, (l16 & 2) != 0);
  fold<4, kDppSwap1>(acc, (l16 & 1) != 0);
  // acc[t] = tile element e = 32*b3 + 16*b2 + 8*b1 + 4*b0 + t (b = bits of l16),
  // i.e. row e / 8 = (l16 >> 1) & 7 and channel e % 8 = 4 * (l16 & 1) + t.
  const int64_t mm = m0 + ((l16 >> 1) & 7);
  const int64_t nb = n0 + 4 * (l16 & 1);
  if (mm >= a.M) return;
  int32_t c[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) c[t] = (nb + t < a.N) ? acc[t] - a.izp * wsum[nb + t] : 0;
  if (a.acc) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (nb + t < a.N) a.acc[mm * a.N + nb + t] = c[t];
    return;
  }
  int q[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bool ok = nb + t < a.N;
    const float sc = ok ? a.wscale[nb + t] : 0.0f;
    const float bv = (ok && a.bias) ? a.bias[nb + t] : 0.0f;
    q[t] = requant(c[t], sc, bv, a.rq);
  }
  int8_t* o = a.out + mm * a.N + nb;
  if (nb + 3 < a.N && ((uintptr_t)o & 3) == 0) {
    *reinterpret_cast<uint32_t*>(o) = pack4(q[0], q[1], q[2], q[3]);
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (nb + t < a.N) o[t] = (int8_t)q[t];
  }
}

// Row sums of W into a stream-ordered workspace, then the GEMM.
template <int LW, bool PIPE>
hipError_t launch_t(const LinearArgs& a, hipStream_t s, int64_t group, int xcd) {
  const int64_t tiles_m = (a.M + 7) / 8;
  const int64_t tiles_n = (a.N + 7) / 8;
  const int64_t BM = (tiles_m + 1) / 2, BN = (tiles_n + 1) / 2;
  const int64_t blocks = BM * (xcd ? (BN + 7) / 8 * 8 : BN);
  if (group < 1) group = 1;
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, (size_t)a.N * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_row_sums, dim3((unsigned)((a.N + 3) / 4)), dim3(kThreads), 0, s, a.w, a.N,
                     a.K, (int32_t*)ws);
  e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL((k_dot4_gemm<8, 8, LW, PIPE>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       s, a, tiles_m, tiles_n, group, xcd, (const int32_t*)ws);
    e = hipGetLastError();
  }
  hipError_t f = hipFreeAsync(ws, s);
  return e != hipSuccess ? e : f;
}

// Row sums of W, then the grouped GEMM.
template <int LW, bool PIPE>
hipError_t launch_g(const LinearArgs& a, hipStream_t s, int64_t group, int xcd) {
  const uint32_t BMb = (uint32_t)((a.M + 31) / 32), BNb = (uint32_t)((a.N + 31) / 32);
  const int64_t blocks = (int64_t)BMb * (xcd ? ((int64_t)BNb + 7) / 8 * 8 : BNb);
  if (group < 1) group = 1;
  if (group > BMb) group = BMb;
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, (size_t)a.N * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_row_sums, dim3((unsigned)((a.N + 3) / 4)), dim3(kThreads), 0, s, a.w, a.N,
                     a.K, (int32_t*)ws);
  e = hipGetLastError();
  if (e == hipSuccess) {
    hipLaunchKernelGGL((k_dot4_gemm_g<LW, PIPE>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a,
                       BMb, BNb, (uint32_t)group, xcd, (const int32_t*)ws);
    e = hipGetLastError();
  }
  hipError_t f = hipFreeAsync(ws, s);
  return e != hipSuccess ? e : f;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool gemm_dot4_supported(const LinearArgs& a) {
  const int64_t blocks = ((a.M + 15) / 16) * (((a.N + 15) / 16 + 7) / 8 * 8);
  // K < 2^28 keeps the grouped kernel's 32-bit lane offsets (< 9 K + 256) in range.
  return (a.K % 16) == 0 && a.K < ((int64_t)1 << 28) && aligned16(a.x) && aligned16(a.w) &&
         blocks < ((int64_t)1 << 31);
}

// Variant: Q8TA_DOT4_CFG = "[G]<LW><P|S>[:group[:x]]".  G = the grouped
// kernel (16 lanes per K split, 32 x 32 blocks), otherwise the whole-wave K
// split (16 x 16 blocks); LW = 2 or 4 dwords per lane per row; P = two-slice
// pipeline (LW = 2 only), S = single slice; group = block-rows walked
// together; x = one weight strip per XCD.  Default: "G4S:16", with XCD strips
// when N >= 1024.
hipError_t launch_gemm_dot4(const LinearArgs& a, hipStream_t s) {
  bool grouped = true;
  int lw = 4;
  bool pipe = false;
  int64_t group = 16;
  int xcd = a.N >= 1024;
  if (const char* e = getenv("Q8TA_DOT4_CFG")) {
    grouped = e[0] == 'G';
    if (grouped) ++e;
    if (e[0] == '2') lw = 2;
    if (e[0] && e[1] == 'P') pipe = true;
    if (const char* c = strchr(e, ':')) {
      group = atoll(c + 1);
      xcd = strchr(c + 1, 'x') != nullptr;
    } else if (!grouped) {
      group = 32;
    }
  }
  // The two-slice pipeline is built only with 2 dwords per lane: with 4 it
  // needs more than 256 vector registers.
  if (grouped) {
    if (lw == 2)
      return pipe ? launch_g<2, true>(a, s, group, xcd) : launch_g<2, false>(a, s, group, xcd);
    return launch_g<4, false>(a, s, group, xcd);
  }
  if (lw == 2)
    return pipe ? launch_t<2, true>(a, s, group, xcd) : launch_t<2, false>(a, s, group, xcd);
  return launch_t<4, false>(a, s, group, xcd);
}

}  // namespace q8ta
