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

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool gemm_dot4_supported(const LinearArgs& a) {
  const int64_t blocks = ((a.M + 15) / 16) * (((a.N + 15) / 16 + 7) / 8 * 8);
  return (a.K % 16) == 0 && aligned16(a.x) && aligned16(a.w) && blocks < ((int64_t)1 << 31);
}

// Variant: Q8TA_DOT4_CFG = "<LW><P|S>[:group[:x]]" (LW = 2 or 4 dwords per
// lane per row, P = two-slice pipeline (LW = 2 only), S = single slice; group =
// block-rows walked together; x = one weight strip per XCD).  Default: "4S:32",
// with XCD strips when there are at least 64 block-columns.
hipError_t launch_gemm_dot4(const LinearArgs& a, hipStream_t s) {
  int lw = 4;
  bool pipe = false;
  int64_t group = 32;
  int xcd = ((a.N + 15) / 16) >= 64;
  if (const char* e = getenv("Q8TA_DOT4_CFG")) {
    if (e[0] == '2') lw = 2;
    if (e[0] && e[1] == 'P') pipe = true;
    if (const char* c = strchr(e, ':')) {
      group = atoll(c + 1);
      xcd = strchr(c + 1, 'x') != nullptr;
    }
  }
  // The two-slice pipeline is built only with 2 dwords per lane: with 4 it
  // needs more than 256 vector registers.
  if (lw == 2)
    return pipe ? launch_t<2, true>(a, s, group, xcd) : launch_t<2, false>(a, s, group, xcd);
  return launch_t<4, false>(a, s, group, xcd);
}

}  // namespace q8ta
