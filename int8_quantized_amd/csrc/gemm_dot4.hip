// q8ta_linear for M > 4 on the vector ALU: a register-tiled int8 GEMM built
// on the packed dot-product instruction v_dot4 ("Add q8ta_linear op",
// Solution: acc[m,n] = sum_k (x[m,k] - izp) * w[n,k] in int32, then the
// per-channel epilogue).
//
// Each wave owns an RN x RM tile (RN weight rows, RM activation rows).  The
// 64 lanes split K: in one pass lane l reads bytes [16 l, 16 l + 16) of a
// 1 KiB slice of every one of the RN + RM rows (each load instruction moves
// 1 KiB of contiguous bytes), and accumulates RN*RM partial dot products plus
// the RN partial row sums of W (v_dot4 against 0x01010101) in registers.  The
// zero-point term is folded as sum x*w - izp*sum w.  At the end the RN*RM
// partials are summed over the 64 lanes with a transposing butterfly: at each
// of the 6 steps a lane keeps half of its values, sends the other half to its
// partner and adds what it receives, so after 63 exchanges lane l holds the
// complete sum of tile element l (RN*RM == 64).  Lane l then requantizes that
// element.  Waves with consecutive indices share their weight rows, so those
// rows are served from the CU's cache while the activation tile changes.
#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int RN, int RM>
__global__ __launch_bounds__(kThreads) void k_dot4_gemm(LinearArgs a, int64_t tiles_m,
                                                        int64_t tiles_n) {
  static_assert(RN * RM == 64, "one tile element per lane after the reduction");
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (t >= tiles_m * tiles_n) return;
  const int64_t m0 = (t % tiles_m) * RM;
  const int64_t n0 = (t / tiles_m) * RN;
  const int64_t M = a.M, N = a.N, K = a.K;

  int32_t acc[RN * RM];
  int32_t sw[RN];
#pragma unroll
  for (int i = 0; i < RN * RM; ++i) acc[i] = 0;
#pragma unroll
  for (int r = 0; r < RN; ++r) sw[r] = 0;

  for (int64_t k0 = 0; k0 < K; k0 += 1024) {
    const int64_t kk = k0 + lane * 16;
    const bool ok = kk < K;
    v4i wv[RN], xv[RM];
#pragma unroll
    for (int r = 0; r < RN; ++r)
      wv[r] = (ok && n0 + r < N) ? *reinterpret_cast<const v4i*>(a.w + (n0 + r) * K + kk)
                                 : v4i{0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < RM; ++m)
      xv[m] = (ok && m0 + m < M) ? *reinterpret_cast<const v4i*>(a.x + (m0 + m) * K + kk)
                                 : v4i{0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int r = 0; r < RN; ++r) {
        sw[r] = __builtin_amdgcn_sdot4(wv[r][d], 0x01010101, sw[r], false);
#pragma unroll
        for (int m = 0; m < RM; ++m)
          acc[r * RM + m] = __builtin_amdgcn_sdot4(xv[m][d], wv[r][d], acc[r * RM + m], false);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RN; ++r)
#pragma unroll
    for (int m = 0; m < RM; ++m) acc[r * RM + m] -= a.izp * sw[r];

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
  if (n < N && mm < M) {
    if (a.acc) {
      a.acc[mm * N + n] = acc[0];
    } else {
      const float b = a.bias ? a.bias[n] : 0.0f;
      a.out[mm * N + n] = (int8_t)requant(acc[0], a.wscale[n], b, a.rq);
    }
  }
}

template <int RN, int RM>
hipError_t launch_t(const LinearArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + RM - 1) / RM;
  const int64_t tiles_n = (a.N + RN - 1) / RN;
  const int64_t blocks = (tiles_m * tiles_n + kWaves - 1) / kWaves;
  hipLaunchKernelGGL((k_dot4_gemm<RN, RM>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a,
                     tiles_m, tiles_n);
  return hipGetLastError();
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool gemm_dot4_supported(const LinearArgs& a) {
  const int64_t tiles = ((a.M + 7) / 8) * ((a.N + 7) / 8);
  return (a.K % 16) == 0 && aligned16(a.x) && aligned16(a.w) &&
         (tiles + kWaves - 1) / kWaves < ((int64_t)1 << 31);
}

hipError_t launch_gemm_dot4(const LinearArgs& a, hipStream_t s) {
  return launch_t<8, 8>(a, s);
}

}  // namespace q8ta
