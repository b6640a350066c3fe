// q8ta_linear GEMM on the int8 matrix cores with v_mfma_i32_32x32x32_i8
// ("Add q8ta_linear op", Solution: acc[m,n] = sum_k (x[m,k] - izp) * w[n,k]
// in int32, then the per-channel dequant/requant epilogue; Constraints (2):
// x [M,K] and w [N,K] both K-contiguous).
//
// The structure of the 16x16x64 kernel in gemm.hip (register-staged K steps
// through two LDS buffers, XOR-swizzled 16-byte chunks, W as the A operand,
// per-channel constants staged through LDS, XCD-aware tile order), with the
// wave tile built from 32 x 32 products: on gfx950 a register-only loop of
// 32x32x32 products issues at ~4.4 POP/s against ~2.4 for 16x16x64 ones.
// Lane l supplies row l % 32 of each operand with K bytes 16*(l/32) .. +15 of
// the 32-byte slice; accumulator register r of lane l holds row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32, so registers 4g .. 4g+3 are four
// consecutive output channels n of one row m.
#include <cstdlib>
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

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

template <int BN_, int BM_, int BK_, int WAVES_N_, int WAVES_M_>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, BK = BK_;
  static constexpr int WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int NT = 64 * WAVES_N * WAVES_M;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int FN = WN / 32, FM = WM / 32;
  static constexpr int CPR = BK / 16;
  static constexpr int A_LD = BN * CPR / NT;
  static constexpr int B_LD = BM * CPR / NT;
  static constexpr int STAGE = (BN + BM) * BK;
  static_assert(BK == 128, "BK");
  static_assert(WN % 32 == 0 && WM % 32 == 0, "wave tile");
  static_assert((BN * CPR) % NT == 0 && (BM * CPR) % NT == 0, "loader");
  static_assert(BN <= NT, "one channel per thread in the epilogue staging");
};

// chunk c of LDS row r sits at position c ^ (r & 7)
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 7); }

template <class C, bool PRE>
__global__ __launch_bounds__(C::NT, 1) void k_gemm32(LinearArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * C::STAGE];
  __shared__ float epi[2 * C::BN];
  __shared__ int32_t epi_ws[C::BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / C::WAVES_M;
  const int wm = wave % C::WAVES_M;

  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int per = T / 8;
  int t = b;
  if (b < per * 8) t = (b % 8) * per + (b / 8);
  const int tm = t % tiles_m;
  const int tn = t / tiles_m;
  const int64_t bn0 = (int64_t)tn * C::BN;
  const int64_t bm0 = (int64_t)tm * C::BM;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = (int)((K + C::BK - 1) / C::BK);

  v4i ra[C::A_LD], rb[C::B_LD];
  auto load_global = [&](int kt) {
    const int64_t kbase = (int64_t)kt * C::BK;
    Static<0, C::A_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      const int64_t n = bn0 + row, k = kbase + c * 16;
      ra[i] = (n < N && k < K) ? *reinterpret_cast<const v4i*>(a.w + n * K + k)
                               : v4i{0, 0, 0, 0};
    });
    Static<0, C::B_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      const int64_t m = bm0 + row, k = kbase + c * 16;
      rb[i] = (m < M && k < K) ? *reinterpret_cast<const v4i*>(a.x + m * K + k)
                               : v4i{0, 0, 0, 0};
    });
  };
  auto store_lds = [&](int buf) {
    int8_t* As = smem + buf * C::STAGE;
    int8_t* Bs = As + C::BN * C::BK;
    Static<0, C::A_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      *reinterpret_cast<v4i*>(As + row * C::BK + 16 * swz(row, c)) = ra[i];
    });
    Static<0, C::B_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      *reinterpret_cast<v4i*>(Bs + row * C::BK + 16 * swz(row, c)) = rb[i];
    });
  };

  v16i acc[C::FN][C::FM];
  Static<0, C::FN>::each([&](auto I) {
    Static<0, C::FM>::each([&](auto J) { acc[decltype(I)::value][decltype(J)::value] = v16i{}; });
  });
  int32_t wsum[C::FN];
  Static<0, C::FN>::each([&](auto I) { wsum[decltype(I)::value] = 0; });

  // per-channel constants of tile row tid, fetched before the K loop
  float e_sc = 0.0f, e_bi = 0.0f;
  int32_t e_ws = 0;
  if (tid < C::BN && !a.acc && bn0 + tid < N) {
    e_sc = a.wscale[bn0 + tid];
    e_bi = a.bias ? a.bias[bn0 + tid] : 0.0f;
  }
  if (PRE && tid < C::BN && bn0 + tid < N) e_ws = a.wsum_pre[bn0 + tid];

  load_global(0);
  store_lds(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int kg = lane >> 5;
  const int a_row0 = (wn * C::WN + lrow) * C::BK;
  const int b_row0 = C::BN * C::BK + (wm * C::WM + lrow) * C::BK;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
    const int8_t* S = smem + cur * C::STAGE;
    Static<0, C::BK / 32>::each([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      // fragment rows differ from lrow by multiples of 32: same swizzle
      const int cpos = 16 * swz(lrow, 2 * ks + kg);
      v4i af[C::FN], bf[C::FM];
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        af[i] = *reinterpret_cast<const v4i*>(S + a_row0 + i * 32 * C::BK + cpos);
      });
      Static<0, C::FM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        bf[j] = *reinterpret_cast<const v4i*>(S + b_row0 + j * 32 * C::BK + cpos);
      });
      if constexpr (!PRE) {
        Static<0, C::FN>::each([&](auto I) {
          constexpr int i = decltype(I)::value;
          wsum[i] = __builtin_amdgcn_sdot4(af[i][0], 0x01010101, wsum[i], false);
          wsum[i] = __builtin_amdgcn_sdot4(af[i][1], 0x01010101, wsum[i], false);
          wsum[i] = __builtin_amdgcn_sdot4(af[i][2], 0x01010101, wsum[i], false);
          wsum[i] = __builtin_amdgcn_sdot4(af[i][3], 0x01010101, wsum[i], false);
        });
      }
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        Static<0, C::FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        });
      });
    });
    if (kt + 1 < KT) store_lds(cur ^ 1);
    __syncthreads();
  }

  // Row sums: lane l holds row l % 32's partial over its 16-byte halves;
  // lanes l and l ^ 32 together cover the row.
  if constexpr (!PRE) {
    Static<0, C::FN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      int32_t v = wsum[i];
      v += __shfl_xor(v, 32, 64);
      wsum[i] = v;
    });
  }
  if (tid < C::BN) {
    epi[tid] = e_sc;
    epi[C::BN + tid] = e_bi;
    if constexpr (PRE) epi_ws[tid] = e_ws;
  }
  if constexpr (!PRE) {
    // waves with wm == 0 publish the sums of their fragment rows
    if (wm == 0 && kg == 0) {
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        epi_ws[wn * C::WN + i * 32 + lrow] = wsum[i];
      });
    }
  }
  __syncthreads();

  const bool vec_out = (N % 4) == 0 && ((uintptr_t)a.out & 3) == 0;
  Static<0, C::FN>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    Static<0, 4>::each([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int lr = wn * C::WN + i * 32 + 8 * g + 4 * kg;
      const int64_t nb = bn0 + lr;
      int32_t ws4[4];
      float sc[4], bi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ws4[r] = epi_ws[lr + r];
        sc[r] = epi[lr + r];
        bi[r] = epi[C::BN + lr + r];
      }
      Static<0, C::FM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int64_t m = bm0 + wm * C::WM + j * 32 + lrow;
        if (m >= M) return;
        int32_t c[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = acc[i][j][4 * g + r] - a.izp * ws4[r];
        if (a.acc) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) a.acc[m * N + nb + r] = c[r];
          return;
        }
        int q[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) q[r] = requant(c[r], sc[r], bi[r], a.rq);
        if (a.outf) {
          float* of = a.outf + m * N + nb;
          if (nb + 3 < N && ((uintptr_t)of & 15) == 0) {
            *reinterpret_cast<v4f*>(of) =
                v4f{dequant1(q[0], a.dq_zp, a.dq_scale), dequant1(q[1], a.dq_zp, a.dq_scale),
                    dequant1(q[2], a.dq_zp, a.dq_scale), dequant1(q[3], a.dq_zp, a.dq_scale)};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (nb + r < N) of[r] = dequant1(q[r], a.dq_zp, a.dq_scale);
          }
        } else if (vec_out && nb + 3 < N) {
          *reinterpret_cast<uint32_t*>(a.out + m * N + nb) = pack4(q[0], q[1], q[2], q[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) a.out[m * N + nb + r] = (int8_t)q[r];
        }
      });
    });
  });
}

using C32V = Cfg<256, 128, 128, 4, 2>;   // 64 x 64 per wave, 8 waves
using C32M = Cfg<128, 128, 128, 2, 2>;   // 64 x 64 per wave, 4 waves

template <class C>
hipError_t launch32(const LinearArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
  const int T = tiles_m * tiles_n;
  if (a.wsum_pre)
    hipLaunchKernelGGL((k_gemm32<C, true>), dim3((unsigned)T), dim3(C::NT), 0, s, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((k_gemm32<C, false>), dim3((unsigned)T), dim3(C::NT), 0, s, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

// Q8TA_GEMM32_CFG = V | M picks 256 x 128 (8 waves) or 128 x 128 (4 waves).
hipError_t launch_gemm32(const LinearArgs& a, hipStream_t s) {
  const char* e = getenv("Q8TA_GEMM32_CFG");
  if (e && e[0] == 'M') return launch32<C32M>(a, s);
  return launch32<C32V>(a, s);
}

}  // namespace q8ta
