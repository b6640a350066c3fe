// q8ta_linear GEMM for large M x N on CDNA4 int8 matrix cores with
// v_mfma_i32_32x32x32_i8 ("Add q8ta_linear op", Solution: acc[m,n] =
// sum_k (x[m,k] - izp) * w[n,k] in int32, then the per-channel dequant /
// requant epilogue; Constraints (2): x [M,K] and w [N,K] both K-contiguous).
//
//  * Instruction: on gfx950 the 32x32x32 int8 product issues at about twice
//    the rate per operation of the 16x16x64 one (a register-only loop reaches
//    ~4.5 POP/s against ~2.5), so the wave tiles are built from 32 x 32
//    products.  Lane l supplies row l % 32 of each operand with K bytes
//    16*(l/32) .. +15 of the 32-byte slice; accumulator register r of lane l
//    holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.  W is the A operand
//    and X the B operand, so a lane's registers 4g .. 4g+3 are four
//    consecutive output channels n of one row m: the epilogue stores 16 bytes
//    (fp32) or 4 bytes (int8) per group.
//  * A workgroup of WAVES_N x WAVES_M waves computes a BN x BM tile; each wave
//    owns (BN/WAVES_N) x (BM/WAVES_M) of it in accumulator registers.  K
//    advances BK bytes per step through two LDS buffers: the next step's slab
//    is fetched into registers (16 B per load, rows past M/N/K zero-filled)
//    while the current buffer feeds the matrix cores, then written to the
//    other buffer; one barrier per step.
//  * 16-byte chunk c of LDS row r sits at chunk position c ^ f(r), so lanes
//    reading consecutive rows at one chunk spread over the banks.
//  * Zero point: x - izp does not fit int8, so the matrix cores form
//    sum x*w and the epilogue subtracts izp * sum w (exact in int32).  The
//    row sums come from the W chunks while they pass through registers on
//    their way to LDS (v_dot4 against 0x01010101, off the matrix cores'
//    operand path), are reduced over the 8 threads that load one row and
//    handed to the epilogue through LDS.
//  * Every register array is indexed with compile-time constants (Static): a
//    loop the compiler left rolled would put the accumulators in scratch.
//  * Workgroups are dispatched round-robin over the 8 XCDs; tile ids are
//    remapped so that each XCD walks a contiguous run of tiles (M fastest),
//    which share W and X slabs in that XCD's L2.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Calls f(std::integral_constant<int, I>) for I = B .. E-1.
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

template <int BN_, int BM_, int BK_, int WAVES_N_, int WAVES_M_, int OCC_ = 1>
struct Cfg32 {
  static constexpr int BN = BN_, BM = BM_, BK = BK_;
  static constexpr int OCC = OCC_;   // waves per SIMD the register budget is cut for
  static constexpr int WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int NT = 64 * WAVES_N * WAVES_M;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int FN = WN / 32, FM = WM / 32;   // 32-row fragments per wave
  static constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
  static constexpr int A_LD = BN * CPR / NT;         // W chunks per thread per step
  static constexpr int B_LD = BM * CPR / NT;         // X chunks per thread per step
  static constexpr int STAGE = (BN + BM) * BK;       // bytes per LDS buffer
  static constexpr int LDS = 2 * STAGE;
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(WN % 32 == 0 && WM % 32 == 0, "wave tile");
  static_assert((BN * CPR) % NT == 0 && (BM * CPR) % NT == 0, "loader");
};

template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (CPR == 8) return c ^ (row & 7);
  else return c ^ ((row >> 1) & 3);
}

template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void k_gemm32(LinearArgs a, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];

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
  int32_t wpart[C::A_LD];   // partial row sums of the W chunks this thread loads
  Static<0, C::A_LD>::each([&](auto I) { wpart[decltype(I)::value] = 0; });
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
      *reinterpret_cast<v4i*>(As + row * C::BK + 16 * swz<C::CPR>(row, c)) = ra[i];
      wpart[i] = __builtin_amdgcn_sdot4(ra[i][0], 0x01010101, wpart[i], false);
      wpart[i] = __builtin_amdgcn_sdot4(ra[i][1], 0x01010101, wpart[i], false);
      wpart[i] = __builtin_amdgcn_sdot4(ra[i][2], 0x01010101, wpart[i], false);
      wpart[i] = __builtin_amdgcn_sdot4(ra[i][3], 0x01010101, wpart[i], false);
    });
    Static<0, C::B_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      *reinterpret_cast<v4i*>(Bs + row * C::BK + 16 * swz<C::CPR>(row, c)) = rb[i];
    });
  };

  v16i acc[C::FN][C::FM];
  Static<0, C::FN>::each([&](auto I) {
    Static<0, C::FM>::each([&](auto J) { acc[decltype(I)::value][decltype(J)::value] = v16i{}; });
  });

  load_global(0);
  store_lds(0);
  __syncthreads();

  const int lrow = lane & 31;   // operand row supplied by this lane
  const int kg = lane >> 5;     // which 16 bytes of a 32-byte K slice
  // Fragment i of this wave covers LDS rows wn*WN + 32*i + lrow; the swizzle
  // depends on the row modulo 8 only, i.e. on lrow.
  const int a_row0 = (wn * C::WN + lrow) * C::BK;
  const int b_row0 = C::BN * C::BK + (wm * C::WM + lrow) * C::BK;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
    const int8_t* S = smem + cur * C::STAGE;
    Static<0, C::BK / 32>::each([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      const int cpos = 16 * swz<C::CPR>(lrow, 2 * ks + kg);
      v4i af[C::FN], bf[C::FM];
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        af[i] = *reinterpret_cast<const v4i*>(S + a_row0 + i * 32 * C::BK + cpos);
      });
      Static<0, C::FM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        bf[j] = *reinterpret_cast<const v4i*>(S + b_row0 + j * 32 * C::BK + cpos);
      });
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

  // Row sums of W: the CPR consecutive threads that load one row add their
  // partials (lane-xor butterfly inside the wave), the first of them stores
  // the row's sum into LDS (free after the last barrier of the loop).
  int32_t* wsum_lds = reinterpret_cast<int32_t*>(smem);
  Static<0, C::A_LD>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    int32_t v = wpart[i];
#pragma unroll
    for (int d = 1; d < C::CPR; d <<= 1) v += __shfl_xor(v, d, 64);
    const int q = tid + i * C::NT;
    if (q % C::CPR == 0) wsum_lds[q / C::CPR] = v;
  });
  __syncthreads();

  const bool vec_out = (N % 4) == 0 && ((uintptr_t)a.out & 3) == 0;
  Static<0, C::FN>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    Static<0, 4>::each([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int r0 = 8 * g + 4 * kg;   // first fragment row of register group g
      const int lr = wn * C::WN + i * 32 + r0;   // tile row of that register
      int32_t ws4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ws4[r] = wsum_lds[lr + r];
      const int64_t nb = bn0 + lr;
      // Scales and bias exist only for the requantizing calls (the
      // accumulator entry point passes no weight_scales).
      float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, bi[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (!a.acc) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = nb + r < N;
          sc[r] = ok ? a.wscale[nb + r] : 0.0f;
          bi[r] = (ok && a.bias) ? a.bias[nb + r] : 0.0f;
        }
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
          // fused dequantize: fp32 out[m, n] = (q - zp) * scale of the output
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

using Big = Cfg32<256, 256, 128, 2, 2>;      // 128 x 128 per wave, 1 wave per SIMD
using Mid = Cfg32<256, 128, 64, 2, 2, 2>;    // 128 x 64 per wave, 2 workgroups per CU
using Tall = Cfg32<128, 256, 64, 2, 2, 2>;   // 64 x 128 per wave, 2 workgroups per CU
using Sq = Cfg32<128, 128, 64, 2, 2, 2>;     // 64 x 64 per wave
using SqK = Cfg32<128, 128, 128, 2, 2, 2>;   // 64 x 64 per wave, 128-byte K steps
using MidK = Cfg32<256, 128, 128, 2, 2>;     // 128 x 64 per wave, 128-byte K steps

template <class C>
hipError_t launch32(const LinearArgs& a, hipStream_t s) {
  if (C::LDS > 64 * 1024) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)k_gemm32<C>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
  hipLaunchKernelGGL(k_gemm32<C>, dim3((unsigned)(tiles_m * tiles_n)), dim3(C::NT), C::LDS, s,
                     a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

bool gemm_big_supported(const LinearArgs& a) {
  return (a.K % 16) == 0 && ((uintptr_t)a.x & 15) == 0 && ((uintptr_t)a.w & 15) == 0 &&
         a.M <= (int64_t)1 << 30 && a.N <= (int64_t)1 << 30 &&
         ((a.M + 127) / 128) * ((a.N + 127) / 128) < ((int64_t)1 << 31);
}

// Q8TA_GEMM32_CFG = B | D | T | Q picks the tile (256x256 / 256x128 /
// 128x256 / 128x128, weight rows x activation rows); default 256 x 128.
hipError_t launch_gemm_big(const LinearArgs& a, hipStream_t s) {
  const char* e = getenv("Q8TA_GEMM32_CFG");
  const char pick = (e && strchr("BDTQKM", e[0])) ? e[0] : 'D';
  switch (pick) {
    case 'B': return launch32<Big>(a, s);
    case 'T': return launch32<Tall>(a, s);
    case 'Q': return launch32<Sq>(a, s);
    case 'K': return launch32<SqK>(a, s);
    case 'M': return launch32<MidK>(a, s);
    default: return launch32<Mid>(a, s);
  }
}

}  // namespace q8ta
