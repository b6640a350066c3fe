// q8ta_linear GEMM for large M x N: int8 matrix cores (v_mfma_i32_32x32x32_i8)
// fed through a ring of LDS stages filled by direct global->LDS loads
// ("Add q8ta_linear op", Solution: acc[m,n] = sum_k (x[m,k] - izp) * w[n,k]
// in int32, then the per-channel dequant / requant epilogue; Constraints (2):
// x [M,K] and w [N,K] both K-contiguous).
//
//  * Loads: global_load_lds_dwordx4 writes 16 bytes per lane straight into
//    LDS, lane l at byte 16*l of the 1 KiB the wave instruction targets; the
//    global address of each lane is free, so lane l fetches the chunk that
//    belongs at its LDS slot.  No registers hold the slabs and no ds_write
//    runs, so STAGES-1 K steps are in flight while the matrix cores work on
//    the oldest one.  Each wave waits for its own loads of a stage (vmcnt),
//    then a barrier makes every wave's loads visible; the same barrier tells
//    that the buffer refilled next is no longer read.
//  * LDS layout per stage: W tile [BN rows][BK bytes] then X tile [BM][BK];
//    16-byte chunk c of row r sits at position c ^ f(r) (the lane that writes
//    position p of row r fetches chunk p ^ f(r)), so the lanes reading 32
//    consecutive rows at one chunk spread over the banks.  Rows past M or N
//    read the last row (their products land in discarded outputs); K must be
//    a multiple of BK.
//  * MFMA operand layout (32x32x32 int8): lane l supplies row l % 32 with K
//    bytes 16*(l/32) .. +15 of the 32-byte slice; accumulator register r of
//    lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.  W is the A
//    operand and X the B operand, so registers 4g .. 4g+3 are four
//    consecutive output channels n of one row m.
//  * Zero point: the matrix cores form sum x*w; the epilogue subtracts
//    izp * sum_k w[n,k], taken from a row-sum pass over W that runs before.
//  * The tile's per-channel row sums, scales and biases are fetched into
//    registers before the K loop (their latency hides behind it) and passed
//    to the epilogue through LDS: read from global memory inside the
//    epilogue, each would cost a full memory latency with one wave per SIMD.
//  * Register arrays are indexed with compile-time constants only (Static).
//  * Tiles are remapped so that each XCD walks a contiguous run (M fastest).
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) void* gvoid;
typedef __attribute__((address_space(3))) void* lvoid;

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

template <int BN_, int BM_, int BK_, int WAVES_N_, int WAVES_M_, int STAGES_, int OCC_>
struct CfgDL {
  static constexpr int BN = BN_, BM = BM_, BK = BK_, STAGES = STAGES_, OCC = OCC_;
  static constexpr int WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int NW = WAVES_N * WAVES_M, NT = 64 * NW;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int FN = WN / 32, FM = WM / 32;
  static constexpr int CPR = BK / 16;          // 16-byte chunks per LDS row
  static constexpr int RPL = 64 / CPR;         // rows one wave load instruction fills
  static constexpr int A_LOADS = BN / (RPL * NW), B_LOADS = BM / (RPL * NW);
  static constexpr int LOADS = A_LOADS + B_LOADS;   // load instructions per wave per stage
  static constexpr int STAGE = (BN + BM) * BK;
  static constexpr int EPI = 3 * BN * 4;     // per-channel wsum, scale, bias of the tile
  static constexpr int LDS = STAGES * STAGE + EPI;
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(BN % (RPL * NW) == 0 && BM % (RPL * NW) == 0, "loader");
  static_assert(WN % 32 == 0 && WM % 32 == 0, "wave tile");
  static_assert(STAGES >= 2 && LOADS * (STAGES - 1) <= 63, "vmcnt range");
};

// Chunk swizzle: distinct positions for the rows one LDS cycle serves under
// both an 8-lanes-per-cycle / 32-bank and a 16-lanes-per-cycle / 64-bank
// reading of ds_read_b128; depends on row bits 0..4 only.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPR == 8) return (row ^ (row >> 3)) & 7;
  else return ((row >> 1) ^ (row >> 3)) & 3;
}

// s_waitcnt with vmcnt <= N and the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <class C>
__global__ __launch_bounds__(C::NT, C::OCC) void k_gemm_dl(LinearArgs a, int tiles_m, int tiles_n,
                                                           const int32_t* __restrict__ wsum) {
  extern __shared__ __attribute__((aligned(1024))) int8_t smem[];

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
  const int KT = (int)(K / C::BK);

  // Global source of each load instruction of this lane (at k = 0).
  const int rr = lane / C::CPR, pos = lane % C::CPR;
  const int8_t* ga[C::A_LOADS];
  const int8_t* gb[C::B_LOADS];
  Static<0, C::A_LOADS>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int r = (i * C::NW + wave) * C::RPL + rr;
    const int64_t n = bn0 + r < N ? bn0 + r : N - 1;
    ga[i] = a.w + n * K + 16 * (pos ^ swz<C::CPR>(r));
  });
  Static<0, C::B_LOADS>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int r = (i * C::NW + wave) * C::RPL + rr;
    const int64_t m = bm0 + r < M ? bm0 + r : M - 1;
    gb[i] = a.x + m * K + 16 * (pos ^ swz<C::CPR>(r));
  });
  auto issue = [&](int stage, int kt) {
    int8_t* base = smem + stage * C::STAGE;
    const int64_t ko = (int64_t)kt * C::BK;
    Static<0, C::A_LOADS>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      __builtin_amdgcn_global_load_lds((gvoid)(ga[i] + ko), (lvoid)(base + (i * C::NW + wave) * 1024),
                                       16, 0, 0);
    });
    Static<0, C::B_LOADS>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      __builtin_amdgcn_global_load_lds((gvoid)(gb[i] + ko),
                                       (lvoid)(base + C::BN * C::BK + (i * C::NW + wave) * 1024),
                                       16, 0, 0);
    });
  };

  v16i acc[C::FN][C::FM];
  Static<0, C::FN>::each([&](auto I) {
    Static<0, C::FM>::each([&](auto J) { acc[decltype(I)::value][decltype(J)::value] = v16i{}; });
  });

  // per-channel constants of tile row tid (read before the K loop)
  int32_t e_ws = 0;
  float e_sc = 0.0f, e_bi = 0.0f;
  if (tid < C::BN && bn0 + tid < N) {
    e_ws = wsum[bn0 + tid];
    if (!a.acc) {
      e_sc = a.wscale[bn0 + tid];
      e_bi = a.bias ? a.bias[bn0 + tid] : 0.0f;
    }
  }

  Static<0, C::STAGES - 1>::each([&](auto S) {
    constexpr int s = decltype(S)::value;
    if (s < KT) issue(s, s);
  });

  const int lrow = lane & 31;
  const int kg = lane >> 5;
  const int a_row0 = (wn * C::WN + lrow) * C::BK;
  const int b_row0 = C::BN * C::BK + (wm * C::WM + lrow) * C::BK;
  const int sw = swz<C::CPR>(lrow);   // fragment rows differ from lrow by multiples of 32
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + C::STAGES - 2 < KT) wait_vmcnt<(C::STAGES - 2) * C::LOADS>();
    else wait_vmcnt<0>();
    // s_barrier without the fence __syncthreads() adds (the fence would wait
    // for every load in flight, later stages included); the empty asm keeps
    // the compiler from moving LDS accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + C::STAGES - 1 < KT) issue((kt + C::STAGES - 1) % C::STAGES, kt + C::STAGES - 1);
    const int8_t* S = smem + (kt % C::STAGES) * C::STAGE;
    // Fragments of slice ks+1 are requested before the products of slice ks
    // are issued (two register sets); the compiler schedules freely (pinning
    // the order with sched_barrier measured ~5 % slower).
    v4i af[2][C::FN], bf[2][C::FM];
    auto read_slice = [&](auto KS, v4i (&fa)[C::FN], v4i (&fb)[C::FM]) {
      constexpr int ks = decltype(KS)::value;
      const int cpos = 16 * ((2 * ks + kg) ^ sw);
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        fa[i] = *reinterpret_cast<const v4i*>(S + a_row0 + i * 32 * C::BK + cpos);
      });
      Static<0, C::FM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        fb[j] = *reinterpret_cast<const v4i*>(S + b_row0 + j * 32 * C::BK + cpos);
      });
    };
    read_slice(std::integral_constant<int, 0>{}, af[0], bf[0]);
    Static<0, C::BK / 32>::each([&](auto KS) {
      constexpr int ks = decltype(KS)::value;
      if constexpr (ks + 1 < C::BK / 32)
        read_slice(std::integral_constant<int, ks + 1>{}, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        Static<0, C::FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks & 1][i], bf[ks & 1][j], acc[i][j],
                                                            0, 0, 0);
        });
      });
    });
  }

  int32_t* e_lds = reinterpret_cast<int32_t*>(smem + C::STAGES * C::STAGE);
  if (tid < C::BN) {
    e_lds[tid] = e_ws;
    e_lds[C::BN + tid] = __float_as_int(e_sc);
    e_lds[2 * C::BN + tid] = __float_as_int(e_bi);
  }
  __syncthreads();

  const bool vec_out = (N % 4) == 0 && ((uintptr_t)a.out & 3) == 0;
  Static<0, C::FN>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    Static<0, 4>::each([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int lr = wn * C::WN + i * 32 + 8 * g + 4 * kg;   // tile row of register group g
      const int64_t nb = bn0 + lr;
      int32_t ws4[4];
      float sc[4], bi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ws4[r] = e_lds[lr + r];
        sc[r] = __int_as_float(e_lds[C::BN + lr + r]);
        bi[r] = __int_as_float(e_lds[2 * C::BN + lr + r]);
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

using DLBig = CfgDL<256, 256, 64, 2, 2, 4, 1>;   // 128 x 128 per wave, 4 stages (128 KiB)
using DLMid = CfgDL<256, 128, 64, 2, 2, 3, 2>;   // 128 x 64 per wave, 3 stages, 2 per CU
using DLSq = CfgDL<128, 128, 64, 2, 2, 4, 2>;    // 64 x 64 per wave, 4 stages

template <class C>
hipError_t launch_dl(const LinearArgs& a, hipStream_t s) {
  if (C::LDS > 64 * 1024) {
    static bool attr_set = false;
    if (!attr_set) {
      hipError_t e = hipFuncSetAttribute((const void*)k_gemm_dl<C>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
      if (e != hipSuccess) return e;
      attr_set = true;
    }
  }
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
  if (a.wsum_pre) {   // the caller's row sums: no pre-pass, no workspace
    hipLaunchKernelGGL(k_gemm_dl<C>, dim3((unsigned)(tiles_m * tiles_n)), dim3(C::NT), C::LDS, s,
                       a, tiles_m, tiles_n, a.wsum_pre);
    return hipGetLastError();
  }
  void* ws = nullptr;
  hipError_t e = workspace_acquire(&ws, (size_t)a.N * sizeof(int32_t), s);
  if (e != hipSuccess) return e;
  e = launch_row_sums(a.w, a.N, a.K, (int32_t*)ws, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_gemm_dl<C>, dim3((unsigned)(tiles_m * tiles_n)), dim3(C::NT), C::LDS, s,
                       a, tiles_m, tiles_n, (const int32_t*)ws);
    e = hipGetLastError();
  }
  hipError_t f = workspace_release(ws, s);
  return e != hipSuccess ? e : f;
}

}  // namespace

bool gemm_dl_supported(const LinearArgs& a) {
  return (a.K % 64) == 0 && a.K < ((int64_t)1 << 30) && ((uintptr_t)a.x & 15) == 0 &&
         ((uintptr_t)a.w & 15) == 0 && a.M >= 1 && a.N >= 1 && a.M <= (int64_t)1 << 30 &&
         a.N <= (int64_t)1 << 30 && ((a.M + 127) / 128) * ((a.N + 127) / 128) < ((int64_t)1 << 31);
}

// Q8TA_GEMM_DL_CFG = B | D | Q picks the tile (256x256 / 256x128 / 128x128,
// weight rows x activation rows); default 256 x 256.
hipError_t launch_gemm_dl(const LinearArgs& a, hipStream_t s) {
  const char* e = getenv("Q8TA_GEMM_DL_CFG");
  const char pick = (e && strchr("BDQ", e[0])) ? e[0] : 'B';
  switch (pick) {
    case 'D': return launch_dl<DLMid>(a, s);
    case 'Q': return launch_dl<DLSq>(a, s);
    default: return launch_dl<DLBig>(a, s);
  }
}

}  // namespace q8ta
