// q8ta_linear GEMM on CDNA4 int8 matrix cores ("Add q8ta_linear op",
// Solution: acc[m,n] = sum_k (x[m,k] - izp) * w[n,k] in int32, then the
// per-channel dequant/requant epilogue; Constraints (2): x [M,K] and
// w [N,K] both row-major, i.e. both K-contiguous).
//
// Design (gfx950):
//  * v_mfma_i32_16x16x64_i8 computes D[16 n][16 m] += W[16 n][64 k] * X[64 k][16 m].
//    The weight tile is the MFMA A operand and the activation tile the B
//    operand, so each lane's four accumulator rows are four consecutive
//    output channels n of one row m: the requantized bytes leave as one
//    32-bit store into row-major out[m, n..n+3].
//  * A workgroup computes a BN x BM tile with WAVES_N x WAVES_M waves, each
//    owning a (BN/WAVES_N) x (BM/WAVES_M) sub-tile held in accumulator
//    registers.  K advances BK bytes per step; the W and X slabs of the next
//    step are fetched into registers (16 B per load, whole 16 B chunks, rows
//    padded with zeros past M/N/K) while the matrix cores work on the current
//    LDS buffer, then written to the other of two LDS buffers.
//  * LDS rows hold BK bytes; the 16-byte chunk c of row r is stored at chunk
//    position c ^ f(r), so the 16 lanes that read 16 consecutive rows at the
//    same k hit distinct banks.
//  * Zero point: x - izp does not fit int8, so the matrix cores form sum x*w
//    and each wave also sums its W fragments with v_dot4 against 0x01010101;
//    the epilogue subtracts izp * sum w (exact in int32).
//  * Workgroups are dispatched round-robin over the 8 XCDs; the block index is
//    remapped so that each XCD walks a contiguous run of tiles (M fastest),
//    which share W and X slabs in that XCD's L2.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

template <int BN_, int BM_, int BK_, int WAVES_N_, int WAVES_M_>
struct Cfg {
  static constexpr int BN = BN_, BM = BM_, BK = BK_;
  static constexpr int WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int NT = 64 * WAVES_N * WAVES_M;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int FN = WN / 16, FM = WM / 16;
  static constexpr int CPR = BK / 16;                 // 16-byte chunks per row
  static constexpr int A_LD = BN * CPR / NT;          // W chunks per thread per step
  static constexpr int B_LD = BM * CPR / NT;          // X chunks per thread per step
  static constexpr int STAGE = (BN + BM) * BK;        // bytes per LDS buffer
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(WN % 16 == 0 && WM % 16 == 0, "wave tile");
  static_assert((BN * CPR) % NT == 0 && (BM * CPR) % NT == 0, "loader");
};

template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (CPR == 8) return c ^ (row & 7);
  else return c ^ ((row >> 1) & 3);
}

// PRE: the row sums of W come from a.wsum_pre (trusted, precomputed by the
// caller) instead of v_dot4 over the W fragments.
template <class C, bool PRE>
__global__ __launch_bounds__(C::NT, 1) void k_gemm(LinearArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * C::STAGE];
  __shared__ float epi[2 * C::BN];   // per-channel scale and bias of the tile
  __shared__ int32_t epi_ws[PRE ? C::BN : 1];   // per-channel row sums (PRE)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave / C::WAVES_M;
  const int wm = wave % C::WAVES_M;

  // XCD-aware tile order: block b runs on XCD b % 8; give each XCD a
  // contiguous run of tile ids.
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
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      const int64_t n = bn0 + row, k = kbase + c * 16;
      ra[i] = (n < N && k < K) ? *reinterpret_cast<const v4i*>(a.w + n * K + k)
                               : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      const int64_t m = bm0 + row, k = kbase + c * 16;
      rb[i] = (m < M && k < K) ? *reinterpret_cast<const v4i*>(a.x + m * K + k)
                               : v4i{0, 0, 0, 0};
    }
  };
  auto store_lds = [&](int buf) {
    int8_t* As = smem + buf * C::STAGE;
    int8_t* Bs = As + C::BN * C::BK;
#pragma unroll
    for (int i = 0; i < C::A_LD; ++i) {
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      *reinterpret_cast<v4i*>(As + row * C::BK + 16 * swz<C::CPR>(row, c)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_LD; ++i) {
      const int q = tid + i * C::NT;
      const int row = q / C::CPR, c = q % C::CPR;
      *reinterpret_cast<v4i*>(Bs + row * C::BK + 16 * swz<C::CPR>(row, c)) = rb[i];
    }
  };

  v4i acc[C::FN][C::FM];
#pragma unroll
  for (int i = 0; i < C::FN; ++i)
#pragma unroll
    for (int j = 0; j < C::FM; ++j) acc[i][j] = v4i{0, 0, 0, 0};
  int32_t wsum[C::FN];
#pragma unroll
  for (int i = 0; i < C::FN; ++i) wsum[i] = 0;

  // The epilogue's per-channel scale and bias (tile row tid), fetched before
  // the K loop so that their latency hides behind it; handed over through LDS
  // after the loop.
  static_assert(C::BN <= C::NT, "one channel per thread");
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

  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_global(kt + 1);
    const int8_t* As = smem + cur * C::STAGE;
    const int8_t* Bs = As + C::BN * C::BK;
#pragma unroll
    for (int kk = 0; kk < C::BK / 64; ++kk) {
      const int c = kk * 4 + lgrp;
      v4i af[C::FN], bf[C::FM];
#pragma unroll
      for (int i = 0; i < C::FN; ++i) {
        const int row = wn * C::WN + i * 16 + lrow;
        af[i] = *reinterpret_cast<const v4i*>(As + row * C::BK + 16 * swz<C::CPR>(row, c));
      }
#pragma unroll
      for (int j = 0; j < C::FM; ++j) {
        const int row = wm * C::WM + j * 16 + lrow;
        bf[j] = *reinterpret_cast<const v4i*>(Bs + row * C::BK + 16 * swz<C::CPR>(row, c));
      }
      if constexpr (!PRE) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i) {
          wsum[i] = __builtin_amdgcn_sdot4(af[i][0], 0x01010101, wsum[i], false);
          wsum[i] = __builtin_amdgcn_sdot4(af[i][1], 0x01010101, wsum[i], false);
          wsum[i] = __builtin_amdgcn_sdot4(af[i][2], 0x01010101, wsum[i], false);
          wsum[i] = __builtin_amdgcn_sdot4(af[i][3], 0x01010101, wsum[i], false);
        }
      }
#pragma unroll
      for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_lds(cur ^ 1);
    __syncthreads();
  }

  if (tid < C::BN) {
    epi[tid] = e_sc;
    epi[C::BN + tid] = e_bi;
    if constexpr (PRE) epi_ws[tid] = e_ws;
  }
  __syncthreads();

  // Row sums of W: lane l holds a partial for row (l & 15) of each fragment;
  // add the four k-groups, then fetch the sums of the four rows this lane's
  // accumulators belong to (rows 4*(l>>4) .. +3 of the fragment).
  int32_t ws4[C::FN][4];
#pragma unroll
  for (int i = 0; i < C::FN; ++i) {
    if constexpr (PRE) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ws4[i][r] = epi_ws[wn * C::WN + i * 16 + 4 * lgrp + r];
    } else {
      int32_t v = wsum[i];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
#pragma unroll
      for (int r = 0; r < 4; ++r) ws4[i][r] = __shfl(v, 4 * lgrp + r, 64);
    }
  }

  const bool vec_store = (N % 4) == 0 && ((uintptr_t)a.out & 3) == 0;
#pragma unroll
  for (int i = 0; i < C::FN; ++i) {
    const int lr = wn * C::WN + i * 16 + 4 * lgrp;   // tile row of this lane's registers
    const int64_t nb = bn0 + lr;
    // Scales and bias exist only for the requantizing calls: the accumulator
    // entry point passes no weight_scales (NULL), so none was read then.
    float sc[4], bi[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[r] = epi[lr + r];
      bi[r] = epi[C::BN + lr + r];
    }
#pragma unroll
    for (int j = 0; j < C::FM; ++j) {
      const int64_t m = bm0 + wm * C::WM + j * 16 + lrow;
      if (m >= M) continue;
      int32_t cacc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) cacc[r] = acc[i][j][r] - a.izp * ws4[i][r];
      if (a.acc) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb + r < N) a.acc[m * N + nb + r] = cacc[r];
      } else {
        int q[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) q[r] = requant(cacc[r], sc[r], bi[r], a.rq);
        if (a.outf) {
          // fused dequantize: fp32 out[m, n] = (q - zp) * scale of the output
          float* of = a.outf + m * N + nb;
          if (nb + 3 < N && ((uintptr_t)of & 15) == 0) {
            typedef float v4f __attribute__((ext_vector_type(4)));
            *reinterpret_cast<v4f*>(of) =
                v4f{dequant1(q[0], a.dq_zp, a.dq_scale), dequant1(q[1], a.dq_zp, a.dq_scale),
                    dequant1(q[2], a.dq_zp, a.dq_scale), dequant1(q[3], a.dq_zp, a.dq_scale)};
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (nb + r < N) of[r] = dequant1(q[r], a.dq_zp, a.dq_scale);
          }
        } else if (vec_store && nb + 3 < N) {
          *reinterpret_cast<uint32_t*>(a.out + m * N + nb) = pack4(q[0], q[1], q[2], q[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb + r < N) a.out[m * N + nb + r] = (int8_t)q[r];
        }
      }
    }
  }
}

using CfgM = Cfg<128, 128, 64, 2, 2>;   // 64x64 per wave
using CfgS = Cfg<128, 64, 64, 2, 1>;    // 64x64 per wave, 2 waves

template <class C>
hipError_t launch_cfg(const LinearArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
  const int T = tiles_m * tiles_n;
  // With the caller's row sums the K loop drops its v_dot4 (same result).
  if (a.wsum_pre) {
    hipLaunchKernelGGL((k_gemm<C, true>), dim3((unsigned)T), dim3(C::NT), 0, s, a, tiles_m,
                       tiles_n);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm<C, false>), dim3((unsigned)T), dim3(C::NT), 0, s, a, tiles_m, tiles_n);
  return hipGetLastError();
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

// The epilogue once read weight_scales[n] also for the accumulator entry
// point, which passes NULL there: a read near address 0, the illegal memory
// access of the first launch.  Scales and bias are now read only when the
// call requantizes.
constexpr bool kMfmaGemmEnabled = true;

bool gemm_mfma_supported(const LinearArgs& a) {
  return kMfmaGemmEnabled && (a.K % 16) == 0 && aligned16(a.x) && aligned16(a.w) &&
         a.M <= (int64_t)1 << 30 && a.N <= (int64_t)1 << 30;
}

// Tile choice for a long K (>= 1024): the eight-wave kernel of gemm_w8.hip
// for problems whose 256 x 256 tiles fill the 256 CUs at least once (whole
// rounds of them, the remaining columns as 256 x 128 tiles in the same
// launch) or whose 256 x 128 tiles fill half to all of them in one round (on
// 2048 x 4096 x N with the fused dequantize, same boxes: 100.6-104.9 us
// against 119.8-120.7 us for gemm_mx.hip at N = 11008, 69.4-70.9 against
// 83.4-84.3 at 8192, 42.8 against 45.8 at 4096, 32.9 against 38.3 at 2048);
// the others that fill the CUs with 256 x 128 tiles the two-workgroup kernel
// of gemm_mx.hip; the rest the 128 x 128 tile of this file, or the 128 x 64
// tile for few rows.
hipError_t launch_gemm_mfma(const LinearArgs& a, hipStream_t s, char kind) {
  const int64_t tv = ((a.M + 127) / 128) * ((a.N + 255) / 256);
  const int64_t tm = ((a.M + 127) / 128) * ((a.N + 127) / 128);
  if (kind == 'x') return launch_gemm_mx(a, s);
  if ((kind == 'w' && gemm_w8_supported(a)) || (kind == 0 && gemm_w8_preferred(a)))
    return launch_gemm_w8(a, s);
  if (tv >= 256 && a.K >= 1024) return launch_gemm_mx(a, s);
  if (tm >= 256 || a.M > 64) return launch_cfg<CfgM>(a, s);
  return launch_cfg<CfgS>(a, s);
}

}  // namespace q8ta
