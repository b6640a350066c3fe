// q8ta_linear GEMM on the int8 matrix cores with v_mfma_i32_32x32x32_i8 and
// large per-wave tiles ("Add q8ta_linear op", Solution: acc[m,n] =
// sum_k (x[m,k] - izp) * w[n,k] in int32, then the per-channel
// dequant/requant epilogue; Constraints (1): the zero-point term folded as
// sum x*w - izp * sum w; Constraints (2): x [M,K] and w [N,K] K-contiguous).
//
// Why this shape on gfx950:
//  * A register-only loop of v_mfma_i32_32x32x32_i8 issues at ~4.3 POP/s
//    (3.7-3.9 with one or two waves per SIMD), one of v_mfma_i32_16x16x64_i8
//    at ~2.4-3.0, so only the 32x32x32 form can approach the 5.0 POP/s dense
//    int8 peak.
//  * Each wave owns a WN x WM = 128 x 64 (or 64 x 128) sub-tile: 8
//    accumulator fragments of 16 registers.  Every K byte then costs the wave
//    WN + WM = 192 bytes of LDS fragment reads for 2 * WN * WM = 16384
//    operations, 85 operations per LDS byte; the 64 x 64 wave tile of the
//    16x16x64 kernel reads 128 bytes for 8192 (64 per byte), which puts the
//    LDS port at the matrix cores' speed.
//  * Two workgroups of four waves share a CU (up to 256 registers per wave,
//    two waves per SIMD, 2 x 24 KiB of LDS buffers): their barriers and
//    epilogues are independent, so one workgroup's requantize and stores run
//    while the other keeps the matrix cores busy.  (The one-workgroup
//    variant keeps a whole SIMD per wave and 128-byte K steps.)
//  * K advances BK bytes per step through two LDS buffers; the slabs are
//    staged in registers (16 B per load; rows past M/N read the last row,
//    chunks past K are zeroed) and written to the buffer the matrix cores are
//    not reading; one barrier per step.  The default loop (PD = 3) writes
//    step k + 1's registers to LDS at the top of step k and refills them with
//    step k + 3 at once.  The 16-byte chunk c of LDS row r sits at chunk
//    position c ^ f(r), f chosen so that the 16 lanes one ds_read_b128 cycle
//    serves hit distinct banks.
//  * Lane l supplies row l % 32 of each operand with K bytes 16 * (l / 32)
//    .. +15 of each 32-byte slice; accumulator register r of lane l holds row
//    8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32 of the product.
//    For int8 output W is the A operand and X the B operand, so registers
//    4g .. 4g+3 are four consecutive output channels of one row (one 32-bit
//    store); for fp32 output (fused dequantize) the operands swap, so lane l
//    holds one channel and each half-wave store writes 32 consecutive floats
//    of one row, a whole 128-byte line.
//  * sum w comes from v_dot4 against 0x01010101 over the W fragments while
//    they are in registers; the waves sharing a W strip split the K slices
//    between them and add their partial sums through LDS after the loop.
//  * Workgroups are dispatched round-robin over the 8 XCDs; the block index
//    is remapped so that each XCD walks a contiguous run of tiles (M
//    fastest), which share W and X slabs in that XCD's L2.
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

template <int BN_, int BM_, int BK_, int WAVES_N_, int WAVES_M_, int BLOCKS_PER_CU_, int PD_ = 1>
struct MxCfg {
  // 1: one register set, loads one step ahead; 2: two sets, loads two steps
  // ahead; 3: two sets, the LDS write of step k + 1 moved to the top of
  // step k (see the K loop)
  static constexpr int PD = PD_;
  static constexpr int BN = BN_, BM = BM_, BK = BK_;
  static constexpr int WAVES_N = WAVES_N_, WAVES_M = WAVES_M_;
  static constexpr int BLOCKS_PER_CU = BLOCKS_PER_CU_;
  static constexpr int NT = 64 * WAVES_N * WAVES_M;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int FN = WN / 32, FM = WM / 32;
  static constexpr int CPR = BK / 16;            // 16-byte chunks per LDS row
  static constexpr int KS = BK / 32;             // 32-byte MFMA slices per step
  static constexpr int A_LD = BN * CPR / NT;     // W chunks per thread per step
  static constexpr int B_LD = BM * CPR / NT;     // X chunks per thread per step
  static constexpr int STAGE = (BN + BM) * BK;   // bytes per LDS buffer
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(PD >= 1 && PD <= 3, "prefetch mode");
  static_assert(WN % 32 == 0 && WM % 32 == 0, "wave tile");
  static_assert((BN * CPR) % NT == 0 && (BM * CPR) % NT == 0, "loader");
  static_assert(NT % CPR == 0, "a thread keeps its chunk column");
  static_assert(BN <= NT, "one channel per thread in the epilogue staging");
  static_assert(KS % WAVES_M == 0 || WAVES_M == 1, "row-sum split");
};

// Chunk position of chunk c in LDS row r: c ^ f(r), f from row bits 1..4
// only, so rows 32 apart (the fragments of one wave) share the pattern.
// Measured on gfx950 with an LDS probe (SQ_LDS_BANK_CONFLICT over 29 lane
// patterns): a ds_read_b128 serves 16 lanes per cycle over 64 banks, and the
// 16 lanes of a cycle are the lane quads (lanes 4q .. 4q+3) of one half-wave
// whose quad index q has even parity, or those with odd parity.  For the
// 32x32x32 pattern (lane l reads row l % 32 at one chunk per half-wave) the
// 16 rows of a cycle are then 4 rows in each residue class r % 4 (64-byte
// rows) or r % 2 (128-byte rows); f = (r >> 2) & 3, resp. (r >> 1) & 7,
// sends them to distinct chunk positions.  The earlier swizzles measured 4
// conflict cycles per read.  The loader's ds_write_b128 (CPR lanes per row)
// measured conflict-free with any of them.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CPR == 4) return c ^ ((r >> 2) & 3);
  else return c ^ ((r >> 1) & 7);
}

// The requantized code as a float in [qmin, 127] (the steps of requant()).
__device__ __forceinline__ float requant_code(int32_t acc, float wscale, float b,
                                              const Requant& r) {
  float v = (float)acc;
  v = v * r.s_in;
  v = v * wscale;
  v = v + b;
  float t = v * r.inv_out;
  float q = __builtin_rintf(t);
  q = q + r.ozp;
  q = __builtin_amdgcn_fmed3f(q, r.qmin, 127.0f);
  return q;
}

// LDS slot of the per-channel constant of tile row r: the four rows of one
// register group (r % 4 = 0..3) sit BN / 4 words apart, so the epilogue reads
// them as separate 32-bit broadcasts; side by side they would merge into one
// 16-byte broadcast read, which measured LDS bank conflicts.
template <int BN>
__device__ __forceinline__ int cslot(int r) { return (r & 3) * (BN / 4) + (r >> 2); }

// PRE: the row sums of W come from a.wsum_pre (trusted, precomputed by the
// caller) instead of v_dot4 over the W fragments.
// TR (fp32 output only): X is the A operand and W the B operand, so lane l
// holds output channel l % 32 of its fragments and the 32 lanes of a
// half-wave store 32 consecutive floats (one whole 128-byte line) of one
// output row per register; in the other form each store instruction writes
// 16-byte pieces of 32 rows, which the L2 has to merge.
template <class C, bool PRE, bool KFULL, bool TR>
__global__ __launch_bounds__(C::NT, C::BLOCKS_PER_CU) void k_gemm_mx(LinearArgs a, int tiles_m,
                                                                      int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * C::STAGE];
  __shared__ __attribute__((aligned(16))) float epi_sc[C::BN];
  __shared__ __attribute__((aligned(16))) float epi_bi[C::BN];
  __shared__ __attribute__((aligned(16))) int32_t epi_ws[C::WAVES_M][C::BN];

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

  // Loader geometry: thread tid copies chunk column lc of rows lr + i * RSTEP.
  // Rows past N (or M) are clamped to the last row: their products land only
  // in accumulators of channels (rows) that are never stored.  Every load is
  // unconditional, so the loop carries no branches and the compiler's wait
  // counts stay exact; with KFULL false the chunks past K are read at a
  // clamped offset and replaced by zeros.
  constexpr int RSTEP = C::NT / C::CPR;
  const int lc = tid % C::CPR;
  const int lr = tid / C::CPR;
  const int8_t* wrow[C::A_LD];
  const int8_t* xrow[C::B_LD];
  Static<0, C::A_LD>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int64_t n = bn0 + lr + i * RSTEP;
    wrow[i] = a.w + (n < N ? n : N - 1) * K + lc * 16;
  });
  Static<0, C::B_LD>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int64_t m = bm0 + lr + i * RSTEP;
    xrow[i] = a.x + (m < M ? m : M - 1) * K + lc * 16;
  });

  // PD register sets of staged chunks: with PD = 2 the loads of step kt + 2
  // are issued while step kt is computed and step kt + 1 waits in the other
  // set, so each load has two steps to arrive.
  constexpr int SETS = C::PD == 1 ? 1 : 2;
  v4i ra[SETS][C::A_LD], rb[SETS][C::B_LD];
  auto load_global = [&](int kt, auto SET) {
    constexpr int st = decltype(SET)::value;
    int64_t ko = (int64_t)kt * C::BK;
    bool kin = true;
    if constexpr (!KFULL) {
      kin = ko + lc * 16 < K;
      if (!kin) ko = K - 16 - lc * 16;
    }
    Static<0, C::A_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const v4i v = *reinterpret_cast<const v4i*>(wrow[i] + ko);
      ra[st][i] = kin ? v : v4i{0, 0, 0, 0};
    });
    Static<0, C::B_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const v4i v = *reinterpret_cast<const v4i*>(xrow[i] + ko);
      rb[st][i] = kin ? v : v4i{0, 0, 0, 0};
    });
  };
  auto store_lds = [&](int buf, auto SET) {
    constexpr int st = decltype(SET)::value;
    int8_t* As = smem + buf * C::STAGE;
    int8_t* Bs = As + C::BN * C::BK;
    Static<0, C::A_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int row = lr + i * RSTEP;
      *reinterpret_cast<v4i*>(As + row * C::BK + 16 * swz<C::CPR>(row, lc)) = ra[st][i];
    });
    Static<0, C::B_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int row = lr + i * RSTEP;
      *reinterpret_cast<v4i*>(Bs + row * C::BK + 16 * swz<C::CPR>(row, lc)) = rb[st][i];
    });
  };

  v16i acc[C::FN][C::FM];
  Static<0, C::FN>::each([&](auto I) {
    Static<0, C::FM>::each([&](auto J) { acc[decltype(I)::value][decltype(J)::value] = v16i{}; });
  });
  int32_t wsum[C::FN];
  Static<0, C::FN>::each([&](auto I) { wsum[decltype(I)::value] = 0; });

  // Per-channel constants of tile row tid, fetched before the K loop so their
  // latency hides behind it.  Scales and bias exist only for the requantizing
  // calls (the accumulator entry point passes no weight_scales).
  float e_sc = 0.0f, e_bi = 0.0f;
  int32_t e_ws = 0;
  if (tid < C::BN && !a.acc && bn0 + tid < N) {
    e_sc = a.wscale[bn0 + tid];
    e_bi = a.bias ? a.bias[bn0 + tid] : 0.0f;
  }
  if (PRE && tid < C::BN && bn0 + tid < N) e_ws = a.wsum_pre[bn0 + tid];

  const int lrow = lane & 31;
  const int kg = lane >> 5;
  const int a_off = (wn * C::WN + lrow) * C::BK;
  const int b_off = C::BN * C::BK + (wm * C::WM + lrow) * C::BK;
  auto compute = [&](int buf) {
    const int8_t* S = smem + buf * C::STAGE;
    Static<0, C::KS>::each([&](auto KSI) {
      constexpr int ks = decltype(KSI)::value;
      const int cpos = 16 * swz<C::CPR>(lrow, 2 * ks + kg);
      v4i af[C::FN], bf[C::FM];
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        af[i] = *reinterpret_cast<const v4i*>(S + a_off + i * 32 * C::BK + cpos);
      });
      Static<0, C::FM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        bf[j] = *reinterpret_cast<const v4i*>(S + b_off + j * 32 * C::BK + cpos);
      });
      if constexpr (!PRE) {
        // the WAVES_M waves of one W strip take turns over the K slices
        if (C::WAVES_M == 1 || ks % C::WAVES_M == wm) {
          Static<0, C::FN>::each([&](auto I) {
            constexpr int i = decltype(I)::value;
            wsum[i] = __builtin_amdgcn_sdot4(af[i][0], 0x01010101, wsum[i], false);
            wsum[i] = __builtin_amdgcn_sdot4(af[i][1], 0x01010101, wsum[i], false);
            wsum[i] = __builtin_amdgcn_sdot4(af[i][2], 0x01010101, wsum[i], false);
            wsum[i] = __builtin_amdgcn_sdot4(af[i][3], 0x01010101, wsum[i], false);
          });
        }
      }
      Static<0, C::FN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        Static<0, C::FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          if constexpr (TR)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        });
      });
    });
  };

  // Loads and LDS writes are issued on every step, also past the last one
  // (the step index is clamped: a repeated fetch of the last slab, written to
  // the buffer no one reads any more), so the loop carries no branch around
  // them.
  constexpr std::integral_constant<int, 0> S0{};
  load_global(0, S0);
  store_lds(0, S0);
  if constexpr (C::PD == 1) {
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      load_global(min(kt + 1, KT - 1), S0);
      compute(cur);
      store_lds(cur ^ 1, S0);
      __syncthreads();
    }
  } else if constexpr (C::PD == 2) {
    constexpr std::integral_constant<int, 1> S1{};
    load_global(min(1, KT - 1), S1);
    __syncthreads();
    // step kt reads LDS buffer kt % 2 and register set (kt + 1) % 2 holds
    // step kt + 1; the body always runs both halves (a break between them
    // would leave a path on which the wait counts turn conservative)
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      load_global(min(kt + 2, KT - 1), S0);
      compute(0);
      store_lds(1, S1);
      __syncthreads();
      load_global(min(kt + 3, KT - 1), S1);
      compute(1);
      store_lds(0, S0);
      __syncthreads();
    }
    if (kt < KT) compute(0);   // odd KT: the last step sits in buffer 0
  } else {
    // Store first: at the top of step kt the set holding step kt + 1 (loaded
    // two steps earlier) is written to buffer (kt + 1) % 2 -- read last in
    // step kt - 1, before the barrier that ended it -- and immediately
    // refilled with step kt + 3; then step kt is computed from buffer
    // kt % 2.  The LDS writes overlap the step's matrix-core work instead of
    // delaying the barrier, and each load still has two steps to arrive.
    constexpr std::integral_constant<int, 1> S1{};
    load_global(min(1, KT - 1), S1);
    load_global(min(2, KT - 1), S0);
    __syncthreads();
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      store_lds(1, S1);
      load_global(min(kt + 3, KT - 1), S1);
      compute(0);
      __syncthreads();
      store_lds(0, S0);
      load_global(min(kt + 4, KT - 1), S0);
      compute(1);
      __syncthreads();
    }
    if (kt < KT) compute(0);   // odd KT: the last step sits in buffer 0
  }

  // Row sums: lane l holds a partial of row l % 32 of fragment i over its
  // 16-byte halves (l / 32) of this wave's K slices; lanes l and l ^ 32 cover
  // the row, the WAVES_M waves of the strip cover K.
  if constexpr (!PRE) {
    Static<0, C::FN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      int32_t v = wsum[i];
      v += __shfl_xor(v, 32, 64);
      if (kg == 0) epi_ws[wm][cslot<C::BN>(wn * C::WN + i * 32 + lrow)] = v;
    });
  } else {
    if (tid < C::BN) epi_ws[0][cslot<C::BN>(tid)] = e_ws;
  }
  if (tid < C::BN) {
    epi_sc[cslot<C::BN>(tid)] = e_sc;
    epi_bi[cslot<C::BN>(tid)] = e_bi;
  }
  __syncthreads();

  constexpr int NWS = PRE ? 1 : C::WAVES_M;
  // Interior tiles of an output with fewer than 2^31 elements take the store
  // path without bounds checks: each lane's element offset is one 32-bit
  // value per channel, and the row offsets c * N are wave-uniform (scalar).
  const bool fast = bm0 + C::BM <= M && bn0 + C::BN <= N && M * N <= (int64_t)INT32_MAX;
  if constexpr (TR) {
    // lane l: channel n of tile row wn*WN + i*32 + l % 32; register r: output
    // row m of fragment j at 8 * (r / 4) + 4 * (l / 32) + r % 4
    const float dq_zpf = (float)a.dq_zp;
    Static<0, C::FN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int rr = wn * C::WN + i * 32 + lrow;
      const int sl = cslot<C::BN>(rr);
      int32_t ws = epi_ws[0][sl];
      Static<1, NWS>::each([&](auto W) { ws += epi_ws[decltype(W)::value][sl]; });
      const int32_t zc = a.izp * ws;
      const float sc = epi_sc[sl], bi = epi_bi[sl];
      const int64_t n = bn0 + rr;
      if (fast) {
        const uint32_t lane_off = (uint32_t)((bm0 + wm * C::WM + 4 * kg) * N + n);
        Static<0, C::FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          Static<0, 16>::each([&](auto R) {
            constexpr int r = decltype(R)::value;
            constexpr int c = j * 32 + 8 * (r / 4) + r % 4;
            const float q = requant_code(acc[i][j][r] - zc, sc, bi, a.rq);
            float* rb = a.outf + (int64_t)c * N;   // wave-uniform row base
            rb[lane_off] = (q - dq_zpf) * a.dq_scale;
          });
        });
      } else if (n < N) {
        Static<0, C::FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          Static<0, 16>::each([&](auto R) {
            constexpr int r = decltype(R)::value;
            const int64_t m = bm0 + wm * C::WM + j * 32 + 8 * (r / 4) + 4 * kg + r % 4;
            if (m < M) {
              const float q = requant_code(acc[i][j][r] - zc, sc, bi, a.rq);
              a.outf[m * N + n] = (q - dq_zpf) * a.dq_scale;
            }
          });
        });
      }
    });
    return;
  }
  // int8 (or int32 accumulator) output
  const bool vec_out = (N % 4) == 0 && ((uintptr_t)a.out & 3) == 0;
  Static<0, C::FN>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    Static<0, 4>::each([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int rr = wn * C::WN + i * 32 + 8 * g + 4 * kg;   // tile row of registers 4g..4g+3
      const int64_t nb = bn0 + rr;
      int32_t wsv[4];
      float sc[4], bi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sl = cslot<C::BN>(rr + r);
        wsv[r] = epi_ws[0][sl];
        Static<1, NWS>::each([&](auto W) { wsv[r] += epi_ws[decltype(W)::value][sl]; });
        sc[r] = epi_sc[sl];
        bi[r] = epi_bi[sl];
      }
      int32_t zc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) zc[r] = a.izp * wsv[r];
      if (fast && vec_out && !a.acc) {
        const uint32_t lane_off = (uint32_t)((bm0 + wm * C::WM + lrow) * N + nb);
        Static<0, C::FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          float q[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) q[r] = requant_code(acc[i][j][4 * g + r] - zc[r], sc[r], bi[r], a.rq);
          int8_t* rb = a.out + (int64_t)(j * 32) * N;   // wave-uniform row base
          *reinterpret_cast<uint32_t*>(rb + lane_off) = pack4((int)q[0], (int)q[1], (int)q[2], (int)q[3]);
        });
        return;
      }
      Static<0, C::FM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int64_t m = bm0 + wm * C::WM + j * 32 + lrow;
        if (m < M) {
          int32_t c[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) c[r] = acc[i][j][4 * g + r] - zc[r];
          if (a.acc) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (nb + r < N) a.acc[m * N + nb + r] = c[r];
          } else {
            float q[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) q[r] = requant_code(c[r], sc[r], bi[r], a.rq);
            if (vec_out && nb + 3 < N) {
              *reinterpret_cast<uint32_t*>(a.out + m * N + nb) =
                  pack4((int)q[0], (int)q[1], (int)q[2], (int)q[3]);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (nb + r < N) a.out[m * N + nb + r] = (int8_t)(int)q[r];
            }
          }
        }
      });
    });
  });
}

// Two workgroups per CU: 256 x 128 tiles, 128 x 64 per wave, 64-byte K steps,
// store-first K loop (loads three steps ahead).
using MxY3 = MxCfg<256, 128, 64, 2, 2, 2, 3>;

template <class C, bool PRE>
hipError_t launch_mx2(const LinearArgs& a, int tiles_m, int tiles_n, hipStream_t s) {
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  // fp32 output (fused dequantize): the transposed form, whole-line stores
  const bool tr = a.outf != nullptr && a.acc == nullptr;
  if (a.K % C::BK == 0) {
    if (tr)
      hipLaunchKernelGGL((k_gemm_mx<C, PRE, true, true>), grid, dim3(C::NT), 0, s, a, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((k_gemm_mx<C, PRE, true, false>), grid, dim3(C::NT), 0, s, a, tiles_m,
                         tiles_n);
  } else {
    if (tr)
      hipLaunchKernelGGL((k_gemm_mx<C, PRE, false, true>), grid, dim3(C::NT), 0, s, a, tiles_m,
                         tiles_n);
    else
      hipLaunchKernelGGL((k_gemm_mx<C, PRE, false, false>), grid, dim3(C::NT), 0, s, a, tiles_m,
                         tiles_n);
  }
  return hipGetLastError();
}

template <class C>
hipError_t launch_mx(const LinearArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.N + C::BN - 1) / C::BN);
  if (a.wsum_pre) return launch_mx2<C, true>(a, tiles_m, tiles_n, s);
  return launch_mx2<C, false>(a, tiles_m, tiles_n, s);
}

}  // namespace

hipError_t launch_gemm_mx(const LinearArgs& a, hipStream_t s) { return launch_mx<MxY3>(a, s); }

}  // namespace q8ta
