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
//  * Each wave owns a 128 x 64 sub-tile (W rows x X rows): 8 accumulator
//    fragments of 16 registers.  Every K byte then costs the wave 192 bytes
//    of LDS fragment reads for 16384 operations.
//  * Two workgroups of four waves share a CU (up to 256 registers per wave,
//    two waves per SIMD, 2 x 24 KiB of LDS buffers): their barriers and
//    epilogues are independent.  A lone workgroup on a CU (the last partial
//    wave of tiles) runs a tile in about half the time of a pair, so the CU's
//    throughput is the same with one or two.
//  * K advances 64 bytes per step through two LDS buffers.  The slabs are
//    staged in registers (16 B per load; rows past M/N read the last row,
//    chunks past K are zeroed), loaded two steps ahead and written to the
//    buffer the matrix cores are not reading; one barrier per step.  Within
//    a step the issue order is fixed with scheduling barriers: slice 0's
//    fragment reads, then the 16 products, the first six each followed by
//    one LDS write of the next step's slab, the load refilling that register
//    and one fragment read of slice 1.  (Measured on 2048 x 4096 x 11008:
//    116-123 us against 124-131 us for the compiler's own order; loading
//    the slabs straight into LDS with global_load_lds_dwordx4 over three
//    stages measured 122-126 us, and 128-byte steps with one workgroup per
//    CU 135 us.)
//  * The 16-byte chunk c of LDS row r sits at chunk position c ^ f(r), f
//    chosen so that the 16 lanes one ds_read_b128 cycle serves hit distinct
//    banks.
//  * Lane l supplies row l % 32 of each operand with K bytes 16 * (l / 32)
//    .. +15 of each 32-byte slice; accumulator register r of lane l holds row
//    8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32 of the product.
//    For int8 output W is the A operand and X the B operand, so registers
//    4g .. 4g+3 are four consecutive output channels of one row (one 32-bit
//    store); for fp32 output (fused dequantize) the operands swap, so lane l
//    holds one channel and each half-wave store writes 32 consecutive floats
//    of one row, a whole 128-byte line.
//  * sum w is taken in the loader: each thread sums the bytes of the W
//    chunks it passes from global memory to LDS with v_dot4 against
//    0x01010101 (steps past the last one, repeated fetches of the last slab,
//    are masked out), and the four threads of a row add their partials after
//    the loop.
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

// 256 x 128 tiles (W rows x X rows), 2 x 2 waves of 128 x 64, 64-byte K
// steps, two workgroups per CU.
struct Cfg {
  static constexpr int BN = 256, BM = 128, BK = 64;
  static constexpr int WAVES_N = 2, WAVES_M = 2, BLOCKS_PER_CU = 2;
  static constexpr int NT = 64 * WAVES_N * WAVES_M;
  static constexpr int WN = BN / WAVES_N, WM = BM / WAVES_M;
  static constexpr int FN = WN / 32, FM = WM / 32;
  static constexpr int CPR = BK / 16;            // 16-byte chunks per LDS row
  static constexpr int KS = BK / 32;             // 32-byte MFMA slices per step
  static constexpr int A_LD = BN * CPR / NT;     // W chunks per thread per step
  static constexpr int B_LD = BM * CPR / NT;     // X chunks per thread per step
  static constexpr int STAGE = (BN + BM) * BK;   // bytes per LDS buffer
  static_assert(KS == 2, "two slices per step");
  static_assert((BN * CPR) % NT == 0 && (BM * CPR) % NT == 0, "loader");
  static_assert(NT % CPR == 0, "a thread keeps its chunk column");
  static_assert(BN <= NT, "one channel per thread in the epilogue staging");
  static_assert(A_LD + B_LD <= FN * FM && FN + FM <= A_LD + B_LD, "interleave slots");
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

// PRE: the row sums of W come from a.wsum_pre (trusted, precomputed by the
// caller) instead of the loader's v_dot4.
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
  __shared__ __attribute__((aligned(16))) int32_t epi_ws[C::BN];

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

  // Two register sets of staged chunks: while step kt is computed, the set
  // holding step kt + 1 is written to LDS and refilled with step kt + 3.
  v4i ra[2][C::A_LD], rb[2][C::B_LD];
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

  v16i acc[C::FN][C::FM];
  Static<0, C::FN>::each([&](auto I) {
    Static<0, C::FM>::each([&](auto J) { acc[decltype(I)::value][decltype(J)::value] = v16i{}; });
  });
  // sum w in the loader: thread tid passes the W chunks of rows lr + i * RSTEP,
  // chunk column lc, through its registers and sums their bytes with v_dot4
  // as it writes them to LDS.
  int32_t lsum[C::A_LD];
  Static<0, C::A_LD>::each([&](auto I) { lsum[decltype(I)::value] = 0; });

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

  // LDS write of staged chunk m of register set SET into buffer buf (W chunks
  // first), with its row sums when it is a W chunk of a real step
  auto write_chunk = [&](int8_t* As, auto SET, auto MI, int ones) {
    constexpr int st = decltype(SET)::value, m = decltype(MI)::value;
    int8_t* Bs = As + C::BN * C::BK;
    if constexpr (m < C::A_LD) {
      const int row = lr + m * RSTEP;
      *reinterpret_cast<v4i*>(As + row * C::BK + 16 * swz<C::CPR>(row, lc)) = ra[st][m];
      if constexpr (!PRE) {
        Static<0, 4>::each([&](auto D) {
          lsum[m] = __builtin_amdgcn_sdot4(ra[st][m][decltype(D)::value], ones, lsum[m], false);
        });
      }
    } else {
      constexpr int q = m - C::A_LD;
      const int row = lr + q * RSTEP;
      *reinterpret_cast<v4i*>(Bs + row * C::BK + 16 * swz<C::CPR>(row, lc)) = rb[st][q];
    }
  };
  auto load_chunk = [&](auto SET, auto MI, int64_t ko, bool kin) {
    constexpr int st = decltype(SET)::value, m = decltype(MI)::value;
    if constexpr (m < C::A_LD) {
      const v4i v = *reinterpret_cast<const v4i*>(wrow[m] + ko);
      ra[st][m] = kin ? v : v4i{0, 0, 0, 0};
    } else {
      constexpr int q = m - C::A_LD;
      const v4i v = *reinterpret_cast<const v4i*>(xrow[q] + ko);
      rb[st][q] = kin ? v : v4i{0, 0, 0, 0};
    }
  };
  auto product = [&](const v4i (&af)[C::FN], const v4i (&bf)[C::FM], auto I, auto J) {
    constexpr int i = decltype(I)::value, j = decltype(J)::value;
    if constexpr (TR)
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
  };
  auto read_frag = [&](const int8_t* S, v4i (&af)[C::FN], v4i (&bf)[C::FM], auto KSI, auto R) {
    constexpr int ks = decltype(KSI)::value, r = decltype(R)::value;
    const int cpos = 16 * swz<C::CPR>(lrow, 2 * ks + kg);
    if constexpr (r < C::FN)
      af[r] = *reinterpret_cast<const v4i*>(S + a_off + r * 32 * C::BK + cpos);
    else
      bf[r - C::FN] = *reinterpret_cast<const v4i*>(S + b_off + (r - C::FN) * 32 * C::BK + cpos);
  };
  constexpr int NR = C::FN + C::FM;          // fragment reads per slice
  constexpr int NW = C::A_LD + C::B_LD;      // staged chunks per step
  constexpr int NP = C::FN * C::FM;          // products per slice
  constexpr std::integral_constant<int, 0> K0{};
  constexpr std::integral_constant<int, 1> K1{};

  // Step on LDS buffer buf: its products, interleaved with writing register
  // set SET (step st_step) into buffer nbuf and refilling SET with step
  // ld_step.  The order is fixed with scheduling barriers (see the header).
  auto step = [&](int buf, int nbuf, auto SET, int st_step, int ld_step) {
    const int8_t* S = smem + buf * C::STAGE;
    int8_t* As = smem + nbuf * C::STAGE;
    v4i af[2][C::FN], bf[2][C::FM];
    const int ones = st_step < KT ? 0x01010101 : 0;
    int64_t ko = (int64_t)ld_step * C::BK;
    bool kin = true;
    if constexpr (!KFULL) {
      kin = ko + lc * 16 < K;
      if (!kin) ko = K - 16 - lc * 16;
    }
    Static<0, NR>::each([&](auto R) { read_frag(S, af[0], bf[0], K0, R); });
    __builtin_amdgcn_sched_barrier(0);
    Static<0, 2 * NP>::each([&](auto MI) {
      constexpr int m = decltype(MI)::value;
      constexpr int ks = m / NP, i = (m % NP) / C::FM, j = m % C::FM;
      product(af[ks], bf[ks], std::integral_constant<int, i>{}, std::integral_constant<int, j>{});
      if constexpr (m < NW) {
        write_chunk(As, SET, MI, ones);
        load_chunk(SET, MI, ko, kin);
      }
      if constexpr (m < NR) read_frag(S, af[1], bf[1], K1, MI);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // a whole step from LDS buffer 0 without staging work (an odd last step)
  auto step_last = [&]() {
    v4i af[2][C::FN], bf[2][C::FM];
    Static<0, NR>::each([&](auto R) {
      read_frag(smem, af[0], bf[0], K0, R);
      read_frag(smem, af[1], bf[1], K1, R);
    });
    Static<0, 2 * NP>::each([&](auto MI) {
      constexpr int m = decltype(MI)::value;
      constexpr int ks = m / NP, i = (m % NP) / C::FM, j = m % C::FM;
      product(af[ks], bf[ks], std::integral_constant<int, i>{}, std::integral_constant<int, j>{});
    });
  };

  // Loads and LDS writes are issued on every step, also past the last one
  // (the step index is clamped: a repeated fetch of the last slab, written to
  // the buffer no one reads any more), so the loop carries no branch around
  // them.  Step kt reads LDS buffer kt % 2; at its top the register set
  // holding step kt + 1 (loaded two steps earlier) goes to buffer (kt + 1) % 2
  // -- read last in step kt - 1, before the barrier that ended it.
  constexpr std::integral_constant<int, 0> S0{};
  constexpr std::integral_constant<int, 1> S1{};
  load_global(0, S0);
  Static<0, NW>::each([&](auto MI) { write_chunk(smem, S0, MI, 0x01010101); });
  load_global(min(1, KT - 1), S1);
  load_global(min(2, KT - 1), S0);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    step(0, 1, S1, kt + 1, min(kt + 3, KT - 1));
    __syncthreads();
    step(1, 0, S0, kt + 2, min(kt + 4, KT - 1));
    __syncthreads();
  }
  if (kt < KT) step_last();   // odd KT: the last step sits in buffer 0

  // Row sums: the CPR threads of a row (consecutive lanes) add their chunk
  // columns.
  if constexpr (!PRE) {
    Static<0, C::A_LD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      int32_t v = lsum[i];
      Static<1, C::CPR>::each([&](auto B) {
        constexpr int bit = decltype(B)::value;
        if constexpr ((bit & (bit - 1)) == 0) v += __shfl_xor(v, bit, 64);
      });
      if (lc == 0) epi_ws[cslot<C::BN>(lr + i * RSTEP)] = v;
    });
  } else {
    if (tid < C::BN) epi_ws[cslot<C::BN>(tid)] = e_ws;
  }
  if (tid < C::BN) {
    epi_sc[cslot<C::BN>(tid)] = e_sc;
    epi_bi[cslot<C::BN>(tid)] = e_bi;
  }
  __syncthreads();

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
      const int32_t zc = a.izp * epi_ws[sl];
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
        wsv[r] = epi_ws[sl];
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


template <bool PRE>
hipError_t launch_mx2(const LinearArgs& a, int tiles_m, int tiles_n, hipStream_t s) {
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  // fp32 output (fused dequantize): the transposed form, whole-line stores
  const bool tr = a.outf != nullptr && a.acc == nullptr;
  if (a.K % Cfg::BK == 0) {
    if (tr)
      hipLaunchKernelGGL((k_gemm_mx<Cfg, PRE, true, true>), grid, dim3(Cfg::NT), 0, s, a, tiles_m,
                         tiles_n);
    else
      hipLaunchKernelGGL((k_gemm_mx<Cfg, PRE, true, false>), grid, dim3(Cfg::NT), 0, s, a, tiles_m,
                         tiles_n);
  } else {
    if (tr)
      hipLaunchKernelGGL((k_gemm_mx<Cfg, PRE, false, true>), grid, dim3(Cfg::NT), 0, s, a, tiles_m,
                         tiles_n);
    else
      hipLaunchKernelGGL((k_gemm_mx<Cfg, PRE, false, false>), grid, dim3(Cfg::NT), 0, s, a,
                         tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const LinearArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + Cfg::BM - 1) / Cfg::BM);
  const int tiles_n = (int)((a.N + Cfg::BN - 1) / Cfg::BN);
  if (a.wsum_pre) return launch_mx2<true>(a, tiles_m, tiles_n, s);
  return launch_mx2<false>(a, tiles_m, tiles_n, s);
}

}  // namespace q8ta
