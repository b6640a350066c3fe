// q8ta_linear GEMM for problems that fill the GPU, eight waves per CU
// ("Add q8ta_linear op", Solution: acc[m,n] = sum_k (x[m,k] - izp) * w[n,k]
// in int32, then the per-channel dequant/requant epilogue; Constraints (1):
// the zero-point term folded as sum x*w - izp * sum w; Constraints (2): x
// [M,K] and w [N,K] K-contiguous).
//
// Why this shape on gfx950:
//  * One workgroup of eight waves per CU owns a 256 x 256 output tile (256
//    weight rows x 256 activation rows), two waves per SIMD, each wave 128 x
//    64 (4 x 2 fragments of 32 x 32; wave w takes weight rows 128 * (w / 4)
//    and activation rows 64 * (w % 4)).  Each 64-byte K step moves 32 KiB
//    into LDS for 4 Mi multiply-adds, 1.5 times the operations per byte of
//    L2 reads of a 256 x 128 tile.  The accumulators of a 256 x 256 tile are
//    as much as two waves per SIMD can hold, so a larger tile per CU would
//    need one wave per SIMD -- which measured slower (a 4-wave form with 128 x
//    128 per wave and the accumulators in AGPRs: 75.1 us against 70.9 us on
//    2048 x 4096 x 8192), the second wave's latency hiding being worth more
//    than the third of the fragment reads it would save.
//  * On 2048 x 4096 x 8192 (256 tiles, one per CU) the kernel takes 68.6-70.9
//    us; without the stores 61, without the slab loads 59, without the
//    fragment reads 63, the matrix-core work alone 39 us (2.75 POP/s, close
//    to what a register-only v_mfma loop sustains on operands with the bit
//    statistics of quantized data: 2.9-3.1 POP/s).
//  * Problems whose tiles do not fill the CUs a whole number of times would
//    run a partial last round (2048 x 11008: 344 tiles, 88 in the last).
//    Instead the columns left after whole rounds are covered by 256 x 128
//    tiles (eight waves of 64 x 64) when those fit one round, in the same
//    launch after the 256 x 256 ones, so that they start on the CUs the first
//    whole tiles free (C3: 176 half tiles; 100.6-104.9 us, against ~120 us
//    with 88 whole tiles in the last round and 109-114 us with the half
//    tiles as a second launch).  Problems of at most 128 whole tiles run as
//    256 x 128 tiles throughout when that fills more CUs.  Splitting the
//    last tiles along K over two workgroups instead measured slower (132 us
//    against 112 us): each piece's int32 partial tile (256 KiB) has to go
//    through memory to the other piece, as much traffic as the split saves.
//  * The slabs go straight from global memory into LDS
//    (global_load_lds_dwordx4: each instruction moves 16 rows x 64 bytes;
//    lane l's 16 bytes land at LDS offset 16 * l of the instruction's base;
//    the address is a wave-uniform scalar base plus a 32-bit lane offset)
//    through three LDS stages.  Each stage is a separate __shared__ object
//    and each step of the unrolled loop names its stages at compile time:
//    with a runtime stage index the compiler cannot tell the stage being
//    loaded from the one being read and waits for every load in flight
//    before each fragment read.  The waits for the slabs are explicit
//    (s_waitcnt vmcnt before the one barrier per step), and the barrier is
//    the bare s_barrier (__syncthreads would also wait for the loads of the
//    next steps).  The barrier sits in the middle of a step, between the
//    products of its two 32-byte slices, so that the fragment reads always
//    run behind products and the slab of step k + 3 is requested as soon as
//    stage k % 3 is free.
//  * The 16-byte chunk c of LDS row r sits at chunk position c ^ ((r >> 2) &
//    3), conflict-free for the 32x32x32 fragment reads; the swizzle is
//    applied on the global side (lane l of a load instruction fetches the
//    chunk that belongs at its fixed LDS position).
//  * Lane l supplies row l % 32 of each operand with K bytes 16 * (l / 32)
//    .. +15 of each 32-byte slice; accumulator register r of lane l holds row
//    8 * (r / 4) + 4 * (l / 32) + r % 4 and column l % 32 of the product.
//    For int8 output W is the A operand and X the B operand (registers 4g ..
//    4g+3 are four consecutive channels of one row: one 32-bit store); for
//    fp32 output the operands swap, so each half-wave store writes 32
//    consecutive floats of one row.
//  * sum w is taken from the W fragments the waves read anyway, with v_dot4
//    against 0x01010101 co-issued with the products: of the four waves that
//    read the same weight rows, each sums one slice of half the fragments
//    (the same work on every SIMD: with two of the four waves summing every
//    fragment the kernel measured 3 us slower on 2048 x 4096 x 8192), and
//    the partials meet in LDS after the loop.
//  * Rows past M or N read the last row (their products land in outputs
//    that are not stored); K must be a multiple of 64 (no partial steps).
#include <type_traits>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
#define Q8TA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

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

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt 0, expcnt any.
constexpr int wait_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// TN x BM tile, 64-byte K steps, WAVES_N x WAVES_M waves of FN x FM
// fragments of 32 x 32 (wave (wn, wm) owns weight rows 32 * FN * wn .. and
// activation rows 32 * FM * wm ..).
template <int WAVES_N_, int WAVES_M_, int FN_, int FM_>
struct Tile {
  static constexpr int WAVES_N = WAVES_N_, WAVES_M = WAVES_M_, FN = FN_, FM = FM_;
  static constexpr int WAVES = WAVES_N * WAVES_M, NT = 64 * WAVES;
  static constexpr int TN = 32 * FN * WAVES_N, BM = 32 * FM * WAVES_M, BK = 64;
  static constexpr int NBW = TN / 16, NBX = BM / 16;   // 16-row blocks of one step
  static constexpr int NQ = (NBW + NBX + WAVES - 1) / WAVES;   // load instructions per wave per step
  // bytes per stage: the blocks at 1 KiB each (W first, then X), then the
  // landing place of the padding loads that even out the waves' counts
  static constexpr int STAGE = WAVES * NQ * 1024;
  static constexpr int CR = (TN + NT - 1) / NT;   // per-channel constants per thread
};

__device__ __forceinline__ int swz4(int r, int c) { return c ^ ((r >> 2) & 3); }

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
// register group sit TN / 4 words apart (separate 32-bit broadcast reads).
template <int TN>
__device__ __forceinline__ int cslot(int r) { return (r & 3) * (TN / 4) + (r >> 2); }

struct Smem {
  int8_t* st0;
  int8_t* st1;
  int8_t* st2;
  float* sc;
  float* bi;
  int32_t* ws;
};

// K loop and epilogue of one wave with FN weight fragments (32 rows each)
// starting at tile row wr0 and activation rows xr0 .. xr0 + 63.  SUMK: the W
// slice this wave sums for sum w (-1: none; PRE: never).
template <class T, int SUMK, int SPAR, bool PRE, bool TR, bool PK>
__device__ __forceinline__ void run(const LinearArgs& a, const Smem& sm,
                                    const int8_t* const (&gb)[T::NQ], const uint32_t (&voff)[T::NQ],
                                    const int (&ldo)[T::NQ], const int (&kst)[T::NQ],
                                    int wr0, int xr0, int lane, int tid, int KT, int64_t bm0,
                                    int64_t bn0, const float (&e_sc)[T::CR],
                                    const float (&e_bi)[T::CR]) {
  constexpr int FN = T::FN, FM = T::FM;
  constexpr int NR = FN + FM;   // fragment reads per slice
  constexpr int NP = FN * FM;   // products per slice
  const int64_t M = a.M, N = a.N;
  const int lrow = lane & 31, kg = lane >> 5;
  const int a_off = (wr0 + lrow) * T::BK;
  const int b_off = T::TN * T::BK + (xr0 + lrow) * T::BK;

  auto stage = [&](auto SI) -> int8_t* {
    constexpr int si = decltype(SI)::value;
    if constexpr (si == 0) return sm.st0;
    else if constexpr (si == 1) return sm.st1;
    else return sm.st2;
  };
  auto issue = [&](int k, auto SI) {
    int8_t* d = stage(SI);
    Static<0, T::NQ>::each([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      __builtin_amdgcn_global_load_lds((const void*)(gb[q] + (int64_t)k * kst[q] + voff[q]),
                                       Q8TA_LDS(d + ldo[q]), 16, 0, 0);
    });
  };

  v16i acc[FN][FM];
  Static<0, FN>::each([&](auto I) {
    Static<0, FM>::each([&](auto J) { acc[decltype(I)::value][decltype(J)::value] = v16i{}; });
  });
  int32_t wsum[FN];
  Static<0, FN>::each([&](auto I) { wsum[decltype(I)::value] = 0; });

  auto read_frag = [&](const int8_t* S, v4i (&af)[FN], v4i (&bf)[FM], auto KSI, auto R) {
    constexpr int ks = decltype(KSI)::value, r = decltype(R)::value;
    const int cpos = 16 * swz4(lrow, 2 * ks + kg);
    if constexpr (r < FN && PK)   // 1 KiB fragments (32-row block, slice) in lane order
      af[r] = *reinterpret_cast<const v4i*>(S + ((wr0 / 32 + r) * 2 + ks) * 1024 + 16 * lane);
    else if constexpr (r < FN)
      af[r] = *reinterpret_cast<const v4i*>(S + a_off + r * 32 * T::BK + cpos);
    else
      bf[r - FN] = *reinterpret_cast<const v4i*>(S + b_off + (r - FN) * 32 * T::BK + cpos);
  };
  auto product = [&](const v4i (&af)[FN], const v4i (&bf)[FM], auto I, auto J) {
    constexpr int i = decltype(I)::value, j = decltype(J)::value;
    if constexpr (TR)
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], af[i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
  };
  constexpr std::integral_constant<int, 0> K0{};
  constexpr std::integral_constant<int, 1> K1{};

  // Step k (its slab in stage SI = k % 3, slice 0's fragments already in
  // registers) in two halves around the step's one barrier:
  //   first half: the products of slice 0, each followed by one fragment read
  //     of slice 1;
  //   wait for this wave's part of step k + 1 (step k + 2 may stay in flight)
  //     and for its fragment reads; barrier: every wave's part of step k + 1
  //     has landed and every wave is done reading stage SI;
  //   second half: load step k + 3 into stage SI, then the products of slice
  //     1, each followed by one fragment read of step k + 1's slice 0.
  // The fragment reads thus run behind products, never right after the
  // barrier, and the loads are issued about two and a half steps ahead.  The
  // summing waves add the v_dot4 of one W fragment after a product of the
  // half whose fragments they sum.
  v4i af[2][FN], bf[2][FM];
  auto sum_frag = [&](auto KSI, auto MI) {
    constexpr int ks = decltype(KSI)::value, m = decltype(MI)::value;
    if constexpr (!PRE && SUMK == ks && m < FN && (SPAR < 0 || m % 2 == SPAR)) {
      Static<0, 4>::each([&](auto D) {
        wsum[m] = __builtin_amdgcn_sdot4(af[ks][m][decltype(D)::value], 0x01010101, wsum[m], false);
      });
    }
  };
  auto body = [&](int k, auto SI) {
    constexpr int si = decltype(SI)::value;
    using SNX = std::integral_constant<int, (si + 1) % 3>;
    const int8_t* S = stage(SI);
    const int8_t* SN = stage(SNX{});
    Static<0, NP>::each([&](auto MI) {
      constexpr int m = decltype(MI)::value;
      product(af[0], bf[0], std::integral_constant<int, m / FM>{}, std::integral_constant<int, m % FM>{});
      if constexpr (m < NR) read_frag(S, af[1], bf[1], K1, MI);
      sum_frag(K0, MI);
      __builtin_amdgcn_sched_barrier(0);
    });
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(T::NQ));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(k + 3 < KT ? k + 3 : KT - 1, SI);
    __builtin_amdgcn_sched_barrier(0);
    Static<0, NP>::each([&](auto MI) {
      constexpr int m = decltype(MI)::value;
      product(af[1], bf[1], std::integral_constant<int, m / FM>{}, std::integral_constant<int, m % FM>{});
      if constexpr (m < NR) read_frag(SN, af[0], bf[0], K0, MI);
      sum_frag(K1, MI);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  constexpr std::integral_constant<int, 0> S0{};
  constexpr std::integral_constant<int, 1> S1{};
  constexpr std::integral_constant<int, 2> S2{};
  issue(0, S0);
  issue(KT > 1 ? 1 : 0, S1);
  issue(KT > 2 ? 2 : KT - 1, S2);
  __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * T::NQ));   // this wave's part of step 0
  __builtin_amdgcn_s_barrier();
  Static<0, NR>::each([&](auto R) { read_frag(sm.st0, af[0], bf[0], K0, R); });
  int k = 0;
  for (; k + 3 <= KT; k += 3) {
    body(k, S0);
    body(k + 1, S1);
    body(k + 2, S2);
  }
  if (k < KT) body(k, S0);
  if (k + 1 < KT) body(k + 1, S1);
  __builtin_amdgcn_s_waitcnt(0);

  // sum w: the two lanes of a row (two K halves) and the two waves that
  // summed its two slices meet in LDS (zeroed before the loop).
  if constexpr (!PRE && SUMK >= 0) {
    Static<0, FN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (SPAR < 0 || i % 2 == SPAR)
        atomicAdd(&sm.ws[cslot<T::TN>(wr0 + i * 32 + lrow)], wsum[i]);
    });
  }
  Static<0, T::CR>::each([&](auto C) {
    constexpr int c = decltype(C)::value;
    const int row = tid + c * T::NT;
    if (row < T::TN) {
      sm.sc[cslot<T::TN>(row)] = e_sc[c];
      sm.bi[cslot<T::TN>(row)] = e_bi[c];
    }
  });
  __syncthreads();

  // Interior tiles of an output with fewer than 2^31 elements store without
  // bounds checks: one 32-bit element offset per lane, wave-uniform row bases.
  const bool fast = bm0 + T::BM <= M && bn0 + T::TN <= N && M * N <= (int64_t)INT32_MAX;
  if constexpr (TR) {
    // lane l: channel n of tile row wr0 + i*32 + l % 32; register r: output
    // row xr0 + j*32 + 8 * (r / 4) + 4 * (l / 32) + r % 4
    const float dq_zpf = (float)a.dq_zp;
    Static<0, FN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int rr = wr0 + i * 32 + lrow;
      const int sl = cslot<T::TN>(rr);
      const int32_t zc = a.izp * sm.ws[sl];
      const float sc = sm.sc[sl], bi = sm.bi[sl];
      const int64_t n = bn0 + rr;
      if (fast) {
        const uint32_t lane_off = (uint32_t)((bm0 + xr0 + 4 * kg) * N + n);
        Static<0, FM>::each([&](auto J) {
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
        Static<0, FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          Static<0, 16>::each([&](auto R) {
            constexpr int r = decltype(R)::value;
            const int64_t m = bm0 + xr0 + j * 32 + 8 * (r / 4) + 4 * kg + r % 4;
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
  // int8 output of an interior tile with 16-byte aligned rows: the codes go
  // through LDS (the free stages 0 and 1: tile row m of 256 bytes at m * 256,
  // its 16-byte chunk c at chunk position c ^ (m % 16), which keeps the 32
  // rows one ds_write_b32 instruction covers on distinct banks but for pairs)
  // and leave as whole 256-byte row segments, 16 bytes per lane.  Stored
  // straight from the accumulators, each store instruction would cover 32
  // rows with 8 bytes each.
  if (fast && !a.acc && (N % 16) == 0 && ((uintptr_t)a.out & 15) == 0) {
    constexpr int RPS = T::STAGE / T::TN;   // tile rows per stage
    static_assert(3 * RPS >= T::BM, "the int8 tile fits the three stages");
    auto row = [&](int m) {
      return (m < RPS ? sm.st0 : (m < 2 * RPS ? sm.st1 : sm.st2)) + (m % RPS) * T::TN;
    };
    // the four codes of a register group packed in offset form (code + 128)
    // by the conversion itself (one instantiation with the lower clamp, which
    // is 0 without relu: a second copy of this loop costs registers)
    const float ozp128 = a.rq.ozp + 128.0f, qmin128 = a.rq.qmin + 128.0f;
    Static<0, FN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      Static<0, 4>::each([&](auto G) {
        constexpr int g = decltype(G)::value;
        const int rr = wr0 + i * 32 + 8 * g + 4 * kg;   // tile row of registers 4g..4g+3
        int32_t zc[4];
        float sc[4], bi[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sl = cslot<T::TN>(rr + r);
          zc[r] = a.izp * sm.ws[sl];
          sc[r] = sm.sc[sl];
          bi[r] = sm.bi[sl];
        }
        Static<0, FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          const int m = xr0 + j * 32 + lrow;
          uint32_t wd = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            wd = requant_u8<true>(acc[i][j][4 * g + r] - zc[r], sc[r], bi[r], a.rq, ozp128,
                                  qmin128, r, wd);
          *reinterpret_cast<uint32_t*>(row(m) + 16 * ((rr >> 4) ^ (m & (T::TN / 16 - 1))) +
                                       (rr & 15)) = wd ^ 0x80808080u;
        });
      });
    });
    __syncthreads();
    constexpr int CH = T::BM * T::TN / 16;   // 16-byte chunks of the tile
    static_assert(CH % T::NT == 0, "whole chunks per thread");
#pragma unroll
    for (int u = 0; u < CH / T::NT; ++u) {
      const int id = tid + u * T::NT;
      const int m = id / (T::TN / 16), c = id % (T::TN / 16);
      const v4i v = *reinterpret_cast<const v4i*>(row(m) + 16 * (c ^ (m & (T::TN / 16 - 1))));
      *reinterpret_cast<v4i*>(a.out + (bm0 + m) * N + bn0 + 16 * c) = v;
    }
    return;
  }
  // int8 (or int32 accumulator) output, lane by lane
  const bool vec_out = (N % 4) == 0 && ((uintptr_t)a.out & 3) == 0;
  Static<0, FN>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    Static<0, 4>::each([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int rr = wr0 + i * 32 + 8 * g + 4 * kg;   // tile row of registers 4g..4g+3
      const int64_t nb = bn0 + rr;
      int32_t zc[4];
      float sc[4], bi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sl = cslot<T::TN>(rr + r);
        zc[r] = a.izp * sm.ws[sl];
        sc[r] = sm.sc[sl];
        bi[r] = sm.bi[sl];
      }
      if (fast && vec_out && !a.acc) {
        const uint32_t lane_off = (uint32_t)((bm0 + xr0 + lrow) * N + nb);
        Static<0, FM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          float q[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            q[r] = requant_code(acc[i][j][4 * g + r] - zc[r], sc[r], bi[r], a.rq);
          int8_t* rb = a.out + (int64_t)(j * 32) * N;   // wave-uniform row base
          *reinterpret_cast<uint32_t*>(rb + lane_off) =
              pack4((int)q[0], (int)q[1], (int)q[2], (int)q[3]);
        });
        return;
      }
      Static<0, FM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int64_t m = bm0 + xr0 + j * 32 + lrow;
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

// One tile of shape T: tile t of a grid of tiles_m x tiles_n tiles (M
// fastest) covering output columns n0 .. (tile column tn at n0 + tn * TN).
template <class T, bool PRE, bool TR, bool PK>
__device__ __forceinline__ void gemm_tile(const LinearArgs& a, const Smem& sm, int t, int tiles_m,
                                          int64_t n0) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / T::WAVES_M, wm = wave % T::WAVES_M;
  const int KT = (int)(a.K / T::BK);
  const int tm = t % tiles_m;
  const int tn = t / tiles_m;
  const int64_t bn0 = n0 + (int64_t)tn * T::TN;
  const int64_t bm0 = (int64_t)tm * T::BM;
  const int64_t M = a.M, N = a.N, K = a.K;

  // Load instruction q of this wave moves 16-row block wave * NQ + q of a
  // step: W blocks, then X blocks, then padding (a repeat of the tile's first
  // X rows into the stage's tail).  Lane l takes row l / 4 of the block and
  // the chunk that belongs at chunk position l % 4 of that LDS row.
  // The block's base address is wave-uniform (scalar registers) and each
  // lane adds a 32-bit offset within the tile, so a load is one scalar base
  // plus one vector register and a step advances only the scalar base.
  // With a prepacked weight (PK) the W blocks are its 1 KiB fragments
  // instead: block 2j + s of a step is slice s of 32-row block j of the tile,
  // fetched whole (lane l: bytes 16 l ..), two fragments per K step.
  const int8_t* gb[T::NQ];
  uint32_t voff[T::NQ];
  int ldo[T::NQ];
  int kst[T::NQ];   // bytes a step advances the block's source
  {
    const int br = lane >> 2;
    const int chunk = swz4(br, lane & 3);
    Static<0, T::NQ>::each([&](auto Q) {
      constexpr int q = decltype(Q)::value;
      const int blk = wave * T::NQ + q;
      ldo[q] = blk * 1024;
      kst[q] = T::BK;
      if (blk < T::NBW && PK) {
        const int64_t KS = 2 * (K / 64), NB = (N + 31) / 32;
        const int64_t nb = bn0 / 32 + blk / 2;
        gb[q] = a.wpk;
        voff[q] = (uint32_t)(((nb < NB ? nb : NB - 1) * KS + (blk & 1)) * 1024 + 16 * lane);
        kst[q] = 2048;
      } else if (blk < T::NBW) {
        const int64_t n = bn0 + 16 * blk + br;
        gb[q] = a.w + bn0 * K;
        voff[q] = (uint32_t)(((n < N ? n : N - 1) - bn0) * K + 16 * chunk);
      } else {
        const int xb = blk < T::NBW + T::NBX ? blk - T::NBW : 0;
        const int64_t m = bm0 + 16 * xb + br;
        gb[q] = a.x + bm0 * K;
        voff[q] = (uint32_t)(((m < M ? m : M - 1) - bm0) * K + 16 * chunk);
      }
    });
  }

  // Per-channel constants of tile rows tid, tid + NT, .., fetched before the
  // K loop; sum w starts at zero (the summing waves add into it) or is the
  // caller's.
  float e_sc[T::CR], e_bi[T::CR];
  Static<0, T::CR>::each([&](auto C) {
    constexpr int c = decltype(C)::value;
    const int row = tid + c * T::NT;
    e_sc[c] = 0.0f;
    e_bi[c] = 0.0f;
    if (row < T::TN) {
      const int64_t n = bn0 + row;
      if (!a.acc && n < N) {
        e_sc[c] = a.wscale[n];
        e_bi[c] = a.bias ? a.bias[n] : 0.0f;
      }
      sm.ws[cslot<T::TN>(row)] = PRE && n < N ? a.wsum_pre[n] : 0;
    }
  });

  const int xr0 = 32 * T::FM * wm;
  const int wr0 = 32 * T::FN * wn;
  // sum w: of the WAVES_M waves that read the same weight rows, wave wm sums
  // slice wm % 2 of the W fragments of parity wm / 2 (of every fragment when
  // there are two such waves), so the v_dot4 work is the same on every SIMD.
  static_assert(T::WAVES_M == 2 || T::WAVES_M == 4, "sum w split");
  if (PRE) {
    run<T, -1, -1, PRE, TR, PK>(a, sm, gb, voff, ldo, kst, wr0, xr0, lane, tid, KT, bm0, bn0, e_sc, e_bi);
  } else if constexpr (T::WAVES_M == 2) {
    if (wm == 0)
      run<T, 0, -1, PRE, TR, PK>(a, sm, gb, voff, ldo, kst, wr0, xr0, lane, tid, KT, bm0, bn0, e_sc, e_bi);
    else
      run<T, 1, -1, PRE, TR, PK>(a, sm, gb, voff, ldo, kst, wr0, xr0, lane, tid, KT, bm0, bn0, e_sc, e_bi);
  } else {
    switch (wm) {
      case 0: run<T, 0, 0, PRE, TR, PK>(a, sm, gb, voff, ldo, kst, wr0, xr0, lane, tid, KT, bm0, bn0, e_sc, e_bi); break;
      case 1: run<T, 1, 0, PRE, TR, PK>(a, sm, gb, voff, ldo, kst, wr0, xr0, lane, tid, KT, bm0, bn0, e_sc, e_bi); break;
      case 2: run<T, 0, 1, PRE, TR, PK>(a, sm, gb, voff, ldo, kst, wr0, xr0, lane, tid, KT, bm0, bn0, e_sc, e_bi); break;
      default: run<T, 1, 1, PRE, TR, PK>(a, sm, gb, voff, ldo, kst, wr0, xr0, lane, tid, KT, bm0, bn0, e_sc, e_bi); break;
    }
  }
}

// Workgroups below nta take tiles of shape TA (tiles_ma x tiles_na, from
// column 0), the rest tiles of shape TB (tiles_mb x tiles_nb from column
// n0b): the columns left after whole rounds of TA tiles, in one launch, so
// that TB tiles start on the CUs the first TA tiles free.  Within each part
// the workgroups are dispatched round-robin over the 8 XCDs; they are
// renumbered so that XCD x walks a contiguous run of tiles (M fastest),
// which share slabs in its L2.
template <class TA, class TB, bool PRE, bool TR, bool PK>
__global__ __launch_bounds__(TA::NT, 1) void k_gemm_w8(LinearArgs a, int tiles_ma, int tiles_na,
                                                        int tiles_mb, int tiles_nb, int64_t n0b) {
  static_assert(TA::NT == TB::NT, "one block size");
  constexpr int STAGE = TA::STAGE > TB::STAGE ? TA::STAGE : TB::STAGE;
  constexpr int TN = TA::TN > TB::TN ? TA::TN : TB::TN;
  __shared__ __attribute__((aligned(16))) int8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) int8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) int8_t st2[STAGE];
  __shared__ __attribute__((aligned(16))) float epi_sc[TN];
  __shared__ __attribute__((aligned(16))) float epi_bi[TN];
  __shared__ __attribute__((aligned(16))) int32_t epi_ws[TN];
  const Smem sm{st0, st1, st2, epi_sc, epi_bi, epi_ws};
  auto remap = [](int b, int nt) {
    const int per = nt / 8;
    return b < per * 8 ? (b % 8) * per + (b / 8) : b;
  };
  const int nta = tiles_ma * tiles_na;
  const int b = blockIdx.x;
  if (b < nta)
    gemm_tile<TA, PRE, TR, PK>(a, sm, remap(b, nta), tiles_ma, 0);
  else
    gemm_tile<TB, PRE, TR, PK>(a, sm, remap(b - nta, tiles_mb * tiles_nb), tiles_mb, n0b);
}

using T256 = Tile<2, 4, 4, 2>;   // 256 x 256, waves of 128 x 64
using T128 = Tile<4, 2, 2, 2>;   // 256 W rows x 128 X rows, waves of 64 x 64

template <bool PRE, bool PK>
hipError_t launch_plan(const LinearArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + T256::BM - 1) / T256::BM;
  const int64_t tiles_n = (a.N + T256::TN - 1) / T256::TN;
  const int64_t tiles = tiles_m * tiles_n;
  // Whole rounds of 256 x 256 tiles over the 256 CUs, then the remaining
  // columns as 256 x 128 tiles when those fit one round: the last round then
  // keeps twice as many CUs busy, each with half a tile.
  // Problems of at most 128 such tiles run as 256 x 128 tiles throughout
  // when those fill more CUs within one round.
  int64_t cols = tiles_n, rest = 0;
  const int64_t tiles_mb = (a.M + T128::BM - 1) / T128::BM;
  if (tiles % 256 != 0 && 256 % tiles_m == 0 && tiles > 256) {
    const int64_t c = tiles / 256 * 256 / tiles_m;
    if ((tiles_n - c) * tiles_mb <= 256) {
      cols = c;
      rest = tiles_n - c;
    }
  } else if (tiles <= 128 && tiles_mb * tiles_n <= 256 && tiles_mb > tiles_m) {
    cols = 0;
    rest = tiles_n;
  }
  const dim3 grid((unsigned)(tiles_m * cols + tiles_mb * rest));
  const int64_t n0b = cols * T256::TN;
  // fp32 output (fused dequantize): the transposed form, whole-line stores
  if (a.outf != nullptr && a.acc == nullptr)
    hipLaunchKernelGGL((k_gemm_w8<T256, T128, PRE, true, PK>), grid, dim3(T256::NT), 0, s, a,
                       (int)tiles_m, (int)cols, (int)tiles_mb, (int)rest, n0b);
  else
    hipLaunchKernelGGL((k_gemm_w8<T256, T128, PRE, false, PK>), grid, dim3(T256::NT), 0, s, a,
                       (int)tiles_m, (int)cols, (int)tiles_mb, (int)rest, n0b);
  return hipGetLastError();
}

}  // namespace

bool gemm_w8_supported(const LinearArgs& a) {
  const int8_t* w = a.wpk ? a.wpk : a.w;
  const bool al = (((uintptr_t)a.x | (uintptr_t)w) & 15) == 0;
  // a prepacked weight comes with its sums; its fragment offsets are 32-bit
  const bool pk_ok = !a.wpk || (a.wsum_pre && (a.N + 31) / 32 * 32 * a.K < ((int64_t)1 << 32));
  // the lane offsets within a tile (up to 256 rows of K bytes) are 32-bit
  return a.K % 64 == 0 && a.K > 0 && a.K < ((int64_t)1 << 24) && al && pk_ok && a.M > 0 &&
         a.N > 0 && a.M <= (int64_t)1 << 30 && a.N <= (int64_t)1 << 30;
}

bool gemm_w8_preferred(const LinearArgs& a) {
  if (!gemm_w8_supported(a) || a.K < 1024) return false;
  const int64_t tiles_n = (a.N + T256::TN - 1) / T256::TN;
  const int64_t tiles = ((a.M + T256::BM - 1) / T256::BM) * tiles_n;
  const int64_t half = ((a.M + T128::BM - 1) / T128::BM) * tiles_n;
  return tiles >= 256 || (tiles <= 128 && half >= 128 && half <= 256);
}

hipError_t launch_gemm_w8(const LinearArgs& a, hipStream_t s) {
  if (!gemm_w8_supported(a)) return hipErrorInvalidValue;
  if (a.wpk) return launch_plan<true, true>(a, s);
  return a.wsum_pre ? launch_plan<true, false>(a, s) : launch_plan<false, false>(a, s);
}

}  // namespace q8ta
