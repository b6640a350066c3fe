// q8ta_linear on prepacked weights ("Add q8ta_linear op", Solution: acc[m,n] =
// sum_k (x[m,k] - izp) * w[n,k] in int32, then the per-channel dequant /
// requant epilogue; Constraints (1): the zero-point term as sum x*w - izp *
// sum w with the sums precomputed, the way the Vulkan op the page mirrors
// takes them; Constraints (2): x [M,K] and w [N,K] K-contiguous).
//
// Packed weight layout (q8ta_weight_prepack): the weight is cut into
// fragments of 32 rows x 32 K bytes, each stored as the 1 KiB operand of one
// v_mfma_i32_32x32x32_i8 A fragment: byte 16 * l + j of fragment (nb, s) is
// w[32 * nb + l % 32][32 * s + 16 * (l / 32) + j] (lane l's 16 bytes), zero
// past N or K.  Fragment (nb, s) sits at byte (nb * KS + s) * 1024 with
// KS = 2 * ceil(K / 64); the buffer holds ceil(N / 32) * 32 rows of
// 64 * ceil(K / 64) bytes.
//
// Kernel: a workgroup of 4 waves computes a 256 x 128 tile (weight rows x
// activation rows); each wave owns 64 weight rows x all 128 activation rows
// (2 x 4 accumulator fragments).  No two waves share a weight row, so each
// wave reads its W fragments straight from global memory into registers: one
// fully coalesced 1 KiB load per fragment per 32-byte K slice, issued two K
// steps ahead (the compiler's own placement of these loads measured faster
// than pinning them with scheduling barriers: 111.7 vs 115-118 us on
// 2048 x 4096 x 11008).  Only the activation tile goes through LDS (two 8 KiB
// buffers, the same XOR swizzle as gemm_mx.hip), so per K byte the LDS takes
// 128 bytes of writes per workgroup instead of 384 and every wave reads
// 128 bytes instead of 192, and W makes no register -> LDS -> register round
// trip.  Two workgroups share a CU.  sum w comes from the caller (required).
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

constexpr int kBN = 256, kBM = 128, kBK = 64, kWaves = 4, kNT = 64 * kWaves;
constexpr int kWN = kBN / kWaves;           // 64 weight rows per wave
constexpr int kFN = kWN / 32, kFM = kBM / 32;
constexpr int kCPR = kBK / 16;               // 16-byte chunks per LDS row
constexpr int kBLD = kBM * kCPR / kNT;       // activation chunks per thread per step
constexpr int kStage = kBM * kBK;            // LDS bytes per buffer
constexpr int kRstep = kNT / kCPR;

// Chunk position of chunk c in LDS row r (the conflict-free layout for the
// 32x32x32 fragment reads, measured on gfx950; see gemm_mx.hip).
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 2) & 3); }

// Per-channel constants of tile row r, four rows of a register group BN / 4
// words apart (32-bit broadcast reads).
__device__ __forceinline__ int cslot(int r) { return (r & 3) * (kBN / 4) + (r >> 2); }

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

// One thread per 16-byte chunk of the packed buffer.
__global__ __launch_bounds__(256) void k_prepack(const int8_t* __restrict__ w, int64_t N,
                                                 int64_t K, int64_t KS, int64_t chunks,
                                                 v4i* __restrict__ packed) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int64_t per_nb = KS * 64;   // chunks per 32-row fragment column
  const int64_t nb = c / per_nb;
  const int64_t rem = c - nb * per_nb;
  const int64_t s = rem / 64;
  const int lane = (int)(rem % 64);
  const int64_t row = nb * 32 + lane % 32;
  const int64_t col = s * 32 + 16 * (lane / 32);
  v4i v = v4i{0, 0, 0, 0};
  if (row < N && col < K) v = *reinterpret_cast<const v4i*>(w + row * K + col);
  packed[c] = v;
}

// TR (fp32 output): X is the A operand and W the B operand, so the 32 lanes of
// a half-wave hold 32 consecutive output channels of one row and each store
// writes a whole 128-byte line (measured 2-2.5 us faster per call on
// 2048 x 4096 x 11008 than 16-byte pieces of 32 rows per store).
template <bool KFULL, bool TR>
__global__ __launch_bounds__(kNT, 2) void k_gemm_pk(LinearArgs a, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t smem[2 * kStage];
  __shared__ __attribute__((aligned(16))) float epi_sc[kBN];
  __shared__ __attribute__((aligned(16))) float epi_bi[kBN];
  __shared__ __attribute__((aligned(16))) int32_t epi_ws[kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);

  // XCD-aware tile order (each XCD walks a contiguous run, M fastest)
  const int T = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int per = T / 8;
  int t = b;
  if (b < per * 8) t = (b % 8) * per + (b / 8);
  const int tm = t % tiles_m;
  const int tn = t / tiles_m;
  const int64_t bn0 = (int64_t)tn * kBN;
  const int64_t bm0 = (int64_t)tm * kBM;
  const int64_t M = a.M, N = a.N, K = a.K;
  const int KT = (int)((K + kBK - 1) / kBK);
  const int64_t KS = 2 * (int64_t)KT;          // 32-byte slices per packed row
  const int64_t NB = (N + 31) / 32;

  // W fragments of this wave: fragment columns nb0, nb0 + 1 (clamped: past N
  // their products land in channels that are never stored).
  const int8_t* wbase[kFN];
  Static<0, kFN>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    int64_t nb = bn0 / 32 + wn * kFN + i;
    if (nb > NB - 1) nb = NB - 1;
    wbase[i] = a.wpk + nb * KS * 1024 + lane * 16;
  });
  // wv[p][ks][i]: fragment i of slice ks of a step with parity p
  v4i wv[2][2][kFN];
  auto load_w = [&](int kt, auto P, auto KSI) {
    constexpr int p = decltype(P)::value, ks = decltype(KSI)::value;
    Static<0, kFN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      wv[p][ks][i] = *reinterpret_cast<const v4i*>(wbase[i] + ((int64_t)2 * kt + ks) * 1024);
    });
  };

  // Activation loader: thread tid copies chunk column lc of rows lr + i * 64
  // (rows past M read the last row; chunks past K are zeroed when !KFULL).
  const int lc = tid % kCPR;
  const int lr = tid / kCPR;
  const int8_t* xrow[kBLD];
  Static<0, kBLD>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int64_t m = bm0 + lr + i * kRstep;
    xrow[i] = a.x + (m < M ? m : M - 1) * K + lc * 16;
  });
  v4i rb[2][kBLD];
  auto load_x = [&](int kt, auto SET) {
    constexpr int st = decltype(SET)::value;
    int64_t ko = (int64_t)kt * kBK;
    bool kin = true;
    if constexpr (!KFULL) {
      kin = ko + lc * 16 < K;
      if (!kin) ko = K - 16 - lc * 16;
    }
    Static<0, kBLD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const v4i v = *reinterpret_cast<const v4i*>(xrow[i] + ko);
      rb[st][i] = kin ? v : v4i{0, 0, 0, 0};
    });
  };
  auto store_x = [&](int buf, auto SET) {
    constexpr int st = decltype(SET)::value;
    int8_t* Bs = smem + buf * kStage;
    Static<0, kBLD>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int row = lr + i * kRstep;
      *reinterpret_cast<v4i*>(Bs + row * kBK + 16 * swz(row, lc)) = rb[st][i];
    });
  };

  v16i acc[kFN][kFM];
  Static<0, kFN>::each([&](auto I) {
    Static<0, kFM>::each([&](auto J) { acc[decltype(I)::value][decltype(J)::value] = v16i{}; });
  });

  // per-channel constants of tile row tid, fetched before the K loop
  float e_sc = 0.0f, e_bi = 0.0f;
  int32_t e_ws = 0;
  if (bn0 + tid < N) {
    e_ws = a.wsum_pre[bn0 + tid];
    if (!a.acc) {
      e_sc = a.wscale[bn0 + tid];
      e_bi = a.bias ? a.bias[bn0 + tid] : 0.0f;
    }
  }

  const int lrow = lane & 31;
  const int kg = lane >> 5;
  // Step on LDS buffer buf with the W fragments of parity P; with LOAD, each
  // slice's W registers are refilled with step `next` right after its
  // products are issued.
  auto compute = [&](int buf, auto P, int next, auto LOAD) {
    const int8_t* S = smem + buf * kStage;
    Static<0, 2>::each([&](auto KSI) {
      constexpr int ks = decltype(KSI)::value;
      constexpr int p = decltype(P)::value;
      const int cpos = 16 * swz(lrow, 2 * ks + kg);
      v4i bf[kFM];
      Static<0, kFM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        bf[j] = *reinterpret_cast<const v4i*>(S + (j * 32 + lrow) * kBK + cpos);
      });
      Static<0, kFN>::each([&](auto I) {
        constexpr int i = decltype(I)::value;
        Static<0, kFM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          if constexpr (TR)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[j], wv[p][ks][i], acc[i][j], 0,
                                                              0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wv[p][ks][i], bf[j], acc[i][j], 0,
                                                              0, 0);
        });
      });
      if constexpr (decltype(LOAD)::value) load_w(next, P, KSI);
    });
  };

  constexpr std::integral_constant<int, 0> I0{};
  constexpr std::integral_constant<int, 1> I1{};
  constexpr std::true_type LD{};
  constexpr std::false_type NOLD{};
  // Loads are issued on every step (step indices clamped to KT - 1: repeated
  // fetches of the last slab, written to a buffer no one reads any more), so
  // the loop carries no branch around them.
  load_x(0, I0);
  store_x(0, I0);
  load_x(min(1, KT - 1), I1);
  load_w(0, I0, I0);
  load_w(0, I0, I1);
  load_w(min(1, KT - 1), I1, I0);
  load_w(min(1, KT - 1), I1, I1);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    load_x(min(kt + 2, KT - 1), I0);
    compute(0, I0, min(kt + 2, KT - 1), LD);
    store_x(1, I1);
    __syncthreads();
    load_x(min(kt + 3, KT - 1), I1);
    compute(1, I1, min(kt + 3, KT - 1), LD);
    store_x(0, I0);
    __syncthreads();
  }
  if (kt < KT) compute(0, I0, 0, NOLD);   // odd KT: the last step sits in buffer 0

  epi_ws[cslot(tid)] = e_ws;
  epi_sc[cslot(tid)] = e_sc;
  epi_bi[cslot(tid)] = e_bi;
  __syncthreads();

  const bool fast = bm0 + kBM <= M && bn0 + kBN <= N && M * N <= (int64_t)INT32_MAX;
  if constexpr (TR) {
    // lane l: channel of tile row wn*64 + i*32 + l % 32; register r: output
    // row m of fragment j at 8 * (r / 4) + 4 * (l / 32) + r % 4
    const float dq_zpf = (float)a.dq_zp;
    Static<0, kFN>::each([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int rr = wn * kWN + i * 32 + lrow;
      const int sl = cslot(rr);
      const int32_t zc = a.izp * epi_ws[sl];
      const float sc = epi_sc[sl], bi = epi_bi[sl];
      const int64_t n = bn0 + rr;
      if (fast) {
        // interior tile: one 32-bit lane offset, wave-uniform row bases
        const uint32_t lane_off = (uint32_t)((bm0 + 4 * kg) * N + n);
        Static<0, kFM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          Static<0, 16>::each([&](auto R) {
            constexpr int r = decltype(R)::value;
            constexpr int c = j * 32 + 8 * (r / 4) + r % 4;
            const float q = requant_code(acc[i][j][r] - zc, sc, bi, a.rq);
            float* rb = a.outf + (int64_t)c * N;
            rb[lane_off] = (q - dq_zpf) * a.dq_scale;
          });
        });
      } else if (n < N) {
        Static<0, kFM>::each([&](auto J) {
          constexpr int j = decltype(J)::value;
          Static<0, 16>::each([&](auto R) {
            constexpr int r = decltype(R)::value;
            const int64_t m = bm0 + j * 32 + 8 * (r / 4) + 4 * kg + r % 4;
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
  Static<0, kFN>::each([&](auto I) {
    constexpr int i = decltype(I)::value;
    Static<0, 4>::each([&](auto G) {
      constexpr int g = decltype(G)::value;
      const int rr = wn * kWN + i * 32 + 8 * g + 4 * kg;   // tile row of registers 4g..4g+3
      const int64_t nb = bn0 + rr;
      int32_t zc[4];
      float sc[4], bi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int sl = cslot(rr + r);
        zc[r] = a.izp * epi_ws[sl];
        sc[r] = epi_sc[sl];
        bi[r] = epi_bi[sl];
      }
      Static<0, kFM>::each([&](auto J) {
        constexpr int j = decltype(J)::value;
        const int64_t m = bm0 + j * 32 + lrow;
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

}  // namespace

int64_t prepacked_bytes(int64_t N, int64_t K) {
  return ((N + 31) / 32) * 32 * (((K + 63) / 64) * 64);
}

hipError_t launch_prepack(const int8_t* w, int64_t N, int64_t K, int8_t* packed, hipStream_t s) {
  const int64_t KS = 2 * ((K + 63) / 64);
  const int64_t chunks = prepacked_bytes(N, K) / 16;
  const int64_t blocks = (chunks + 255) / 256;
  hipLaunchKernelGGL(k_prepack, dim3((unsigned)blocks), dim3(256), 0, s, w, N, K, KS, chunks,
                     reinterpret_cast<v4i*>(packed));
  return hipGetLastError();
}

// a.wpk: packed weight; a.wsum_pre: the weight's row sums (both required).
hipError_t launch_gemm_pk(const LinearArgs& a, hipStream_t s) {
  const int tiles_m = (int)((a.M + kBM - 1) / kBM);
  const int tiles_n = (int)((a.N + kBN - 1) / kBN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const bool tr = a.outf != nullptr && a.acc == nullptr;
  if (a.K % kBK == 0) {
    if (tr) hipLaunchKernelGGL((k_gemm_pk<true, true>), grid, dim3(kNT), 0, s, a, tiles_m, tiles_n);
    else hipLaunchKernelGGL((k_gemm_pk<true, false>), grid, dim3(kNT), 0, s, a, tiles_m, tiles_n);
  } else {
    if (tr) hipLaunchKernelGGL((k_gemm_pk<false, true>), grid, dim3(kNT), 0, s, a, tiles_m, tiles_n);
    else hipLaunchKernelGGL((k_gemm_pk<false, false>), grid, dim3(kNT), 0, s, a, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace q8ta
