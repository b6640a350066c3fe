// q8ta_linear for M <= 4 rows of activations (q8ta_linear_gemv is M == 1):
// a weight-streaming, HBM-bound kernel ("Add q8ta_linear op", Solution: the
// M == 1 case of the same contraction and epilogue).
//
// Each wave owns ROWS consecutive weight rows.  In one pass over K the 64
// lanes read CH consecutive 1 KiB slices of each row (lane l takes bytes
// [16 l, 16 l + 16) of a slice), so every load instruction moves 1 KiB of
// contiguous weight bytes; all ROWS*CH weight loads of a pass are issued
// before any arithmetic, keeping ROWS*CH*1 KiB in flight per wave.  The
// activation row(s) are small and stay in cache.  The dot products use the
// packed int8 dot instruction (v_dot4): sum x*w and, against 0x01010101,
// sum w; the zero-point term is folded as sum x*w - izp*sum w, then each
// row's partial is reduced across the wave and requantized.  With fp32
// activations (the fused quantize -> linear chain) each lane loads its 16
// values as four float4 and quantizes them with the quantize_per_tensor
// formula into LDS, once per workgroup and chunk (the four waves share it),
// before the dot products, so the int8 activations never go to HBM.
#include <cstdlib>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int MR, int ROWS, int CH, bool XF>
__global__ __launch_bounds__(kThreads) void k_skinny(LinearArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int64_t n0 = wave * ROWS;
  // No early exit: a wave past the last row reads row N - 1 and stores
  // nothing (a branch ahead of the weight stream would put a second round of
  // argument reads before its first load; the fp32 form also shares each
  // chunk's codes through LDS and meets barriers).
  const int64_t K = a.K;
  int32_t dot[MR][ROWS];
  int32_t sw[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    sw[r] = 0;
#pragma unroll
    for (int m = 0; m < MR; ++m) dot[m][r] = 0;
  }
  // K >= 1 (the entry points check it): the first pass runs unconditionally,
  // so no branch sits ahead of its loads
  int64_t k0 = 0;
  do {
    v4i wv[ROWS][CH];
    v4i xv[MR][CH];
    int ones[CH];  // 0x01010101 where the lane's slice is inside K, else 0
    if constexpr (XF) {
      // the int8 form allocates no LDS
      __shared__ v4i xs[MR * CH * 64];
      // The chunk's fp32 activations are loaded first (the quantize below
      // waits only for them), then the weight stream, with every load
      // unconditional: rows past N read row N - 1 (never stored), slices past
      // K read the row's first bytes and are cancelled by zero activation
      // codes and a zero ones-vector in sum w.  The workgroup quantizes the
      // MR x 1024*CH activations once: slot i = (m, c, lane) of the register
      // layout, 16 values each.
      constexpr int SLOTS = MR * CH * 64;
      constexpr int SL = (SLOTS + kThreads - 1) / kThreads;
      v4f xr[SL][4];
      bool xok[SL];
#pragma unroll
      for (int j = 0; j < SL; ++j) {
        const int i = threadIdx.x + j * kThreads;
        const int m = (i < SLOTS ? i : 0) / (CH * 64);
        const int64_t kk = k0 + (int64_t)(i % (CH * 64)) * 16;
        xok[j] = i < SLOTS && kk < K;
        const v4f* p = reinterpret_cast<const v4f*>(a.xf + m * K + (xok[j] ? kk : 0));
#pragma unroll
        for (int d = 0; d < 4; ++d) xr[j][d] = p[d];
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int64_t kk = k0 + c * 1024 + lane * 16;
        const bool ok = kk < K;
        ones[c] = ok ? 0x01010101 : 0;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const int64_t n = n0 + r < a.N ? n0 + r : a.N - 1;
          wv[r][c] = __builtin_nontemporal_load(
              reinterpret_cast<const v4i*>(a.w + n * K + (ok ? kk : 0)));
        }
      }
      if (k0 != 0) __syncthreads();  // every wave has read the last chunk
#pragma unroll
      for (int j = 0; j < SL; ++j) {
        v4i q;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          q[d] = (int)pack4(quantize1(xr[j][d][0], a.inv_in, (float)a.izp),
                            quantize1(xr[j][d][1], a.inv_in, (float)a.izp),
                            quantize1(xr[j][d][2], a.inv_in, (float)a.izp),
                            quantize1(xr[j][d][3], a.inv_in, (float)a.izp));
        if (SLOTS % kThreads == 0 || threadIdx.x + j * kThreads < SLOTS)
          xs[threadIdx.x + j * kThreads] = xok[j] ? q : v4i{0, 0, 0, 0};
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < CH; ++c) {
#pragma unroll
        for (int m = 0; m < MR; ++m) xv[m][c] = xs[(m * CH + c) * 64 + lane];
      }
    } else {
      // every load unconditional (no branch between them): rows past N
      // read row N - 1, slices past K read the row's first bytes; both are
      // cancelled by zero activations and a zero ones-vector
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int64_t kk = k0 + c * 1024 + lane * 16;
        const bool ok = kk < K;
        ones[c] = ok ? 0x01010101 : 0;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
          const int64_t n = n0 + r < a.N ? n0 + r : a.N - 1;
          wv[r][c] = __builtin_nontemporal_load(
              reinterpret_cast<const v4i*>(a.w + n * K + (ok ? kk : 0)));
        }
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int64_t kk = k0 + c * 1024 + lane * 16;
        const bool ok = kk < K;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const v4i v = *reinterpret_cast<const v4i*>(a.x + m * K + (ok ? kk : 0));
          xv[m][c] = ok ? v : v4i{0, 0, 0, 0};
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          sw[r] = __builtin_amdgcn_sdot4(wv[r][c][d], ones[c], sw[r], false);
#pragma unroll
          for (int m = 0; m < MR; ++m)
            dot[m][r] = __builtin_amdgcn_sdot4(xv[m][c][d], wv[r][c][d], dot[m][r], false);
        }
      }
    }
    k0 += 1024 * CH;
  } while (k0 < K);
  int32_t mine = 0;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      int32_t t = wave_total(dot[m][r] - a.izp * sw[r]);
      if (lane == m * ROWS + r) mine = t;
    }
  }
  if (lane < MR * ROWS) {
    const int m = lane / ROWS, r = lane % ROWS;
    const int64_t n = n0 + r;
    if (n < a.N) {
      if (a.acc) {
        a.acc[m * a.N + n] = mine;
      } else {
        const int q = requant(mine, a.wscale[n], a.bias ? a.bias[n] : 0.0f, a.rq);
        if (a.outf)
          a.outf[m * a.N + n] = dequant1(q, a.dq_zp, a.dq_scale);
        else
          a.out[m * a.N + n] = (int8_t)q;
      }
    }
  }
}

// CH: consecutive 1 KiB slices a wave reads per pass over K: 4, or 1 when
// K <= 1024 (one pass either way; the single slice wastes no loads or
// quantize work on slices past K).
template <int MR, int ROWS>
hipError_t launch_rows(const LinearArgs& a, hipStream_t s) {
  const int64_t waves = (a.N + ROWS - 1) / ROWS;
  const int64_t blocks = (waves + kWaves - 1) / kWaves;
  const dim3 g((unsigned)blocks), t(kThreads);
  if (a.K <= 1024) {
    if (a.xf) hipLaunchKernelGGL((k_skinny<MR, ROWS, 1, true>), g, t, 0, s, a);
    else hipLaunchKernelGGL((k_skinny<MR, ROWS, 1, false>), g, t, 0, s, a);
  } else {
    if (a.xf) hipLaunchKernelGGL((k_skinny<MR, ROWS, 4, true>), g, t, 0, s, a);
    else hipLaunchKernelGGL((k_skinny<MR, ROWS, 4, false>), g, t, 0, s, a);
  }
  return hipGetLastError();
}

template <int MR>
hipError_t launch_mr(const LinearArgs& a, hipStream_t s, int rows) {
  switch (rows) {
    case 1: return launch_rows<MR, 1>(a, s);
    default: return launch_rows<MR, 4>(a, s);
  }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

bool gemv_supported(const LinearArgs& a) {
  return a.M >= 1 && a.M <= 4 && (a.K % 16) == 0 && aligned16(a.xf ? (const void*)a.xf : a.x) &&
         aligned16(a.w);
}

// rows: weight rows per wave.  One for int8 activations (1 x 4096 x 4096:
// 4.7-4.9 us against 4.9-5.2 us for 2 rows and 6.1 for 4).  The fp32 form
// takes 4 rows for M > 1, where each workgroup's quantize pass grows with M:
// on 4 x 4096 x 4096, 7.1 us against 7.2 for 2 rows and 9.7 for 1 (M = 1:
// 5.3 us with 1 row, 6.0 with 4).
hipError_t launch_gemv(const LinearArgs& a, hipStream_t s) {
  const int rows = (a.xf && a.M > 1) ? 4 : 1;
  switch (a.M) {
    case 1: return launch_mr<1>(a, s, rows);
    case 2: return launch_mr<2>(a, s, rows);
    case 3: return launch_mr<3>(a, s, rows);
    default: return launch_mr<4>(a, s, rows);
  }
}

}  // namespace q8ta
