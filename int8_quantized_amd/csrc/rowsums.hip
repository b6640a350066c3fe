// sum_k w[n, k] for every weight row: the precomputed weight sums of the
// zero-point fold ("Add q8ta_linear op", Constraints (1): sum (x - zp) * w =
// sum x * w - zp * sum w; the pages' op ignores a precomputed weight_sums,
// q8ta_weight_sums offers it as an opt-in).  One wave per row, lanes split K,
// v_dot4 against 0x01010101, then a reduction across the wave.
#include "q8ta_internal.h"

namespace q8ta {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_row_sums(const int8_t* __restrict__ w, int64_t N,
                                                       int64_t K, int32_t* __restrict__ out) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t n = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (n >= N) return;
  int32_t s = 0;
  for (int64_t k = (int64_t)lane * 16; k < K; k += 1024) {
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(w + n * K + k));
#pragma unroll
    for (int d = 0; d < 4; ++d) s = __builtin_amdgcn_sdot4(v[d], 0x01010101, s, false);
  }
  s = wave_total(s);
  if (lane == 0) out[n] = s;
}

}  // namespace

// K % 16 == 0 and w 16-byte aligned (q8ta_weight_sums checks both).
hipError_t launch_row_sums(const int8_t* w, int64_t N, int64_t K, int32_t* out, hipStream_t s) {
  hipLaunchKernelGGL(k_row_sums, dim3((unsigned)((N + 3) / 4)), dim3(kThreads), 0, s, w, N, K, out);
  return hipGetLastError();
}

}  // namespace q8ta
