// Calibration kernels for the benchmark: they measure what the chip reaches
// on the two resources the q8ta kernels are bound by, next to the published
// peaks.  Not part of the q8ta op family.
//
//  q8ta_calib_mfma: a register-only loop of independent int8 MFMAs per wave
//    (the matrix-core issue ceiling).
//  q8ta_calib_mfma_data: the same 32x32x32 loop with every lane's operands
//    taken from given int8 data: the matrix cores draw more power, and the
//    chip runs them slower, on operands with many toggling bits (quantized
//    data) than on the near-constant ones of q8ta_calib_mfma.
//  q8ta_calib_copy: 16-byte grid-stride copy of n16 chunks; bytes = 32 * n16.
//  q8ta_calib_read: read-only stream of n16 16-byte chunks, 8 per thread in
//    the access pattern of the GEMV's weight stream (each load instruction of
//    a wave covers 1 KiB); bytes = 16 * n16.
//  q8ta_calib_empty: a launch of `blocks` blocks that do no work (the floor
//    of one launch in a back-to-back sequence).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// MFMA issue ceiling: each wave runs `iters` rounds of 16 independent int8
// matrix products into 16 accumulators held in registers.  kind 0:
// v_mfma_i32_16x16x64_i8 (32768 ops each), kind 1: v_mfma_i32_32x32x32_i8
// (65536 ops each).
template <int KIND>
__global__ __launch_bounds__(256) void k_mfma_loop(int32_t* out, int iters, int seed) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const v4i a = v4i{(int)(t * 0x9E3779B1u) ^ seed, t, seed, 7};
  const v4i b = v4i{t ^ 0x5a5a5a5a, seed, (int)(t * 0x85EBCA6Bu), 3};
  int s = 0;
  if constexpr (KIND == 0) {
    v4i acc[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = v4i{k, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) s ^= acc[k][0] ^ acc[k][3];
  } else {
    typedef int v16i __attribute__((ext_vector_type(16)));
    v16i acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc[k] = v16i{};
      acc[k][0] = k;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[k], 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s ^= acc[k][0] ^ acc[k][15];
  }
  out[t] = s;
}

// kind 1's loop on operands from memory: lane t of the grid takes A = the
// 16 bytes at 16 * (t % na16) of a and B = those at 16 * (t % nb16) of b.
__global__ __launch_bounds__(256) void k_mfma_data(const v4i* __restrict__ a, int64_t na16,
                                                   const v4i* __restrict__ b, int64_t nb16,
                                                   int iters, int32_t* out) {
  typedef int v16i __attribute__((ext_vector_type(16)));
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const v4i av = a[t % na16];
  const v4i bv = b[t % nb16];
  v16i acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = v16i{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc[k], 0, 0, 0);
  }
  int s = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) s ^= acc[k][0] ^ acc[k][15];
  out[t] = s;
}

__global__ __launch_bounds__(256) void k_copy16(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                                int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

__global__ __launch_bounds__(256) void k_read16(const v4i* __restrict__ src, int64_t n16,
                                                int32_t* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * 256 * 8 + threadIdx.x;
  v4i v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t i = base + u * 256;
    v[u] = i < n16 ? __builtin_nontemporal_load(&src[i]) : v4i{0, 0, 0, 0};
  }
  int s = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) s ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (s == 0x7fffffff) out[0] = s;  // keeps the loads; almost never taken
}

__global__ __launch_bounds__(256) void k_empty(int32_t* out, int flag) {
  if (flag) out[threadIdx.x] = 0;
}

}  // namespace

extern "C" {

// out: int32 device buffer of blocks * 256 entries.
// ops = blocks * 4 waves * iters * (16 * 32768 for kind 0, 8 * 65536 for kind 1)
int q8ta_calib_mfma(int32_t* out, int blocks, int iters, int kind, hipStream_t s) {
  if (kind == 0)
    hipLaunchKernelGGL(k_mfma_loop<0>, dim3(blocks), dim3(256), 0, s, out, iters, 12345);
  else
    hipLaunchKernelGGL(k_mfma_loop<1>, dim3(blocks), dim3(256), 0, s, out, iters, 12345);
  return (int)hipGetLastError();
}

// a, b: device buffers of na16 / nb16 16-byte chunks; out: int32 device
// buffer of blocks * 256 entries.  ops = blocks * 4 waves * iters * 8 * 65536.
int q8ta_calib_mfma_data(const void* a, int64_t na16, const void* b, int64_t nb16, int32_t* out,
                         int blocks, int iters, hipStream_t s) {
  if (!a || !b || !out || na16 < 1 || nb16 < 1 || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(k_mfma_data, dim3(blocks), dim3(256), 0, s, (const v4i*)a, na16,
                     (const v4i*)b, nb16, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// src, dst: device buffers of n16 16-byte chunks each.
int q8ta_calib_copy(const void* src, void* dst, int64_t n16, int blocks, hipStream_t s) {
  if (!src || !dst || n16 < 1 || blocks < 1) return 1;
  hipLaunchKernelGGL(k_copy16, dim3(blocks), dim3(256), 0, s, (const v4i*)src, (v4i*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// src: device buffer of n16 16-byte chunks; out: int32 device scratch (>= 1).
int q8ta_calib_read(const void* src, int64_t n16, int32_t* out, hipStream_t s) {
  if (!src || !out || n16 < 1) return 1;
  const int64_t blocks = (n16 + 256 * 8 - 1) / (256 * 8);
  hipLaunchKernelGGL(k_read16, dim3((unsigned)blocks), dim3(256), 0, s, (const v4i*)src, n16, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int q8ta_calib_empty(int32_t* out, int blocks, hipStream_t s) {
  if (!out || blocks < 1) return 1;
  hipLaunchKernelGGL(k_empty, dim3(blocks), dim3(256), 0, s, out, 0);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
