// Calibration kernels for the benchmark: they measure what the chip reaches
// on the two resources the q8ta kernels are bound by, next to the published
// peaks.  Not part of the q8ta op family.
//
//  q8ta_calib_dot4: each thread runs `iters` rounds of 16 independent v_dot4
//    accumulations on registers (no memory traffic inside the loop) and writes
//    one int32; ops = threads * iters * 16 * 8.
//  q8ta_calib_copy: 16-byte grid-stride copy of n16 chunks; bytes = 32 * n16.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void k_dot4_loop(int32_t* out, int iters, int seed) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  int a[16], acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    a[k] = (t * 0x9E3779B1u) ^ (k * 0x85EBCA6Bu) ^ seed;
    acc[k] = k;
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = __builtin_amdgcn_sdot4(a[k], a[(k + 1) & 15], acc[k], false);
  }
  int s = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) s ^= acc[k];
  out[t] = s;
}

__global__ __launch_bounds__(256) void k_copy16(const v4i* __restrict__ src, v4i* __restrict__ dst,
                                                int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

}  // namespace

extern "C" {

// out: int32 device buffer of blocks * 256 entries.
int q8ta_calib_dot4(int32_t* out, int blocks, int iters, hipStream_t s) {
  if (!out || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(k_dot4_loop, dim3(blocks), dim3(256), 0, s, out, iters, 12345);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// src, dst: device buffers of n16 16-byte chunks each.
int q8ta_calib_copy(const void* src, void* dst, int64_t n16, int blocks, hipStream_t s) {
  if (!src || !dst || n16 < 1 || blocks < 1) return 1;
  hipLaunchKernelGGL(k_copy16, dim3(blocks), dim3(256), 0, s, (const v4i*)src, (v4i*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
