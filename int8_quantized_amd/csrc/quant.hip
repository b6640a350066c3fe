// quantize_per_tensor / dequantize_per_tensor: streaming, HBM-bound kernels.
//
// quantize ("Add quantize_per_tensor op (int8 buffer path)", commit message):
//   q = clamp(round(x * inv_scale) + zero_point, -128, 127), inv_scale formed
//   on the host as (float)(1.0 / scale).
// dequantize (the decomposed op the q8ta subgraph ends with):
//   y = (float)(q - zero_point) * (float)scale.
//
// Layout: each thread moves U groups of 4 elements (U = 4 for dequantize); within one group
// instruction the 64 lanes of a wave touch 64 consecutive groups, so every
// global load and store instruction is fully coalesced (1 KiB of fp32 and
// 256 B of int8 per wave per instruction).  All loads of a thread are issued
// before any arithmetic so each wave keeps U requests in flight.
#include <cstdlib>

#include "q8ta_internal.h"

namespace q8ta {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__device__ __forceinline__ int quant1(float x, float inv, float zp) { return quantize1(x, inv, zp); }

// x: fp32, 16-byte aligned; out: int8, 4-byte aligned.  n4 = numel / 4 groups;
// block 0 also converts the numel % 4 trailing elements one by one.
template <int U>
__global__ __launch_bounds__(kThreads) void k_quantize_x4(const v4f* __restrict__ x,
                                                          uint32_t* __restrict__ out, int64_t n4,
                                                          int64_t numel, float inv, float zp) {
  const int64_t base = (int64_t)blockIdx.x * (kThreads * U) + threadIdx.x;
  if (base + (U - 1) * kThreads < n4) {
    v4f v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&x[base + u * kThreads]);
#pragma unroll
    for (int u = 0; u < U; ++u)
      out[base + u * kThreads] = pack4(quant1(v[u].x, inv, zp), quant1(v[u].y, inv, zp),
                                       quant1(v[u].z, inv, zp), quant1(v[u].w, inv, zp));
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t c = base + u * kThreads;
      if (c < n4) {
        v4f v = x[c];
        out[c] = pack4(quant1(v.x, inv, zp), quant1(v.y, inv, zp), quant1(v.z, inv, zp),
                       quant1(v.w, inv, zp));
      }
    }
  }
  if (blockIdx.x == 0) {
    int64_t e = n4 * 4 + threadIdx.x;
    if (e < numel) {
      const float* xs = reinterpret_cast<const float*>(x);
      int8_t* os = reinterpret_cast<int8_t*>(out);
      os[e] = (int8_t)quant1(xs[e], inv, zp);
    }
  }
}

// Any alignment: one element per thread.
__global__ __launch_bounds__(kThreads) void k_quantize_x1(const float* __restrict__ x,
                                                          int8_t* __restrict__ out, int64_t numel,
                                                          float inv, float zp) {
  int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e < numel) out[e] = (int8_t)quant1(x[e], inv, zp);
}

__device__ __forceinline__ v4f dequant4(uint32_t p, float scale, int zp) {
  v4f r;
  r.x = (float)((int)(int8_t)(p & 0xff) - zp) * scale;
  r.y = (float)((int)(int8_t)((p >> 8) & 0xff) - zp) * scale;
  r.z = (float)((int)(int8_t)((p >> 16) & 0xff) - zp) * scale;
  r.w = (float)((int)(int8_t)(p >> 24) - zp) * scale;
  return r;
}

// x: int8, 4-byte aligned; out: fp32, 16-byte aligned.
__global__ __launch_bounds__(kThreads) void k_dequantize_x4(const uint32_t* __restrict__ x,
                                                            v4f* __restrict__ out, int64_t n4,
                                                            int64_t numel, float scale, int zp) {
  constexpr int64_t kGroupsPerBlock = (int64_t)kThreads * kUnroll;
  const int64_t base = (int64_t)blockIdx.x * kGroupsPerBlock + threadIdx.x;
  if (base + (kUnroll - 1) * kThreads < n4) {
    uint32_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(&x[base + u * kThreads]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_nontemporal_store(dequant4(v[u], scale, zp), &out[base + u * kThreads]);
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      int64_t c = base + u * kThreads;
      if (c < n4) out[c] = dequant4(x[c], scale, zp);
    }
  }
  if (blockIdx.x == 0) {
    int64_t e = n4 * 4 + threadIdx.x;
    if (e < numel) {
      const int8_t* xs = reinterpret_cast<const int8_t*>(x);
      float* os = reinterpret_cast<float*>(out);
      os[e] = (float)((int)xs[e] - zp) * scale;
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_dequantize_x1(const int8_t* __restrict__ x,
                                                            float* __restrict__ out, int64_t numel,
                                                            float scale, int zp) {
  int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (e < numel) out[e] = (float)((int)x[e] - zp) * scale;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

template <int U>
void launch_quantize_u(const float* x, int8_t* out, int64_t numel, float inv_scale, float zp,
                       hipStream_t s) {
  const int64_t n4 = numel / 4;
  int64_t blocks = (n4 + (int64_t)kThreads * U - 1) / ((int64_t)kThreads * U);
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_quantize_x4<U>, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     reinterpret_cast<const v4f*>(x), reinterpret_cast<uint32_t*>(out), n4, numel,
                     inv_scale, zp);
}

}  // namespace

// Four groups of 4 elements per thread (unrolls of 2 and 8 measured no
// better on [8,256,64,64]).
hipError_t launch_quantize(const float* x, int8_t* out, int64_t numel, float inv_scale, float zp,
                           hipStream_t s) {
  if (aligned(x, 16) && aligned(out, 4)) {
    launch_quantize_u<4>(x, out, numel, inv_scale, zp, s);
  } else {
    int64_t blocks = (numel + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_quantize_x1, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, out, numel,
                       inv_scale, zp);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const int8_t* x, float* out, int64_t numel, float scale, int zp,
                             hipStream_t s) {
  if (aligned(x, 4) && aligned(out, 16)) {
    int64_t n4 = numel / 4;
    int64_t blocks = (n4 + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_dequantize_x4, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint32_t*>(x), reinterpret_cast<v4f*>(out), n4,
                       numel, scale, zp);
  } else {
    int64_t blocks = (numel + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(k_dequantize_x1, dim3((unsigned)blocks), dim3(kThreads), 0, s, x, out,
                       numel, scale, zp);
  }
  return hipGetLastError();
}

}  // namespace q8ta
