// Internal declarations shared by the libq8ta host code and its gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8ta {

// Scalars of the dequant/requant epilogue, prepared on the host:
// s_in = (float)input_scale, inv_out = (float)(1.0 / output_scale),
// ozp = (float)output_zero_point, qmin = the lowest code: -128, or the output
// zero point for the relu-fused activation.
struct Requant {
  float s_in;
  float inv_out;
  float ozp;
  float qmin;
};

// The per-channel epilogue of q8ta_linear / q8ta_conv2d_transposed
// ("Add q8ta_linear op" and "Add q8ta_conv2d_transposed op", Solution):
// v = acc * input_scale * weight_scale + bias, then
// q = clamp(round(v * inv_output_scale) + output_zero_point, -128, 127).
// Evaluated left to right in float with one rounding per operation (every
// source is built with -ffp-contract=off, so no multiply-add is fused);
// rint rounds half to even.  A missing bias is passed as 0.0f, which gives
// the same code as skipping the add.  Relu fused (the follow-up both pages
// leave fail-loud) requantizes max(v, 0): for v <= 0 that code is the output
// zero point and the plain code is at most the zero point, for v > 0 the plain
// code is already at least the zero point, so it equals clamping the plain
// code from below at the zero point (r.qmin) for every finite v.
__device__ __forceinline__ int requant(int32_t acc, float wscale, float b, const Requant& r) {
  float v = (float)acc;
  v = v * r.s_in;
  v = v * wscale;
  v = v + b;
  float t = v * r.inv_out;
  float q = __builtin_rintf(t);
  q = q + r.ozp;
  q = __builtin_amdgcn_fmed3f(q, r.qmin, 127.0f);   // clamp to [qmin, 127] in one instruction
  return (int)q;
}

// requant() with the code written into byte `sel` of `old` in offset form
// (code + 128, so byte b of the result XOR 0x80 is the int8 code).  The same
// left-to-right float steps up to the rounding; then u = rint(t) + (zp + 128),
// exact for |rint(t)| < 2^24 - 256 and beyond that saturating either way,
// goes through v_cvt_pk_u8_f32, which saturates at 0 and 255 (u is integral,
// so its round-to-nearest-even is exact) and inserts the byte: the code of
// requant() for every finite v.  The lower clamp at -128 is that saturation;
// RELU adds the clamp at qmin + 128 (qmin128) for the relu-fused epilogue.
// ozp128 is r.ozp + 128.
template <bool RELU>
__device__ __forceinline__ uint32_t requant_u8(int32_t acc, float wscale, float b, const Requant& r,
                                               float ozp128, float qmin128, uint32_t sel,
                                               uint32_t old) {
  float v = (float)acc;
  v = v * r.s_in;
  v = v * wscale;
  v = v + b;
  float t = v * r.inv_out;
  float u = __builtin_rintf(t);
  u = u + ozp128;
  if constexpr (RELU) u = __builtin_fmaxf(u, qmin128);
  return __builtin_amdgcn_cvt_pk_u8_f32(u, sel, old);
}

// quantize_per_tensor of one value ("Add quantize_per_tensor op (int8 buffer
// path)", commit message): clamp(rint(x * inv) + zp, -128, 127), inv formed on
// the host as (float)(1.0 / scale).
__device__ __forceinline__ int quantize1(float x, float inv, float zp) {
  float t = x * inv;
  float r = __builtin_rintf(t);
  float u = r + zp;
  u = __builtin_amdgcn_fmed3f(u, -128.0f, 127.0f);
  return (int)u;
}

// dequantize_per_tensor of one int8 value: (float)(q - zp) * scale.
__device__ __forceinline__ float dequant1(int q, int zp, float scale) {
  return (float)(q - zp) * scale;
}

// Low bytes of a, b, c, d as one little-endian word (three byte permutes).
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)b, (uint32_t)a, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)d, (uint32_t)c, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Lane moves inside a row of 16 lanes (DPP controls of the gfx9 encoding).
constexpr int kDppSwap1 = 0xB1;      // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppRev4 = 0x1B;       // quad_perm [3,2,1,0]: lane ^ 3
constexpr int kDppMirror8 = 0x141;   // row_half_mirror:     lane ^ 7
constexpr int kDppMirror16 = 0x140;  // row_mirror:          lane ^ 15

template <int CTRL>
__device__ __forceinline__ int32_t row_move(int32_t v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Sum of v over the 64 lanes of a wave, returned wave-uniform.  Every lane of
// the wave must be active.  Four DPP steps (lane masks 15, 7, 3, 1 span the 16
// lanes of a row) leave each row's sum in all of its lanes; the four row sums
// are then read out with v_readlane.
__device__ __forceinline__ int32_t wave_total(int32_t v) {
  v += row_move<kDppMirror16>(v);
  v += row_move<kDppMirror8>(v);
  v += row_move<kDppRev4>(v);
  v += row_move<kDppSwap1>(v);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Transposing butterfly of the register-tiled contractions: a lane holds 64
// partial sums of an 8 x 8 tile and the LPG lanes of a group (inside one DPP
// row) together cover the whole K range.  One step over HALF value pairs: keep
// the upper or lower half by `upper`, receive the partner's copy of the kept
// half and add it.
template <int HALF, int CTRL>
__device__ __forceinline__ void fold(int32_t (&acc)[64], bool upper) {
#pragma unroll
  for (int i = 0; i < HALF; ++i) {
    const int32_t lo = acc[i], hi = acc[i + HALF];
    const int32_t keep = upper ? hi : lo;
    const int32_t send = upper ? lo : hi;
    acc[i] = keep + row_move<CTRL>(send);
  }
}

// Butterfly over the LPG lanes of a group: 64 values -> 64/LPG values.
template <int LPG>
__device__ __forceinline__ void reduce_group(int32_t (&acc)[64], int lg) {
  if constexpr (LPG == 16) {
    fold<32, kDppMirror16>(acc, (lg & 8) != 0);
    fold<16, kDppMirror8>(acc, (lg & 4) != 0);
    fold<8, kDppRev4>(acc, (lg & 2) != 0);
    fold<4, kDppSwap1>(acc, (lg & 1) != 0);
  } else if constexpr (LPG == 8) {
    fold<32, kDppMirror8>(acc, (lg & 4) != 0);
    fold<16, kDppRev4>(acc, (lg & 2) != 0);
    fold<8, kDppSwap1>(acc, (lg & 1) != 0);
  } else {
    static_assert(LPG == 4, "LPG");
    fold<32, kDppRev4>(acc, (lg & 2) != 0);
    fold<16, kDppSwap1>(acc, (lg & 1) != 0);
  }
}

// Global pointer kept in scalar registers (wave-uniform).
typedef const __attribute__((address_space(1))) int8_t* gptr;

__device__ __forceinline__ gptr uniform_ptr(const int8_t* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (gptr)(((uint64_t)hi << 32) | lo);
}

// Scratch device memory ordered on stream s, released with workspace_release
// on the same stream and thread once the call's kernels are launched.  The
// library keeps one buffer per (device, stream) and nesting depth, grown on
// demand (after a synchronization of s) and held until the process ends:
// a per-call hipMallocAsync / hipFreeAsync pair costs ~15 us of stream time.
// Requests above 256 MiB, deeper nesting and streams under graph capture take
// stream-ordered memory from the device's default pool instead (kept up to
// 1 GiB after frees).  Between acquire and release the library holds a lock.
hipError_t workspace_acquire(void** p, size_t bytes, hipStream_t s);
hipError_t workspace_release(void* p, hipStream_t s);

// ---- launchers (host functions; each returns hipGetLastError() after launch)
hipError_t launch_quantize(const float* x, int8_t* out, int64_t numel, float inv_scale, float zp,
                           hipStream_t s);
hipError_t launch_dequantize(const int8_t* x, float* out, int64_t numel, float scale, int zp,
                             hipStream_t s);

struct LinearArgs {
  const int8_t* x;
  const int8_t* w;
  const float* wscale;
  const float* bias;  // may be NULL
  int8_t* out;        // int8 [M, N] (NULL when acc or outf is set)
  int32_t* acc;       // int32 [M, N] accumulator output (NULL for the int8 op)
  int64_t M, K, N;
  int32_t izp;
  Requant rq;
  // Fused dequantize: when set, the kernels write fp32 [M, N] =
  // (float)(q - dq_zp) * dq_scale of the requantized q instead of q itself.
  float* outf = nullptr;
  float dq_scale = 0.0f;
  int32_t dq_zp = 0;
  // Trusted per-row sums sum_k w[n, k] supplied by the caller (the
  // precomputed weight_sums of the presummed entry points); NULL: the kernels
  // form them.
  const int32_t* wsum_pre = nullptr;
  // Prepacked weight (the MFMA-fragment layout of q8ta_weight_prepack); set
  // only by the prepacked entry points, which also supply wsum_pre.
  const int8_t* wpk = nullptr;
  // Fused quantize: when xf is set (x NULL), the activations are fp32 [M, K]
  // and are quantized with inv_in = (float)(1/input_scale) and the input zero
  // point before the contraction (the M <= 4 kernel does it while it loads
  // them; launch_quantize_linear sends the other shapes through a workspace).
  const float* xf = nullptr;
  float inv_in = 0.0f;
};
hipError_t launch_linear(const LinearArgs& a, hipStream_t s);
hipError_t launch_quantize_linear(LinearArgs a, hipStream_t s, int8_t* staging = nullptr);

struct DeconvArgs {
  const int8_t* x;
  const int8_t* w;
  const float* wscale;
  const float* bias;
  int8_t* out;
  int32_t* acc;
  int64_t N, IC, H_in, W_in, OC, Kh, Kw, ldw;
  int64_t sh, sw, ph, pw;
  int64_t H_out, W_out;
  int32_t izp;
  Requant rq;
  int64_t dil_h = 1, dil_w = 1;
  int64_t groups = 1;  // IC and OC split into equal groups (weight rows hold IC/groups channels)
  // Fused quantize: when xf is set (x NULL), the input is fp32 NCHW and is
  // quantized on the fly with inv_in = (float)(1/input_scale) and the input
  // zero point, exactly as quantize_per_tensor would.
  const float* xf = nullptr;
  float inv_in = 0.0f;
  // Prepacked weight (the fragment layout of
  // q8ta_conv2d_transposed_weight_prepack); set only by the prepacked entry
  // point, which takes the compile-time-pattern kernel.
  const int8_t* wpk = nullptr;
};
// The same arguments describe the forward q8ta_conv2d (stride, padding and
// dilation of the forward index relation).
hipError_t launch_deconv(const DeconvArgs& a, hipStream_t s);
hipError_t launch_conv2d(const DeconvArgs& a, hipStream_t s);
hipError_t launch_quantize_deconv(DeconvArgs a, hipStream_t s);
// Transposed-conv weight [OC, ldw] -> fragment layout (IC % 64 == 0, 16-byte
// aligned weight and packed, ldw % 16 == 0); its size in bytes.
hipError_t launch_deconv_wprepack(const int8_t* w, int64_t OC, int64_t IC, int64_t Kh, int64_t Kw,
                                  int64_t ldw, int8_t* packed, hipStream_t s);
int64_t deconv_prepacked_bytes(int64_t OC, int64_t IC, int64_t Kh, int64_t Kw);

// Stride phases of a transposed conv, built on the host: for row residue r
// (output rows oh = r + s_h*i) the nth[r] qualifying kernel rows thk[r][t] read
// input rows ih = i + thd[r][t]; likewise for columns.  jb, ib and ocb are tile
// counts filled in by the launchers that use them.
constexpr int kMaxS = 8;    // largest stride taken
constexpr int kMaxT = 16;   // largest number of taps per residue
struct Phases {
  int nth[kMaxS], thk[kMaxS][kMaxT], thd[kMaxS][kMaxT];
  int ntw[kMaxS], twk[kMaxS][kMaxT], twd[kMaxS][kMaxT];
  int jb;     // blocks of 64 phase columns
  int ib;     // blocks of phase rows
  int ocb;    // blocks of output channels
};
// False when a stride or a residue's tap count exceeds the limits above.
bool make_phases(const DeconvArgs& a, Phases& p);

// Individual paths (used by the dispatchers above).
hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t s);
hipError_t launch_gemv(const LinearArgs& a, hipStream_t s);
bool gemv_supported(const LinearArgs& a);
// kind: 0 the default choice; 'x' the 32x32x32 kernel of gemm_mx.hip for any
// shape; 'w' the eight-wave kernel of gemm_w8.hip where it applies (else the
// default choice).
hipError_t launch_gemm_mfma(const LinearArgs& a, hipStream_t s, char kind = 0);
bool gemm_mfma_supported(const LinearArgs& a);
// 32x32x32 matrix-core GEMM for large problems (same operand requirements as
// launch_gemm_mfma, which chooses it).
hipError_t launch_gemm_mx(const LinearArgs& a, hipStream_t s);
// Eight-wave 256 x 256-tile matrix-core GEMM with slab loads straight into
// LDS (gemm_w8.hip): K a multiple of 64, x and w 16-byte aligned.
bool gemm_w8_supported(const LinearArgs& a);
// The default choice takes it (K >= 1024 and its tiles keep most CUs busy).
bool gemm_w8_preferred(const LinearArgs& a);
hipError_t launch_gemm_w8(const LinearArgs& a, hipStream_t s);
int64_t prepacked_bytes(int64_t N, int64_t K);
hipError_t launch_prepack(const int8_t* w, int64_t N, int64_t K, int8_t* packed, hipStream_t s);
hipError_t launch_gemm_pk(const LinearArgs& a, hipStream_t s);
// out[n] = sum_k w[n, k] for an [N, K] int8 matrix (K % 16 == 0, w 16-byte aligned).
hipError_t launch_row_sums(const int8_t* w, int64_t N, int64_t K, int32_t* out, hipStream_t s);
// Same for any K and alignment, rows ldw bytes apart (one thread per row).
hipError_t launch_row_sums_generic(const int8_t* w, int64_t N, int64_t K, int64_t ldw, int32_t* out,
                                   hipStream_t s);
hipError_t launch_deconv_generic(const DeconvArgs& a, hipStream_t s);
hipError_t launch_deconv_fixed(const DeconvArgs& a, hipStream_t s);
bool deconv_fixed_supported(const DeconvArgs& a);
bool deconv_fixed_preferred(const DeconvArgs& a);
hipError_t launch_conv_fixed(const DeconvArgs& a, hipStream_t s);
bool conv_fixed_supported(const DeconvArgs& a);
hipError_t launch_deconv_mx(const DeconvArgs& a, hipStream_t s);
bool deconv_mx_supported(const DeconvArgs& a);
hipError_t launch_conv_mx(const DeconvArgs& a, hipStream_t s);
bool conv_mx_supported(const DeconvArgs& a);
bool conv_mx_preferred(const DeconvArgs& a);
hipError_t launch_deconv_mfma(const DeconvArgs& a, hipStream_t s);
bool deconv_mfma_supported(const DeconvArgs& a);
hipError_t launch_conv_mfma(const DeconvArgs& a, hipStream_t s);
bool conv_mfma_supported(const DeconvArgs& a);
hipError_t launch_deconv_dot4(const DeconvArgs& a, hipStream_t s);
bool deconv_dot4_supported(const DeconvArgs& a);
hipError_t launch_deconv_igemm(const DeconvArgs& a, hipStream_t s);
bool deconv_igemm_supported(const DeconvArgs& a);
hipError_t launch_conv_igemm(const DeconvArgs& a, hipStream_t s);
bool conv_igemm_supported(const DeconvArgs& a);
hipError_t launch_conv2d_generic(const DeconvArgs& a, hipStream_t s);
hipError_t launch_depthwise(const DeconvArgs& a, hipStream_t s);
bool depthwise_supported(const DeconvArgs& a);

}  // namespace q8ta
