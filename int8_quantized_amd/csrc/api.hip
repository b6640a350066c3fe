// libq8ta C ABI: argument checks, kernel choice, launch.
//
// Every entry point validates all of its arguments before touching the HIP
// runtime, so invalid calls fail (loudly, with a status and a message) even
// on a machine without a GPU, and nothing is launched for them.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>
#include <cstdlib>

#include "../../include/q8ta.h"

#include "q8ta_internal.h"

namespace q8ta {
// Kernel-family choice forced through q8ta_select_kernel (0 = default).
extern std::atomic<char> g_sel_linear, g_sel_deconv, g_sel_conv;
}  // namespace q8ta

using namespace q8ta;

namespace {

thread_local char g_err[512] = "no error";

q8ta_status fail(q8ta_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

q8ta_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return Q8TA_OK;
  return fail(Q8TA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool scale_ok(double s) { return std::isfinite(s) && s > 0.0; }
bool zp_ok(int64_t z) { return z >= -128 && z <= 127; }

// Tensors up to 2^40 elements: every kernel forms its addresses in 64 bits.
constexpr int64_t kMaxElems = (int64_t)1 << 40;

// Reciprocal of a scale as the quantize page defines it: divide in double,
// round once to float.
float recip(double s) { return (float)(1.0 / s); }

q8ta_status check_qparams(const char* op, double scale, int64_t zp) {
  if (!scale_ok(scale)) return fail(Q8TA_ERR_QPARAM, "%s: scale must be finite and > 0 (got %g)", op, scale);
  if (!zp_ok(zp)) return fail(Q8TA_ERR_QPARAM, "%s: zero_point must be in [-128, 127] (got %lld)", op, (long long)zp);
  return Q8TA_OK;
}

// "none" or "relu" (the relu-fused variant the pages name as a follow-up);
// anything else, NULL included, fails.
q8ta_status check_activation(const char* op, const char* activation, bool* relu) {
  if (!activation)
    return fail(Q8TA_ERR_UNSUPPORTED, "%s: activation is NULL (\"none\" or \"relu\")", op);
  if (strcmp(activation, "none") == 0) {
    *relu = false;
  } else if (strcmp(activation, "relu") == 0) {
    *relu = true;
  } else {
    return fail(Q8TA_ERR_UNSUPPORTED, "%s: activation \"%.64s\" is not supported (\"none\" or \"relu\")",
                op, activation);
  }
  return Q8TA_OK;
}

Requant make_requant(double input_scale, double output_scale, int64_t output_zero_point, bool relu) {
  const float ozp = (float)output_zero_point;
  return Requant{(float)input_scale, recip(output_scale), ozp, relu ? ozp : -128.0f};
}

// Dilation and groups of the convolutions: dilation >= 1, groups dividing IC
// and OC.
q8ta_status check_dil_groups(const char* op, int64_t IC, int64_t OC, int64_t dh, int64_t dw,
                             int64_t groups) {
  if (groups < 1 || IC < 1 || OC < 1 || IC % groups != 0 || OC % groups != 0)
    return fail(Q8TA_ERR_SHAPE, "%s: groups (%lld) must divide IC and OC", op, (long long)groups);
  if (dh < 1 || dw < 1 || dh > 4096 || dw > 4096)
    return fail(Q8TA_ERR_SHAPE, "%s: dilation must be in [1, 4096]", op);
  return Q8TA_OK;
}

q8ta_status linear_checks(const char* op, const void* x, int64_t M, int64_t K, const int8_t* weight,
                          int64_t N, const void* out) {
  if (!x || !weight || !out) return fail(Q8TA_ERR_NULL, "%s: x, weight and out must not be NULL", op);
  if (M < 1 || K < 1 || N < 1) return fail(Q8TA_ERR_SHAPE, "%s: M, K, N must be >= 1 (got %lld, %lld, %lld)", op,
                                           (long long)M, (long long)K, (long long)N);
  if (M > kMaxElems / K || N > kMaxElems / K || M > kMaxElems / N || K >= ((int64_t)1 << 31))
    return fail(Q8TA_ERR_SHAPE, "%s: sizes too large", op);
  return Q8TA_OK;
}

// Scratch of the allocation-free entry point q8ta_quantize_linear_noalloc:
// the quantized activations of one call (M * K bytes) before its GEMM.  A
// file-scope device array, so each GPU the library runs on holds its own copy
// from module load until the process ends.  In host code `scratch` names a
// host-side stand-in: kernels get the device address noalloc_scratch returns.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;

}  // namespace

static __device__ __align__(256) int8_t scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress, with that device current) and kept.
hipError_t noalloc_scratch(void** p) {
  *p = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!q) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = q;
  }
  *p = g_scratch_ptr[dev];
  return hipSuccess;
}

// out: int8 [M, N]; or, with outf set (out NULL), fp32 [M, N] = the
// dequantized int8 result (fused dequantize_per_tensor with the output's own
// scale and zero point).
q8ta_status linear_impl(const char* op, bool gemv_only, const int8_t* x, int64_t M, int64_t K,
                        double input_scale, int64_t input_zero_point, const int8_t* weight, int64_t N,
                        const float* weight_scales, const float* bias, double output_scale,
                        int64_t output_zero_point, const char* activation, int8_t* out,
                        hipStream_t stream, float* outf = nullptr,
                        const int32_t* wsum_pre = nullptr, bool packed = false,
                        const float* xf = nullptr, bool noalloc = false) {
  q8ta_status st = linear_checks(op, xf ? (const void*)xf : x, M, K, weight, N,
                                 outf ? (const void*)outf : out);
  if (st) return st;
  if (packed && (K % 16 != 0 || ((uintptr_t)x & 15) != 0 || ((uintptr_t)weight & 15) != 0))
    return fail(Q8TA_ERR_UNSUPPORTED,
                "%s: needs K %% 16 == 0 and 16-byte aligned x and packed weight (K = %lld)", op,
                (long long)K);
  if (gemv_only && M != 1) return fail(Q8TA_ERR_SHAPE, "%s: M must be 1 (got %lld)", op, (long long)M);
  if (!weight_scales) return fail(Q8TA_ERR_NULL, "%s: weight_scales must not be NULL", op);
  if ((st = check_qparams(op, input_scale, input_zero_point))) return st;
  if ((st = check_qparams(op, output_scale, output_zero_point))) return st;
  bool relu = false;
  if ((st = check_activation(op, activation, &relu))) return st;

  LinearArgs a{};
  a.x = x; a.w = weight; a.wscale = weight_scales; a.bias = bias; a.out = out; a.acc = nullptr;
  a.M = M; a.K = K; a.N = N; a.izp = (int32_t)input_zero_point;
  a.rq = make_requant(input_scale, output_scale, output_zero_point, relu);
  a.outf = outf;
  a.dq_scale = (float)output_scale;
  a.dq_zp = (int32_t)output_zero_point;
  a.wsum_pre = wsum_pre;
  if (packed) {
    // the eight-wave kernel where the default choice (or the selection) takes
    // it, else the 256 x 128-tile kernel of gemm_pk.hip
    a.wpk = weight;
    const char k = g_sel_linear.load(std::memory_order_relaxed);
    const bool w8 = k == 'w' ? gemm_w8_supported(a) : (k == 0 && gemm_w8_preferred(a));
    return hip_status(w8 ? launch_gemm_w8(a, stream) : launch_gemm_pk(a, stream), op);
  }
  if (xf) {
    a.xf = xf;
    a.inv_in = recip(input_scale);
    if (noalloc) {
      // Only the shapes the M <= 4 kernel refuses stage the quantized
      // activations (M * K bytes); they must fit the static scratch array.
      if (!gemv_supported(a) && (uint64_t)M * (uint64_t)K > kNoAllocScratchBytes)
        return fail(Q8TA_ERR_SHAPE,
                    "%s: M * K = %lld bytes of quantized activations exceed the static scratch "
                    "of %llu bytes", op, (long long)(M * K), (unsigned long long)kNoAllocScratchBytes);
      void* scratch_ptr = nullptr;
      if ((st = hip_status(noalloc_scratch(&scratch_ptr), op))) return st;
      return hip_status(launch_quantize_linear(a, stream, (int8_t*)scratch_ptr), op);
    }
    return hip_status(launch_quantize_linear(a, stream), op);
  }
  return hip_status(launch_linear(a, stream), op);
}

}  // namespace

namespace q8ta {

namespace {

hipError_t pool_alloc(void** p, size_t bytes, hipStream_t s) {
  static std::atomic<uint64_t> pools_set{0};   // one bit per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && !(pools_set.load() & (1ull << dev))) {
    hipMemPool_t pool;
    e = hipDeviceGetDefaultMemPool(&pool, dev);
    uint64_t keep = (uint64_t)1 << 30;
    if (e == hipSuccess) e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) return e;
    pools_set.fetch_or(1ull << dev);
  }
  return hipMallocAsync(p, bytes, s);
}

constexpr int kWsSlots = 4;                          // cached buffers per device
constexpr size_t kWsCachedMax = (size_t)256 << 20;   // larger requests use the pool
constexpr size_t kWsGrain = (size_t)1 << 20;

// A cached workspace buffer.  While `busy` it belongs to one call (between its
// workspace_acquire and workspace_release); `done` is recorded on that call's
// stream at release, after the call's kernels, so that the next holder --
// on any stream -- is ordered after them.
struct WsSlot {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;
  bool busy = false;
};
struct WsDevice {
  WsSlot slot[kWsSlots];
};

// Guards the slot tables only (lookups and flag updates); never held across
// a HIP call that waits or launches.
std::mutex g_ws_mu;
std::map<int, WsDevice> g_ws;

}  // namespace

// Takes a cached buffer of at least `bytes` for stream s without blocking the
// host: a buffer last used on another stream (or by a stream since destroyed)
// is ordered after that use with hipStreamWaitEvent; one that is too small is
// freed and replaced in stream order (hipFreeAsync / hipMallocAsync on s, after
// that wait), so work already queued keeps the memory it was given.  When every
// slot is taken, under graph capture and for requests above 256 MiB the call
// gets its own stream-ordered allocation, freed by workspace_release.
hipError_t workspace_acquire(void** p, size_t bytes, hipStream_t s) {
  *p = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(s, &cap);
  if (e != hipSuccess) return e;
  if (cap != hipStreamCaptureStatusNone || bytes > kWsCachedMax) return pool_alloc(p, bytes, s);

  WsSlot* sl = nullptr;
  WsSlot mine;
  {
    std::lock_guard<std::mutex> g(g_ws_mu);
    WsDevice& d = g_ws[dev];
    // the smallest free buffer that fits, else the largest free one (to grow)
    for (WsSlot& c : d.slot) {
      if (c.busy) continue;
      if (!sl) { sl = &c; continue; }
      const bool c_fits = c.bytes >= bytes, s_fits = sl->bytes >= bytes;
      if (c_fits ? (!s_fits || c.bytes < sl->bytes) : (!s_fits && c.bytes > sl->bytes)) sl = &c;
    }
    if (sl) {
      sl->busy = true;
      mine = *sl;
    }
  }
  if (!sl) return pool_alloc(p, bytes, s);

  if (!mine.done) e = hipEventCreateWithFlags(&mine.done, hipEventDisableTiming);
  if (e == hipSuccess && mine.ptr) {
    const hipError_t q = hipEventQuery(mine.done);   // never recorded: hipSuccess
    if (q == hipErrorNotReady) e = hipStreamWaitEvent(s, mine.done, 0);
    else if (q != hipSuccess) e = q;
  }
  if (e == hipSuccess && mine.bytes < bytes) {
    if (mine.ptr) e = hipFreeAsync(mine.ptr, s);
    mine.ptr = nullptr;
    mine.bytes = 0;
    if (e == hipSuccess) {
      const size_t want = (bytes + kWsGrain - 1) / kWsGrain * kWsGrain;
      e = pool_alloc(&mine.ptr, want, s);
      if (e == hipSuccess) mine.bytes = want;
      else mine.ptr = nullptr;
    }
  }
  {
    std::lock_guard<std::mutex> g(g_ws_mu);
    sl->ptr = mine.ptr;
    sl->bytes = mine.bytes;
    sl->done = mine.done;
    if (e != hipSuccess) sl->busy = false;
  }
  if (e != hipSuccess) return e;
  *p = mine.ptr;
  return hipSuccess;
}

// Returns a buffer from workspace_acquire once the call's kernels are queued
// on s: a cached one is marked free after its event is recorded on s, any
// other is freed in stream order.
hipError_t workspace_release(void* p, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  WsSlot* sl = nullptr;
  hipEvent_t done = nullptr;
  {
    std::lock_guard<std::mutex> g(g_ws_mu);
    auto it = g_ws.find(dev);
    if (it != g_ws.end())
      for (WsSlot& c : it->second.slot)
        if (c.busy && c.ptr == p) {
          sl = &c;
          done = c.done;
          break;
        }
  }
  if (!sl) return p ? hipFreeAsync(p, s) : hipSuccess;
  e = hipEventRecord(done, s);
  std::lock_guard<std::mutex> g(g_ws_mu);
  sl->busy = false;
  return e;
}

// Kernel-family choice forced through q8ta_select_kernel (0 = default).
std::atomic<char> g_sel_linear{0}, g_sel_deconv{0}, g_sel_conv{0};

hipError_t launch_linear(const LinearArgs& a, hipStream_t s) {
  const char k = g_sel_linear.load(std::memory_order_relaxed);
  if (k == 'g') return launch_linear_generic(a, s);
  if (gemv_supported(a)) return launch_gemv(a, s);
  if (gemm_mfma_supported(a)) return launch_gemm_mfma(a, s, k);
  return launch_linear_generic(a, s);
}

// quantize_per_tensor -> linear with fp32 activations (a.xf): the M <= 4
// kernel quantizes while it loads them; other shapes quantize into an int8
// buffer of M * K bytes -- `staging` when given (the allocation-free entry
// point's static scratch), else a workspace -- and take the usual path.
hipError_t launch_quantize_linear(LinearArgs a, hipStream_t s, int8_t* staging) {
  if (gemv_supported(a)) return launch_gemv(a, s);
  const int64_t numel = a.M * a.K;
  void* ws = staging;
  hipError_t e = staging ? hipSuccess : workspace_acquire(&ws, (size_t)numel, s);
  if (e != hipSuccess) return e;
  e = launch_quantize(a.xf, (int8_t*)ws, numel, a.inv_in, (float)a.izp, s);
  if (e == hipSuccess) {
    a.x = (const int8_t*)ws;
    a.xf = nullptr;
    e = launch_linear(a, s);
  }
  if (staging) return e;
  hipError_t f = workspace_release(ws, s);
  return e != hipSuccess ? e : f;
}

// Transposed conv: the compile-time-pattern 32x32x32 kernel for 3x3 and 4x4
// stride-2 shapes with at least one workgroup per CU, then the tiled
// 16x16x64 matrix-core kernel for every shape it supports, then the implicit
// GEMM (three launches' worth of fixed cost: input copy, then the GEMM) from
// about 2^28 multiply-adds, then the direct tiled kernel, then the
// shape-general one.  q8ta_select_kernel can force one family ('f' pattern,
// 'x' 32x32x32, 'm' 16x16x64, 'i' implicit GEMM, 't' tiled, 'g' generic)
// where the shape allows it.
// The forced family when it takes the shape, else 0 (the default choice).
static char deconv_family(const DeconvArgs& a) {
  const char k = g_sel_deconv.load(std::memory_order_relaxed);
  switch (k) {
    case 'f': return deconv_fixed_supported(a) ? k : 0;
    case 'x': return deconv_mx_supported(a) ? k : 0;
    case 'm': return deconv_mfma_supported(a) ? k : 0;
    case 'i': return deconv_igemm_supported(a) ? k : 0;
    case 't': return deconv_dot4_supported(a) ? k : 0;
    default: return k;   // 0 or 'g' (the generic kernel takes every shape)
  }
}

static bool deconv_wants_igemm(const DeconvArgs& a) {
  const char k = deconv_family(a);
  const double macs = (double)a.N * a.OC * a.H_out * a.W_out * a.IC * a.Kh * a.Kw /
                      ((double)a.sh * a.sw);
  return (k ? k == 'i' : macs >= (double)(1 << 28)) && deconv_igemm_supported(a);
}

hipError_t launch_deconv(const DeconvArgs& a, hipStream_t s) {
  const char k = deconv_family(a);
  if ((k == 0 && deconv_fixed_preferred(a)) || (k == 'f' && deconv_fixed_supported(a)))
    return launch_deconv_fixed(a, s);
  if (k == 'x' && deconv_mx_supported(a)) return launch_deconv_mx(a, s);
  if ((k == 0 || k == 'm') && deconv_mfma_supported(a)) return launch_deconv_mfma(a, s);
  if (deconv_wants_igemm(a)) return launch_deconv_igemm(a, s);
  if (k != 'g' && deconv_dot4_supported(a)) return launch_deconv_dot4(a, s);
  return launch_deconv_generic(a, s);
}

// quantize_per_tensor -> transposed conv with an fp32 input (a.xf): the
// compile-time-pattern kernel and the implicit GEMM quantize while they stage
// or copy the input; the other paths quantize into a stream-ordered int8
// workspace.
hipError_t launch_quantize_deconv(DeconvArgs a, hipStream_t s) {
  const char k = deconv_family(a);
  if ((k == 0 && deconv_fixed_preferred(a)) || (k == 'f' && deconv_fixed_supported(a)))
    return launch_deconv_fixed(a, s);
  const bool mfma = ((k == 0 || k == 'm') && deconv_mfma_supported(a)) ||
                    (k == 0 && deconv_fixed_preferred(a)) ||
                    (k == 'x' && deconv_mx_supported(a)) ||
                    (k == 'f' && deconv_fixed_supported(a));
  if (!mfma && k != 'm' && k != 'x' && k != 'f' && deconv_wants_igemm(a))
    return launch_deconv_igemm(a, s);
  const int64_t numel = a.N * a.IC * a.H_in * a.W_in;
  void* ws = nullptr;
  hipError_t e = workspace_acquire(&ws, (size_t)numel, s);
  if (e != hipSuccess) return e;
  e = launch_quantize(a.xf, (int8_t*)ws, numel, a.inv_in, (float)a.izp, s);
  if (e == hipSuccess) {
    a.x = (const int8_t*)ws;
    a.xf = nullptr;
    e = launch_deconv(a, s);
  }
  hipError_t f = workspace_release(ws, s);
  return e != hipSuccess ? e : f;
}

// Forward conv: the 32x32x32 kernel for large stride-1 shapes (IC % 32 == 0,
// W_in % 4 == 0), the 16x16x64 matrix-core kernel (groups 1, stride 1, IC % 16 == 0),
// the implicit GEMM on v_dot4 (groups 1, IC % 64 == 0), the depthwise kernel
// (groups == IC == OC), or the shape-general kernel.  q8ta_select_kernel can
// force one ('m', 'i', 'g') where the shape allows it.
hipError_t launch_conv2d(const DeconvArgs& a, hipStream_t s) {
  char k = g_sel_conv.load(std::memory_order_relaxed);
  // a forced family that does not take the shape falls back to the default
  if ((k == 'f' && !conv_fixed_supported(a)) || (k == 'x' && !conv_mx_supported(a)) ||
      (k == 'm' && !conv_mfma_supported(a)) || (k == 'i' && !conv_igemm_supported(a)))
    k = 0;
  if (k == 'f' && conv_fixed_supported(a)) return launch_conv_fixed(a, s);
  if ((k == 0 && conv_mx_preferred(a)) || (k == 'x' && conv_mx_supported(a)))
    return launch_conv_mx(a, s);
  if ((k == 0 || k == 'm') && conv_mfma_supported(a)) return launch_conv_mfma(a, s);
  if ((k == 0 || k == 'i') && conv_igemm_supported(a)) return launch_conv_igemm(a, s);
  if (k == 'g') return launch_conv2d_generic(a, s);
  if (depthwise_supported(a)) return launch_depthwise(a, s);
  return launch_conv2d_generic(a, s);
}

}  // namespace q8ta

extern "C" {

const char* q8ta_last_error(void) { return g_err; }

q8ta_status q8ta_select_kernel(const char* op, const char* kernel) {
  if (!op || !kernel) return fail(Q8TA_ERR_NULL, "q8ta_select_kernel: op and kernel must not be NULL");
  struct Name { const char* name; char code; };
  static const Name linear[] = {{"default", 0}, {"mfma32", 'x'}, {"mfma32_8w", 'w'}, {"generic", 'g'}};
  static const Name deconv[] = {{"default", 0}, {"fixed", 'f'}, {"mfma32", 'x'}, {"mfma", 'm'},
                                {"igemm", 'i'}, {"tiled", 't'}, {"generic", 'g'}};
  static const Name conv[] = {{"default", 0}, {"fixed", 'f'}, {"mfma32", 'x'}, {"mfma", 'm'},
                              {"igemm", 'i'}, {"generic", 'g'}};
  const Name* tab = nullptr;
  size_t n = 0;
  std::atomic<char>* dst = nullptr;
  if (strcmp(op, "linear") == 0) { tab = linear; n = 4; dst = &g_sel_linear; }
  else if (strcmp(op, "conv2d_transposed") == 0) { tab = deconv; n = 7; dst = &g_sel_deconv; }
  else if (strcmp(op, "conv2d") == 0) { tab = conv; n = 6; dst = &g_sel_conv; }
  else return fail(Q8TA_ERR_UNSUPPORTED, "q8ta_select_kernel: unknown op \"%.64s\"", op);
  for (size_t i = 0; i < n; ++i)
    if (strcmp(kernel, tab[i].name) == 0) {
      dst->store(tab[i].code, std::memory_order_relaxed);
      return Q8TA_OK;
    }
  return fail(Q8TA_ERR_UNSUPPORTED, "q8ta_select_kernel: unknown kernel \"%.64s\" for %s", kernel, op);
}

q8ta_status q8ta_quantize_per_tensor(const float* x, int8_t* out, int64_t numel, double scale,
                                     int64_t zero_point, hipStream_t stream) {
  const char* op = "q8ta_quantize_per_tensor";
  if (numel < 0 || numel > kMaxElems) return fail(Q8TA_ERR_SHAPE, "%s: numel out of range (%lld)", op, (long long)numel);
  q8ta_status st = check_qparams(op, scale, zero_point);
  if (st) return st;
  if (numel == 0) return Q8TA_OK;
  if (!x || !out) return fail(Q8TA_ERR_NULL, "%s: x and out must not be NULL", op);
  return hip_status(launch_quantize(x, out, numel, recip(scale), (float)zero_point, stream), op);
}

q8ta_status q8ta_dequantize_per_tensor(const int8_t* x, float* out, int64_t numel, double scale,
                                       int64_t zero_point, hipStream_t stream) {
  const char* op = "q8ta_dequantize_per_tensor";
  if (numel < 0 || numel > kMaxElems) return fail(Q8TA_ERR_SHAPE, "%s: numel out of range (%lld)", op, (long long)numel);
  q8ta_status st = check_qparams(op, scale, zero_point);
  if (st) return st;
  if (numel == 0) return Q8TA_OK;
  if (!x || !out) return fail(Q8TA_ERR_NULL, "%s: x and out must not be NULL", op);
  return hip_status(launch_dequantize(x, out, numel, (float)scale, (int)zero_point, stream), op);
}

q8ta_status q8ta_linear(const int8_t* x, int64_t M, int64_t K, double input_scale,
                        int64_t input_zero_point, const int8_t* weight, int64_t N,
                        const int32_t* weight_sums, const float* weight_scales, const float* bias,
                        double output_scale, int64_t output_zero_point, const char* activation,
                        int8_t* out, hipStream_t stream) {
  (void)weight_sums;
  return linear_impl("q8ta_linear", false, x, M, K, input_scale, input_zero_point, weight, N,
                     weight_scales, bias, output_scale, output_zero_point, activation, out, stream);
}

q8ta_status q8ta_linear_gemv(const int8_t* x, int64_t M, int64_t K, double input_scale,
                             int64_t input_zero_point, const int8_t* weight, int64_t N,
                             const int32_t* weight_sums, const float* weight_scales,
                             const float* bias, double output_scale, int64_t output_zero_point,
                             const char* activation, int8_t* out, hipStream_t stream) {
  (void)weight_sums;
  return linear_impl("q8ta_linear_gemv", true, x, M, K, input_scale, input_zero_point, weight, N,
                     weight_scales, bias, output_scale, output_zero_point, activation, out, stream);
}

q8ta_status q8ta_linear_dq(const int8_t* x, int64_t M, int64_t K, double input_scale,
                           int64_t input_zero_point, const int8_t* weight, int64_t N,
                           const int32_t* weight_sums, const float* weight_scales,
                           const float* bias, double output_scale, int64_t output_zero_point,
                           const char* activation, float* out, hipStream_t stream) {
  (void)weight_sums;
  return linear_impl("q8ta_linear_dq", false, x, M, K, input_scale, input_zero_point, weight, N,
                     weight_scales, bias, output_scale, output_zero_point, activation, nullptr,
                     stream, out);
}

q8ta_status q8ta_quantize_linear(const float* x, int64_t M, int64_t K, double input_scale,
                                 int64_t input_zero_point, const int8_t* weight, int64_t N,
                                 const int32_t* weight_sums, const float* weight_scales,
                                 const float* bias, double output_scale,
                                 int64_t output_zero_point, const char* activation, int8_t* out,
                                 hipStream_t stream) {
  (void)weight_sums;
  return linear_impl("q8ta_quantize_linear", false, nullptr, M, K, input_scale, input_zero_point,
                     weight, N, weight_scales, bias, output_scale, output_zero_point, activation,
                     out, stream, nullptr, nullptr, false, x);
}

q8ta_status q8ta_quantize_linear_dq(const float* x, int64_t M, int64_t K, double input_scale,
                                    int64_t input_zero_point, const int8_t* weight, int64_t N,
                                    const int32_t* weight_sums, const float* weight_scales,
                                    const float* bias, double output_scale,
                                    int64_t output_zero_point, const char* activation, float* out,
                                    hipStream_t stream) {
  (void)weight_sums;
  return linear_impl("q8ta_quantize_linear_dq", false, nullptr, M, K, input_scale,
                     input_zero_point, weight, N, weight_scales, bias, output_scale,
                     output_zero_point, activation, nullptr, stream, out, nullptr, false, x);
}

q8ta_status q8ta_quantize_linear_noalloc(const float* x, int64_t M, int64_t K,
                                         double input_scale, int64_t input_zero_point,
                                         const int8_t* weight, int64_t N,
                                         const int32_t* weight_sums, const float* weight_scales,
                                         const float* bias, double output_scale,
                                         int64_t output_zero_point, const char* activation,
                                         int8_t* out, hipStream_t stream) {
  (void)weight_sums;
  return linear_impl("q8ta_quantize_linear_noalloc", false, nullptr, M, K, input_scale,
                     input_zero_point, weight, N, weight_scales, bias, output_scale,
                     output_zero_point, activation, out, stream, nullptr, nullptr, false, x, true);
}

q8ta_status q8ta_weight_sums(const int8_t* weight, int64_t N, int64_t K, int32_t* sums,
                             hipStream_t stream) {
  const char* op = "q8ta_weight_sums";
  if (!weight || !sums) return fail(Q8TA_ERR_NULL, "%s: weight and sums must not be NULL", op);
  if (N < 1 || K < 1 || N > kMaxElems / K || K >= ((int64_t)1 << 31))
    return fail(Q8TA_ERR_SHAPE, "%s: N and K must be >= 1 (got %lld, %lld)", op, (long long)N,
                (long long)K);
  if (K % 16 == 0 && ((uintptr_t)weight & 15) == 0)
    return hip_status(launch_row_sums(weight, N, K, sums, stream), op);
  return hip_status(launch_row_sums_generic(weight, N, K, K, sums, stream), op);
}

q8ta_status q8ta_linear_presummed(const int8_t* x, int64_t M, int64_t K, double input_scale,
                                  int64_t input_zero_point, const int8_t* weight, int64_t N,
                                  const int32_t* weight_sums, const float* weight_scales,
                                  const float* bias, double output_scale,
                                  int64_t output_zero_point, const char* activation, int8_t* out,
                                  hipStream_t stream) {
  const char* op = "q8ta_linear_presummed";
  if (!weight_sums) return fail(Q8TA_ERR_NULL, "%s: weight_sums must not be NULL", op);
  return linear_impl(op, false, x, M, K, input_scale, input_zero_point, weight, N, weight_scales,
                     bias, output_scale, output_zero_point, activation, out, stream, nullptr,
                     weight_sums);
}

q8ta_status q8ta_linear_dq_presummed(const int8_t* x, int64_t M, int64_t K, double input_scale,
                                     int64_t input_zero_point, const int8_t* weight, int64_t N,
                                     const int32_t* weight_sums, const float* weight_scales,
                                     const float* bias, double output_scale,
                                     int64_t output_zero_point, const char* activation, float* out,
                                     hipStream_t stream) {
  const char* op = "q8ta_linear_dq_presummed";
  if (!weight_sums) return fail(Q8TA_ERR_NULL, "%s: weight_sums must not be NULL", op);
  return linear_impl(op, false, x, M, K, input_scale, input_zero_point, weight, N, weight_scales,
                     bias, output_scale, output_zero_point, activation, nullptr, stream, out,
                     weight_sums);
}

int64_t q8ta_weight_prepacked_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 1 || N > kMaxElems / K || K >= ((int64_t)1 << 31)) return -1;
  return prepacked_bytes(N, K);
}

q8ta_status q8ta_weight_prepack(const int8_t* weight, int64_t N, int64_t K, int8_t* packed,
                                hipStream_t stream) {
  const char* op = "q8ta_weight_prepack";
  if (!weight || !packed) return fail(Q8TA_ERR_NULL, "%s: weight and packed must not be NULL", op);
  if (q8ta_weight_prepacked_bytes(N, K) < 0)
    return fail(Q8TA_ERR_SHAPE, "%s: N and K must be >= 1 (got %lld, %lld)", op, (long long)N,
                (long long)K);
  if (K % 16 != 0 || ((uintptr_t)weight & 15) != 0 || ((uintptr_t)packed & 15) != 0)
    return fail(Q8TA_ERR_UNSUPPORTED,
                "%s: needs K %% 16 == 0 and 16-byte aligned weight and packed (K = %lld)", op,
                (long long)K);
  return hip_status(launch_prepack(weight, N, K, packed, stream), op);
}

q8ta_status q8ta_linear_prepacked(const int8_t* x, int64_t M, int64_t K, double input_scale,
                                  int64_t input_zero_point, const int8_t* packed_weight, int64_t N,
                                  const int32_t* weight_sums, const float* weight_scales,
                                  const float* bias, double output_scale,
                                  int64_t output_zero_point, const char* activation, int8_t* out,
                                  hipStream_t stream) {
  const char* op = "q8ta_linear_prepacked";
  if (!weight_sums) return fail(Q8TA_ERR_NULL, "%s: weight_sums must not be NULL", op);
  return linear_impl(op, false, x, M, K, input_scale, input_zero_point, packed_weight, N,
                     weight_scales, bias, output_scale, output_zero_point, activation, out, stream,
                     nullptr, weight_sums, true);
}

q8ta_status q8ta_linear_dq_prepacked(const int8_t* x, int64_t M, int64_t K, double input_scale,
                                     int64_t input_zero_point, const int8_t* packed_weight,
                                     int64_t N, const int32_t* weight_sums,
                                     const float* weight_scales, const float* bias,
                                     double output_scale, int64_t output_zero_point,
                                     const char* activation, float* out, hipStream_t stream) {
  const char* op = "q8ta_linear_dq_prepacked";
  if (!weight_sums) return fail(Q8TA_ERR_NULL, "%s: weight_sums must not be NULL", op);
  return linear_impl(op, false, x, M, K, input_scale, input_zero_point, packed_weight, N,
                     weight_scales, bias, output_scale, output_zero_point, activation, nullptr,
                     stream, out, weight_sums, true);
}

q8ta_status q8ta_linear_acc(const int8_t* x, int64_t M, int64_t K, int64_t input_zero_point,
                            const int8_t* weight, int64_t N, int32_t* acc, hipStream_t stream) {
  const char* op = "q8ta_linear_acc";
  q8ta_status st = linear_checks(op, x, M, K, weight, N, acc);
  if (st) return st;
  if (!zp_ok(input_zero_point)) return fail(Q8TA_ERR_QPARAM, "%s: input_zero_point out of range", op);
  LinearArgs a{};
  a.x = x; a.w = weight; a.acc = acc; a.M = M; a.K = K; a.N = N;
  a.izp = (int32_t)input_zero_point;
  return hip_status(launch_linear(a, stream), op);
}

}  // extern "C"

namespace {

// icg: input channels per weight row (IC, or IC / groups for a grouped conv).
q8ta_status deconv_checks(const char* op, const int8_t* x, int64_t N, int64_t IC, int64_t H_in,
                          int64_t W_in, const int8_t* weight, int64_t OC, int64_t Kh, int64_t Kw,
                          int64_t ldw, int64_t sh, int64_t sw, int64_t ph, int64_t pw,
                          const void* out, int64_t H_out, int64_t W_out, int64_t icg) {
  if (!x || !weight || !out) return fail(Q8TA_ERR_NULL, "%s: x, weight and out must not be NULL", op);
  if (N < 1 || IC < 1 || H_in < 1 || W_in < 1 || OC < 1 || Kh < 1 || Kw < 1 || H_out < 1 || W_out < 1)
    return fail(Q8TA_ERR_SHAPE, "%s: all sizes must be >= 1", op);
  const int64_t lim = (int64_t)1 << 24;
  if (N > lim || IC > lim || H_in > lim || W_in > lim || OC > lim || Kh > 4096 || Kw > 4096 ||
      H_out > lim || W_out > lim)
    return fail(Q8TA_ERR_SHAPE, "%s: a size is too large", op);
  if (Kh * Kw > kMaxElems / IC) return fail(Q8TA_ERR_SHAPE, "%s: Kh*Kw*IC too large", op);
  if (ldw < Kh * Kw * icg)
    return fail(Q8TA_ERR_SHAPE, "%s: weight_row_stride (%lld) must be >= Kh*Kw*%s (%lld)", op,
                (long long)ldw, icg == IC ? "IC" : "IC/groups", (long long)(Kh * Kw * icg));
  if (sh < 1 || sw < 1 || sh > 4096 || sw > 4096) return fail(Q8TA_ERR_SHAPE, "%s: stride must be >= 1", op);
  if (ph < 0 || pw < 0 || ph > lim || pw > lim) return fail(Q8TA_ERR_SHAPE, "%s: padding must be >= 0", op);
  const double xe = (double)N * IC * H_in * W_in, oe = (double)N * OC * H_out * W_out,
               we = (double)OC * ldw;
  if (xe > (double)kMaxElems || oe > (double)kMaxElems || we > (double)kMaxElems)
    return fail(Q8TA_ERR_SHAPE, "%s: tensors too large", op);
  return Q8TA_OK;
}

}  // namespace

extern "C" {

q8ta_status q8ta_conv2d_transposed(const int8_t* x, int64_t N, int64_t IC, int64_t H_in, int64_t W_in,
                                   double input_scale, int64_t input_zero_point, const int8_t* weight,
                                   int64_t OC, int64_t Kh, int64_t Kw, int64_t weight_row_stride,
                                   const int32_t* weight_sums, const float* weight_scales,
                                   const float* bias, double output_scale, int64_t output_zero_point,
                                   int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                                   int64_t output_padding_h, int64_t output_padding_w,
                                   int64_t dilation_h, int64_t dilation_w, int64_t groups,
                                   const char* activation, int8_t* out, int64_t H_out, int64_t W_out,
                                   hipStream_t stream) {
  const char* op = "q8ta_conv2d_transposed";
  (void)weight_sums;
  (void)output_padding_h;
  (void)output_padding_w;
  q8ta_status st = check_dil_groups(op, IC, OC, dilation_h, dilation_w, groups);
  if (st) return st;
  st = deconv_checks(op, x, N, IC, H_in, W_in, weight, OC, Kh, Kw, weight_row_stride, stride_h,
                     stride_w, pad_h, pad_w, out, H_out, W_out, IC / groups);
  if (st) return st;
  if (!weight_scales) return fail(Q8TA_ERR_NULL, "%s: weight_scales must not be NULL", op);
  if ((st = check_qparams(op, input_scale, input_zero_point))) return st;
  if ((st = check_qparams(op, output_scale, output_zero_point))) return st;
  bool relu = false;
  if ((st = check_activation(op, activation, &relu))) return st;

  DeconvArgs a{};
  a.x = x; a.w = weight; a.wscale = weight_scales; a.bias = bias; a.out = out; a.acc = nullptr;
  a.N = N; a.IC = IC; a.H_in = H_in; a.W_in = W_in; a.OC = OC; a.Kh = Kh; a.Kw = Kw;
  a.ldw = weight_row_stride; a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w;
  a.dil_h = dilation_h; a.dil_w = dilation_w; a.groups = groups;
  a.H_out = H_out; a.W_out = W_out; a.izp = (int32_t)input_zero_point;
  a.rq = make_requant(input_scale, output_scale, output_zero_point, relu);
  return hip_status(launch_deconv(a, stream), op);
}

int64_t q8ta_conv2d_transposed_weight_prepacked_bytes(int64_t OC, int64_t IC, int64_t Kh,
                                                      int64_t Kw) {
  const int64_t lim = (int64_t)1 << 24;
  if (OC < 1 || IC < 1 || Kh < 1 || Kw < 1 || OC > lim || IC > lim || Kh > 4096 || Kw > 4096)
    return -1;
  if (IC % 64 != 0 || Kh * Kw > kMaxElems / IC || (OC + 31) / 32 * 32 > kMaxElems / (Kh * Kw * IC))
    return -1;
  return deconv_prepacked_bytes(OC, IC, Kh, Kw);
}

q8ta_status q8ta_conv2d_transposed_weight_prepack(const int8_t* weight, int64_t OC, int64_t IC,
                                                  int64_t Kh, int64_t Kw,
                                                  int64_t weight_row_stride, int8_t* packed,
                                                  hipStream_t stream) {
  const char* op = "q8ta_conv2d_transposed_weight_prepack";
  if (!weight || !packed) return fail(Q8TA_ERR_NULL, "%s: weight and packed must not be NULL", op);
  if (OC < 1 || IC < 1 || Kh < 1 || Kw < 1)
    return fail(Q8TA_ERR_SHAPE, "%s: OC, IC, Kh and Kw must be >= 1", op);
  if (q8ta_conv2d_transposed_weight_prepacked_bytes(OC, IC, Kh, Kw) < 0)
    return fail(Q8TA_ERR_UNSUPPORTED, "%s: needs IC %% 64 == 0 and sizes in range (IC = %lld)", op,
                (long long)IC);
  if (weight_row_stride < Kh * Kw * IC || (double)OC * weight_row_stride > (double)kMaxElems)
    return fail(Q8TA_ERR_SHAPE, "%s: weight_row_stride (%lld) must be >= Kh*Kw*IC (%lld)", op,
                (long long)weight_row_stride, (long long)(Kh * Kw * IC));
  if (weight_row_stride % 16 != 0 || ((uintptr_t)weight & 15) != 0 || ((uintptr_t)packed & 15) != 0)
    return fail(Q8TA_ERR_UNSUPPORTED,
                "%s: needs weight_row_stride %% 16 == 0 and 16-byte aligned weight and packed", op);
  return hip_status(launch_deconv_wprepack(weight, OC, IC, Kh, Kw, weight_row_stride, packed,
                                           stream), op);
}

q8ta_status q8ta_conv2d_transposed_prepacked(
    const int8_t* x, int64_t N, int64_t IC, int64_t H_in, int64_t W_in, double input_scale,
    int64_t input_zero_point, const int8_t* packed_weight, int64_t OC, int64_t Kh, int64_t Kw,
    const int32_t* weight_sums, const float* weight_scales, const float* bias, double output_scale,
    int64_t output_zero_point, int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
    int64_t output_padding_h, int64_t output_padding_w, int64_t dilation_h, int64_t dilation_w,
    int64_t groups, const char* activation, int8_t* out, int64_t H_out, int64_t W_out,
    hipStream_t stream) {
  const char* op = "q8ta_conv2d_transposed_prepacked";
  (void)weight_sums;
  (void)output_padding_h;
  (void)output_padding_w;
  q8ta_status st = check_dil_groups(op, IC, OC, dilation_h, dilation_w, groups);
  if (st) return st;
  st = deconv_checks(op, x, N, IC, H_in, W_in, packed_weight, OC, Kh, Kw, Kh * Kw * IC, stride_h,
                     stride_w, pad_h, pad_w, out, H_out, W_out, IC / groups);
  if (st) return st;
  if (!weight_scales) return fail(Q8TA_ERR_NULL, "%s: weight_scales must not be NULL", op);
  if ((st = check_qparams(op, input_scale, input_zero_point))) return st;
  if ((st = check_qparams(op, output_scale, output_zero_point))) return st;
  bool relu = false;
  if ((st = check_activation(op, activation, &relu))) return st;
  DeconvArgs a{};
  a.x = x; a.w = packed_weight; a.wpk = packed_weight; a.wscale = weight_scales; a.bias = bias;
  a.out = out; a.acc = nullptr;
  a.N = N; a.IC = IC; a.H_in = H_in; a.W_in = W_in; a.OC = OC; a.Kh = Kh; a.Kw = Kw;
  a.ldw = Kh * Kw * IC; a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w;
  a.dil_h = dilation_h; a.dil_w = dilation_w; a.groups = groups;
  a.H_out = H_out; a.W_out = W_out; a.izp = (int32_t)input_zero_point;
  a.rq = make_requant(input_scale, output_scale, output_zero_point, relu);
  if (!deconv_fixed_supported(a))
    return fail(Q8TA_ERR_UNSUPPORTED,
                "%s: takes the 3x3 / 4x4 stride-2 shapes of the compile-time-pattern kernel only "
                "(groups 1, dilation 1, equal padding parities, IC %% 64 == 0 with the input halo "
                "of a tile in LDS, W_in %% 4 == 0, 4-byte aligned x, 16-byte aligned "
                "packed_weight); use q8ta_conv2d_transposed", op);
  return hip_status(launch_deconv_fixed(a, stream), op);
}

q8ta_status q8ta_conv2d_transposed_acc(const int8_t* x, int64_t N, int64_t IC, int64_t H_in,
                                       int64_t W_in, int64_t input_zero_point, const int8_t* weight,
                                       int64_t OC, int64_t Kh, int64_t Kw, int64_t weight_row_stride,
                                       int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
                                       int64_t dilation_h, int64_t dilation_w, int64_t groups,
                                       int32_t* acc, int64_t H_out, int64_t W_out, hipStream_t stream) {
  const char* op = "q8ta_conv2d_transposed_acc";
  q8ta_status st = check_dil_groups(op, IC, OC, dilation_h, dilation_w, groups);
  if (st) return st;
  st = deconv_checks(op, x, N, IC, H_in, W_in, weight, OC, Kh, Kw, weight_row_stride, stride_h,
                     stride_w, pad_h, pad_w, acc, H_out, W_out, IC / groups);
  if (st) return st;
  if (!zp_ok(input_zero_point)) return fail(Q8TA_ERR_QPARAM, "%s: input_zero_point out of range", op);
  DeconvArgs a{};
  a.x = x; a.w = weight; a.acc = acc;
  a.N = N; a.IC = IC; a.H_in = H_in; a.W_in = W_in; a.OC = OC; a.Kh = Kh; a.Kw = Kw;
  a.ldw = weight_row_stride; a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w;
  a.dil_h = dilation_h; a.dil_w = dilation_w; a.groups = groups;
  a.H_out = H_out; a.W_out = W_out; a.izp = (int32_t)input_zero_point;
  return hip_status(launch_deconv(a, stream), op);
}


q8ta_status q8ta_conv2d(const int8_t* x, int64_t N, int64_t IC, int64_t H_in, int64_t W_in,
                        double input_scale, int64_t input_zero_point, const int8_t* weight,
                        int64_t OC, int64_t Kh, int64_t Kw, int64_t weight_row_stride,
                        const int32_t* weight_sums, const float* weight_scales, const float* bias,
                        double output_scale, int64_t output_zero_point, int64_t stride_h,
                        int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dilation_h,
                        int64_t dilation_w, int64_t groups, const char* activation, int8_t* out,
                        int64_t H_out, int64_t W_out, hipStream_t stream) {
  const char* op = "q8ta_conv2d";
  (void)weight_sums;
  q8ta_status st = check_dil_groups(op, IC, OC, dilation_h, dilation_w, groups);
  if (st) return st;
  st = deconv_checks(op, x, N, IC, H_in, W_in, weight, OC, Kh, Kw, weight_row_stride, stride_h,
                     stride_w, pad_h, pad_w, out, H_out, W_out, IC / groups);
  if (st) return st;
  if (!weight_scales) return fail(Q8TA_ERR_NULL, "%s: weight_scales must not be NULL", op);
  if ((st = check_qparams(op, input_scale, input_zero_point))) return st;
  if ((st = check_qparams(op, output_scale, output_zero_point))) return st;
  bool relu = false;
  if ((st = check_activation(op, activation, &relu))) return st;

  DeconvArgs a{};
  a.x = x; a.w = weight; a.wscale = weight_scales; a.bias = bias; a.out = out; a.acc = nullptr;
  a.N = N; a.IC = IC; a.H_in = H_in; a.W_in = W_in; a.OC = OC; a.Kh = Kh; a.Kw = Kw;
  a.ldw = weight_row_stride; a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w;
  a.dil_h = dilation_h; a.dil_w = dilation_w; a.groups = groups;
  a.H_out = H_out; a.W_out = W_out; a.izp = (int32_t)input_zero_point;
  a.rq = make_requant(input_scale, output_scale, output_zero_point, relu);
  return hip_status(launch_conv2d(a, stream), op);
}

q8ta_status q8ta_conv2d_acc(const int8_t* x, int64_t N, int64_t IC, int64_t H_in, int64_t W_in,
                            int64_t input_zero_point, const int8_t* weight, int64_t OC, int64_t Kh,
                            int64_t Kw, int64_t weight_row_stride, int64_t stride_h,
                            int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t dilation_h,
                            int64_t dilation_w, int64_t groups, int32_t* acc, int64_t H_out,
                            int64_t W_out, hipStream_t stream) {
  const char* op = "q8ta_conv2d_acc";
  q8ta_status st = check_dil_groups(op, IC, OC, dilation_h, dilation_w, groups);
  if (st) return st;
  st = deconv_checks(op, x, N, IC, H_in, W_in, weight, OC, Kh, Kw, weight_row_stride, stride_h,
                     stride_w, pad_h, pad_w, acc, H_out, W_out, IC / groups);
  if (st) return st;
  if (!zp_ok(input_zero_point)) return fail(Q8TA_ERR_QPARAM, "%s: input_zero_point out of range", op);
  DeconvArgs a{};
  a.x = x; a.w = weight; a.acc = acc;
  a.N = N; a.IC = IC; a.H_in = H_in; a.W_in = W_in; a.OC = OC; a.Kh = Kh; a.Kw = Kw;
  a.ldw = weight_row_stride; a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w;
  a.dil_h = dilation_h; a.dil_w = dilation_w; a.groups = groups;
  a.H_out = H_out; a.W_out = W_out; a.izp = (int32_t)input_zero_point;
  return hip_status(launch_conv2d(a, stream), op);
}


q8ta_status q8ta_quantize_conv2d_transposed(
    const float* x, int64_t N, int64_t IC, int64_t H_in, int64_t W_in, double input_scale,
    int64_t input_zero_point, const int8_t* weight, int64_t OC, int64_t Kh, int64_t Kw,
    int64_t weight_row_stride, const int32_t* weight_sums, const float* weight_scales,
    const float* bias, double output_scale, int64_t output_zero_point, int64_t stride_h,
    int64_t stride_w, int64_t pad_h, int64_t pad_w, int64_t output_padding_h,
    int64_t output_padding_w, int64_t dilation_h, int64_t dilation_w, int64_t groups,
    const char* activation, int8_t* out, int64_t H_out, int64_t W_out, hipStream_t stream) {
  const char* op = "q8ta_quantize_conv2d_transposed";
  (void)weight_sums;
  (void)output_padding_h;
  (void)output_padding_w;
  q8ta_status st = check_dil_groups(op, IC, OC, dilation_h, dilation_w, groups);
  if (st) return st;
  st = deconv_checks(op, (const int8_t*)x, N, IC, H_in, W_in, weight, OC, Kh, Kw,
                     weight_row_stride, stride_h, stride_w, pad_h, pad_w, out, H_out, W_out,
                     IC / groups);
  if (st) return st;
  if (!weight_scales) return fail(Q8TA_ERR_NULL, "%s: weight_scales must not be NULL", op);
  if ((st = check_qparams(op, input_scale, input_zero_point))) return st;
  if ((st = check_qparams(op, output_scale, output_zero_point))) return st;
  bool relu = false;
  if ((st = check_activation(op, activation, &relu))) return st;

  DeconvArgs a{};
  a.x = nullptr; a.xf = x; a.inv_in = recip(input_scale);
  a.w = weight; a.wscale = weight_scales; a.bias = bias; a.out = out; a.acc = nullptr;
  a.N = N; a.IC = IC; a.H_in = H_in; a.W_in = W_in; a.OC = OC; a.Kh = Kh; a.Kw = Kw;
  a.ldw = weight_row_stride; a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w;
  a.dil_h = dilation_h; a.dil_w = dilation_w; a.groups = groups;
  a.H_out = H_out; a.W_out = W_out; a.izp = (int32_t)input_zero_point;
  a.rq = make_requant(input_scale, output_scale, output_zero_point, relu);
  return hip_status(launch_quantize_deconv(a, stream), op);
}

q8ta_status q8ta_quantize_conv2d_transposed_prepacked(
    const float* x, int64_t N, int64_t IC, int64_t H_in, int64_t W_in, double input_scale,
    int64_t input_zero_point, const int8_t* packed_weight, int64_t OC, int64_t Kh, int64_t Kw,
    const int32_t* weight_sums, const float* weight_scales, const float* bias, double output_scale,
    int64_t output_zero_point, int64_t stride_h, int64_t stride_w, int64_t pad_h, int64_t pad_w,
    int64_t output_padding_h, int64_t output_padding_w, int64_t dilation_h, int64_t dilation_w,
    int64_t groups, const char* activation, int8_t* out, int64_t H_out, int64_t W_out,
    hipStream_t stream) {
  const char* op = "q8ta_quantize_conv2d_transposed_prepacked";
  (void)weight_sums;
  (void)output_padding_h;
  (void)output_padding_w;
  q8ta_status st = check_dil_groups(op, IC, OC, dilation_h, dilation_w, groups);
  if (st) return st;
  st = deconv_checks(op, (const int8_t*)x, N, IC, H_in, W_in, packed_weight, OC, Kh, Kw,
                     Kh * Kw * IC, stride_h, stride_w, pad_h, pad_w, out, H_out, W_out, IC / groups);
  if (st) return st;
  if (!weight_scales) return fail(Q8TA_ERR_NULL, "%s: weight_scales must not be NULL", op);
  if ((st = check_qparams(op, input_scale, input_zero_point))) return st;
  if ((st = check_qparams(op, output_scale, output_zero_point))) return st;
  bool relu = false;
  if ((st = check_activation(op, activation, &relu))) return st;
  DeconvArgs a{};
  a.x = nullptr; a.xf = x; a.inv_in = recip(input_scale);
  a.w = packed_weight; a.wpk = packed_weight; a.wscale = weight_scales; a.bias = bias;
  a.out = out; a.acc = nullptr;
  a.N = N; a.IC = IC; a.H_in = H_in; a.W_in = W_in; a.OC = OC; a.Kh = Kh; a.Kw = Kw;
  a.ldw = Kh * Kw * IC; a.sh = stride_h; a.sw = stride_w; a.ph = pad_h; a.pw = pad_w;
  a.dil_h = dilation_h; a.dil_w = dilation_w; a.groups = groups;
  a.H_out = H_out; a.W_out = W_out; a.izp = (int32_t)input_zero_point;
  a.rq = make_requant(input_scale, output_scale, output_zero_point, relu);
  if (!deconv_fixed_supported(a))
    return fail(Q8TA_ERR_UNSUPPORTED,
                "%s: takes the 3x3 / 4x4 stride-2 shapes of the compile-time-pattern kernel only "
                "(groups 1, dilation 1, equal padding parities, IC %% 64 == 0 with the input halo "
                "of a tile in LDS, W_in %% 4 == 0, 16-byte aligned x and packed_weight); use "
                "q8ta_quantize_conv2d_transposed", op);
  return hip_status(launch_deconv_fixed(a, stream), op);
}

}  // extern "C"
