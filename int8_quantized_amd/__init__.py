"""int8_quantized_amd -- Python binding of libq8ta (MI355X / gfx950).

Thin ctypes marshalling over the C ABI declared in ``include/q8ta.h``: every
function here has the name of the C entry point it calls, checks that its
tensors are dense device tensors of the right dtype, and passes their data
pointers, sizes and the current HIP stream.  All arithmetic runs in the HIP
kernels of ``libq8ta.so``; there is no fallback.  If the library has not been
built, loading fails loudly (build it with ``python -m int8_quantized_amd.build``).

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq8ta.so")

Q8TA_OK = 0
Q8TA_ERR_NULL = 1
Q8TA_ERR_SHAPE = 2
Q8TA_ERR_QPARAM = 3
Q8TA_ERR_UNSUPPORTED = 4
Q8TA_ERR_HIP = 5

STATUS_NAMES = {0: "Q8TA_OK", 1: "Q8TA_ERR_NULL", 2: "Q8TA_ERR_SHAPE", 3: "Q8TA_ERR_QPARAM",
                4: "Q8TA_ERR_UNSUPPORTED", 5: "Q8TA_ERR_HIP"}


class Q8taError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_I64 = ctypes.c_int64
_DBL = ctypes.c_double
_P = ctypes.c_void_p
_S = ctypes.c_char_p

# argument types of every exported entry point, in declaration order
SIGNATURES = {
    "q8ta_last_error": ([], ctypes.c_char_p),
    "q8ta_select_kernel": ([_S, _S], ctypes.c_int),
    "q8ta_quantize_per_tensor": ([_P, _P, _I64, _DBL, _I64, _P], ctypes.c_int),
    "q8ta_dequantize_per_tensor": ([_P, _P, _I64, _DBL, _I64, _P], ctypes.c_int),
    "q8ta_linear": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64, _S, _P, _P],
                    ctypes.c_int),
    "q8ta_linear_gemv": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64, _S, _P,
                          _P], ctypes.c_int),
    "q8ta_conv2d_transposed": ([_P, _I64, _I64, _I64, _I64, _DBL, _I64, _P, _I64, _I64, _I64, _I64,
                                _P, _P, _P, _DBL, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                _I64, _I64, _S, _P, _I64, _I64, _P], ctypes.c_int),
    "q8ta_linear_dq": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64, _S, _P, _P],
                       ctypes.c_int),
    "q8ta_quantize_linear": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64, _S,
                              _P, _P], ctypes.c_int),
    "q8ta_quantize_linear_dq": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64,
                                 _S, _P, _P], ctypes.c_int),
    "q8ta_quantize_linear_noalloc": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL,
                                      _I64, _S, _P, _P], ctypes.c_int),
    "q8ta_weight_sums": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "q8ta_linear_presummed": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64, _S,
                               _P, _P], ctypes.c_int),
    "q8ta_linear_dq_presummed": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64,
                                  _S, _P, _P], ctypes.c_int),
    "q8ta_weight_prepacked_bytes": ([_I64, _I64], ctypes.c_int64),
    "q8ta_conv2d_transposed_weight_prepacked_bytes": ([_I64, _I64, _I64, _I64], ctypes.c_int64),
    "q8ta_conv2d_transposed_weight_prepack": ([_P, _I64, _I64, _I64, _I64, _I64, _P, _P],
                                              ctypes.c_int),
    "q8ta_conv2d_transposed_prepacked": ([_P, _I64, _I64, _I64, _I64, _DBL, _I64, _P, _I64, _I64,
                                          _I64, _P, _P, _P, _DBL, _I64, _I64, _I64, _I64, _I64,
                                          _I64, _I64, _I64, _I64, _I64, _S, _P, _I64, _I64, _P],
                                         ctypes.c_int),
    "q8ta_quantize_conv2d_transposed_prepacked": ([_P, _I64, _I64, _I64, _I64, _DBL, _I64, _P, _I64,
                                                   _I64, _I64, _P, _P, _P, _DBL, _I64, _I64, _I64,
                                                   _I64, _I64, _I64, _I64, _I64, _I64, _I64, _S,
                                                   _P, _I64, _I64, _P], ctypes.c_int),
    "q8ta_weight_prepack": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "q8ta_linear_prepacked": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64, _S,
                               _P, _P], ctypes.c_int),
    "q8ta_linear_dq_prepacked": ([_P, _I64, _I64, _DBL, _I64, _P, _I64, _P, _P, _P, _DBL, _I64,
                                  _S, _P, _P], ctypes.c_int),
    "q8ta_quantize_conv2d_transposed": ([_P, _I64, _I64, _I64, _I64, _DBL, _I64, _P, _I64, _I64,
                                         _I64, _I64, _P, _P, _P, _DBL, _I64, _I64, _I64, _I64,
                                         _I64, _I64, _I64, _I64, _I64, _I64, _S, _P, _I64, _I64,
                                         _P], ctypes.c_int),
    "q8ta_linear_acc": ([_P, _I64, _I64, _I64, _P, _I64, _P, _P], ctypes.c_int),
    "q8ta_conv2d_transposed_acc": ([_P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _I64, _I64,
                                    _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P],
                                   ctypes.c_int),
    "q8ta_conv2d": ([_P, _I64, _I64, _I64, _I64, _DBL, _I64, _P, _I64, _I64, _I64, _I64,
                     _P, _P, _P, _DBL, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                     _I64, _S, _P, _I64, _I64, _P], ctypes.c_int),
    "q8ta_conv2d_acc": ([_P, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _I64, _I64,
                         _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P, _I64, _I64, _P],
                        ctypes.c_int),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libq8ta.so with argument types set (raises if not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libq8ta.so not found at {LIB_PATH}: build it with "
                "`python -m int8_quantized_amd.build` (there is no CPU fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.argtypes = args
            fn.restype = res
        _lib = l
    return _lib


def q8ta_last_error() -> str:
    return lib().q8ta_last_error().decode()


def _check(status: int):
    if status != Q8TA_OK:
        raise Q8taError(status, q8ta_last_error())


def q8ta_select_kernel(op: str, kernel: str) -> None:
    """Force one kernel family of ``op`` ("linear", "conv2d_transposed",
    "conv2d") where the shape allows it; "default" restores the normal choice."""
    _check(lib().q8ta_select_kernel(op.encode(), kernel.encode()))


def _torch():
    import torch
    return torch


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _opt(t, dtype, name):
    return None if t is None else _dev(t, dtype, name)


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _act(activation):
    return None if activation is None else activation.encode()


# ---------------------------------------------------------------------------
def q8ta_quantize_per_tensor(x, out, scale: float, zero_point: int, stream=None):
    """out (int8) = clamp(rint(x * (float)(1/scale)) + zero_point, -128, 127)."""
    torch = _torch()
    if x.numel() != out.numel():
        raise ValueError("x and out must have the same number of elements")
    _check(lib().q8ta_quantize_per_tensor(_dev(x, torch.float32, "x"), _dev(out, torch.int8, "out"),
                                          x.numel(), float(scale), int(zero_point), _stream(stream)))
    return out


def q8ta_dequantize_per_tensor(x, out, scale: float, zero_point: int, stream=None):
    """out (fp32) = (float)(x - zero_point) * (float)scale."""
    torch = _torch()
    if x.numel() != out.numel():
        raise ValueError("x and out must have the same number of elements")
    _check(lib().q8ta_dequantize_per_tensor(_dev(x, torch.int8, "x"), _dev(out, torch.float32, "out"),
                                            x.numel(), float(scale), int(zero_point), _stream(stream)))
    return out


def _linear(fn, x, input_scale, input_zero_point, weight, weight_sums, weight_scales, bias,
            output_scale, output_zero_point, activation, out, stream):
    torch = _torch()
    if x.dim() != 2 or weight.dim() != 2 or out.dim() != 2:
        raise ValueError("x [M,K], weight [N,K] and out [M,N] must be 2-D")
    M, K = x.shape
    N = weight.shape[0]
    if weight.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, weight {tuple(weight.shape)}, "
                         f"out {tuple(out.shape)}")
    _check(fn(_dev(x, torch.int8, "x"), M, K, float(input_scale), int(input_zero_point),
              _dev(weight, torch.int8, "weight"), N, _opt(weight_sums, torch.int32, "weight_sums"),
              _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
              float(output_scale), int(output_zero_point), _act(activation),
              _dev(out, torch.int8, "out"), _stream(stream)))
    return out


def q8ta_linear(x, input_scale, input_zero_point, weight, weight_sums, weight_scales, bias,
                output_scale, output_zero_point, activation, out, stream=None):
    """int8 [M,K] x int8 [N,K] -> int8 [M,N] with the per-channel epilogue."""
    return _linear(lib().q8ta_linear, x, input_scale, input_zero_point, weight, weight_sums,
                   weight_scales, bias, output_scale, output_zero_point, activation, out, stream)


def q8ta_linear_gemv(x, input_scale, input_zero_point, weight, weight_sums, weight_scales, bias,
                     output_scale, output_zero_point, activation, out, stream=None):
    """q8ta_linear for M == 1."""
    return _linear(lib().q8ta_linear_gemv, x, input_scale, input_zero_point, weight, weight_sums,
                   weight_scales, bias, output_scale, output_zero_point, activation, out, stream)


def q8ta_weight_sums(weight, sums, stream=None):
    """sums[n] = sum_k weight[n, k] (int32 [N]) for int8 weight [N, K]."""
    torch = _torch()
    if weight.dim() != 2 or tuple(sums.shape) != (weight.shape[0],):
        raise ValueError("weight [N, K] and sums [N] expected")
    _check(lib().q8ta_weight_sums(_dev(weight, torch.int8, "weight"), weight.shape[0],
                                  weight.shape[1], _dev(sums, torch.int32, "sums"),
                                  _stream(stream)))
    return sums


def q8ta_linear_presummed(x, input_scale, input_zero_point, weight, weight_sums, weight_scales,
                          bias, output_scale, output_zero_point, activation, out, stream=None):
    """q8ta_linear with the caller's (trusted) weight_sums."""
    if weight_sums is None:
        raise ValueError("weight_sums is required")
    return _linear(lib().q8ta_linear_presummed, x, input_scale, input_zero_point, weight,
                   weight_sums, weight_scales, bias, output_scale, output_zero_point, activation,
                   out, stream)


def q8ta_linear_dq_presummed(x, input_scale, input_zero_point, weight, weight_sums, weight_scales,
                             bias, output_scale, output_zero_point, activation, out, stream=None):
    """q8ta_linear_dq with the caller's (trusted) weight_sums: fp32 out [M, N]."""
    torch = _torch()
    if weight_sums is None:
        raise ValueError("weight_sums is required")
    M, K = x.shape
    N = weight.shape[0]
    if weight.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("weight [N, K] and out [M, N] expected")
    _check(lib().q8ta_linear_dq_presummed(
        _dev(x, torch.int8, "x"), M, K, float(input_scale), int(input_zero_point),
        _dev(weight, torch.int8, "weight"), N, _dev(weight_sums, torch.int32, "weight_sums"),
        _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
        float(output_scale), int(output_zero_point), _act(activation),
        _dev(out, torch.float32, "out"), _stream(stream)))
    return out


def q8ta_weight_prepacked_bytes(N: int, K: int) -> int:
    """Size in bytes of the prepacked layout of an int8 [N, K] weight (-1 if invalid)."""
    return int(lib().q8ta_weight_prepacked_bytes(int(N), int(K)))


def q8ta_weight_prepack(weight, packed, stream=None):
    """Rearrange int8 weight [N, K] into the matrix-core fragment layout
    (packed: int8 device tensor of q8ta_weight_prepacked_bytes(N, K) bytes)."""
    torch = _torch()
    if weight.dim() != 2:
        raise ValueError("weight [N, K] expected")
    N, K = weight.shape
    if packed.numel() != q8ta_weight_prepacked_bytes(N, K):
        raise ValueError(f"packed must hold {q8ta_weight_prepacked_bytes(N, K)} bytes")
    _check(lib().q8ta_weight_prepack(_dev(weight, torch.int8, "weight"), N, K,
                                     _dev(packed, torch.int8, "packed"), _stream(stream)))
    return packed


def _linear_pk(fn, out_dtype, x, input_scale, input_zero_point, packed, N, weight_sums,
               weight_scales, bias, output_scale, output_zero_point, activation, out, stream):
    torch = _torch()
    if weight_sums is None:
        raise ValueError("weight_sums is required")
    if x.dim() != 2 or tuple(out.shape) != (x.shape[0], N):
        raise ValueError("x [M, K] and out [M, N] expected")
    M, K = x.shape
    if packed.numel() != q8ta_weight_prepacked_bytes(N, K):
        raise ValueError("packed does not hold an [N, K] prepacked weight")
    _check(fn(_dev(x, torch.int8, "x"), M, K, float(input_scale), int(input_zero_point),
              _dev(packed, torch.int8, "packed"), int(N),
              _dev(weight_sums, torch.int32, "weight_sums"),
              _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
              float(output_scale), int(output_zero_point), _act(activation),
              _dev(out, out_dtype, "out"), _stream(stream)))
    return out


def q8ta_linear_prepacked(x, input_scale, input_zero_point, packed, N, weight_sums, weight_scales,
                          bias, output_scale, output_zero_point, activation, out, stream=None):
    """q8ta_linear_presummed on a prepacked weight of N rows: int8 out [M, N]."""
    return _linear_pk(lib().q8ta_linear_prepacked, _torch().int8, x, input_scale,
                      input_zero_point, packed, N, weight_sums, weight_scales, bias, output_scale,
                      output_zero_point, activation, out, stream)


def q8ta_linear_dq_prepacked(x, input_scale, input_zero_point, packed, N, weight_sums,
                             weight_scales, bias, output_scale, output_zero_point, activation, out,
                             stream=None):
    """q8ta_linear_dq_presummed on a prepacked weight of N rows: fp32 out [M, N]."""
    return _linear_pk(lib().q8ta_linear_dq_prepacked, _torch().float32, x, input_scale,
                      input_zero_point, packed, N, weight_sums, weight_scales, bias, output_scale,
                      output_zero_point, activation, out, stream)


def q8ta_linear_acc(x, input_zero_point, weight, acc, stream=None):
    """int32 accumulator of q8ta_linear: acc[m,n] = sum_k (x[m,k]-izp)*w[n,k]."""
    torch = _torch()
    M, K = x.shape
    N = weight.shape[0]
    if weight.shape[1] != K or tuple(acc.shape) != (M, N):
        raise ValueError("shape mismatch")
    _check(lib().q8ta_linear_acc(_dev(x, torch.int8, "x"), M, K, int(input_zero_point),
                                 _dev(weight, torch.int8, "weight"), N,
                                 _dev(acc, torch.int32, "acc"), _stream(stream)))
    return acc


def q8ta_linear_dq(x, input_scale, input_zero_point, weight, weight_sums, weight_scales, bias,
                   output_scale, output_zero_point, activation, out, stream=None):
    """q8ta_linear then dequantize_per_tensor of its output, in one call:
    fp32 out [M, N]."""
    torch = _torch()
    M, K = x.shape
    N = weight.shape[0]
    if weight.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError("weight [N, K] and out [M, N] expected")
    _check(lib().q8ta_linear_dq(
        _dev(x, torch.int8, "x"), M, K, float(input_scale), int(input_zero_point),
        _dev(weight, torch.int8, "weight"), N, _opt(weight_sums, torch.int32, "weight_sums"),
        _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
        float(output_scale), int(output_zero_point), _act(activation),
        _dev(out, torch.float32, "out"), _stream(stream)))
    return out


def _quantize_linear(fn, out_dtype, x, input_scale, input_zero_point, weight, weight_sums,
                     weight_scales, bias, output_scale, output_zero_point, activation, out, stream):
    torch = _torch()
    if x.dim() != 2 or weight.dim() != 2 or out.dim() != 2:
        raise ValueError("x [M,K], weight [N,K] and out [M,N] must be 2-D")
    M, K = x.shape
    N = weight.shape[0]
    if weight.shape[1] != K or tuple(out.shape) != (M, N):
        raise ValueError(f"shape mismatch: x {tuple(x.shape)}, weight {tuple(weight.shape)}, "
                         f"out {tuple(out.shape)}")
    _check(fn(_dev(x, torch.float32, "x"), M, K, float(input_scale), int(input_zero_point),
              _dev(weight, torch.int8, "weight"), N, _opt(weight_sums, torch.int32, "weight_sums"),
              _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
              float(output_scale), int(output_zero_point), _act(activation),
              _dev(out, out_dtype, "out"), _stream(stream)))
    return out


def q8ta_quantize_linear(x, input_scale, input_zero_point, weight, weight_sums, weight_scales,
                         bias, output_scale, output_zero_point, activation, out, stream=None):
    """quantize_per_tensor of fp32 x [M, K] (input_scale, input_zero_point), then
    q8ta_linear, in one call: int8 out [M, N]."""
    return _quantize_linear(lib().q8ta_quantize_linear, _torch().int8, x, input_scale,
                            input_zero_point, weight, weight_sums, weight_scales, bias,
                            output_scale, output_zero_point, activation, out, stream)


def q8ta_quantize_linear_noalloc(x, input_scale, input_zero_point, weight, weight_sums,
                                 weight_scales, bias, output_scale, output_zero_point, activation,
                                 out, stream=None):
    """q8ta_quantize_linear without any device allocation (the quantized
    activations go through the library's static scratch; M * K <= 16 MiB)."""
    return _quantize_linear(lib().q8ta_quantize_linear_noalloc, _torch().int8, x, input_scale,
                            input_zero_point, weight, weight_sums, weight_scales, bias,
                            output_scale, output_zero_point, activation, out, stream)


def q8ta_quantize_linear_dq(x, input_scale, input_zero_point, weight, weight_sums, weight_scales,
                            bias, output_scale, output_zero_point, activation, out, stream=None):
    """quantize_per_tensor -> q8ta_linear -> dequantize_per_tensor of fp32 x [M, K]
    in one call: fp32 out [M, N]."""
    return _quantize_linear(lib().q8ta_quantize_linear_dq, _torch().float32, x, input_scale,
                            input_zero_point, weight, weight_sums, weight_scales, bias,
                            output_scale, output_zero_point, activation, out, stream)


def q8ta_conv2d_transposed(x, input_scale, input_zero_point, weight, Kh, Kw, weight_sums,
                           weight_scales, bias, output_scale, output_zero_point, stride, padding,
                           output_padding, dilation, groups, activation, out, stream=None):
    """int8 NCHW x int8 [OC, ldw] -> int8 NCHW out (H_out, W_out taken from out)."""
    torch = _torch()
    if x.dim() != 4 or weight.dim() != 2 or out.dim() != 4:
        raise ValueError("x [N,IC,H,W], weight [OC, ldw] and out [N,OC,H_out,W_out] expected")
    N, IC, H_in, W_in = x.shape
    OC, ldw = weight.shape
    if out.shape[0] != N or out.shape[1] != OC:
        raise ValueError("out must be [N, OC, H_out, W_out]")
    H_out, W_out = out.shape[2], out.shape[3]
    _check(lib().q8ta_conv2d_transposed(
        _dev(x, torch.int8, "x"), N, IC, H_in, W_in, float(input_scale), int(input_zero_point),
        _dev(weight, torch.int8, "weight"), OC, int(Kh), int(Kw), ldw,
        _opt(weight_sums, torch.int32, "weight_sums"),
        _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
        float(output_scale), int(output_zero_point), int(stride[0]), int(stride[1]),
        int(padding[0]), int(padding[1]), int(output_padding[0]), int(output_padding[1]),
        int(dilation[0]), int(dilation[1]), int(groups), _act(activation),
        _dev(out, torch.int8, "out"), H_out, W_out, _stream(stream)))
    return out


def q8ta_conv2d_transposed_weight_prepacked_bytes(OC: int, IC: int, Kh: int, Kw: int) -> int:
    """Size in bytes of the prepacked transposed-conv weight (-1 if unsupported)."""
    return int(lib().q8ta_conv2d_transposed_weight_prepacked_bytes(int(OC), int(IC), int(Kh),
                                                                   int(Kw)))


def q8ta_conv2d_transposed_weight_prepack(weight, IC, Kh, Kw, packed, stream=None):
    """Rearrange the int8 [OC, ldw] transposed-conv weight into its fragment
    layout (packed: int8 device tensor of the prepacked size)."""
    torch = _torch()
    if weight.dim() != 2:
        raise ValueError("weight [OC, ldw] expected")
    OC, ldw = weight.shape
    nb = q8ta_conv2d_transposed_weight_prepacked_bytes(OC, IC, Kh, Kw)
    if packed.numel() != nb:
        raise ValueError(f"packed must hold {nb} bytes")
    _check(lib().q8ta_conv2d_transposed_weight_prepack(
        _dev(weight, torch.int8, "weight"), OC, int(IC), int(Kh), int(Kw), ldw,
        _dev(packed, torch.int8, "packed"), _stream(stream)))
    return packed


def q8ta_conv2d_transposed_prepacked(x, input_scale, input_zero_point, packed, OC, Kh, Kw,
                                     weight_sums, weight_scales, bias, output_scale,
                                     output_zero_point, stride, padding, output_padding, dilation,
                                     groups, activation, out, stream=None):
    """q8ta_conv2d_transposed on a prepacked weight (H_out, W_out taken from out);
    with an fp32 x, q8ta_quantize_conv2d_transposed_prepacked."""
    torch = _torch()
    fp32 = x.dtype == torch.float32
    fn = (lib().q8ta_quantize_conv2d_transposed_prepacked if fp32
          else lib().q8ta_conv2d_transposed_prepacked)
    if x.dim() != 4 or out.dim() != 4:
        raise ValueError("x [N,IC,H,W] and out [N,OC,H_out,W_out] expected")
    N, IC, H_in, W_in = x.shape
    if out.shape[0] != N or out.shape[1] != OC:
        raise ValueError("out must be [N, OC, H_out, W_out]")
    if packed.numel() != q8ta_conv2d_transposed_weight_prepacked_bytes(OC, IC, Kh, Kw):
        raise ValueError("packed does not hold an [OC, Kh*Kw*IC] prepacked weight")
    _check(fn(
        _dev(x, torch.float32 if fp32 else torch.int8, "x"), N, IC, H_in, W_in,
        float(input_scale), int(input_zero_point),
        _dev(packed, torch.int8, "packed"), int(OC), int(Kh), int(Kw),
        _opt(weight_sums, torch.int32, "weight_sums"),
        _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
        float(output_scale), int(output_zero_point), int(stride[0]), int(stride[1]),
        int(padding[0]), int(padding[1]), int(output_padding[0]), int(output_padding[1]),
        int(dilation[0]), int(dilation[1]), int(groups), _act(activation),
        _dev(out, torch.int8, "out"), out.shape[2], out.shape[3], _stream(stream)))
    return out


def q8ta_quantize_conv2d_transposed(x, input_scale, input_zero_point, weight, Kh, Kw,
                                    weight_sums, weight_scales, bias, output_scale,
                                    output_zero_point, stride, padding, output_padding, dilation,
                                    groups, activation, out, stream=None):
    """quantize_per_tensor of the fp32 NCHW x, then q8ta_conv2d_transposed, in
    one call (H_out, W_out taken from out)."""
    torch = _torch()
    if x.dim() != 4 or weight.dim() != 2 or out.dim() != 4:
        raise ValueError("x [N,IC,H,W], weight [OC, ldw] and out [N,OC,H_out,W_out] expected")
    N, IC, H_in, W_in = x.shape
    OC, ldw = weight.shape
    if out.shape[0] != N or out.shape[1] != OC:
        raise ValueError("out must be [N, OC, H_out, W_out]")
    _check(lib().q8ta_quantize_conv2d_transposed(
        _dev(x, torch.float32, "x"), N, IC, H_in, W_in, float(input_scale),
        int(input_zero_point), _dev(weight, torch.int8, "weight"), OC, int(Kh), int(Kw), ldw,
        _opt(weight_sums, torch.int32, "weight_sums"),
        _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
        float(output_scale), int(output_zero_point), int(stride[0]), int(stride[1]),
        int(padding[0]), int(padding[1]), int(output_padding[0]), int(output_padding[1]),
        int(dilation[0]), int(dilation[1]), int(groups), _act(activation),
        _dev(out, torch.int8, "out"), out.shape[2], out.shape[3], _stream(stream)))
    return out


def q8ta_conv2d_transposed_acc(x, input_zero_point, weight, Kh, Kw, stride, padding, acc,
                               stream=None, dilation=(1, 1), groups=1):
    """int32 accumulator of q8ta_conv2d_transposed (NCHW [N, OC, H_out, W_out])."""
    torch = _torch()
    N, IC, H_in, W_in = x.shape
    OC, ldw = weight.shape
    if acc.dim() != 4 or acc.shape[0] != N or acc.shape[1] != OC:
        raise ValueError("acc must be [N, OC, H_out, W_out]")
    _check(lib().q8ta_conv2d_transposed_acc(
        _dev(x, torch.int8, "x"), N, IC, H_in, W_in, int(input_zero_point),
        _dev(weight, torch.int8, "weight"), OC, int(Kh), int(Kw), ldw, int(stride[0]),
        int(stride[1]), int(padding[0]), int(padding[1]), int(dilation[0]), int(dilation[1]),
        int(groups), _dev(acc, torch.int32, "acc"), acc.shape[2], acc.shape[3],
        _stream(stream)))
    return acc


def q8ta_conv2d(x, input_scale, input_zero_point, weight, Kh, Kw, weight_sums, weight_scales,
                bias, output_scale, output_zero_point, stride, padding, dilation, groups,
                activation, out, stream=None):
    """Forward conv: int8 NCHW x int8 [OC, ldw] -> int8 NCHW out (H_out, W_out
    taken from out)."""
    torch = _torch()
    if x.dim() != 4 or weight.dim() != 2 or out.dim() != 4:
        raise ValueError("x [N,IC,H,W], weight [OC, ldw] and out [N,OC,H_out,W_out] expected")
    N, IC, H_in, W_in = x.shape
    OC, ldw = weight.shape
    if out.shape[0] != N or out.shape[1] != OC:
        raise ValueError("out must be [N, OC, H_out, W_out]")
    _check(lib().q8ta_conv2d(
        _dev(x, torch.int8, "x"), N, IC, H_in, W_in, float(input_scale), int(input_zero_point),
        _dev(weight, torch.int8, "weight"), OC, int(Kh), int(Kw), ldw,
        _opt(weight_sums, torch.int32, "weight_sums"),
        _dev(weight_scales, torch.float32, "weight_scales"), _opt(bias, torch.float32, "bias"),
        float(output_scale), int(output_zero_point), int(stride[0]), int(stride[1]),
        int(padding[0]), int(padding[1]), int(dilation[0]), int(dilation[1]), int(groups),
        _act(activation), _dev(out, torch.int8, "out"), out.shape[2], out.shape[3],
        _stream(stream)))
    return out


def q8ta_conv2d_acc(x, input_zero_point, weight, Kh, Kw, stride, padding, dilation, acc,
                    groups=1, stream=None):
    """int32 accumulator of q8ta_conv2d (NCHW [N, OC, H_out, W_out])."""
    torch = _torch()
    N, IC, H_in, W_in = x.shape
    OC, ldw = weight.shape
    if acc.dim() != 4 or acc.shape[0] != N or acc.shape[1] != OC:
        raise ValueError("acc must be [N, OC, H_out, W_out]")
    _check(lib().q8ta_conv2d_acc(
        _dev(x, torch.int8, "x"), N, IC, H_in, W_in, int(input_zero_point),
        _dev(weight, torch.int8, "weight"), OC, int(Kh), int(Kw), ldw, int(stride[0]),
        int(stride[1]), int(padding[0]), int(padding[1]), int(dilation[0]), int(dilation[1]),
        int(groups), _dev(acc, torch.int32, "acc"), acc.shape[2], acc.shape[3],
        _stream(stream)))
    return acc


__all__ = [
    "Q8taError", "lib", "q8ta_last_error", "q8ta_quantize_per_tensor", "q8ta_dequantize_per_tensor",
    "q8ta_linear", "q8ta_linear_gemv", "q8ta_linear_dq", "q8ta_linear_acc", "q8ta_conv2d_transposed",
    "q8ta_quantize_linear", "q8ta_quantize_linear_dq",
    "q8ta_weight_sums", "q8ta_linear_presummed", "q8ta_linear_dq_presummed",
    "q8ta_weight_prepacked_bytes", "q8ta_weight_prepack", "q8ta_linear_prepacked",
    "q8ta_linear_dq_prepacked",
    "q8ta_conv2d_transposed_acc", "q8ta_quantize_conv2d_transposed", "q8ta_conv2d",
    "q8ta_conv2d_acc", "q8ta_conv2d_transposed_weight_prepacked_bytes",
    "q8ta_conv2d_transposed_weight_prepack", "q8ta_conv2d_transposed_prepacked",
    "q8ta_quantize_conv2d_transposed_prepacked",
]
