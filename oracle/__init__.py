"""q8ta CPU oracle -- TEST INFRASTRUCTURE ONLY.

A numpy-facing wrapper around ``q8ta_oracle.c``: plain, slow, obviously
correct CPU definitions of the int8 quantized-activation operations from the
ExecuTorch WebGPU pull-request pages "Add quantize_per_tensor op (int8 buffer
path)" (#21187), "Add q8ta_linear op (int8 quantized linear)" (#21197) and
"Add q8ta_conv2d_transposed op (int8 transposed conv)" (#21205).  Each function
names the passage it follows.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``int8_quantized_amd``) and imports nothing from it.

Every function is pinned by ``tests/test_oracle_pins.py`` against values fixed
by the pages or by mathematics: torch's decomposed quantize/dequantize ops,
float64 matmul / conv_transpose2d, brute force on tiny inputs, hand-derived
fixtures under ``tests/golden/``, and the error bound of the float epilogue.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8ta_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# Tests that plant a mistake in a copy of the oracle point this at the copy.
_LIB_OVERRIDE = os.environ.get("Q8TA_ORACLE_LIB")

OK, BAD_ARG, OVERFLOW = 0, 1, 2

_c_i64 = ctypes.c_int64
_c_dbl = ctypes.c_double
_c_ptr = ctypes.c_void_p


GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
             "-shared", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """gcc-compile an oracle C source into a shared library at `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc"] + GCC_FLAGS + ["-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    """Compile ``q8ta_oracle.c`` with gcc (no FMA contraction, no fast-math)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    return compile_source(_SRC, _LIB)


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            lib = ctypes.CDLL(_LIB)
        for name in ("oracle_quantize_per_tensor", "oracle_dequantize_per_tensor",
                     "oracle_epilogue", "oracle_linear_acc", "oracle_linear_acc_folded",
                     "oracle_linear", "oracle_deconv_acc_gather", "oracle_deconv_acc_scatter",
                     "oracle_deconv_acc_zpfill", "oracle_conv2d_transposed",
                     "oracle_conv2d_acc", "oracle_conv2d"):
            getattr(lib, name).restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _chk(rc, what):
    if rc == OVERFLOW:
        raise OverflowError(f"{what}: an accumulator left the int32 range")
    if rc != OK:
        raise ValueError(f"{what}: bad argument (rc={rc})")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _relu_flag(activation: str) -> int:
    """"none" -> 0, "relu" -> 1 (the relu-fused follow-up of #21197/#21205)."""
    if activation not in ("none", "relu"):
        raise ValueError(f"unknown activation {activation!r}")
    return 1 if activation == "relu" else 0


# ---------------------------------------------------------------------------
def quantize_per_tensor(x, scale: float, zero_point: int) -> np.ndarray:
    """#21187 Solution/Implementation: clamp(round(x*inv_scale)+zp, -128, 127),
    inv_scale = float(1.0/scale) taken in double, round half to even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.int8)
    _chk(_load().oracle_quantize_per_tensor(_p(x), _p(out), _c_i64(x.size), _c_dbl(scale),
                                            _c_i64(zero_point)), "quantize")
    return out


def dequantize_per_tensor(q, scale: float, zero_point: int) -> np.ndarray:
    """Decomposed dequantize (named, not printed, by #21197/#21205 Problem):
    float(q - zp) * float(scale)."""
    q = _c(q, np.int8)
    out = np.empty(q.shape, np.float32)
    _chk(_load().oracle_dequantize_per_tensor(_p(q), _p(out), _c_i64(q.size), _c_dbl(scale),
                                              _c_i64(zero_point)), "dequantize")
    return out


def epilogue(acc, channels: int, inner: int, input_scale: float, weight_scales, bias,
             output_scale: float, output_zero_point: int, return_pre: bool = False,
             activation: str = "none"):
    """#21197/#21205 Solution: v = acc*input_scale*weight_scales[c] + bias[c];
    q = clamp(round(v*inv_output_scale) + output_zero_point, -128, 127).
    Element e belongs to channel (e // inner) % channels.  activation="relu"
    (the pages' relu-fused follow-up) requantizes max(v, 0) instead of v;
    return_pre gives v before the rectifier."""
    acc = _c(acc, np.int32)
    ws = _c(weight_scales, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty(acc.shape, np.int8)
    pre = np.empty(acc.shape, np.float32) if return_pre else None
    _chk(_load().oracle_epilogue(_p(acc), _c_i64(acc.size), _c_i64(channels), _c_i64(inner),
                                 _c_dbl(input_scale), _p(ws), _p(b), _c_dbl(output_scale),
                                 _c_i64(output_zero_point), _c_i64(_relu_flag(activation)),
                                 _p(out), _p(pre)), "epilogue")
    return (out, pre) if return_pre else out


def linear_acc(x, w, input_zero_point: int, folded: bool = False) -> np.ndarray:
    """#21197 Solution: acc[m,n] = sum_k (x[m,k]-izp)*w[n,k] (int32).
    folded=True evaluates sum x*w - izp*sum w instead (#21197 Constraints (1))."""
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    M, K = x.shape
    N, ldw = w.shape
    acc = np.empty((M, N), np.int32)
    fn = _load().oracle_linear_acc_folded if folded else _load().oracle_linear_acc
    _chk(fn(_p(x), _c_i64(M), _c_i64(K), _c_i64(input_zero_point), _p(w), _c_i64(N),
            _c_i64(ldw), _p(acc)), "linear_acc")
    return acc


def weight_sums(w, K: int | None = None) -> np.ndarray:
    """sum_k w[n, k] over the first K columns (all by default), int32: the
    zero-point term's factor of #21197 Constraints (1) (sum(x-zp)w = sum xw -
    zp * sum w).  Formed in int64 and checked to fit int32."""
    w = _c(w, np.int8)
    K = w.shape[1] if K is None else K
    s = w[:, :K].astype(np.int64).sum(axis=1)
    if s.size and (s.max() > np.iinfo(np.int32).max or s.min() < np.iinfo(np.int32).min):
        raise OverflowError("weight_sums: a sum left the int32 range")
    return s.astype(np.int32)


def linear(x, w, weight_scales, bias, input_scale: float, input_zero_point: int,
           output_scale: float, output_zero_point: int, return_acc: bool = False,
           activation: str = "none"):
    """q8ta_linear (#21197 Solution): contraction then per-channel epilogue.
    x int8 [M,K] row-major, w int8 [N,ldw] row-major (only [:, :K] is read)."""
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    M, K = x.shape
    N, ldw = w.shape
    ws = _c(weight_scales, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((M, N), np.int8)
    acc = np.empty((M, N), np.int32) if return_acc else None
    _chk(_load().oracle_linear(_p(x), _c_i64(M), _c_i64(K), _c_dbl(input_scale),
                               _c_i64(input_zero_point), _p(w), _c_i64(N), _c_i64(ldw),
                               _p(ws), _p(b), _c_dbl(output_scale), _c_i64(output_zero_point),
                               _c_i64(_relu_flag(activation)), _p(out), _p(acc)), "linear")
    return (out, acc) if return_acc else out


def _deconv_args(x, w, Kh, Kw, stride, padding, dilation):
    x = _c(x, np.int8)
    w = _c(w, np.int8)
    N, IC, H_in, W_in = x.shape
    OC, ldw = w.shape
    sh, sw = stride
    ph, pw = padding
    dh, dw = dilation
    return x, w, (N, IC, H_in, W_in, OC, ldw, sh, sw, ph, pw, dh, dw)


def deconv_acc(x, w, input_zero_point: int, Kh: int, Kw: int, stride, padding, dilation,
               H_out: int, W_out: int, method: str = "gather", groups: int = 1) -> np.ndarray:
    """#21205 Solution gather (method="gather"); the scatter and zero-point-fill
    formulations ("scatter", "zpfill") exist only to check it.  With groups,
    output channel oc sums over the input channels of its group only,
    w[oc, (kh*Kw+kw)*(IC/groups) + icg]."""
    x, w, (N, IC, H_in, W_in, OC, ldw, sh, sw, ph, pw, dh, dw) = _deconv_args(
        x, w, Kh, Kw, stride, padding, dilation)
    acc = np.empty((N, OC, H_out, W_out), np.int32)
    fn = {"gather": _load().oracle_deconv_acc_gather,
          "scatter": _load().oracle_deconv_acc_scatter,
          "zpfill": _load().oracle_deconv_acc_zpfill}[method]
    _chk(fn(_p(x), _c_i64(N), _c_i64(IC), _c_i64(H_in), _c_i64(W_in), _c_i64(input_zero_point),
            _p(w), _c_i64(OC), _c_i64(Kh), _c_i64(Kw), _c_i64(ldw), _c_i64(sh), _c_i64(sw),
            _c_i64(ph), _c_i64(pw), _c_i64(dh), _c_i64(dw), _c_i64(groups), _c_i64(H_out),
            _c_i64(W_out), _p(acc)), "deconv_acc")
    return acc


def conv2d_transposed(x, w, weight_scales, bias, input_scale: float, input_zero_point: int,
                      output_scale: float, output_zero_point: int, Kh: int, Kw: int,
                      stride, padding, dilation, H_out: int, W_out: int,
                      return_acc: bool = False, groups: int = 1, activation: str = "none"):
    """q8ta_conv2d_transposed (#21205 Solution): gather contraction then the
    per-channel epilogue with channel = oc.  x int8 NCHW, w int8 [OC, ldw] with
    w[oc, (kh*Kw+kw)*IC + ic] (IC/groups per row when grouped); output int8 NCHW
    [N, OC, H_out, W_out]."""
    x, w, (N, IC, H_in, W_in, OC, ldw, sh, sw, ph, pw, dh, dw) = _deconv_args(
        x, w, Kh, Kw, stride, padding, dilation)
    ws = _c(weight_scales, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((N, OC, H_out, W_out), np.int8)
    acc = np.empty((N, OC, H_out, W_out), np.int32) if return_acc else None
    _chk(_load().oracle_conv2d_transposed(
        _p(x), _c_i64(N), _c_i64(IC), _c_i64(H_in), _c_i64(W_in), _c_dbl(input_scale),
        _c_i64(input_zero_point), _p(w), _c_i64(OC), _c_i64(Kh), _c_i64(Kw), _c_i64(ldw),
        _p(ws), _p(b), _c_dbl(output_scale), _c_i64(output_zero_point), _c_i64(sh),
        _c_i64(sw), _c_i64(ph), _c_i64(pw), _c_i64(dh), _c_i64(dw), _c_i64(groups),
        _c_i64(H_out), _c_i64(W_out), _c_i64(_relu_flag(activation)), _p(out), _p(acc)),
        "conv2d_transposed")
    return (out, acc) if return_acc else out


def conv2d_acc(x, w, input_zero_point: int, Kh: int, Kw: int, stride, padding, dilation,
               H_out: int, W_out: int, groups: int = 1) -> np.ndarray:
    """Forward q8ta_conv2d contraction (the general conv whose scaffold #21205
    Solution says the transposed op reuses): ih = oh*stride - pad + kh*dil,
    taken only inside the input; with groups, output channel oc sums over the
    input channels of its group only, w[oc, (kh*Kw+kw)*(IC/groups) + icg]."""
    x, w, (N, IC, H_in, W_in, OC, ldw, sh, sw, ph, pw, dh, dw) = _deconv_args(
        x, w, Kh, Kw, stride, padding, dilation)
    acc = np.empty((N, OC, H_out, W_out), np.int32)
    _chk(_load().oracle_conv2d_acc(
        _p(x), _c_i64(N), _c_i64(IC), _c_i64(H_in), _c_i64(W_in), _c_i64(input_zero_point),
        _p(w), _c_i64(OC), _c_i64(Kh), _c_i64(Kw), _c_i64(ldw), _c_i64(sh), _c_i64(sw),
        _c_i64(ph), _c_i64(pw), _c_i64(dh), _c_i64(dw), _c_i64(groups), _c_i64(H_out),
        _c_i64(W_out), _p(acc)), "conv2d_acc")
    return acc


def conv2d(x, w, weight_scales, bias, input_scale: float, input_zero_point: int,
           output_scale: float, output_zero_point: int, Kh: int, Kw: int, stride, padding,
           dilation, H_out: int, W_out: int, return_acc: bool = False, groups: int = 1,
           activation: str = "none"):
    """Forward q8ta_conv2d: contraction then the per-channel epilogue with
    channel = oc.  x int8 NCHW, w int8 [OC, ldw] with w[oc, (kh*Kw+kw)*IC + ic];
    output int8 NCHW [N, OC, H_out, W_out]."""
    x, w, (N, IC, H_in, W_in, OC, ldw, sh, sw, ph, pw, dh, dw) = _deconv_args(
        x, w, Kh, Kw, stride, padding, dilation)
    ws = _c(weight_scales, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((N, OC, H_out, W_out), np.int8)
    acc = np.empty((N, OC, H_out, W_out), np.int32) if return_acc else None
    _chk(_load().oracle_conv2d(
        _p(x), _c_i64(N), _c_i64(IC), _c_i64(H_in), _c_i64(W_in), _c_dbl(input_scale),
        _c_i64(input_zero_point), _p(w), _c_i64(OC), _c_i64(Kh), _c_i64(Kw), _c_i64(ldw),
        _p(ws), _p(b), _c_dbl(output_scale), _c_i64(output_zero_point), _c_i64(sh),
        _c_i64(sw), _c_i64(ph), _c_i64(pw), _c_i64(dh), _c_i64(dw), _c_i64(groups),
        _c_i64(H_out), _c_i64(W_out), _c_i64(_relu_flag(activation)), _p(out), _p(acc)),
        "conv2d")
    return (out, acc) if return_acc else out
