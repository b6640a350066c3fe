"""Seeded synthetic inputs for the q8ta operations.

This module only draws numbers: it holds none of the operations' arithmetic and
is the one piece shared by the CPU oracle's tests and the GPU library's tests
and benchmark.  Every array is produced on the host with numpy's PCG64
generator, so the oracle and the GPU see the same bytes.

Distributions (the workloads the int8 op family is measured on):
  x_fp32 ~ N(0, 1); int8 activations ~ U{-128..127}; int8 weights ~ U{-127..127};
  weight_scales ~ U[0.005, 0.02) (float32); bias ~ N(0, 0.1) (float32);
  input scale 0.02, input zero point 3, output zero point -5, and the output
  scale 1.7 * input_scale * sqrt(Kred) evaluated in double, Kred being the
  number of products summed per output in the interior of the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

IN_SCALE = 0.02
IN_ZP = 3
OUT_ZP = -5


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def out_scale_for(kred: float, in_scale: float = IN_SCALE) -> float:
    return 1.7 * in_scale * math.sqrt(kred)


def x_fp32(g, shape):
    return g.standard_normal(size=shape, dtype=np.float32)


def x_int8(g, shape):
    return g.integers(-128, 128, size=shape, dtype=np.int8)


def w_int8(g, shape):
    return g.integers(-127, 128, size=shape, dtype=np.int8)


def scales(g, n):
    return g.uniform(0.005, 0.02, size=n).astype(np.float32)


def bias(g, n):
    return g.normal(0.0, 0.1, size=n).astype(np.float32)


@dataclass
class LinearCase:
    x: np.ndarray            # int8 [M, K]
    w: np.ndarray            # int8 [N, ldw]
    weight_scales: np.ndarray
    bias: np.ndarray | None
    in_scale: float
    in_zp: int
    out_scale: float
    out_zp: int
    x_fp32: np.ndarray | None = None   # set when x came from a quantize step

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return self.w.shape[0]


def linear_case(seed: int, M: int, K: int, N: int, ldw: int | None = None,
                with_bias: bool = True, in_zp: int = IN_ZP, out_zp: int = OUT_ZP,
                in_scale: float = IN_SCALE) -> LinearCase:
    g = rng(seed)
    ldw = K if ldw is None else ldw
    x = x_int8(g, (M, K))
    w = w_int8(g, (N, ldw))
    ws = scales(g, N)
    b = bias(g, N) if with_bias else None
    return LinearCase(x, w, ws, b, in_scale, in_zp, out_scale_for(K, in_scale), out_zp)


@dataclass
class DeconvCase:
    x: np.ndarray            # int8 [N, IC, H_in, W_in]
    w: np.ndarray            # int8 [OC, ldw], ldw >= Kh*Kw*IC
    weight_scales: np.ndarray
    bias: np.ndarray | None
    in_scale: float
    in_zp: int
    out_scale: float
    out_zp: int
    Kh: int
    Kw: int
    stride: tuple
    padding: tuple
    output_padding: tuple
    dilation: tuple
    H_out: int
    W_out: int
    x_fp32: np.ndarray | None = None


def deconv_out_size(in_size, k, s, p, op, d=1):
    """Conventional transposed-conv output size (PyTorch's formula)."""
    return (in_size - 1) * s - 2 * p + d * (k - 1) + op + 1


def deconv_case(seed: int, N: int, IC: int, H_in: int, W_in: int, OC: int, Kh: int, Kw: int,
                stride=(2, 2), padding=(1, 1), output_padding=(0, 0), H_out=None, W_out=None,
                ldw=None, with_bias=True, in_zp=IN_ZP, out_zp=OUT_ZP,
                x_from_fp32: bool = False, in_scale: float = IN_SCALE, dilation=(1, 1),
                groups: int = 1) -> DeconvCase:
    """Transposed-conv inputs; the weight has Kh*Kw*IC/groups columns."""
    g = rng(seed)
    if H_out is None:
        H_out = deconv_out_size(H_in, Kh, stride[0], padding[0], output_padding[0], dilation[0])
    if W_out is None:
        W_out = deconv_out_size(W_in, Kw, stride[1], padding[1], output_padding[1], dilation[1])
    ldw = Kh * Kw * (IC // groups) if ldw is None else ldw
    xf = None
    if x_from_fp32:
        xf = x_fp32(g, (N, IC, H_in, W_in))
        x = np.zeros((N, IC, H_in, W_in), np.int8)   # filled by the caller's quantize
    else:
        x = x_int8(g, (N, IC, H_in, W_in))
    w = w_int8(g, (OC, ldw))
    ws = scales(g, OC)
    b = bias(g, OC) if with_bias else None
    kred = (IC // groups) * Kh * Kw / (stride[0] * stride[1])
    c = DeconvCase(x, w, ws, b, in_scale, in_zp, out_scale_for(kred, in_scale), out_zp,
                   Kh, Kw, tuple(stride), tuple(padding), tuple(output_padding), tuple(dilation),
                   H_out, W_out, xf)
    c.groups = groups
    return c


def conv_out_size(in_size, k, s, p, d=1):
    """Conventional convolution output size (PyTorch's formula)."""
    return (in_size + 2 * p - d * (k - 1) - 1) // s + 1


def conv_case(seed: int, N: int, IC: int, H_in: int, W_in: int, OC: int, Kh: int, Kw: int,
              stride=(1, 1), padding=(1, 1), dilation=(1, 1), H_out=None, W_out=None, ldw=None,
              with_bias=True, in_zp=IN_ZP, out_zp=OUT_ZP, x_from_fp32: bool = False,
              in_scale: float = IN_SCALE, groups: int = 1) -> DeconvCase:
    """Forward conv inputs, in the same container as the transposed conv's
    (output_padding unused, (0, 0)); the weight has Kh*Kw*IC/groups columns."""
    g = rng(seed)
    if H_out is None:
        H_out = conv_out_size(H_in, Kh, stride[0], padding[0], dilation[0])
    if W_out is None:
        W_out = conv_out_size(W_in, Kw, stride[1], padding[1], dilation[1])
    ldw = Kh * Kw * (IC // groups) if ldw is None else ldw
    xf = None
    if x_from_fp32:
        xf = x_fp32(g, (N, IC, H_in, W_in))
        x = np.zeros((N, IC, H_in, W_in), np.int8)   # filled by the caller's quantize
    else:
        x = x_int8(g, (N, IC, H_in, W_in))
    w = w_int8(g, (OC, ldw))
    ws = scales(g, OC)
    b = bias(g, OC) if with_bias else None
    kred = (IC // groups) * Kh * Kw
    c = DeconvCase(x, w, ws, b, in_scale, in_zp, out_scale_for(kred, in_scale), out_zp,
                   Kh, Kw, tuple(stride), tuple(padding), (0, 0), tuple(dilation),
                   H_out, W_out, xf)
    c.groups = groups
    return c


# --- the five named workloads -------------------------------------------------
@dataclass
class Workload:
    key: str
    description: str
    seed: int
    params: dict = field(default_factory=dict)


WORKLOADS = {
    "chain_small": Workload(
        "chain_small", "quantize_per_tensor [4,64] -> q8ta_linear M=4 K=64 N=32", 1001,
        dict(M=4, K=64, N=32)),
    "gemv": Workload(
        "gemv", "q8ta_linear gemv M=1 K=4096 N=4096", 1002, dict(M=1, K=4096, N=4096)),
    "gemm": Workload(
        "gemm", "q8ta_linear GEMM M=2048 K=4096 N=11008 -> dequantize_per_tensor", 1003,
        dict(M=2048, K=4096, N=11008)),
    "deconv_small": Workload(
        "deconv_small", "q8ta_conv2d_transposed [1,64,32,32] K4 s2 p1 -> [1,32,64,64]", 1004,
        dict(N=1, IC=64, H_in=32, W_in=32, OC=32, Kh=4, Kw=4, stride=(2, 2), padding=(1, 1),
             output_padding=(0, 0))),
    "deconv_large": Workload(
        "deconv_large",
        "quantize_per_tensor [8,256,64,64] -> q8ta_conv2d_transposed K3 s2 p1 op1 -> "
        "[8,128,128,128]", 1005,
        dict(N=8, IC=256, H_in=64, W_in=64, OC=128, Kh=3, Kw=3, stride=(2, 2),
             padding=(1, 1), output_padding=(1, 1))),
    # Not a workload of the pages (they measure none for the forward conv): the
    # same-size 3x3 conv on the large transposed conv's input, for the forward
    # op's measurement.
    "conv2d_large": Workload(
        "conv2d_large", "q8ta_conv2d [8,256,64,64] K3 s1 p1 -> [8,128,64,64]", 1006,
        dict(N=8, IC=256, H_in=64, W_in=64, OC=128, Kh=3, Kw=3, stride=(1, 1),
             padding=(1, 1), dilation=(1, 1))),
    # Likewise ours: the depthwise 3x3 conv on the same input.
    "depthwise_large": Workload(
        "depthwise_large", "q8ta_conv2d depthwise [8,256,64,64] K3 s1 p1 -> [8,256,64,64]", 1007,
        dict(N=8, IC=256, H_in=64, W_in=64, OC=256, Kh=3, Kw=3, stride=(1, 1),
             padding=(1, 1), dilation=(1, 1), groups=256)),
}


def make_chain_small():
    wl = WORKLOADS["chain_small"]
    g = rng(wl.seed)
    M, K, N = wl.params["M"], wl.params["K"], wl.params["N"]
    xf = x_fp32(g, (M, K))
    w = w_int8(g, (N, K))
    ws = scales(g, N)
    b = bias(g, N)
    c = LinearCase(np.zeros((M, K), np.int8), w, ws, b, IN_SCALE, IN_ZP,
                   out_scale_for(K), OUT_ZP, x_fp32=xf)
    return c


def make_gemv():
    wl = WORKLOADS["gemv"]
    return linear_case(wl.seed, **wl.params)


def make_gemm():
    wl = WORKLOADS["gemm"]
    return linear_case(wl.seed, **wl.params)


def make_deconv_small():
    wl = WORKLOADS["deconv_small"]
    return deconv_case(wl.seed, **wl.params)


def make_deconv_large():
    wl = WORKLOADS["deconv_large"]
    return deconv_case(wl.seed, x_from_fp32=True, **wl.params)


def make_conv2d_large():
    wl = WORKLOADS["conv2d_large"]
    return conv_case(wl.seed, **wl.params)


def make_depthwise_large():
    wl = WORKLOADS["depthwise_large"]
    return conv_case(wl.seed, **wl.params)
