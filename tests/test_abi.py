"""C-ABI tests that need no GPU: the library loads, exports every entry point
the header declares, and rejects every invalid argument before any HIP call.

No call here passes a complete set of valid arguments with fake pointers
(that would launch a kernel on fake addresses on a GPU machine); the one test
that launches is skipped wherever a GPU is present.
"""
import ctypes
import os
import re
import subprocess

import pytest

import int8_quantized_amd as q8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q8ta.h")

FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q8ta_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ["q8ta_quantize_per_tensor", "q8ta_dequantize_per_tensor", "q8ta_linear",
              "q8ta_linear_gemv", "q8ta_conv2d_transposed", "q8ta_conv2d", "q8ta_conv2d_acc",
              "q8ta_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = q8.lib()
    for n in _declared():
        assert hasattr(lib, n), n
        assert n in q8.SIGNATURES, n


def test_exported_dynamic_symbols_with_nm():
    out = subprocess.run(["nm", "-D", "--defined-only", q8.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    syms = set(re.findall(r"\bT (q8ta_\w+)", out))
    assert set(_declared()) <= syms


def test_last_error_is_never_null():
    assert isinstance(q8.q8ta_last_error(), str)


def _st(rc, status, needle=None):
    assert rc == status, (rc, q8.q8ta_last_error())
    if needle:
        assert needle in q8.q8ta_last_error()


# ---------------------------------------------------------------- quantize / dequantize
@pytest.mark.parametrize("fn", ["q8ta_quantize_per_tensor", "q8ta_dequantize_per_tensor"])
def test_quant_errors(fn):
    f = getattr(q8.lib(), fn)
    _st(f(None, FAKE, 16, 0.02, 3, None), q8.Q8TA_ERR_NULL)
    _st(f(FAKE, None, 16, 0.02, 3, None), q8.Q8TA_ERR_NULL)
    _st(f(FAKE, FAKE, -1, 0.02, 3, None), q8.Q8TA_ERR_SHAPE)
    _st(f(FAKE, FAKE, 16, 0.0, 3, None), q8.Q8TA_ERR_QPARAM)
    _st(f(FAKE, FAKE, 16, -1.0, 3, None), q8.Q8TA_ERR_QPARAM)
    _st(f(FAKE, FAKE, 16, float("nan"), 3, None), q8.Q8TA_ERR_QPARAM)
    _st(f(FAKE, FAKE, 16, float("inf"), 3, None), q8.Q8TA_ERR_QPARAM)
    _st(f(FAKE, FAKE, 16, 0.02, 128, None), q8.Q8TA_ERR_QPARAM)
    _st(f(FAKE, FAKE, 16, 0.02, -129, None), q8.Q8TA_ERR_QPARAM)


@pytest.mark.parametrize("fn", ["q8ta_quantize_per_tensor", "q8ta_dequantize_per_tensor"])
def test_quant_empty_is_noop_without_launch(fn):
    f = getattr(q8.lib(), fn)
    assert f(None, None, 0, 0.02, 3, None) == q8.Q8TA_OK


# ---------------------------------------------------------------- linear
def _lin(fn="q8ta_linear", x=FAKE, M=4, K=64, s_in=0.02, izp=3, w=FAKE, N=32, ws=None,
         scales=FAKE, bias=FAKE, s_out=0.27, ozp=-5, act=b"none", out=FAKE):
    return getattr(q8.lib(), fn)(x, M, K, s_in, izp, w, N, ws, scales, bias, s_out, ozp, act, out,
                                 None)


@pytest.mark.parametrize("fn", ["q8ta_linear", "q8ta_linear_gemv"])
def test_linear_errors(fn):
    M = 1
    _st(_lin(fn, x=None, M=M), q8.Q8TA_ERR_NULL)
    _st(_lin(fn, w=None, M=M), q8.Q8TA_ERR_NULL)
    _st(_lin(fn, out=None, M=M), q8.Q8TA_ERR_NULL)
    _st(_lin(fn, scales=None, M=M), q8.Q8TA_ERR_NULL)
    _st(_lin(fn, M=0), q8.Q8TA_ERR_SHAPE)
    _st(_lin(fn, M=M, K=0), q8.Q8TA_ERR_SHAPE)
    _st(_lin(fn, M=M, N=-3), q8.Q8TA_ERR_SHAPE)
    _st(_lin(fn, M=M, s_in=0.0), q8.Q8TA_ERR_QPARAM)
    _st(_lin(fn, M=M, s_out=float("inf")), q8.Q8TA_ERR_QPARAM)
    _st(_lin(fn, M=M, izp=200), q8.Q8TA_ERR_QPARAM)
    _st(_lin(fn, M=M, ozp=-129), q8.Q8TA_ERR_QPARAM)
    _st(_lin(fn, M=M, act=b"gelu"), q8.Q8TA_ERR_UNSUPPORTED, "gelu")
    _st(_lin(fn, M=M, act=b"RELU"), q8.Q8TA_ERR_UNSUPPORTED)
    _st(_lin(fn, M=M, act=None), q8.Q8TA_ERR_UNSUPPORTED)
    _st(_lin(fn, M=M, act=b"None"), q8.Q8TA_ERR_UNSUPPORTED)


def test_linear_gemv_requires_single_row():
    _st(_lin("q8ta_linear_gemv", M=4), q8.Q8TA_ERR_SHAPE, "M must be 1")


def test_linear_acc_errors():
    f = q8.lib().q8ta_linear_acc
    _st(f(None, 4, 64, 3, FAKE, 32, FAKE, None), q8.Q8TA_ERR_NULL)
    _st(f(FAKE, 4, 64, 3, FAKE, 32, None, None), q8.Q8TA_ERR_NULL)
    _st(f(FAKE, 4, 0, 3, FAKE, 32, FAKE, None), q8.Q8TA_ERR_SHAPE)
    _st(f(FAKE, 4, 64, 300, FAKE, 32, FAKE, None), q8.Q8TA_ERR_QPARAM)


# ---------------------------------------------------------------- conv2d_transposed
DC = dict(x=FAKE, N=1, IC=64, H_in=32, W_in=32, s_in=0.02, izp=3, w=FAKE, OC=32, Kh=4, Kw=4,
          ldw=1024, ws=None, scales=FAKE, bias=FAKE, s_out=0.54, ozp=-5, sh=2, sw=2, ph=1, pw=1,
          oph=0, opw=0, dh=1, dw=1, groups=1, act=b"none", out=FAKE, H_out=64, W_out=64)


def _dc(**kw):
    a = dict(DC)
    a.update(kw)
    return q8.lib().q8ta_conv2d_transposed(
        a["x"], a["N"], a["IC"], a["H_in"], a["W_in"], a["s_in"], a["izp"], a["w"], a["OC"],
        a["Kh"], a["Kw"], a["ldw"], a["ws"], a["scales"], a["bias"], a["s_out"], a["ozp"],
        a["sh"], a["sw"], a["ph"], a["pw"], a["oph"], a["opw"], a["dh"], a["dw"], a["groups"],
        a["act"], a["out"], a["H_out"], a["W_out"], None)


def test_deconv_errors():
    _st(_dc(x=None), q8.Q8TA_ERR_NULL)
    _st(_dc(w=None), q8.Q8TA_ERR_NULL)
    _st(_dc(out=None), q8.Q8TA_ERR_NULL)
    _st(_dc(scales=None), q8.Q8TA_ERR_NULL)
    for k in ["N", "IC", "H_in", "W_in", "OC", "Kh", "Kw", "H_out", "W_out"]:
        _st(_dc(**{k: 0}), q8.Q8TA_ERR_SHAPE)
    _st(_dc(ldw=1023), q8.Q8TA_ERR_SHAPE, "weight_row_stride")
    _st(_dc(sh=0), q8.Q8TA_ERR_SHAPE)
    _st(_dc(sw=-1), q8.Q8TA_ERR_SHAPE)
    _st(_dc(ph=-1), q8.Q8TA_ERR_SHAPE)
    _st(_dc(dw=0), q8.Q8TA_ERR_SHAPE, "dilation")
    _st(_dc(dh=5000), q8.Q8TA_ERR_SHAPE, "dilation")
    _st(_dc(groups=0), q8.Q8TA_ERR_SHAPE, "groups")
    _st(_dc(groups=3), q8.Q8TA_ERR_SHAPE, "groups")          # does not divide IC = 64
    _st(_dc(groups=64), q8.Q8TA_ERR_SHAPE, "groups")         # does not divide OC = 32
    _st(_dc(groups=2, ldw=511), q8.Q8TA_ERR_SHAPE, "weight_row_stride")
    _st(_dc(act=b"sigmoid"), q8.Q8TA_ERR_UNSUPPORTED)
    _st(_dc(act=None), q8.Q8TA_ERR_UNSUPPORTED)
    _st(_dc(izp=128), q8.Q8TA_ERR_QPARAM)
    _st(_dc(s_out=-0.5), q8.Q8TA_ERR_QPARAM)
    _st(_dc(s_in=float("nan")), q8.Q8TA_ERR_QPARAM)


def test_deconv_acc_errors():
    f = q8.lib().q8ta_conv2d_transposed_acc
    args = [FAKE, 1, 64, 32, 32, 3, FAKE, 32, 4, 4, 1024, 2, 2, 1, 1, 1, 1, 1, FAKE, 64, 64, None]
    a = list(args); a[0] = None
    _st(f(*a), q8.Q8TA_ERR_NULL)
    a = list(args); a[18] = None
    _st(f(*a), q8.Q8TA_ERR_NULL)
    a = list(args); a[10] = 100
    _st(f(*a), q8.Q8TA_ERR_SHAPE)
    a = list(args); a[15] = 0
    _st(f(*a), q8.Q8TA_ERR_SHAPE, "dilation")
    a = list(args); a[17] = 3
    _st(f(*a), q8.Q8TA_ERR_SHAPE, "groups")
    a = list(args); a[5] = -200
    _st(f(*a), q8.Q8TA_ERR_QPARAM)


# ---------------------------------------------------------------- forward conv2d
CV = dict(x=FAKE, N=1, IC=64, H_in=32, W_in=32, s_in=0.02, izp=3, w=FAKE, OC=32, Kh=3, Kw=3,
          ldw=576, ws=None, scales=FAKE, bias=FAKE, s_out=0.54, ozp=-5, sh=1, sw=1, ph=1, pw=1,
          dh=1, dw=1, groups=1, act=b"none", out=FAKE, H_out=32, W_out=32)


def _cv(**kw):
    a = dict(CV)
    a.update(kw)
    return q8.lib().q8ta_conv2d(
        a["x"], a["N"], a["IC"], a["H_in"], a["W_in"], a["s_in"], a["izp"], a["w"], a["OC"],
        a["Kh"], a["Kw"], a["ldw"], a["ws"], a["scales"], a["bias"], a["s_out"], a["ozp"],
        a["sh"], a["sw"], a["ph"], a["pw"], a["dh"], a["dw"], a["groups"], a["act"], a["out"],
        a["H_out"], a["W_out"], None)


def test_conv2d_errors():
    _st(_cv(x=None), q8.Q8TA_ERR_NULL)
    _st(_cv(w=None), q8.Q8TA_ERR_NULL)
    _st(_cv(out=None), q8.Q8TA_ERR_NULL)
    _st(_cv(scales=None), q8.Q8TA_ERR_NULL)
    for k in ["N", "IC", "H_in", "W_in", "OC", "Kh", "Kw", "H_out", "W_out"]:
        _st(_cv(**{k: 0}), q8.Q8TA_ERR_SHAPE)
    _st(_cv(ldw=575), q8.Q8TA_ERR_SHAPE, "weight_row_stride")
    _st(_cv(sh=0), q8.Q8TA_ERR_SHAPE)
    _st(_cv(ph=-1), q8.Q8TA_ERR_SHAPE)
    _st(_cv(dh=0), q8.Q8TA_ERR_SHAPE, "dilation")
    _st(_cv(dw=5000), q8.Q8TA_ERR_SHAPE, "dilation")
    _st(_cv(groups=0), q8.Q8TA_ERR_SHAPE, "groups")
    _st(_cv(groups=3), q8.Q8TA_ERR_SHAPE, "groups")          # does not divide IC = 64
    _st(_cv(groups=64), q8.Q8TA_ERR_SHAPE, "groups")         # does not divide OC = 32
    _st(_cv(groups=2, ldw=287), q8.Q8TA_ERR_SHAPE, "weight_row_stride")
    _st(_cv(act=b"tanh"), q8.Q8TA_ERR_UNSUPPORTED)
    _st(_cv(izp=-129), q8.Q8TA_ERR_QPARAM)
    _st(_cv(s_out=0.0), q8.Q8TA_ERR_QPARAM)


def test_conv2d_acc_errors():
    f = q8.lib().q8ta_conv2d_acc
    args = [FAKE, 1, 64, 32, 32, 3, FAKE, 32, 3, 3, 576, 1, 1, 1, 1, 1, 1, 1, FAKE, 32, 32, None]
    a = list(args); a[18] = None
    _st(f(*a), q8.Q8TA_ERR_NULL)
    a = list(args); a[17] = 5
    _st(f(*a), q8.Q8TA_ERR_SHAPE)
    a = list(args); a[15] = 0
    _st(f(*a), q8.Q8TA_ERR_SHAPE)
    a = list(args); a[5] = 200
    _st(f(*a), q8.Q8TA_ERR_QPARAM)


def test_fused_entry_points_errors():
    l = q8.lib()
    # q8ta_linear_dq: same checks as q8ta_linear
    _st(l.q8ta_linear_dq(FAKE, 4, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", None,
                         None), q8.Q8TA_ERR_NULL)
    _st(l.q8ta_linear_dq(FAKE, 0, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", FAKE,
                         None), q8.Q8TA_ERR_SHAPE)
    _st(l.q8ta_linear_dq(FAKE, 4, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"relu6", FAKE,
                         None), q8.Q8TA_ERR_UNSUPPORTED)
    # q8ta_quantize_linear(_dq): same checks as q8ta_linear, x fp32
    for fn in (l.q8ta_quantize_linear, l.q8ta_quantize_linear_dq):
        _st(fn(None, 4, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_NULL)
        _st(fn(FAKE, 4, 64, 0.02, 3, FAKE, 32, None, None, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_NULL)
        _st(fn(FAKE, 4, 0, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_SHAPE)
        _st(fn(FAKE, 4, 64, 0.0, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_QPARAM)
        _st(fn(FAKE, 4, 64, 0.02, 300, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_QPARAM)
        _st(fn(FAKE, 4, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"gelu", FAKE, None),
            q8.Q8TA_ERR_UNSUPPORTED)
    # q8ta_quantize_conv2d_transposed: same checks as q8ta_conv2d_transposed
    args = [FAKE, 1, 64, 32, 32, 0.02, 3, FAKE, 32, 4, 4, 1024, None, FAKE, FAKE, 0.54, -5, 2, 2,
            1, 1, 0, 0, 1, 1, 1, b"none", FAKE, 64, 64, None]
    a = list(args); a[0] = None
    _st(l.q8ta_quantize_conv2d_transposed(*a), q8.Q8TA_ERR_NULL)
    a = list(args); a[23] = 0
    _st(l.q8ta_quantize_conv2d_transposed(*a), q8.Q8TA_ERR_SHAPE, "dilation")
    a = list(args); a[25] = 5
    _st(l.q8ta_quantize_conv2d_transposed(*a), q8.Q8TA_ERR_SHAPE, "groups")
    a = list(args); a[5] = -1.0
    _st(l.q8ta_quantize_conv2d_transposed(*a), q8.Q8TA_ERR_QPARAM)


def test_presummed_entry_points_errors():
    l = q8.lib()
    _st(l.q8ta_weight_sums(None, 32, 64, FAKE, None), q8.Q8TA_ERR_NULL)
    _st(l.q8ta_weight_sums(FAKE, 32, 64, None, None), q8.Q8TA_ERR_NULL)
    _st(l.q8ta_weight_sums(FAKE, 0, 64, FAKE, None), q8.Q8TA_ERR_SHAPE)
    _st(l.q8ta_weight_sums(FAKE, 32, 0, FAKE, None), q8.Q8TA_ERR_SHAPE)
    for fn in (l.q8ta_linear_presummed, l.q8ta_linear_dq_presummed):
        # weight_sums is required
        _st(fn(FAKE, 4, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_NULL, "weight_sums")
        # the rest as for q8ta_linear
        _st(fn(FAKE, 0, 64, 0.02, 3, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_SHAPE)
        _st(fn(FAKE, 4, 64, 0.02, 3, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"gelu", FAKE, None),
            q8.Q8TA_ERR_UNSUPPORTED)
        _st(fn(FAKE, 4, 64, 0.02, 300, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_QPARAM)


def test_prepacked_size_formula():
    """ceil(N/32)*32 rows of ceil(K/64)*64 bytes; -1 for invalid sizes."""
    l = q8.lib()
    for N, K in [(1, 1), (32, 64), (33, 64), (11008, 4096), (100, 1040), (7, 48)]:
        assert l.q8ta_weight_prepacked_bytes(N, K) == -(-N // 32) * 32 * (-(-K // 64) * 64)
    assert l.q8ta_weight_prepacked_bytes(0, 64) == -1
    assert l.q8ta_weight_prepacked_bytes(32, 0) == -1
    assert l.q8ta_weight_prepacked_bytes(32, 1 << 31) == -1


def test_prepacked_entry_points_errors():
    l = q8.lib()
    odd = ctypes.c_void_p(4096 + 8)   # not 16-byte aligned
    _st(l.q8ta_weight_prepack(None, 32, 64, FAKE, None), q8.Q8TA_ERR_NULL)
    _st(l.q8ta_weight_prepack(FAKE, 32, 64, None, None), q8.Q8TA_ERR_NULL)
    _st(l.q8ta_weight_prepack(FAKE, 0, 64, FAKE, None), q8.Q8TA_ERR_SHAPE)
    _st(l.q8ta_weight_prepack(FAKE, 32, 40, FAKE, None), q8.Q8TA_ERR_UNSUPPORTED, "K % 16")
    _st(l.q8ta_weight_prepack(odd, 32, 64, FAKE, None), q8.Q8TA_ERR_UNSUPPORTED)
    _st(l.q8ta_weight_prepack(FAKE, 32, 64, odd, None), q8.Q8TA_ERR_UNSUPPORTED)
    for fn in (l.q8ta_linear_prepacked, l.q8ta_linear_dq_prepacked):
        _st(fn(FAKE, 4, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_NULL, "weight_sums")
        _st(fn(FAKE, 4, 40, 0.02, 3, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_UNSUPPORTED, "K % 16")
        _st(fn(odd, 4, 64, 0.02, 3, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_UNSUPPORTED)
        _st(fn(FAKE, 4, 64, 0.02, 3, odd, 32, FAKE, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_UNSUPPORTED)
        _st(fn(FAKE, 0, 64, 0.02, 3, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_SHAPE)
        _st(fn(FAKE, 4, 64, 0.02, 3, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"gelu", FAKE, None),
            q8.Q8TA_ERR_UNSUPPORTED)
        _st(fn(FAKE, 4, 64, 0.02, 300, FAKE, 32, FAKE, FAKE, None, 0.5, -5, b"none", FAKE, None),
            q8.Q8TA_ERR_QPARAM)


def test_deconv_prepacked_size_formula():
    """ceil(OC/32)*32 rows of Kh*Kw*IC bytes; -1 for IC % 64 != 0 or sizes < 1."""
    l = q8.lib()
    for OC, IC, K in [(32, 64, 3), (33, 64, 4), (128, 256, 3), (1, 128, 3), (160, 192, 4)]:
        assert l.q8ta_conv2d_transposed_weight_prepacked_bytes(OC, IC, K, K) == \
            -(-OC // 32) * 32 * K * K * IC
    assert l.q8ta_conv2d_transposed_weight_prepacked_bytes(32, 48, 3, 3) == -1
    assert l.q8ta_conv2d_transposed_weight_prepacked_bytes(0, 64, 3, 3) == -1
    assert l.q8ta_conv2d_transposed_weight_prepacked_bytes(32, 64, 0, 3) == -1


def test_deconv_prepacked_entry_points_errors():
    l = q8.lib()
    odd = ctypes.c_void_p(4096 + 8)   # not 16-byte aligned
    pk = l.q8ta_conv2d_transposed_weight_prepack
    _st(pk(None, 32, 64, 3, 3, 576, FAKE, None), q8.Q8TA_ERR_NULL)
    _st(pk(FAKE, 32, 64, 3, 3, 576, None, None), q8.Q8TA_ERR_NULL)
    _st(pk(FAKE, 0, 64, 3, 3, 576, FAKE, None), q8.Q8TA_ERR_SHAPE)
    _st(pk(FAKE, 32, 48, 3, 3, 432, FAKE, None), q8.Q8TA_ERR_UNSUPPORTED, "IC % 64")
    _st(pk(FAKE, 32, 64, 3, 3, 500, FAKE, None), q8.Q8TA_ERR_SHAPE, "weight_row_stride")
    _st(pk(FAKE, 32, 64, 3, 3, 584, FAKE, None), q8.Q8TA_ERR_UNSUPPORTED)
    _st(pk(odd, 32, 64, 3, 3, 576, FAKE, None), q8.Q8TA_ERR_UNSUPPORTED)
    _st(pk(FAKE, 32, 64, 3, 3, 576, odd, None), q8.Q8TA_ERR_UNSUPPORTED)

    def call(**kw):
        d = dict(x=FAKE, N=1, IC=64, H_in=32, W_in=32, s_in=0.02, izp=3, w=FAKE, OC=32, Kh=3,
                 Kw=3, ws=None, scales=FAKE, bias=FAKE, s_out=0.54, ozp=-5, sh=2, sw=2, ph=1,
                 pw=1, oph=1, opw=1, dh=1, dw=1, groups=1, act=b"none", out=FAKE, H_out=64,
                 W_out=64)
        d.update(kw)
        return l.q8ta_conv2d_transposed_prepacked(*d.values(), None)

    _st(call(x=None), q8.Q8TA_ERR_NULL)
    _st(call(w=None), q8.Q8TA_ERR_NULL)
    _st(call(out=None), q8.Q8TA_ERR_NULL)
    _st(call(scales=None), q8.Q8TA_ERR_NULL)
    _st(call(N=0), q8.Q8TA_ERR_SHAPE)
    _st(call(izp=300), q8.Q8TA_ERR_QPARAM)
    _st(call(act=b"gelu"), q8.Q8TA_ERR_UNSUPPORTED)
    # shapes outside the compile-time-pattern kernel
    for kw in (dict(Kh=5, Kw=5), dict(Kh=3, Kw=4), dict(sh=1, sw=1), dict(IC=48), dict(W_in=30),
               dict(ph=1, pw=0), dict(groups=2), dict(dh=2, dw=2), dict(w=odd),
               dict(x=ctypes.c_void_p(4096 + 2))):
        _st(call(**kw), q8.Q8TA_ERR_UNSUPPORTED, "use q8ta_conv2d_transposed")
    qf = l.q8ta_quantize_conv2d_transposed_prepacked
    _st(qf(None, 1, 64, 32, 32, 0.02, 3, FAKE, 32, 3, 3, None, FAKE, FAKE, 0.54, -5, 2, 2, 1, 1, 1,
           1, 1, 1, 1, b"none", FAKE, 64, 64, None), q8.Q8TA_ERR_NULL)
    _st(qf(ctypes.c_void_p(4096 + 4), 1, 64, 32, 32, 0.02, 3, FAKE, 32, 3, 3, None, FAKE, FAKE,
           0.54, -5, 2, 2, 1, 1, 1, 1, 1, 1, 1, b"none", FAKE, 64, 64, None),
        q8.Q8TA_ERR_UNSUPPORTED, "use q8ta_quantize_conv2d_transposed")
    _st(qf(FAKE, 1, 64, 32, 32, 0.02, 3, FAKE, 32, 5, 5, None, FAKE, FAKE, 0.54, -5, 2, 2, 1, 1, 1,
           1, 1, 1, 1, b"none", FAKE, 64, 64, None), q8.Q8TA_ERR_UNSUPPORTED)


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_gpu_present(), reason="launches on fake pointers; only meaningful without a GPU")
def test_valid_call_without_gpu_reports_hip_error():
    rc = q8.lib().q8ta_quantize_per_tensor(FAKE, FAKE, 16, 0.02, 3, None)
    assert rc == q8.Q8TA_ERR_HIP, q8.q8ta_last_error()
    assert "HIP error" in q8.q8ta_last_error()


@pytest.mark.skipif(_gpu_present(), reason="launches on fake pointers; only meaningful without a GPU")
def test_relu_dilation_and_groups_pass_validation():
    """relu on every op, dilation and groups on the transposed conv are
    accepted: without a GPU such calls get as far as the HIP runtime."""
    for fn in ("q8ta_linear", "q8ta_linear_gemv"):
        _st(_lin(fn, M=1, act=b"relu"), q8.Q8TA_ERR_HIP, "HIP error")
    _st(_dc(act=b"relu"), q8.Q8TA_ERR_HIP, "HIP error")
    _st(_dc(dh=2, dw=3), q8.Q8TA_ERR_HIP, "HIP error")
    _st(_dc(groups=2, ldw=512), q8.Q8TA_ERR_HIP, "HIP error")
    _st(_dc(groups=32, ldw=32), q8.Q8TA_ERR_HIP, "HIP error")
    _st(_cv(act=b"relu"), q8.Q8TA_ERR_HIP, "HIP error")
    _st(q8.lib().q8ta_weight_sums(FAKE, 32, 64, FAKE, None), q8.Q8TA_ERR_HIP, "HIP error")
    _st(q8.lib().q8ta_linear_presummed(FAKE, 4, 64, 0.02, 3, FAKE, 32, FAKE, FAKE, None, 0.5, -5,
                                       b"none", FAKE, None), q8.Q8TA_ERR_HIP, "HIP error")


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(16, dtype=torch.float32)
    out = torch.zeros(16, dtype=torch.int8)
    with pytest.raises(ValueError, match="device tensor"):
        q8.q8ta_quantize_per_tensor(x, out, 0.02, 3)


def test_quantize_linear_binding_checks_shapes_before_the_call():
    """The fused quantize -> linear bindings reject mismatched shapes and host
    tensors before anything reaches the library."""
    import torch
    x = torch.zeros((4, 64), dtype=torch.float32)
    w = torch.zeros((32, 64), dtype=torch.int8)
    s = torch.ones(32, dtype=torch.float32)
    for fn, dt in ((q8.q8ta_quantize_linear, torch.int8),
                   (q8.q8ta_quantize_linear_dq, torch.float32)):
        with pytest.raises(ValueError, match="shape mismatch"):
            fn(x, 0.02, 3, w, None, s, None, 0.5, -5, "none", torch.zeros((4, 31), dtype=dt))
        with pytest.raises(ValueError, match="2-D"):
            fn(x.view(-1), 0.02, 3, w, None, s, None, 0.5, -5, "none",
               torch.zeros((4, 32), dtype=dt))
        with pytest.raises(ValueError, match="device tensor"):
            fn(x, 0.02, 3, w, None, s, None, 0.5, -5, "none", torch.zeros((4, 32), dtype=dt))


def test_select_kernel_names():
    """q8ta_select_kernel accepts the documented op and kernel names, rejects
    others (leaving the choice unchanged) and makes no HIP call."""
    lib = q8.lib()
    for op, kernels in (("linear", ("mfma32", "mfma32_8w", "generic")),
                        ("conv2d_transposed", ("fixed", "mfma32", "mfma", "igemm", "tiled",
                                               "generic")),
                        ("conv2d", ("fixed", "mfma32", "mfma", "igemm", "generic"))):
        for k in kernels + ("default",):
            _st(lib.q8ta_select_kernel(op.encode(), k.encode()), q8.Q8TA_OK)
        _st(lib.q8ta_select_kernel(op.encode(), b"dot4"), q8.Q8TA_ERR_UNSUPPORTED, "unknown kernel")
    _st(lib.q8ta_select_kernel(b"gemm", b"default"), q8.Q8TA_ERR_UNSUPPORTED, "unknown op")
    _st(lib.q8ta_select_kernel(None, b"default"), q8.Q8TA_ERR_NULL)
    _st(lib.q8ta_select_kernel(b"linear", None), q8.Q8TA_ERR_NULL)
    q8.q8ta_select_kernel("linear", "default")
    with pytest.raises(q8.Q8taError, match="unknown kernel"):
        q8.q8ta_select_kernel("conv2d", "tiled")


def test_noalloc_rejects_staging_beyond_the_static_scratch():
    """q8ta_quantize_linear_noalloc refuses, before any HIP call, a shape whose
    staged activations (M * K bytes) exceed its 16 MiB static scratch."""
    lib = q8.lib()
    M, K = 4097, 4096
    rc = lib.q8ta_quantize_linear_noalloc(FAKE, M, K, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5,
                                          b"none", FAKE, None)
    _st(rc, q8.Q8TA_ERR_SHAPE, "static scratch")
    # the usual argument checks come first
    _st(lib.q8ta_quantize_linear_noalloc(None, 8, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5,
                                         b"none", FAKE, None), q8.Q8TA_ERR_NULL)
    _st(lib.q8ta_quantize_linear_noalloc(FAKE, 8, 64, 0.02, 3, FAKE, 32, None, FAKE, None, 0.5, -5,
                                         b"gelu", FAKE, None), q8.Q8TA_ERR_UNSUPPORTED)
