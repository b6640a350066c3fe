"""Pins for the CPU oracle: each test checks ``oracle`` against something other
than itself -- values derived by hand from the pages' definitions
(``tests/golden``), torch's decomposed quantize/dequantize ops (which the
quantize page says it bit-matches), exact float64 matmul / conv_transpose2d /
conv2d on integer data, brute force on tiny inputs, identities the pages state,
and the error bound of the float32 epilogue.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.ao.quantization.fx import _decomposed  # noqa: F401  (registers quantized_decomposed ops)

import oracle
import q8ta_inputs as qi

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = 2.0 ** -24  # float32 unit roundoff


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _torch_quant(x, scale, zp):
    return torch.ops.quantized_decomposed.quantize_per_tensor(
        torch.from_numpy(np.ascontiguousarray(x, np.float32)), scale, zp, -128, 127,
        torch.int8).numpy()


def _torch_dequant(q, scale, zp):
    return torch.ops.quantized_decomposed.dequantize_per_tensor(
        torch.from_numpy(np.ascontiguousarray(q, np.int8)), scale, zp, -128, 127,
        torch.int8).numpy()


# --------------------------------------------------------------------------- quantize
def test_quantize_hand_vectors():
    g = _gold("quantize_hand.json")
    for scale, zp, x, q in g["cases"]:
        xv = np.array([float(x)], np.float32)
        got = oracle.quantize_per_tensor(xv, scale, zp)
        assert int(got[0]) == q, (scale, zp, x, q, int(got[0]))


SCALES = [0.02, 0.272, 2.176, 0.544, qi.out_scale_for(4096), qi.out_scale_for(576), 1.0 / 3.0, 0.1]


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("zp", [0, 3, -5, -128, 127])
def test_quantize_matches_torch_decomposed(scale, zp):
    g = qi.rng(7)
    # a spread of values plus values placed on and next to every rounding tie
    x = np.concatenate([
        (g.standard_normal(20000) * 80 * scale).astype(np.float32),
        ((np.arange(-140, 141) + 0.5) * scale).astype(np.float32),
        np.nextafter(((np.arange(-140, 141) + 0.5) * scale).astype(np.float32), np.float32(np.inf)),
        np.nextafter(((np.arange(-140, 141) + 0.5) * scale).astype(np.float32), np.float32(-np.inf)),
        np.array([0.0, -0.0, 1e30, -1e30, np.inf, -np.inf], np.float32),
    ])
    np.testing.assert_array_equal(oracle.quantize_per_tensor(x, scale, zp), _torch_quant(x, scale, zp))


def test_quantize_reciprocal_is_taken_in_double():
    """The quantize page says the reciprocal is formed in double and then
    rounded to float; a float reciprocal differs for the 0.272 output scale and
    gives different codes on the tie grid, which torch and the oracle agree on."""
    scale = 0.272
    inv_double = np.float32(1.0 / scale)
    inv_float = np.float32(1.0) / np.float32(scale)
    assert inv_double != inv_float
    x = np.concatenate([((np.arange(-140, 141) + 0.5) * scale).astype(np.float32)] +
                       [(g * scale).astype(np.float32) for g in [np.linspace(-140, 140, 200001)]])
    ref = _torch_quant(x, scale, 0)
    wrong = np.clip(np.rint(x * inv_float), -128, 127).astype(np.int8)
    assert (wrong != ref).any()
    np.testing.assert_array_equal(oracle.quantize_per_tensor(x, scale, 0), ref)


def test_quantize_large_workload_matches_torch():
    c = qi.make_deconv_large()
    np.testing.assert_array_equal(oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp),
                                  _torch_quant(c.x_fp32, c.in_scale, c.in_zp))


def test_quantize_empty():
    assert oracle.quantize_per_tensor(np.zeros(0, np.float32), 0.02, 3).shape == (0,)


# --------------------------------------------------------------------------- dequantize
@pytest.mark.parametrize("scale,zp", [(0.02, 3), (0.272, -5), (1.0 / 3.0, 0), (2.176, -128), (0.1, 127)])
def test_dequantize_matches_torch_decomposed(scale, zp):
    q = np.arange(-128, 128, dtype=np.int16).astype(np.int8)
    np.testing.assert_array_equal(oracle.dequantize_per_tensor(q, scale, zp), _torch_dequant(q, scale, zp))


def test_dequantize_hand():
    got = oracle.dequantize_per_tensor(np.array([5, -128, 3, 127], np.int8), 0.5, 3)
    np.testing.assert_array_equal(got, np.array([1.0, -65.5, 0.0, 62.0], np.float32))


# --------------------------------------------------------------------------- linear contraction
def test_linear_acc_bruteforce_tiny():
    g = qi.rng(11)
    M, K, N, zp = 3, 5, 4, 3
    x = qi.x_int8(g, (M, K))
    w = qi.w_int8(g, (N, K))
    ref = [[sum((int(x[m, k]) - zp) * int(w[n, k]) for k in range(K)) for n in range(N)]
           for m in range(M)]
    np.testing.assert_array_equal(oracle.linear_acc(x, w, zp), np.array(ref, np.int32))


@pytest.mark.parametrize("zp", [3, 0, -128, 127])
@pytest.mark.parametrize("M,K,N", [(37, 300, 53), (1, 4096, 64), (64, 64, 32)])
def test_linear_acc_matches_f64_matmul(M, K, N, zp):
    g = qi.rng(M * 1000 + K + N)
    x = qi.x_int8(g, (M, K))
    w = g.integers(-128, 128, size=(N, K), dtype=np.int8)
    ref = (torch.from_numpy(x).double() - zp) @ torch.from_numpy(w).double().T
    np.testing.assert_array_equal(oracle.linear_acc(x, w, zp), ref.numpy().astype(np.int32))


def test_linear_zero_point_fold_identity():
    g = qi.rng(12)
    x = qi.x_int8(g, (17, 257))
    w = qi.w_int8(g, (29, 257))
    for zp in (3, -128, 127, 0):
        np.testing.assert_array_equal(oracle.linear_acc(x, w, zp),
                                      oracle.linear_acc(x, w, zp, folded=True))


def test_linear_gemv_is_a_gemm_row():
    c = qi.linear_case(13, 9, 320, 48)
    full = oracle.linear(c.x, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale, c.out_zp)
    for m in range(c.M):
        row = oracle.linear(c.x[m:m + 1], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                            c.out_scale, c.out_zp)
        np.testing.assert_array_equal(row[0], full[m])


def test_linear_reads_only_first_K_columns_of_padded_weight():
    c = qi.linear_case(14, 5, 100, 12, ldw=128)
    a = oracle.linear_acc(c.x, c.w, c.in_zp)
    b = oracle.linear_acc(c.x, np.ascontiguousarray(c.w[:, :100]), c.in_zp)
    np.testing.assert_array_equal(a, b)


def test_linear_overflow_is_detected():
    K = 70000  # (127 + 128) * 127 * 70000 > 2**31 - 1
    x = np.full((1, K), 127, np.int8)
    w = np.full((1, K), 127, np.int8)
    with pytest.raises(OverflowError):
        oracle.linear_acc(x, w, -128)


# --------------------------------------------------------------------------- epilogue
def test_epilogue_hand_vectors():
    g = _gold("epilogue_hand.json")
    for acc, s_in, w_s, b, s_out, ozp, q in g["cases"]:
        got = oracle.epilogue(np.array([acc], np.int32), 1, 1, s_in, np.array([w_s], np.float32),
                              None if b is None else np.array([b], np.float32), s_out, ozp)
        assert int(got[0]) == q, (acc, b, ozp, q, int(got[0]))


def _round_binary(x, mant, emin):
    """Nearest value of a binary floating-point format (``mant`` fraction
    bits, smallest normal exponent ``emin``) to the rational x, ties to even:
    the IEEE 754 default rounding written out from its definition."""
    from fractions import Fraction
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, emin) - mant)
    n = a / quantum
    k = n.numerator // n.denominator
    if n - k > Fraction(1, 2) or (n - k == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return (k if x > 0 else -k) * quantum


def _r32(x):
    return _round_binary(x, 23, -126)


def _r64(x):
    return _round_binary(x, 52, -1022)


def _rne_int(t):
    k = t.numerator // t.denominator
    if t - k > 0.5 or (t - k == 0.5 and k % 2 == 1):
        k += 1
    return k


def test_epilogue_order_derivation_is_exact():
    """Checks the hand derivation in epilogue_order_hand.json step by step in
    exact rational arithmetic (each stated intermediate is the correctly
    rounded binary32 result of the exact operation on the previous ones), and
    that each of the four other readings of the expression lands on a
    different code on at least two rows -- so the codes pin the order."""
    from fractions import Fraction as Fr
    g = _gold("epilogue_order_hand.json")
    caught = {}
    for row in g["rows"]:
        h = lambda key: Fr(float.fromhex(row[key]))
        s_in_d = _r64(Fr(row["input_scale"]))
        assert h("s_in_f32") == _r32(s_in_d)
        assert h("weight_scale_f32") == _r32(Fr(row["weight_scale"]))
        assert h("bias_f32") == _r32(Fr(row["bias"]))
        assert h("inv_out_f32") == _r32(1 / _r64(Fr(row["output_scale"])))
        a = _r32(Fr(row["acc"]))
        assert a == row["acc"]  # |acc| < 2**24: exact
        assert h("p1") == _r32(a * h("s_in_f32"))
        assert h("p2") == _r32(h("p1") * h("weight_scale_f32"))
        assert h("v") == _r32(h("p2") + h("bias_f32"))
        assert h("t") == _r32(h("v") * h("inv_out_f32"))
        q = max(-128, min(127, _rne_int(h("t")) + row["output_zero_point"]))
        assert q == row["q"]
        ws, b, inv, s_in = h("weight_scale_f32"), h("bias_f32"), h("inv_out_f32"), h("s_in_f32")
        others = {
            "prefolded_scales": _r32(_r32(a * _r32(s_in * ws)) + b),
            "fma_weight_scale_bias": _r32(h("p1") * ws + b),
            "scales_swapped": _r32(_r32(_r32(a * ws) * s_in) + b),
            "input_scale_in_double": _r32(_r32(_r32(_r64(a * s_in_d)) * ws) + b),
        }
        for name, vm in others.items():
            st = row["other_orders"][name]
            assert Fr(float.fromhex(st["v"])) == vm, (row["acc"], name)
            tm = _r32(vm * inv)
            assert Fr(float.fromhex(st["t"])) == tm
            qm = max(-128, min(127, _rne_int(tm) + row["output_zero_point"]))
            assert qm == st["q"]
            if qm != q:
                caught[name] = caught.get(name, 0) + 1
    assert set(caught) == {"prefolded_scales", "fma_weight_scale_bias", "scales_swapped",
                           "input_scale_in_double"}
    assert min(caught.values()) >= 2, caught


def test_epilogue_order_hand_vectors():
    """The oracle's epilogue reproduces every hand-derived code, alone and at
    the end of the full linear (a 1x1 contraction that yields the row's acc)."""
    g = _gold("epilogue_order_hand.json")
    for row in g["rows"]:
        args = (row["input_scale"], row["weight_scale"], row["bias"], row["output_scale"],
                row["output_zero_point"])
        s_in, w_s, b, s_out, ozp = (float(args[0]), np.float32(args[1]), np.float32(args[2]),
                                    float(args[3]), args[4])
        got = oracle.epilogue(np.array([row["acc"]], np.int32), 1, 1, s_in,
                              np.array([w_s], np.float32), np.array([b], np.float32), s_out, ozp)
        assert int(got[0]) == row["q"], (row["acc"], row["q"], int(got[0]))
        # the same value through oracle.linear: acc = 127 * S + r with 0 <= r < 127,
        # S spread over terms x * 127 with |x| <= 127, then one term r * 1
        acc = row["acc"]
        r = acc % 127
        S = (acc - r) // 127
        xs_l, ws_l = [], []
        while S != 0:
            step = max(-127, min(127, S))
            xs_l.append(step)
            ws_l.append(127)
            S -= step
        xs_l.append(r)
        ws_l.append(1)
        xs = np.array([xs_l], np.int8)
        wv = np.array([ws_l], np.int8)
        assert int((xs.astype(np.int64) * wv).sum()) == acc
        ql = oracle.linear(xs, wv, np.array([w_s], np.float32), np.array([b], np.float32), s_in,
                           0, s_out, ozp)
        assert int(ql[0, 0]) == row["q"]


def _linear_random_acc(seed, M, N, spread):
    g = qi.rng(seed)
    return g.integers(-spread, spread + 1, size=(M, N)).astype(np.int32)


@pytest.mark.parametrize("out_scale", [qi.out_scale_for(64), qi.out_scale_for(4096), 0.544, 2.176])
def test_epilogue_requant_matches_torch_quantize(out_scale):
    """The requantize half of the epilogue is the page's quantize rule applied
    to the dequantized value v: it must bit-match torch's quantize_per_tensor."""
    g = qi.rng(21)
    M, N = 64, 96
    acc = _linear_random_acc(22, M, N, 400000)
    ws = qi.scales(g, N)
    b = qi.bias(g, N)
    q, pre = oracle.epilogue(acc, N, 1, 0.02, ws, b, out_scale, -5, return_pre=True)
    np.testing.assert_array_equal(q, _torch_quant(pre, out_scale, -5))


@pytest.mark.parametrize("out_scale", [0.272, 2.176, 0.544, 1.0 / 3.0])
def test_epilogue_requant_tie_grid_matches_torch_quantize(out_scale):
    """With acc = 0 the epilogue's value is the bias exactly, so feeding the
    quantize tie grid through the bias pins the requantize reciprocal (taken
    in double, as the quantize page states for its inverse scale) on exactly
    the values where a float reciprocal would round differently."""
    grid = ((np.arange(-140, 141) + 0.5) * out_scale).astype(np.float32)
    v = np.concatenate([grid, np.nextafter(grid, np.float32(np.inf)),
                        np.nextafter(grid, np.float32(-np.inf))])
    acc = np.zeros(v.size, np.int32)
    q = oracle.epilogue(acc, v.size, 1, 1.0, np.ones(v.size, np.float32), v, out_scale, -5)
    np.testing.assert_array_equal(q, _torch_quant(v, out_scale, -5))


@pytest.mark.parametrize("with_bias", [True, False])
def test_epilogue_dequant_within_float_error_bound(with_bias):
    g = qi.rng(23)
    M, N = 50, 70
    acc = _linear_random_acc(24, M, N, 10 ** 6)
    ws = qi.scales(g, N)
    b = qi.bias(g, N) if with_bias else None
    _, pre = oracle.epilogue(acc, N, 1, 0.02, ws, b, 1.0, 0, return_pre=True)
    s_in = float(np.float32(0.02))
    prod = acc.astype(np.float64) * s_in * ws.astype(np.float64)[None, :]
    exact = prod + (b.astype(np.float64)[None, :] if with_bias else 0.0)
    bound = 3 * U * (np.abs(prod) + (np.abs(b.astype(np.float64))[None, :] if with_bias else 0)) + 1e-30
    assert (np.abs(pre.astype(np.float64) - exact) <= bound).all()


def test_epilogue_output_within_one_step_of_exact_rounding():
    """Against the exact (float64) requantization: at most one code apart, and
    identical wherever the exact value is not within 1e-3 of a rounding tie."""
    c = qi.linear_case(25, 48, 512, 80)
    q, acc = oracle.linear(c.x, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                           c.out_zp, return_acc=True)
    v = acc.astype(np.float64) * c.in_scale * c.weight_scales.astype(np.float64)[None, :] + \
        c.bias.astype(np.float64)[None, :]
    t = v / c.out_scale
    exact = np.clip(np.rint(t) + c.out_zp, -128, 127)
    d = np.abs(q.astype(np.float64) - exact)
    assert d.max() <= 1
    far = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-3
    assert (d[far] == 0).all()
    # the workload's output scale keeps most outputs inside the int8 range
    assert (np.abs(q.astype(int)) < 127).mean() > 0.9


def test_epilogue_channel_of_nchw_element():
    """Element e of an NCHW tensor belongs to channel (e // (H*W)) % C."""
    Nb, C, H, W = 2, 3, 2, 2
    acc = np.full((Nb, C, H, W), 8, np.int32)
    ws = np.array([0.25, 0.5, 1.0], np.float32)
    q = oracle.epilogue(acc, C, H * W, 1.0, ws, None, 1.0, 0)
    for n in range(Nb):
        for ch, expect in enumerate([2, 4, 8]):
            assert (q[n, ch] == expect).all()


def test_epilogue_null_bias_equals_zero_bias():
    c = qi.linear_case(26, 8, 64, 16)
    a = oracle.linear(c.x, c.w, c.weight_scales, None, c.in_scale, c.in_zp, c.out_scale, c.out_zp)
    b = oracle.linear(c.x, c.w, c.weight_scales, np.zeros(16, np.float32), c.in_scale, c.in_zp,
                      c.out_scale, c.out_zp)
    np.testing.assert_array_equal(a, b)


def test_chain_small_against_torch_pieces():
    """quantize -> linear on the small chain workload, with quantize taken from
    torch and the contraction from float64 matmul."""
    c = qi.make_chain_small()
    xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
    np.testing.assert_array_equal(xq, _torch_quant(c.x_fp32, c.in_scale, c.in_zp))
    q, acc = oracle.linear(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                           c.out_zp, return_acc=True)
    ref = (torch.from_numpy(xq).double() - c.in_zp) @ torch.from_numpy(c.w).double().T
    np.testing.assert_array_equal(acc, ref.numpy().astype(np.int32))


# --------------------------------------------------------------------------- deconv
def _orig_weight(w, OC, Kh, Kw, IC):
    """Undo the ahead-of-time reshape weight[oc,(kh*Kw+kw)*IC+ic] = orig[ic,oc,kh,kw]."""
    return torch.from_numpy(np.ascontiguousarray(w[:, :Kh * Kw * IC])).reshape(
        OC, Kh, Kw, IC).permute(3, 0, 1, 2).contiguous()


def _torch_deconv_acc(x, w, zp, Kh, Kw, stride, padding, output_padding, dilation):
    N, IC, H, W = x.shape
    OC = w.shape[0]
    wo = _orig_weight(w, OC, Kh, Kw, IC).double()
    xs = torch.from_numpy(x).double() - zp
    return F.conv_transpose2d(xs, wo, stride=stride, padding=padding,
                              output_padding=output_padding, dilation=dilation).numpy()


def test_deconv_hand_cases():
    for c in _gold("deconv_hand.json")["cases"]:
        x = np.array(c["x"], np.int8).reshape(c["N"], c["IC"], c["H_in"], c["W_in"])
        w = np.array(c["w"], np.int8).reshape(c["OC"], -1)
        for method in ("gather", "scatter", "zpfill"):
            acc = oracle.deconv_acc(x, w, c["zp"], c["Kh"], c["Kw"], c["stride"], c["pad"], (1, 1),
                                    c["H_out"], c["W_out"], method=method)
            np.testing.assert_array_equal(acc.reshape(-1), np.array(c["acc"]), err_msg=c["name"])


DECONV_SHAPES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad, dil
    (1, 5, 6, 7, 3, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1)),
    (2, 4, 5, 5, 6, 4, 4, (2, 2), (1, 1), (0, 0), (1, 1)),
    (1, 3, 4, 6, 2, 3, 2, (3, 2), (0, 1), (2, 1), (1, 1)),
    (1, 2, 5, 4, 3, 1, 1, (1, 1), (0, 0), (0, 0), (1, 1)),
    (1, 3, 4, 4, 2, 5, 3, (2, 3), (2, 1), (1, 0), (1, 1)),
    (1, 2, 4, 5, 2, 3, 3, (2, 2), (1, 2), (1, 0), (2, 2)),
    (2, 3, 3, 3, 4, 2, 2, (1, 1), (1, 0), (0, 0), (1, 1)),
]


@pytest.mark.parametrize("shape", DECONV_SHAPES)
def test_deconv_matches_torch_conv_transpose2d(shape):
    N, IC, H, W, OC, Kh, Kw, s, p, op, d = shape
    g = qi.rng(sum(shape[:7]))
    x = qi.x_int8(g, (N, IC, H, W))
    w = g.integers(-128, 128, size=(OC, Kh * Kw * IC), dtype=np.int8)
    ref = _torch_deconv_acc(x, w, 3, Kh, Kw, s, p, op, d)
    H_out, W_out = ref.shape[2:]
    assert H_out == qi.deconv_out_size(H, Kh, s[0], p[0], op[0], d[0])
    assert W_out == qi.deconv_out_size(W, Kw, s[1], p[1], op[1], d[1])
    for method in ("gather", "scatter", "zpfill"):
        acc = oracle.deconv_acc(x, w, 3, Kh, Kw, s, p, d, H_out, W_out, method=method)
        np.testing.assert_array_equal(acc, ref.astype(np.int32), err_msg=method)


@pytest.mark.parametrize("H_out,W_out", [(3, 17), (20, 9), (1, 1), (0, 5)])
def test_deconv_gather_scatter_zpfill_agree_for_any_output_size(H_out, W_out):
    """The output size is given explicitly; for any size the three
    formulations of the sum agree."""
    g = qi.rng(31 + H_out * 7 + W_out)
    x = qi.x_int8(g, (2, 3, 5, 4))
    w = qi.w_int8(g, (4, 3 * 3 * 3 + 5))  # padded weight rows
    a = oracle.deconv_acc(x, w, -7, 3, 3, (2, 2), (1, 1), (1, 1), H_out, W_out, "gather")
    b = oracle.deconv_acc(x, w, -7, 3, 3, (2, 2), (1, 1), (1, 1), H_out, W_out, "scatter")
    c = oracle.deconv_acc(x, w, -7, 3, 3, (2, 2), (1, 1), (1, 1), H_out, W_out, "zpfill")
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_deconv_adjoint_identity():
    """<convT(x'), y> == <x', conv2d(y)> for x' = x - zp (integers, exact in float64)."""
    g = qi.rng(41)
    N, IC, H, W, OC, K = 2, 4, 5, 6, 3, 3
    s, p, op = (2, 2), (1, 1), (1, 1)
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, K * K * IC))
    Ho, Wo = qi.deconv_out_size(H, K, 2, 1, 1), qi.deconv_out_size(W, K, 2, 1, 1)
    acc = oracle.deconv_acc(x, w, 3, K, K, s, p, (1, 1), Ho, Wo)
    y = torch.from_numpy(g.integers(-50, 51, size=(N, OC, Ho, Wo))).double()
    wo = _orig_weight(w, OC, K, K, IC).double()
    back = F.conv2d(y, wo, stride=s, padding=p)  # [N, IC, H, W]
    lhs = float((torch.from_numpy(acc).double() * y).sum())
    rhs = float(((torch.from_numpy(x).double() - 3) * back[:, :, :H, :W]).sum())
    assert lhs == rhs


def test_deconv_1x1_stride1_is_linear_on_nhwc():
    g = qi.rng(42)
    N, IC, H, W, OC = 2, 40, 3, 5, 24
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, IC))
    acc = oracle.deconv_acc(x, w, 3, 1, 1, (1, 1), (0, 0), (1, 1), H, W)
    lin = oracle.linear_acc(x.transpose(0, 2, 3, 1).reshape(-1, IC), w, 3)
    np.testing.assert_array_equal(acc.transpose(0, 2, 3, 1).reshape(-1, OC), lin)


def test_deconv_epilogue_channel_is_oc():
    c = qi.deconv_case(43, 2, 6, 5, 4, 5, 3, 3, (2, 2), (1, 1), (1, 1))
    q, acc = oracle.conv2d_transposed(c.x, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                                      c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding,
                                      c.dilation, c.H_out, c.W_out, return_acc=True)
    v = acc.astype(np.float64) * c.in_scale * c.weight_scales.astype(np.float64)[None, :, None, None] \
        + c.bias.astype(np.float64)[None, :, None, None]
    t = v / c.out_scale
    exact = np.clip(np.rint(t) + c.out_zp, -128, 127)
    d = np.abs(q.astype(np.float64) - exact)
    assert d.max() <= 1
    far = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-3
    assert (d[far] == 0).all()


def test_deconv_small_workload_matches_torch():
    c = qi.make_deconv_small()
    assert (c.H_out, c.W_out) == (64, 64)
    acc = oracle.deconv_acc(c.x, c.w, c.in_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation,
                            c.H_out, c.W_out)
    ref = _torch_deconv_acc(c.x, c.w, c.in_zp, c.Kh, c.Kw, c.stride, c.padding,
                            c.output_padding, c.dilation)
    np.testing.assert_array_equal(acc, ref.astype(np.int32))


def test_deconv_large_workload_output_size():
    c = qi.make_deconv_large()
    assert (c.H_out, c.W_out) == (128, 128)
    assert c.w.shape == (128, 9 * 256)


# --------------------------------------------------------------------------- forward conv2d
def _torch_conv2d_acc(x, w, zp, Kh, Kw, stride, padding, dilation, groups=1):
    """Exact float64 torch conv2d of (x - zp) with the weight reshape
    w[oc, (kh*Kw+kw)*ICg + icg] = orig[oc, icg, kh, kw] undone (ICg = IC/groups)."""
    N, IC, H, W = x.shape
    OC = w.shape[0]
    ICg = IC // groups
    wo = torch.from_numpy(np.ascontiguousarray(w[:, :Kh * Kw * ICg])).reshape(
        OC, Kh, Kw, ICg).permute(0, 3, 1, 2).contiguous().double()
    xs = torch.from_numpy(x).double() - zp
    return F.conv2d(xs, wo, stride=stride, padding=padding, dilation=dilation,
                    groups=groups).numpy()


def test_conv2d_hand_cases():
    for c in _gold("conv2d_hand.json")["cases"]:
        x = np.array(c["x"], np.int8).reshape(c["N"], c["IC"], c["H_in"], c["W_in"])
        w = np.array(c["w"], np.int8).reshape(c["OC"], -1)
        acc = oracle.conv2d_acc(x, w, c["zp"], c["Kh"], c["Kw"], c["stride"], c["pad"], c["dil"],
                                c["H_out"], c["W_out"], groups=c["groups"])
        np.testing.assert_array_equal(acc.reshape(-1), np.array(c["acc"]), err_msg=c["name"])


CONV2D_SHAPES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, dil
    (1, 5, 7, 6, 3, 3, 3, (1, 1), (1, 1), (1, 1)),
    (2, 4, 9, 8, 5, 3, 3, (2, 2), (1, 1), (1, 1)),
    (1, 3, 8, 9, 2, 5, 3, (2, 3), (2, 0), (1, 1)),
    (1, 3, 9, 7, 4, 3, 2, (1, 2), (0, 1), (2, 3)),
    (1, 2, 5, 5, 3, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 2, 4, 5, 2, 3, 3, (1, 1), (4, 3), (1, 1)),      # pad larger than the kernel
    (2, 3, 6, 6, 2, 4, 4, (3, 3), (1, 2), (1, 1)),
]


@pytest.mark.parametrize("shape", CONV2D_SHAPES)
def test_conv2d_matches_torch_conv2d(shape):
    N, IC, H, W, OC, Kh, Kw, s, p, d = shape
    g = qi.rng(sum(shape[:7]) + 1)
    x = qi.x_int8(g, (N, IC, H, W))
    w = g.integers(-128, 128, size=(OC, Kh * Kw * IC), dtype=np.int8)
    ref = _torch_conv2d_acc(x, w, -5, Kh, Kw, s, p, d)
    H_out, W_out = ref.shape[2:]
    assert H_out == qi.conv_out_size(H, Kh, s[0], p[0], d[0])
    assert W_out == qi.conv_out_size(W, Kw, s[1], p[1], d[1])
    acc = oracle.conv2d_acc(x, w, -5, Kh, Kw, s, p, d, H_out, W_out)
    np.testing.assert_array_equal(acc, ref.astype(np.int32))


def test_conv2d_brute_force_tiny():
    """Pure-Python loops over the definition on a tiny input."""
    g = qi.rng(77)
    N, IC, H, W, OC, Kh, Kw, s, p, d, zp = 1, 2, 4, 5, 2, 2, 3, (2, 1), (1, 1), (1, 2), 7
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, Kh * Kw * IC + 3))
    Ho, Wo = qi.conv_out_size(H, Kh, s[0], p[0], d[0]), qi.conv_out_size(W, Kw, s[1], p[1], d[1])
    ref = np.zeros((N, OC, Ho, Wo), np.int64)
    for n in range(N):
        for oc in range(OC):
            for oh in range(Ho):
                for ow in range(Wo):
                    t = 0
                    for ic in range(IC):
                        for kh in range(Kh):
                            for kw in range(Kw):
                                ih, iw = oh * s[0] - p[0] + kh * d[0], ow * s[1] - p[1] + kw * d[1]
                                if 0 <= ih < H and 0 <= iw < W:
                                    t += (int(x[n, ic, ih, iw]) - zp) * int(w[oc, (kh * Kw + kw) * IC + ic])
                    ref[n, oc, oh, ow] = t
    np.testing.assert_array_equal(oracle.conv2d_acc(x, w, zp, Kh, Kw, s, p, d, Ho, Wo), ref)


def test_conv2d_is_the_adjoint_of_the_transposed_conv():
    """<conv2d(x - zp), y> == <x - zp, conv_transpose(y)> with the channel axes
    of the weight swapped: ties the forward oracle to the (separately pinned)
    transposed one; integers, exact in int64."""
    g = qi.rng(78)
    N, IC, H, W, OC, Kh, Kw, s, p, d = 2, 5, 9, 8, 4, 3, 2, (2, 3), (1, 1), (1, 2)
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, Kh * Kw * IC))
    Ho, Wo = qi.conv_out_size(H, Kh, s[0], p[0], d[0]), qi.conv_out_size(W, Kw, s[1], p[1], d[1])
    acc = oracle.conv2d_acc(x, w, 3, Kh, Kw, s, p, d, Ho, Wo).astype(np.int64)
    y = qi.x_int8(g, (N, OC, Ho, Wo))
    wt = w.reshape(OC, Kh * Kw, IC).transpose(2, 1, 0).reshape(IC, Kh * Kw * OC)
    back = oracle.deconv_acc(y, wt, 0, Kh, Kw, s, p, d, H, W).astype(np.int64)
    lhs = int((acc * y.astype(np.int64)).sum())
    rhs = int(((x.astype(np.int64) - 3) * back).sum())
    assert lhs == rhs


def test_conv2d_1x1_stride1_is_linear_on_nhwc():
    g = qi.rng(79)
    N, IC, H, W, OC = 2, 40, 3, 5, 24
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, IC))
    acc = oracle.conv2d_acc(x, w, 3, 1, 1, (1, 1), (0, 0), (1, 1), H, W)
    lin = oracle.linear_acc(x.transpose(0, 2, 3, 1).reshape(-1, IC), w, 3)
    np.testing.assert_array_equal(acc.transpose(0, 2, 3, 1).reshape(-1, OC), lin)


def test_conv2d_epilogue_matches_the_shared_epilogue():
    c = qi.conv_case(80, 2, 6, 7, 5, 5, 3, 3, (2, 2), (1, 1), (1, 1))
    q, acc = oracle.conv2d(c.x, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                           c.out_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation, c.H_out, c.W_out,
                           return_acc=True)
    ref = oracle.epilogue(acc, c.w.shape[0], c.H_out * c.W_out, c.in_scale, c.weight_scales,
                          c.bias, c.out_scale, c.out_zp)
    np.testing.assert_array_equal(q, ref)


GROUPED_SHAPES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, dil, groups
    (1, 6, 7, 6, 4, 3, 3, (1, 1), (1, 1), (1, 1), 2),
    (2, 8, 9, 8, 12, 3, 2, (2, 1), (1, 0), (1, 2), 4),
    (1, 5, 8, 9, 5, 3, 3, (1, 1), (1, 1), (1, 1), 5),      # depthwise
    (1, 4, 9, 7, 8, 5, 3, (2, 2), (2, 1), (1, 1), 4),      # depthwise, channel multiplier 2
    (2, 6, 6, 6, 6, 3, 3, (2, 2), (1, 1), (2, 2), 6),      # depthwise, dilated, strided
]


@pytest.mark.parametrize("shape", GROUPED_SHAPES)
def test_grouped_conv2d_matches_torch(shape):
    N, IC, H, W, OC, Kh, Kw, s, p, d, G = shape
    g = qi.rng(sum(shape[:7]) + 3)
    x = qi.x_int8(g, (N, IC, H, W))
    w = g.integers(-128, 128, size=(OC, Kh * Kw * (IC // G)), dtype=np.int8)
    ref = _torch_conv2d_acc(x, w, 9, Kh, Kw, s, p, d, groups=G)
    H_out, W_out = ref.shape[2:]
    acc = oracle.conv2d_acc(x, w, 9, Kh, Kw, s, p, d, H_out, W_out, groups=G)
    np.testing.assert_array_equal(acc, ref.astype(np.int32))


def test_grouped_conv2d_is_per_group_ungrouped_conv():
    """A grouped conv equals the ungrouped conv of each group's channel slice."""
    g = qi.rng(81)
    N, IC, H, W, OC, K, G = 2, 6, 7, 5, 9, 3, 3
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, K * K * (IC // G) + 4))
    acc = oracle.conv2d_acc(x, w, -3, K, K, (1, 2), (1, 1), (1, 1), 7, 3, groups=G)
    for gi in range(G):
        xs = x[:, gi * (IC // G):(gi + 1) * (IC // G)]
        ws = w[gi * (OC // G):(gi + 1) * (OC // G)]
        part = oracle.conv2d_acc(xs, ws, -3, K, K, (1, 2), (1, 1), (1, 1), 7, 3)
        np.testing.assert_array_equal(acc[:, gi * (OC // G):(gi + 1) * (OC // G)], part)


def test_depthwise_brute_force_tiny():
    g = qi.rng(82)
    N, C, H, W, Kh, Kw, s, p, d, zp = 1, 3, 5, 4, 3, 2, (2, 1), (1, 1), (1, 1), 5
    x = qi.x_int8(g, (N, C, H, W))
    w = qi.w_int8(g, (C, Kh * Kw))
    Ho, Wo = qi.conv_out_size(H, Kh, s[0], p[0], d[0]), qi.conv_out_size(W, Kw, s[1], p[1], d[1])
    ref = np.zeros((N, C, Ho, Wo), np.int64)
    for c in range(C):
        for oh in range(Ho):
            for ow in range(Wo):
                t = 0
                for kh in range(Kh):
                    for kw in range(Kw):
                        ih, iw = oh * s[0] - p[0] + kh * d[0], ow * s[1] - p[1] + kw * d[1]
                        if 0 <= ih < H and 0 <= iw < W:
                            t += (int(x[0, c, ih, iw]) - zp) * int(w[c, kh * Kw + kw])
                ref[0, c, oh, ow] = t
    np.testing.assert_array_equal(oracle.conv2d_acc(x, w, zp, Kh, Kw, s, p, d, Ho, Wo, groups=C),
                                  ref)


# --------------------------------------------------------------------------- relu-fused epilogue
def test_relu_epilogue_hand_vectors():
    g = _gold("epilogue_relu_hand.json")
    for acc, s_in, w_s, b, s_out, ozp, q_relu, q_none in g["cases"]:
        args = (np.array([acc], np.int32), 1, 1, s_in, np.array([w_s], np.float32),
                None if b is None else np.array([b], np.float32), s_out, ozp)
        assert int(oracle.epilogue(*args, activation="relu")[0]) == q_relu, (acc, b, ozp)
        assert int(oracle.epilogue(*args)[0]) == q_none, (acc, b, ozp)


@pytest.mark.parametrize("ozp", [-128, -5, 0, 3, 127])
def test_relu_epilogue_is_torch_quantize_of_relu(ozp):
    """Relu-fused output == torch's decomposed quantize of torch.relu(v), v the
    real-valued output before requantization; and == max(plain output, zp)."""
    g = qi.rng(1091 + ozp)
    acc = _linear_random_acc(1092 + ozp, 64, 48, 300000)
    ws = g.uniform(0.005, 0.02, 48).astype(np.float32)
    b = g.normal(0, 0.1, 48).astype(np.float32)
    s_out = qi.out_scale_for(4096)
    q_none, pre = oracle.epilogue(acc, 48, 1, 0.02, ws, b, s_out, ozp, return_pre=True)
    q_relu = oracle.epilogue(acc, 48, 1, 0.02, ws, b, s_out, ozp, activation="relu")
    assert (pre < 0).mean() > 0.3 and (pre > 0).mean() > 0.3
    ref = _torch_quant(torch.relu(torch.from_numpy(pre)).numpy(), s_out, ozp)
    np.testing.assert_array_equal(q_relu, ref)
    np.testing.assert_array_equal(q_relu, np.maximum(q_none, ozp))


def test_relu_reaches_every_op():
    """linear, the transposed conv and the forward conv pass the activation to
    the epilogue: their relu outputs are max(plain output, zp)."""
    c = qi.linear_case(93, 5, 64, 24)
    for act_out, plain in [
        (oracle.linear(c.x, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                       c.out_zp, activation="relu"),
         oracle.linear(c.x, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                       c.out_zp))]:
        np.testing.assert_array_equal(act_out, np.maximum(plain, c.out_zp))
    d = qi.deconv_case(94, 1, 4, 5, 5, 6, 3, 3, (2, 2), (1, 1), (1, 1))
    args = (d.x, d.w, d.weight_scales, d.bias, d.in_scale, d.in_zp, d.out_scale, d.out_zp, d.Kh,
            d.Kw, d.stride, d.padding, d.dilation, d.H_out, d.W_out)
    np.testing.assert_array_equal(oracle.conv2d_transposed(*args, activation="relu"),
                                  np.maximum(oracle.conv2d_transposed(*args), d.out_zp))
    f = qi.conv_case(95, 1, 4, 7, 6, 5, 3, 3, (1, 1), (1, 1), (1, 1))
    args = (f.x, f.w, f.weight_scales, f.bias, f.in_scale, f.in_zp, f.out_scale, f.out_zp, f.Kh,
            f.Kw, f.stride, f.padding, f.dilation, f.H_out, f.W_out)
    relu = oracle.conv2d(*args, activation="relu")
    np.testing.assert_array_equal(relu, np.maximum(oracle.conv2d(*args), f.out_zp))
    assert (relu == f.out_zp).mean() > 0.2


# --------------------------------------------------------------------------- transposed conv: dilation, groups
def _torch_deconv_acc_grouped(x, w, zp, Kh, Kw, stride, padding, output_padding, dilation, groups):
    """Exact float64 torch conv_transpose2d of (x - zp) with the grouped reshape
    w[oc, (kh*Kw+kw)*ICg + icg] = orig[g*ICg + icg, oc - g*OCg, kh, kw] undone."""
    N, IC, H, W = x.shape
    OC = w.shape[0]
    ICg, OCg = IC // groups, OC // groups
    wo = torch.from_numpy(np.ascontiguousarray(w[:, :Kh * Kw * ICg])).reshape(
        groups, OCg, Kh, Kw, ICg).permute(0, 4, 1, 2, 3).reshape(IC, OCg, Kh, Kw)
    xs = torch.from_numpy(x).double() - zp
    return F.conv_transpose2d(xs, wo.contiguous().double(), stride=stride, padding=padding,
                              output_padding=output_padding, dilation=dilation,
                              groups=groups).numpy()


DECONV_GROUPED_SHAPES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad, dil, groups
    (1, 4, 5, 6, 6, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), 2),
    (2, 6, 4, 5, 3, 4, 4, (2, 2), (1, 1), (0, 0), (1, 1), 3),
    (1, 5, 5, 4, 5, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), 5),      # depthwise
    (1, 3, 4, 5, 6, 3, 2, (2, 1), (1, 0), (1, 0), (1, 1), 3),      # depthwise, multiplier 2
    (1, 4, 5, 5, 4, 3, 3, (2, 2), (2, 2), (1, 1), (2, 2), 2),      # grouped and dilated
    (1, 3, 6, 5, 2, 3, 3, (1, 1), (2, 1), (0, 0), (2, 3), 1),      # dilated, stride 1
    (2, 2, 4, 4, 3, 3, 3, (3, 2), (2, 1), (2, 1), (2, 2), 1),      # dilated, stride 3 x 2
]


@pytest.mark.parametrize("shape", DECONV_GROUPED_SHAPES)
def test_grouped_dilated_deconv_matches_torch(shape):
    N, IC, H, W, OC, Kh, Kw, s, p, op, d, G = shape
    g = qi.rng(sum(shape[:7]) + 5)
    x = qi.x_int8(g, (N, IC, H, W))
    w = g.integers(-128, 128, size=(OC, Kh * Kw * (IC // G)), dtype=np.int8)
    ref = _torch_deconv_acc_grouped(x, w, -6, Kh, Kw, s, p, op, d, G)
    H_out, W_out = ref.shape[2:]
    assert H_out == qi.deconv_out_size(H, Kh, s[0], p[0], op[0], d[0])
    for method in ("gather", "scatter", "zpfill"):
        acc = oracle.deconv_acc(x, w, -6, Kh, Kw, s, p, d, H_out, W_out, method=method, groups=G)
        np.testing.assert_array_equal(acc, ref.astype(np.int32), err_msg=method)


def test_grouped_deconv_is_per_group_ungrouped_deconv():
    g = qi.rng(96)
    N, IC, H, W, OC, K, G = 2, 6, 5, 4, 9, 3, 3
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, K * K * (IC // G) + 3))
    acc = oracle.deconv_acc(x, w, 4, K, K, (2, 2), (1, 1), (1, 2), 10, 9, groups=G)
    for gi in range(G):
        xs = x[:, gi * (IC // G):(gi + 1) * (IC // G)]
        ws = w[gi * (OC // G):(gi + 1) * (OC // G)]
        part = oracle.deconv_acc(xs, ws, 4, K, K, (2, 2), (1, 1), (1, 2), 10, 9)
        np.testing.assert_array_equal(acc[:, gi * (OC // G):(gi + 1) * (OC // G)], part)


def test_grouped_dilated_deconv_is_the_adjoint_of_the_grouped_conv():
    """<conv2d_g(x - zp), y> == <x - zp, convT_g(y)>, the transposed weight
    holding each group's block with its channel axes swapped; exact in int64."""
    g = qi.rng(97)
    N, IC, H, W, OC, Kh, Kw, s, p, d, G = 2, 6, 9, 8, 4, 3, 2, (2, 3), (1, 1), (2, 2), 2
    ICg, OCg, T = IC // G, OC // G, Kh * Kw
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, T * ICg))
    Ho, Wo = qi.conv_out_size(H, Kh, s[0], p[0], d[0]), qi.conv_out_size(W, Kw, s[1], p[1], d[1])
    acc = oracle.conv2d_acc(x, w, 3, Kh, Kw, s, p, d, Ho, Wo, groups=G).astype(np.int64)
    y = qi.x_int8(g, (N, OC, Ho, Wo))
    wt = w.reshape(G, OCg, T, ICg).transpose(0, 3, 2, 1).reshape(IC, T * OCg)
    back = oracle.deconv_acc(y, wt, 0, Kh, Kw, s, p, d, H, W, groups=G).astype(np.int64)
    lhs = int((acc * y.astype(np.int64)).sum())
    rhs = int(((x.astype(np.int64) - 3) * back).sum())
    assert lhs == rhs


def test_grouped_dilated_deconv_brute_force_tiny():
    """Pure-Python loops over the gather as the page states it (numerator
    checked for sign and divisibility before dividing), per group."""
    g = qi.rng(98)
    N, IC, H, W, OC, Kh, Kw, s, p, d, G, zp = 1, 4, 3, 4, 6, 3, 2, (2, 3), (1, 2), (2, 1), 2, -9
    ICg, OCg = IC // G, OC // G
    x = qi.x_int8(g, (N, IC, H, W))
    w = qi.w_int8(g, (OC, Kh * Kw * ICg + 2))
    Ho, Wo = 8, 11
    ref = np.zeros((N, OC, Ho, Wo), np.int64)
    for oc in range(OC):
        gi = oc // OCg
        for oh in range(Ho):
            for ow in range(Wo):
                t = 0
                for icg in range(ICg):
                    for kh in range(Kh):
                        nh = oh + p[0] - kh * d[0]
                        if nh < 0 or nh % s[0] or nh // s[0] >= H:
                            continue
                        for kw in range(Kw):
                            nw = ow + p[1] - kw * d[1]
                            if nw < 0 or nw % s[1] or nw // s[1] >= W:
                                continue
                            t += (int(x[0, gi * ICg + icg, nh // s[0], nw // s[1]]) - zp) * \
                                int(w[oc, (kh * Kw + kw) * ICg + icg])
                ref[0, oc, oh, ow] = t
    for method in ("gather", "scatter", "zpfill"):
        np.testing.assert_array_equal(
            oracle.deconv_acc(x, w, zp, Kh, Kw, s, p, d, Ho, Wo, method=method, groups=G), ref)


# --------------------------------------------------------------------------- weight sums (precomputed, opt-in)
def test_weight_sums_brute_force_and_zero_point_identity():
    """sum_k w[n,k] by pure-Python loops on a tiny matrix, and through the
    contraction: acc(zp = 0) - acc(zp) == zp * sum_k w (the page's fold)."""
    g = qi.rng(99)
    w = qi.w_int8(g, (5, 37))
    ref = [sum(int(v) for v in row) for row in w]
    np.testing.assert_array_equal(oracle.weight_sums(w), np.array(ref, np.int32))
    np.testing.assert_array_equal(oracle.weight_sums(w, K=20), np.array([sum(int(v) for v in row[:20]) for row in w], np.int32))
    x = qi.x_int8(g, (3, 37))
    d = oracle.linear_acc(x, w, 0).astype(np.int64) - oracle.linear_acc(x, w, 7).astype(np.int64)
    np.testing.assert_array_equal(d, 7 * np.broadcast_to(oracle.weight_sums(w).astype(np.int64), d.shape))
