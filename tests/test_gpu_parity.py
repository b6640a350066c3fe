"""GPU parity: libq8ta's HIP kernels, called through the C ABI, against the CPU
oracle on the same seeded inputs.  int8 outputs and int32 accumulators must be
bit-exact (integer sums are order-free and the float epilogue is evaluated in
the same operation order on both sides, without fused multiply-add).
"""
import contextlib
import os
import sys

import numpy as np
import pytest

import oracle
import q8ta_inputs as qi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import int8_quantized_amd as q8  # noqa: E402


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


class kernel:
    """Force one kernel family of an op (q8ta_select_kernel) inside a block;
    "default" (or "") keeps the library's own choice."""

    def __init__(self, op, name):
        self.op, self.name = op, name or "default"

    def __enter__(self):
        q8.q8ta_select_kernel(self.op, self.name)

    def __exit__(self, *exc):
        q8.q8ta_select_kernel(self.op, "default")


# ============================================================================ quantize
@pytest.mark.parametrize("numel", [1, 3, 4, 5, 255, 1024, 1027, 4096 + 13, 300001])
@pytest.mark.parametrize("offset", [0, 1])
def test_quantize_ragged(numel, offset):
    _say(f"quantize numel={numel} offset={offset}")
    g = qi.rng(numel + offset)
    x = (g.standard_normal(numel) * 3).astype(np.float32)
    xb = torch.zeros(numel + offset, dtype=torch.float32, device="cuda")
    xb[offset:] = dev(x)
    ob = torch.zeros(numel + offset, dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_per_tensor(xb[offset:], ob[offset:], 0.02, 3)
    np.testing.assert_array_equal(host(ob[offset:]), oracle.quantize_per_tensor(x, 0.02, 3))


@pytest.mark.parametrize("numel", [5, 4096 + 13, 300001, 2 * 256 * 8 * 4 + 7, 256 * 16 * 3 + 4])
def test_quantize_grid_tails(numel):
    """Sizes around the vector kernel's per-thread and per-block strides."""
    _say(f"quantize numel={numel}")
    x = (qi.rng(numel + 17).standard_normal(numel) * 3).astype(np.float32)
    ob = torch.zeros(numel, dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_per_tensor(dev(x), ob, 0.02, 3)
    np.testing.assert_array_equal(host(ob), oracle.quantize_per_tensor(x, 0.02, 3))


def test_quantize_ties_and_saturation():
    import json
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantize_hand.json")))["cases"]
    for scale, zp, x, q in cases:
        xs = torch.full((8,), float(x), dtype=torch.float32, device="cuda")
        out = torch.empty(8, dtype=torch.int8, device="cuda")
        q8.q8ta_quantize_per_tensor(xs, out, scale, zp)
        assert (host(out) == q).all(), (scale, zp, x, q, host(out))


@pytest.mark.parametrize("scale", [0.02, 0.272, 2.176, 0.544, qi.out_scale_for(4096)])
def test_quantize_scales(scale):
    g = qi.rng(5)
    x = np.concatenate([(g.standard_normal(100000) * 90 * scale).astype(np.float32),
                        ((np.arange(-140, 141) + 0.5) * scale).astype(np.float32)])
    out = torch.empty(x.size, dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_per_tensor(dev(x), out, scale, -5)
    np.testing.assert_array_equal(host(out), oracle.quantize_per_tensor(x, scale, -5))


def test_quantize_large_workload():
    c = qi.make_deconv_large()
    _say("quantize [8,256,64,64]")
    out = torch.empty(c.x_fp32.shape, dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_per_tensor(dev(c.x_fp32), out, c.in_scale, c.in_zp)
    np.testing.assert_array_equal(host(out), oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp))


def test_quantize_empty():
    x = torch.empty(0, dtype=torch.float32, device="cuda")
    o = torch.empty(0, dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_per_tensor(x, o, 0.02, 3)


# ============================================================================ dequantize
@pytest.mark.parametrize("numel", [1, 7, 1024, 1029, 65536 + 3])
@pytest.mark.parametrize("offset", [0, 1])
def test_dequantize_ragged(numel, offset):
    _say(f"dequantize numel={numel} offset={offset}")
    g = qi.rng(numel * 3 + offset)
    q = qi.x_int8(g, numel)
    qb = torch.zeros(numel + offset, dtype=torch.int8, device="cuda")
    qb[offset:] = dev(q)
    ob = torch.zeros(numel + offset, dtype=torch.float32, device="cuda")
    q8.q8ta_dequantize_per_tensor(qb[offset:], ob[offset:], 0.272, -5)
    np.testing.assert_array_equal(host(ob[offset:]), oracle.dequantize_per_tensor(q, 0.272, -5))


# ============================================================================ linear
def _run_linear(c, fn=None, bias=True, activation="none"):
    fn = fn or q8.q8ta_linear
    out = torch.empty((c.M, c.N), dtype=torch.int8, device="cuda")
    b = dev(c.bias) if (bias and c.bias is not None) else None
    fn(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales), b, c.out_scale,
       c.out_zp, activation, out)
    return host(out)


def _oracle_linear(c, bias=True, activation="none"):
    return oracle.linear(c.x, c.w, c.weight_scales, c.bias if bias else None, c.in_scale, c.in_zp,
                         c.out_scale, c.out_zp, activation=activation)


def _acc_linear(c):
    acc = torch.empty((c.M, c.N), dtype=torch.int32, device="cuda")
    q8.q8ta_linear_acc(dev(c.x), c.in_zp, dev(c.w), acc)
    return host(acc)


LINEAR_SHAPES = [
    # skinny / gemv path (M <= 4, K % 16 == 0)
    (1, 4096, 4096), (1, 16, 1), (1, 1040, 37), (2, 1024, 100), (3, 48, 17), (4, 4096, 64),
    (4, 64, 32),
    # matrix-core path: ragged M, N and K (K % 64 != 0); (5, 64, 32) is the case whose accumulator
    # call once read weight_scales through a NULL pointer (fixed: the epilogue reads no scale then)
    (5, 64, 32), (65, 320, 97), (300, 1040, 257), (256, 4096, 512), (513, 256, 1000),
    (129, 2064, 129),
    # shape-general path (K % 16 != 0)
    (7, 33, 5), (1, 100, 9), (40, 100, 70),
]


@pytest.mark.parametrize("M,K,N", LINEAR_SHAPES)
def test_linear_parity(M, K, N):
    _say(f"linear M={M} K={K} N={N}")
    c = qi.linear_case(M * 7 + K * 3 + N, M, K, N)
    np.testing.assert_array_equal(_run_linear(c), _oracle_linear(c))
    np.testing.assert_array_equal(_acc_linear(c), oracle.linear_acc(c.x, c.w, c.in_zp))


@pytest.mark.parametrize("izp", [-128, 127, 0])
@pytest.mark.parametrize("M,K,N", [(1, 512, 64), (70, 512, 80)])
def test_linear_zero_points_and_no_bias(M, K, N, izp):
    _say(f"linear zp M={M} izp={izp}")
    c = qi.linear_case(300 + izp, M, K, N, in_zp=izp, out_zp=127 if izp < 0 else -128)
    np.testing.assert_array_equal(_run_linear(c, bias=False), _oracle_linear(c, bias=False))
    np.testing.assert_array_equal(_run_linear(c), _oracle_linear(c))


# Shapes that reach each GEMM tile of the default dispatch: the 128 x 64 tile
# (M <= 64 with few tiles), the 128 x 128 tile, the 32x32x32 256 x 128 tile
# (>= 256 such tiles and K >= 1024; one of them with ragged M, N and K tail),
# and the shape-general kernel (K % 16 != 0); plus every shape forced onto the
# shape-general kernel.
GEMM_TILE_SHAPES = [(64, 128, 64), (70, 48, 300), (300, 1040, 257), (512, 4096, 768),
                    (1024, 1024, 8192), (1000, 1040, 8100), (33, 100, 70)]


@pytest.mark.parametrize("path", ["default", "mfma32", "mfma32_8w", "generic"])
@pytest.mark.parametrize("M,K,N", GEMM_TILE_SHAPES)
def test_linear_every_gemm_tile(path, M, K, N):
    _say(f"gemm {path} M={M} K={K} N={N}")
    if path == "generic" and M * K * N > 1 << 31:
        pytest.skip("the shape-general kernel is checked on the smaller shapes")
    c = qi.linear_case(M + N + len(path), M, K, N)
    with kernel("linear", path):
        np.testing.assert_array_equal(_run_linear(c), _oracle_linear(c))
        np.testing.assert_array_equal(_acc_linear(c), oracle.linear_acc(c.x, c.w, c.in_zp))
        # fp32 output (fused dequantize; the 32x32x32 kernel stores it in its
        # transposed form)
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        q8.q8ta_linear_dq(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                          dev(c.bias), c.out_scale, c.out_zp, "relu", out)
        ref = oracle.dequantize_per_tensor(_oracle_linear(c, activation="relu"), c.out_scale,
                                           c.out_zp)
        np.testing.assert_array_equal(host(out).view(np.uint32), ref.view(np.uint32))


# The eight-wave kernel: one K step (64), two, three (one pass of its three
# LDS stages), a tail of one and of two steps after whole passes, ragged M and
# N in one and in several tiles, a grid that is not a multiple of 8 (its XCD
# remapping leaves the last tiles in place), and 258 tiles of 256 x 256: one
# launch of 256 of them, then the last column of tiles as 256 x 128 tiles
# (ragged in M and N).
W8_SHAPES = [(256, 64, 256), (257, 128, 255), (512, 192, 512), (300, 1088, 257),
             (70, 256, 1000), (1000, 1024, 900), (769, 640, 2304), (300, 1088, 33000)]


@pytest.mark.parametrize("M,K,N", W8_SHAPES)
def test_linear_w8_edges(M, K, N):
    _say(f"gemm w8 M={M} K={K} N={N}")
    c = qi.linear_case(M * 7 + K + N, M, K, N)
    ref = _oracle_linear(c, activation="relu")
    wd = dev(c.w)
    sums = torch.empty(N, dtype=torch.int32, device="cuda")
    q8.q8ta_weight_sums(wd, sums)
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    outf = torch.empty((M, N), dtype=torch.float32, device="cuda")
    dq = oracle.dequantize_per_tensor(ref, c.out_scale, c.out_zp)
    with kernel("linear", "mfma32_8w"):
        q8.q8ta_linear(dev(c.x), c.in_scale, c.in_zp, wd, None, dev(c.weight_scales),
                       dev(c.bias), c.out_scale, c.out_zp, "relu", out)
        np.testing.assert_array_equal(host(out), ref)
        np.testing.assert_array_equal(_acc_linear(c), oracle.linear_acc(c.x, c.w, c.in_zp))
        q8.q8ta_linear_dq(dev(c.x), c.in_scale, c.in_zp, wd, None, dev(c.weight_scales),
                          dev(c.bias), c.out_scale, c.out_zp, "relu", outf)
        np.testing.assert_array_equal(host(outf).view(np.uint32), dq.view(np.uint32))
        out.zero_()
        q8.q8ta_linear_presummed(dev(c.x), c.in_scale, c.in_zp, wd, sums, dev(c.weight_scales),
                                 dev(c.bias), c.out_scale, c.out_zp, "relu", out)
        np.testing.assert_array_equal(host(out), ref)
        outf.zero_()
        q8.q8ta_linear_dq_presummed(dev(c.x), c.in_scale, c.in_zp, wd, sums,
                                    dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp,
                                    "relu", outf)
        np.testing.assert_array_equal(host(outf).view(np.uint32), dq.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 2048), (3, 4096), (1, 5136), (4, 48), (2, 16), (1, 4112),
                                 (1, 11008)])
def test_gemv_k_slices(M, K):
    """The skinny GEMM (M <= 4) and, for M == 1 from K = 2048, the kernel in
    which a workgroup owns 8 weight rows; K spans partial slices and several
    passes, N = 1001 leaves a partly filled last row group."""
    _say(f"gemv M={M} K={K}")
    c = qi.linear_case(78 + M + K, M, K, 1001)
    np.testing.assert_array_equal(_run_linear(c), _oracle_linear(c))
    np.testing.assert_array_equal(_acc_linear(c), oracle.linear_acc(c.x, c.w, c.in_zp))


def test_linear_gemv_entry_and_gemm_row_identity():
    """q8ta_linear_gemv is the M == 1 case: identical to q8ta_linear's row."""
    c = qi.linear_case(91, 8, 1024, 96)
    full = _run_linear(c)
    for m in (0, 5, 7):
        cm = qi.LinearCase(c.x[m:m + 1].copy(), c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                           c.out_scale, c.out_zp)
        np.testing.assert_array_equal(_run_linear(cm, fn=q8.q8ta_linear_gemv)[0], full[m])


def test_linear_gemv_rejects_m_gt_1():
    c = qi.linear_case(92, 2, 64, 8)
    with pytest.raises(q8.Q8taError, match="M must be 1"):
        _run_linear(c, fn=q8.q8ta_linear_gemv)


@pytest.mark.parametrize("M", [1, 8])
@pytest.mark.parametrize("out_scale", [0.272, 2.176, 1.0 / 3.0])
def test_linear_epilogue_on_rounding_ties(M, out_scale):
    """x == input zero point makes every accumulator 0, so the bias alone
    carries values placed on and beside every rounding tie through the
    kernel's epilogue (reciprocal in double, round half to even)."""
    grid = ((np.arange(-140, 141) + 0.5) * out_scale).astype(np.float32)
    b = np.concatenate([grid, np.nextafter(grid, np.float32(np.inf)),
                        np.nextafter(grid, np.float32(-np.inf))])
    N, K = b.size, 64
    g = qi.rng(17)
    c = qi.LinearCase(np.full((M, K), 3, np.int8), qi.w_int8(g, (N, K)), qi.scales(g, N), b,
                      0.02, 3, out_scale, -5)
    np.testing.assert_array_equal(_run_linear(c), _oracle_linear(c))


def test_linear_unaligned_pointers():
    c = qi.linear_case(93, 33, 256, 40)
    xb = torch.zeros(c.M * c.K + 1, dtype=torch.int8, device="cuda")
    xb[1:] = dev(c.x.reshape(-1))
    out = torch.empty((c.M, c.N), dtype=torch.int8, device="cuda")
    q8.q8ta_linear(xb[1:].view(c.M, c.K), c.in_scale, c.in_zp, dev(c.w), None,
                   dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, "none", out)
    np.testing.assert_array_equal(host(out), _oracle_linear(c))


def test_chain_small_workload():
    """quantize_per_tensor [4,64] -> q8ta_linear M=4 K=64 N=32."""
    c = qi.make_chain_small()
    xq = torch.empty((c.M, c.K), dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_per_tensor(dev(c.x_fp32), xq, c.in_scale, c.in_zp)
    ref_xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
    np.testing.assert_array_equal(host(xq), ref_xq)
    out = torch.empty((c.M, c.N), dtype=torch.int8, device="cuda")
    q8.q8ta_linear(xq, c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales), dev(c.bias),
                   c.out_scale, c.out_zp, "none", out)
    ref = oracle.linear(ref_xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                        c.out_zp)
    np.testing.assert_array_equal(host(out), ref)


def test_gemv_workload():
    c = qi.make_gemv()
    _say("gemv 1x4096x4096")
    np.testing.assert_array_equal(_run_linear(c), _oracle_linear(c))
    np.testing.assert_array_equal(_run_linear(c, fn=q8.q8ta_linear_gemv), _oracle_linear(c))
    np.testing.assert_array_equal(_acc_linear(c), oracle.linear_acc(c.x, c.w, c.in_zp))


_gemm_reference = {}


def _gemm_full_reference(c):
    """The oracle's whole int8 output of the 2048 x 4096 x 11008 workload
    (computed once per process)."""
    if "q" not in _gemm_reference:
        _gemm_reference["q"] = oracle.linear(c.x, c.w, c.weight_scales, c.bias, c.in_scale,
                                             c.in_zp, c.out_scale, c.out_zp)
    return _gemm_reference["q"]


@pytest.mark.parametrize("path", ["default"])
def test_gemm_workload_full(path):
    """GEMM M=2048 K=4096 N=11008 in the benchmark's launch configuration,
    every output element against the oracle, int8 (q8ta_linear) and fp32
    (q8ta_linear_dq)."""
    c = qi.make_gemm()
    _say(f"gemm full {path} 2048x4096x11008")
    ref = _gemm_full_reference(c)
    out = torch.empty((c.M, c.N), dtype=torch.int8, device="cuda")
    y = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    with kernel("linear", path):
        q8.q8ta_linear(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                       dev(c.bias), c.out_scale, c.out_zp, "none", out)
        q8.q8ta_linear_dq(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                          dev(c.bias), c.out_scale, c.out_zp, "none", y)
    np.testing.assert_array_equal(host(out), ref)
    dq = oracle.dequantize_per_tensor(ref, c.out_scale, c.out_zp)
    np.testing.assert_array_equal(host(y).view(np.uint32), dq.view(np.uint32))


def test_gemm_workload_sampled_rows_and_dequantize():
    """GEMM M=2048 K=4096 N=11008 in the benchmark's launch configuration:
    every output of 40 sampled rows (first, last and spread) is compared with
    the oracle; the dequantize of the whole int8 output is compared in full."""
    c = qi.make_gemm()
    _say("gemm 2048x4096x11008")
    out = torch.empty((c.M, c.N), dtype=torch.int8, device="cuda")
    q8.q8ta_linear(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                   dev(c.bias), c.out_scale, c.out_zp, "none", out)
    y = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    q8.q8ta_dequantize_per_tensor(out, y, c.out_scale, c.out_zp)
    got = host(out)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 1023, 2046, 2047],
                                     qi.rng(3).integers(0, c.M, 33)]))
    ref = oracle.linear(c.x[rows], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                        c.out_zp)
    np.testing.assert_array_equal(got[rows], ref)
    np.testing.assert_array_equal(host(y), oracle.dequantize_per_tensor(got, c.out_scale, c.out_zp))
    # the output scale keeps the codes mostly unsaturated
    assert (np.abs(got.astype(int)) < 127).mean() > 0.9


# ============================================================================ conv2d_transposed
def _run_deconv(c, bias=True, activation="none"):
    out = torch.empty((c.x.shape[0], c.w.shape[0], c.H_out, c.W_out), dtype=torch.int8, device="cuda")
    b = dev(c.bias) if (bias and c.bias is not None) else None
    q8.q8ta_conv2d_transposed(dev(c.x), c.in_scale, c.in_zp, dev(c.w), c.Kh, c.Kw, None,
                              dev(c.weight_scales), b, c.out_scale, c.out_zp, c.stride, c.padding,
                              c.output_padding, c.dilation, c.groups, activation, out)
    return host(out)


def _acc_deconv(c):
    acc = torch.empty((c.x.shape[0], c.w.shape[0], c.H_out, c.W_out), dtype=torch.int32, device="cuda")
    q8.q8ta_conv2d_transposed_acc(dev(c.x), c.in_zp, dev(c.w), c.Kh, c.Kw, c.stride, c.padding, acc,
                                  dilation=c.dilation, groups=c.groups)
    return host(acc)


def _oracle_deconv(c, bias=True, activation="none"):
    return oracle.conv2d_transposed(c.x, c.w, c.weight_scales, c.bias if bias else None, c.in_scale,
                                    c.in_zp, c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding,
                                    c.dilation, c.H_out, c.W_out, groups=c.groups,
                                    activation=activation)


def _oracle_deconv_acc(c):
    return oracle.deconv_acc(c.x, c.w, c.in_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation,
                             c.H_out, c.W_out, groups=c.groups)


DECONV_CASES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad, H_out, W_out, ldw_extra
    (1, 64, 32, 32, 32, 4, 4, (2, 2), (1, 1), (0, 0), None, None, 0),      # small workload shape
    (2, 32, 9, 12, 48, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 0),
    (1, 16, 5, 8, 20, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 32),       # padded weight rows
    (1, 48, 7, 6, 17, 4, 3, (2, 3), (1, 0), (0, 2), None, None, 0),        # mixed strides
    (1, 16, 6, 8, 16, 1, 1, (1, 1), (0, 0), (0, 0), None, None, 0),        # 1x1, stride 1
    (1, 32, 4, 8, 16, 5, 5, (3, 3), (2, 2), (1, 1), None, None, 0),        # stride 3
    (1, 16, 4, 4, 16, 2, 2, (4, 4), (0, 0), (0, 0), None, None, 0),        # phases with no taps
    (1, 64, 5, 20, 70, 3, 3, (2, 2), (4, 4), (0, 0), None, None, 0),       # pad > K
    (2, 32, 6, 7, 24, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 0),        # W_in % 4 != 0
    (1, 32, 8, 8, 32, 3, 3, (2, 2), (1, 1), (1, 1), 21, 9, 0),             # explicit H_out/W_out
    (1, 32, 8, 8, 32, 3, 3, (2, 2), (1, 1), (1, 1), 3, 40, 0),
    (1, 128, 16, 80, 96, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 0),     # several column tiles
    (1, 80, 6, 8, 40, 2, 2, (2, 2), (0, 0), (0, 0), None, None, 0),        # IC not a multiple of 64
    (1, 320, 3, 4, 24, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 0),
    (1, 24, 5, 6, 8, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 0),         # IC % 16 != 0 (general)
    (1, 16, 4, 4, 8, 3, 3, (5, 5), (1, 1), (0, 0), None, None, 0),         # stride 5 (general)
]


@pytest.mark.parametrize("case", DECONV_CASES, ids=[str(i) for i in range(len(DECONV_CASES))])
def test_deconv_parity(case):
    N, IC, H, W, OC, Kh, Kw, s, p, op, Ho, Wo, extra = case
    _say(f"deconv case={case}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, Kh, Kw]), N, IC, H, W, OC, Kh, Kw, s, p, op,
                       H_out=Ho, W_out=Wo, ldw=Kh * Kw * IC + extra)
    np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))
    np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))


# Shapes for the implicit-GEMM path (IC a multiple of 64): zero-point border on
# every side, output channels not a multiple of 32, phases without taps, tall
# and wide inputs, explicit (cropped) output sizes.
DECONV_IGEMM_CASES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad, H_out, W_out, ldw_extra
    (1, 64, 5, 7, 32, 4, 4, (2, 2), (1, 1), (0, 0), None, None, 0),
    (2, 64, 6, 5, 40, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 16),
    (1, 128, 4, 9, 64, 3, 3, (1, 1), (1, 1), (0, 0), None, None, 0),
    (1, 64, 3, 4, 96, 5, 3, (3, 2), (2, 0), (0, 0), None, None, 0),
    (1, 64, 7, 3, 8, 3, 5, (2, 3), (0, 2), (1, 1), None, None, 0),
    (1, 64, 33, 5, 33, 4, 4, (2, 2), (1, 1), (0, 0), None, None, 0),
    (1, 64, 4, 40, 32, 2, 2, (2, 2), (0, 0), (0, 0), None, None, 0),
    (1, 64, 3, 3, 16, 1, 1, (4, 4), (0, 0), (3, 3), None, None, 0),
    (1, 64, 5, 5, 32, 3, 3, (2, 2), (1, 1), (1, 1), 7, 6, 0),
    (3, 192, 9, 70, 130, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 64),
]


@pytest.mark.parametrize("case", DECONV_IGEMM_CASES,
                         ids=[str(i) for i in range(len(DECONV_IGEMM_CASES))])
@pytest.mark.parametrize("path", ["igemm", "tiled", "mfma"])
def test_deconv_igemm_parity(case, path):
    N, IC, H, W, OC, Kh, Kw, s, p, op, Ho, Wo, extra = case
    _say(f"deconv {path} case={case}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, Kh, Kw]) + 1, N, IC, H, W, OC, Kh, Kw, s, p, op,
                       H_out=Ho, W_out=Wo, ldw=Kh * Kw * IC + extra)
    with kernel("conv2d_transposed", path):
        np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))
        np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))


# Shapes that reach each tile plan of the matrix-core transposed conv: phase
# columns per wave (16, 32, 64: W_out / stride below 32, below 64, at least
# 64), output-channel fragments per wave (OC below 32 or not), and the
# one-fragment plan for problems that leave the chip mostly idle.
DECONV_PLAN_SHAPES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad   (256 workgroups or more unless noted)
    (8, 32, 64, 24, 16, 3, 3, (2, 2), (1, 1), (1, 1)),    # 24 phase columns, OC 16
    (8, 32, 64, 40, 48, 3, 3, (2, 2), (1, 1), (1, 1)),    # 40 phase columns, 2 fragments
    (8, 32, 64, 70, 40, 3, 3, (2, 2), (1, 1), (1, 1)),    # 70 phase columns
    (2, 64, 10, 36, 72, 3, 3, (2, 2), (1, 1), (1, 1)),    # 24 workgroups: one-fragment plan
]


@pytest.mark.parametrize("shape", DECONV_PLAN_SHAPES, ids=[str(i) for i in range(4)])
def test_deconv_every_tile(shape):
    _say(f"deconv tile plan shape={shape}")
    c = qi.deconv_case(500 + sum(shape[:5]), *shape)
    with kernel("conv2d_transposed", "mfma"):
        np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))
        np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))


@pytest.mark.parametrize("case", [DECONV_CASES[1], DECONV_CASES[3], DECONV_CASES[6], DECONV_CASES[11],
                                  DECONV_CASES[13]],
                         ids=["k3s2", "mixed_strides", "empty_phases", "wide", "ic320"])
def test_deconv_tiled_kernel(case):
    N, IC, H, W, OC, Kh, Kw, s, p, op, Ho, Wo, extra = case
    _say(f"deconv tiled case={case}")
    c = qi.deconv_case(7 + 8 + 1, N, IC, H, W, OC, Kh, Kw, s, p, op, H_out=Ho,
                       W_out=Wo, ldw=Kh * Kw * IC + extra)
    with kernel("conv2d_transposed", "tiled"):
        np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))
        np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))


# Shapes the 32x32x32 matrix-core transposed conv takes (IC % 32 == 0,
# W_in % 4 == 0, strides up to 2): several channel tiles and a partly empty
# last one, ragged column tiles, one-sided strides, dilation, phases without
# taps, padding beyond the kernel, cropped and enlarged outputs, IC not a
# multiple of 64, and a padded weight row.
DECONV_MX_CASES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad, dilation, H_out, W_out, ldw_extra
    (2, 64, 12, 20, 160, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), None, None, 0),
    (1, 96, 9, 36, 33, 4, 4, (2, 2), (1, 1), (0, 0), (1, 1), None, None, 32),
    (1, 32, 7, 16, 40, 3, 3, (1, 2), (1, 1), (0, 1), (1, 1), None, None, 0),
    (1, 64, 6, 16, 48, 3, 4, (2, 1), (0, 2), (1, 0), (1, 1), None, None, 0),
    (1, 64, 5, 136, 48, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), None, None, 0),
    (1, 64, 8, 12, 32, 3, 3, (2, 2), (2, 2), (1, 1), (2, 2), None, None, 0),
    (1, 32, 5, 8, 32, 1, 1, (2, 2), (0, 0), (1, 1), (1, 1), None, None, 0),
    (2, 128, 6, 8, 64, 5, 5, (2, 2), (4, 4), (1, 1), (1, 1), None, None, 0),
    (1, 64, 8, 8, 32, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), 9, 21, 0),
    (1, 32, 4, 12, 24, 4, 4, (2, 2), (1, 1), (0, 0), (1, 1), 12, 40, 0),
    (2, 256, 5, 16, 128, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), None, None, 16),
    (1, 64, 32, 32, 32, 4, 4, (2, 2), (1, 1), (0, 0), (1, 1), None, None, 0),
]


@pytest.mark.parametrize("case", DECONV_MX_CASES, ids=[str(i) for i in range(len(DECONV_MX_CASES))])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_deconv_mfma32_parity(case, act):
    N, IC, H, W, OC, Kh, Kw, s, p, op, d, Ho, Wo, extra = case
    _say(f"deconv mfma32 case={case} act={act}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, Kh, Kw]) + 31, N, IC, H, W, OC, Kh, Kw, s, p, op,
                       H_out=Ho, W_out=Wo, ldw=Kh * Kw * IC + extra, dilation=d)
    with kernel("conv2d_transposed", "mfma32"):
        np.testing.assert_array_equal(_run_deconv(c, activation=act),
                                      _oracle_deconv(c, activation=act))
        if act == "none":
            np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))
            np.testing.assert_array_equal(_run_deconv(c, bias=False), _oracle_deconv(c, bias=False))


CONV2D_MX_CASES = [
    # N, IC, H, W, OC, Kh, Kw, pad, dil, ldw_extra
    (2, 64, 10, 12, 40, 3, 3, (1, 1), (1, 1), 0),
    (1, 32, 7, 16, 160, 5, 5, (2, 2), (1, 1), 16),
    (1, 64, 9, 8, 48, 3, 3, (2, 2), (2, 2), 0),
    (1, 128, 7, 40, 64, 1, 1, (0, 0), (1, 1), 0),
    (1, 96, 6, 132, 32, 3, 3, (0, 1), (1, 1), 0),
    (2, 256, 8, 8, 128, 3, 3, (1, 1), (1, 1), 0),
]


@pytest.mark.parametrize("case", CONV2D_MX_CASES, ids=[str(i) for i in range(len(CONV2D_MX_CASES))])
def test_conv2d_mfma32_parity(case):
    N, IC, H, W, OC, Kh, Kw, p, d, extra = case
    _say(f"conv2d mfma32 case={case}")
    c = qi.conv_case(sum([N, IC, H, W, OC, Kh, Kw]) + 41, N, IC, H, W, OC, Kh, Kw, (1, 1), p, d,
                     ldw=Kh * Kw * IC + extra)
    with kernel("conv2d", "mfma32"):
        np.testing.assert_array_equal(_run_conv(c), _oracle_conv(c))
        np.testing.assert_array_equal(_acc_conv(c), oracle.conv2d_acc(
            c.x, c.w, c.in_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation, c.H_out, c.W_out))
        np.testing.assert_array_equal(_run_conv(c, activation="relu"),
                                      _oracle_conv(c, activation="relu"))


# Shapes the compile-time-pattern transposed conv takes (3x3 and 4x4, stride
# 2, IC % 64 == 0, W_in % 4 == 0): several channel tiles (the last partly
# empty), OC not a multiple of 32, several and ragged column tiles with
# byte-wise stores, both parities of the padding, odd output sizes, a padded
# weight row.
DECONV_FIXED_CASES = [
    # N, IC, H, W, OC, K, pad, out_pad
    (2, 64, 12, 20, 160, 3, (1, 1), (1, 1)),
    (1, 128, 9, 36, 33, 4, (1, 1), (0, 0)),
    (1, 64, 7, 136, 48, 3, (0, 0), (1, 1)),
    (1, 64, 6, 16, 64, 4, (2, 2), (0, 0)),
    (2, 192, 5, 12, 130, 3, (2, 2), (1, 1)),
    (1, 64, 8, 8, 32, 4, (3, 3), (1, 1)),
    (1, 64, 32, 32, 32, 4, (1, 1), (0, 0)),
]


@pytest.mark.parametrize("case", DECONV_FIXED_CASES, ids=[str(i) for i in range(len(DECONV_FIXED_CASES))])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_deconv_fixed_parity(case, act):
    N, IC, H, W, OC, K, p, op = case
    _say(f"deconv fixed case={case} act={act}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, K]) + 61, N, IC, H, W, OC, K, K, (2, 2), p, op,
                       ldw=K * K * IC + 16)
    with kernel("conv2d_transposed", "fixed"):
        np.testing.assert_array_equal(_run_deconv(c, activation=act),
                                      _oracle_deconv(c, activation=act))
        if act == "none":
            np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))
            np.testing.assert_array_equal(_run_deconv(c, bias=False), _oracle_deconv(c, bias=False))


@pytest.mark.parametrize("case", DECONV_FIXED_CASES, ids=[str(i) for i in range(len(DECONV_FIXED_CASES))])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_quantize_deconv_fixed_parity(case, act):
    """The fused quantize -> transposed conv on the compile-time-pattern
    kernel, which quantizes the fp32 input while it stages the halo."""
    N, IC, H, W, OC, K, p, op = case
    _say(f"quantize+deconv fixed case={case} act={act}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, K]) + 67, N, IC, H, W, OC, K, K, (2, 2), p, op,
                       ldw=K * K * IC + 16, x_from_fp32=True)
    out = torch.empty((N, OC, c.H_out, c.W_out), dtype=torch.int8, device="cuda")
    with kernel("conv2d_transposed", "fixed"):
        q8.q8ta_quantize_conv2d_transposed(dev(c.x_fp32), c.in_scale, c.in_zp, dev(c.w), c.Kh,
                                           c.Kw, None, dev(c.weight_scales), dev(c.bias),
                                           c.out_scale, c.out_zp, c.stride, c.padding,
                                           c.output_padding, (1, 1), 1, act, out)
    xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
    ref = oracle.conv2d_transposed(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                                   c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding, (1, 1),
                                   c.H_out, c.W_out, activation=act)
    np.testing.assert_array_equal(host(out), ref)


def _deconv_pack_reference(w, OC, IC, K):
    """The prepacked transposed-conv weight written out from the header's
    formula: byte 16 l + j of fragment (ob, kh, kw, kc) is
    w[32 ob + l % 32, (kh K + kw) IC + 32 kc + 16 (l // 32) + j], zero past OC."""
    nob, nk = -(-OC // 32), IC // 32
    out = np.zeros((nob, K, K, nk, 64, 16), np.int8)
    for ob in range(nob):
        for kh in range(K):
            for kw in range(K):
                for kc in range(nk):
                    for l in range(64):
                        row = 32 * ob + l % 32
                        if row < OC:
                            s0 = (kh * K + kw) * IC + 32 * kc + 16 * (l // 32)
                            out[ob, kh, kw, kc, l] = w[row, s0:s0 + 16]
    return out.reshape(-1)


def _deconv_prepack(c):
    OC, IC, K = c.w.shape[0], c.x.shape[1], c.Kh
    packed = torch.empty(q8.q8ta_conv2d_transposed_weight_prepacked_bytes(OC, IC, K, K),
                         dtype=torch.int8, device="cuda")
    q8.q8ta_conv2d_transposed_weight_prepack(dev(c.w), IC, K, K, packed)
    return packed


@pytest.mark.parametrize("case", DECONV_FIXED_CASES, ids=[str(i) for i in range(len(DECONV_FIXED_CASES))])
@pytest.mark.parametrize("act", ["none", "relu"])
def test_deconv_prepacked_parity(case, act):
    """q8ta_conv2d_transposed_weight_prepack writes the header's layout, and
    q8ta_conv2d_transposed_prepacked on it equals the oracle (padded weight
    rows, OC not a multiple of 32 or 128, several column tiles)."""
    N, IC, H, W, OC, K, p, op = case
    _say(f"deconv prepacked case={case} act={act}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, K]) + 61, N, IC, H, W, OC, K, K, (2, 2), p, op,
                       ldw=K * K * IC + 16)
    packed = _deconv_prepack(c)
    np.testing.assert_array_equal(host(packed), _deconv_pack_reference(c.w, OC, IC, K))
    out = torch.empty((N, OC, c.H_out, c.W_out), dtype=torch.int8, device="cuda")
    q8.q8ta_conv2d_transposed_prepacked(dev(c.x), c.in_scale, c.in_zp, packed, OC, K, K, None,
                                        dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp,
                                        c.stride, c.padding, c.output_padding, (1, 1), 1, act, out)
    np.testing.assert_array_equal(host(out), _oracle_deconv(c, activation=act))


@pytest.mark.parametrize("case", DECONV_FIXED_CASES, ids=[str(i) for i in range(len(DECONV_FIXED_CASES))])
def test_quantize_deconv_prepacked_parity(case):
    """q8ta_quantize_conv2d_transposed_prepacked: the fp32 input quantized in
    the same call, on the packed weight, against the oracle's chain."""
    N, IC, H, W, OC, K, p, op = case
    _say(f"quantize+deconv prepacked case={case}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, K]) + 67, N, IC, H, W, OC, K, K, (2, 2), p, op,
                       ldw=K * K * IC + 16, x_from_fp32=True)
    packed = _deconv_prepack(c)
    out = torch.empty((N, OC, c.H_out, c.W_out), dtype=torch.int8, device="cuda")
    q8.q8ta_conv2d_transposed_prepacked(dev(c.x_fp32), c.in_scale, c.in_zp, packed, OC, K, K, None,
                                        dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp,
                                        c.stride, c.padding, c.output_padding, (1, 1), 1, "relu",
                                        out)
    xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
    ref = oracle.conv2d_transposed(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                                   c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding, (1, 1),
                                   c.H_out, c.W_out, activation="relu")
    np.testing.assert_array_equal(host(out), ref)


def test_deconv_prepacked_large_workload_full():
    """[8,256,64,64] -> [8,128,128,128] on the prepacked weight, every output
    against the oracle."""
    c, xq_ref, ref = _c5_reference()
    _say("deconv prepacked [8,256,64,64] -> [8,128,128,128], full output")
    packed = _deconv_prepack(c)
    out = torch.empty((8, 128, 128, 128), dtype=torch.int8, device="cuda")
    q8.q8ta_conv2d_transposed_prepacked(dev(xq_ref), c.in_scale, c.in_zp, packed, 128, c.Kh, c.Kw,
                                        None, dev(c.weight_scales), dev(c.bias), c.out_scale,
                                        c.out_zp, c.stride, c.padding, c.output_padding, (1, 1), 1,
                                        "none", out)
    np.testing.assert_array_equal(host(out), ref)
    out.zero_()
    q8.q8ta_conv2d_transposed_prepacked(dev(c.x_fp32), c.in_scale, c.in_zp, packed, 128, c.Kh,
                                        c.Kw, None, dev(c.weight_scales), dev(c.bias), c.out_scale,
                                        c.out_zp, c.stride, c.padding, c.output_padding, (1, 1), 1,
                                        "none", out)
    np.testing.assert_array_equal(host(out), ref)


CONV2D_FIXED_CASES = [
    # N, IC, H, W, OC, pad
    (2, 64, 10, 12, 40, (1, 1)),
    (1, 128, 7, 132, 160, (0, 1)),
    (2, 256, 8, 8, 128, (1, 1)),
    (1, 64, 9, 8, 48, (2, 2)),
]


@pytest.mark.parametrize("case", CONV2D_FIXED_CASES, ids=[str(i) for i in range(len(CONV2D_FIXED_CASES))])
def test_conv2d_fixed_parity(case):
    N, IC, H, W, OC, p = case
    _say(f"conv2d fixed case={case}")
    c = qi.conv_case(sum([N, IC, H, W, OC]) + 71, N, IC, H, W, OC, 3, 3, (1, 1), p, (1, 1))
    with kernel("conv2d", "fixed"):
        np.testing.assert_array_equal(_run_conv(c), _oracle_conv(c))
        np.testing.assert_array_equal(_acc_conv(c), oracle.conv2d_acc(
            c.x, c.w, c.in_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation, c.H_out, c.W_out))
        np.testing.assert_array_equal(_run_conv(c, activation="relu"),
                                      _oracle_conv(c, activation="relu"))


def test_deconv_epilogue_on_rounding_ties():
    """x == input zero point everywhere: the accumulator is 0 and the bias (one
    value per output channel, on and beside rounding ties) is requantized."""
    out_scale = 0.272
    grid = ((np.arange(-140, 141) + 0.5) * out_scale).astype(np.float32)
    b = np.concatenate([grid, np.nextafter(grid, np.float32(np.inf))])
    OC = b.size
    c = qi.deconv_case(23, 1, 16, 4, 4, OC, 3, 3, (2, 2), (1, 1), (1, 1))
    c.x[...] = 3
    c.bias = b
    c.out_scale = out_scale
    np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))


@pytest.mark.parametrize("izp", [-128, 127])
def test_deconv_zero_points_and_no_bias(izp):
    c = qi.deconv_case(600 + izp, 1, 32, 8, 8, 24, 3, 3, (2, 2), (1, 1), (1, 1), in_zp=izp)
    np.testing.assert_array_equal(_run_deconv(c, bias=False), _oracle_deconv(c, bias=False))
    np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))


def test_deconv_small_workload():
    c = qi.make_deconv_small()
    _say("deconv [1,64,32,32] -> [1,32,64,64]")
    np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))


_C5_REF = {}


def _c5_reference():
    """The oracle's quantize and transposed conv of the large workload, over
    every output (computed once per test session)."""
    if not _C5_REF:
        c = qi.make_deconv_large()
        xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
        ref = oracle.conv2d_transposed(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                                       c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding,
                                       (1, 1), c.H_out, c.W_out)
        _C5_REF.update(c=c, xq=xq, ref=ref)
    return _C5_REF["c"], _C5_REF["xq"], _C5_REF["ref"]


def test_deconv_large_workload_full():
    """quantize [8,256,64,64] -> deconv -> [8,128,128,128] in the benchmark's
    launch configuration, every output compared with the oracle."""
    c, xq_ref, ref = _c5_reference()
    _say("quantize + deconv [8,256,64,64] -> [8,128,128,128], full output")
    xq = torch.empty(c.x_fp32.shape, dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_per_tensor(dev(c.x_fp32), xq, c.in_scale, c.in_zp)
    out = torch.empty((8, 128, 128, 128), dtype=torch.int8, device="cuda")
    q8.q8ta_conv2d_transposed(xq, c.in_scale, c.in_zp, dev(c.w), c.Kh, c.Kw, None,
                              dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, c.stride,
                              c.padding, c.output_padding, (1, 1), 1, "none", out)
    np.testing.assert_array_equal(host(xq), xq_ref)
    got = host(out)
    np.testing.assert_array_equal(got, ref)
    assert (np.abs(got.astype(int)) < 127).mean() > 0.9


# ============================================================================ forward conv2d
def _run_conv(c, bias=True, activation="none"):
    out = torch.empty((c.x.shape[0], c.w.shape[0], c.H_out, c.W_out), dtype=torch.int8, device="cuda")
    b = dev(c.bias) if (bias and c.bias is not None) else None
    q8.q8ta_conv2d(dev(c.x), c.in_scale, c.in_zp, dev(c.w), c.Kh, c.Kw, None,
                   dev(c.weight_scales), b, c.out_scale, c.out_zp, c.stride, c.padding,
                   c.dilation, getattr(c, "groups", 1), activation, out)
    return host(out)


def _acc_conv(c):
    acc = torch.empty((c.x.shape[0], c.w.shape[0], c.H_out, c.W_out), dtype=torch.int32, device="cuda")
    q8.q8ta_conv2d_acc(dev(c.x), c.in_zp, dev(c.w), c.Kh, c.Kw, c.stride, c.padding, c.dilation,
                       acc, groups=getattr(c, "groups", 1))
    return host(acc)


def _oracle_conv(c, bias=True, activation="none"):
    return oracle.conv2d(c.x, c.w, c.weight_scales, c.bias if bias else None, c.in_scale, c.in_zp,
                         c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation,
                         c.H_out, c.W_out, groups=getattr(c, "groups", 1), activation=activation)


CONV2D_CASES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, dil, H_out, W_out, ldw_extra
    (1, 64, 9, 11, 32, 3, 3, (1, 1), (1, 1), (1, 1), None, None, 0),
    (2, 64, 10, 9, 40, 3, 3, (2, 2), (1, 1), (1, 1), None, None, 16),     # OC % 32 != 0
    (1, 128, 7, 40, 64, 1, 1, (1, 1), (0, 0), (1, 1), None, None, 0),     # pointwise
    (1, 64, 9, 9, 16, 3, 2, (1, 2), (2, 0), (2, 3), None, None, 0),       # dilation, mixed strides
    (1, 64, 12, 70, 33, 5, 5, (3, 2), (2, 2), (1, 1), None, None, 0),     # several column tiles
    (1, 64, 4, 5, 32, 3, 3, (1, 1), (4, 3), (1, 1), None, None, 0),       # pad larger than K
    (1, 64, 6, 6, 32, 3, 3, (1, 1), (1, 1), (1, 1), 4, 9, 0),             # explicit output size
    (3, 192, 17, 33, 130, 3, 3, (1, 1), (1, 1), (1, 1), None, None, 64),
    (1, 24, 7, 7, 8, 3, 3, (1, 1), (1, 1), (1, 1), None, None, 0),        # IC % 64 != 0 (general)
    (1, 3, 16, 16, 16, 7, 7, (2, 2), (3, 3), (1, 1), None, None, 0),      # stem-like (general)
]


@pytest.mark.parametrize("case", CONV2D_CASES, ids=[str(i) for i in range(len(CONV2D_CASES))])
@pytest.mark.parametrize("path", ["mfma", "igemm"])
def test_conv2d_parity(case, path):
    N, IC, H, W, OC, Kh, Kw, s, p, d, Ho, Wo, extra = case
    _say(f"conv2d path={path} case={case}")
    c = qi.conv_case(sum([N, IC, H, W, OC, Kh, Kw]) + 2, N, IC, H, W, OC, Kh, Kw, s, p, d,
                     H_out=Ho, W_out=Wo, ldw=Kh * Kw * IC + extra)
    with kernel("conv2d", path):
        np.testing.assert_array_equal(_run_conv(c), _oracle_conv(c))
        np.testing.assert_array_equal(_acc_conv(c), oracle.conv2d_acc(
            c.x, c.w, c.in_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation, c.H_out, c.W_out))


@pytest.mark.parametrize("izp", [-128, 127, 0])
def test_conv2d_zero_points_and_no_bias(izp):
    c = qi.conv_case(700 + izp, 1, 64, 8, 8, 24, 3, 3, (1, 1), (1, 1), (1, 1), in_zp=izp)
    np.testing.assert_array_equal(_run_conv(c, bias=False), _oracle_conv(c, bias=False))
    np.testing.assert_array_equal(_run_conv(c), _oracle_conv(c))


def test_conv2d_large_workload_sampled():
    """[8,256,64,64] K3 s1 p1 -> [8,128,64,64] in the benchmark's launch
    configuration; the oracle recomputes images 0 and 7 for 24 output channels."""
    c = qi.make_conv2d_large()
    _say("conv2d [8,256,64,64] -> [8,128,64,64]")
    got = _run_conv(c)
    chans = np.array(sorted(set([0, 1, 2, 63, 64, 65, 126, 127] + list(range(5, 128, 8)))))[:24]
    for n in (0, 7):
        ref = oracle.conv2d(c.x[n:n + 1], c.w[chans], c.weight_scales[chans], c.bias[chans],
                            c.in_scale, c.in_zp, c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride,
                            c.padding, c.dilation, c.H_out, c.W_out)
        np.testing.assert_array_equal(got[n:n + 1, chans], ref)


GROUPED_CASES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, dil, groups, H_out, W_out
    (1, 64, 9, 11, 64, 3, 3, (1, 1), (1, 1), (1, 1), 64, None, None),    # depthwise
    (2, 32, 10, 9, 32, 3, 3, (2, 2), (1, 1), (1, 1), 32, None, None),    # depthwise, strided
    (1, 16, 9, 9, 16, 5, 5, (1, 2), (2, 2), (2, 1), 16, None, None),     # depthwise, dilated
    (1, 12, 13, 5, 12, 3, 2, (1, 1), (0, 1), (1, 1), 12, None, None),    # W_out % 4 != 0
    (1, 16, 6, 6, 16, 3, 3, (1, 1), (1, 1), (1, 1), 16, 4, 9),           # explicit output size
    (1, 16, 11, 13, 16, 5, 5, (1, 1), (2, 2), (1, 1), 16, None, None),   # depthwise 5x5
    (1, 16, 12, 9, 16, 5, 5, (2, 2), (2, 2), (1, 1), 16, None, None),    # depthwise 5x5 s2
    (2, 8, 7, 10, 8, 3, 3, (2, 2), (0, 0), (1, 1), 8, None, None),       # depthwise 3x3 s2 p0
    (1, 8, 9, 9, 8, 3, 3, (1, 1), (1, 1), (1, 1), 8, 11, 5),             # output past the input
    (1, 8, 7, 6, 16, 3, 3, (1, 1), (1, 1), (1, 1), 8, None, None),       # channel multiplier 2
    (2, 64, 8, 8, 32, 3, 3, (1, 1), (1, 1), (1, 1), 4, None, None),      # grouped
    # wide rows (W % 16 == 0), large planes, outputs past the input
    (2, 8, 9, 16, 8, 3, 3, (1, 1), (1, 1), (1, 1), 8, None, None),       # ragged last block
    (1, 4, 5, 32, 4, 5, 5, (1, 1), (2, 2), (1, 1), 4, None, None),       # 5x5, W 32
    (1, 4, 8, 16, 4, 3, 3, (1, 1), (1, 1), (1, 1), 4, 11, 20),           # output past the input
    (1, 4, 4, 16, 4, 3, 3, (1, 1), (3, 3), (1, 1), 4, None, None),       # pad larger than K
    (1, 2, 128, 128, 2, 3, 3, (1, 1), (1, 1), (1, 1), 2, None, None),    # 128 x 128 plane
    (1, 2, 129, 128, 2, 3, 3, (1, 1), (1, 1), (1, 1), 2, None, None),    # 129 x 128 plane
    (1, 3, 16, 48, 3, 3, 3, (1, 1), (0, 0), (1, 1), 3, None, None),      # p0, W_out % 4 != 0
]


@pytest.mark.parametrize("case", GROUPED_CASES, ids=[str(i) for i in range(len(GROUPED_CASES))])
def test_grouped_conv2d_parity(case):
    N, IC, H, W, OC, Kh, Kw, s, p, d, G, Ho, Wo = case
    _say(f"grouped conv2d case={case}")
    c = qi.conv_case(sum([N, IC, H, W, OC, Kh, Kw, G]), N, IC, H, W, OC, Kh, Kw, s, p, d,
                     H_out=Ho, W_out=Wo, groups=G)
    np.testing.assert_array_equal(_run_conv(c), _oracle_conv(c))
    np.testing.assert_array_equal(_acc_conv(c), oracle.conv2d_acc(
        c.x, c.w, c.in_zp, c.Kh, c.Kw, c.stride, c.padding, c.dilation, c.H_out, c.W_out,
        groups=G))


def test_depthwise_large_workload():
    """[8,256,64,64] depthwise 3x3 s1 p1, every output against the oracle."""
    c = qi.make_depthwise_large()
    _say("depthwise [8,256,64,64]")
    np.testing.assert_array_equal(_run_conv(c), _oracle_conv(c))


# ============================================================================ fused chains
DQ_SHAPES = [(1, 4096, 4096), (3, 48, 17), (4, 64, 32), (65, 320, 97), (300, 1040, 257),
             (129, 2064, 129), (7, 33, 5), (40, 100, 70), (64, 128, 64)]


@pytest.mark.parametrize("M,K,N", DQ_SHAPES)
@pytest.mark.parametrize("path", ["default", "mfma32", "mfma32_8w", "generic"])
def test_linear_dq_equals_linear_then_dequantize(M, K, N, path):
    """q8ta_linear_dq == dequantize_per_tensor(q8ta_linear(...)) bit for bit,
    against the oracle's two steps (default and shape-general kernels)."""
    _say(f"linear_dq {path} M={M} K={K} N={N}")
    c = qi.linear_case(M * 3 + K + N, M, K, N)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    with kernel("linear", path):
        q8.q8ta_linear_dq(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                          dev(c.bias), c.out_scale, c.out_zp, "none", out)
    ref = oracle.dequantize_per_tensor(_oracle_linear(c), c.out_scale, c.out_zp)
    np.testing.assert_array_equal(host(out).view(np.uint32), ref.view(np.uint32))


def test_linear_dq_gemm_workload_sampled():
    c = qi.make_gemm()
    _say("linear_dq 2048x4096x11008")
    out = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    q8.q8ta_linear_dq(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                      dev(c.bias), c.out_scale, c.out_zp, "none", out)
    got = host(out)
    rows = np.array([0, 1, 2, 511, 1024, 1025, 2046, 2047])
    q = oracle.linear(c.x[rows], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                      c.out_zp)
    ref = oracle.dequantize_per_tensor(q, c.out_scale, c.out_zp)
    np.testing.assert_array_equal(got[rows].view(np.uint32), ref.view(np.uint32))


# M <= 4 with K % 16 == 0: quantized inside the weight-streaming kernel; the
# rest (ragged K, M > 4, the GEMM shapes) through the int8 workspace.
QLIN_SHAPES = [(1, 4096, 4096), (4, 5136, 33), (2, 48, 17), (3, 1040, 300), (1, 4112, 7),
               (4, 36, 9), (5, 64, 32), (65, 320, 97), (300, 1040, 257), (7, 33, 5)]


@pytest.mark.parametrize("M,K,N", QLIN_SHAPES)
@pytest.mark.parametrize("act", ["none", "relu"])
def test_quantize_linear_equals_the_chain(M, K, N, act):
    """q8ta_quantize_linear == q8ta_linear(quantize_per_tensor(x)) and
    q8ta_quantize_linear_dq == dequantize of it, bit for bit, against the
    oracle's steps; fp32 inputs include values beyond the int8 range so that
    the quantize clamps."""
    _say(f"quantize+linear M={M} K={K} N={N} act={act}")
    g = qi.rng(M * 7 + K + N)
    c = qi.linear_case(M * 5 + K + N, M, K, N)
    xf = (qi.x_fp32(g, (M, K)) * 1.5).astype(np.float32)
    xf.flat[:: 7] *= 3.0
    xq = oracle.quantize_per_tensor(xf, c.in_scale, c.in_zp)
    ref = oracle.linear(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                        c.out_zp, activation=act)
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_linear(dev(xf), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                            dev(c.bias), c.out_scale, c.out_zp, act, out)
    np.testing.assert_array_equal(host(out), ref)
    outf = torch.empty((M, N), dtype=torch.float32, device="cuda")
    q8.q8ta_quantize_linear_dq(dev(xf), c.in_scale, c.in_zp, dev(c.w), None,
                               dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, act, outf)
    refd = oracle.dequantize_per_tensor(ref, c.out_scale, c.out_zp)
    np.testing.assert_array_equal(host(outf).view(np.uint32), refd.view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(1, 5136, 33), (2, 4112, 7), (3, 48, 301), (4, 8192, 65)])
def test_quantize_linear_skinny_shapes(M, K, N):
    """The fp32-activation skinny kernel (one weight row per wave for M = 1,
    four for M > 1; ragged N, K chunks with masked slices) against the
    oracle's quantize -> linear."""
    _say(f"quantize+linear M={M} K={K} N={N}")
    c = qi.linear_case(M * 11 + K + N, M, K, N)
    xf = (qi.x_fp32(qi.rng(K + N), (M, K)) * 2.0).astype(np.float32)
    xq = oracle.quantize_per_tensor(xf, c.in_scale, c.in_zp)
    ref = oracle.linear(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                        c.out_zp)
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_linear(dev(xf), c.in_scale, c.in_zp, dev(c.w), None,
                            dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, "none", out)
    np.testing.assert_array_equal(host(out), ref)


def test_quantize_linear_chain_small_workload():
    """The small chain workload (quantize [4,64] -> linear 4x64x32) in one call."""
    c = qi.make_chain_small()
    _say("quantize+linear chain_small")
    xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
    ref = oracle.linear(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                        c.out_zp)
    out = torch.empty((c.M, c.N), dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_linear(dev(c.x_fp32), c.in_scale, c.in_zp, dev(c.w), None,
                            dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, "none", out)
    np.testing.assert_array_equal(host(out), ref)


def test_quantize_linear_dq_gemm_workload_sampled():
    """fp32 [2048, 4096] -> quantize -> 2048 x 4096 x 11008 GEMM -> dequantize,
    sampled rows against the oracle."""
    c = qi.make_gemm()
    _say("quantize+linear_dq 2048x4096x11008")
    xf = qi.x_fp32(qi.rng(2024), (c.M, c.K))
    out = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    q8.q8ta_quantize_linear_dq(dev(xf), c.in_scale, c.in_zp, dev(c.w), None,
                               dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, "none",
                               out)
    got = host(out)
    rows = np.array([0, 1, 1023, 2047])
    xq = oracle.quantize_per_tensor(xf[rows], c.in_scale, c.in_zp)
    q = oracle.linear(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                      c.out_zp)
    ref = oracle.dequantize_per_tensor(q, c.out_scale, c.out_zp)
    np.testing.assert_array_equal(got[rows].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("case", [DECONV_CASES[1], DECONV_CASES[3], DECONV_IGEMM_CASES[1],
                                  DECONV_IGEMM_CASES[5], DECONV_CASES[14]],
                         ids=["k3s2", "mixed", "igemm_oc40", "igemm_tall", "general"])
@pytest.mark.parametrize("path", ["igemm", "tiled", "mfma"])
def test_quantize_conv2d_transposed_equals_the_chain(case, path):
    N, IC, H, W, OC, Kh, Kw, s, p, op, Ho, Wo, extra = case
    _say(f"quantize+deconv {path} case={case}")
    c = qi.deconv_case(sum([N, IC, H, W, OC]) + 5, N, IC, H, W, OC, Kh, Kw, s, p, op, H_out=Ho,
                       W_out=Wo, ldw=Kh * Kw * IC + extra, x_from_fp32=True)
    out = torch.empty((N, OC, c.H_out, c.W_out), dtype=torch.int8, device="cuda")
    with kernel("conv2d_transposed", path):
        q8.q8ta_quantize_conv2d_transposed(dev(c.x_fp32), c.in_scale, c.in_zp, dev(c.w), c.Kh,
                                           c.Kw, None, dev(c.weight_scales), dev(c.bias),
                                           c.out_scale, c.out_zp, c.stride, c.padding,
                                           c.output_padding, (1, 1), 1, "none", out)
    xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
    ref = oracle.conv2d_transposed(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                                   c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding, (1, 1),
                                   c.H_out, c.W_out)
    np.testing.assert_array_equal(host(out), ref)


def test_quantize_conv2d_transposed_large_workload_full():
    """The fused quantize -> transposed conv on the large workload, every
    output compared with the oracle's quantize then transposed conv."""
    c, _, ref = _c5_reference()
    _say("quantize+deconv fused [8,256,64,64] -> [8,128,128,128], full output")
    out = torch.empty((8, 128, 128, 128), dtype=torch.int8, device="cuda")
    q8.q8ta_quantize_conv2d_transposed(dev(c.x_fp32), c.in_scale, c.in_zp, dev(c.w), c.Kh, c.Kw,
                                       None, dev(c.weight_scales), dev(c.bias), c.out_scale,
                                       c.out_zp, c.stride, c.padding, c.output_padding, (1, 1), 1,
                                       "none", out)
    np.testing.assert_array_equal(host(out), ref)


@pytest.mark.parametrize("path", ["mfma", "igemm", "tiled"])
def test_workspace_reuse_across_calls_and_streams(path):
    """Calls that need scratch memory, queued back to back without a host
    synchronization: small, larger (the stream's buffer grows), small again,
    and one on a second stream.  Every result is checked after one final
    synchronization."""
    _say(f"workspace reuse {path}")
    shapes = [(1, 32, 6, 5, 16), (2, 64, 13, 11, 32), (1, 16, 4, 9, 16)]
    cases = [qi.deconv_case(940 + i, n, ic, h, w, oc, 3, 3, (2, 2), (1, 1), (1, 1),
                            x_from_fp32=True) for i, (n, ic, h, w, oc) in enumerate(shapes)]
    side = torch.cuda.Stream()
    keep, outs = [], []
    with kernel("conv2d_transposed", path):
        for i, c in enumerate(cases + cases[1:2]):
            args = (dev(c.x_fp32), dev(c.w), dev(c.weight_scales), dev(c.bias))
            out = torch.empty((c.x_fp32.shape[0], c.w.shape[0], c.H_out, c.W_out),
                              dtype=torch.int8, device="cuda")
            keep.append(args)
            outs.append(out)
            ctx = torch.cuda.stream(side) if i == 3 else contextlib.nullcontext()
            if i == 3:
                side.wait_stream(torch.cuda.current_stream())
            with ctx:
                q8.q8ta_quantize_conv2d_transposed(args[0], c.in_scale, c.in_zp, args[1], c.Kh,
                                                   c.Kw, None, args[2], args[3], c.out_scale,
                                                   c.out_zp, c.stride, c.padding,
                                                   c.output_padding, (1, 1), 1, "none", out)
    torch.cuda.synchronize()
    for c, out in zip(cases + cases[1:2], outs):
        xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
        ref = oracle.conv2d_transposed(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                                       c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding,
                                       (1, 1), c.H_out, c.W_out)
        np.testing.assert_array_equal(host(out), ref)


def test_quantize_linear_workspace_across_calls_and_streams():
    """q8ta_quantize_linear calls that quantize through the workspace (M > 4,
    and K % 16 != 0 at M <= 4) mixed with in-kernel ones, queued back to back:
    small, larger (the buffer grows), small again, and one on a second
    stream; every result checked after one final synchronization."""
    _say("quantize+linear workspace reuse")
    shapes = [(8, 64, 32), (300, 1040, 257), (2, 36, 9), (1, 4096, 64), (65, 320, 97)]
    cases = []
    for i, (M, K, N) in enumerate(shapes):
        c = qi.linear_case(960 + i, M, K, N)
        cases.append((c, (qi.x_fp32(qi.rng(970 + i), (M, K)) * 1.5).astype(np.float32)))
    side = torch.cuda.Stream()
    keep, outs = [], []
    for i, (c, xf) in enumerate(cases + cases[1:2]):
        args = (dev(xf), dev(c.w), dev(c.weight_scales), dev(c.bias))
        out = torch.empty((c.M, c.N), dtype=torch.int8, device="cuda")
        keep.append(args)
        outs.append(out)
        on_side = i == len(cases)
        if on_side:
            side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side) if on_side else contextlib.nullcontext():
            q8.q8ta_quantize_linear(args[0], c.in_scale, c.in_zp, args[1], None, args[2], args[3],
                                    c.out_scale, c.out_zp, "none", out)
    torch.cuda.synchronize()
    for (c, xf), out in zip(cases + cases[1:2], outs):
        xq = oracle.quantize_per_tensor(xf, c.in_scale, c.in_zp)
        ref = oracle.linear(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                            c.out_zp)
        np.testing.assert_array_equal(host(out), ref)


# ============================================================================ relu, transposed-conv dilation and groups
@pytest.mark.parametrize("M,K,N", [(1, 512, 64), (1, 4096, 4096), (3, 48, 17), (300, 1040, 257),
                                   (7, 33, 5), (64, 128, 64)])
def test_linear_relu(M, K, N):
    """activation "relu" on every linear kernel (GEMV, skinny, grouped GEMM,
    shape-general) and on the fused dequantize."""
    _say(f"linear relu M={M} K={K} N={N}")
    c = qi.linear_case(M * 5 + K + N + 11, M, K, N)
    ref = _oracle_linear(c, activation="relu")
    assert (ref == c.out_zp).mean() > 0.2
    np.testing.assert_array_equal(_run_linear(c, activation="relu"), ref)
    with kernel("linear", "generic"):
        np.testing.assert_array_equal(_run_linear(c, activation="relu"), ref)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    q8.q8ta_linear_dq(dev(c.x), c.in_scale, c.in_zp, dev(c.w), None, dev(c.weight_scales),
                      dev(c.bias), c.out_scale, c.out_zp, "relu", out)
    dq = oracle.dequantize_per_tensor(ref, c.out_scale, c.out_zp)
    np.testing.assert_array_equal(host(out).view(np.uint32), dq.view(np.uint32))
    if M == 1:
        np.testing.assert_array_equal(_run_linear(c, fn=q8.q8ta_linear_gemv, activation="relu"), ref)


@pytest.mark.parametrize("path", ["mfma", "igemm", "tiled", "generic"])
def test_deconv_relu(path):
    _say(f"deconv relu path={path}")
    IC = 6 if path == "generic" else 64   # IC % 4 != 0 takes the one-output-per-thread kernel
    c = qi.deconv_case(811 + IC, 2, IC, 6, 7, 40, 3, 3, (2, 2), (1, 1), (1, 1))
    with kernel("conv2d_transposed", path):
        np.testing.assert_array_equal(_run_deconv(c, activation="relu"),
                                      _oracle_deconv(c, activation="relu"))


@pytest.mark.parametrize("case", ["mfma", "igemm", "depthwise", "generic"])
def test_conv2d_relu(case):
    _say(f"conv2d relu {case}")
    if case in ("mfma", "igemm"):
        c = qi.conv_case(821, 1, 64, 9, 11, 32, 3, 3, (1, 1), (1, 1), (1, 1))
    elif case == "depthwise":
        c = qi.conv_case(822, 2, 16, 12, 16, 16, 3, 3, (1, 1), (1, 1), (1, 1), groups=16)
    else:
        c = qi.conv_case(823, 1, 24, 7, 7, 8, 3, 3, (1, 1), (1, 1), (1, 1))
    with kernel("conv2d", case if case in ("mfma", "igemm") else "default"):
        np.testing.assert_array_equal(_run_conv(c, activation="relu"),
                                      _oracle_conv(c, activation="relu"))


def test_quantize_conv2d_transposed_relu():
    _say("quantize+deconv relu")
    c = qi.deconv_case(831, 1, 64, 5, 7, 32, 4, 4, (2, 2), (1, 1), (0, 0), x_from_fp32=True)
    for path in ("igemm", "tiled"):
        out = torch.empty((1, 32, c.H_out, c.W_out), dtype=torch.int8, device="cuda")
        with kernel("conv2d_transposed", path):
            q8.q8ta_quantize_conv2d_transposed(dev(c.x_fp32), c.in_scale, c.in_zp, dev(c.w), c.Kh,
                                               c.Kw, None, dev(c.weight_scales), dev(c.bias),
                                               c.out_scale, c.out_zp, c.stride, c.padding,
                                               c.output_padding, (1, 1), 1, "relu", out)
        xq = oracle.quantize_per_tensor(c.x_fp32, c.in_scale, c.in_zp)
        ref = oracle.conv2d_transposed(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp,
                                       c.out_scale, c.out_zp, c.Kh, c.Kw, c.stride, c.padding,
                                       (1, 1), c.H_out, c.W_out, activation="relu")
        np.testing.assert_array_equal(host(out), ref, err_msg=path)


# Dilated transposed convs: the stride phases take the dilated taps
# (num = r + pad - kh*dil); some phases get every tap, some none.
DECONV_DILATED_CASES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad, dil
    (1, 64, 6, 7, 32, 3, 3, (2, 2), (2, 2), (1, 1), (2, 2)),
    (1, 64, 5, 5, 40, 3, 3, (1, 1), (2, 2), (0, 0), (2, 2)),
    (2, 128, 4, 9, 64, 3, 3, (2, 2), (1, 1), (1, 1), (2, 1)),
    (1, 64, 5, 4, 16, 4, 4, (3, 2), (3, 2), (0, 0), (2, 3)),
    (1, 64, 4, 4, 16, 3, 3, (2, 2), (0, 0), (0, 0), (4, 4)),
    (1, 64, 3, 6, 24, 2, 3, (2, 2), (1, 2), (1, 1), (3, 3)),
]


@pytest.mark.parametrize("case", DECONV_DILATED_CASES,
                         ids=[str(i) for i in range(len(DECONV_DILATED_CASES))])
@pytest.mark.parametrize("path", ["mfma", "igemm", "tiled"])
def test_deconv_dilated_parity(case, path):
    N, IC, H, W, OC, Kh, Kw, s, p, op, d = case
    _say(f"deconv dilated {path} case={case}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, Kh, Kw]) + 13, N, IC, H, W, OC, Kh, Kw, s, p, op,
                       dilation=d)
    with kernel("conv2d_transposed", path):
        np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))
        np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))


def test_deconv_dilated_general_kernel():
    """IC % 4 != 0: the one-output-per-thread kernel with dilation."""
    _say("deconv dilated general")
    c = qi.deconv_case(841, 1, 6, 5, 6, 8, 3, 3, (2, 2), (1, 1), (1, 1), dilation=(2, 3))
    np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))
    np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))


DECONV_GROUPED_CASES = [
    # N, IC, H, W, OC, Kh, Kw, stride, pad, out_pad, dil, groups
    (1, 16, 5, 6, 16, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), 16),     # depthwise
    (2, 32, 4, 5, 16, 4, 4, (2, 2), (1, 1), (0, 0), (1, 1), 4),
    (1, 8, 6, 5, 16, 3, 3, (2, 2), (1, 1), (1, 1), (2, 2), 8),       # multiplier 2, dilated
    (1, 128, 4, 4, 64, 3, 3, (2, 2), (1, 1), (1, 1), (1, 1), 2),     # IC % 64 == 0, grouped
    (1, 12, 7, 3, 6, 2, 3, (3, 1), (0, 1), (2, 0), (1, 2), 3),
]


@pytest.mark.parametrize("case", DECONV_GROUPED_CASES,
                         ids=[str(i) for i in range(len(DECONV_GROUPED_CASES))])
def test_deconv_grouped_parity(case):
    N, IC, H, W, OC, Kh, Kw, s, p, op, d, G = case
    _say(f"deconv grouped case={case}")
    c = qi.deconv_case(sum([N, IC, H, W, OC, Kh, Kw, G]) + 17, N, IC, H, W, OC, Kh, Kw, s, p, op,
                       dilation=d, groups=G)
    np.testing.assert_array_equal(_run_deconv(c), _oracle_deconv(c))
    np.testing.assert_array_equal(_acc_deconv(c), _oracle_deconv_acc(c))
    np.testing.assert_array_equal(_run_deconv(c, activation="relu"),
                                  _oracle_deconv(c, activation="relu"))


# ============================================================================ precomputed weight sums (opt-in)
@pytest.mark.parametrize("N,K,offset", [(4096, 4096, 0), (257, 1040, 0), (37, 33, 0), (5, 64, 1),
                                        (11008, 4096, 0)])
def test_weight_sums(N, K, offset):
    _say(f"weight sums N={N} K={K} offset={offset}")
    g = qi.rng(N + K + offset)
    w = qi.w_int8(g, (N, K))
    buf = torch.zeros(N * K + offset, dtype=torch.int8, device="cuda")
    buf[offset:] = dev(w.reshape(-1))
    sums = torch.empty(N, dtype=torch.int32, device="cuda")
    q8.q8ta_weight_sums(buf[offset:].view(N, K), sums)
    np.testing.assert_array_equal(host(sums), oracle.weight_sums(w))


@pytest.mark.parametrize("path", ["default", "mfma32", "mfma32_8w", "generic"])
@pytest.mark.parametrize("M,K,N", [(1, 4096, 512), (300, 1024, 257), (65, 320, 97), (512, 4096, 768),
                                   (7, 33, 5), (40, 256, 64), (1024, 1024, 8192)])
def test_linear_presummed_equals_linear(path, M, K, N):
    """With the sums q8ta_weight_sums returns, the presummed calls give the
    same bits as q8ta_linear / q8ta_linear_dq on every kernel; with other sums
    the results move (the sums are used, not recomputed)."""
    _say(f"presummed {path} M={M} K={K} N={N}")
    c = qi.linear_case(M * 11 + K + N + len(path), M, K, N)
    wd = dev(c.w)
    sums = torch.empty(N, dtype=torch.int32, device="cuda")
    q8.q8ta_weight_sums(wd, sums)
    ref = _oracle_linear(c)
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    outf = torch.empty((M, N), dtype=torch.float32, device="cuda")
    with kernel("linear", path):
        q8.q8ta_linear_presummed(dev(c.x), c.in_scale, c.in_zp, wd, sums, dev(c.weight_scales),
                                 dev(c.bias), c.out_scale, c.out_zp, "none", out)
        np.testing.assert_array_equal(host(out), ref)
        q8.q8ta_linear_dq_presummed(dev(c.x), c.in_scale, c.in_zp, wd, sums, dev(c.weight_scales),
                                    dev(c.bias), c.out_scale, c.out_zp, "none", outf)
        dq = oracle.dequantize_per_tensor(ref, c.out_scale, c.out_zp)
        np.testing.assert_array_equal(host(outf).view(np.uint32), dq.view(np.uint32))
        if M > 4 and K % 16 == 0 and path != "generic":
            # the matrix-core GEMM takes the sums (the shape-general kernel forms
            # (x - zp) * w directly): shifted sums shift the accumulator
            wrong = sums + 1000
            q8.q8ta_linear_presummed(dev(c.x), c.in_scale, c.in_zp, wd, wrong, dev(c.weight_scales),
                                     dev(c.bias), c.out_scale, c.out_zp, "none", out)
            assert not np.array_equal(host(out), ref)


# ============================================================================ prepacked weights
def _pack_reference(w):
    """The packed layout as the header defines it, built with numpy indexing:
    byte 16*l + j of fragment (nb, s) = w[32*nb + l % 32][32*s + 16*(l // 32) + j],
    zero past N or K; fragment (nb, s) at (nb * KS + s) * 1024, KS = 2*ceil(K/64)."""
    N, K = w.shape
    NB, KP = -(-N // 32), -(-K // 64) * 64
    wp = np.zeros((NB * 32, KP), dtype=np.int8)
    wp[:N, :K] = w
    KS = KP // 32
    out = np.zeros(NB * 32 * KP, dtype=np.int8)
    for nb in range(NB):
        for s in range(KS):
            frag = np.empty((64, 16), dtype=np.int8)
            for l in range(64):
                frag[l] = wp[32 * nb + l % 32, 32 * s + 16 * (l // 32): 32 * s + 16 * (l // 32) + 16]
            out[(nb * KS + s) * 1024:(nb * KS + s + 1) * 1024] = frag.reshape(-1)
    return out


def _prepack(w):
    N, K = w.shape
    packed = torch.empty(q8.q8ta_weight_prepacked_bytes(N, K), dtype=torch.int8, device="cuda")
    q8.q8ta_weight_prepack(dev(w), packed)
    sums = torch.empty(N, dtype=torch.int32, device="cuda")
    q8.q8ta_weight_sums(dev(w), sums)
    return packed, sums


@pytest.mark.parametrize("N,K", [(32, 64), (33, 80), (100, 1040), (257, 4096), (7, 16)])
def test_weight_prepack_layout(N, K):
    _say(f"prepack N={N} K={K}")
    w = qi.linear_case(N + K, 1, K, N).w
    packed, _ = _prepack(w)
    np.testing.assert_array_equal(host(packed), _pack_reference(w))


PK_SHAPES = [(300, 1040, 257), (64, 128, 64), (512, 4096, 768), (5, 64, 32), (129, 2064, 129),
             (1, 4096, 512), (700, 256, 1100), (256, 192, 256)]


@pytest.mark.parametrize("path", ["default", "mfma32", "mfma32_8w"])
@pytest.mark.parametrize("M,K,N", PK_SHAPES)
def test_linear_prepacked_parity(M, K, N, path):
    """q8ta_linear_prepacked / _dq_prepacked with the weight's own sums: equal
    to the oracle (int8 codes, and their dequantized fp32 values bit for bit),
    on the 256 x 128-tile kernel of gemm_pk.hip ("mfma32") and the eight-wave
    kernel's prepacked mode ("mfma32_8w", K % 64 == 0)."""
    _say(f"linear prepacked {path} M={M} K={K} N={N}")
    c = qi.linear_case(M * 5 + K + N + 11, M, K, N)
    packed, sums = _prepack(c.w)
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    with kernel("linear", path):
        q8.q8ta_linear_prepacked(dev(c.x), c.in_scale, c.in_zp, packed, N, sums,
                                 dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, "none",
                                 out)
    ref = _oracle_linear(c)
    np.testing.assert_array_equal(host(out), ref)
    outf = torch.empty((M, N), dtype=torch.float32, device="cuda")
    with kernel("linear", path):
        q8.q8ta_linear_dq_prepacked(dev(c.x), c.in_scale, c.in_zp, packed, N, sums,
                                    dev(c.weight_scales), None, c.out_scale, c.out_zp, "relu",
                                    outf)
    refr = oracle.dequantize_per_tensor(_oracle_linear(c, bias=False, activation="relu"),
                                        c.out_scale, c.out_zp)
    np.testing.assert_array_equal(host(outf).view(np.uint32), refr.view(np.uint32))


@pytest.mark.parametrize("izp", [-128, 127])
def test_linear_prepacked_zero_points_and_shifted_sums(izp):
    """Extreme input zero points; sums other than the weight's move the result
    (the sums are used, not recomputed)."""
    M, K, N = 200, 512, 300
    c = qi.linear_case(900 + izp, M, K, N, in_zp=izp, out_zp=127 if izp < 0 else -128)
    packed, sums = _prepack(c.w)
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    q8.q8ta_linear_prepacked(dev(c.x), c.in_scale, c.in_zp, packed, N, sums,
                             dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, "none", out)
    np.testing.assert_array_equal(host(out), _oracle_linear(c))
    q8.q8ta_linear_prepacked(dev(c.x), c.in_scale, c.in_zp, packed, N, sums + 1000,
                             dev(c.weight_scales), dev(c.bias), c.out_scale, c.out_zp, "none", out)
    assert not np.array_equal(host(out), _oracle_linear(c))


def test_linear_dq_prepacked_gemm_workload_sampled():
    """The 2048 x 4096 x 11008 workload: fp32 rows checked against the oracle
    one by one, and the whole output against q8ta_linear_dq."""
    c = qi.make_gemm()
    _say("linear_dq prepacked 2048x4096x11008")
    packed, sums = _prepack(c.w)
    out = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    x, sc, bi = dev(c.x), dev(c.weight_scales), dev(c.bias)
    q8.q8ta_linear_dq_prepacked(x, c.in_scale, c.in_zp, packed, c.N, sums, sc, bi, c.out_scale,
                                c.out_zp, "none", out)
    ref_full = torch.empty_like(out)
    q8.q8ta_linear_dq(x, c.in_scale, c.in_zp, dev(c.w), None, sc, bi, c.out_scale, c.out_zp,
                      "none", ref_full)
    assert torch.equal(out.view(torch.int32), ref_full.view(torch.int32))
    got = host(out)
    rows = np.array([0, 1, 127, 128, 1000, 2047])
    q = oracle.linear(c.x[rows], c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                      c.out_zp)
    ref = oracle.dequantize_per_tensor(q, c.out_scale, c.out_zp)
    np.testing.assert_array_equal(got[rows].view(np.uint32), ref.view(np.uint32))
