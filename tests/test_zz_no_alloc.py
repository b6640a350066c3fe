"""The allocation-free entry point q8ta_quantize_linear_noalloc, called through
the C ABI, against the allocating q8ta_quantize_linear and the oracle: two
calls in a row (the second smaller) that stage their quantized activations in
the library's static scratch array, an M <= 4 call that needs none, and the
size limit of that array."""
import ctypes

import numpy as np
import pytest

import oracle
import q8ta_inputs as qi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import int8_quantized_amd as q8  # noqa: E402

SCRATCH_BYTES = 16 << 20


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _call(fn, xf, c, out, act="none"):
    lib = q8.lib()
    M, K = xf.shape
    N = c.w.shape[0]
    args = [ctypes.c_void_p(xf.data_ptr()), M, K, c.in_scale, c.in_zp, ctypes.c_void_p(c.wd.data_ptr()),
            N, None, ctypes.c_void_p(c.sd.data_ptr()), ctypes.c_void_p(c.bd.data_ptr()), c.out_scale,
            c.out_zp, act.encode(), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)]
    return getattr(lib, fn)(*args)


def _case(seed, M, K, N):
    c = qi.linear_case(seed, M, K, N)
    c.xf = (qi.x_fp32(qi.rng(seed + 1), (M, K)) * 2.0).astype(np.float32)
    c.wd = torch.from_numpy(c.w).cuda()
    c.sd = torch.from_numpy(c.weight_scales).cuda()
    c.bd = torch.from_numpy(c.bias).cuda()
    return c


def _oracle(c, act="none"):
    xq = oracle.quantize_per_tensor(c.xf, c.in_scale, c.in_zp)
    return oracle.linear(xq, c.w, c.weight_scales, c.bias, c.in_scale, c.in_zp, c.out_scale,
                         c.out_zp, activation=act)


@pytest.mark.parametrize("act", ["none", "relu"])
def test_noalloc_two_calls_match_the_allocating_entry_point(act):
    # first call: 2048 x 4096 activations (8 MiB staged), second a smaller
    # ragged one; then an M <= 4 call (no staging) and the first shape again
    shapes = [(2048, 4096, 1024), (300, 1040, 257), (3, 512, 70), (2048, 4096, 1024)]
    cases = [_case(4000 + i, *s) for i, s in enumerate(shapes[:3])] 
    cases.append(cases[0])
    for i, (c, (M, K, N)) in enumerate(zip(cases, shapes)):
        print(f"noalloc call {i}: M={M} K={K} N={N} act={act}", flush=True)
        xf = torch.from_numpy(c.xf).cuda()
        out_na = torch.full((M, N), 99, dtype=torch.int8, device="cuda")
        out_ref = torch.full((M, N), -99, dtype=torch.int8, device="cuda")
        assert _call("q8ta_quantize_linear_noalloc", xf, c, out_na, act) == 0, q8.q8ta_last_error()
        assert _call("q8ta_quantize_linear", xf, c, out_ref, act) == 0, q8.q8ta_last_error()
        torch.cuda.synchronize()
        got = out_na.cpu().numpy()
        np.testing.assert_array_equal(got, out_ref.cpu().numpy())
        np.testing.assert_array_equal(got, _oracle(c, act))


def test_noalloc_rejects_more_than_the_scratch_holds():
    M, K, N = 4097, 4096, 32     # 16 MiB + 4 KiB of staged activations
    assert M * K > SCRATCH_BYTES
    xf = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    w = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    s = torch.ones(N, dtype=torch.float32, device="cuda")
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    rc = q8.lib().q8ta_quantize_linear_noalloc(
        xf.data_ptr(), M, K, 0.02, 3, w.data_ptr(), N, None, s.data_ptr(), None, 0.5, -5, b"none",
        out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == q8.Q8TA_ERR_SHAPE
    assert "static scratch" in q8.q8ta_last_error()
    # exactly at the limit is accepted
    M = SCRATCH_BYTES // K
    out = torch.empty((M, N), dtype=torch.int8, device="cuda")
    rc = q8.lib().q8ta_quantize_linear_noalloc(
        xf.data_ptr(), M, K, 0.02, 3, w.data_ptr(), N, None, s.data_ptr(), None, 0.5, -5, b"none",
        out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, q8.q8ta_last_error()
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == np.int8(np.clip(np.rint(0.0) - 5, -128, 127))).all()
