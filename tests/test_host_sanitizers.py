"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two sanitized builds, each exercised in a subprocess with the sanitizer
runtime preloaded (the Python interpreter itself is not instrumented):

* the oracle (``oracle/q8ta_oracle.c``) built by gcc with
  ``-fsanitize=address,undefined``, running the pin suite
  (``tests/test_oracle_pins.py``);
* libq8ta with its host code (argument validation, kernel choice, launch
  planning, workspace bookkeeping) built by hipcc with both sanitizers on the
  host side only -- device code is never instrumented -- running the C-ABI
  tests (``tests/test_abi.py``) and the planning sweep below.

The planning sweep also runs in the plain suite.  On a machine without a GPU a
call with valid arguments and fake device pointers passes validation, kernel
choice and planning and then fails in the HIP runtime (Q8TA_ERR_HIP), so every
shape, kernel family and entry point of the sweep drives the host path without
launching anything; with a GPU present it is skipped (it would launch on fake
addresses).
"""
import ctypes
import glob
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import int8_quantized_amd as q8

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
FAKE = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced on the host


def _gpu_present():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


NO_GPU = pytest.mark.skipif(_gpu_present(), reason="calls with fake device pointers; only "
                                                   "meaningful without a GPU")

KERNELS = {
    "linear": ["default", "mfma32", "mfma32_8w", "generic"],
    "conv2d_transposed": ["default", "fixed", "mfma32", "mfma", "igemm", "tiled", "generic"],
    "conv2d": ["default", "fixed", "mfma32", "mfma", "igemm", "generic"],
}


def _deconv_shapes(n):
    """n seeded transposed-conv configurations (conventional output size)."""
    g = np.random.Generator(np.random.PCG64(2051))
    out = []
    while len(out) < n:
        N = int(g.choice([1, 2, 8]))
        groups = int(g.choice([1, 1, 1, 2, 4]))
        IC = int(g.choice([16, 32, 64, 128, 192, 256])) * (groups if g.random() < 0.5 else 1)
        OC = int(g.choice([8, 32, 33, 48, 64, 128, 130, 160]))
        if IC % groups or OC % groups:
            continue
        H, W = (int(v) for v in g.choice([(5, 12), (8, 8), (9, 36), (32, 32), (64, 64),
                                          (7, 136), (1, 1), (3, 200)]))
        K = int(g.choice([1, 2, 3, 4, 5]))
        s = int(g.choice([1, 2, 2, 3]))
        d = int(g.choice([1, 1, 2]))
        p = int(g.integers(0, K))
        op = int(g.integers(0, max(s, d)))
        H_out = (H - 1) * s - 2 * p + d * (K - 1) + op + 1
        W_out = (W - 1) * s - 2 * p + d * (K - 1) + op + 1
        if H_out < 1 or W_out < 1:
            continue
        out.append((N, IC, H, W, OC, K, s, p, op, d, groups, H_out, W_out))
    return out


def _conv_shapes(n):
    g = np.random.Generator(np.random.PCG64(2052))
    out = []
    while len(out) < n:
        N = int(g.choice([1, 2, 8]))
        groups = int(g.choice([1, 1, 1, 2, 64, 256]))
        IC = int(g.choice([64, 128, 256])) if groups < 64 else groups
        OC = IC if groups >= 64 else int(g.choice([8, 40, 48, 128, 160]))
        if IC % groups or OC % groups:
            continue
        H, W = (int(v) for v in g.choice([(10, 12), (7, 132), (8, 8), (64, 64), (9, 8), (3, 3)]))
        K = int(g.choice([1, 3, 5]))
        s = int(g.choice([1, 1, 2]))
        d = int(g.choice([1, 1, 2]))
        p = int(g.integers(0, K))
        H_out = (H + 2 * p - d * (K - 1) - 1) // s + 1
        W_out = (W + 2 * p - d * (K - 1) - 1) // s + 1
        if H_out < 1 or W_out < 1:
            continue
        out.append((N, IC, H, W, OC, K, s, p, d, groups, H_out, W_out))
    return out


LINEAR_SHAPES = [(M, K, N) for M in (1, 2, 4, 5, 64, 300, 2048)
                 for K in (16, 48, 64, 1040, 4096, 4112) for N in (1, 7, 32, 257, 11008)]


def _reaches_runtime(rc, what):
    assert rc == q8.Q8TA_ERR_HIP, (what, rc, q8.q8ta_last_error())


@NO_GPU
def test_host_planning_sweep():
    """Every entry point, kernel family and a seeded sweep of shapes gets
    through the host path to the HIP runtime without a GPU."""
    l = q8.lib()
    F = FAKE
    try:
        for kern in KERNELS["linear"]:
            q8.q8ta_select_kernel("linear", kern)
            for M, K, N in LINEAR_SHAPES:
                args = (F, M, K, 0.02, 3, F, N, None, F, F, 0.3, -5, b"relu", F, None)
                for fn in ("q8ta_linear", "q8ta_linear_dq", "q8ta_quantize_linear",
                           "q8ta_quantize_linear_dq"):
                    _reaches_runtime(getattr(l, fn)(*args), (fn, M, K, N, kern))
                if M == 1:
                    _reaches_runtime(l.q8ta_linear_gemv(*args), ("gemv", K, N))
                if M * K <= (16 << 20) or M <= 4:
                    _reaches_runtime(l.q8ta_quantize_linear_noalloc(*args), ("noalloc", M, K, N))
                pres = (F, M, K, 0.02, 3, F, N, F, F, None, 0.3, -5, b"none", F, None)
                _reaches_runtime(l.q8ta_linear_presummed(*pres), ("presummed", M, K, N))
                _reaches_runtime(l.q8ta_linear_dq_presummed(*pres), ("dq_presummed", M, K, N))
                _reaches_runtime(l.q8ta_linear_acc(F, M, K, 3, F, N, F, None), ("acc", M, K, N))
                if K % 16 == 0:
                    _reaches_runtime(l.q8ta_linear_prepacked(*pres), ("prepacked", M, K, N))
                    _reaches_runtime(l.q8ta_linear_dq_prepacked(*pres), ("dq_prepacked", M, K, N))
        for kern in KERNELS["conv2d_transposed"]:
            q8.q8ta_select_kernel("conv2d_transposed", kern)
            for (N, IC, H, W, OC, K, s, p, op, d, g, Ho, Wo) in _deconv_shapes(150):
                ldw = K * K * (IC // g) + (16 if IC % 3 == 0 else 0)
                for fn in (l.q8ta_conv2d_transposed, l.q8ta_quantize_conv2d_transposed):
                    rc = fn(F, N, IC, H, W, 0.02, 3, F, OC, K, K, ldw, None, F, F, 0.5, -5, s, s,
                            p, p, op, op, d, d, g, b"none", F, Ho, Wo, None)
                    _reaches_runtime(rc, ("deconv", kern, N, IC, H, W, OC, K, s, p, op, d, g))
                rc = l.q8ta_conv2d_transposed_acc(F, N, IC, H, W, 3, F, OC, K, K, ldw, s, s, p, p,
                                                  d, d, g, F, Ho, Wo, None)
                _reaches_runtime(rc, ("deconv_acc", kern, N, IC, H, W, OC, K, s, p, d, g))
        for kern in KERNELS["conv2d"]:
            q8.q8ta_select_kernel("conv2d", kern)
            for (N, IC, H, W, OC, K, s, p, d, g, Ho, Wo) in _conv_shapes(120):
                ldw = K * K * (IC // g)
                rc = l.q8ta_conv2d(F, N, IC, H, W, 0.02, 3, F, OC, K, K, ldw, None, F, F, 0.5, -5,
                                   s, s, p, p, d, d, g, b"relu", F, Ho, Wo, None)
                _reaches_runtime(rc, ("conv", kern, N, IC, H, W, OC, K, s, p, d, g))
                rc = l.q8ta_conv2d_acc(F, N, IC, H, W, 3, F, OC, K, K, ldw, s, s, p, p, d, d, g,
                                       F, Ho, Wo, None)
                _reaches_runtime(rc, ("conv_acc", kern, N, IC, H, W, OC, K, s, p, d, g))
        for numel in (1, 3, 16, 1000, 1 << 22):
            _reaches_runtime(l.q8ta_quantize_per_tensor(F, F, numel, 0.02, 3, None), numel)
            _reaches_runtime(l.q8ta_dequantize_per_tensor(F, F, numel, 0.02, 3, None), numel)
        _reaches_runtime(l.q8ta_weight_sums(F, 257, 1040, F, None), "sums")
        _reaches_runtime(l.q8ta_weight_prepack(F, 257, 1040, F, None), "prepack")
    finally:
        for op in KERNELS:
            q8.q8ta_select_kernel(op, "default")


# --------------------------------------------------------------------- sanitized builds
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, env, timeout=900):
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=timeout)
    assert r.returncode == 0, (r.stdout[-3000:] + "\n" + r.stderr[-6000:])
    return r.stdout


def test_oracle_pins_under_asan_ubsan():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    import oracle
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "liboracle_san.so")
        flags = [f for f in oracle.GCC_FLAGS if f != "-O2"] + [
            "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
            "-fno-omit-frame-pointer"]
        subprocess.run(["gcc"] + flags + ["-o", lib, os.path.join(ROOT, "oracle", "q8ta_oracle.c"),
                                          "-lm"], check=True)
        env = dict(os.environ, LD_PRELOAD=asan, Q8TA_ORACLE_LIB=lib, OMP_NUM_THREADS="4",
                   PYTHONPATH=ROOT, **SAN_ENV)
        out = _run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider",
                    os.path.join(HERE, "test_oracle_pins.py")], env)
        assert " passed" in out


def _clang_asan_runtime():
    from int8_quantized_amd import build as b
    hipcc = b.hipcc()
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    p = r.stdout.strip()
    if os.path.isabs(p) and os.path.exists(p):
        return p
    hits = glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))),
                                  "llvm", "lib", "clang", "*", "lib", "linux",
                                  "libclang_rt.asan-x86_64.so"))
    hits += glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def test_library_host_code_under_asan_ubsan():
    from int8_quantized_amd import build as b
    asan = _clang_asan_runtime()
    if asan is None:
        pytest.skip("clang's AddressSanitizer runtime is not installed")
    # Host-side instrumentation only: -Xarch_host before every sanitizer flag.
    host = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer", "-g"):
        host += ["-Xarch_host", f]
    cflags = [f for f in b.CFLAGS if f != "-O3"] + ["-O1"] + host
    srcs = sorted(glob.glob(os.path.join(b.CSRC, "*.hip")))
    with tempfile.TemporaryDirectory() as tmp:
        from concurrent.futures import ThreadPoolExecutor

        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            subprocess.run([b.hipcc()] + cflags + ["-I", os.path.join(ROOT, "include"), "-c", src,
                                                   "-o", obj], check=True, capture_output=True)
            return obj
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
            objs = list(ex.map(compile_one, srcs))
        lib = os.path.join(tmp, "libq8ta_san.so")
        subprocess.run([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-o", lib] + objs,
                       check=True, capture_output=True)
        env = dict(os.environ, LD_PRELOAD=asan, PYTHONPATH=ROOT, **SAN_ENV)
        code = ("import sys, pytest, int8_quantized_amd as q8\n"
                f"q8.LIB_PATH = {lib!r}\n"
                "sys.exit(pytest.main(['-x', '-q', '-s', '-p', 'no:cacheprovider', "
                f"{os.path.join(HERE, 'test_abi.py')!r}, "
                f"{os.path.join(HERE, 'test_host_sanitizers.py') + '::test_host_planning_sweep'!r}"
                "]))\n")
        out = _run([sys.executable, "-c", code], env)
        assert " passed" in out
