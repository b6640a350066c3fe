"""The oracle's pins must catch a plausible mistake anywhere in it.

Each case below plants one mistake in a copy of ``oracle/q8ta_oracle.c`` (a
dropped term, a wrong sign or index, a transposed operand, the wrong rounding,
the wrong reciprocal, ...), builds the copy, and runs the pin suite
(``tests/test_oracle_pins.py``) against it in a subprocess: the suite must fail.
CPU only; the real oracle library is never touched.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "q8ta_oracle.c")

# (name, text to replace, replacement, occurrence index (0 = first))
MUTANTS = [
    ("quantize_round_half_away", "float r = nearbyintf(t);", "float r = roundf(t);", 0),
    ("quantize_float_reciprocal", "const float inv_scale = (float)(1.0 / scale);",
     "const float inv_scale = 1.0f / (float)scale;", 0),
    ("quantize_zp_before_round", "float t = x[i] * inv_scale;", "float t = x[i] * inv_scale + zp;"
     " t = t - zp + zp;", 0),
    ("quantize_narrow_clamp", "if (u < -128.0f) u = -128.0f;", "if (u < -127.0f) u = -127.0f;", 0),
    ("dequantize_zp_sign", "int d = (int)q[i] - (int)zero_point;",
     "int d = (int)q[i] + (int)zero_point;", 0),
    ("dequantize_scale_reciprocal", "const float s = (float)scale;",
     "const float s = (float)(1.0 / scale);", 0),
    ("epilogue_channel_index", "int64_t c = (e / inner) % channels;", "int64_t c = e % channels;", 0),
    ("epilogue_bias_sign", "if (bias) v = v + bias[c];", "if (bias) v = v - bias[c];", 0),
    ("epilogue_bias_dropped", "if (bias) v = v + bias[c];", "if (bias) v = v;", 0),
    ("epilogue_input_scale_dropped", "v = v * s_in;", "v = v * 1.0f;", 0),
    # the operation order of acc * input_scale * weight_scales[c] + bias[c]
    ("epilogue_prefolded_scales", "v = v * s_in;\n    v = v * weight_scales[c];",
     "v = v * (s_in * weight_scales[c]);", 0),
    ("epilogue_fma_weight_scale_bias", "v = v * weight_scales[c];\n    if (bias) v = v + bias[c];",
     "if (bias) v = fmaf(v, weight_scales[c], bias[c]);\n    else v = v * weight_scales[c];", 0),
    ("epilogue_scales_swapped", "v = v * s_in;\n    v = v * weight_scales[c];",
     "v = v * weight_scales[c];\n    v = v * s_in;", 0),
    ("epilogue_input_scale_in_double", "v = v * s_in;", "v = (float)((double)v * input_scale);", 0),
    ("epilogue_dequant_in_double", "v = v * s_in;\n    v = v * weight_scales[c];\n"
     "    if (bias) v = v + bias[c];",
     "v = (float)((double)v * (double)s_in * (double)weight_scales[c]"
     " + (bias ? (double)bias[c] : 0.0));", 0),
    ("epilogue_out_zp_sign", "float u = r + ozp;", "float u = r - ozp;", 0),
    ("epilogue_round_half_away", "float r = nearbyintf(t);", "float r = roundf(t);", 1),
    ("epilogue_float_reciprocal", "const float inv_out = (float)(1.0 / output_scale);",
     "const float inv_out = 1.0f / (float)output_scale;", 0),
    ("epilogue_clamp_before_zp", "float u = r + ozp;\n    if (u < -128.0f) u = -128.0f;\n"
     "    if (u > 127.0f) u = 127.0f;", "float u = r;\n    if (u < -128.0f) u = -128.0f;\n"
     "    if (u > 127.0f) u = 127.0f;\n    u = u + ozp;", 0),
    ("linear_zp_sign", "((int64_t)x[m * K + k] - input_zero_point)",
     "((int64_t)x[m * K + k] + input_zero_point)", 0),
    ("linear_weight_row_stride", "(int64_t)w[n * ldw + k];\n      if", "(int64_t)w[n * K + k];\n      if",
     0),
    ("linear_transposed_weight", "* (int64_t)w[n * ldw + k];\n      if (s > INT32_MAX",
     "* (int64_t)w[(k % N) * ldw + (n % K)];\n      if (s > INT32_MAX", 0),
    ("deconv_tap_order", "int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];\n                s +=",
     "int64_t wv = w[oc * ldw + (kw * Kh + kh) * ICg + icg];\n                s +=", 0),
    ("deconv_channel_major_weight", "int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];\n"
     "                s +=", "int64_t wv = w[oc * ldw + icg * Kh * Kw + kh * Kw + kw];\n"
     "                s +=", 0),
    ("deconv_dilation_dropped", "int64_t num = o + pad - k * dil;\n  if (num < 0)",
     "int64_t num = o + pad - k;\n  if (num < 0)", 0),
    ("deconv_group_of_channel", "const int64_t g = oc / OCg;", "const int64_t g = oc % groups;", 0),
    ("deconv_group_channels_interleaved", "const int64_t ic = g * ICg + icg;",
     "const int64_t ic = icg * groups + g;", 0),
    ("deconv_group_weight_stride", "int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];",
     "int64_t wv = w[oc * ldw + (kh * Kw + kw) * IC + icg];", 0),
    ("relu_dropped", "if (relu && v < 0.0f) v = 0.0f;", "", 0),
    ("relu_on_the_code", "if (relu && v < 0.0f) v = 0.0f;\n    float t = v * inv_out;\n"
     "    float r = nearbyintf(t);\n    float u = r + ozp;",
     "float t = v * inv_out;\n    float r = nearbyintf(t);\n    float u = r + ozp;\n"
     "    if (relu && u < 0.0f) u = 0.0f;", 0),
    ("relu_before_bias", "if (bias) v = v + bias[c];\n    if (pre) pre[e] = v;\n"
     "    if (relu && v < 0.0f) v = 0.0f;", "if (relu && v < 0.0f) v = 0.0f;\n"
     "    if (bias) v = v + bias[c];\n    if (pre) pre[e] = v;", 0),
    ("deconv_negative_numerator_allowed", "if (num < 0) return 0;            /* checked before dividing */",
     "", 0),
    ("deconv_last_row_dropped", "if (i >= in_size) return 0;", "if (i >= in_size - 1) return 0;", 0),
    ("deconv_zp_sign", "s += (xv - input_zero_point) * wv;", "s += (xv + input_zero_point) * wv;", 0),
    ("deconv_pad_sign", "int64_t num = o + pad - k * dil;\n  if (num < 0)",
     "int64_t num = o - pad - k * dil;\n  if (num < 0)", 0),
    ("conv_pad_sign", "const int64_t ih = oh * stride_h - pad_h + kh * dil_h;",
     "const int64_t ih = oh * stride_h + pad_h + kh * dil_h;", 0),
    ("conv_dilation_dropped", "const int64_t iw = ow * stride_w - pad_w + kw * dil_w;",
     "const int64_t iw = ow * stride_w - pad_w + kw;", 0),
    ("conv_stride_axis", "const int64_t iw = ow * stride_w - pad_w + kw * dil_w;",
     "const int64_t iw = ow * stride_h - pad_w + kw * dil_w;", 0),
    ("conv_last_column_dropped", "if (iw < 0 || iw >= W_in) continue;",
     "if (iw < 0 || iw >= W_in - 1) continue;", 0),
    ("conv_tap_order", "int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];",
     "int64_t wv = w[oc * ldw + (kw * Kh + kh) * ICg + icg];", 2),
    ("conv_zp_sign", "s += (xv - input_zero_point) * wv;", "s += (xv + input_zero_point) * wv;", 1),
    ("conv_group_of_channel", "const int64_t g = oc / OCg;", "const int64_t g = oc % groups;", 2),
    ("conv_group_channels_interleaved", "const int64_t ic = g * ICg + icg;",
     "const int64_t ic = icg * groups + g;", 2),
    ("conv_group_weight_stride", "int64_t wv = w[oc * ldw + (kh * Kw + kw) * ICg + icg];",
     "int64_t wv = w[oc * ldw + (kh * Kw + kw) * IC + icg];", 2),
]


def _mutate(text, old, new, occ):
    idx = -1
    for _ in range(occ + 1):
        idx = text.index(old, idx + 1)
    return text[:idx] + new + text[idx + len(old):]


def _run_pins_against(name, old, new, occ, tmp):
    text = open(SRC).read()
    mutated = _mutate(text, old, new, occ)
    assert mutated != text
    src = os.path.join(tmp, f"{name}.c")
    with open(src, "w") as f:
        f.write(mutated)
    lib = oracle.compile_source(src, os.path.join(tmp, f"lib{name}.so"))
    env = dict(os.environ, Q8TA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-400:]


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run_pins_against(*m, tmp), MUTANTS))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, f"mistakes no pin caught: {[n for n, _ in survivors]}"


def test_unmutated_copy_passes_the_pins():
    """Control: the same machinery on an unmodified copy passes."""
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.compile_source(SRC, os.path.join(tmp, "libcopy.so"))
        env = dict(os.environ, Q8TA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join(HERE, "test_oracle_pins.py")], cwd=ROOT, env=env,
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-2000:]
