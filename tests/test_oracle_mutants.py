"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a private copy of the oracle's C
source (on the CPU only), builds it, and runs the oracle pin suite against it
in a subprocess: every mutant must make at least one pin fail.  The real oracle
is never modified."""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "aria_oracle.c")
PIN_FILES = ["tests/test_oracle_codec.py", "tests/test_oracle_quant.py", "tests/test_oracle_pack.py",
             "tests/test_oracle_gemm.py", "tests/test_oracle_epilogue.py", "tests/test_oracle_block.py"]

MUTANTS = {
    "rne_ties_up": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "codec_subnormal_quantum": ("if (e < -14) e = -14;", "if (e < -15) e = -15;"),
    "codec_decode_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "no_clamp": ("if (r > qmax) r = qmax;", ""),
    "scale_qmax_plus_one": ("or_f64_to_f16(a / (double)qmax)", "or_f64_to_f16(a / (double)(qmax + 1))"),
    "scale_not_stored": ("double r = or_rne(or_f16_to_f64(v[i * stride]) / sd);",
                         "double r = or_rne(or_f16_to_f64(v[i * stride]) / (a / qmax));"),
    "nibble_order": ("(uint8_t)((qcol[2 * j] & 0xF) | ((qcol[2 * j + 1] & 0xF) << 4))",
                     "(uint8_t)((qcol[2 * j + 1] & 0xF) | ((qcol[2 * j] & 0xF) << 4))"),
    "group_column_stride": ("or_quant_sym(w + g * group * N + n, group, N,", "or_quant_sym(w + g * group + n, group, N,"),
    "gemm_drops_last_k": ("for (int64_t k = 0; k < K; k++) t += (int64_t)xq", "for (int64_t k = 0; k + 1 < K; k++) t += (int64_t)xq"),
    "w8a16_no_scale": ("r[m * N + n] = or_f16_to_f64(sw[n]) * t;", "r[m * N + n] = t;"),
    "w4a16_no_sign_extend": ("int qv = nib >= 8 ? nib - 16 : nib;", "int qv = nib;"),
    "w4a16_group_index": ("sg[n * G + k / group]", "sg[n * G + k % G]"),
    "w8a8_drop_act_scale": ("(double)acc[m * N + n] * or_f16_to_f64(sa[m]) * or_f16_to_f64(sw[n])",
                            "(double)acc[m * N + n] * or_f16_to_f64(sw[n])"),
    "gelu_constant": ("sqrt(2.0 / pi)", "sqrt(pi / 2.0)"),
    "gelu_cubic": ("0.044715 * y * y * y", "0.44715 * y * y * y"),
    "bias_after_gelu": ("if (bias) v += or_f16_to_f64(bias[n]);\n            if (gelu) v = or_gelu_tanh(v);",
                        "if (gelu) v = or_gelu_tanh(v);\n            if (bias) v += or_f16_to_f64(bias[n]);"),
    "steer_sign": ("v += (double)alpha * (double)d[n];", "v -= (double)alpha * (double)d[n];"),
    "steer_always": ("if (d && alpha != 0.0f)", "if (d)"),
    "pack16_not_transposed": ("wt[n * K + k] = w[k * N + n];", "wt[n * K + k] = w[n * K + k];"),
    "w16a16_row_stride": ("t += xr[k] * or_f16_to_f64(wt[n * K + k]);", "t += xr[k] * or_f16_to_f64(wt[k * N + n]);"),
    "layernorm_no_eps": ("double inv = 1.0 / sqrt(var + eps);", "double inv = 1.0 / sqrt(var);"),
    "layernorm_sample_variance": ("var /= (double)W;", "var /= (double)(W - 1);"),
    "layernorm_beta_scaled": ("* or_f16_to_f64(gamma[k]) +\n                           or_f16_to_f64(beta[k]);",
                              "* or_f16_to_f64(gamma[k]) * (1.0 +\n                           or_f16_to_f64(beta[k]));"),
    "attention_no_scale": ("const double scale = 1.0 / sqrt((double)D);", "const double scale = 1.0;"),
    "attention_across_sequences": ("const int64_t kj = (b * S + j) * ld + W + h * D;", "const int64_t kj = (((b + 1) % (M / S)) * S + j) * ld + W + h * D;"),
    "attention_value_head": ("o += sc[j] * or_f16_to_f64(qkv[(b * S + j) * ld + 2 * W + h * D + e]);",
                             "o += sc[j] * or_f16_to_f64(qkv[(b * S + j) * ld + 2 * W + e]);"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    d = os.path.join(tmp, name)
    os.makedirs(d)
    c = os.path.join(d, "m.c")
    so = os.path.join(d, "libm.so")
    open(c, "w").write(src.replace(old, new))
    subprocess.run(["gcc", *oracle._CFLAGS, "-w", c, "-o", so, "-lm"], check=True)
    env = dict(os.environ, ARIA_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-W", "ignore::RuntimeWarning", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_mutant_is_caught():
    tmp = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = dict(ex.map(lambda n: _run_mutant(n, tmp), MUTANTS))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    survivors = [n for n, rc in results.items() if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    # return code 1 = tests failed (not a crash of the runner or a collection error)
    assert all(rc == 1 for rc in results.values()), results


def test_unmutated_copy_passes():
    """Control: the same procedure with no mutation passes, so failures above
    come from the planted mistakes."""
    tmp = tempfile.mkdtemp(prefix="oracle_control_")
    try:
        MUTANTS["_control"] = ("/* C-1  IEEE 754", "/* C-1  IEEE 754")
        name, rc = _run_mutant("_control", tmp)
    finally:
        MUTANTS.pop("_control", None)
        shutil.rmtree(tmp, ignore_errors=True)
    assert rc == 0
