"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a private copy of the oracle (on
the CPU only) and runs the oracle pin suite against it in a subprocess: every
mutant must make at least one pin fail.  C mutants edit the arithmetic in
``aria_oracle.c`` and are built into their own library; Python mutants edit
the block compositions in ``oracle/__init__.py`` (which third of QKV is V,
which tensor each residual reads, where GELU and the steering term go, which
input each norm reads) and run from a private copy of the tree.  The real
oracle is never modified."""
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
             "tests/test_oracle_gemm.py", "tests/test_oracle_epilogue.py", "tests/test_oracle_block.py",
             "tests/test_oracle_chain.py"]
PY_SRC = os.path.join(ROOT, "oracle", "__init__.py")

MUTANTS = {
    "rne_ties_up": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "codec_subnormal_quantum": ("if (e < -14) e = -14;", "if (e < -15) e = -15;"),
    "codec_decode_bias": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "no_clamp": ("if (r > qmax) r = qmax;", ""),
    "scale_qmax_plus_one": ("or_f64_to_f16(a / (double)qmax)", "or_f64_to_f16(a / (double)(qmax + 1))"),
    "scale_not_stored": ("double r = or_rne(or_f16_to_f64(v[i * stride]) / sd);",
                         "double r = or_rne(or_f16_to_f64(v[i * stride]) / (a / qmax));"),
    "q4_sequential_nibbles": ("return (int)((k % 2) * 16 + ((k % 8) / 2) * 4);", "return (int)((k % 8) * 4);"),
    "q4_halves_swapped": ("return (int)((k % 2) * 16 + ((k % 8) / 2) * 4);",
                          "return (int)((1 - k % 2) * 16 + ((k % 8) / 2) * 4);"),
    "group_column_stride": ("or_quant_sym(w + g * group * N + n, group, N,", "or_quant_sym(w + g * group + n, group, N,"),
    "gemm_drops_last_k": ("for (int64_t k = 0; k < K; k++) t += (int64_t)xq", "for (int64_t k = 0; k + 1 < K; k++) t += (int64_t)xq"),
    "w8a16_no_scale": ("r[m * N + n] = or_f16_to_f64(sw[n]) * t;", "r[m * N + n] = t;"),
    "w4a16_no_sign_extend": ("return nib >= 8 ? nib - 16 : nib;", "return nib;"),
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


# Python mutants: name -> list of (old, new, occurrence) edits of oracle/__init__.py
# (occurrence: which match of `old` to replace; the two block functions share
# some lines).  The first two groups follow the identity-attention chain
# (dit_block_w8a8), the last the full block (dit_block_full_w8a8).
_DOWN = 'out64 = qlinear_w8a8(u, *packed["down"], residual=h1, d=d, alpha=alpha)["y"]'
_OUT = 'h1 = f64_to_f16(qlinear_w8a8(a, *packed["o"], residual=h)["y"])'
PY_MUTANTS = {
    "chain_v_slice_k": [("qkv[:, 2 * width:3 * width]", "qkv[:, width:2 * width]", 0)],
    "chain_v_slice_q": [("qkv[:, 2 * width:3 * width]", "qkv[:, 0:width]", 0)],
    "chain_down_residual_h": [(_DOWN, _DOWN.replace("residual=h1", "residual=h"), 1)],
    "chain_steer_on_out": [(_OUT, _OUT.replace("residual=h)", "residual=h, d=d, alpha=alpha)"), 1),
                           (_DOWN, _DOWN.replace(", d=d, alpha=alpha", ""), 1)],
    "chain_gelu_on_down": [('qlinear_w8a8(h1, *packed["up"], gelu=True)', 'qlinear_w8a8(h1, *packed["up"])', 0),
                           (_DOWN, _DOWN.replace("residual=h1,", "residual=h1, gelu=True,"), 1)],
    "chain_out_no_residual": [(_OUT, _OUT.replace(", residual=h", ""), 1)],
    "chain_up_reads_h": [('qlinear_w8a8(h1, *packed["up"], gelu=True)', 'qlinear_w8a8(h, *packed["up"], gelu=True)', 0)],
    "full_qkv_reads_h": [('qlinear_w8a8(n1, *packed["qkv"])', 'qlinear_w8a8(h, *packed["qkv"])', 0)],
    "full_ln1_params": [("n1 = f64_to_f16(layernorm(h, *ln1, eps))", "n1 = f64_to_f16(layernorm(h, *ln2, eps))", 0)],
    "full_ln2_reads_h": [("layernorm(h1, *ln2, eps)", "layernorm(h, *ln2, eps)", 0)],
    "full_attention_one_sequence": [("attention(qkv, heads, seq)", "attention(qkv, heads, qkv.shape[0])", 0)],
    "full_out_residual_n1": [(_OUT, _OUT.replace("residual=h)", "residual=n1)"), 0)],
    "full_down_residual_h": [(_DOWN, _DOWN.replace("residual=h1", "residual=h"), 0)],
    "full_steer_on_out": [(_OUT, _OUT.replace("residual=h)", "residual=h, d=d, alpha=alpha)"), 0),
                          (_DOWN, _DOWN.replace(", d=d, alpha=alpha", ""), 0)],
    "full_gelu_on_down": [('qlinear_w8a8(n2, *packed["up"], gelu=True)', 'qlinear_w8a8(n2, *packed["up"])', 0),
                          (_DOWN, _DOWN.replace("residual=h1,", "residual=h1, gelu=True,"), 0)],
}


def _pytest(cwd, env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-W", "ignore::RuntimeWarning", *PIN_FILES],
                       cwd=cwd, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


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
    return name, _pytest(ROOT, env)


def _replace_nth(src, old, new, n):
    at = -1
    for _ in range(n + 1):
        at = src.find(old, at + 1)
        assert at >= 0, f"mutation site {old!r} has no occurrence {n}"
    return src[:at] + new + src[at + len(old):]


def _run_py_mutant(name, tmp):
    """Copy the tests, the input generators and the oracle package into a
    private tree, edit the copy's __init__.py, run the pins there (their
    conftest puts that tree first on sys.path) against the real C library."""
    d = os.path.join(tmp, name)
    shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(d, "tests"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "synthetic_inputs.py"), d)
    os.makedirs(os.path.join(d, "oracle"))
    src = open(PY_SRC).read()
    for old, new, n in PY_MUTANTS[name]:
        src = _replace_nth(src, old, new, n)
    open(os.path.join(d, "oracle", "__init__.py"), "w").write(src)
    env = dict(os.environ, ARIA_ORACLE_LIB=oracle.build(force=False), OMP_NUM_THREADS="1")
    return name, _pytest(d, env)


def test_every_mutant_is_caught():
    tmp = tempfile.mkdtemp(prefix="oracle_mutants_")
    try:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            jobs = [ex.submit(_run_mutant, n, tmp) for n in MUTANTS]
            jobs += [ex.submit(_run_py_mutant, n, tmp) for n in PY_MUTANTS]
            results = dict(j.result() for j in jobs)
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


def test_unmutated_python_copy_passes():
    """Control for the Python mutants: the private tree with an unedited
    __init__.py passes."""
    tmp = tempfile.mkdtemp(prefix="oracle_control_py_")
    try:
        PY_MUTANTS["_control"] = []
        name, rc = _run_py_mutant("_control", tmp)
    finally:
        PY_MUTANTS.pop("_control", None)
        shutil.rmtree(tmp, ignore_errors=True)
    assert rc == 0
