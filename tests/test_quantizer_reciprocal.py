"""Host proof of the activation quantizer's division-free rounding (CPU only).

The GPU kernel rounds x / s through a per-row reciprocal instead of dividing
per element: rint(x * RN(1/s)), with an exact tie test only where the product
lies within 2^-15 of a half-integer.  quantizer_reciprocal_check.c replays
those fp32 steps for every fp16 row maximum and every |x| <= it and compares
them with rint(x / s) under IEEE division; a mutant without the tie test must
fail, which shows the check can see the cases that matter."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quantizer_reciprocal_check.c")


def _build(tmp_path, extra=()):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / ("qchk_mutant" if extra else "qchk"))
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", *extra, SRC, "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    return exe


def _run(exe):
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)


def test_reciprocal_rounding_matches_division(tmp_path):
    r = _run(_build(tmp_path))
    assert r.returncode == 0, r.stdout + r.stderr
    # every fp16 x with |x| <= a for every positive finite fp16 a, both signs
    assert "pairs 1007713278 " in r.stdout and "mismatches 0" in r.stdout, r.stdout


def test_reciprocal_rounding_needs_the_tie_test(tmp_path):
    r = _run(_build(tmp_path, ("-DDROP_TIE_TEST",)))
    assert r.returncode != 0 and "mismatches 0" not in r.stdout, r.stdout


def test_fast_path_needs_its_margin(tmp_path):
    """With a near-half-integer margin far below the product's error bound
    (2^-30 instead of 2^-15), the fast path keeps wrong roundings."""
    r = _run(_build(tmp_path, ("-DNEAR_MARGIN=0x1p-30f",)))
    assert r.returncode != 0 and "mismatches 0" not in r.stdout, r.stdout
