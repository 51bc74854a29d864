"""Pins for the oracle's symmetric quantizer (C-2) and activation quantizer (a2):
exact integer/rational brute force over the full fp16 grid, hand-derived worked
values (tests/golden/quantizer_worked.csv), the round-trip bound and the
degenerate cases.  Also checks, on the host, the two fp32 facts the GPU
quantizers rely on to be bit-exact with the fp64 definition."""
import os

import numpy as np
import pytest

import oracle
from tests.exact import UNIT, f16_units, fraction_to_f16_bits, quant_exact, rne_div

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantizer_worked.csv")

ALL = np.arange(65536, dtype=np.uint32).astype(np.uint16)
FINITE = ALL[np.isfinite(ALL.view(np.float16))]

# absmax values chosen to give: ordinary scales, exact-tie scales (0.125, 1.0),
# a subnormal scale (with clamping), the largest finite input, random ones
ABSMAX = [0x3C00, 0x4BF0, 0x4700, 0x0400, 0x7BFF, 0x3555, 0x4E21, 0x1234, 0x2A00, 0x0013]


def _grid_vector(a_bits):
    a = f16_units(np.array([a_bits], np.uint16))[0]
    u = f16_units(FINITE)
    sel = FINITE[np.abs(u) <= a]
    return np.concatenate([np.array([a_bits], np.uint16), sel])


@pytest.mark.parametrize("qmax", [127, 7])
@pytest.mark.parametrize("a_bits", ABSMAX)
def test_exhaustive_grid_vs_exact(a_bits, qmax):
    v = _grid_vector(a_bits)
    q, s = oracle.quant_sym(v, qmax)
    qe, se = quant_exact(v, qmax)
    assert int(np.asarray(s).view(np.uint16)) == se
    assert np.array_equal(q.astype(np.int64), qe)


def test_golden_worked_values():
    rows = [ln.split(",") for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 15
    for a, qmax, x, s_exp, q_exp in rows:
        v = np.array([int(a, 16), int(x, 16)], np.uint16)
        q, s = oracle.quant_sym(v, int(qmax))
        assert int(np.asarray(s).view(np.uint16)) == int(s_exp, 16), (a, qmax, x)
        assert int(q[1]) == int(q_exp), (a, qmax, x, int(q[1]))


@pytest.mark.parametrize("qmax,L", [(127, 1536), (127, 256), (7, 32)])
def test_round_trip_bound(qmax, L):
    rng = np.random.default_rng(11)
    for sigma in (1.0, 0.02, 0.01, 30.0):
        v = (rng.standard_normal((64, L)) * sigma).astype(np.float16)
        for row in v:
            q, s = oracle.quant_sym(row, qmax)
            sd = float(s)
            assert sd >= 2.0 ** -14  # normal scale at these sigmas
            err = np.abs(row.astype(np.float64) - q.astype(np.float64) * sd)
            assert np.all(err <= sd / 2), (qmax, sigma, float(err.max()), sd)
            assert np.max(np.abs(q)) == qmax  # the absmax element maps to +-qmax


def test_zero_vector_and_signed_zero():
    for qmax in (127, 7):
        q, s = oracle.quant_sym(np.array([0, 0x8000, 0], np.uint16), qmax)
        assert int(np.asarray(s).view(np.uint16)) == 0 and not q.any()


def test_quant_act_rows():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 96)).astype(np.float16)
    x[4] = 0  # an all-zero token
    xq, sa = oracle.quant_act(x)
    for m in range(x.shape[0]):
        qe, se = quant_exact(x[m].view(np.uint16), 127)
        assert int(sa.view(np.uint16)[m]) == se
        assert np.array_equal(xq[m].astype(np.int64), qe)
    assert not xq[4].any() and sa.view(np.uint16)[4] == 0


def test_nonfinite_rejected():
    with pytest.raises(ValueError):
        oracle.quant_sym(np.array([0x3C00, 0x7C00], np.uint16), 127)


# ---------------------------------------------------------------------------
# fp32 facts the device quantizers use (host-side proofs, no GPU involved)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("qmax", [127, 7])
def test_fp32_scale_equals_fp64_scale(qmax):
    """fp16(fp32(a)/qmax) == fp16_RNE(a/qmax) exactly, for every positive finite a."""
    a = FINITE.view(np.float16)
    a = a[a > 0]
    dev = (a.astype(np.float32) / np.float32(qmax)).astype(np.float16).view(np.uint16)
    ref = oracle.f64_to_f16(a.astype(np.float64) / qmax).view(np.uint16)
    assert np.array_equal(dev, ref)


@pytest.mark.parametrize("a_bits", ABSMAX)
@pytest.mark.parametrize("qmax", [127, 7])
def test_fp32_divide_rint_equals_exact(a_bits, qmax):
    """clamp(rint(fp32(x)/fp32(s))) (IEEE fp32 division, ties-to-even rint)
    equals the exact rounding of x/s for every x on the grid."""
    v = _grid_vector(a_bits)
    qe, se = quant_exact(v, qmax)
    s = np.array([se], np.uint16).view(np.float16).astype(np.float32)[0]
    if s == 0:
        return
    q = np.clip(np.rint(v.view(np.float16).astype(np.float32) / s), -qmax, qmax).astype(np.int64)
    assert np.array_equal(q, qe)


def test_exact_helpers_selfcheck():
    # the exact helpers against hand values (worked values of the golden file)
    from fractions import Fraction
    assert fraction_to_f16_bits(Fraction(1, 127)) == 0x2008
    assert fraction_to_f16_bits(Fraction(1, 7)) == 0x3092
    assert list(rne_div(np.array([1, 3, 5, -1, -3]), 2)) == [0, 2, 2, 0, -2]
    assert f16_units(np.array([0x0001], np.uint16))[0] == 1 and UNIT == 2 ** 24
