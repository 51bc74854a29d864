"""Pins for the oracle's IEEE 754 binary16 codec (C-1) against numpy's own
float16 conversion and hand-derived worked values (tests/golden/fp16_worked.csv)."""
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp16_worked.csv")


def _all_patterns():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_decode_every_pattern():
    h = _all_patterns()
    ours = oracle.f16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(ours[0x8000]) and not np.signbit(ours[0])


def test_encode_every_value_and_midpoint():
    h = _all_patterns()
    v = h.view(np.float16).astype(np.float64)
    fin = np.isfinite(v)
    vals = np.sort(np.unique(v[fin]))
    mids = (vals[:-1] + vals[1:]) / 2.0          # exact in fp64: ties
    quarter = vals[:-1] + (vals[1:] - vals[:-1]) / 4.0
    three_q = vals[:-1] + 3.0 * (vals[1:] - vals[:-1]) / 4.0
    over = np.array([65504.0, 65519.0, 65519.999, 65520.0, 70000.0, 1e300, -65520.0, -1e300])
    x = np.concatenate([vals, mids, quarter, three_q, over, -mids])
    ours = oracle.f64_to_f16(x).view(np.uint16)
    ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r}"


def test_encode_random_doubles():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-30, 17, 200000))
    ours = oracle.f64_to_f16(x).view(np.uint16)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_golden_worked_values():
    rows = [ln.split(",") for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for val, bits in rows:
        x = float.fromhex(val) if "p" in val else float(val)
        got = int(oracle.f64_to_f16([x]).view(np.uint16)[0])
        assert got == int(bits, 16), (val, hex(got), bits)


def test_rne_ties():
    assert [oracle.rne(v) for v in (0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 2.4999, 2.5001)] == \
        [0.0, 2.0, 2.0, -0.0, -2.0, -2.0, 2.0, 3.0]
