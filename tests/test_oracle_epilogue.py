"""Pins for the oracle's epilogue (C-5): the GELU(tanh) closed-form properties,
its distance to the exact Gaussian-CDF GELU, the order scale -> bias -> GELU ->
residual -> alpha*d, and strength 0 giving bit-identical output (project page,
"Results", "Steering is real, inside a narrow window")."""
import math

import numpy as np

import oracle
import synthetic_inputs as si


def _gelu_erf(y):
    return 0.5 * y * (1.0 + math.erf(y / math.sqrt(2.0)))


def test_gelu_special_values():
    assert oracle.gelu_tanh(0.0) == 0.0
    assert abs(oracle.gelu_tanh(10.0) - 10.0) < 1e-12          # -> identity for large y
    assert abs(oracle.gelu_tanh(-10.0)) < 1e-12                 # -> 0 for very negative y
    h = 1e-6                                                     # slope 1/2 at the origin
    assert abs((oracle.gelu_tanh(h) - oracle.gelu_tanh(-h)) / (2 * h) - 0.5) < 1e-9


def test_gelu_odd_part_identity():
    # gelu(y) - gelu(-y) = y exactly in real arithmetic, because tanh is odd
    for y in np.linspace(-8, 8, 4001):
        assert abs(oracle.gelu_tanh(y) - oracle.gelu_tanh(-y) - y) <= 1e-14 * max(1.0, abs(y))


def test_gelu_close_to_exact_gelu():
    # the tanh form approximates x*Phi(x) to within 4.8e-4 everywhere
    worst = max(abs(oracle.gelu_tanh(y) - _gelu_erf(y)) for y in np.linspace(-10, 10, 20001))
    assert 1e-4 < worst < 4.8e-4
    # second-order Taylor coefficient equals exact GELU's 1/sqrt(2 pi)
    h = 1e-3
    c2 = (oracle.gelu_tanh(h) + oracle.gelu_tanh(-h)) / (2 * h * h)
    assert abs(c2 - 1.0 / math.sqrt(2.0 * math.pi)) < 1e-6


def test_epilogue_order():
    M, N = 2, 3
    z = np.zeros((M, N))
    bias = np.array([1.0, -2.0, 0.5], np.float16)
    res = np.array([[0.25, 0.5, -1.0], [2.0, 0.0, 3.0]], np.float16)
    d = np.array([1.0, -0.5, 0.25], np.float32)
    y = oracle.epilogue(z, bias=bias)
    assert np.array_equal(y, np.tile(bias.astype(np.float64), (M, 1)))
    y = oracle.epilogue(z, bias=bias, gelu=True)       # bias goes in before the GELU
    assert np.array_equal(y[0], [oracle.gelu_tanh(1.0), oracle.gelu_tanh(-2.0), oracle.gelu_tanh(0.5)])
    y = oracle.epilogue(z, gelu=True, residual=res)    # residual after the GELU: gelu(0) + r = r
    assert np.array_equal(y, res.astype(np.float64))
    y = oracle.epilogue(z, gelu=True, d=d, alpha=0.5)  # steering after the GELU too
    assert np.array_equal(y, np.tile(0.5 * d.astype(np.float64), (M, 1)))
    y = oracle.epilogue(np.full((M, N), -3.0), gelu=True, residual=res, d=d, alpha=2.0)
    assert np.allclose(y, oracle.gelu_tanh(-3.0) + res.astype(np.float64) + 2.0 * d, rtol=0, atol=1e-15)


def test_alpha_zero_is_bit_identical():
    rng = np.random.default_rng(4)
    y0 = rng.standard_normal((5, 7))
    y0[0, 0] = -0.0
    d = rng.standard_normal(7).astype(np.float32)
    a = oracle.epilogue(y0, gelu=True)
    b = oracle.epilogue(y0, gelu=True, d=d, alpha=0.0)
    assert a.tobytes() == b.tobytes()
    c = oracle.epilogue(y0, d=d, alpha=0.0)
    assert c.tobytes() == y0.tobytes()   # -0.0 stays -0.0


def test_direction_unit_norm():
    d = si.unit_direction(1536, 406)
    assert d.dtype == np.float32 and abs(np.linalg.norm(d.astype(np.float64)) - 1.0) < 1e-7
