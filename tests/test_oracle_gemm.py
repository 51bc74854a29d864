"""Pins for the oracle's contractions (C-4): the exact int32 W8A8 accumulator
against naive Python sums and numpy int64 matmul, the fp64 weight-only
references against numpy float64 (BLAS) matmul of the dequantized weights,
and identity weights through the whole pipeline (closed-form outputs)."""
import numpy as np
import pytest

import oracle
from tests.exact import unpack4_words


def test_k1_all_pairs():
    v = np.arange(-127, 128, dtype=np.int8)
    acc = oracle.gemm_i8(v.reshape(-1, 1), v.reshape(-1, 1))
    exp = np.array([[int(a) * int(b) for b in v] for a in v], np.int64)
    assert np.array_equal(acc.astype(np.int64), exp)


@pytest.mark.parametrize("seed", range(6))
def test_random_tiny_vs_numpy_and_loops(seed):
    rng = np.random.default_rng(seed)
    M, N = rng.integers(1, 18, 2)
    K = int(rng.choice([32, 64, 96]))
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (N, K)).astype(np.int8)
    acc = oracle.gemm_i8(a, b)
    assert np.array_equal(acc.astype(np.int64), a.astype(np.int64) @ b.astype(np.int64).T)
    m, n = int(rng.integers(0, M)), int(rng.integers(0, N))
    assert int(acc[m, n]) == sum(int(a[m, k]) * int(b[n, k]) for k in range(K))


def test_int32_extremes_k8192():
    K = 8192
    a = np.full((2, K), 127, np.int8)
    a[1] = -127
    b = np.full((1, K), 127, np.int8)
    acc = oracle.gemm_i8(a, b)
    assert acc[0, 0] == 127 * 127 * K and acc[1, 0] == -127 * 127 * K


def test_w8a16_vs_blas():
    rng = np.random.default_rng(21)
    M, K, N = 33, 160, 47
    x = rng.standard_normal((M, K)).astype(np.float16)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sw = (rng.random(N) * 1e-3).astype(np.float16)
    r = oracle.ref_w8a16(x, wq, sw)
    ref = (x.astype(np.float64) @ wq.astype(np.float64).T) * sw.astype(np.float64)[None, :]
    assert np.max(np.abs(r - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_w4a16_vs_blas():
    rng = np.random.default_rng(22)
    M, K, N = 19, 128, 37
    x = rng.standard_normal((M, K)).astype(np.float16)
    q4 = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    s4 = (rng.random((N, K // 32)) * 1e-2).astype(np.float16)
    r = oracle.ref_w4a16(x, q4, s4, 32)
    wd = unpack4_words(q4).astype(np.float64)
    wd *= np.repeat(s4.astype(np.float64), 32, axis=1)
    ref = x.astype(np.float64) @ wd.T
    assert np.max(np.abs(r - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_identity_weights_closed_form():
    K = N = 128
    M = 24
    rng = np.random.default_rng(9)
    perm = rng.permutation(N)
    w = np.zeros((K, N), np.float16)
    w[perm, np.arange(N)] = 1.0
    x = rng.standard_normal((M, K)).astype(np.float16)
    xs = x.astype(np.float64)[:, perm]
    # W8A16: y = x[:, perm[n]] * (127 * fp16(1/127))
    wq, sw = oracle.qpack8(w)
    y8 = oracle.qlinear_w8a16(x, wq, sw)
    assert np.array_equal(y8, xs * 0.99993896484375)
    # W4A16: y = x[:, perm[n]] * (7 * fp16(1/7))
    q4, s4 = oracle.qpack4(w, 32)
    y4 = oracle.qlinear_w4a16(x, q4, s4)
    assert np.array_equal(y4, xs * 0.999755859375)
    # W8A8: acc = 127 * xq[:, perm[n]]
    out = oracle.qlinear_w8a8(x, wq, sw)
    assert np.array_equal(out["acc"].astype(np.int64), 127 * out["xq"].astype(np.int64)[:, perm])


def test_w8a8_scale_closed_form():
    acc = np.array([[127 * 127, -1, 0]], np.int32)
    s = np.array([0x2008], np.uint16).view(np.float16)
    y = oracle.scale_w8a8(acc, s, np.repeat(s, 3))
    assert y[0, 0] == 0.99993896484375 ** 2
    assert y[0, 1] == -(0.00787353515625 ** 2) and y[0, 2] == 0.0


# ---- the fp16 rung (W16A16) ----------------------------------------------

def test_pack16_is_the_transpose():
    rng = np.random.default_rng(31)
    w = rng.standard_normal((96, 40)).astype(np.float16)
    wt = oracle.pack16(w)
    assert wt.shape == (40, 96) and wt.dtype == np.float16
    assert np.array_equal(wt.view(np.uint16), np.ascontiguousarray(w.T).view(np.uint16))


def test_w16a16_exact_integers():
    """Small integer-valued fp16 operands: every product and partial sum is an
    exact integer in fp64, so the reference equals Python integer sums."""
    rng = np.random.default_rng(32)
    M, K, N = 7, 96, 11
    x = rng.integers(-20, 21, (M, K))
    w = rng.integers(-20, 21, (K, N))
    r = oracle.ref_w16a16(x.astype(np.float16), oracle.pack16(w.astype(np.float16)))
    for m in range(M):
        for n in range(N):
            assert r[m, n] == sum(int(x[m, k]) * int(w[k, n]) for k in range(K))


def test_w16a16_vs_blas():
    rng = np.random.default_rng(33)
    M, K, N = 21, 224, 45
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    r = oracle.ref_w16a16(x, oracle.pack16(w))
    ref = x.astype(np.float64) @ w.astype(np.float64)
    assert np.max(np.abs(r - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_w16a16_permutation_weights():
    """A permutation matrix as W selects input columns: y = x[:, perm] exactly."""
    rng = np.random.default_rng(34)
    K = 64
    perm = rng.permutation(K)
    w = np.zeros((K, K), np.float16)
    w[perm, np.arange(K)] = 1.0
    x = rng.standard_normal((9, K)).astype(np.float16)
    r = oracle.ref_w16a16(x, oracle.pack16(w))
    assert np.array_equal(r, x.astype(np.float64)[:, perm])
