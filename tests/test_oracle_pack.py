"""Pins for the oracle's weight packers (a1: q8 per-channel, q4 group-32 nibbles):
brute force per column / per group with exact arithmetic, the nibble order from
one-hot weights, every byte through the nibble decoder, and identity weights."""
import numpy as np
import pytest

import oracle
from tests.exact import quant_exact, sign_extend4


def _rand_w(K, N, seed, sigma=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((K, N)) * sigma).astype(np.float16)
    return w


@pytest.mark.parametrize("K,N", [(32, 1), (64, 7), (96, 17), (256, 5)])
def test_qpack8_brute_force(K, N):
    w = _rand_w(K, N, K * 100 + N)
    w[:, 0] = 0  # an all-zero output channel
    q, s = oracle.qpack8(w)
    assert q.shape == (N, K) and s.shape == (N,)
    for n in range(N):
        qe, se = quant_exact(w[:, n].view(np.uint16), 127)
        assert int(s.view(np.uint16)[n]) == se
        assert np.array_equal(q[n].astype(np.int64), qe)


@pytest.mark.parametrize("K,N", [(32, 3), (64, 5), (160, 9)])
def test_qpack4_brute_force(K, N):
    w = _rand_w(K, N, K * 7 + N)
    # give each group a very different magnitude so a wrong group index shows
    for g in range(K // 32):
        w[32 * g:32 * g + 32] *= np.float16(2.0 ** (g - 2))
    w[32:64, 1 % N] = 0 if K >= 64 else w[32:64, 1 % N]
    q4, s4 = oracle.qpack4(w, 32)
    assert q4.shape == (N, K // 2) and s4.shape == (N, K // 32)
    lo = sign_extend4(q4)            # even k
    hi = sign_extend4(q4 >> 4)       # odd k
    for n in range(N):
        for g in range(K // 32):
            qe, se = quant_exact(w[32 * g:32 * g + 32, n].view(np.uint16), 7)
            assert int(s4.view(np.uint16)[n, g]) == se, (n, g)
            got = np.empty(32, np.int64)
            got[0::2] = lo[n, 16 * g:16 * g + 16]
            got[1::2] = hi[n, 16 * g:16 * g + 16]
            assert np.array_equal(got, qe), (n, g)


def test_nibble_order_one_hot():
    K, N = 64, 4
    w = np.zeros((K, N), np.float16)
    w[0, 0] = 1.0     # k = 0  -> low nibble of byte 0
    w[1, 1] = 1.0     # k = 1  -> high nibble of byte 0
    w[2, 2] = -1.0    # k = 2  -> low nibble of byte 1, value -7 = 0b1001
    w[33, 3] = 1.0    # k = 33 -> group 1, high nibble of byte 16
    q4, s4 = oracle.qpack4(w, 32)
    assert q4[0, 0] == 0x07 and not q4[0, 1:].any()
    assert q4[1, 0] == 0x70 and not q4[1, 1:].any()
    assert q4[2, 1] == 0x09 and q4[2, 0] == 0 and not q4[2, 2:].any()
    assert q4[3, 16] == 0x70 and q4[3].sum() == 0x70
    sb = s4.view(np.uint16)
    assert sb[0, 0] == 0x3092 and sb[0, 1] == 0       # 1/7 rounded to fp16
    assert sb[3, 0] == 0 and sb[3, 1] == 0x3092


def test_unpack_every_byte():
    b = np.arange(256, dtype=np.uint8).reshape(1, 256)
    q = oracle.unpack4(b, 512)
    vals = np.arange(256)
    assert np.array_equal(q[0, 0::2].astype(np.int64), sign_extend4(vals))
    assert np.array_equal(q[0, 1::2].astype(np.int64), sign_extend4(vals >> 4))
    # repacking the decoded nibbles gives every byte back
    rep = (q[0, 0::2].astype(np.int64) & 0xF) | ((q[0, 1::2].astype(np.int64) & 0xF) << 4)
    assert np.array_equal(rep, vals)


def test_identity_weights():
    K = N = 96
    perm = np.random.default_rng(5).permutation(N)
    w = np.zeros((K, N), np.float16)
    w[perm, np.arange(N)] = 1.0          # column n holds its 1 at k = perm[n]
    q, s = oracle.qpack8(w)
    assert np.all(s.view(np.uint16) == 0x2008)
    exp = np.zeros((N, K), np.int8)
    exp[np.arange(N), perm] = 127
    assert np.array_equal(q, exp)
    q4, s4 = oracle.qpack4(w, 32)
    full = oracle.unpack4(q4, K)
    exp4 = np.zeros((N, K), np.int8)
    exp4[np.arange(N), perm] = 7
    assert np.array_equal(full, exp4)
    sb = s4.view(np.uint16)
    for n in range(N):
        for g in range(K // 32):
            assert sb[n, g] == (0x3092 if perm[n] // 32 == g else 0)
