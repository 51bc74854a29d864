"""Pins for the oracle's weight packers (a1: q8 per-channel, q4 group-32 nibbles):
brute force per column / per group with exact arithmetic, the nibble positions
from one-hot weights, every byte value in every position through the nibble
decoder, and identity weights."""
import numpy as np
import pytest

import oracle
from tests.exact import quant_exact, sign_extend4, unpack4_words


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
    codes = unpack4_words(q4)
    for n in range(N):
        for g in range(K // 32):
            qe, se = quant_exact(w[32 * g:32 * g + 32, n].view(np.uint16), 7)
            assert int(s4.view(np.uint16)[n, g]) == se, (n, g)
            assert np.array_equal(codes[n, 32 * g:32 * g + 32], qe), (n, g)


def test_nibble_order_one_hot():
    """Where each k lands: word k // 8 of the row, even k in the low half-word
    and odd k in the high one, nibble (k % 8) // 2 of that half-word."""
    K, N = 64, 6
    w = np.zeros((K, N), np.float16)
    w[0, 0] = 1.0     # k = 0  -> byte 0, low nibble
    w[1, 1] = 1.0     # k = 1  -> byte 2, low nibble
    w[2, 2] = -1.0    # k = 2  -> byte 0, high nibble, value -7 = 0b1001
    w[7, 3] = 1.0     # k = 7  -> byte 3, high nibble
    w[33, 4] = 1.0    # k = 33 -> group 1, word 4: byte 18, low nibble
    w[12, 5] = -1.0   # k = 12 -> word 1, even, nibble 2: byte 5, low nibble
    q4, s4 = oracle.qpack4(w, 32)
    expect = {0: (0, 0x07), 1: (2, 0x07), 2: (0, 0x90), 3: (3, 0x70), 4: (18, 0x07), 5: (5, 0x09)}
    for n, (byte, val) in expect.items():
        assert q4[n, byte] == val, (n, q4[n])
        assert int(q4[n].astype(np.int64).sum()) == val, (n, q4[n])
    sb = s4.view(np.uint16)
    assert sb[0, 0] == 0x3092 and sb[0, 1] == 0       # 1/7 rounded to fp16
    assert sb[4, 0] == 0 and sb[4, 1] == 0x3092


def test_unpack_every_byte():
    """Every byte value in each of a word's four byte positions, decoded by
    the oracle and by an independent word reader, and packed back."""
    vals = np.arange(256, dtype=np.int64)
    for pos in range(4):
        b = np.zeros((1, 4 * 256), np.uint8)
        b[0, pos::4] = vals
        q = oracle.unpack4(b, 8 * 256).astype(np.int64)
        assert np.array_equal(q, unpack4_words(b))
        words = q.reshape(256, 8)
        # byte pos holds k = 4 (pos % 2) + pos // 2 in its low nibble and k + 2 in its high one
        k_lo = 4 * (pos % 2) + pos // 2
        assert np.array_equal(words[:, k_lo], sign_extend4(vals))
        assert np.array_equal(words[:, k_lo + 2], sign_extend4(vals >> 4))
        others = [k for k in range(8) if k not in (k_lo, k_lo + 2)]
        assert not words[:, others].any()


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
