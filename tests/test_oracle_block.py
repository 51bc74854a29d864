"""Pins for the oracle's DiT-block steps around the linears: LayerNorm and
multi-head self-attention (readings R21-R23), each against closed forms,
invariances and an independent numpy/scipy formulation."""
import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _f16(a):
    return np.asarray(a, np.float16)


# ---- LayerNorm ----------------------------------------------------------------

def test_layernorm_unit_affine_closed_form():
    """gamma = 1, beta = 0: every row has mean 0 and variance var / (var + eps)."""
    rng = np.random.default_rng(1)
    x = _f16(rng.standard_normal((6, 96)) * 3 + 1)
    eps = 1e-5
    y = oracle.layernorm(x, np.ones(96, np.float16), np.zeros(96, np.float16), eps)
    xf = x.astype(np.float64)
    var = xf.var(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-12
    assert np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-12, atol=0)


def test_layernorm_affine_and_numpy():
    rng = np.random.default_rng(2)
    x = _f16(rng.standard_normal((5, 160)))
    g = _f16(1 + 0.1 * rng.standard_normal(160))
    b = _f16(0.1 * rng.standard_normal(160))
    y = oracle.layernorm(x, g, b, 1e-5)
    xf = x.astype(np.float64)
    ref = (xf - xf.mean(1, keepdims=True)) / np.sqrt(xf.var(1, keepdims=True) + 1e-5)
    ref = ref * g.astype(np.float64) + b.astype(np.float64)
    assert np.max(np.abs(y - ref)) < 1e-12


def test_layernorm_constant_row_gives_beta():
    x = np.full((2, 64), 1.5, np.float16)
    b = _f16(np.linspace(-1, 1, 64))
    y = oracle.layernorm(x, _f16(np.full(64, 3.0)), b, 1e-5)
    assert np.array_equal(y, np.broadcast_to(b.astype(np.float64), (2, 64)))


def test_layernorm_shift_and_scale_invariance():
    """LN(a x + c) = LN(x) up to eps: exact with eps = 0 for power-of-two a."""
    rng = np.random.default_rng(3)
    x = _f16(rng.integers(-64, 64, (3, 128)))
    g, b = np.ones(128, np.float16), np.zeros(128, np.float16)
    y0 = oracle.layernorm(x, g, b, 0.0)
    y1 = oracle.layernorm(_f16(x.astype(np.float64) * 4 + 8), g, b, 0.0)
    assert np.max(np.abs(y0 - y1)) < 1e-12


# ---- attention ------------------------------------------------------------------

def _ref_attention(qkv, heads, seq):
    """Independent formulation: numpy einsum + scipy softmax per sequence."""
    qkv = qkv.astype(np.float64)
    M, W3 = qkv.shape
    W = W3 // 3
    D = W // heads
    q = qkv[:, :W].reshape(M // seq, seq, heads, D)
    k = qkv[:, W:2 * W].reshape(M // seq, seq, heads, D)
    v = qkv[:, 2 * W:].reshape(M // seq, seq, heads, D)
    s = np.einsum("bihd,bjhd->bhij", q, k) / np.sqrt(D)
    p = softmax(s, axis=-1)
    o = np.einsum("bhij,bjhd->bihd", p, v)
    return o.reshape(M, W)


@pytest.mark.parametrize("heads,seq,M", [(2, 16, 32), (3, 24, 24), (4, 8, 40)])
def test_attention_vs_numpy(heads, seq, M):
    rng = np.random.default_rng(heads * 10 + seq)
    W = heads * 16
    qkv = _f16(rng.standard_normal((M, 3 * W)))
    out = oracle.attention(qkv, heads, seq)
    ref = _ref_attention(qkv, heads, seq)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_attention_zero_queries_average_values():
    """Q = 0: every weight is 1/S, so each output is the mean of its sequence's V."""
    rng = np.random.default_rng(5)
    heads, seq, M, W = 2, 12, 36, 32
    qkv = _f16(rng.standard_normal((M, 3 * W)))
    qkv[:, :W] = 0
    out = oracle.attention(qkv, heads, seq)
    v = qkv[:, 2 * W:].astype(np.float64).reshape(M // seq, seq, W)
    exp = np.repeat(v.mean(axis=1), seq, axis=0)
    assert np.max(np.abs(out - exp)) < 1e-12


def test_attention_one_hot_selects_a_value_row():
    """A query aligned with one key and orthogonal to the rest, scaled up,
    puts (almost) all weight on that key: the output is that key's V row."""
    heads, seq, W = 1, 8, 16
    qkv = np.zeros((seq, 3 * W), np.float16)
    for j in range(seq):
        qkv[j, W + (j % W)] = 8.0          # key j along axis j
        qkv[j, 2 * W:] = j + 1             # value row j = (j + 1) * ones
    qkv[:, 3] = 8.0                        # every query along axis 3: picks key 3
    out = oracle.attention(qkv, heads, seq)
    # weight on key 3: e^16 / (e^16 + 7) (s = 64 / sqrt(16) = 16 vs 0)
    w3 = np.exp(16.0) / (np.exp(16.0) + 7)
    exp = w3 * 4 + (1 - w3) * (sum(j + 1 for j in range(seq) if j != 3) / 7)
    assert np.allclose(out, exp, rtol=0, atol=1e-12)


def test_attention_sequences_and_heads_are_independent():
    rng = np.random.default_rng(6)
    heads, seq, W = 2, 10, 32
    qkv = _f16(rng.standard_normal((2 * seq, 3 * W)))
    out = oracle.attention(qkv, heads, seq)
    qkv2 = qkv.copy()
    qkv2[seq:] = _f16(rng.standard_normal((seq, 3 * W)))          # other sequence changed
    qkv2[:seq, 16:32] = _f16(rng.standard_normal((seq, 16)))     # head 1's queries of seq 0 changed
    out2 = oracle.attention(qkv2, heads, seq)
    assert np.array_equal(out[:seq, :16], out2[:seq, :16])         # head 0 of sequence 0 unchanged
    assert not np.array_equal(out[:seq, 16:], out2[:seq, 16:])


def test_attention_softmax_shift_invariance():
    """Adding the same vector to every key of a sequence shifts all scores of
    a query equally: the output does not change."""
    rng = np.random.default_rng(7)
    heads, seq, W = 1, 16, 16
    qkv = _f16(rng.integers(-4, 5, (seq, 3 * W)) * 0.25)
    out = oracle.attention(qkv, heads, seq)
    qkv2 = qkv.copy()
    qkv2[:, W:2 * W] = _f16(qkv2[:, W:2 * W].astype(np.float64) + 0.5)
    out2 = oracle.attention(qkv2, heads, seq)
    assert np.max(np.abs(out - out2)) < 1e-12
