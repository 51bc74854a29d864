"""Pins for the oracle's block compositions: ``oracle.dit_block_w8a8`` (the
W8A8 chain with the identity-attention stand-in) and
``oracle.dit_block_full_w8a8`` (the block with pre-norms and softmax
attention).

The compositions fix the wiring that no single-step pin sees: which third of
the QKV output is V, which tensor each residual add reads, which linear
applies GELU, and that the steering term alpha*d is added only by the
block-output linear (project page, "Results", "Steering is real, inside a
narrow window": the direction is added to one block's residual stream and
alpha = 0 removes it exactly; docshare paper page, Fig. 1, steering site 1 on
the residual stream).

Each linear gets a weight with exactly one nonzero per output column, so its
W8A8 output has a closed form: per-token quantization of the input (computed
here with the brute-force rational quantizer of ``tests/exact.py``), one
product per output (acc[m][n] = qa[m][sel[n]] * qw[n]) and the two scales.
Attention with zero queries and keys weighs every key of a sequence equally,
so its output is the mean of that sequence's values.  LayerNorm and GELU are
written from their definitions with numpy and ``math.tanh``.  Nothing here
calls the oracle except the function under test."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import f16_units, fraction_to_f16_bits, quant_exact, rne_div

ALPHA = np.float32(0.3)


def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16)


# ---- closed forms ---------------------------------------------------------------

def sel_weight(K, N, sel, vals):
    """fp16 W [K][N] with W[sel[n]][n] = vals[n] and zeros elsewhere."""
    w = np.zeros((K, N), np.float16)
    w[np.asarray(sel), np.arange(N)] = _f16(vals)
    return w


def quant_rows_exact(x16):
    """Per-token quantization of fp16 rows by exact rational arithmetic:
    (qa int64 [M][K], s_a float64 [M])."""
    qa, sa = [], []
    for row in np.asarray(x16, np.float16):
        q, sb = quant_exact(row.view(np.uint16), 127)
        qa.append(q)
        sa.append(float(np.array([sb], np.uint16).view(np.float16)[0]))
    return np.array(qa, np.int64), np.array(sa, np.float64)


def weight_codes(vals):
    """int8 code and fp16 scale of a column whose only nonzero is v."""
    codes, scales = [], []
    for v in vals:
        v16 = np.float16(v)
        if v16 == 0:
            codes.append(0)
            scales.append(0.0)
            continue
        units = int(f16_units(np.array([v16]).view(np.uint16))[0])
        sb = fraction_to_f16_bits(Fraction(abs(units), 1 << 24) / 127)
        S = int(f16_units(np.array([sb], np.uint16))[0])
        codes.append(int(np.clip(rne_div(np.array([units]), S)[0], -127, 127)))
        scales.append(float(np.array([sb], np.uint16).view(np.float16)[0]))
    return np.array(codes, np.int64), np.array(scales, np.float64)


def w8a8_sel(x16, sel, vals):
    """fp64 W8A8 output (before any epilogue term) of x through sel_weight."""
    qa, sa = quant_rows_exact(x16)
    qw, sw = weight_codes(vals)
    acc = qa[:, np.asarray(sel)] * qw[None, :]           # one product per output: exact
    return acc.astype(np.float64) * sa[:, None] * sw[None, :]


def gelu(y):
    c = math.sqrt(2.0 / math.pi)
    return np.vectorize(lambda v: 0.5 * v * (1.0 + math.tanh(c * (v + 0.044715 * v ** 3))))(y)


def layer_norm(x16, gamma, beta, eps=1e-5):
    x = np.asarray(x16, np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * gamma.astype(np.float64) + beta.astype(np.float64)


def seq_mean(v16, seq):
    v = np.asarray(v16, np.float64)
    M, W = v.shape
    return np.repeat(v.reshape(M // seq, seq, W).mean(axis=1), seq, axis=0)


def pack(ws):
    return {k: oracle.qpack8(w) for k, w in ws.items()}


def _same16(a, b, what):
    assert np.array_equal(np.asarray(a, np.float16).view(np.uint16), np.asarray(b, np.float16).view(np.uint16)), what


def _close(a, b, what, tol=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert np.max(np.abs(a - b)) <= tol * max(1.0, float(np.max(np.abs(b)))), what


# ---- the identity-attention chain ---------------------------------------------------

W, F, M = 64, 128, 8


def _rng_sel(rng, K, N):
    return rng.permutation(np.resize(np.arange(K), N)) if N > K else rng.permutation(K)[:N]


def _chain_weights(seed, up_zero):
    rng = np.random.default_rng(seed)
    # three thirds of QKV with different selections and magnitudes, so each
    # third is a different function of h
    sel_q, sel_k, sel_v = (rng.permutation(W) for _ in range(3))
    vq = rng.choice([-2.0, 1.5], W)
    vk = rng.choice([0.75, -1.0], W)
    vv = rng.choice([0.5, -1.25, 1.0], W)
    sel_qkv = np.concatenate([sel_q, sel_k, sel_v])
    v_qkv = np.concatenate([vq, vk, vv])
    sel_o, v_o = rng.permutation(W), rng.choice([1.0, -0.75, 0.625], W)
    sel_u, v_u = _rng_sel(rng, W, F), rng.choice([1.0, -1.5, 2.0], F)
    if up_zero:
        v_u = np.zeros(F)
    sel_d, v_d = rng.permutation(F)[:W], rng.choice([0.5, -1.0, 0.875], W)
    return {
        "qkv": (sel_qkv, v_qkv), "o": (sel_o, v_o), "up": (sel_u, v_u), "down": (sel_d, v_d),
    }


def _dense(spec):
    shapes = {"qkv": (W, 3 * W), "o": (W, W), "up": (W, F), "down": (F, W)}
    return {k: sel_weight(*shapes[k], *spec[k]) for k in spec}


def _chain_expected(h, spec, d, alpha):
    qkv = _f16(w8a8_sel(h, *spec["qkv"]))
    a = qkv[:, 2 * W:3 * W]                                 # V third
    h1 = _f16(w8a8_sel(a, *spec["o"]) + h.astype(np.float64))
    u = _f16(gelu(w8a8_sel(h1, *spec["up"])))
    out64 = w8a8_sel(u, *spec["down"]) + h1.astype(np.float64)
    if d is not None and alpha != 0:
        out64 = out64 + np.float64(alpha) * d.astype(np.float64)
    return {"qkv": qkv, "a": a, "h1": h1, "u": u, "out64": out64}


@pytest.mark.parametrize("up_zero", [True, False])
def test_chain_closed_form(up_zero):
    """The whole chain against its closed form.  With MLP-up weights zero the
    MLP contributes exactly nothing, so the block output is h1 + alpha*d:
    that isolates the V third, the out-projection's residual (h) and the
    steering site; with them nonzero GELU's site and MLP-down's residual
    (h1) enter too."""
    rng = np.random.default_rng(11)
    h = _f16(rng.standard_normal((M, W)))
    d = rng.standard_normal(W)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    spec = _chain_weights(12, up_zero)
    got = oracle.dit_block_w8a8(h, pack(_dense(spec)), d=d, alpha=ALPHA)
    exp = _chain_expected(h, spec, d, ALPHA)
    for k in ("qkv", "a", "h1", "u"):
        _same16(got[k], exp[k], k)
    _close(got["out64"], exp["out64"], "out64")
    _same16(got["out"], _f16(exp["out64"]), "out")
    if up_zero:
        assert np.all(exp["u"] == 0)
        _close(got["out64"], exp["h1"].astype(np.float64) + np.float64(ALPHA) * d.astype(np.float64), "h1 + alpha d")


def test_chain_alpha_zero_is_bit_identical():
    """alpha = 0 gives exactly the unsteered block; the steered block differs
    from it only by alpha*d, and only in the block output."""
    rng = np.random.default_rng(21)
    h = _f16(rng.standard_normal((M, W)))
    ws = {"qkv": _f16(rng.standard_normal((W, 3 * W)) * 0.1), "o": _f16(rng.standard_normal((W, W)) * 0.1),
          "up": _f16(rng.standard_normal((W, F)) * 0.1), "down": _f16(rng.standard_normal((F, W)) * 0.1)}
    p = pack(ws)
    d = rng.standard_normal(W)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    r0 = oracle.dit_block_w8a8(h, p)
    rz = oracle.dit_block_w8a8(h, p, d=d, alpha=0.0)
    rs = oracle.dit_block_w8a8(h, p, d=d, alpha=ALPHA)
    for k in ("qkv", "a", "h1", "u", "out"):
        _same16(rz[k], r0[k], k)
    assert np.array_equal(rz["out64"], r0["out64"])
    for k in ("qkv", "a", "h1", "u"):
        _same16(rs[k], r0[k], k)
    _close(rs["out64"] - r0["out64"], np.broadcast_to(np.float64(ALPHA) * d.astype(np.float64), (M, W)),
           "steering adds alpha*d", tol=1e-14)


# ---- the full block (pre-norms, softmax attention) -----------------------------------

WF, HEADS, SEQ, MF = 128, 2, 8, 16     # two sequences of 8 tokens, two heads of 64


def _full_weights(seed, up_zero):
    rng = np.random.default_rng(seed)
    sel_v, v_v = rng.permutation(WF), rng.choice([0.5, -1.25, 1.0], WF)
    # Q and K thirds zero: every score is 0, so attention averages V over the sequence
    sel_qkv = np.concatenate([np.zeros(2 * WF, np.int64), sel_v])
    v_qkv = np.concatenate([np.zeros(2 * WF), v_v])
    sel_o, v_o = rng.permutation(WF), rng.choice([1.0, -0.75, 2.0], WF)
    sel_u, v_u = rng.permutation(np.resize(np.arange(WF), 2 * WF)), rng.choice([1.0, -1.5, 0.75], 2 * WF)
    if up_zero:
        v_u = np.zeros(2 * WF)
    sel_d, v_d = rng.permutation(2 * WF)[:WF], rng.choice([0.5, -1.0, 1.5], WF)
    spec = {"qkv": (sel_qkv, v_qkv), "o": (sel_o, v_o), "up": (sel_u, v_u), "down": (sel_d, v_d)}
    shapes = {"qkv": (WF, 3 * WF), "o": (WF, WF), "up": (WF, 2 * WF), "down": (2 * WF, WF)}
    return spec, {k: sel_weight(*shapes[k], *spec[k]) for k in spec}


@pytest.mark.parametrize("up_zero", [True, False])
def test_full_block_closed_form(up_zero):
    """LN1(h) feeds QKV; attention (zero queries and keys) averages V over
    each sequence; the out-projection adds h; LN2 reads h1 (with its own
    parameters); MLP-up applies GELU; MLP-down adds h1 and alpha*d."""
    rng = np.random.default_rng(31)
    h = _f16(rng.standard_normal((MF, WF)) * 1.5 + 0.25)
    ln1 = (_f16(1 + 0.2 * rng.standard_normal(WF)), _f16(0.2 * rng.standard_normal(WF)))
    ln2 = (_f16(1 + 0.2 * rng.standard_normal(WF)), _f16(0.2 * rng.standard_normal(WF)))
    d = rng.standard_normal(WF)
    d = (d / np.linalg.norm(d)).astype(np.float32)
    spec, dense = _full_weights(32, up_zero)
    got = oracle.dit_block_full_w8a8(h, pack(dense), ln1, ln2, HEADS, SEQ, d=d, alpha=ALPHA)

    n1 = _f16(layer_norm(h, *ln1))
    qkv = _f16(w8a8_sel(n1, *spec["qkv"]))
    assert np.all(qkv[:, :2 * WF] == 0)
    a = _f16(seq_mean(qkv[:, 2 * WF:], SEQ))
    h1 = _f16(w8a8_sel(a, *spec["o"]) + h.astype(np.float64))
    n2 = _f16(layer_norm(h1, *ln2))
    u = _f16(gelu(w8a8_sel(n2, *spec["up"])))
    out64 = w8a8_sel(u, *spec["down"]) + h1.astype(np.float64) + np.float64(ALPHA) * d.astype(np.float64)

    # the fp16 stage outputs agree bit for bit (LayerNorm and the softmax
    # average round differently in the last fp64 bits here and in the oracle,
    # which moves no fp16 value of these draws); the fp64 output to 1e-12
    for k, v in (("n1", n1), ("qkv", qkv), ("a", a), ("h1", h1), ("n2", n2), ("u", u)):
        _same16(got[k], v, k)
    _close(got["out64"], out64, "out64", tol=1e-12)
    if up_zero:
        assert np.all(u == 0)
