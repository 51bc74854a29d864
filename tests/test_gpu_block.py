"""GPU parity of the DiT block's steps around the linears (LayerNorm and
multi-head self-attention) through the C-ABI against the oracle, and of the
full W8A8 block (pre-norms, attention over two 1024-token sequences, 24 heads
of 64) at M = 2048: stage by stage (each GPU stage fed the GPU's own previous
stage, compared with the oracle's step on the same input) and end to end."""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from tests.gpu_util import assert_close, dev, host, log, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_diffusion_transformer_qlinear_amd as m
    return m


@pytest.mark.parametrize("M,W", [(1, 8), (5, 96), (33, 1536), (64, 6144), (3, 16384), (130, 520)])
def test_layernorm(q, M, W):
    rng = np.random.default_rng(M * 7 + W)
    x = (rng.standard_normal((M, W)) * 2 + 0.5).astype(np.float16)
    g = (1 + 0.1 * rng.standard_normal(W)).astype(np.float16)
    b = (0.1 * rng.standard_normal(W)).astype(np.float16)
    log(f"layernorm M={M} W={W}")
    y = q.layernorm(dev(x), dev(g), dev(b), 1e-5)
    assert_close(host(y), oracle.layernorm(x, g, b, 1e-5), f"layernorm {M}x{W}")


def test_layernorm_in_place(q):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((40, 1536)).astype(np.float16)
    g, b = np.ones(1536, np.float16), np.zeros(1536, np.float16)
    xd = dev(x)
    q.layernorm(xd, dev(g), dev(b), 1e-5, y=xd)
    assert_close(host(xd), oracle.layernorm(x, g, b, 1e-5), "layernorm in place")


@pytest.mark.parametrize("M,W", [(1, 32), (5, 96), (33, 1536), (130, 544), (3, 16384), (2051, 1536)])
def test_layernorm_quant(q, M, W):
    """The fused pre-norm + per-token quantization: y close to the oracle's
    LayerNorm, xq / s_a bit-exact with the oracle's quantization of that y,
    and all three bit-identical with the two separate kernels."""
    rng = np.random.default_rng(M * 11 + W)
    x = (rng.standard_normal((M, W)) * 2 + 0.5).astype(np.float16)
    x[0, :: max(1, W // 7)] = 40.0                       # one row with outliers
    g = (1 + 0.1 * rng.standard_normal(W)).astype(np.float16)
    b = (0.1 * rng.standard_normal(W)).astype(np.float16)
    log(f"layernorm_quant M={M} W={W}")
    xd, gd, bd = dev(x), dev(g), dev(b)
    y, xq, sa = q.layernorm_quant(xd, gd, bd, 1e-5, want_y=True)
    yh = host(y)
    assert_close(yh, oracle.layernorm(x, g, b, 1e-5), f"layernorm_quant y {M}x{W}")
    xq_ref, sa_ref = oracle.quant_act(yh)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(sa).view(np.uint16), sa_ref.view(np.uint16))
    y2 = q.layernorm(xd, gd, bd, 1e-5)
    xq2, sa2 = q.quant_act(y2)
    assert np.array_equal(host(y).view(np.uint16), host(y2).view(np.uint16))
    assert np.array_equal(host(xq), host(xq2))
    assert np.array_equal(host(sa).view(np.uint16), host(sa2).view(np.uint16))
    xq3, sa3 = q.layernorm_quant(xd, gd, bd, 1e-5)       # no y written
    assert np.array_equal(host(xq3), host(xq2))
    assert np.array_equal(host(sa3).view(np.uint16), host(sa2).view(np.uint16))


def test_layernorm_quant_in_place(q):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((70, 1536)).astype(np.float16)
    g, b = np.ones(1536, np.float16), np.zeros(1536, np.float16)
    xd = dev(x)
    _, xq, sa = q.layernorm_quant(xd, dev(g), dev(b), 1e-5, y=xd)
    yh = host(xd)
    assert_close(yh, oracle.layernorm(x, g, b, 1e-5), "layernorm_quant in place")
    xq_ref, sa_ref = oracle.quant_act(yh)
    assert np.array_equal(host(xq), xq_ref)
    assert np.array_equal(host(sa).view(np.uint16), sa_ref.view(np.uint16))


@pytest.mark.parametrize("M,K,N", [(1, 32, 8), (77, 1536, 4608), (2048, 1536, 6144), (300, 6144, 1536)])
def test_w8a8_prequant_matches_w8a8(q, M, K, N):
    """The linear on quantized-beforehand activations gives the W8A8 call's
    output bit for bit (same Xq / s_a, same GEMM and epilogue)."""
    import torch
    rng = np.random.default_rng(M + K + N)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    bias = (0.1 * rng.standard_normal(N)).astype(np.float16)
    res = rng.standard_normal((M, N)).astype(np.float16)
    d = rng.standard_normal(N).astype(np.float32)
    alpha = torch.tensor([0.25], dtype=torch.float32, device="cuda:0")
    log(f"w8a8_prequant M={M} K={K} N={N}")
    wq, sw = q.qpack(8, dev(w))
    xd = dev(x)
    epi = dict(bias=dev(bias), gelu=True, residual=dev(res), steer_dir=dev(d), steer_alpha=alpha)
    y_ref = q.qlinear_w8a8(xd, wq, sw, **epi)
    xq, sa = q.quant_act(xd)
    y = q.qlinear_w8a8_prequant(xq, sa, wq, sw, **epi)
    assert np.array_equal(host(y).view(np.uint16), host(y_ref).view(np.uint16))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    q.qlinear_w8a8_prequant(xq, sa, wq, sw, acc_out=acc)
    rows = sample_rows(M, 16, 1)
    assert np.array_equal(host(acc)[rows], oracle.gemm_i8(host(xq)[rows], host(wq)))


# the last shape launches 640 workgroups, past the two-per-CU mark where the
# kernel stops prefetching a block's fragments (both variants are covered);
# 40 and 1000 keys end in a partial key block, 40 in the second of two
@pytest.mark.parametrize("heads,seq,M", [(1, 1, 1), (1, 64, 64), (2, 100, 200), (3, 130, 130), (2, 257, 514),
                                         (4, 64, 256), (8, 128, 10240), (1, 40, 80), (3, 1000, 2000)])
def test_attention(q, heads, seq, M):
    rng = np.random.default_rng(heads * 1000 + seq)
    W = 64 * heads
    qkv = rng.standard_normal((M, 3 * W)).astype(np.float16)
    log(f"attention heads={heads} seq={seq} M={M}")
    out = q.attention(dev(qkv), heads, seq)
    assert_close(host(out), oracle.attention(qkv, heads, seq), f"attention h{heads} s{seq} m{M}")


def test_attention_zero_queries_average_values(q):
    """Q = 0 gives uniform weights: each output row is its sequence's mean V."""
    rng = np.random.default_rng(4)
    heads, seq, M, W = 2, 192, 384, 128
    qkv = rng.standard_normal((M, 3 * W)).astype(np.float16)
    qkv[:, :W] = 0
    out = host(q.attention(dev(qkv), heads, seq))
    v = qkv[:, 2 * W:].astype(np.float64).reshape(M // seq, seq, W)
    assert_close(out, np.repeat(v.mean(axis=1), seq, axis=0), "uniform attention")


def test_attention_large_scores(q):
    """Scores far beyond fp16 range of exp stay finite (the running max is subtracted)."""
    rng = np.random.default_rng(5)
    heads, seq, W = 1, 128, 64
    qkv = (rng.standard_normal((seq, 3 * W)) * 8).astype(np.float16)
    out = host(q.attention(dev(qkv), heads, seq))
    assert_close(out, oracle.attention(qkv, heads, seq), "large scores")


@pytest.fixture(scope="module")
def block(q):
    import torch
    from quantized_diffusion_transformer_qlinear_amd.chain import DitBlockFullW8A8
    blk = si.dit_block()
    norms = si.dit_block_norms()
    packed, opacked = {}, {}
    for k in ("qkv", "o", "up", "down"):
        packed[k] = q.qpack(8, dev(blk[k]))
        opacked[k] = oracle.qpack8(blk[k])
    ln1 = tuple(dev(a) for a in norms["ln1"])
    ln2 = tuple(dev(a) for a in norms["ln2"])
    alpha = torch.tensor([blk["alpha"]], dtype=torch.float32, device="cuda:0")
    chain = DitBlockFullW8A8(packed, ln1, ln2, si.TOKENS, si.WIDTH, si.MLP, si.HEADS, si.SEQ,
                             steer_dir=dev(blk["d"]), steer_alpha=alpha, keep_norms=True)
    chain.run(dev(blk["h"]))
    torch.cuda.synchronize()
    return blk, norms, opacked, chain


def test_block_stagewise(block):
    """Each stage of the GPU block against the oracle's step applied to the
    GPU's own input of that stage (sampled rows where the step is row-local)."""
    blk, norms, op, chain = block
    rows = sample_rows(si.TOKENS, 40, 6)
    h = blk["h"]
    log("block stage ln1")
    assert_close(host(chain.n1)[rows], oracle.layernorm(h[rows], *norms["ln1"]), "ln1")
    n1 = host(chain.n1)
    log("block stage qkv")
    assert_close(host(chain.qkv)[rows], oracle.qlinear_w8a8(n1[rows], *op["qkv"])["y"], "qkv")
    log("block stage attention (2 sequences x 24 heads x 1024 tokens)")
    assert_close(host(chain.a), oracle.attention(host(chain.qkv), si.HEADS, si.SEQ), "attention")
    a = host(chain.a)
    log("block stage out")
    assert_close(host(chain.h1)[rows], oracle.qlinear_w8a8(a[rows], *op["o"], residual=h[rows])["y"], "out")
    h1 = host(chain.h1)
    log("block stage ln2")
    assert_close(host(chain.n2)[rows], oracle.layernorm(h1[rows], *norms["ln2"]), "ln2")
    n2 = host(chain.n2)
    # the fused pre-norm's quantized rows (the up linear's input) are the
    # oracle's per-token quantization of the normalized rows it also wrote
    xq_ref, sa_ref = oracle.quant_act(n2[rows])
    assert np.array_equal(host(chain.xq)[rows], xq_ref), "ln2 xq"
    assert np.array_equal(host(chain.sa)[rows].view(np.uint16), sa_ref.view(np.uint16)), "ln2 s_a"
    log("block stage up")
    assert_close(host(chain.u)[rows], oracle.qlinear_w8a8(n2[rows], *op["up"], gelu=True)["y"], "up")
    u = host(chain.u)
    log("block stage down")
    ref = oracle.qlinear_w8a8(u[rows], *op["down"], residual=h1[rows], d=blk["d"], alpha=blk["alpha"])["y"]
    assert_close(host(chain.out)[rows], ref, "down")


def test_block_end_to_end(block):
    """The whole block against the oracle's own chain (fp16 at every stage).

    Bound: the per-step contract (5e-3 max-abs, 1e-3 Frobenius) is checked
    stage by stage above.  End to end, the GPU and the oracle feed each of the
    four activation quantizers inputs that differ by up to one fp16 ulp
    (2^-11 relative); a code then moves by one step where the input sits
    within an ulp of a rounding boundary — a fraction of about
    ulp / step = 2^-11 * 127 * |x| / max|x| (≈ 2-6 % of the codes) — and each
    such move changes that input's contribution by one quantization step
    (1/127 of the row's absmax).  Summed over K inputs of rms |x| / max|x| ≈ 0.25
    this is ≈ sqrt(0.04) * (1/127) / 0.25 ≈ 6e-3 relative per quantized stage,
    so the block output is held to 1e-2 (Frobenius) and 2e-2 (max-abs)."""
    blk, norms, op, chain = block
    log("block end to end (oracle chain over all 2048 rows)")
    ref = oracle.dit_block_full_w8a8(blk["h"], op, norms["ln1"], norms["ln2"], si.HEADS, si.SEQ,
                                     d=blk["d"], alpha=blk["alpha"])
    out = host(chain.out).astype(np.float64)
    r = ref["out64"]
    maxabs = float(np.max(np.abs(out - r))) / float(np.max(np.abs(r)))
    frob = float(np.linalg.norm(out - r) / np.linalg.norm(r))
    log(f"  block output: max-abs/max|ref| = {maxabs:.3e}, rel-Frobenius = {frob:.3e}")
    assert np.all(np.isfinite(out))
    assert maxabs <= 2e-2 and frob <= 1e-2, (maxabs, frob)
