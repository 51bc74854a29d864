"""The per-token quantization fused into the linears around it (through the
C-ABI): the producer W8A8 call records the row maxima of a column block of its
output, and the consumer W8A8 call quantizes that block while it stages it.

Bit-exact checks:
  - the producer's Y equals the plain W8A8 call's, and its row maxima equal
    the fp16 magnitude bits recomputed on the host from that Y;
  - the consumer's Y and token scales equal the separate strided quantization
    followed by the linear on the quantized input, on GEMM-produced inputs
    and on hand-built inputs full of exact quantization ties;
  - the W8A8 block chain with the fused out-projection gives the same output
    bits as the chain with the separate quantization pass.
Ragged M and several tile shapes are covered.
"""
import numpy as np
import pytest

import synthetic_inputs as si
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_diffusion_transformer_qlinear_amd as m
    return m


def _mag_blocks(y, c0, nc):
    """Host row maxima of |y| over 64-column blocks, as fp16 magnitude bits."""
    b = (y[:, c0:c0 + nc].view(np.uint16) & 0x7FFF).astype(np.int64)
    return b.reshape(y.shape[0], nc // 64, 64).max(axis=2).astype(np.int32)


def _weights(q, K, N, seed, scale=0.05):
    w = (np.random.default_rng(seed).standard_normal((K, N)) * scale).astype(np.float16)
    return q.qpack(8, dev(w))


@pytest.mark.parametrize("M,K,W3,c0,nc", [(300, 256, 768, 512, 256), (2048, 1536, 4608, 3072, 1536),
                                           (77, 128, 384, 0, 384), (130, 512, 1024, 448, 512)])
def test_producer_rowmax(q, M, K, W3, c0, nc):
    log(f"rowmax producer {M}x{K}x{W3} cols [{c0}, {c0 + nc})")
    x = dev(np.random.default_rng(M + K).standard_normal((M, K)).astype(np.float16))
    wq, sw = _weights(q, K, W3, 11 + K)
    y0 = q.qlinear_w8a8(x, wq, sw)
    y, rm = q.qlinear_w8a8_rowmax(x, wq, sw, c0, nc)
    yh = host(y)
    assert np.array_equal(yh.view(np.uint16), host(y0).view(np.uint16))
    assert np.array_equal(host(rm), _mag_blocks(yh, c0, nc))


@pytest.mark.parametrize("M,K,N,epi", [(2048, 1536, 1536, "residual"), (300, 256, 520, "bias_gelu"),
                                       (77, 64, 256, None), (513, 512, 1536, "steer"), (64, 1536, 4608, None),
                                       (256, 1536, 6144, "bias_gelu")])
def test_consumer_matches_quantize_then_linear(q, M, K, N, epi):
    import torch
    log(f"fused consumer {M}x{K}x{N} epi={epi}")
    rng = np.random.default_rng(M * 7 + N)
    W3 = 3 * K
    # a GEMM-produced input: the V third of a W8A8 output, with its row maxima
    x = dev(rng.standard_normal((M, K)).astype(np.float16))
    wq3, sw3 = _weights(q, K, W3, 5 + K)
    src, rm = q.qlinear_w8a8_rowmax(x, wq3, sw3, 2 * K, K)
    wq, sw = _weights(q, K, N, 9 + N)
    kw = {}
    if epi == "residual":
        kw["residual"] = dev(rng.standard_normal((M, N)).astype(np.float16))
    elif epi == "bias_gelu":
        kw.update(bias=dev((rng.standard_normal(N) * 0.1).astype(np.float16)), gelu=True)
    elif epi == "steer":
        kw.update(steer_dir=dev(si.unit_direction(N, 3)),
                  steer_alpha=torch.tensor([0.3], dtype=torch.float32, device="cuda:0"))
    xq, sa = q.quant_act_columns(src, 2 * K, K)
    y_ref = q.qlinear_w8a8_prequant(xq, sa, wq, sw, **kw)
    sa_out = torch.empty((M,), dtype=torch.float16, device="cuda:0")
    y = q.qlinear_w8a8_fused(src, 2 * K, K, rm, wq, sw, sa_out=sa_out, **kw)
    assert np.array_equal(host(sa_out).view(np.uint16), host(sa).view(np.uint16))
    assert np.array_equal(host(y).view(np.uint16), host(y_ref).view(np.uint16))


def test_consumer_on_exact_ties(q):
    """Hand-built rows whose scale is a power of two c (max |x| = 127 c) and
    whose other values are exact ties (k + 1/2) c, mixed with random rows and
    an all-zero row: the quantized codes decide y, so bit-identical y means
    bit-identical codes."""
    import torch
    M, K, N, ld = 192, 256, 256, 320
    rng = np.random.default_rng(4)
    X = np.zeros((M, ld), np.float32)
    for m in range(M):
        if m % 3 == 0:
            c = 2.0 ** int(rng.integers(-12, -2))
            k = rng.integers(-127, 127, ld).astype(np.float64)
            X[m] = (k + 0.5) * c
            X[m, int(rng.integers(0, K))] = 127 * c * (1 if m % 2 else -1)
        elif m % 3 == 1:
            X[m] = rng.standard_normal(ld) * 0.7
    X[5] = 0.0
    Xh = X.astype(np.float16)
    src = dev(Xh)
    # the row maxima a producer would have written for columns [0, K)
    rm = dev(_mag_blocks(Xh, 0, K))
    wq, sw = _weights(q, K, N, 21)
    xq_ref, sa_ref = q.quant_act_columns(src, 0, K)
    y_ref = q.qlinear_w8a8_prequant(xq_ref, sa_ref, wq, sw)
    sa_out = torch.empty((M,), dtype=torch.float16, device="cuda:0")
    y = q.qlinear_w8a8_fused(src, 0, K, rm, wq, sw, sa_out=sa_out)
    assert np.array_equal(host(sa_out).view(np.uint16), host(sa_ref).view(np.uint16))
    assert np.array_equal(host(y).view(np.uint16), host(y_ref).view(np.uint16))
    # the ties really are there: some codes sit at k + 1/2 before rounding
    assert int((np.abs(Xh[::3, :K].astype(np.float64)) > 0).sum()) > 0


def test_chain_with_fused_out_projection_is_bit_identical(q):
    import torch

    from quantized_diffusion_transformer_qlinear_amd.chain import DitBlockW8A8
    log("W8A8 block chain 2048 x 1536: fused out-projection quantization vs separate pass")
    blk = si.dit_block()
    packed = {k: q.qpack(8, dev(blk[k])) for k in ("qkv", "o", "up", "down")}
    alpha = torch.tensor([blk["alpha"]], dtype=torch.float32, device="cuda:0")
    h = dev(blk["h"])
    plain = DitBlockW8A8(packed, 2048, si.WIDTH, si.MLP, steer_dir=dev(blk["d"]), steer_alpha=alpha)
    fused = DitBlockW8A8(packed, 2048, si.WIDTH, si.MLP, steer_dir=dev(blk["d"]), steer_alpha=alpha,
                         fuse_out_quant=True)
    a = host(plain.run(h)).view(np.uint16).copy()
    b = host(fused.run(h)).view(np.uint16).copy()
    assert np.array_equal(host(fused.h1).view(np.uint16), host(plain.h1).view(np.uint16))
    assert np.array_equal(a, b)
