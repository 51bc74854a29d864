"""GPU parity of the W8A8 DiT block chain at full size (M = 2048, width 1536,
MLP 6144, residuals, GELU, steering alpha = 0.3 on the block output).

The chain is row-local (identity-attention stand-in), so the oracle runs it
on sampled token rows.  Two checks:
  - end to end: the GPU block output vs the oracle's fp64 output, within the
    fp tolerance (an upstream 1-ulp fp16 difference may legitimately move a
    downstream int8 code, so this stage is not bit-exact);
  - stage by stage: every GPU stage is fed the oracle's own fp16 stage input
    on the sampled rows, and its int8 activations, token scales and int32
    accumulators must equal the oracle's bit for bit (outputs within tolerance).
"""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from tests.gpu_util import assert_close, dev, host, log, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def setup():
    import torch

    import quantized_diffusion_transformer_qlinear_amd as q
    from quantized_diffusion_transformer_qlinear_amd.chain import DitBlockW8A8
    blk = si.dit_block()
    packed, opacked = {}, {}
    for k in ("qkv", "o", "up", "down"):
        packed[k] = q.qpack(8, dev(blk[k]))
        opacked[k] = oracle.qpack8(blk[k])
        assert np.array_equal(host(packed[k][0]), opacked[k][0]), k
        assert np.array_equal(host(packed[k][1]).view(np.uint16), opacked[k][1].view(np.uint16)), k
    alpha = torch.tensor([blk["alpha"]], dtype=torch.float32, device="cuda:0")
    chain = DitBlockW8A8(packed, 2048, si.WIDTH, si.MLP, steer_dir=dev(blk["d"]), steer_alpha=alpha)
    rows = sample_rows(2048, 40, 4)
    ref = oracle.dit_block_w8a8(blk["h"][rows], opacked, d=blk["d"], alpha=blk["alpha"])
    return q, blk, packed, opacked, chain, alpha, rows, ref


def test_chain_end_to_end(setup):
    q, blk, packed, opacked, chain, alpha, rows, ref = setup
    log("w8a8 DiT block chain 2048 x 1536 end to end")
    out = host(chain.run(dev(blk["h"])))
    assert_close(out[rows], ref["out64"], "chain output")


def test_chain_stagewise_bit_exact(setup):
    import torch
    q, blk, packed, opacked, chain, alpha, rows, ref = setup
    h = dev(blk["h"])
    chain.run(h)
    torch.cuda.synchronize()
    hh = blk["h"][rows]
    stages = [  # name, GPU stage input, oracle stage input, weights, epilogue (GPU buffers / oracle arrays)
        ("qkv", None, None, "qkv", {}),
        ("out", None, ref["a"], "o", {"residual": (h, hh)}),   # identity attention: the V third of qkv
        ("up", chain.h1, ref["h1"], "up", {"gelu": True}),
        ("down", chain.u, ref["u"], "down", {"residual": (chain.h1, ref["h1"]), "d": True}),
    ]
    for name, gin, oin, wk, e in stages:
        log(f"stage {name}")
        if name == "qkv":
            x_host, oin = blk["h"].copy(), hh
        else:
            W = packed["o"][0].shape[1]
            x_host = (host(chain.qkv)[:, 2 * W:] if name == "out" else host(gin)).copy()
            x_host[rows] = oin                    # the oracle's own stage input on the sampled rows
        x = dev(x_host)
        kw, okw = {}, {}
        if "residual" in e:
            rg, ro = e["residual"]
            r_host = host(rg).copy()
            r_host[rows] = ro
            kw["residual"] = dev(r_host)
            okw["residual"] = ro
        if e.get("gelu"):
            kw["gelu"] = okw["gelu"] = True
        if e.get("d"):
            kw["steer_dir"], kw["steer_alpha"] = dev(blk["d"]), alpha
            okw["d"], okw["alpha"] = blk["d"], blk["alpha"]
        M, N = x.shape[0], packed[wk][0].shape[0]
        acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
        xq_g, sa_g = q.quant_act(x)
        y = q.qlinear_w8a8(x, *packed[wk], acc_out=acc, **kw)
        o = oracle.qlinear_w8a8(oin, *opacked[wk], **okw)
        assert np.array_equal(host(xq_g)[rows], o["xq"]), name
        assert np.array_equal(host(sa_g)[rows].view(np.uint16), o["sa"].view(np.uint16)), name
        assert np.array_equal(host(acc)[rows], o["acc"]), name
        assert_close(host(y)[rows], o["y"], f"stage {name}")


def test_chain_alpha_zero_matches_unsteered(setup):
    import torch

    from quantized_diffusion_transformer_qlinear_amd.chain import DitBlockW8A8
    q, blk, packed, opacked, chain, alpha, rows, ref = setup
    h = dev(blk["h"])
    zero = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    c0 = DitBlockW8A8(packed, 2048, si.WIDTH, si.MLP, steer_dir=dev(blk["d"]), steer_alpha=zero)
    c1 = DitBlockW8A8(packed, 2048, si.WIDTH, si.MLP)
    a, b = host(c0.run(h)), host(c1.run(h))
    assert a.tobytes() == b.tobytes()
