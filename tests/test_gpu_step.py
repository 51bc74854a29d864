"""GPU parity of the 1.2B-parameter-scale denoising step: 24 blocks x {QKV
2048->6144, out 2048->2048, MLP-up 2048->8192, MLP-down 8192->2048}, every
linear packed at 8 and at 4 bits on the GPU (fp16 copy released right after
packing), run over M = 2048 tokens in W8A16, W4A16 and W8A8.

Packed bytes are compared bit-exactly with the oracle on sampled output
channels (each channel is packed independently), and every output is compared
on sampled (row, channel) blocks, which the oracle computes from the sampled
rows and the sampled channels alone.  The resident footprint after packing
equals the packed sizes exactly (project page, "What aria is": the
full-precision copy is released once packed)."""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from tests.gpu_util import assert_close, dev, host, log, sample_rows

pytestmark = pytest.mark.gpu

ROWS = sample_rows(2048, 13, 5)          # 16 rows
NCOLS = 96


@pytest.fixture(scope="module")
def xs():
    return {k: si.step_x(k) for k in (si.STEP_WIDTH, si.STEP_MLP)}


@pytest.fixture(scope="module")
def xs_dev(xs):
    return {k: dev(v) for k, v in xs.items()}


@pytest.mark.parametrize("block", range(si.STEP_BLOCKS))
def test_step_block(block, xs, xs_dev):
    import torch

    import quantized_diffusion_transformer_qlinear_amd as q
    for layer, (name, K, N) in enumerate(si.STEP_LAYERS):
        log(f"block {block} {name} {K}->{N}")
        w = si.step_weight(block, layer)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        wd = dev(w)
        q8 = q.qpack(8, wd)
        q4 = q.qpack(4, wd)
        del wd
        torch.cuda.synchronize()
        qb8, sb8 = q.qpack_bytes(8, 0, K, N)
        qb4, sb4 = q.qpack_bytes(4, 32, K, N)
        assert torch.cuda.memory_allocated() - base == qb8 + sb8 + qb4 + sb4, "fp16 copy not released"

        cols = np.sort(np.random.default_rng(block * 10 + layer).choice(N, NCOLS, replace=False))
        wc = np.ascontiguousarray(w[:, cols])
        o8, os8 = oracle.qpack8(wc)
        o4, os4 = oracle.qpack4(wc, 32)
        assert np.array_equal(host(q8[0])[cols], o8) and np.array_equal(host(q8[1])[cols].view(np.uint16), os8.view(np.uint16))
        assert np.array_equal(host(q4[0])[cols], o4) and np.array_equal(host(q4[1])[cols].view(np.uint16), os4.view(np.uint16))

        x, xd = xs[K], xs_dev[K]
        xr = x[ROWS]
        y8 = host(q.qlinear_w8a16(xd, *q8))[ROWS][:, cols]
        assert_close(y8, oracle.ref_w8a16(xr, o8, os8), f"w8a16 b{block} {name}")
        y4 = host(q.qlinear_w4a16(xd, *q4))[ROWS][:, cols]
        assert_close(y4, oracle.ref_w4a16(xr, o4, os4, 32), f"w4a16 b{block} {name}")
        acc = torch.empty((2048, N), dtype=torch.int32, device="cuda:0")
        ya = host(q.qlinear_w8a8(xd, *q8, acc_out=acc))[ROWS][:, cols]
        ref = oracle.qlinear_w8a8(xr, o8, os8)
        assert np.array_equal(host(acc)[ROWS][:, cols], ref["acc"])
        assert_close(ya, ref["y"], f"w8a8 b{block} {name}")
        del q8, q4, acc
