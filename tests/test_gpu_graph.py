"""The C-ABI calls capture into a HIP graph and replay correctly.

The pages replay the denoising loop as one captured graph and change the
steering strength while streaming, inside the captured graph (project page,
"What aria is": the loop is replayed as one graph; "Results", "Live steering
while streaming").  Here the W8A8 block chain plus a W8A16 and a W4A16 layer
are captured once; every replay (with unrelated eager work in between) must
match the eager result bit for bit, and writing a new alpha into the device
scalar between replays must change the steered output exactly as an eager
call with that alpha does.  Captured on one stream, and as the benchmark
captures its step: the chain on a forked stream, the weight-only layers on
the capturing stream, as parallel branches of the graph."""
import numpy as np
import pytest

import synthetic_inputs as si
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("branched", [False, True])
def test_graph_replay_matches_eager(branched):
    import torch

    import quantized_diffusion_transformer_qlinear_amd as q
    from quantized_diffusion_transformer_qlinear_amd.chain import DitBlockW8A8
    M = 512
    blk = si.dit_block()
    packed = {k: q.qpack(8, dev(blk[k])) for k in ("qkv", "o", "up", "down")}
    alpha = torch.tensor([0.3], dtype=torch.float32, device="cuda:0")
    chain = DitBlockW8A8(packed, M, si.WIDTH, si.MLP, steer_dir=dev(blk["d"]), steer_alpha=alpha)
    h = dev(blk["h"][:M])
    lin = si.mlp_up_w8a16()
    x2, b2 = dev(lin.x[:M]), dev(lin.bias)
    wq2, sw2 = q.qpack(8, dev(lin.w))
    wq4, sg4 = q.qpack(4, dev(si.w4a16_w()))
    x4 = dev(si.w4a16_sweep_x()[:16])
    y2 = torch.empty((M, si.MLP), dtype=torch.float16, device="cuda:0")
    y4 = torch.empty((16, si.MLP), dtype=torch.float16, device="cuda:0")

    side = torch.cuda.Stream()

    def step(fork=False):
        cur = torch.cuda.current_stream()
        if fork:
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                chain.run(h)
        else:
            chain.run(h)
        q.qlinear_w8a16(x2, wq2, sw2, y=y2, bias=b2, gelu=True)
        q.qlinear_w4a16(x4, wq4, sg4, y=y4)
        if fork:
            cur.wait_stream(side)

    def outputs():
        return host(chain.out).tobytes(), host(y2).tobytes(), host(y4).tobytes()

    step()
    eager = outputs()
    alpha.fill_(0.0)
    step()
    eager_a0 = outputs()
    alpha.fill_(0.3)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step(fork=branched)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()

    other = dev(np.random.default_rng(0).standard_normal((64, si.WIDTH)).astype(np.float16))
    for rep in range(4):
        log(f"replay {rep} (branched {branched})")
        for buf in (chain.out, y2, y4):
            buf.fill_(0)
        q.qlinear_w8a16(other, wq2, sw2)   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert outputs() == eager, f"replay {rep} differs from the eager result"

    alpha.fill_(0.0)                       # live steering change, no re-capture
    g.replay()
    torch.cuda.synchronize()
    assert outputs() == eager_a0
    alpha.fill_(0.3)
    g.replay()
    torch.cuda.synchronize()
    assert outputs() == eager
