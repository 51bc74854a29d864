"""GPU parity of the grouped small-M call (several independent weight-only
linears in one launch per 16 problems) through the C-ABI: every problem's
output within tolerance of the oracle and bit-identical to the single call
on the same problem; ragged shapes, every epilogue term, more problems than
one launch takes, an in-place residual, graph capture, and the 4-bit layer of
the width-1536 block at M = 16 in full."""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from tests.gpu_util import assert_close, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_diffusion_transformer_qlinear_amd as m
    return m


def _problem(q, bits, M, K, N, seed, epi=()):
    import torch
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    wq, s = q.qpack(bits, dev(w))
    p = {"x": dev(x), "wq": wq, "s": s}
    e = {}
    if "bias" in epi:
        e["bias"] = (rng.standard_normal(N) * 0.1).astype(np.float16)
        p["bias"] = dev(e["bias"])
    if "gelu" in epi:
        e["gelu"] = True
        p["gelu"] = True
    if "residual" in epi:
        e["residual"] = rng.standard_normal((M, N)).astype(np.float16)
        p["residual"] = dev(e["residual"])
    if "steer" in epi:
        e["d"], e["alpha"] = si.unit_direction(N, seed + 3), 0.3
        p["steer_dir"] = dev(e["d"])
        p["steer_alpha"] = torch.tensor([0.3], dtype=torch.float32, device="cuda:0")
    return x, w, e, p


def _oracle(bits, x, w, e):
    if bits == 8:
        rq, rs = oracle.qpack8(w)
        r = oracle.ref_w8a16(x, rq, rs)
    else:
        rq, rs = oracle.qpack4(w, 32)
        r = oracle.ref_w4a16(x, rq, rs, 32)
    return oracle.epilogue(r, bias=e.get("bias"), gelu=e.get("gelu", False), residual=e.get("residual"),
                           d=e.get("d"), alpha=e.get("alpha", 0.0))


def _single(q, bits, p):
    f = q.qlinear_w8a16 if bits == 8 else q.qlinear_w4a16
    kw = {k: v for k, v in p.items() if k not in ("x", "wq", "s", "y")}
    return f(p["x"], p["wq"], p["s"], **kw)


MIXED = [(1, 32, 1, ()), (5, 96, 33, ("bias",)), (16, 256, 130, ("gelu",)), (33, 160, 64, ("residual",)),
         (64, 288, 257, ("steer",)), (17, 1536, 520, ("bias", "gelu", "residual", "steer")), (2, 64, 16, ())]


@pytest.mark.parametrize("bits", [8, 4])
def test_grouped_mixed(q, bits):
    probs = [_problem(q, bits, M, K, N, 900 + 13 * i + bits, epi) for i, (M, K, N, epi) in enumerate(MIXED)]
    log(f"grouped w{bits}a16: {len(probs)} problems")
    outs = q.qlinear_grouped(bits, [p for _, _, _, p in probs])
    for i, ((x, w, e, p), y) in enumerate(zip(probs, outs)):
        M, K, N, _ = MIXED[i]
        assert_close(host(y), _oracle(bits, x, w, e), f"grouped w{bits}a16 #{i} {M}x{K}x{N}")
        assert host(y).tobytes() == host(_single(q, bits, p)).tobytes(), f"problem {i} differs from the single call"


def test_grouped_more_than_one_launch(q):
    """37 problems: two launches of at most 32; each equals its single call."""
    shapes = [(1 + (i * 7) % 64, 32 * (1 + i % 5), 1 + (i * 29) % 300) for i in range(37)]
    probs = [_problem(q, 4, M, K, N, 3000 + i) for i, (M, K, N) in enumerate(shapes)]
    log(f"grouped w4a16: {len(probs)} problems")
    outs = q.qlinear_grouped(4, [p for _, _, _, p in probs])
    for i, ((x, w, e, p), y) in enumerate(zip(probs, outs)):
        assert host(y).tobytes() == host(_single(q, 4, p)).tobytes(), f"problem {i} {shapes[i]}"
    for i in (0, 17, 36):
        x, w, e, _ = probs[i]
        assert_close(host(outs[i]), _oracle(4, x, w, e), f"grouped #{i} {shapes[i]}")


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N,epi", [(9, 512, 4104, ("bias", "gelu", "residual", "steer")),
                                       (16, 1536, 6144, ()), (16, 256, 8192, ("residual",))])
def test_single_call_two_groups(q, bits, M, K, N, epi):
    """Widths where the single call at M > 8 gives each workgroup two 16-channel
    groups (one to two workgroups per CU on a 256-CU device; N = 4104 leaves
    the last workgroup half a group): within tolerance of the oracle and
    bit-identical to the grouped call, whose workgroups take more groups."""
    x, w, e, p = _problem(q, bits, M, K, N, 4100 + M + bits, epi)
    log(f"single w{bits}a16 {M}x{K}x{N} {epi}")
    y = _single(q, bits, p)
    assert_close(host(y), _oracle(bits, x, w, e), f"single w{bits}a16 {M}x{K}x{N}")
    g = q.qlinear_grouped(bits, [p])[0]
    assert host(y).tobytes() == host(g).tobytes(), "single and grouped calls differ"


def test_grouped_in_place_residual(q):
    x, w, e, p = _problem(q, 4, 24, 320, 96, 77, ("residual",))
    h = p["residual"]
    p["y"] = h
    q.qlinear_grouped(4, [p])
    assert_close(host(h), _oracle(4, x, w, e), "grouped in-place residual")


def test_grouped_graph_replay(q):
    import torch
    probs = [_problem(q, 4, M, K, N, 500 + i) for i, (M, K, N) in enumerate([(16, 256, 192), (8, 512, 64), (16, 96, 33)])]
    ps = [p for _, _, _, p in probs]
    eager = [host(y).tobytes() for y in q.qlinear_grouped(4, ps)]
    for p in ps:
        p["y"] = torch.zeros((p["x"].shape[0], p["wq"].shape[0]), dtype=torch.float16, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            q.qlinear_grouped(4, ps)
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        for p in ps:
            p["y"].fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert [host(p["y"]).tobytes() for p in ps] == eager, f"replay {rep}"


def test_grouped_w4a16_block_width_m16(q):
    """Three 1536 -> 6144 4-bit layers (the W4A16 workload's weight shape) at
    M = 16 in one launch, every output element against the oracle."""
    x = si.w4a16_sweep_x()[:16]
    ws = [si.w4a16_w()] + [(np.random.default_rng(310 + i).standard_normal((1536, 6144)) * 0.02).astype(np.float16)
                          for i in range(2)]
    ps = []
    for w in ws:
        wq, s = q.qpack(4, dev(w))
        ps.append({"x": dev(x), "wq": wq, "s": s})
    log("grouped w4a16 3 x 16x1536x6144")
    outs = q.qlinear_grouped(4, ps)
    for i, (w, y) in enumerate(zip(ws, outs)):
        rq, rs = oracle.qpack4(w, 32)
        assert_close(host(y), oracle.ref_w4a16(x, rq, rs, 32), f"layer {i}")
