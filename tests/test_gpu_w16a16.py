"""GPU parity of the fp16 rung (W16A16) through the C-ABI against the oracle:
the transposed weight copy bit-exact, the output within tolerance of the fp64
reference, across ragged shapes on both kernels (M <= 64 and tiled), every
epilogue term, steering strength 0 bit-identical, and the 1536 -> 6144 layer
at M = 2048 (sampled rows)."""
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


def _case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, K)).astype(np.float16), (rng.standard_normal((K, N)) * 0.05).astype(np.float16)


def run(q, x, w, e, rows=None):
    import torch
    wt, _ = q.qpack(16, dev(w))
    ref_wt = oracle.pack16(w)
    assert np.array_equal(host(wt).view(np.uint16), ref_wt.view(np.uint16)), "fp16 weight layout differs"
    kw = {}
    if "bias" in e:
        kw["bias"] = dev(e["bias"])
    if e.get("gelu"):
        kw["gelu"] = True
    if "residual" in e:
        kw["residual"] = dev(e["residual"])
    if "d" in e:
        kw["steer_dir"] = dev(e["d"])
        kw["steer_alpha"] = torch.tensor([e["alpha"]], dtype=torch.float32, device="cuda:0")
    y = q.qlinear_w16a16(dev(x), wt, **kw)
    rows = np.arange(x.shape[0]) if rows is None else rows
    res = e.get("residual")
    yref = oracle.epilogue(oracle.ref_w16a16(x[rows], ref_wt), bias=e.get("bias"), gelu=e.get("gelu", False),
                           residual=None if res is None else res[rows], d=e.get("d"), alpha=e.get("alpha", 0.0))
    return host(y)[rows], yref


SHAPES = [(1, 32, 1), (5, 96, 33), (16, 256, 130), (33, 1600, 64), (64, 288, 257), (65, 64, 96),
          (130, 544, 200), (257, 96, 129), (300, 1024, 160), (513, 320, 260), (700, 128, 384)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w16a16_ragged(q, M, K, N):
    log(f"w16a16 M={M} K={K} N={N}")
    x, w = _case(M, K, N, M * 41 + K * 3 + N)
    out, ref = run(q, x, w, {})
    assert_close(out, ref, f"w16a16 {M}x{K}x{N}")


@pytest.mark.parametrize("M", [16, 200])
@pytest.mark.parametrize("epi", ["bias", "gelu", "residual", "steer", "all"])
def test_w16a16_epilogue(q, M, epi):
    K, N = 192, 160
    x, w = _case(M, K, N, 5000 + M)
    rng = np.random.default_rng(7)
    e = {}
    if epi in ("bias", "all"):
        e["bias"] = (rng.standard_normal(N) * 0.1).astype(np.float16)
    if epi in ("gelu", "all"):
        e["gelu"] = True
    if epi in ("residual", "all"):
        e["residual"] = rng.standard_normal((M, N)).astype(np.float16)
    if epi in ("steer", "all"):
        e["d"], e["alpha"] = si.unit_direction(N, 11), 0.3
    out, ref = run(q, x, w, e)
    assert_close(out, ref, f"w16a16 {epi} M={M}")


@pytest.mark.parametrize("M", [16, 256])
def test_w16a16_alpha_zero_bit_identical(q, M):
    import torch
    x, w = _case(M, 256, 192, 99)
    wt, _ = q.qpack(16, dev(w))
    xd = dev(x)
    plain = q.qlinear_w16a16(xd, wt, gelu=True)
    alpha = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    s0 = q.qlinear_w16a16(xd, wt, gelu=True, steer_dir=dev(si.unit_direction(192, 4)), steer_alpha=alpha)
    assert host(plain).tobytes() == host(s0).tobytes()


def test_w16a16_full_width_m2048(q):
    """The 1536 -> 6144 layer at M = 2048 with bias and GELU (sampled rows)."""
    lin = si.mlp_up_w8a16()
    rows = sample_rows(lin.x.shape[0])
    log("w16a16 2048x1536x6144")
    out, ref = run(q, lin.x, lin.w, {"bias": lin.bias, "gelu": True}, rows)
    assert_close(out, ref, "w16a16 2048x1536x6144")


TILES = ["256x192x4x3", "256x256x4x4", "256x192x4x2", "256x128x4x2", "128x256x2x4", "128x192x2x2", "128x128x2x2",
         "64x192x2x2", "128x64x2x2", "64x128x2x2", "64x64x2x2", "64x96x2x3", "128x96x2x3", "128x128x2x4",
         # two K groups per workgroup (the fifth number)
         "64x192x2x2x2", "128x128x2x2x2", "128x64x2x2x2", "64x128x2x2x2", "64x96x2x3x2"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("N,K", [(460, 352), (520, 416), (460, 32)])
def test_w16a16_every_tile_variant(q, tile, N, K, monkeypatch):
    """Every macro-tile variant in fp16 mode (forced through the tuning
    override), with an even (K = 352: 6 K-steps of 64) and an odd (K = 416: 7)
    number of K-steps, the one-step case (K = 32), and both epilogue forms."""
    rng = np.random.default_rng(N + K)
    monkeypatch.setenv("ARIA_QLINEAR_TILE", tile)
    M = 300
    log(f"w16a16 tile {tile} {M}x{K}x{N}")
    x, w = _case(M, K, N, 4300 + N + K)
    e = {"bias": (rng.standard_normal(N) * 0.1).astype(np.float16), "gelu": True,
         "residual": rng.standard_normal((M, N)).astype(np.float16)}
    out, ref = run(q, x, w, e)
    assert_close(out, ref, f"w16a16 {tile} {M}x{K}x{N}")
