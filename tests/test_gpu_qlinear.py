"""GPU parity of the three qlinear modes through the C-ABI against the oracle:
W8A8 (per-token int8 activations and the int32 accumulators bit-exact, fp16
output within tolerance), W8A16 and W4A16 (fp16 output within tolerance of the
fp64 reference of the same quantized weights); ragged shapes spanning several
tiles, every epilogue term, steering strength 0 bit-identical to no steering,
and the DiT-width layers at their full sizes (sampled rows)."""
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


def _rand(M, K, N, seed, wsig=0.05):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((K, N)) * wsig).astype(np.float16)
    return x, w


def _epi_inputs(M, N, seed, bias=False, gelu=False, residual=False, steer=False, alpha=0.3):
    rng = np.random.default_rng(seed + 17)
    e = {}
    if bias:
        e["bias"] = (rng.standard_normal(N) * 0.1).astype(np.float16)
    if gelu:
        e["gelu"] = True
    if residual:
        e["residual"] = rng.standard_normal((M, N)).astype(np.float16)
    if steer:
        e["d"] = si.unit_direction(N, seed + 5)
        e["alpha"] = alpha
    return e


def _dev_epi(e):
    import torch
    out = {}
    if "bias" in e:
        out["bias"] = dev(e["bias"])
    if e.get("gelu"):
        out["gelu"] = True
    if "residual" in e:
        out["residual"] = dev(e["residual"])
    if "d" in e:
        out["steer_dir"] = dev(e["d"])
        out["steer_alpha"] = torch.tensor([e["alpha"]], dtype=torch.float32, device="cuda:0")
    return out


def run_w8a8(q, x, w, e, rows=None):
    """GPU and oracle W8A8; rows = sampled rows for the oracle's contraction."""
    import torch
    M, K = x.shape
    N = w.shape[1]
    wq, sw = q.qpack(8, dev(w))
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
    y = q.qlinear_w8a8(dev(x), wq, sw, acc_out=acc, **_dev_epi(e))
    ref_q, ref_s = oracle.qpack8(w)
    assert np.array_equal(host(wq), ref_q) and np.array_equal(host(sw).view(np.uint16), ref_s.view(np.uint16))
    rows = np.arange(M) if rows is None else rows
    xq, sa = oracle.quant_act(x)
    ref_acc = oracle.gemm_i8(xq[rows], ref_q)
    gacc = host(acc)[rows]
    assert np.array_equal(gacc, ref_acc), f"int32 accumulators differ at {np.argwhere(gacc != ref_acc)[:4]}"
    res = e.get("residual")
    yref = oracle.epilogue(oracle.scale_w8a8(ref_acc, sa[rows], ref_s), bias=e.get("bias"), gelu=e.get("gelu", False),
                           residual=None if res is None else res[rows], d=e.get("d"), alpha=e.get("alpha", 0.0))
    return host(y)[rows], yref


def run_wxa16(q, bits, x, w, e, rows=None):
    M, K = x.shape
    wq, s = q.qpack(bits, dev(w))
    f = q.qlinear_w8a16 if bits == 8 else q.qlinear_w4a16
    y = f(dev(x), wq, s, **_dev_epi(e))
    if bits == 8:
        ref_q, ref_s = oracle.qpack8(w)
    else:
        ref_q, ref_s = oracle.qpack4(w, 32)
    assert np.array_equal(host(wq), ref_q) and np.array_equal(host(s).view(np.uint16), ref_s.view(np.uint16))
    rows = np.arange(M) if rows is None else rows
    r = oracle.ref_w8a16(x[rows], ref_q, ref_s) if bits == 8 else oracle.ref_w4a16(x[rows], ref_q, ref_s, 32)
    res = e.get("residual")
    yref = oracle.epilogue(r, bias=e.get("bias"), gelu=e.get("gelu", False),
                           residual=None if res is None else res[rows], d=e.get("d"), alpha=e.get("alpha", 0.0))
    return host(y)[rows], yref


SHAPES = [(1, 32, 1), (5, 96, 33), (16, 256, 130), (33, 160, 64), (64, 288, 257), (65, 64, 96),
          (130, 544, 200), (257, 96, 129), (300, 1024, 160), (513, 320, 260), (700, 128, 384)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w8a8_ragged(q, M, K, N):
    log(f"w8a8 M={M} K={K} N={N}")
    x, w = _rand(M, K, N, M * 31 + K * 7 + N)
    out, ref = run_w8a8(q, x, w, {})
    assert_close(out, ref, f"w8a8 {M}x{K}x{N}")


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_wxa16_ragged(q, bits, M, K, N):
    log(f"w{bits}a16 M={M} K={K} N={N}")
    x, w = _rand(M, K, N, M * 37 + K * 5 + N + bits)
    out, ref = run_wxa16(q, bits, x, w, {})
    assert_close(out, ref, f"w{bits}a16 {M}x{K}x{N}")


EPIS = [dict(bias=True), dict(gelu=True), dict(bias=True, gelu=True), dict(residual=True),
        dict(steer=True), dict(bias=True, gelu=True, residual=True, steer=True)]


@pytest.mark.parametrize("mode", ["w8a8", "w8a16", "w4a16"])
@pytest.mark.parametrize("M", [16, 48, 200])
@pytest.mark.parametrize("ei", range(len(EPIS)))
def test_epilogue_terms(q, mode, M, ei):
    K, N = 192, 160
    log(f"{mode} epilogue {EPIS[ei]} M={M}")
    x, w = _rand(M, K, N, 1000 + ei + M)
    e = _epi_inputs(M, N, ei, **EPIS[ei])
    if mode == "w8a8":
        out, ref = run_w8a8(q, x, w, e)
    else:
        out, ref = run_wxa16(q, 8 if mode == "w8a16" else 4, x, w, e)
    assert_close(out, ref, f"{mode} epi{ei}")


@pytest.mark.parametrize("mode", ["w8a8", "w8a16", "w4a16"])
@pytest.mark.parametrize("M", [16, 256])
def test_alpha_zero_bit_identical(q, mode, M):
    """Strength 0 removes the steering term with bit-identical output."""
    import torch
    K, N = 256, 192
    x, w = _rand(M, K, N, 77 + M)
    res = np.random.default_rng(1).standard_normal((M, N)).astype(np.float16)
    bits = 4 if mode == "w4a16" else 8
    wq, s = q.qpack(bits, dev(w))
    f = {"w8a8": q.qlinear_w8a8, "w8a16": q.qlinear_w8a16, "w4a16": q.qlinear_w4a16}[mode]
    xd, rd = dev(x), dev(res)
    plain = f(xd, wq, s, gelu=True, residual=rd)
    alpha = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    steered0 = f(xd, wq, s, gelu=True, residual=rd, steer_dir=dev(si.unit_direction(N, 3)), steer_alpha=alpha)
    assert host(plain).tobytes() == host(steered0).tobytes()
    alpha.fill_(0.5)  # the same call with a changed device-side alpha now differs
    steered = f(xd, wq, s, gelu=True, residual=rd, steer_dir=dev(si.unit_direction(N, 3)), steer_alpha=alpha)
    assert host(plain).tobytes() != host(steered).tobytes()


@pytest.mark.parametrize("mode", ["w8a8", "w8a16", "w4a16"])
def test_residual_in_place(q, mode):
    """residual == y: h += linear(x) in place."""
    M, K, N = 96, 128, 160
    x, w = _rand(M, K, N, 55)
    h = np.random.default_rng(2).standard_normal((M, N)).astype(np.float16)
    bits = 4 if mode == "w4a16" else 8
    wq, s = q.qpack(bits, dev(w))
    hd = dev(h)
    f = {"w8a8": q.qlinear_w8a8, "w8a16": q.qlinear_w8a16, "w4a16": q.qlinear_w4a16}[mode]
    f(dev(x), wq, s, y=hd, residual=hd)
    if mode == "w8a8":
        xq, sa = oracle.quant_act(x)
        rq, rs = oracle.qpack8(w)
        ref = oracle.epilogue(oracle.scale_w8a8(oracle.gemm_i8(xq, rq), sa, rs), residual=h)
    elif mode == "w8a16":
        rq, rs = oracle.qpack8(w)
        ref = oracle.epilogue(oracle.ref_w8a16(x, rq, rs), residual=h)
    else:
        rq, rs = oracle.qpack4(w, 32)
        ref = oracle.epilogue(oracle.ref_w4a16(x, rq, rs, 32), residual=h)
    assert_close(host(hd), ref, f"{mode} in-place residual")


def test_identity_weights(q):
    """Permutation weights give closed-form outputs through every mode."""
    M, K = 96, 256
    perm = np.random.default_rng(8).permutation(K)
    w = np.zeros((K, K), np.float16)
    w[perm, np.arange(K)] = 1.0
    x = np.random.default_rng(9).standard_normal((M, K)).astype(np.float16)
    xs = x.astype(np.float64)[:, perm]
    out, _ = run_wxa16(q, 8, x, w, {})
    assert_close(out, xs * 0.99993896484375, "w8a16 identity")
    out, _ = run_wxa16(q, 4, x, w, {})
    assert_close(out, xs * 0.999755859375, "w4a16 identity")
    import torch
    wq, sw = q.qpack(8, dev(w))
    acc = torch.empty((M, K), dtype=torch.int32, device="cuda:0")
    q.qlinear_w8a8(dev(x), wq, sw, acc_out=acc)
    xq, _ = oracle.quant_act(x)
    assert np.array_equal(host(acc), 127 * xq.astype(np.int32)[:, perm])


# ---------------------------------------------------------------------------
# the DiT-width workloads at full size (oracle on sampled rows)
# ---------------------------------------------------------------------------
def test_small_w8a8_full(q):
    lin = si.small_w8a8()
    log("w8a8 64x256x256 (all outputs)")
    out, ref = run_w8a8(q, lin.x, lin.w, {})
    assert_close(out, ref, "w8a8 64x256x256")


def test_mlp_up_w8a16_full_size(q):
    lin = si.mlp_up_w8a16()
    rows = sample_rows(lin.x.shape[0], 40, 1)
    log("w8a16 2048x1536x6144 + bias + GELU")
    out, ref = run_wxa16(q, 8, lin.x, lin.w, {"bias": lin.bias, "gelu": True}, rows)
    assert_close(out, ref, "w8a16 2048x1536x6144")


@pytest.mark.parametrize("M", si.W4A16_M_SWEEP)
def test_w4a16_sweep_full_size(q, M):
    x = si.w4a16_sweep_x()[:M]
    w = si.w4a16_w()
    rows = None if M <= 256 else sample_rows(M, 40, 2)
    log(f"w4a16 {M}x1536x6144")
    out, ref = run_wxa16(q, 4, x, w, {}, rows)
    assert_close(out, ref, f"w4a16 {M}x1536x6144")


def test_w8a8_mlp_up_full_size(q):
    blk = si.dit_block()
    rows = sample_rows(2048, 40, 3)
    log("w8a8 2048x1536x6144 + GELU")
    out, ref = run_w8a8(q, blk["h"], blk["up"], {"gelu": True}, rows)
    assert_close(out, ref, "w8a8 2048x1536x6144")


TILES = ["256x192x4x3", "256x256x4x4", "256x192x4x2", "256x128x4x2", "128x256x2x4", "128x192x2x2", "128x128x2x2",
         "64x192x2x2", "128x64x2x2", "64x128x2x2", "64x64x2x2", "64x96x2x3", "128x96x2x3", "128x128x2x4",
         # two K groups per workgroup (the fifth number)
         "64x192x2x2x2", "128x128x2x2x2", "128x64x2x2x2", "64x128x2x2x2", "64x96x2x3x2"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("mode", ["w8a8", "w8a16", "w4a16"])
@pytest.mark.parametrize("N,K", [(460, 352), (520, 352), (520, 416), (460, 32)])
def test_every_tile_variant(q, tile, mode, N, K, monkeypatch):
    """Every macro-tile variant of the tiled kernel (forced through the tuning
    override) on ragged shapes that span several tiles and a K tail; N = 460
    takes the element-wise epilogue (N % 8 != 0), N = 520 the vector one with
    a partial last tile.  K = 352 and 416 give an odd and an even number of
    K-steps in each mode (128 int8 k or 64 fp16 k per step: the 4-wave tiles
    alternate two register sets, so both parities and the one-step case,
    K = 32, are covered)."""
    monkeypatch.setenv("ARIA_QLINEAR_TILE", tile)
    M = 300
    log(f"{mode} tile {tile} {M}x{K}x{N}")
    x, w = _rand(M, K, N, 4242)
    e = _epi_inputs(M, N, 9, bias=True, gelu=True, residual=True, steer=True)
    if mode == "w8a8":
        out, ref = run_w8a8(q, x, w, e)
    else:
        out, ref = run_wxa16(q, 8 if mode == "w8a16" else 4, x, w, e)
    assert_close(out, ref, f"{mode} {tile}")
