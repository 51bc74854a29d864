"""Guard bands: every output is written into the middle of a larger buffer
pre-filled with a pattern, and after the call the bands on both sides must be
untouched and the output identical, bit for bit, to the same call on a plain
buffer.  Ragged shapes (partial last tiles, N % 8 != 0, K tails) exercise the
kernels' edge handling, where a stray store would land just past the end of a
row or of the tensor."""
import numpy as np
import pytest

import synthetic_inputs as si
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu

BAND = 4096          # elements of guard on each side
PAT16 = 0x7E5A       # fp16 / int16 fill pattern (a NaN payload as fp16)


@pytest.fixture(scope="module")
def q():
    import quantized_diffusion_transformer_qlinear_amd as m
    return m


def guarded(torch, shape, dtype):
    """(view of `shape` inside a pattern-filled buffer, the whole buffer)."""
    n = int(np.prod(shape))
    itemsize = torch.empty(0, dtype=dtype).element_size()
    raw = torch.empty((2 * BAND + n) * itemsize, dtype=torch.uint8, device="cuda:0")
    pat = np.frombuffer(np.array([PAT16], np.uint16).tobytes() * ((raw.numel() + 1) // 2), np.uint8)[:raw.numel()]
    raw.copy_(torch.from_numpy(pat.copy()))
    view = raw[BAND * itemsize:(BAND + n) * itemsize].view(dtype).view(shape)
    return view, raw


def bands_intact(raw, n, itemsize):
    b = host(raw)
    pat = np.frombuffer(np.array([PAT16], np.uint16).tobytes() * ((b.size + 1) // 2), np.uint8)[:b.size]
    lo, hi = BAND * itemsize, (BAND + n) * itemsize
    return np.array_equal(b[:lo], pat[:lo]) and np.array_equal(b[hi:], pat[hi:])


def _inputs(M, K, N, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    return x, w


@pytest.mark.parametrize("mode", ["w8a8", "w8a16", "w4a16", "w16a16"])
@pytest.mark.parametrize("M,K,N", [(300, 352, 460), (300, 416, 520), (37, 352, 460), (5, 96, 520), (12, 256, 4104)])
def test_output_guard_bands(q, mode, M, K, N):
    import torch
    log(f"guard {mode} {M}x{K}x{N}")
    x, w = _inputs(M, K, N, 77 + M + N)
    xd = dev(x)
    rng = np.random.default_rng(5)
    bias = dev((rng.standard_normal(N) * 0.1).astype(np.float16))
    res = dev(rng.standard_normal((M, N)).astype(np.float16))
    d = dev(si.unit_direction(N, 8))
    alpha = torch.tensor([0.3], dtype=torch.float32, device="cuda:0")
    epi = dict(bias=bias, gelu=True, residual=res, steer_dir=d, steer_alpha=alpha)
    if mode in ("w8a8", "w8a16"):
        packed = q.qpack(8, dev(w))
    elif mode == "w4a16":
        packed = q.qpack(4, dev(w))
    else:
        packed = (q.qpack(16, dev(w))[0],)
    fn = {"w8a8": q.qlinear_w8a8, "w8a16": q.qlinear_w8a16, "w4a16": q.qlinear_w4a16,
          "w16a16": q.qlinear_w16a16}[mode]
    y_plain = fn(xd, *packed, **epi)
    y, raw = guarded(torch, (M, N), torch.float16)
    extra = {}
    if mode == "w8a8":
        acc, acc_raw = guarded(torch, (M, N), torch.int32)
        acc_plain = torch.empty((M, N), dtype=torch.int32, device="cuda:0")
        fn(xd, *packed, y=y_plain, acc_out=acc_plain, **epi)
        extra = dict(acc_out=acc)
    fn(xd, *packed, y=y, **epi, **extra)
    assert bands_intact(raw, M * N, 2), f"{mode}: a store landed outside y"
    assert np.array_equal(host(y).view(np.uint16), host(y_plain).view(np.uint16))
    if mode == "w8a8":
        assert bands_intact(acc_raw, M * N, 4), "a store landed outside acc_out"
        assert np.array_equal(host(acc), host(acc_plain))


@pytest.mark.parametrize("M,K", [(300, 352), (7, 96), (64, 6144)])
def test_quantizer_guard_bands(q, M, K):
    import torch
    x = dev(np.random.default_rng(M + K).standard_normal((M, K)).astype(np.float16))
    xq0, sa0 = q.quant_act(x)
    xq, xq_raw = guarded(torch, (M, K), torch.int8)
    sa, sa_raw = guarded(torch, (M,), torch.float16)
    q.quant_act(x, xq=xq, sa=sa)
    assert bands_intact(xq_raw, M * K, 1) and bands_intact(sa_raw, M, 2)
    assert np.array_equal(host(xq), host(xq0)) and np.array_equal(host(sa).view(np.uint16), host(sa0).view(np.uint16))
    # the column block of a wider tensor, read in place
    wide = dev(np.random.default_rng(K).standard_normal((M, 3 * K)).astype(np.float16))
    xq1, sa1 = q.quant_act_columns(wide, 2 * K, K)
    q.quant_act_columns(wide, 2 * K, K, xq=xq, sa=sa)
    assert bands_intact(xq_raw, M * K, 1) and bands_intact(sa_raw, M, 2)
    assert np.array_equal(host(xq), host(xq1))


def test_grouped_and_pack_guard_bands(q):
    import torch
    probs, outs, raws = [], [], []
    for i, (M, K, N) in enumerate([(16, 1536, 460), (5, 256, 520), (1, 352, 72)]):
        x, w = _inputs(M, K, N, 300 + i)
        wq, s = q.qpack(4, dev(w))
        y, raw = guarded(torch, (M, N), torch.float16)
        probs.append({"x": dev(x), "wq": wq, "s": s, "y": y})
        outs.append(q.qlinear_w4a16(dev(x), wq, s))
        raws.append((raw, M * N))
    q.qlinear_grouped(4, probs)
    for p, ref, (raw, n) in zip(probs, outs, raws):
        assert bands_intact(raw, n, 2)
        assert np.array_equal(host(p["y"]).view(np.uint16), host(ref).view(np.uint16))
    # packing: the packed weights and scales of ragged layers (N % 8 != 0 and
    # N % 8 == 0 take different kernels)
    for K, N in ((352, 460), (352, 456)):
        w = dev(_inputs(1, K, N, 9)[1])
        for bits, qshape, qtype, sshape in ((8, (N, K), torch.int8, (N,)), (4, (N, K // 2), torch.uint8, (N, K // 32))):
            qb, qraw = guarded(torch, qshape, qtype)
            sb, sraw = guarded(torch, sshape, torch.float16)
            q0, s0 = q.qpack(bits, w)
            q.qpack(bits, w, q=qb, s=sb)
            assert bands_intact(qraw, int(np.prod(qshape)), 1) and bands_intact(sraw, int(np.prod(sshape)), 2)
            assert np.array_equal(host(qb), host(q0)) and np.array_equal(host(sb).view(np.uint16), host(s0).view(np.uint16))
