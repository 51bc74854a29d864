"""The allocation-free W8A8 entry point, aria_qlinear_w8a8_noalloc, through
the C-ABI against aria_qlinear_w8a8 with a caller workspace: the same int32
accumulators and fp16 output bit for bit, on calls in a row whose inputs
shrink (each later call runs on the scratch the previous one left behind),
plus the accumulators against the oracle.  No torch allocation happens in the
call (every buffer is allocated beforehand)."""
import ctypes

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


# largest first, then smaller ones: MLP-down at DiT width, a ragged shape, a tiny one
SHAPES = [(2048, 6144, 1536, dict(residual=True, steer=True)),
          (300, 1536, 832, dict(bias=True, gelu=True)),
          (70, 256, 200, dict(residual=True, steer=True))]


def _inputs(M, K, N, seed, bias=False, gelu=False, residual=False, steer=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float16)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float16)
    e = {}
    if bias:
        e["bias"] = (rng.standard_normal(N) * 0.1).astype(np.float16)
    if gelu:
        e["gelu"] = True
    if residual:
        e["residual"] = rng.standard_normal((M, N)).astype(np.float16)
    if steer:
        e["d"] = si.unit_direction(N, seed + 5)
        e["alpha"] = 0.3
    return x, w, e


def test_noalloc_matches_workspace_call(q):
    import torch
    L = q.lib
    for i, (M, K, N, opts) in enumerate(SHAPES):
        log(f"noalloc call {i}: M={M} K={K} N={N} {sorted(opts)}")
        x, w, e = _inputs(M, K, N, 900 + i, **opts)
        xd = dev(x)
        wq, sw = q.qpack(8, dev(w))
        alpha = torch.tensor([e.get("alpha", 0.0)], dtype=torch.float32, device="cuda:0")
        bd = dev(e["bias"]) if "bias" in e else None
        rd = dev(e["residual"]) if "residual" in e else None
        dd = dev(e["d"]) if "d" in e else None
        ys = [torch.empty((M, N), dtype=torch.float16, device="cuda:0") for _ in range(2)]
        accs = [torch.empty((M, N), dtype=torch.int32, device="cuda:0") for _ in range(2)]
        ws = torch.empty(q.workspace_bytes(q.ARIA_W8A8, M, K, N), dtype=torch.uint8, device="cuda:0")
        stream = torch.cuda.current_stream().cuda_stream
        epis = [q.binding.Epilogue(None if bd is None else bd.data_ptr(), int(e.get("gelu", False)), 0,
                                   None if rd is None else rd.data_ptr(), None if dd is None else dd.data_ptr(),
                                   None if dd is None else alpha.data_ptr(), accs[j].data_ptr()) for j in range(2)]
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        rc = L.aria_qlinear_w8a8_noalloc(xd.data_ptr(), M, K, N, wq.data_ptr(), sw.data_ptr(),
                                         ctypes.byref(epis[0]), ys[0].data_ptr(), stream)
        assert rc == 0, q.status_string(rc)
        assert torch.cuda.memory_allocated() == before
        rc = L.aria_qlinear_w8a8(xd.data_ptr(), M, K, N, wq.data_ptr(), sw.data_ptr(), ctypes.byref(epis[1]),
                                 ys[1].data_ptr(), ws.data_ptr(), ws.numel(), stream)
        assert rc == 0, q.status_string(rc)
        acc_n, acc_w = host(accs[0]), host(accs[1])
        y_n, y_w = host(ys[0]), host(ys[1])
        assert np.array_equal(acc_n, acc_w), "accumulators differ from the workspace call"
        assert np.array_equal(y_n.view(np.uint16), y_w.view(np.uint16)), "output differs from the workspace call"
        if M * N <= 300 * 832:
            ref = oracle.qlinear_w8a8(x, *oracle.qpack8(w), bias=e.get("bias"), gelu=e.get("gelu", False),
                                      residual=e.get("residual"), d=e.get("d"), alpha=e.get("alpha", 0.0))
            assert np.array_equal(acc_n, ref["acc"]), "accumulators differ from the oracle"
            assert_close(y_n, ref["y"], f"noalloc {M}x{K}x{N}")


def test_noalloc_rejects_shapes_past_the_scratch(q):
    """A shape whose quantized activations exceed the scratch is refused on
    the host, before anything is launched."""
    L = q.lib
    X, W, S, Y = 1 << 20, 2 << 20, 3 << 20, 1 << 36      # never dereferenced
    assert L.aria_qlinear_w8a8_noalloc(X, 2048, 12288, 256, W, S, None, Y, None) == -8
    assert L.aria_qlinear_w8a8_noalloc(X, 4096, 8192, 256, W, S, None, Y, None) == -8
