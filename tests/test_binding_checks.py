"""The Python binding checks every operand's dtype, shape and device against
the call's M, K, N before anything reaches the C-ABI (which receives raw
pointers and cannot size-check them).  Runs on the CPU: the library object is
replaced by a stub that fails the test if any entry point other than the
host-only workspace-size query is called, so every case below must be
refused by the wrapper itself."""
import pytest
import torch

import quantized_diffusion_transformer_qlinear_amd as q
from quantized_diffusion_transformer_qlinear_amd import binding


class _NoCalls:
    """Stands in for the loaded library: only host-only queries pass through."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in ("aria_qlinear_workspace_bytes", "aria_status_string", "aria_qpack_bytes"):
            return getattr(self._real, name)

        def called(*a, **k):
            raise AssertionError(f"{name} reached the library")
        return called


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    monkeypatch.setattr(binding, "lib", _NoCalls(binding.lib))


f16, i8, u8, i32, f32 = torch.float16, torch.int8, torch.uint8, torch.int32, torch.float32
M, K, N = 64, 256, 192


def t(*shape, dtype=f16):
    return torch.zeros(shape, dtype=dtype)


@pytest.mark.parametrize("kw", [
    dict(wq=t(N, K + 32, dtype=i8)),                 # wq K differs from x
    dict(sw=t(N + 1)),
    dict(y=t(M, N + 8)),
    dict(bias=t(N - 1)),
    dict(residual=t(M + 1, N)),
    dict(steer_dir=t(N, dtype=f32), steer_alpha=t(2, dtype=f32)),
    dict(steer_dir=t(N + 4, dtype=f32), steer_alpha=t(1, dtype=f32)),
    dict(acc_out=t(M, N - 8, dtype=i32)),
])
def test_w8a8_shapes(kw):
    args = dict(x=t(M, K), wq=t(N, K, dtype=i8), sw=t(N))
    args.update(kw)
    with pytest.raises(ValueError):
        q.qlinear_w8a8(**args)
    with pytest.raises(ValueError):
        q.qlinear_w8a8_noalloc(**args)


@pytest.mark.parametrize("kw,err", [
    (dict(x=t(M, K, dtype=f32)), TypeError),
    (dict(wq=t(N, K, dtype=u8)), TypeError),
    (dict(sw=t(N, dtype=f32)), TypeError),
    (dict(acc_out=t(M, N, dtype=f32)), TypeError),
    (dict(bias=t(N, dtype=f32)), TypeError),
    (dict(x=t(M * K)), ValueError),                  # not 2-D
])
def test_w8a8_dtypes(kw, err):
    args = dict(x=t(M, K), wq=t(N, K, dtype=i8), sw=t(N))
    args.update(kw)
    with pytest.raises(err):
        q.qlinear_w8a8(**args)


def test_valid_cpu_tensors_are_refused_as_not_on_the_gpu():
    with pytest.raises(ValueError, match="GPU"):
        q.qlinear_w8a8(t(M, K), t(N, K, dtype=i8), t(N))


def test_weight_only_shapes():
    with pytest.raises(ValueError):
        q.qlinear_w8a16(t(M, K), t(N, K // 2, dtype=i8), t(N))
    with pytest.raises(ValueError):
        q.qlinear_w4a16(t(M, K), t(N, K, dtype=u8), t(N, K // 32))          # nibbles are K/2 bytes
    with pytest.raises(ValueError):
        q.qlinear_w4a16(t(M, K), t(N, K // 2, dtype=u8), t(N, K // 16))     # group scales K/32
    with pytest.raises(ValueError):
        q.qlinear_w4a16(t(M, K), t(N, K // 2, dtype=u8), t(N, K // 32), group=64)
    with pytest.raises(ValueError):
        q.qlinear_w16a16(t(M, K), t(N, K - 32), bias=t(N))
    with pytest.raises(ValueError):
        q.qlinear_w8a16(t(M, K), t(N, K, dtype=i8), t(N), residual=t(N, M))
    with pytest.raises(TypeError):
        q.qlinear_w16a16(t(M, K), t(N, K, dtype=i8))


def test_grouped_shapes():
    ok = dict(x=t(16, K), wq=t(N, K // 2, dtype=u8), s=t(N, K // 32))
    with pytest.raises(ValueError):
        q.qlinear_grouped(4, [ok, dict(ok, s=t(N, K // 64))])
    with pytest.raises(ValueError):
        q.qlinear_grouped(4, [dict(ok, y=t(16, N - 1))])
    with pytest.raises(ValueError):
        q.qlinear_grouped(8, [dict(x=t(16, K), wq=t(N, K + 32, dtype=i8), s=t(N))])
    with pytest.raises(ValueError):
        q.qlinear_grouped(2, [ok])


def test_quantizer_and_pack_shapes():
    with pytest.raises(ValueError):
        q.quant_act(t(M, K), xq=t(M, K - 32, dtype=i8))
    with pytest.raises(ValueError):
        q.quant_act(t(M, K), sa=t(M - 1))
    with pytest.raises(ValueError):
        q.quant_act_columns(t(M, 3 * K), 2 * K + 32, K)                     # past the last column
    with pytest.raises(ValueError):
        q.quant_act_columns(t(M, 3 * K), 2 * K, K, xq=t(M, 2 * K, dtype=i8))
    with pytest.raises(ValueError):
        q.qpack(8, t(K, N), q=t(K, N, dtype=i8))                          # [N][K], not [K][N]
    with pytest.raises(ValueError):
        q.qpack(4, t(K, N), s=t(N, K // 16))
    with pytest.raises(ValueError):
        q.qpack(3, t(K, N))


def test_block_step_shapes():
    with pytest.raises(ValueError):
        q.layernorm(t(M, K), t(K - 8), t(K))
    with pytest.raises(ValueError):
        q.layernorm(t(M, K), t(K), t(K), y=t(M, K + 8))
    with pytest.raises(ValueError):
        q.layernorm_quant(t(M, K), t(K), t(K), xq=t(M, K - 32, dtype=i8))
    with pytest.raises(ValueError):
        q.layernorm_quant(t(M, K), t(K), t(K), sa=t(2 * M))
    with pytest.raises(ValueError):
        q.qlinear_w8a8_prequant(t(M, K, dtype=i8), t(M + 1), t(N, K, dtype=i8), t(N))
    with pytest.raises(ValueError):
        q.qlinear_w8a8_prequant(t(M, K, dtype=i8), t(M), t(N, K, dtype=i8), t(N), residual=t(M, K))
    with pytest.raises(ValueError):
        q.attention(t(M, 3 * 128 + 1), 2, 32)
    with pytest.raises(ValueError):
        q.attention(t(M, 3 * 128), 2, 32, out=t(M, 3 * 128))
