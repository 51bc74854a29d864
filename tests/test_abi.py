"""The C-ABI library loads, exports every function include/aria_qlinear.h
declares, and rejects bad arguments on the host before any launch (no GPU
needed: every call here fails validation, so nothing reaches the device)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "aria_qlinear.h")
LIB = os.environ.get("ARIA_QLINEAR_LIB",
                     os.path.join(ROOT, "quantized_diffusion_transformer_qlinear_amd", "libaria_qlinear.so"))

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="HIP library not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(aria_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def q():
    import quantized_diffusion_transformer_qlinear_amd as m
    return m


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 19, names
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (aria_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert getattr(lib, n) is not None


def test_status_strings(q):
    for code in range(-8, 1):
        assert q.status_string(code) and q.status_string(code) != "unknown status"
    assert q.status_string(-99) == "unknown status"
    assert q.lib.aria_abi_version() == 1


def test_qpack_bytes(q):
    assert q.qpack_bytes(8, 0, 1536, 6144) == (1536 * 6144, 2 * 6144)
    assert q.qpack_bytes(4, 32, 1536, 6144) == (1536 * 6144 // 2, 2 * 6144 * 48)
    assert q.qpack_bytes(16, 0, 1536, 6144) == (2 * 1536 * 6144, 0)
    for bits, group in ((8, 32), (4, 0), (4, 64), (2, 32), (16, 32)):
        with pytest.raises(q.AriaError) as e:
            q.qpack_bytes(bits, group, 64, 64)
        assert e.value.code == -4
    with pytest.raises(q.AriaError) as e:
        q.qpack_bytes(8, 0, 48, 64)       # K % 32 != 0
    assert e.value.code == -2


def _w8a8(q, x=16, M=64, K=256, N=256, wq=32, sw=48, epi=None, y=4096, ws=1 << 20, ws_bytes=1 << 30):
    e = ctypes.byref(epi) if epi is not None else None
    return q.lib.aria_qlinear_w8a8(x, M, K, N, wq, sw, e, y, ws, ws_bytes, None)


def test_validation_codes(q):
    L = q.lib
    X, W, S, Y, WS = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20  # never dereferenced
    big = 1 << 40
    # null pointers
    assert _w8a8(q, x=None) == -1
    assert _w8a8(q, wq=None) == -1
    assert _w8a8(q, y=None) == -1
    # shapes
    for M, K, N in ((0, 256, 256), (64, 0, 256), (64, 256, 0), (64, 48, 256), (64, 32768, 256),
                    (64, 32, 1 << 26), ((1 << 30) + 1, 256, 256)):
        assert _w8a8(q, X, M, K, N, W, S, None, Y, WS, big) == -2, (M, K, N)
    # alignment
    assert _w8a8(q, X + 2, 64, 256, 256, W, S, None, Y, WS, big) == -3
    assert _w8a8(q, X, 64, 256, 256, W, S + 8, None, Y, WS, big) == -3
    # workspace
    need = q.workspace_bytes(q.ARIA_W8A8, 64, 256, 256)
    assert need >= 64 * 256 + 128
    assert _w8a8(q, X, 64, 256, 256, W, S, None, Y, WS, need - 1) == -5
    assert _w8a8(q, X, 64, 256, 256, W, S, None, Y, None, big) == -5
    # x overlapping y
    assert _w8a8(q, X, 64, 256, 256, W, S, None, X + 1024, WS, big) == -7
    # epilogue options
    E = q.binding.Epilogue
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 2, 0, None, None, None, None), Y, WS, big) == -4
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 1, None, None, None, None), Y, WS, big) == -4
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 0, None, 7 << 20, None, None), Y, WS, big) == -1
    assert _w8a8(q, X, 64, 256, 256, W, S, E(S + 2, 0, 0, None, None, None, None), Y, WS, big) == -3
    # residual partly overlapping y is rejected, exact aliasing is allowed past validation
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 0, Y + 512, None, None, None), Y, WS, big) == -7
    # the workspace is written while x, the weights and the epilogue operands
    # are read and y is written: it may overlap none of them
    assert _w8a8(q, X, 64, 256, 256, W, S, None, Y, X + 4096, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, None, Y, Y + 4096, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, None, Y, W + 4096, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, None, Y, S - 256, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, E(WS + 1024, 0, 0, None, None, None, None), Y, WS, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 0, WS + 1024, None, None, None), Y, WS, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 0, None, 7 << 20, WS + 64, None), Y, WS, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 0, None, None, None, WS + 4096), Y, WS, big) == -7
    # the raw accumulators may overlap neither y nor another epilogue operand
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 0, None, None, None, Y + 256), Y, WS, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, E(None, 0, 0, 9 << 20, None, None, (9 << 20) + 1024), Y, WS, big) == -7
    assert _w8a8(q, X, 64, 256, 256, W, S, E(9 << 20, 0, 0, None, None, None, (9 << 20) - 256), Y, WS, big) == -7
    assert L.aria_qlinear_w8a8_prequant(1 << 24, 2 << 24, 64, 256, 256, W, S,
                                        ctypes.byref(E(None, 0, 0, None, None, None, Y + 1024)), Y, None) == -7
    # the allocation-free W8A8 call: the W8A8 checks, then the scratch limit,
    # all before any device call
    N0 = L.aria_qlinear_w8a8_noalloc
    assert N0(None, 64, 256, 256, W, S, None, Y, None) == -1
    assert N0(X, 64, 48, 256, W, S, None, Y, None) == -2
    assert N0(X + 2, 64, 256, 256, W, S, None, Y, None) == -3
    assert N0(X, 64, 256, 256, W, S, None, X + 1024, None) == -7
    assert N0(X, 64, 256, 256, W, S, E(None, 2, 0, None, None, None, None), Y, None) == -4
    assert N0(X, 64, 256, 256, W, S, E(None, 0, 0, None, None, None, Y + 256), Y, None) == -7
    far = 1 << 36
    assert N0(X, 2048, 12288, 256, W, S, None, far, None) == -8     # 24 MiB of int8 + the scales
    assert N0(X, 4096, 8192, 256, W, S, None, far, None) == -8
    assert N0(X, 1 << 20, 64, 64, W, S, None, far, None) == -8
    # acc_out only for W8A8; group must be 32 for W4A16
    ep = E(None, 0, 0, None, None, None, 6 << 20)
    assert L.aria_qlinear_w8a16(X, 64, 256, 256, W, S, ctypes.byref(ep), Y, None, 0, None) == -4
    assert L.aria_qlinear_w4a16(X, 64, 256, 256, W, S, 64, None, Y, None, 0, None) == -4
    assert L.aria_qlinear_w4a16(None, 64, 256, 256, W, S, 32, None, Y, None, 0, None) == -1
    # packing and activation quantization
    assert L.aria_qpack(8, 0, None, 64, 64, W, S, None) == -1
    assert L.aria_qpack(8, 0, X, 64, 64, W + 1, S, None) == -3
    assert L.aria_qpack(3, 0, X, 64, 64, W, S, None) == -4
    assert L.aria_qpack(8, 0, X, 64, 64, X + 64, S, None) == -7
    assert L.aria_quant_act(X, 64, 33, W, S, None) == -2
    assert L.aria_quant_act(X, 64, 64, None, S, None) == -1
    assert L.aria_quant_act_strided(X, 32, 64, 64, W, S, None) == -2        # ldx < K
    assert L.aria_quant_act_strided(X, 100, 64, 64, W, S, None) == -2       # ldx % 8
    assert L.aria_quant_act_strided(X, 192, 64, 64, None, S, None) == -1
    assert L.aria_quant_act_strided(X + 2, 192, 64, 64, W, S, None) == -3
    assert L.aria_quant_act_strided(X, 192, 64, 64, X + 1024, S, None) == -7     # xq inside the rows read
    assert L.aria_quant_act_strided(X, 192, 64, 64, W, W + 1024, None) == -7     # s_a inside xq
    # the fp16 rung
    assert L.aria_qlinear_w16a16(X, 64, 256, 256, None, None, Y, None, 0, None) == -1
    assert L.aria_qlinear_w16a16(X, 64, 48, 256, W, None, Y, None, 0, None) == -2
    assert L.aria_qlinear_w16a16(X, 64, 16384, 65536, W, None, Y, None, 0, None) == -2   # 2 K N >= 2^31
    assert L.aria_qlinear_w16a16(X + 4, 64, 256, 256, W, None, Y, None, 0, None) == -3
    assert L.aria_qlinear_w16a16(X, 64, 256, 256, W, ctypes.byref(ep), Y, None, 0, None) == -4   # acc_out
    assert L.aria_qpack(16, 32, X, 64, 64, W, None, None) == -4
    assert L.aria_qpack(16, 0, None, 64, 64, W, None, None) == -1
    # block steps around the linears
    assert L.aria_layernorm(X, 64, 100, W, S, 1e-5, Y, None) == -2          # W % 8
    assert L.aria_layernorm(X, 64, 32768, W, S, 1e-5, Y, None) == -2
    assert L.aria_layernorm(X, 64, 256, W, S, -1.0, Y, None) == -4
    assert L.aria_layernorm(X, 64, 256, None, S, 1e-5, Y, None) == -1
    assert L.aria_layernorm(X, 64, 256, W, S + 2, 1e-5, Y, None) == -3
    assert L.aria_layernorm(X, 64, 256, W, S, 1e-5, X + 512, None) == -7     # partial overlap
    # fused pre-norm + quantization (W8A8 shape rules on W), and the linear on
    # activations quantized beforehand
    Q, SA = 6 << 20, 7 << 20
    assert L.aria_layernorm_quant(X, 64, 80, W, S, 1e-5, None, Q, SA, None) == -2      # W % 32
    assert L.aria_layernorm_quant(X, 64, 256, W, S, 2.0, None, Q, SA, None) == -4
    assert L.aria_layernorm_quant(X, 64, 256, W, S, 1e-5, None, None, SA, None) == -1
    assert L.aria_layernorm_quant(X, 64, 256, W, S, 1e-5, Y + 2, Q, SA, None) == -3
    assert L.aria_layernorm_quant(X, 64, 256, W, S, 1e-5, None, X + 256, SA, None) == -7
    assert L.aria_layernorm_quant(X, 64, 256, W, S, 1e-5, None, Q, Q + 64, None) == -7
    assert L.aria_layernorm_quant(X, 64, 256, W, S, 1e-5, X + 512, Q, SA, None) == -7
    assert L.aria_layernorm_quant(X, 64, 256, W, S, 1e-5, Y, Q, Y + 256, None) == -7
    assert L.aria_qlinear_w8a8_prequant(Q, SA, 64, 48, 256, W, S, None, Y, None) == -2
    assert L.aria_qlinear_w8a8_prequant(Q, None, 64, 256, 256, W, S, None, Y, None) == -1
    assert L.aria_qlinear_w8a8_prequant(Q, SA + 2, 64, 256, 256, W, S, None, Y, None) == -3
    assert L.aria_qlinear_w8a8_prequant(Q, SA, 64, 256, 256, W, S, None, Q + 64, None) == -7
    ep2 = E(None, 3, 0, None, None, None, None)
    assert L.aria_qlinear_w8a8_prequant(Q, SA, 64, 256, 256, W, S, ctypes.byref(ep2), Y, None) == -4
    assert L.aria_attention(X, 64, 96, 2, 32, Y, None) == -4                 # head dim 48
    assert L.aria_attention(X, 64, 128, 2, 48, Y, None) == -2                # M % seq
    assert L.aria_attention(None, 64, 128, 2, 32, Y, None) == -1
    assert L.aria_attention(X, 64, 128, 2, 32, X + 1024, None) == -7
    assert L.aria_attention(X, 64, 128, 2, 32, Y + 8, None) == -3
    assert L.aria_qlinear_workspace_bytes(9, 64, 64, 64) == 0
    assert L.aria_qlinear_workspace_bytes(0, 64, 40, 64) == 0


def test_fused_quant_validation_codes(q):
    """The producer (W8A8 + row maxima of a column block) and the consumer
    (W8A8 quantizing its fp16 input with those maxima): every rejection on the
    host, before any launch."""
    L = q.lib
    X, W, S, Y, WS, R = 1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20, 6 << 20
    big = 1 << 40
    P = L.aria_qlinear_w8a8_rowmax
    # the W8A8 checks first
    assert P(None, 64, 256, 768, W, S, None, Y, WS, big, R, 512, 256, None) == -1
    assert P(X, 64, 48, 768, W, S, None, Y, WS, big, R, 512, 256, None) == -2
    # the column block: 64-column blocks inside [0, N), N % 8 == 0
    for c0, nc in ((512, 0), (512, 32), (500, 256), (512, 200), (640, 256), (-64, 128)):
        assert P(X, 64, 256, 768, W, S, None, Y, WS, big, R, c0, nc, None) == -2, (c0, nc)
    assert P(X, 64, 256, 772, W, S, None, Y, WS, big, R, 512, 256, None) == -2         # N % 8
    assert P(X, 64, 256, 768, W, S, None, Y, WS, big, None, 512, 256, None) == -1
    assert P(X, 64, 256, 768, W, S, None, Y, WS, big, R + 4, 512, 256, None) == -3
    assert P(X, 64, 256, 768, W, S, None, Y, WS, 100, R, 512, 256, None) == -5
    # rowmax may overlap nothing else
    for r in (X + 64, Y + 1024, WS + 256, W + 64, S - 128):
        assert P(X, 64, 256, 768, W, S, None, Y, WS, big, r, 512, 256, None) == -7, hex(r)
    E = q.binding.Epilogue
    assert P(X, 64, 256, 768, W, S, E(None, 0, 0, R + 64, None, None, None), Y, WS, big, R, 512, 256, None) == -7
    F = L.aria_qlinear_w8a8_fused
    # (x, ldx, rowmax, M, K, N, wq, sw, epi, y, s_a_out, stream)
    assert F(None, 768, R, 64, 256, 256, W, S, None, Y, None, None) == -1
    assert F(X, 768, None, 64, 256, 256, W, S, None, Y, None, None) == -1
    assert F(X, 768, R, 64, 224, 256, W, S, None, Y, None, None) == -2       # K % 64
    assert F(X, 192, R, 64, 256, 256, W, S, None, Y, None, None) == -2       # ldx < K
    assert F(X, 772, R, 64, 256, 256, W, S, None, Y, None, None) == -2       # ldx % 8
    assert F(X + 2, 768, R, 64, 256, 256, W, S, None, Y, None, None) == -3
    assert F(X, 768, R, 64, 256, 256, W, S, None, Y, 7 << 20 | 2, None) == -3
    assert F(X, 768, R, 64, 256, 256, W, S, None, X + 4096, None, None) == -7        # y inside the rows read
    assert F(X, 768, R, 64, 256, 256, W, S, None, R + 64, None, None) == -7          # y over rowmax
    for sa in (Y + 64, X + 1024, R + 16, W + 64, S - 64):
        assert F(X, 768, R, 64, 256, 256, W, S, None, Y, sa, None) == -7, hex(sa)
    assert F(X, 768, R, 64, 256, 256, W, S, E(None, 2, 0, None, None, None, None), Y, None, None) == -4


def test_grouped_validation_codes(q):
    L = q.lib
    P = q.binding.LinearProblem
    E = q.binding.Epilogue
    X, W, S, Y = 1 << 20, 2 << 20, 3 << 20, 4 << 20  # never dereferenced

    def call(bits, group, probs):
        arr = (P * max(len(probs), 1))(*probs)
        return L.aria_qlinear_grouped(bits, group, arr, len(probs), None)

    ok = P(X, 16, 256, 128, W, S, None, Y)   # valid on its own; every call below fails validation
    assert call(4, 16, [ok]) == -4 and call(8, 32, [ok]) == -4 and call(3, 0, [ok]) == -4
    assert L.aria_qlinear_grouped(4, 32, None, 1, None) == -1
    assert call(4, 32, []) == -2
    assert call(4, 32, [P(X, 65, 256, 128, W, S, None, Y)]) == -4           # M > 64: not the small-M path
    assert call(4, 32, [P(X, 16, 48, 128, W, S, None, Y)]) == -2            # K % 32
    assert call(4, 32, [P(None, 16, 256, 128, W, S, None, Y)]) == -1
    assert call(4, 32, [P(X + 2, 16, 256, 128, W, S, None, Y)]) == -3
    assert call(4, 32, [P(X, 16, 256, 128, W, S, None, X + 64)]) == -7      # own x / y overlap
    ep = E(None, 0, 0, None, None, None, 6 << 20)
    assert call(4, 32, [P(X, 16, 256, 128, W, S, ctypes.pointer(ep), Y)]) == -4   # acc_out
    # across problems: y of one may not overlap x, weights, scales or y of another
    Y2 = 8 << 20
    assert call(4, 32, [P(X, 16, 256, 128, W, S, None, Y), P(Y, 16, 256, 128, W, S, None, Y2)]) == -7
    assert call(4, 32, [P(X, 16, 256, 128, W, S, None, Y), P(X, 16, 256, 128, Y + 64, S, None, Y2)]) == -7
    assert call(4, 32, [P(X, 16, 256, 128, W, S, None, Y), P(X, 16, 256, 128, W, S, None, Y + 2048)]) == -7
    assert call(8, 0, [P(X, 16, 256, 128, W, S, None, Y)] * 1025) == -2
