"""ctypes binding of the C-ABI in include/aria_qlinear.h (same names, minus
the ``aria_`` prefix).  Arguments are torch tensors on the GPU (or raw device
addresses as ints); nothing here computes any part of the layer."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libaria_qlinear.so")

if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is not built; run __graft_entry__.build() "
                      "(or python quantized_diffusion_transformer_qlinear_amd/build.py)")

lib = ctypes.CDLL(library_path)

ARIA_W8A8, ARIA_W8A16, ARIA_W4A16, ARIA_W16A16 = 0, 1, 2, 3
_P, _I64, _SZ, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int


class Epilogue(ctypes.Structure):
    _fields_ = [("bias", _P), ("gelu", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("residual", _P), ("steer_dir", _P), ("steer_alpha", _P), ("acc_out", _P)]


lib.aria_status_string.argtypes = [_I]
lib.aria_status_string.restype = ctypes.c_char_p
lib.aria_abi_version.argtypes = []
lib.aria_abi_version.restype = _I
lib.aria_qpack_bytes.argtypes = [_I, _I, _I64, _I64, ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)]
lib.aria_qpack_bytes.restype = _I
lib.aria_qpack.argtypes = [_I, _I, _P, _I64, _I64, _P, _P, _P]
lib.aria_qpack.restype = _I
lib.aria_quant_act.argtypes = [_P, _I64, _I64, _P, _P, _P]
lib.aria_quant_act.restype = _I
lib.aria_quant_act_strided.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P]
lib.aria_quant_act_strided.restype = _I
lib.aria_qlinear_workspace_bytes.argtypes = [_I, _I64, _I64, _I64]
lib.aria_qlinear_workspace_bytes.restype = _SZ
for _name in ("aria_qlinear_w8a8", "aria_qlinear_w8a16"):
    getattr(lib, _name).argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.POINTER(Epilogue), _P, _P, _SZ, _P]
    getattr(lib, _name).restype = _I
lib.aria_qlinear_w4a16.argtypes = [_P, _I64, _I64, _I64, _P, _P, _I, ctypes.POINTER(Epilogue), _P, _P, _SZ, _P]
lib.aria_qlinear_w4a16.restype = _I
lib.aria_qlinear_w16a16.argtypes = [_P, _I64, _I64, _I64, _P, ctypes.POINTER(Epilogue), _P, _P, _SZ, _P]
lib.aria_qlinear_w16a16.restype = _I


lib.aria_layernorm.argtypes = [_P, _I64, _I64, _P, _P, ctypes.c_float, _P, _P]
lib.aria_layernorm.restype = _I
lib.aria_layernorm_quant.argtypes = [_P, _I64, _I64, _P, _P, ctypes.c_float, _P, _P, _P, _P]
lib.aria_layernorm_quant.restype = _I
lib.aria_qlinear_w8a8_prequant.argtypes = [_P, _P, _I64, _I64, _I64, _P, _P, ctypes.POINTER(Epilogue), _P, _P]
lib.aria_qlinear_w8a8_prequant.restype = _I
lib.aria_attention.argtypes = [_P, _I64, _I64, _I64, _I64, _P, _P]
lib.aria_attention.restype = _I


class LinearProblem(ctypes.Structure):
    _fields_ = [("x_f16", _P), ("M", _I64), ("K", _I64), ("N", _I64), ("wq", _P), ("s_f16", _P),
                ("epi", ctypes.POINTER(Epilogue)), ("y_f16", _P)]


lib.aria_qlinear_grouped.argtypes = [_I, _I, ctypes.POINTER(LinearProblem), _I, _P]
lib.aria_qlinear_grouped.restype = _I


class AriaError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {status_string(code)} ({code})")
        self.code = code


def status_string(code: int) -> str:
    return lib.aria_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise AriaError(code, what)


def _torch():
    import torch
    return torch


def _addr(t):
    """Device address of a tensor (None -> NULL); ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous GPU tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _dt(t, dtype, name):
    if t is not None and not isinstance(t, int) and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def qpack_bytes(bits: int, group: int, K: int, N: int):
    qb, sb = _SZ(), _SZ()
    _check(lib.aria_qpack_bytes(bits, group, K, N, ctypes.byref(qb), ctypes.byref(sb)), "qpack_bytes")
    return qb.value, sb.value


def qpack(bits: int, w, q=None, s=None, stream=None):
    """Pack fp16 W [K][N]: bits 8 -> (Wq int8 [N][K], s fp16 [N]);
    bits 4 -> (Wq4 uint8 [N][K/2], s fp16 [N][K/32]); bits 16 -> (Wt fp16 [N][K], None)."""
    torch = _torch()
    _dt(w, torch.float16, "w")
    K, N = w.shape
    group = 32 if bits == 4 else 0
    if q is None:
        shape = (N, K // 2) if bits == 4 else (N, K)
        dtype = {8: torch.int8, 4: torch.uint8, 16: torch.float16}[bits]
        q = torch.empty(shape, dtype=dtype, device=w.device)
    if s is None and bits != 16:
        s = torch.empty((N,) if bits == 8 else (N, K // group), dtype=torch.float16, device=w.device)
    _check(lib.aria_qpack(bits, group, _addr(w), K, N, _addr(q), _addr(s), _stream(stream)), "qpack")
    return q, s


def quant_act(x, xq=None, sa=None, stream=None):
    torch = _torch()
    _dt(x, torch.float16, "x")
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device) if xq is None else xq
    sa = torch.empty((M,), dtype=torch.float16, device=x.device) if sa is None else sa
    _check(lib.aria_quant_act(_addr(x), M, K, _addr(xq), _addr(sa), _stream(stream)), "quant_act")
    return xq, sa


def quant_act_columns(src, col0: int, ncols: int, xq=None, sa=None, stream=None):
    """Per-token quantization of the column block src[:, col0:col0+ncols] of a
    contiguous fp16 [M][W] tensor, read in place (row stride W)."""
    torch = _torch()
    _dt(src, torch.float16, "src")
    M, W = src.shape
    if not (0 <= col0 and col0 + ncols <= W):
        raise ValueError("column block outside the tensor")
    xq = torch.empty((M, ncols), dtype=torch.int8, device=src.device) if xq is None else xq
    sa = torch.empty((M,), dtype=torch.float16, device=src.device) if sa is None else sa
    _check(lib.aria_quant_act_strided(_addr(src) + 2 * col0, W, M, ncols, _addr(xq), _addr(sa), _stream(stream)),
           "quant_act_strided")
    return xq, sa


def workspace_bytes(mode: int, M: int, K: int, N: int) -> int:
    return int(lib.aria_qlinear_workspace_bytes(mode, M, K, N))


def _epi(bias, gelu, residual, steer_dir, steer_alpha, acc_out):
    torch = _torch()
    _dt(bias, torch.float16, "bias")
    _dt(residual, torch.float16, "residual")
    _dt(steer_dir, torch.float32, "steer_dir")
    _dt(steer_alpha, torch.float32, "steer_alpha")
    _dt(acc_out, torch.int32, "acc_out")
    return Epilogue(_addr(bias), int(bool(gelu)), 0, _addr(residual), _addr(steer_dir), _addr(steer_alpha),
                    _addr(acc_out))


def _ws(mode, M, K, N, ws, device):
    need = workspace_bytes(mode, M, K, N)
    if ws is None and need:
        ws = _torch().empty(need, dtype=_torch().uint8, device=device)
    nbytes = 0 if ws is None else (ws.numel() * ws.element_size() if not isinstance(ws, int) else need)
    return ws, nbytes


def _out(x, N, y):
    return _torch().empty((x.shape[0], N), dtype=_torch().float16, device=x.device) if y is None else y


def qlinear_w8a8(x, wq, sw, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                 steer_alpha=None, acc_out=None, stream=None):
    torch = _torch()
    _dt(x, torch.float16, "x"), _dt(wq, torch.int8, "wq"), _dt(sw, torch.float16, "sw")
    M, K = x.shape
    N = wq.shape[0]
    y = _out(x, N, y)
    ws, nb = _ws(ARIA_W8A8, M, K, N, ws, x.device)
    e = _epi(bias, gelu, residual, steer_dir, steer_alpha, acc_out)
    _check(lib.aria_qlinear_w8a8(_addr(x), M, K, N, _addr(wq), _addr(sw), ctypes.byref(e), _addr(y), _addr(ws),
                                 nb, _stream(stream)), "qlinear_w8a8")
    return y


def qlinear_w8a16(x, wq, sw, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                  steer_alpha=None, stream=None):
    torch = _torch()
    _dt(x, torch.float16, "x"), _dt(wq, torch.int8, "wq"), _dt(sw, torch.float16, "sw")
    M, K = x.shape
    N = wq.shape[0]
    y = _out(x, N, y)
    ws, nb = _ws(ARIA_W8A16, M, K, N, ws, x.device)
    e = _epi(bias, gelu, residual, steer_dir, steer_alpha, None)
    _check(lib.aria_qlinear_w8a16(_addr(x), M, K, N, _addr(wq), _addr(sw), ctypes.byref(e), _addr(y), _addr(ws),
                                  nb, _stream(stream)), "qlinear_w8a16")
    return y


def qlinear_w4a16(x, wq4, sg, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                  steer_alpha=None, stream=None, group: int = 32):
    torch = _torch()
    _dt(x, torch.float16, "x"), _dt(wq4, torch.uint8, "wq4"), _dt(sg, torch.float16, "sg")
    M, K = x.shape
    N = wq4.shape[0]
    y = _out(x, N, y)
    ws, nb = _ws(ARIA_W4A16, M, K, N, ws, x.device)
    e = _epi(bias, gelu, residual, steer_dir, steer_alpha, None)
    _check(lib.aria_qlinear_w4a16(_addr(x), M, K, N, _addr(wq4), _addr(sg), group, ctypes.byref(e), _addr(y),
                                  _addr(ws), nb, _stream(stream)), "qlinear_w4a16")
    return y


def qlinear_w16a16(x, wt, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                   steer_alpha=None, stream=None):
    """The fp16 rung: Y = epilogue(X Wt^T) with Wt fp16 [N][K] from qpack(16, W)."""
    torch = _torch()
    _dt(x, torch.float16, "x"), _dt(wt, torch.float16, "wt")
    M, K = x.shape
    N = wt.shape[0]
    y = _out(x, N, y)
    ws, nb = _ws(ARIA_W16A16, M, K, N, ws, x.device)
    e = _epi(bias, gelu, residual, steer_dir, steer_alpha, None)
    _check(lib.aria_qlinear_w16a16(_addr(x), M, K, N, _addr(wt), ctypes.byref(e), _addr(y), _addr(ws), nb,
                                   _stream(stream)), "qlinear_w16a16")
    return y


def qlinear_grouped(bits: int, problems, stream=None):
    """Several independent weight-only linears at small M in one call.
    ``problems``: a list of dicts with keys x, wq, s and optionally y, bias,
    gelu, residual, steer_dir, steer_alpha (as for qlinear_w8a16 /
    qlinear_w4a16).  bits 8 -> W8A16, bits 4 -> W4A16 (group 32).  Returns the
    list of outputs."""
    torch = _torch()
    arr = (LinearProblem * len(problems))()
    keep, outs = [], []
    for i, p in enumerate(problems):
        x, wq, s = p["x"], p["wq"], p["s"]
        _dt(x, torch.float16, "x"), _dt(wq, torch.int8 if bits == 8 else torch.uint8, "wq"), _dt(s, torch.float16, "s")
        M, K = x.shape
        N = wq.shape[0]
        y = _out(x, N, p.get("y"))
        e = _epi(p.get("bias"), p.get("gelu", False), p.get("residual"), p.get("steer_dir"),
                 p.get("steer_alpha"), None)
        keep.append(e)
        outs.append(y)
        arr[i] = LinearProblem(_addr(x), M, K, N, _addr(wq), _addr(s), ctypes.pointer(e), _addr(y))
    _check(lib.aria_qlinear_grouped(bits, 0 if bits == 8 else 32, arr, len(problems), _stream(stream)),
           "qlinear_grouped")
    return outs


def layernorm(x, gamma, beta, eps: float = 1e-5, y=None, stream=None):
    """LayerNorm of every row of x fp16 [M][W] (y may be x)."""
    torch = _torch()
    _dt(x, torch.float16, "x"), _dt(gamma, torch.float16, "gamma"), _dt(beta, torch.float16, "beta")
    M, W = x.shape
    y = torch.empty_like(x) if y is None else y
    _check(lib.aria_layernorm(_addr(x), M, W, _addr(gamma), _addr(beta), float(eps), _addr(y), _stream(stream)),
           "layernorm")
    return y


def layernorm_quant(x, gamma, beta, eps: float = 1e-5, y=None, xq=None, sa=None, want_y: bool = False,
                    stream=None):
    """LayerNorm of x fp16 [M][W] and the per-token quantization of the
    result in one pass: returns (xq, sa) or, with want_y / a given y,
    (y, xq, sa)."""
    torch = _torch()
    _dt(x, torch.float16, "x"), _dt(gamma, torch.float16, "gamma"), _dt(beta, torch.float16, "beta")
    M, W = x.shape
    if y is None and want_y:
        y = torch.empty_like(x)
    xq = torch.empty((M, W), dtype=torch.int8, device=x.device) if xq is None else xq
    sa = torch.empty((M,), dtype=torch.float16, device=x.device) if sa is None else sa
    _check(lib.aria_layernorm_quant(_addr(x), M, W, _addr(gamma), _addr(beta), float(eps), _addr(y), _addr(xq),
                                    _addr(sa), _stream(stream)), "layernorm_quant")
    return (xq, sa) if y is None else (y, xq, sa)


def qlinear_w8a8_prequant(xq, sa, wq, sw, y=None, bias=None, gelu=False, residual=None, steer_dir=None,
                          steer_alpha=None, acc_out=None, stream=None):
    """The W8A8 linear on activations quantized beforehand (xq int8 [M][K],
    sa fp16 [M])."""
    torch = _torch()
    _dt(xq, torch.int8, "xq"), _dt(sa, torch.float16, "sa"), _dt(wq, torch.int8, "wq"), _dt(sw, torch.float16, "sw")
    M, K = xq.shape
    N = wq.shape[0]
    y = torch.empty((M, N), dtype=torch.float16, device=xq.device) if y is None else y
    e = _epi(bias, gelu, residual, steer_dir, steer_alpha, acc_out)
    _check(lib.aria_qlinear_w8a8_prequant(_addr(xq), _addr(sa), M, K, N, _addr(wq), _addr(sw), ctypes.byref(e),
                                          _addr(y), _stream(stream)), "qlinear_w8a8_prequant")
    return y


def attention(qkv, heads: int, seq: int, out=None, stream=None):
    """Multi-head self-attention over [Q | K | V] = qkv fp16 [M][3W] within
    sequences of `seq` rows; returns out fp16 [M][W]."""
    torch = _torch()
    _dt(qkv, torch.float16, "qkv")
    M, W3 = qkv.shape
    W = W3 // 3
    out = torch.empty((M, W), dtype=torch.float16, device=qkv.device) if out is None else out
    _check(lib.aria_attention(_addr(qkv), M, W, int(heads), int(seq), _addr(out), _stream(stream)), "attention")
    return out
