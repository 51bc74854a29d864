"""ctypes binding of the C-ABI in include/aria_qlinear.h (same names, minus
the ``aria_`` prefix).  Arguments are contiguous torch tensors on one GPU;
nothing here computes any part of the layer.  The C-ABI receives raw pointers
and cannot tell a buffer's size, so every wrapper checks each tensor's
dtype, shape and device against the call's M, K, N before anything reaches
the library (TypeError for a wrong dtype, ValueError for a wrong shape or
device)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ARIA_QLINEAR_LIB selects another build of the same library (e.g. one whose
# host code carries address and undefined-behaviour sanitizers)
library_path = os.environ.get("ARIA_QLINEAR_LIB", os.path.join(HERE, "libaria_qlinear.so"))

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
lib.aria_qlinear_w8a8_noalloc.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.POINTER(Epilogue), _P, _P]
lib.aria_qlinear_w8a8_rowmax.restype = _I
lib.aria_qlinear_w8a8_rowmax.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.POINTER(Epilogue), _P, _P, _SZ, _P,
                                         _I64, _I64, _P]
lib.aria_qlinear_w8a8_fused.restype = _I
lib.aria_qlinear_w8a8_fused.argtypes = [_P, _I64, _P, _I64, _I64, _I64, _P, _P, ctypes.POINTER(Epilogue), _P, _P, _P]
lib.aria_qlinear_w8a8_noalloc.restype = _I
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
    """Device address of a checked tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous GPU tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _arg(t, dtype, shape, name, device=None):
    """Check an operand: a torch tensor (or None) of `dtype`, exactly `shape`,
    on `device` when given.  Returns t."""
    if t is None:
        return t
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, the other operands on {device}")
    return t


def _mat(t, dtype, name):
    """A 2-D operand whose shape defines the call: returns (rows, cols)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D tensor, got shape {tuple(t.shape)}")
    return t.shape


def qpack_bytes(bits: int, group: int, K: int, N: int):
    qb, sb = _SZ(), _SZ()
    _check(lib.aria_qpack_bytes(bits, group, K, N, ctypes.byref(qb), ctypes.byref(sb)), "qpack_bytes")
    return qb.value, sb.value


def qpack(bits: int, w, q=None, s=None, stream=None):
    """Pack fp16 W [K][N]: bits 8 -> (Wq int8 [N][K], s fp16 [N]);
    bits 4 -> (Wq4 uint8 [N][K/2], s fp16 [N][K/32]); bits 16 -> (Wt fp16 [N][K], None)."""
    torch = _torch()
    if bits not in (4, 8, 16):
        raise ValueError(f"bits must be 4, 8 or 16, got {bits}")
    K, N = _mat(w, torch.float16, "w")
    group = 32 if bits == 4 else 0
    qshape = (N, K // 2) if bits == 4 else (N, K)
    qtype = {8: torch.int8, 4: torch.uint8, 16: torch.float16}[bits]
    sshape = (N,) if bits == 8 else (N, K // 32)
    q = torch.empty(qshape, dtype=qtype, device=w.device) if q is None else _arg(q, qtype, qshape, "q", w.device)
    if bits == 16:
        s = None
    else:
        s = (torch.empty(sshape, dtype=torch.float16, device=w.device) if s is None
             else _arg(s, torch.float16, sshape, "s", w.device))
    _check(lib.aria_qpack(bits, group, _addr(w), K, N, _addr(q), _addr(s), _stream(stream)), "qpack")
    return q, s


def quant_act(x, xq=None, sa=None, stream=None):
    torch = _torch()
    M, K = _mat(x, torch.float16, "x")
    xq = torch.empty((M, K), dtype=torch.int8, device=x.device) if xq is None else xq
    sa = torch.empty((M,), dtype=torch.float16, device=x.device) if sa is None else sa
    _arg(xq, torch.int8, (M, K), "xq", x.device), _arg(sa, torch.float16, (M,), "sa", x.device)
    _check(lib.aria_quant_act(_addr(x), M, K, _addr(xq), _addr(sa), _stream(stream)), "quant_act")
    return xq, sa


def quant_act_columns(src, col0: int, ncols: int, xq=None, sa=None, stream=None):
    """Per-token quantization of the column block src[:, col0:col0+ncols] of a
    contiguous fp16 [M][W] tensor, read in place (row stride W)."""
    torch = _torch()
    M, W = _mat(src, torch.float16, "src")
    if not (0 <= col0 and 0 < ncols and col0 + ncols <= W):
        raise ValueError("column block outside the tensor")
    xq = torch.empty((M, ncols), dtype=torch.int8, device=src.device) if xq is None else xq
    sa = torch.empty((M,), dtype=torch.float16, device=src.device) if sa is None else sa
    _arg(xq, torch.int8, (M, ncols), "xq", src.device), _arg(sa, torch.float16, (M,), "sa", src.device)
    _check(lib.aria_quant_act_strided(_addr(src) + 2 * col0, W, M, ncols, _addr(xq), _addr(sa), _stream(stream)),
           "quant_act_strided")
    return xq, sa


def workspace_bytes(mode: int, M: int, K: int, N: int) -> int:
    return int(lib.aria_qlinear_workspace_bytes(mode, M, K, N))


def _epi(M, N, device, bias, gelu, residual, steer_dir, steer_alpha, acc_out):
    torch = _torch()
    _arg(bias, torch.float16, (N,), "bias", device)
    _arg(residual, torch.float16, (M, N), "residual", device)
    _arg(steer_dir, torch.float32, (N,), "steer_dir", device)
    if steer_alpha is not None:
        if not isinstance(steer_alpha, torch.Tensor) or steer_alpha.numel() != 1:
            raise ValueError("steer_alpha: expected a one-element device tensor")
        _arg(steer_alpha, torch.float32, tuple(steer_alpha.shape), "steer_alpha", device)
    _arg(acc_out, torch.int32, (M, N), "acc_out", device)
    return Epilogue(_addr(bias), int(bool(gelu)), 0, _addr(residual), _addr(steer_dir), _addr(steer_alpha),
                    _addr(acc_out))


def _ws(mode, M, K, N, ws, device):
    need = workspace_bytes(mode, M, K, N)
    if ws is None:
        ws = _torch().empty(need, dtype=_torch().uint8, device=device) if need else None
    elif not isinstance(ws, _torch().Tensor) or ws.device != device:
        raise ValueError("ws: expected a tensor on the operands' device")
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def _out(M, N, y, device, name="y"):
    torch = _torch()
    if y is None:
        return torch.empty((M, N), dtype=torch.float16, device=device)
    return _arg(y, torch.float16, (M, N), name, device)


def qlinear_w8a8(x, wq, sw, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                 steer_alpha=None, acc_out=None, stream=None):
    torch = _torch()
    M, K = _mat(x, torch.float16, "x")
    N, _ = _mat(wq, torch.int8, "wq")
    _arg(wq, torch.int8, (N, K), "wq", x.device), _arg(sw, torch.float16, (N,), "sw", x.device)
    y = _out(M, N, y, x.device)
    e = _epi(M, N, x.device, bias, gelu, residual, steer_dir, steer_alpha, acc_out)
    ws, nb = _ws(ARIA_W8A8, M, K, N, ws, x.device)
    _check(lib.aria_qlinear_w8a8(_addr(x), M, K, N, _addr(wq), _addr(sw), ctypes.byref(e), _addr(y), _addr(ws),
                                 nb, _stream(stream)), "qlinear_w8a8")
    return y


def qlinear_w8a8_noalloc(x, wq, sw, y=None, bias=None, gelu=False, residual=None, steer_dir=None,
                         steer_alpha=None, acc_out=None, stream=None):
    """qlinear_w8a8 without a workspace: the library's fixed device scratch
    holds the quantized activations (calls overlapping on one GPU race)."""
    torch = _torch()
    M, K = _mat(x, torch.float16, "x")
    N, _ = _mat(wq, torch.int8, "wq")
    _arg(wq, torch.int8, (N, K), "wq", x.device), _arg(sw, torch.float16, (N,), "sw", x.device)
    y = _out(M, N, y, x.device)
    e = _epi(M, N, x.device, bias, gelu, residual, steer_dir, steer_alpha, acc_out)
    _check(lib.aria_qlinear_w8a8_noalloc(_addr(x), M, K, N, _addr(wq), _addr(sw), ctypes.byref(e), _addr(y),
                                         _stream(stream)), "qlinear_w8a8_noalloc")
    return y


def qlinear_w8a8_rowmax(x, wq, sw, col0: int, ncols: int, y=None, ws=None, rowmax=None, bias=None, gelu=False,
                        residual=None, steer_dir=None, steer_alpha=None, acc_out=None, stream=None):
    """qlinear_w8a8 that also records the row maxima of the output columns
    [col0, col0 + ncols) in 64-column blocks (uint32 [M][ncols / 64], fp16
    magnitude bits) for qlinear_w8a8_fused.  Returns (y, rowmax)."""
    torch = _torch()
    M, K = _mat(x, torch.float16, "x")
    N, _ = _mat(wq, torch.int8, "wq")
    _arg(wq, torch.int8, (N, K), "wq", x.device), _arg(sw, torch.float16, (N,), "sw", x.device)
    if not (0 <= col0 and 64 <= ncols and col0 % 64 == 0 and ncols % 64 == 0 and col0 + ncols <= N):
        raise ValueError(f"rowmax columns [{col0}, {col0 + ncols}) are not 64-column blocks inside [0, {N})")
    y = _out(M, N, y, x.device)
    rowmax = torch.empty((M, ncols // 64), dtype=torch.int32, device=x.device) if rowmax is None else rowmax
    _arg(rowmax, torch.int32, (M, ncols // 64), "rowmax", x.device)
    e = _epi(M, N, x.device, bias, gelu, residual, steer_dir, steer_alpha, acc_out)
    ws, nb = _ws(ARIA_W8A8, M, K, N, ws, x.device)
    _check(lib.aria_qlinear_w8a8_rowmax(_addr(x), M, K, N, _addr(wq), _addr(sw), ctypes.byref(e), _addr(y),
                                        _addr(ws), nb, _addr(rowmax), int(col0), int(ncols), _stream(stream)),
           "qlinear_w8a8_rowmax")
    return y, rowmax


def qlinear_w8a8_fused(src, col0: int, ncols: int, rowmax, wq, sw, y=None, sa_out=None, bias=None, gelu=False,
                       residual=None, steer_dir=None, steer_alpha=None, acc_out=None, stream=None):
    """The W8A8 linear over the column block src[:, col0:col0+ncols] of a
    contiguous fp16 [M][W] tensor (read in place, row stride W), quantized
    per token inside the contraction with the scales from `rowmax` (the
    producer's qlinear_w8a8_rowmax output for exactly those columns)."""
    torch = _torch()
    M, W = _mat(src, torch.float16, "src")
    if not (0 <= col0 and 0 < ncols and col0 + ncols <= W):
        raise ValueError("column block outside the tensor")
    K = ncols
    N, _ = _mat(wq, torch.int8, "wq")
    _arg(wq, torch.int8, (N, K), "wq", src.device), _arg(sw, torch.float16, (N,), "sw", src.device)
    _arg(rowmax, torch.int32, (M, K // 64), "rowmax", src.device)
    _arg(sa_out, torch.float16, (M,), "sa_out", src.device)
    y = _out(M, N, y, src.device)
    e = _epi(M, N, src.device, bias, gelu, residual, steer_dir, steer_alpha, acc_out)
    _check(lib.aria_qlinear_w8a8_fused(_addr(src) + 2 * col0, W, _addr(rowmax), M, K, N, _addr(wq), _addr(sw),
                                       ctypes.byref(e), _addr(y), _addr(sa_out), _stream(stream)),
           "qlinear_w8a8_fused")
    return y


def _wxa16(bits, fn, name, x, wq, s, y, ws, bias, gelu, residual, steer_dir, steer_alpha, stream, group=None):
    torch = _torch()
    M, K = _mat(x, torch.float16, "x")
    wtype = {8: torch.int8, 4: torch.uint8, 16: torch.float16}[bits]
    N, _ = _mat(wq, wtype, "wq")
    _arg(wq, wtype, (N, K // 2) if bits == 4 else (N, K), "wq", x.device)
    if bits == 8:
        _arg(s, torch.float16, (N,), "s", x.device)
    elif bits == 4:
        _arg(s, torch.float16, (N, K // 32), "s", x.device)
    y = _out(M, N, y, x.device)
    e = _epi(M, N, x.device, bias, gelu, residual, steer_dir, steer_alpha, None)
    mode = {8: ARIA_W8A16, 4: ARIA_W4A16, 16: ARIA_W16A16}[bits]
    ws, nb = _ws(mode, M, K, N, ws, x.device)
    if bits == 16:
        rc = fn(_addr(x), M, K, N, _addr(wq), ctypes.byref(e), _addr(y), _addr(ws), nb, _stream(stream))
    elif bits == 4:
        rc = fn(_addr(x), M, K, N, _addr(wq), _addr(s), group, ctypes.byref(e), _addr(y), _addr(ws), nb,
                _stream(stream))
    else:
        rc = fn(_addr(x), M, K, N, _addr(wq), _addr(s), ctypes.byref(e), _addr(y), _addr(ws), nb, _stream(stream))
    _check(rc, name)
    return y


def qlinear_w8a16(x, wq, sw, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                  steer_alpha=None, stream=None):
    return _wxa16(8, lib.aria_qlinear_w8a16, "qlinear_w8a16", x, wq, sw, y, ws, bias, gelu, residual, steer_dir,
                  steer_alpha, stream)


def qlinear_w4a16(x, wq4, sg, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                  steer_alpha=None, stream=None, group: int = 32):
    if group != 32:
        raise ValueError(f"group must be 32, got {group}")
    return _wxa16(4, lib.aria_qlinear_w4a16, "qlinear_w4a16", x, wq4, sg, y, ws, bias, gelu, residual, steer_dir,
                  steer_alpha, stream, group)


def qlinear_w16a16(x, wt, y=None, ws=None, bias=None, gelu=False, residual=None, steer_dir=None,
                   steer_alpha=None, stream=None):
    """The fp16 rung: Y = epilogue(X Wt^T) with Wt fp16 [N][K] from qpack(16, W)."""
    return _wxa16(16, lib.aria_qlinear_w16a16, "qlinear_w16a16", x, wt, None, y, ws, bias, gelu, residual,
                  steer_dir, steer_alpha, stream)


def qlinear_grouped(bits: int, problems, stream=None):
    """Several independent weight-only linears at small M in one call.
    ``problems``: a list of dicts with keys x, wq, s and optionally y, bias,
    gelu, residual, steer_dir, steer_alpha (as for qlinear_w8a16 /
    qlinear_w4a16).  bits 8 -> W8A16, bits 4 -> W4A16 (group 32).  Returns the
    list of outputs."""
    torch = _torch()
    if bits not in (4, 8):
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    arr = (LinearProblem * len(problems))()
    keep, outs = [], []
    wtype = torch.int8 if bits == 8 else torch.uint8
    for i, p in enumerate(problems):
        x, wq, s = p["x"], p["wq"], p["s"]
        M, K = _mat(x, torch.float16, f"problems[{i}].x")
        N, _ = _mat(wq, wtype, f"problems[{i}].wq")
        _arg(wq, wtype, (N, K) if bits == 8 else (N, K // 2), f"problems[{i}].wq", x.device)
        _arg(s, torch.float16, (N,) if bits == 8 else (N, K // 32), f"problems[{i}].s", x.device)
        y = _out(M, N, p.get("y"), x.device, f"problems[{i}].y")
        e = _epi(M, N, x.device, p.get("bias"), p.get("gelu", False), p.get("residual"), p.get("steer_dir"),
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
    M, W = _mat(x, torch.float16, "x")
    _arg(gamma, torch.float16, (W,), "gamma", x.device), _arg(beta, torch.float16, (W,), "beta", x.device)
    y = torch.empty_like(x) if y is None else _arg(y, torch.float16, (M, W), "y", x.device)
    _check(lib.aria_layernorm(_addr(x), M, W, _addr(gamma), _addr(beta), float(eps), _addr(y), _stream(stream)),
           "layernorm")
    return y


def layernorm_quant(x, gamma, beta, eps: float = 1e-5, y=None, xq=None, sa=None, want_y: bool = False,
                    stream=None):
    """LayerNorm of x fp16 [M][W] and the per-token quantization of the
    result in one pass: returns (xq, sa) or, with want_y / a given y,
    (y, xq, sa)."""
    torch = _torch()
    M, W = _mat(x, torch.float16, "x")
    _arg(gamma, torch.float16, (W,), "gamma", x.device), _arg(beta, torch.float16, (W,), "beta", x.device)
    if y is None and want_y:
        y = torch.empty_like(x)
    _arg(y, torch.float16, (M, W), "y", x.device)
    xq = torch.empty((M, W), dtype=torch.int8, device=x.device) if xq is None else xq
    sa = torch.empty((M,), dtype=torch.float16, device=x.device) if sa is None else sa
    _arg(xq, torch.int8, (M, W), "xq", x.device), _arg(sa, torch.float16, (M,), "sa", x.device)
    _check(lib.aria_layernorm_quant(_addr(x), M, W, _addr(gamma), _addr(beta), float(eps), _addr(y), _addr(xq),
                                    _addr(sa), _stream(stream)), "layernorm_quant")
    return (xq, sa) if y is None else (y, xq, sa)


def qlinear_w8a8_prequant(xq, sa, wq, sw, y=None, bias=None, gelu=False, residual=None, steer_dir=None,
                          steer_alpha=None, acc_out=None, stream=None):
    """The W8A8 linear on activations quantized beforehand (xq int8 [M][K],
    sa fp16 [M])."""
    torch = _torch()
    M, K = _mat(xq, torch.int8, "xq")
    _arg(sa, torch.float16, (M,), "sa", xq.device)
    N, _ = _mat(wq, torch.int8, "wq")
    _arg(wq, torch.int8, (N, K), "wq", xq.device), _arg(sw, torch.float16, (N,), "sw", xq.device)
    y = _out(M, N, y, xq.device)
    e = _epi(M, N, xq.device, bias, gelu, residual, steer_dir, steer_alpha, acc_out)
    _check(lib.aria_qlinear_w8a8_prequant(_addr(xq), _addr(sa), M, K, N, _addr(wq), _addr(sw), ctypes.byref(e),
                                          _addr(y), _stream(stream)), "qlinear_w8a8_prequant")
    return y


def attention(qkv, heads: int, seq: int, out=None, stream=None):
    """Multi-head self-attention over [Q | K | V] = qkv fp16 [M][3W] within
    sequences of `seq` rows; returns out fp16 [M][W]."""
    torch = _torch()
    M, W3 = _mat(qkv, torch.float16, "qkv")
    if W3 % 3:
        raise ValueError(f"qkv: {W3} columns is not three blocks of equal width")
    W = W3 // 3
    out = _out(M, W, out, qkv.device, "out")
    _check(lib.aria_attention(_addr(qkv), M, W, int(heads), int(seq), _addr(out), _stream(stream)), "attention")
    return out
