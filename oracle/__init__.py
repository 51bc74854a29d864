"""aria qlinear ORACLE — test infrastructure only.

A plain CPU model (fp64 reals, exact int64 integers) of the quantized linear
layer of the aria runtime ("A Quantized Native Runtime for On-Device Semantic
Audio Generation", project page: "What aria is" — weights packed from fp16 to
8 or 4 bits; "Results" — the q8 / W8A8 / q4 precision table and the steering
add on one block's residual stream).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never calls it and
shares no code with it.  The arithmetic lives in ``aria_oracle.c``; this module
only marshals numpy arrays (fp16 travels as its raw 16-bit pattern) and
composes the C steps in the order the method applies them.

Every function here is pinned by ``tests/test_oracle_*.py`` against something
other than itself (numpy's own fp16 conversion, exact rational arithmetic,
brute-force loops, numpy int64/fp64 matmul, closed forms).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "aria_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra"]

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile ``aria_oracle.c`` into ``liboracle.so`` with gcc (no fast-math,
    no FMA contraction) and return its path."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        # a test may point the wrapper at a deliberately broken copy of the
        # oracle (mutation testing of the pins); normal use loads liboracle.so
        path = os.environ.get("ARIA_ORACLE_LIB", _LIB_PATH)
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.or_f16_to_f64.restype = ctypes.c_double
        lib.or_f64_to_f16.argtypes = [ctypes.c_double]
        lib.or_f64_to_f16.restype = ctypes.c_uint16
        lib.or_rne.argtypes = [ctypes.c_double]
        lib.or_rne.restype = ctypes.c_double
        lib.or_gelu_tanh.argtypes = [ctypes.c_double]
        lib.or_gelu_tanh.restype = ctypes.c_double
        sigs = {
            "or_f16_to_f64_array": [P, P, I64],
            "or_f64_to_f16_array": [P, P, I64],
            "or_quant_sym": [P, I64, I64, ctypes.c_int, P, P],
            "or_qpack8": [P, I64, I64, P, P],
            "or_qpack4": [P, I64, I64, I64, P, P],
            "or_unpack4": [P, I64, I64, P],
            "or_quant_act": [P, I64, I64, P, P],
            "or_gemm_i8": [P, P, I64, I64, I64, P],
            "or_ref_w8a16": [P, P, P, I64, I64, I64, P],
            "or_ref_w4a16": [P, P, P, I64, I64, I64, I64, P],
            "or_pack16": [P, I64, I64, P],
            "or_ref_w16a16": [P, P, I64, I64, I64, P],
            "or_scale_w8a8": [P, P, P, I64, I64, P],
            "or_layernorm": [P, P, P, ctypes.c_double, I64, I64, P],
            "or_attention": [P, I64, I64, I64, I64, P],
            "or_epilogue": [P, I64, I64, P, ctypes.c_int, P, P, ctypes.c_float],
        }
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} failed with code {rc}")


def _bits(a) -> np.ndarray:
    """fp16 array (or its uint16 pattern) -> C-contiguous uint16 pattern."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError(f"expected float16/uint16, got {a.dtype}")
    return np.ascontiguousarray(a)


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return np.ascontiguousarray(a)


# --------------------------------------------------------------------------
# C-1 binary16 codec
# --------------------------------------------------------------------------
def f16_to_f64(h) -> np.ndarray:
    h = _bits(h)
    out = np.empty(h.shape, np.float64)
    _check(_load().or_f16_to_f64_array(_ptr(h), _ptr(out), h.size), "f16_to_f64")
    return out


def f64_to_f16(x) -> np.ndarray:
    """fp64 -> fp16 (RNE), returned as numpy float16."""
    x = np.ascontiguousarray(np.asarray(x, np.float64))
    out = np.empty(x.shape, np.uint16)
    _check(_load().or_f64_to_f16_array(_ptr(x), _ptr(out), x.size), "f64_to_f16")
    return out.view(np.float16)


def rne(x: float) -> float:
    return _load().or_rne(float(x))


def gelu_tanh(y: float) -> float:
    return _load().or_gelu_tanh(float(y))


# --------------------------------------------------------------------------
# C-2 quantizer, a1 packing, a2 activation quantization
# --------------------------------------------------------------------------
def quant_sym(v, qmax: int):
    """Quantize one vector of fp16 values: returns (q int8[L], s float16)."""
    v = _bits(v).ravel()
    q = np.empty(v.size, np.int8)
    s = np.zeros(1, np.uint16)
    _check(_load().or_quant_sym(_ptr(v), v.size, 1, int(qmax), _ptr(q), _ptr(s)), "quant_sym")
    return q, s.view(np.float16)[0]


def qpack8(w):
    """W fp16 [K][N] -> (Wq int8 [N][K], s_w fp16 [N])."""
    w = _bits(w)
    K, N = w.shape
    q = np.empty((N, K), np.int8)
    s = np.empty(N, np.uint16)
    _check(_load().or_qpack8(_ptr(w), K, N, _ptr(q), _ptr(s)), "qpack8")
    return q, s.view(np.float16)


def qpack4(w, group: int = 32):
    """W fp16 [K][N] -> (Wq4 uint8 [N][K/2], s4 fp16 [N][K/group])."""
    w = _bits(w)
    K, N = w.shape
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // group), np.uint16)
    _check(_load().or_qpack4(_ptr(w), K, N, int(group), _ptr(q), _ptr(s)), "qpack4")
    return q, s.view(np.float16)


def unpack4(q4, K: int) -> np.ndarray:
    q4 = _c(q4, np.uint8)
    N = q4.shape[0]
    q = np.empty((N, K), np.int8)
    _check(_load().or_unpack4(_ptr(q4), K, N, _ptr(q)), "unpack4")
    return q


def quant_act(x):
    """X fp16 [M][K] -> (Xq int8 [M][K], s_a fp16 [M])."""
    x = _bits(x)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.uint16)
    _check(_load().or_quant_act(_ptr(x), M, K, _ptr(q), _ptr(s)), "quant_act")
    return q, s.view(np.float16)


# --------------------------------------------------------------------------
# C-4 contractions, C-5 epilogue
# --------------------------------------------------------------------------
def gemm_i8(xq, wq) -> np.ndarray:
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K
    acc = np.empty((M, N), np.int32)
    _check(_load().or_gemm_i8(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc)), "gemm_i8")
    return acc


def ref_w8a16(x, wq, sw) -> np.ndarray:
    x = _bits(x)
    wq = _c(wq, np.int8)
    sw = _bits(sw)
    M, K = x.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and sw.shape == (N,)
    r = np.empty((M, N), np.float64)
    _check(_load().or_ref_w8a16(_ptr(x), _ptr(wq), _ptr(sw), M, N, K, _ptr(r)), "ref_w8a16")
    return r


def ref_w4a16(x, q4, s4, group: int = 32) -> np.ndarray:
    x = _bits(x)
    q4 = _c(q4, np.uint8)
    s4 = _bits(s4)
    M, K = x.shape
    N = q4.shape[0]
    assert q4.shape[1] * 2 == K and s4.shape == (N, K // group)
    r = np.empty((M, N), np.float64)
    _check(_load().or_ref_w4a16(_ptr(x), _ptr(q4), _ptr(s4), int(group), M, N, K, _ptr(r)),
           "ref_w4a16")
    return r


def pack16(w):
    """W fp16 [K][N] -> Wt fp16 [N][K] (the fp16 rung's weight layout)."""
    w = _bits(w)
    K, N = w.shape
    wt = np.empty((N, K), np.uint16)
    _check(_load().or_pack16(_ptr(w), K, N, _ptr(wt)), "pack16")
    return wt.view(np.float16)


def ref_w16a16(x, wt) -> np.ndarray:
    x = _bits(x)
    wt = _bits(wt)
    M, K = x.shape
    N = wt.shape[0]
    assert wt.shape[1] == K
    r = np.empty((M, N), np.float64)
    _check(_load().or_ref_w16a16(_ptr(x), _ptr(wt), M, N, K, _ptr(r)), "ref_w16a16")
    return r


def scale_w8a8(acc, sa, sw) -> np.ndarray:
    acc = _c(acc, np.int32)
    sa = _bits(sa)
    sw = _bits(sw)
    M, N = acc.shape
    y = np.empty((M, N), np.float64)
    _check(_load().or_scale_w8a8(_ptr(acc), _ptr(sa), _ptr(sw), M, N, _ptr(y)), "scale_w8a8")
    return y


def epilogue(y, bias=None, gelu=False, residual=None, d=None, alpha=0.0) -> np.ndarray:
    """Returns a new fp64 array: y (+bias) (gelu) (+residual) (+alpha*d)."""
    y = np.array(y, np.float64, order="C", copy=True)
    M, N = y.shape
    b = None if bias is None else _bits(bias)
    r = None if residual is None else _bits(residual)
    dd = None if d is None else _c(d, np.float32)
    if b is not None:
        assert b.shape == (N,)
    if r is not None:
        assert r.shape == (M, N)
    if dd is not None:
        assert dd.shape == (N,)
    _check(_load().or_epilogue(_ptr(y), M, N, _ptr(b), int(bool(gelu)), _ptr(r), _ptr(dd),
                               ctypes.c_float(float(alpha))), "epilogue")
    return y


# --------------------------------------------------------------------------
# Whole modes: the layer as the method applies it
# --------------------------------------------------------------------------
def qlinear_w8a8(x, wq, sw, **epi):
    """act-quant -> exact int GEMM -> acc*s_a*s_w -> epilogue.
    Returns dict(xq, sa, acc, y) with y fp64."""
    xq, sa = quant_act(x)
    acc = gemm_i8(xq, wq)
    y = epilogue(scale_w8a8(acc, sa, sw), **epi)
    return {"xq": xq, "sa": sa, "acc": acc, "y": y}


def qlinear_w8a16(x, wq, sw, **epi) -> np.ndarray:
    return epilogue(ref_w8a16(x, wq, sw), **epi)


def qlinear_w16a16(x, wt, **epi) -> np.ndarray:
    return epilogue(ref_w16a16(x, wt), **epi)


def qlinear_w4a16(x, q4, s4, group=32, **epi) -> np.ndarray:
    return epilogue(ref_w4a16(x, q4, s4, group), **epi)


def layernorm(x, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm over each row of x fp16 [M][W] with fp16 gamma, beta [W] (fp64 out)."""
    x = _bits(x)
    gamma = _bits(gamma)
    beta = _bits(beta)
    M, W = x.shape
    assert gamma.shape == (W,) and beta.shape == (W,)
    y = np.empty((M, W), np.float64)
    _check(_load().or_layernorm(_ptr(x), _ptr(gamma), _ptr(beta), float(eps), M, W, _ptr(y)), "layernorm")
    return y


def attention(qkv, heads: int, seq: int) -> np.ndarray:
    """Multi-head softmax self-attention over [Q | K | V] = qkv fp16 [M][3W]
    within each sequence of `seq` rows (fp64 out [M][W])."""
    qkv = _bits(qkv)
    M, W3 = qkv.shape
    W = W3 // 3
    out = np.empty((M, W), np.float64)
    _check(_load().or_attention(_ptr(qkv), M, W, int(heads), int(seq), _ptr(out)), "attention")
    return out


def dit_block_full_w8a8(h, packed, ln1, ln2, heads: int, seq: int, d=None, alpha=0.0, eps: float = 1e-5):
    """The W8A8 DiT block with its attention core and norms, rounding to fp16
    at every stage boundary as the device stores it:
      n1 = LN1(h);  qkv = n1.Wqkv;  a = attention(qkv);  h1 = h + a.Wo;
      n2 = LN2(h1);  u = gelu(n2.Wup);  out = h1 + u.Wdown + alpha*d.
    ``ln1`` / ``ln2`` are (gamma, beta) pairs.  Returns the fp16 stage outputs
    and the fp64 value of the last stage."""
    h = np.asarray(h, np.float16)
    n1 = f64_to_f16(layernorm(h, *ln1, eps))
    qkv = f64_to_f16(qlinear_w8a8(n1, *packed["qkv"])["y"])
    a = f64_to_f16(attention(qkv, heads, seq))
    h1 = f64_to_f16(qlinear_w8a8(a, *packed["o"], residual=h)["y"])
    n2 = f64_to_f16(layernorm(h1, *ln2, eps))
    u = f64_to_f16(qlinear_w8a8(n2, *packed["up"], gelu=True)["y"])
    out64 = qlinear_w8a8(u, *packed["down"], residual=h1, d=d, alpha=alpha)["y"]
    return {"n1": n1, "qkv": qkv, "a": a, "h1": h1, "n2": n2, "u": u, "out": f64_to_f16(out64), "out64": out64}


def dit_block_w8a8(h, packed, d=None, alpha=0.0):
    """The W8A8 block chain, end to end, rounding to fp16 at every stage
    boundary as the device stores it:
      qkv = h.Wqkv;  a = V slice of qkv (identity attention: each token
      attends only to itself);  h1 = h + a.Wo;  u = gelu(h1.Wup);
      out = h1 + u.Wdown + alpha*d  (steering on the block output only).
    ``packed`` maps 'qkv','o','up','down' to (Wq, s_w).  Returns dict of the
    fp16 stage outputs and the fp64 value of the last stage."""
    h = np.asarray(h, np.float16)
    width = h.shape[1]
    qkv = f64_to_f16(qlinear_w8a8(h, *packed["qkv"])["y"])
    a = np.ascontiguousarray(qkv[:, 2 * width:3 * width])
    h1 = f64_to_f16(qlinear_w8a8(a, *packed["o"], residual=h)["y"])
    u = f64_to_f16(qlinear_w8a8(h1, *packed["up"], gelu=True)["y"])
    out64 = qlinear_w8a8(u, *packed["down"], residual=h1, d=d, alpha=alpha)["y"]
    return {"qkv": qkv, "a": a, "h1": h1, "u": u, "out": f64_to_f16(out64), "out64": out64}
