"""The W8A8 diffusion-transformer block chain built from qlinear calls.

The aria pages run the denoising step's transformer blocks at W8A8 and add the
steering direction to one block's residual stream (project page, "Results":
"Steering is real, inside a narrow window"; the CLI form
``--steer residual:<block>:<file>:<alpha>:<steps>``).  The block here is
QKV -> attention -> out-projection (+ residual) -> MLP-up (GELU) -> MLP-down
(+ residual + alpha * d).  The attention core is not a quantized linear; it is
stood in for by identity attention (each token attends only to itself, so the
attention output is the V third of the QKV output), which keeps the chain
data-dependent and row-local.  The out-projection's per-token quantization
reads that third in place (a row-strided act-quant), so the stand-in costs no
copy; every arithmetic step runs in the qlinear kernels.
"""
from __future__ import annotations

from . import binding as B


class DitBlockW8A8:
    """Preallocated W8A8 block: ``run(h)`` enqueues the chain on the stream and
    returns the block output (fp16 [M][width])."""

    def __init__(self, packed: dict, M: int, width: int, mlp: int, steer_dir=None, steer_alpha=None,
                 fuse_out_quant: bool = False):
        import torch
        dev = packed["qkv"][0].device
        self.packed, self.M, self.width, self.mlp = packed, M, width, mlp
        self.steer_dir, self.steer_alpha = steer_dir, steer_alpha
        # fuse_out_quant: the QKV linear records the V third's row maxima and
        # the out-projection quantizes V inside its contraction (no separate
        # quantization pass; bit-identical output)
        self.fuse_out_quant = fuse_out_quant
        self.rowmax = torch.empty((M, width // 64), dtype=torch.int32, device=dev) if fuse_out_quant else None
        f16 = torch.float16
        self.qkv = torch.empty((M, 3 * width), dtype=f16, device=dev)
        self.xq = torch.empty((M, width), dtype=torch.int8, device=dev)   # quantized V third
        self.sa = torch.empty((M,), dtype=f16, device=dev)
        self.h1 = torch.empty((M, width), dtype=f16, device=dev)
        self.u = torch.empty((M, mlp), dtype=f16, device=dev)
        self.out = torch.empty((M, width), dtype=f16, device=dev)
        need = max(B.workspace_bytes(B.ARIA_W8A8, M, k, n)
                   for k, n in ((width, 3 * width), (width, width), (width, mlp), (mlp, width)))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def _qkv(self, h, stream):
        p = self.packed
        if self.fuse_out_quant:
            B.qlinear_w8a8_rowmax(h, *p["qkv"], 2 * self.width, self.width, y=self.qkv, ws=self.ws,
                                  rowmax=self.rowmax, stream=stream)
        else:
            B.qlinear_w8a8(h, *p["qkv"], y=self.qkv, ws=self.ws, stream=stream)

    def _out(self, h, stream):
        # identity attention: the out-projection's input is the V third of qkv
        if self.fuse_out_quant:
            B.qlinear_w8a8_fused(self.qkv, 2 * self.width, self.width, self.rowmax, *self.packed["o"], y=self.h1,
                                 residual=h, stream=stream)
            return
        B.quant_act_columns(self.qkv, 2 * self.width, self.width, xq=self.xq, sa=self.sa, stream=stream)
        B.qlinear_w8a8_prequant(self.xq, self.sa, *self.packed["o"], y=self.h1, residual=h, stream=stream)

    def calls(self, h, stream=None):
        """The stages as (name, callable) pairs, in order; each call enqueues one
        stage on the stream (re-running one alone recomputes it from the
        buffers the previous stage left).  Each linear's stage includes its
        activation quantization."""
        p = self.packed
        return [
            ("qkv", lambda: self._qkv(h, stream)),
            ("out", lambda: self._out(h, stream)),
            ("up", lambda: B.qlinear_w8a8(self.h1, *p["up"], y=self.u, ws=self.ws, gelu=True, stream=stream)),
            ("down", lambda: B.qlinear_w8a8(self.u, *p["down"], y=self.out, ws=self.ws, residual=self.h1,
                                            steer_dir=self.steer_dir, steer_alpha=self.steer_alpha,
                                            stream=stream)),
        ]

    def stages(self, h, stream=None):
        """Yields after each stage (for per-stage timing or checks)."""
        for name, fn in self.calls(h, stream):
            fn()
            yield name

    def run(self, h, stream=None):
        for _ in self.stages(h, stream):
            pass
        return self.out


class DitBlockFullW8A8:
    """The W8A8 block with its attention core and pre-norms (docshare paper
    page, Fig. 1 "DiT blocks"):
      n1 = LN1(h);  qkv = n1.Wqkv;  a = attention(qkv);  h1 = h + a.Wo;
      n2 = LN2(h1); u = gelu(n2.Wup); out = h1 + u.Wdown + alpha*d,
    with `heads` 64-dimensional heads over sequences of `seq` tokens (the M
    rows hold M / seq sequences, e.g. two guidance branches).  Every step runs
    in the library's kernels; ``run(h)`` returns the block output.  Each
    pre-norm is fused with the per-token quantization of the W8A8 linear it
    feeds (the normalized rows stay in registers); ``keep_norms`` also writes
    the fp16 normalized rows to ``n1`` / ``n2`` for inspection."""

    def __init__(self, packed: dict, ln1, ln2, M: int, width: int, mlp: int, heads: int, seq: int,
                 steer_dir=None, steer_alpha=None, eps: float = 1e-5, keep_norms: bool = False):
        import torch
        dev = packed["qkv"][0].device
        self.packed, self.ln1, self.ln2, self.eps = packed, ln1, ln2, eps
        self.M, self.width, self.mlp, self.heads, self.seq = M, width, mlp, heads, seq
        self.steer_dir, self.steer_alpha = steer_dir, steer_alpha
        f16 = torch.float16
        self.n1 = torch.empty((M, width), dtype=f16, device=dev) if keep_norms else None
        self.n2 = torch.empty((M, width), dtype=f16, device=dev) if keep_norms else None
        self.xq = torch.empty((M, width), dtype=torch.int8, device=dev)   # quantized n1, then n2
        self.sa = torch.empty((M,), dtype=f16, device=dev)
        self.qkv = torch.empty((M, 3 * width), dtype=f16, device=dev)
        self.a = torch.empty((M, width), dtype=f16, device=dev)
        self.h1 = torch.empty((M, width), dtype=f16, device=dev)
        self.u = torch.empty((M, mlp), dtype=f16, device=dev)
        self.out = torch.empty((M, width), dtype=f16, device=dev)
        need = max(B.workspace_bytes(B.ARIA_W8A8, M, k, n)
                   for k, n in ((width, 3 * width), (width, width), (width, mlp), (mlp, width)))
        self.ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def calls(self, h, stream=None):
        """The stages as (name, callable) pairs, in order (see DitBlockW8A8.calls)."""
        p = self.packed
        return [
            ("ln1", lambda: B.layernorm_quant(h, *self.ln1, eps=self.eps, y=self.n1, xq=self.xq, sa=self.sa,
                                              stream=stream)),
            ("qkv", lambda: B.qlinear_w8a8_prequant(self.xq, self.sa, *p["qkv"], y=self.qkv, stream=stream)),
            ("attention", lambda: B.attention(self.qkv, self.heads, self.seq, out=self.a, stream=stream)),
            ("out", lambda: B.qlinear_w8a8(self.a, *p["o"], y=self.h1, ws=self.ws, residual=h, stream=stream)),
            ("ln2", lambda: B.layernorm_quant(self.h1, *self.ln2, eps=self.eps, y=self.n2, xq=self.xq, sa=self.sa,
                                              stream=stream)),
            ("up", lambda: B.qlinear_w8a8_prequant(self.xq, self.sa, *p["up"], y=self.u, gelu=True,
                                                   stream=stream)),
            ("down", lambda: B.qlinear_w8a8(self.u, *p["down"], y=self.out, ws=self.ws, residual=self.h1,
                                            steer_dir=self.steer_dir, steer_alpha=self.steer_alpha,
                                            stream=stream)),
        ]

    def stages(self, h, stream=None):
        for name, fn in self.calls(h, stream):
            fn()
            yield name

    def run(self, h, stream=None):
        for _ in self.stages(h, stream):
            pass
        return self.out
