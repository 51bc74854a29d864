"""Quantized linear layer ("qlinear") of a diffusion-transformer denoising step,
for AMD Instinct MI355X (gfx950): W8A8, W8A16 and W4A16 with a fused epilogue
(bias, GELU(tanh), residual, steering add alpha*d).

Every step runs in the HIP library ``libaria_qlinear.so`` behind the C-ABI of
``include/aria_qlinear.h``; this package only marshals arguments (device
pointers of torch tensors, sizes, the current HIP stream) and, for
convenience, allocates outputs with torch.  There is no fallback: importing
the binding without the built library raises.
"""
from .binding import (  # noqa: F401
    ARIA_W4A16, ARIA_W8A16, ARIA_W8A8, ARIA_W16A16, AriaError, attention, layernorm, layernorm_quant, lib,
    library_path, qlinear_grouped, qlinear_w4a16, qlinear_w8a8, qlinear_w8a8_fused, qlinear_w8a8_noalloc,
    qlinear_w8a8_prequant, qlinear_w8a8_rowmax, qlinear_w8a16,
    qlinear_w16a16, qpack, qpack_bytes, quant_act, quant_act_columns, status_string, workspace_bytes,
)
