"""Helpers for the GPU parity tests: host<->device copies and the tolerance of
the floating-point outputs (max-abs error <= 5e-3 * max|ref| and relative
Frobenius error <= 1e-3, against the fp64 oracle of the same quantized
weights)."""
import sys

import numpy as np

MAXABS_TOL = 5e-3
FROB_TOL = 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_close(out, ref, what=""):
    out = np.asarray(out)
    o = out.astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert o.shape == ref.shape, (what, o.shape, ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    err = np.abs(o - ref)
    mx = float(np.max(np.abs(ref)))
    maxabs = float(err.max()) / mx if mx > 0 else float(err.max())
    frob = float(np.linalg.norm(o - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"  {what}: max-abs/max|ref| = {maxabs:.3e}, rel-Frobenius = {frob:.3e}")
    assert maxabs <= MAXABS_TOL, f"{what}: max-abs {maxabs:.3e} > {MAXABS_TOL}"
    assert frob <= FROB_TOL, f"{what}: rel-Frobenius {frob:.3e} > {FROB_TOL}"
    return maxabs, frob


def sample_rows(M, n=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = {0, M - 1, M // 2}
    rows.update(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(rows))
