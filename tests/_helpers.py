"""Shared helpers for the parity tests (not a test module)."""

import numpy as np
import torch

# Tolerances for the bf16 output of the linear against the unrounded float64 oracle:
# elementwise |gpu - ref| <= ELEM_TOL * (|ref| + 1) and relative Frobenius error
# <= FRO_TOL. The bf16 rounding of the output alone costs about 1.7e-3 relative
# Frobenius, so these bounds leave room for fp32 accumulation and epilogue
# rounding only, not for a second low-precision rounding.
ELEM_TOL = 1e-2
FRO_TOL = 2e-3


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("this test needs a gfx950 GPU: the HIP library is the only implementation")
    return torch.device("cuda", 0)


def bf16_out_to_f64(t):
    return t.detach().float().cpu().double().numpy()


def linear_errors(gpu_f64, ref):
    diff = np.abs(gpu_f64 - ref)
    elem = float(np.max(diff / (np.abs(ref) + 1.0))) if ref.size else 0.0
    den = float(np.linalg.norm(ref))
    fro = float(np.linalg.norm(gpu_f64 - ref) / den) if den > 0 else float(np.linalg.norm(gpu_f64 - ref))
    return elem, fro


def assert_linear_close(gpu_out, ref, label=""):
    got = bf16_out_to_f64(gpu_out) if isinstance(gpu_out, torch.Tensor) else gpu_out
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    elem, fro = linear_errors(got, ref)
    assert elem <= ELEM_TOL, f"{label}: max |gpu-ref|/(|ref|+1) = {elem:.3e} > {ELEM_TOL}"
    assert fro <= FRO_TOL, f"{label}: relative Frobenius error {fro:.3e} > {FRO_TOL}"
    return elem, fro


def sample_rows(m, tile=256, count=192, seed=0):
    """Rows to check at full size: the first tile's rows, the ragged last tile, and random ones."""
    rng = np.random.default_rng(seed)
    head = np.arange(min(m, 32))
    last_tile = (m - 1) // tile * tile
    tail = np.arange(max(0, min(last_tile, m - 48)), m)
    rand = rng.choice(m, size=min(m, count), replace=False)
    return np.unique(np.concatenate([head, tail, rand]))
