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


def assert_linear_close_rows(out_gpu, ref_rows, label="", chunk=4096):
    """Whole-output parity of a GPU output [m, n] against the oracle, row block by row block.

    ref_rows(r0, r1) returns the oracle's unrounded float64 rows [r0, r1). Every element
    must meet the elementwise bound, and the relative Frobenius error is accumulated over
    the whole [m, n] output (not per block)."""
    m = out_gpu.shape[0]
    worst, num, den = 0.0, 0.0, 0.0
    for r0 in range(0, m, chunk):
        r1 = min(m, r0 + chunk)
        ref = ref_rows(r0, r1)
        got = bf16_out_to_f64(out_gpu[r0:r1])
        assert got.shape == ref.shape, (got.shape, ref.shape)
        assert np.all(np.isfinite(got)), f"{label}: non-finite output in rows {r0}..{r1}"
        diff = got - ref
        worst = max(worst, float(np.max(np.abs(diff) / (np.abs(ref) + 1.0))) if ref.size else 0.0)
        num += float(np.sum(diff * diff))
        den += float(np.sum(ref * ref))
    fro = float(np.sqrt(num) / np.sqrt(den)) if den > 0 else float(np.sqrt(num))
    assert worst <= ELEM_TOL, f"{label}: max |gpu-ref|/(|ref|+1) = {worst:.3e} > {ELEM_TOL}"
    assert fro <= FRO_TOL, f"{label}: relative Frobenius error {fro:.3e} > {FRO_TOL} over the whole output"
    return worst, fro


def assert_codes_equal(q_gpu, s_gpu, eq, es, label=""):
    """Bit-exact comparison of per-row codes [m, k] and scales [m] with the oracle's."""
    q = q_gpu.cpu().numpy() if isinstance(q_gpu, torch.Tensor) else q_gpu
    s = s_gpu.cpu().numpy() if isinstance(s_gpu, torch.Tensor) else s_gpu
    assert np.array_equal(s.view(np.uint32), np.asarray(es, np.float32).view(np.uint32)), f"{label}: scales differ"
    bad = np.argwhere(q != eq)
    assert bad.size == 0, f"{label}: {len(bad)} codes differ, first at {bad[0]}"
