"""Helpers shared by the GPU tests: run the library, run the oracle, compare."""
import os

import numpy as np
import torch

import newton_schulz_04_amd as ns
from oracle import oracle

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def coeffs32(c=ns.QUINTIC):
    return tuple(float(np.float32(v)) for v in c)


def gpu_run(mats, steps=5, coeffs=ns.QUINTIC, device="cuda"):
    """Copy CPU matrices to the GPU, orthogonalize them in one batched call,
    return CPU copies of the results."""
    dev = [m.to(device).contiguous() for m in mats]
    ns.orthogonalize(dev, steps=steps, coeffs=coeffs)
    torch.cuda.synchronize()
    return [d.cpu() for d in dev]


def oracle_run(mat, steps=5, coeffs=ns.QUINTIC):
    return oracle.newton_schulz(mat.float().numpy(), steps=steps, coeffs=coeffs32(coeffs))


def rel_err(y, ref, rows=None):
    y = y.float().numpy().astype(np.float64) if isinstance(y, torch.Tensor) else np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if rows is not None:
        y, ref = y[rows], ref[rows]
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def zero_bits(t):
    """True when every element is +0.0 (bit pattern all zero)."""
    t = t.contiguous()
    if t.numel() == 0:
        return True
    iv = t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    return not bool(iv.any())


def load_golden(name):
    path = os.path.join(GOLDEN, f"oracle_{name}.npz")
    if not os.path.exists(path):
        return None
    return np.load(path, allow_pickle=False)


def check_against_golden(y, g, tol=2e-2):
    """Compare a full-size result with the stored oracle sample.

    Band samples (one stored row per 256-row band and one stored column per
    256-column band, so every 256 x 256 output tile has a stored row and a
    stored column through it): each stored row and each stored column on its
    own, element by element, relative Frobenius error <= tol, and the whole
    row and column sets likewise. Older samples hold a few rows only. The +-1
    sketch checks the whole matrix (E ||dY w||^2 = ||dY||_F^2 for w with
    independent +-1 entries), and the norm."""
    yf = y.float().numpy().astype(np.float64)
    rows = g["rows_idx"]
    ref_rows = g["rows"].astype(np.float64)
    got_rows = yf[rows]
    e_rows = np.linalg.norm(got_rows - ref_rows) / np.linalg.norm(ref_rows)
    worst = 0.0
    for k in range(len(rows)):
        nr = np.linalg.norm(ref_rows[k])
        if nr > 0:
            ek = np.linalg.norm(got_rows[k] - ref_rows[k]) / nr
            assert ek <= tol, f"row {int(rows[k])}: rel err {ek:.3e}"
            worst = max(worst, ek)
    if "cols_idx" in g.files:
        cols = g["cols_idx"]
        ref_cols = g["cols"].astype(np.float64)
        got_cols = yf[:, cols]
        e_cols = np.linalg.norm(got_cols - ref_cols) / np.linalg.norm(ref_cols)
        assert e_cols <= tol, f"sampled columns rel err {e_cols:.3e}"
        for k in range(len(cols)):
            nc = np.linalg.norm(ref_cols[:, k])
            if nc > 0:
                ek = np.linalg.norm(got_cols[:, k] - ref_cols[:, k]) / nc
                assert ek <= tol, f"column {int(cols[k])}: rel err {ek:.3e}"
                worst = max(worst, ek)
    om = g["omega"].astype(np.float64)
    sk = yf @ om
    e_sketch = np.linalg.norm(sk - g["sketch"]) / np.linalg.norm(g["sketch"])
    e_fro = abs(np.linalg.norm(yf) - float(g["fro"])) / float(g["fro"])
    assert e_rows <= tol, f"sampled rows rel err {e_rows:.3e}"
    assert e_sketch <= tol, f"sketch rel err {e_sketch:.3e}"
    assert e_fro <= tol, f"norm rel err {e_fro:.3e}"
    return e_rows, e_sketch, e_fro, worst
