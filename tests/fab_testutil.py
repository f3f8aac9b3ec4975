"""Shared helpers for the parity tests: error metrics and device transfer.

Error measure (the reading used throughout): per-row normwise relative error
max_i ||g_i - r_i||_inf / ||r_i||_inf over rows (one d-vector per batch, head
and token for attention; one matrix row for the MLP), where rows whose
reference norm is below 1e-3 of the largest row norm are compared against that
floor instead.  The floor exists because some gradient rows vanish by exact
cancellation (the causal first query's dQ: its only score has dS = P (dP - D)
= 0), and rounding noise relative to an exact zero is no error measure.  Tolerances: 1e-2 for bf16 inputs with fp32 accumulation,
1e-5 for the fp32 path.  LSE uses absolute error: 1e-3 (bf16), 1e-5 (fp32).
"""
import numpy as np

TOL = {"bf16": 1e-2, "f32": 1e-5}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}


def row_rel_err(got, ref):
    """max over rows of ||got_i - ref_i||_inf / max(||ref_i||_inf, floor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    rn = np.abs(r).max(axis=1)
    floor = 1e-3 * max(rn.max(), 1e-300)
    err = np.abs(g - r).max(axis=1) / np.maximum(rn, floor)
    return float(err.max()) if err.size else 0.0


def to_device(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return t.cuda()


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(name, got, ref, dtype, tol=None):
    tol = TOL[dtype] if tol is None else tol
    err = row_rel_err(got, ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: row-relative error {err:.3e} > {tol:.1e}"
    return err


def assert_lse(got, ref, dtype):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if np.size(ref) else 0.0
    assert err <= LSE_TOL[dtype], f"lse: abs error {err:.3e} > {LSE_TOL[dtype]:.1e}"
    return err
