"""Shared helpers for the parity tests: error metrics and device transfer.

Error measure (the reading used throughout): normwise max relative error per
slice, max |g - r| / max |r| over one slice, where a slice is one (batch, head)
pair of a [batch, rows, heads, d] attention tensor and the whole matrix for the
MLP.  Tolerances: 1e-2 for bf16 inputs with fp32 accumulation, 1e-5 for the
fp32 path; the LSE uses absolute error 1e-3 (bf16) and 1e-5 (fp32).

Why per slice and not per row: the backward forms D_i = rowsum(dO_i * O_i) from
the O the forward returned (bf16), so dS = P (dP - D) carries an absolute error
of order 2^-9 |O_i| |dO_i|.  Rows whose dS nearly cancels (in the extreme, the
causal first query's dQ is exactly zero) then have small norms and large
row-relative errors that say nothing about the kernel.  The per-row relative
error is still computed and printed as a diagnostic.  A slice whose reference
is identically zero (e.g. dQ, dK for a single key) is compared in absolute
terms against `zero_scale` times the tolerance.
"""
import numpy as np

TOL = {"bf16": 1e-2, "f32": 1e-5}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}


def _slices(x):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 4:
        b, n, h, d = x.shape
        return x.transpose(0, 2, 1, 3).reshape(b * h, n * d)
    return x.reshape(1, -1)


def slice_rel_err(got, ref, zero_scale=None):
    """max over slices of max|got - ref| / max|ref| (see module docstring)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    g, r = _slices(got), _slices(ref)
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    zero = den == 0
    if zero.any():
        assert zero_scale is not None and zero_scale > 0, "all-zero reference needs zero_scale"
        den = np.where(zero, zero_scale, den)
    return float((num / den).max())


def row_rel_err(got, ref):
    """Diagnostic: max over rows of ||got_i - ref_i||_inf / ||ref_i||_inf
    (rows below 1e-3 of the largest row norm use that floor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    rn = np.abs(r).max(axis=1)
    floor = 1e-3 * max(rn.max(), 1e-300) if rn.size else 1.0
    err = np.abs(g - r).max(axis=1) / np.maximum(rn, floor)
    return float(err.max()) if err.size else 0.0


def to_device(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return t.cuda()


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(name, got, ref, dtype, tol=None, zero_scale=None):
    tol = TOL[dtype] if tol is None else tol
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = slice_rel_err(got, ref, zero_scale)
    rows = row_rel_err(got, ref) if np.size(ref) else 0.0
    print(f"  {name}: max rel err {err:.2e} (per-row diagnostic {rows:.2e})")
    assert err <= tol, f"{name}: max relative error {err:.3e} > {tol:.1e}"
    return err


def assert_lse(got, ref, dtype):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if np.size(ref) else 0.0
    assert err <= LSE_TOL[dtype], f"lse: abs error {err:.3e} > {LSE_TOL[dtype]:.1e}"
    return err
