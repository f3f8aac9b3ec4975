"""Shared helpers for the parity tests: error gates and device transfer.

The gate ("max relative error" of the benchmark spec's bound, read per row): for
every row i -- one d-vector per (batch, head, token) of an attention tensor,
one matrix row of the MLP --

    ||got_i - ref_i||_inf / max(||ref_i||_inf, floor_i)  <=  tol,

tol = 1e-2 for bf16 inputs with fp32 accumulation and 1e-5 for the fp32 path.
The default floor is 1e-6 of the largest reference row norm of the tensor
(it only matters for rows that are exactly or almost zero).  The LSE is
checked in absolute terms (1e-3 bf16, 1e-5 fp32).

dQ and dK get a floor from the rounding of D.  The backward forms
D_i = rowsum(dO_i * O_i) from the O the forward returned, and
dQ_i = scale (sum_j P_ij dP_ij K_j - D_i (P K)_i),
dK_j = scale sum_i P_ij (dP_ij - D_i) Q_i.
A relative perturbation u of each element of O changes D_i by at most
u w_i with w_i = sum_d |dO_id O_id|, hence dQ_i by at most
u scale w_i ||(P K)_i||_inf and dK_j by at most
u scale ||sum_i P_ij w_i |Q_i| ||_inf (summed over the query heads sharing
the key's head).  Rows whose value nearly cancels between the two terms
cannot be more accurate, relative to their own size, than D itself, so their
error is measured against that D-term magnitude when it exceeds the row norm:

    floor_i(dQ) = scale w_i ||(P K)_i||_inf,
    floor_j(dK) = scale ||sum_{h in group} sum_i P^h_ij w^h_i |Q^h_i| ||_inf.

Both are computed with the oracle (P K is attention with K as the values;
sum_i P_ij x_i is the oracle's dV for dO = x).  The normwise figure over a
whole (batch, head) slice is printed beside the gate as a secondary number.
"""
import numpy as np

TOL = {"bf16": 1e-2, "f32": 1e-5}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}
FLOOR_REL = 1e-6  # default floor: this fraction of the largest reference row norm


def _slices(x):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 4:
        b, n, h, d = x.shape
        return x.transpose(0, 2, 1, 3).reshape(b * h, n * d)
    return x.reshape(1, -1)


def slice_rel_err(got, ref):
    """Secondary figure: max over (batch, head) slices of max|got - ref| /
    max|ref| (whole matrix for 2-d tensors); slices with an all-zero
    reference count their absolute error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    g, r = _slices(got), _slices(ref)
    num = np.abs(g - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def row_errors(got, ref, floor=None):
    """Per-row ||got_i - ref_i||_inf / max(||ref_i||_inf, floor_i) over the
    last axis.  floor: None, a scalar, or an array of the row shape; it is
    raised to at least FLOOR_REL times the largest reference row norm.  A row
    whose reference and floor are both zero must match exactly (error inf
    otherwise)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref).max(axis=-1)
    rn = np.abs(ref).max(axis=-1)
    base = FLOOR_REL * float(rn.max()) if rn.size else 0.0
    fl = np.maximum(base, 0.0 if floor is None else np.asarray(floor, dtype=np.float64))
    den = np.maximum(rn, fl)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(den > 0, err / np.where(den > 0, den, 1.0), np.where(err > 0, np.inf, 0.0))
    return out


def to_device(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    return t.cuda()


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(name, got, ref, dtype, tol=None, floor=None):
    """Per-row gate (module docstring); prints the largest row error, how many
    rows the floor decided, and the per-slice figure."""
    tol = TOL[dtype] if tol is None else tol
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:
        return 0.0
    errs = row_errors(got, ref, floor)
    worst = float(errs.max())
    note = ""
    if floor is not None:
        rn = np.abs(np.asarray(ref, np.float64)).max(axis=-1)
        floored = int(np.sum(np.asarray(floor) > rn))
        plain = float(row_errors(got, ref).max())
        note = (f" ({floored} rows measured against the D-term floor; "
                f"{plain:.2e} against the row norms alone)")
    print(f"  {name}: per-row max rel err {worst:.2e} over {errs.size} rows{note}; "
          f"per-slice {slice_rel_err(got, ref):.2e}")
    if worst > tol:
        idx = np.unravel_index(int(np.argmax(errs)), errs.shape)
        raise AssertionError(f"{name}: row {idx} relative error {worst:.3e} > {tol:.1e}")
    return worst


def assert_lse(got, ref, dtype):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if not np.size(ref):
        return 0.0
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)) and np.all(got[~fin] == ref[~fin]), \
        "lse: infinite entries differ"
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= LSE_TOL[dtype], f"lse: abs error {err:.3e} > {LSE_TOL[dtype]:.1e}"
    return err


def _abs_dot(do, o):
    """w_i = sum_d |dO_id O_id| for every row: [..., d] -> [...]."""
    return np.abs(np.asarray(do, np.float64) * np.asarray(o, np.float64)).sum(axis=-1)


def grad_floors(x, scale, causal, o_ref=None, q_offset=0, k_offset=0):
    """D-term floors (module docstring) for every row of dQ [b, m, hq] and of
    dK [b, n, hkv], from the oracle."""
    import oracle
    if o_ref is None:
        o_ref, _ = oracle.attention_forward(x["q"], x["k"], x["v"], scale, causal,
                                            q_offset=q_offset, k_offset=k_offset)
    w = _abs_dot(x["do"], o_ref)
    pk, _ = oracle.attention_forward(x["q"], x["k"], x["k"], scale, causal,
                                     q_offset=q_offset, k_offset=k_offset)
    fq = scale * w * np.abs(pk).max(axis=-1)
    wq = w[..., None] * np.abs(np.asarray(x["q"], np.float64))
    _, _, pt = oracle.attention_backward(x["q"], x["k"], x["v"], wq, scale, causal,
                                         q_offset=q_offset, k_offset=k_offset)
    fk = scale * np.abs(pt).max(axis=-1)
    return fq, fk


def dq_floor_rows(x, scale, causal, b, h, rows):
    """D-term floor of dQ for selected query rows of one (batch, head)."""
    import oracle
    o, _ = oracle.attention_forward_rows(x["q"], x["k"], x["v"], scale, causal, b, h, rows)
    pk, _ = oracle.attention_forward_rows(x["q"], x["k"], x["k"], scale, causal, b, h, rows)
    w = _abs_dot(np.asarray(x["do"])[b, rows, h], o)
    return scale * w * np.abs(pk).max(axis=-1)


def dk_floor_keys(x, scale, causal, b, g, keys):
    """D-term floor of dK for selected keys of one (batch, kv head); with the
    causal mask only query rows i >= min(keys) enter, so the late keys of a
    long sequence are cheap."""
    import oracle
    q = np.asarray(x["q"])
    m, hq = q.shape[1], q.shape[2]
    grp = hq // np.asarray(x["k"]).shape[2]
    first = int(np.min(keys)) if causal else 0
    rows = np.arange(first, m)
    wq = np.zeros(q.shape, dtype=np.float32)  # rows before `first` never enter
    for h in range(g * grp, (g + 1) * grp):
        o, _ = oracle.attention_forward_rows(x["q"], x["k"], x["v"], scale, causal, b, h, rows)
        w = _abs_dot(np.asarray(x["do"])[b, rows, h], o)
        wq[b, rows, h] = w[:, None] * np.abs(q[b, rows, h])
    _, pt = oracle.attention_backward_keys(x["q"], x["k"], x["v"], wq, scale, causal, b, g, keys)
    return scale * np.abs(pt).max(axis=-1)
