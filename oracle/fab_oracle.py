"""Plain fp64 CPU oracle for the fused two-matmul block O = f(A.B).C.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
executes this module; only the test suite, the smoke check and the CPU-baseline
leg of the benchmark do.  It shares no code, tables or helpers with the HIP
library.

What it computes (the plain definition, not the tiled algorithm):

* The unit itself: two consecutive matrix products with a function between
  them, O = f(A B) C -- "Memory-efficient tensor parallelism" abstract
  (FITEE 10.1631/FITEE.2400602).
* f = scaled row softmax over the key axis (attention).  Tiling in the style of
  FlashAttention leaves the result unchanged and only avoids storing the score
  matrix -- "Ulysses Sequence Parallelism: training with million-token
  contexts", section "Contexte Technique".  So the oracle materialises every
  score row at full width and normalises it directly.
* Optional causal mask, an index-defined mask on the score matrix --
  "AutoSP: Unlocking Long-Context LLM Training Via Compiler-Based Sequence
  Parallelism", section 2.A (index recomputation).  Reading taken: key j is
  visible to query i iff j <= i, in global indices, since a rank holds the full
  sequence for its heads (Ulysses page, "Contexte Technique"; AutoSP 2.A,
  buffer resizing).  For a slice of the sequence (a key range passed around a
  ring of ranks: Ulysses page, "Analyse") the global positions are
  q_offset + i and k_offset + j, i.e. key j is visible iff
  j <= i + diag with diag = q_offset - k_offset.  A query row that sees no
  key has O = 0 and LSE = -inf.
* Merging two results over disjoint key sets of the same queries:
  LSE = log(e^LSE_a + e^LSE_b), O = e^(LSE_a - LSE) O_a + e^(LSE_b - LSE) O_b,
  which is the softmax over the union (it follows from the definition of the
  softmax as exp(S - LSE)).
* f = GeLU in its erf form, applied elementwise (the MLP block of AutoSP 2.A
  and 2.B).  Phi is the standard normal CDF.
* Backward passes are the derivative of the same definitions; recomputing the
  intermediate instead of storing it (AutoSP 2.B) does not change them.
* The Ulysses exchange layout (pack before and unpack after the all-to-all
  exchanges): plain index copies, and for a head held by several ranks the
  sum of their blocks (see the section below).

Layouts: attention tensors are [batch, seq, heads, dim] ("BSHD"); query head h
uses key/value head h // (Hq // Hkv).  LSE is [batch, Hq, m], natural log.
MLP: A [m, k], Bt [n, k] (B transposed), C [n, p], O [m, p].

All arithmetic is float64.  Callers pass the exact scale value the device
path receives (a float32 value widened exactly).

Parity: pinned by the CPU tests against closed forms, invariants, brute-force
loops, central finite differences and torch's float64 CPU attention/GeLU.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
from scipy.special import erf as _erf

try:  # keep BLAS single-threaded inside the worker pool
    from threadpoolctl import threadpool_limits as _tp_limits
except ImportError:  # pragma: no cover
    _tp_limits = None

_ROW_BLOCK_ELEMS = 1 << 22  # fp64 elements of one materialised score block


def _workers(workers):
    if workers is None:
        return max(1, len(os.sched_getaffinity(0)))
    return max(1, int(workers))


def _run(tasks, workers):
    """Run zero-argument callables, in a pool when workers > 1."""
    workers = _workers(workers)
    if workers == 1 or len(tasks) <= 1:
        return [t() for t in tasks]
    ctx = _tp_limits(limits=1) if _tp_limits is not None else None
    if ctx is not None:
        ctx.__enter__()
    try:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(lambda t: t(), tasks))
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def _blocks(m, n, block_rows):
    if block_rows is None:
        block_rows = max(1, _ROW_BLOCK_ELEMS // max(1, n))
    return [(r, min(m, r + block_rows)) for r in range(0, m, block_rows)]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _kv_of(h, hq, hkv):
    if hq % hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return h // (hq // hkv)


# ---------------------------------------------------------------------------
# softmax attention
# ---------------------------------------------------------------------------

def attention_probs(qh, kh, scale, causal, rows, diag=0):
    """Full-width probability rows P[rows, :] for one (batch, head).

    qh: [|rows|, d] query rows; kh: [n, d] keys; rows: query indices; causal:
    key j visible iff j <= row + diag.  Returns (P, M, Z): P_ij =
    exp(S_ij - M_i) / Z_i with S = scale * q k^T, M_i = max_j S_ij and
    Z_i = sum_j exp(S_ij - M_i).  A row with no visible key has P = 0,
    M = 0, Z = 0 (so M + log Z = -inf).
    """
    s = float(scale) * (qh @ kh.T)
    if causal:
        cols = np.arange(kh.shape[0])
        s[cols[None, :] > np.asarray(rows)[:, None] + int(diag)] = -np.inf
    mx = s.max(axis=1)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.exp(s - mx[:, None])
    z = e.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(z[:, None] > 0, e / np.where(z > 0, z, 1.0)[:, None], 0.0)
    return p, mx, z


def _lse(mx, z):
    with np.errstate(divide="ignore"):
        return mx + np.log(z)


def _attn_fwd_block(q, k, v, scale, causal, b, h, hkv, r0, r1, o, lse, diag=0):
    g = _kv_of(h, q.shape[2], hkv)
    rows = np.arange(r0, r1)
    p, mx, z = attention_probs(q[b, r0:r1, h], k[b, :, g], scale, causal, rows, diag)
    o[b, r0:r1, h] = p @ v[b, :, g]
    lse[b, h, r0:r1] = _lse(mx, z)


def attention_forward(q, k, v, scale, causal=False, workers=None, block_rows=None,
                      q_offset=0, k_offset=0):
    """O = softmax(scale * Q K^T [+ causal mask]) V and LSE, per (batch, head).

    q [b, m, Hq, d], k [b, n, Hkv, d], v [b, n, Hkv, dv] -> (o [b, m, Hq, dv],
    lse [b, Hq, m]).  Causal positions: query i at q_offset + i, key j at
    k_offset + j.
    """
    diag = int(q_offset) - int(k_offset)
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, m, hq, _ = q.shape
    hkv = k.shape[2]
    o = np.empty((b, m, hq, v.shape[3]))
    lse = np.empty((b, hq, m))
    tasks = []
    for bi in range(b):
        for h in range(hq):
            for r0, r1 in _blocks(m, k.shape[1], block_rows):
                tasks.append(lambda bi=bi, h=h, r0=r0, r1=r1: _attn_fwd_block(
                    q, k, v, scale, causal, bi, h, hkv, r0, r1, o, lse, diag))
    _run(tasks, workers)
    return o, lse


def attention_forward_rows(q, k, v, scale, causal, b, h, rows):
    """O and LSE for selected query rows of one (batch, query head)."""
    rows = np.asarray(rows, dtype=np.int64)
    g = _kv_of(h, q.shape[2], k.shape[2])
    qh = _f64(q[b, rows, h])
    p, mx, z = attention_probs(qh, _f64(k[b, :, g]), scale, causal, rows)
    return p @ _f64(v[b, :, g]), _lse(mx, z)


def _attn_bwd_rows(qh, kh, vh, doh, scale, causal, rows, diag=0):
    """Gradient pieces for a set of full query rows of one head.

    dP = dO V^T; D_i = sum_j P_ij dP_ij; dS = P * (dP - D);
    dQ = scale dS K; dK = scale dS^T Q; dV = P^T dO.
    """
    p, _, _ = attention_probs(qh, kh, scale, causal, rows, diag)
    dp = doh @ vh.T
    dd = (p * dp).sum(axis=1)
    ds = p * (dp - dd[:, None])
    dq = float(scale) * (ds @ kh)
    dk = float(scale) * (ds.T @ qh)
    dv = p.T @ doh
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal=False, workers=None, block_rows=None,
                       q_offset=0, k_offset=0):
    """(dQ, dK, dV) of L = <dO, O> for O = attention_forward(q, k, v) (same
    causal positions)."""
    diag = int(q_offset) - int(k_offset)
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b, m, hq, _ = q.shape
    n, hkv = k.shape[1], k.shape[2]
    dq = np.empty_like(q)
    parts = []

    def task(bi, h, r0, r1):
        g = _kv_of(h, hq, hkv)
        dqb, dkb, dvb = _attn_bwd_rows(q[bi, r0:r1, h], k[bi, :, g], v[bi, :, g],
                                       do[bi, r0:r1, h], scale, causal,
                                       np.arange(r0, r1), diag)
        dq[bi, r0:r1, h] = dqb
        return bi, g, dkb, dvb

    tasks = []
    for bi in range(b):
        for h in range(hq):
            for r0, r1 in _blocks(m, n, block_rows):
                tasks.append(lambda bi=bi, h=h, r0=r0, r1=r1: task(bi, h, r0, r1))
    parts = _run(tasks, workers)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi, g, dkb, dvb in parts:
        dk[bi, :, g] += dkb
        dv[bi, :, g] += dvb
    return dq, dk, dv


def attention_backward_rows(q, k, v, do, scale, causal, b, h, rows):
    """dQ for selected query rows of one (batch, query head)."""
    rows = np.asarray(rows, dtype=np.int64)
    g = _kv_of(h, q.shape[2], k.shape[2])
    dq, _, _ = _attn_bwd_rows(_f64(q[b, rows, h]), _f64(k[b, :, g]), _f64(v[b, :, g]),
                              _f64(do[b, rows, h]), scale, causal, rows)
    return dq


def attention_backward_keys(q, k, v, do, scale, causal, b, g, keys, block_rows=None):
    """dK and dV for selected key rows of one (batch, key/value head).

    Sums over every query head of the group and every query row that can see
    the keys (all rows, or rows i >= min(keys) under the causal mask).
    """
    keys = np.asarray(keys, dtype=np.int64)
    b_, m, hq, _ = q.shape
    hkv = k.shape[2]
    grp = hq // hkv
    kh, vh = _f64(k[b, :, g]), _f64(v[b, :, g])
    dk = np.zeros((len(keys), k.shape[3]))
    dv = np.zeros((len(keys), v.shape[3]))
    first = int(keys.min()) if causal else 0
    for h in range(g * grp, (g + 1) * grp):
        for r0, r1 in _blocks(m - first, k.shape[1], block_rows):
            rows = np.arange(first + r0, first + r1)
            qh, doh = _f64(q[b, rows, h]), _f64(do[b, rows, h])
            p, _, _ = attention_probs(qh, kh, scale, causal, rows)
            dp = doh @ vh.T
            dd = (p * dp).sum(axis=1)
            ds = p[:, keys] * (dp[:, keys] - dd[:, None])
            dk += float(scale) * (ds.T @ qh)
            dv += p[:, keys].T @ doh
    return dk, dv


def attention_merge(o_a, lse_a, o_b, lse_b):
    """Softmax result over the union of two disjoint key sets from the two
    parts' results: LSE = log(e^LSE_a + e^LSE_b), O = sum_x e^(LSE_x - LSE) O_x.
    o_* [b, m, Hq, dv], lse_* [b, Hq, m]; rows with both LSE = -inf give O = 0,
    LSE = -inf."""
    o_a, o_b, lse_a, lse_b = _f64(o_a), _f64(o_b), _f64(lse_a), _f64(lse_b)
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = np.logaddexp(lse_a, lse_b)
        wa = np.where(np.isfinite(lse), np.exp(lse_a - lse), 0.0)
        wb = np.where(np.isfinite(lse), np.exp(lse_b - lse), 0.0)
    # weights [b, Hq, m] -> [b, m, Hq, 1]
    wa, wb = wa.transpose(0, 2, 1)[..., None], wb.transpose(0, 2, 1)[..., None]
    return wa * o_a + wb * o_b, lse


# ---------------------------------------------------------------------------
# GeLU MLP
# ---------------------------------------------------------------------------

def gelu(x):
    """GeLU, erf form: x * Phi(x) with Phi(x) = (1 + erf(x / sqrt 2)) / 2."""
    x = _f64(x)
    return x * 0.5 * (1.0 + _erf(x / math.sqrt(2.0)))


def gelu_grad(x):
    """d/dx GeLU = Phi(x) + x * phi(x), phi(x) = exp(-x^2 / 2) / sqrt(2 pi)."""
    x = _f64(x)
    cdf = 0.5 * (1.0 + _erf(x / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return cdf + x * pdf


def mlp_forward(a, bt, c, scale=1.0, workers=None, block_rows=None):
    """O = GeLU(scale * A Bt^T) C for A [m, k], Bt [n, k], C [n, p]."""
    a, bt, c = _f64(a), _f64(bt), _f64(c)
    m, n = a.shape[0], bt.shape[0]
    o = np.empty((m, c.shape[1]))

    def task(r0, r1):
        o[r0:r1] = gelu(float(scale) * (a[r0:r1] @ bt.T)) @ c

    _run([lambda r0=r0, r1=r1: task(r0, r1) for r0, r1 in _blocks(m, n, block_rows)],
         workers)
    return o


def mlp_forward_rows(a, bt, c, scale, rows):
    """Selected rows of O = GeLU(scale * A Bt^T) C."""
    rows = np.asarray(rows, dtype=np.int64)
    return gelu(float(scale) * (_f64(a[rows]) @ _f64(bt).T)) @ _f64(c)


def mlp_backward(a, bt, c, do, scale=1.0, workers=None, block_rows=None):
    """(dA, dBt, dC) of L = <dO, O> for O = GeLU(scale * A Bt^T) C.

    H = scale A Bt^T; dG = dO C^T; dH = dG * GeLU'(H);
    dA = scale dH Bt; dBt = scale dH^T A; dC = GeLU(H)^T dO.
    """
    a, bt, c, do = _f64(a), _f64(bt), _f64(c), _f64(do)
    m, n = a.shape[0], bt.shape[0]
    da = np.empty_like(a)

    def task(r0, r1):
        hh = float(scale) * (a[r0:r1] @ bt.T)
        dh = (do[r0:r1] @ c.T) * gelu_grad(hh)
        da[r0:r1] = float(scale) * (dh @ bt)
        return float(scale) * (dh.T @ a[r0:r1]), gelu(hh).T @ do[r0:r1]

    parts = _run([lambda r0=r0, r1=r1: task(r0, r1)
                  for r0, r1 in _blocks(m, n, block_rows)], workers)
    dbt = np.zeros_like(bt)
    dc = np.zeros_like(c)
    for dbt_p, dc_p in parts:
        dbt += dbt_p
        dc += dc_p
    return da, dbt, dc


# ---------------------------------------------------------------------------
# brute-force scalar loops (tiny shapes only)
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# Ulysses sequence parallelism: the exchange layout
# ---------------------------------------------------------------------------
# "Ulysses Sequence Parallelism", sections "Contexte Technique" and "Analyse":
# the sequence is split into p chunks, one per rank; an all-to-all then gives
# every rank all positions for a subset of the heads, and a second all-to-all
# after attention returns to the sequence split ("AutoSP" section 2 inserts
# these exchanges at the attention boundaries).  Readings taken: rank j owns
# tokens j n_local .. j n_local + n_local - 1 and heads
# floor(j H / p) .. floor(j H / p) + Hl - 1 with Hl = H / p when p divides H;
# when H < p (grouped-query key/value heads) a head goes to the p / H ranks
# whose query heads read it, and the gradients those ranks return for it are
# summed.  One rank's exchange buffer is [p, n_local, b, Hl, d]: block j goes
# to (or came from) rank j.


def ulysses_heads_per_rank(heads, ranks):
    """Hl, the heads each rank holds after the exchange."""
    if heads % ranks and ranks % heads:
        raise ValueError(f"heads {heads} and ranks {ranks}: one must divide the other")
    return heads // ranks if heads >= ranks else 1


def ulysses_pack(x, ranks):
    """Send buffer [p, n_local, b, Hl, d] of one rank whose tokens are
    x [b, n_local, H, d]: block j holds, for every local token, the heads
    rank j computes attention for."""
    b, nl, heads, d = x.shape
    hl = ulysses_heads_per_rank(heads, ranks)
    out = np.empty((ranks, nl, b, hl, d), dtype=x.dtype)
    for j in range(ranks):
        h0 = (j * heads) // ranks
        out[j] = np.transpose(x[:, :, h0:h0 + hl, :], (1, 0, 2, 3))
    return out


def all_to_all(sends):
    """The exchange itself (equal splits): sends[s][j] goes to rank j, and
    rank j's receive buffer holds, as block s, what rank s sent it."""
    p = len(sends)
    return [np.stack([sends[s][j] for s in range(p)]) for j in range(p)]


def ulysses_unpack(recv, heads):
    """x [b, n_local, H, d] (float64) from a receive buffer [p, n_local, b,
    Hl, d] of the return exchange: block j carries rank j's result for its
    heads; heads held by several ranks get the sum of their blocks."""
    p, nl, b, hl, d = recv.shape
    if ulysses_heads_per_rank(heads, p) != hl:
        raise ValueError("buffer does not match heads / ranks")
    out = np.zeros((b, nl, heads, d), dtype=np.float64)
    for j in range(p):
        h0 = (j * heads) // p
        out[:, :, h0:h0 + hl, :] += np.transpose(_f64(recv[j]), (1, 0, 2, 3))
    return out


def ulysses_sequence_view(recv):
    """A receive buffer of the first exchange read as [b, n, Hl, d]: block s
    holds tokens s n_local .. s n_local + n_local - 1."""
    p, nl, b, hl, d = recv.shape
    return np.transpose(recv.reshape(p * nl, b, hl, d), (1, 0, 2, 3))


def brute_attention_forward(q, k, v, scale, causal=False, q_offset=0, k_offset=0):
    """Scalar-loop attention with math.exp; same layouts as attention_forward."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, m, hq, d = q.shape
    n, hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    o = np.zeros((b, m, hq, dv))
    lse = np.zeros((b, hq, m))
    for bi in range(b):
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(m):
                keys = [j for j in range(n) if not (causal and k_offset + j > q_offset + i)]
                if not keys:  # no visible key: O = 0, LSE = -inf
                    lse[bi, h, i] = -math.inf
                    continue
                s = {}
                for j in keys:
                    acc = 0.0
                    for t in range(d):
                        acc += q[bi, i, h, t] * k[bi, j, g, t]
                    s[j] = float(scale) * acc
                top = max(s.values())
                w = {j: math.exp(s[j] - top) for j in keys}
                z = sum(w.values())
                for c in range(dv):
                    o[bi, i, h, c] = sum(w[j] * v[bi, j, g, c] for j in keys) / z
                lse[bi, h, i] = top + math.log(z)
    return o, lse


def brute_attention_backward(q, k, v, do, scale, causal=False, q_offset=0, k_offset=0):
    """Scalar-loop gradients of <dO, O> by the chain rule through softmax."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b, m, hq, d = q.shape
    n, hkv, dvd = k.shape[1], k.shape[2], v.shape[3]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for bi in range(b):
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(m):
                keys = [j for j in range(n) if not (causal and k_offset + j > q_offset + i)]
                if not keys:  # the row sees no key: no gradient flows through it
                    continue
                s = {j: float(scale) * sum(q[bi, i, h, t] * k[bi, j, g, t]
                                           for t in range(d)) for j in keys}
                top = max(s.values())
                z = sum(math.exp(s[j] - top) for j in keys)
                p = {j: math.exp(s[j] - top) / z for j in keys}
                # dL/dP_ij = sum_c dO_ic V_jc ; softmax Jacobian gives dS
                gp = {j: sum(do[bi, i, h, c] * v[bi, j, g, c] for c in range(dvd))
                      for j in keys}
                mean = sum(p[j] * gp[j] for j in keys)
                for j in keys:
                    ds = p[j] * (gp[j] - mean)
                    for t in range(d):
                        dq[bi, i, h, t] += float(scale) * ds * k[bi, j, g, t]
                        dk[bi, j, g, t] += float(scale) * ds * q[bi, i, h, t]
                    for c in range(dvd):
                        dv[bi, j, g, c] += p[j] * do[bi, i, h, c]
    return dq, dk, dv


def brute_mlp_forward(a, bt, c, scale=1.0):
    """Scalar-loop GeLU MLP with math.erf."""
    a, bt, c = _f64(a), _f64(bt), _f64(c)
    m, kk = a.shape
    n, p = bt.shape[0], c.shape[1]
    o = np.zeros((m, p))
    for i in range(m):
        for j in range(n):
            hv = float(scale) * sum(a[i, t] * bt[j, t] for t in range(kk))
            gv = hv * 0.5 * (1.0 + math.erf(hv / math.sqrt(2.0)))
            for c_ in range(p):
                o[i, c_] += gv * c[j, c_]
    return o
