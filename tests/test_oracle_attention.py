"""Pins for the softmax-attention half of the oracle (CPU only).

Each check ties the oracle to something other than itself: a hand-worked
example, closed forms, invariants of softmax, scalar brute-force loops,
central finite differences and torch's float64 CPU attention with autograd.
"""
import math
import os

import numpy as np
import pytest

from oracle import (attention_backward, attention_backward_keys,
                    attention_backward_rows, attention_forward,
                    attention_forward_rows, attention_merge, attention_probs,
                    brute_attention_backward, brute_attention_forward)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def qkv(seed, b=1, m=9, n=9, hq=2, hkv=1, d=5, dv=None):
    dv = d if dv is None else dv
    return (rnd(seed, b, m, hq, d), rnd(seed + 1, b, n, hkv, d),
            rnd(seed + 2, b, n, hkv, dv), rnd(seed + 3, b, m, hq, dv))


def test_hand_worked_two_keys():
    rows = {}
    with open(os.path.join(GOLDEN, "attention_two_keys.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                name, *vals = line.split()
                rows[name] = [float(x) for x in vals]
    q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    k = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 2, 1, 2)
    v = np.array([[1.0, 2.0], [3.0, -1.0]]).reshape(1, 2, 1, 2)
    for case, causal in (("full", False), ("causal", True)):
        o, lse = attention_forward(q, k, v, 1.0, causal)
        np.testing.assert_allclose(o[0, 0, 0], rows[case][:2], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[0, 0, 0], rows[case][2], rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k, _, _ = qkv(1, m=33, n=33, hq=1, d=7)
    p, _, _ = attention_probs(q[0, :, 0], k[0, :, 0], 0.3, causal, np.arange(33))
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
    if causal:
        assert np.all(np.triu(p, 1) == 0)


@pytest.mark.parametrize("causal", [False, True])
def test_value_ones_gives_ones(causal):
    q, k, _, _ = qkv(2, m=17, n=17, hq=4, hkv=2, d=6)
    v = np.ones((1, 17, 2, 3))
    o, _ = attention_forward(q * 3.0, k, v, 0.7, causal)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)


def test_zero_scores_average_values():
    _, k, v, _ = qkv(3, m=11, n=11, hq=1, d=4)
    q = np.zeros((1, 11, 1, 4))
    o, lse = attention_forward(q, k, v, 0.5, False)
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v[0, :, 0].mean(axis=0), (11, 4)),
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(11), rtol=0, atol=1e-14)
    o, lse = attention_forward(q, k, v, 0.5, True)
    prefix = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, 12)[:, None]
    np.testing.assert_allclose(o[0, :, 0], prefix, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(np.arange(1, 12)), rtol=0, atol=1e-14)


def test_causal_first_row():
    q, k, v, _ = qkv(4, m=13, n=13, hq=3, hkv=3, d=8)
    scale = 0.37
    o, lse = attention_forward(q, k, v, scale, True)
    for h in range(3):
        np.testing.assert_allclose(o[0, 0, h], v[0, 0, h], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[0, h, 0], scale * q[0, 0, h] @ k[0, 0, h],
                                   rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    q, k, v, _ = qkv(5, m=10, n=10, hq=2, hkv=1, d=6)
    u = rnd(99, 6)
    scale = 0.4
    o0, l0 = attention_forward(q, k, v, scale, causal)
    o1, l1 = attention_forward(q, k + u, v, scale, causal)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    shift = scale * np.einsum("bmhd,d->bhm", q, u)
    np.testing.assert_allclose(l1, l0 + shift, rtol=0, atol=1e-12)


def test_large_scores_pick_argmax_value():
    q, k, v, _ = qkv(6, m=8, n=12, hq=1, d=5)
    o, lse = attention_forward(q * 1e3, k, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    best = np.argmax(q[0, :, 0] @ k[0, :, 0].T, axis=1)
    np.testing.assert_allclose(o[0, :, 0], v[0, best, 0], rtol=0, atol=1e-9)


def test_key_permutation_invariance():
    q, k, v, _ = qkv(7, m=9, n=14, hq=2, hkv=2, d=4)
    perm = np.random.default_rng(0).permutation(14)
    o0, l0 = attention_forward(q, k, v, 0.8, False)
    o1, l1 = attention_forward(q, k[:, perm], v[:, perm], 0.8, False)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2), (3, 1)])
def test_brute_force_forward_and_backward(causal, hq, hkv):
    q, k, v, do = qkv(8, b=2, m=5, n=5, hq=hq, hkv=hkv, d=3, dv=4)
    scale = 0.6
    o, lse = attention_forward(q, k, v, scale, causal)
    ob, lb = brute_attention_forward(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)
    grads = attention_backward(q, k, v, do, scale, causal)
    brute = brute_attention_backward(q, k, v, do, scale, causal)
    for g, gb in zip(grads, brute):
        np.testing.assert_allclose(g, gb, rtol=0, atol=1e-12)


def _torch_reference(q, k, v, do, scale, causal):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    hq, hkv = q.shape[2], k.shape[2]
    tq = torch.tensor(q).permute(0, 2, 1, 3).requires_grad_(True)
    tk = torch.tensor(k).permute(0, 2, 1, 3).requires_grad_(True)
    tv = torch.tensor(v).permute(0, 2, 1, 3).requires_grad_(True)
    kk = tk.repeat_interleave(hq // hkv, dim=1)
    vv = tv.repeat_interleave(hq // hkv, dim=1)
    o = F.scaled_dot_product_attention(tq, kk, vv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do).permute(0, 2, 1, 3))
    back = lambda t: t.permute(0, 2, 1, 3).detach().numpy()
    return back(o), back(tq.grad), back(tk.grad), back(tv.grad)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1), (6, 2)])
def test_against_torch_float64(causal, hq, hkv):
    q, k, v, do = qkv(9, b=2, m=37, n=37, hq=hq, hkv=hkv, d=16)
    scale = 0.25
    o, _ = attention_forward(q, k, v, scale, causal, block_rows=8)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal, block_rows=8)
    to, tdq, tdk, tdv = _torch_reference(q, k, v, do, scale, causal)
    for a, b in ((o, to), (dq, tdq), (dk, tdk), (dv, tdv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    q, k, v, do = qkv(10, m=6, n=6, hq=2, hkv=1, d=3)
    scale = 0.9
    grads = attention_backward(q, k, v, do, scale, causal)
    h = 1e-6

    def loss(q_, k_, v_):
        return float(np.sum(attention_forward(q_, k_, v_, scale, causal)[0] * do))

    rng = np.random.default_rng(1)
    for which, g in enumerate(grads):
        base = [q, k, v]
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in base[which].shape)
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (loss(*plus) - loss(*minus)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (which, idx, fd, g[idx])


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(causal):
    q, k, v, do = qkv(11, b=1, m=40, n=40, hq=4, hkv=2, d=8)
    scale = 0.3
    o, _ = attention_forward(q, k, v, scale, causal)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    grp = 2
    for g in range(2):
        heads = slice(g * grp, (g + 1) * grp)
        # P rows sum to one -> column sums of dV equal summed dO over the group
        np.testing.assert_allclose(dv[0, :, g].sum(axis=0), do[0, :, heads].sum(axis=(0, 1)),
                                   rtol=0, atol=1e-11)
        # dS rows sum to zero -> dK sums to zero
        np.testing.assert_allclose(dk[0, :, g].sum(axis=0), 0.0, rtol=0, atol=1e-11)
    # O is linear in V
    np.testing.assert_allclose(np.sum(dv * v), np.sum(do * o), rtol=1e-12)
    # invariance under Q -> a Q, K -> K / a
    np.testing.assert_allclose(np.sum(dq * q), np.sum(dk * k), rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("causal", [False, True])
def test_row_and_key_helpers_match_full(causal):
    q, k, v, do = qkv(12, b=2, m=50, n=50, hq=4, hkv=2, d=8)
    scale = 0.35
    o, lse = attention_forward(q, k, v, scale, causal)
    dq, dk, dv = attention_backward(q, k, v, do, scale, causal)
    rows = np.array([0, 7, 31, 49])
    for b in range(2):
        for h in range(4):
            orow, lrow = attention_forward_rows(q, k, v, scale, causal, b, h, rows)
            np.testing.assert_allclose(orow, o[b, rows, h], rtol=0, atol=1e-13)
            np.testing.assert_allclose(lrow, lse[b, h, rows], rtol=0, atol=1e-13)
            dqr = attention_backward_rows(q, k, v, do, scale, causal, b, h, rows)
            np.testing.assert_allclose(dqr, dq[b, rows, h], rtol=0, atol=1e-12)
        for g in range(2):
            keys = np.array([3, 40, 48, 49])
            dkk, dvk = attention_backward_keys(q, k, v, do, scale, causal, b, g, keys,
                                               block_rows=7)
            np.testing.assert_allclose(dkk, dk[b, keys, g], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dvk, dv[b, keys, g], rtol=0, atol=1e-12)


def test_row_blocks_do_not_change_result():
    q, k, v, do = qkv(13, b=1, m=70, n=70, hq=2, hkv=1, d=4)
    a = attention_forward(q, k, v, 0.5, True, block_rows=70, workers=1)
    b = attention_forward(q, k, v, 0.5, True, block_rows=3, workers=4)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-14)
    ga = attention_backward(q, k, v, do, 0.5, True, block_rows=70, workers=1)
    gb = attention_backward(q, k, v, do, 0.5, True, block_rows=5, workers=3)
    for x, y in zip(ga, gb):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# causal positions for a slice of the sequence (q_offset / k_offset) and the
# merge of results over disjoint key sets
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("q_offset,k_offset", [(0, 0), (7, 3), (3, 7), (0, 5), (100, 0),
                                               (0, 100)])
def test_offset_mask_brute_force(q_offset, k_offset):
    q, k, v, do = qkv(21, b=1, m=6, n=5, hq=2, hkv=1, d=3, dv=4)
    scale = 0.7
    o, lse = attention_forward(q, k, v, scale, True, q_offset=q_offset, k_offset=k_offset)
    ob, lb = brute_attention_forward(q, k, v, scale, True, q_offset, k_offset)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
    grads = attention_backward(q, k, v, do, scale, True, q_offset=q_offset, k_offset=k_offset)
    brute = brute_attention_backward(q, k, v, do, scale, True, q_offset, k_offset)
    for g, gb in zip(grads, brute):
        np.testing.assert_allclose(g, gb, rtol=0, atol=1e-12)


def test_offset_mask_against_torch_explicit_mask():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v, do = qkv(22, b=1, m=11, n=17, hq=2, hkv=2, d=8)
    scale, q_offset, k_offset = 0.3, 9, 2  # every row sees >= 8 keys
    o, lse = attention_forward(q, k, v, scale, True, q_offset=q_offset, k_offset=k_offset)
    allow = (k_offset + np.arange(17))[None, :] <= (q_offset + np.arange(11))[:, None]
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3) for x in (q, k, v))
    to = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(allow), scale=scale)
    np.testing.assert_allclose(o, to.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-12)


def test_offset_limits():
    q, k, v, _ = qkv(23, b=1, m=6, n=8, hq=1, hkv=1, d=4)
    full, lf = attention_forward(q, k, v, 0.5, False)
    # every row sees every key once q_offset - k_offset >= n - 1
    o, lse = attention_forward(q, k, v, 0.5, True, q_offset=7, k_offset=0)
    np.testing.assert_allclose(o, full, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lf, rtol=0, atol=1e-14)
    # no row sees a key once q_offset + m - 1 < k_offset
    o, lse = attention_forward(q, k, v, 0.5, True, q_offset=0, k_offset=6)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(5,), (3, 8), (1, 2, 11)])
def test_key_split_merge_equals_full(causal, cuts):
    """Splitting the keys into ranges (each placed by its k_offset), then merging
    the per-range results pairwise in any order, gives the full result."""
    q, k, v, _ = qkv(24, b=2, m=12, n=12, hq=4, hkv=2, d=6)
    scale = 0.45
    full, lf = attention_forward(q, k, v, scale, causal)
    bounds = [0, *cuts, 12]
    parts = [attention_forward(q, k[:, a:b], v[:, a:b], scale, causal, q_offset=0, k_offset=a)
             for a, b in zip(bounds[:-1], bounds[1:])]
    o, lse = parts[-1]
    for po, pl in reversed(parts[:-1]):  # right to left
        o, lse = attention_merge(po, pl, o, lse)
    np.testing.assert_allclose(o, full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lf, rtol=0, atol=1e-13)


def test_merge_closed_form_and_empty_rows():
    # a 2-key softmax split into two 1-key parts: O_x = V_x, LSE_x = S_x
    o_a = np.full((1, 1, 1, 2), 3.0)
    o_b = np.full((1, 1, 1, 2), -1.0)
    la, lb = np.array([[[0.25]]]), np.array([[[1.0]]])
    o, lse = attention_merge(o_a, la, o_b, lb)
    pa = math.exp(0.25) / (math.exp(0.25) + math.exp(1.0))
    np.testing.assert_allclose(o[0, 0, 0], [3 * pa - (1 - pa)] * 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, math.log(math.exp(0.25) + math.exp(1.0)), rtol=0, atol=1e-15)
    # an empty part leaves the other unchanged; two empty parts give O = 0, -inf
    o, lse = attention_merge(o_a, la, np.zeros_like(o_b), np.array([[[-np.inf]]]))
    np.testing.assert_array_equal(o, o_a)
    np.testing.assert_array_equal(lse, la)
    o, lse = attention_merge(np.zeros_like(o_a), np.array([[[-np.inf]]]), np.zeros_like(o_b),
                             np.array([[[-np.inf]]]))
    assert np.all(o == 0) and np.isneginf(lse).all()
