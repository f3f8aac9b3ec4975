"""Pins for the Ulysses exchange layout of the oracle (CPU only).

The layout steps have no formula of their own on the pages; what the pages fix
is what the exchanges achieve ("Ulysses Sequence Parallelism", "Contexte
Technique": after the redistribution each rank holds every position of a
subset of the heads, and attention computed that way is the attention of the
whole sequence).  So the checks are: hand-worked placements, the attention and
its gradients computed rank by rank through pack / exchange / unpack equal the
single-device result, a round trip restores the input, and every element
travels exactly once.
"""
import numpy as np
import pytest

from oracle import (all_to_all, attention_backward, attention_forward,
                    ulysses_heads_per_rank, ulysses_pack,
                    ulysses_sequence_view, ulysses_unpack)


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def shards(x, p):
    nl = x.shape[1] // p
    return [x[:, j * nl:(j + 1) * nl] for j in range(p)]


def to_send(y, p):
    """Per-rank result y [b, n, Hl, d] laid out as the return exchange's
    send buffer [p, n_local, b, Hl, d] (block s = token chunk s)."""
    b, n, hl, d = y.shape
    return np.transpose(y, (1, 0, 2, 3)).reshape(p, n // p, b, hl, d)


def test_hand_worked_two_ranks():
    # b = 1, n = 4 tokens, H = 2 heads, d = 1, p = 2; value = 10 token + head.
    full = np.array([[[[10.0 * t + h] for h in range(2)] for t in range(4)]])
    recv = all_to_all([ulysses_pack(x, 2) for x in shards(full, 2)])
    # rank 0 holds head 0 of all four tokens, rank 1 head 1, in token order
    assert ulysses_sequence_view(recv[0]).ravel().tolist() == [0, 10, 20, 30]
    assert ulysses_sequence_view(recv[1]).ravel().tolist() == [1, 11, 21, 31]
    # the buffer a rank sends: block j is for rank j
    send0 = ulysses_pack(shards(full, 2)[0], 2)
    assert send0[0].ravel().tolist() == [0, 10]
    assert send0[1].ravel().tolist() == [1, 11]


def test_hand_worked_replicated_head():
    # one key/value head, two ranks: both receive it for all tokens, and the
    # return exchange sums what both send back for it.
    full = np.array([[[[1.0]], [[2.0]], [[3.0]], [[4.0]]]])  # [1, 4, 1, 1]
    assert ulysses_heads_per_rank(1, 2) == 1
    recv = all_to_all([ulysses_pack(x, 2) for x in shards(full, 2)])
    for j in range(2):
        assert ulysses_sequence_view(recv[j]).ravel().tolist() == [1, 2, 3, 4]
    back = all_to_all([np.full((2, 2, 1, 1, 1), 10.0 ** j) for j in range(2)])
    assert ulysses_unpack(back[0], 1).ravel().tolist() == [11.0, 11.0]


def test_heads_per_rank_rules():
    assert ulysses_heads_per_rank(32, 8) == 4
    assert ulysses_heads_per_rank(8, 8) == 1
    assert ulysses_heads_per_rank(2, 8) == 1
    with pytest.raises(ValueError):
        ulysses_heads_per_rank(6, 4)


@pytest.mark.parametrize("b,nl,h,d,p", [(1, 3, 4, 2, 2), (2, 2, 6, 3, 3), (1, 4, 8, 1, 8),
                                        (2, 3, 5, 2, 1)])
def test_every_element_travels_once(b, nl, h, d, p):
    xs = [rnd(10 + j, b, nl, h, d) for j in range(p)]
    sent = np.concatenate([ulysses_pack(x, p).ravel() for x in xs])
    assert np.array_equal(np.sort(sent), np.sort(np.concatenate([x.ravel() for x in xs])))


@pytest.mark.parametrize("b,nl,h,d,p", [(1, 3, 4, 2, 2), (2, 2, 6, 3, 3), (1, 2, 2, 2, 4),
                                        (2, 1, 1, 3, 4)])
def test_round_trip(b, nl, h, d, p):
    xs = [rnd(20 + j, b, nl, h, d) for j in range(p)]
    recv = all_to_all([ulysses_pack(x, p) for x in xs])
    back = all_to_all(recv)  # send each received block back where it came from
    reps = p // h if p > h else 1
    for j in range(p):
        np.testing.assert_array_equal(ulysses_unpack(back[j], h), reps * xs[j])


CASES = [  # b, n, hq, hkv, d, p
    (1, 12, 4, 4, 3, 2),
    (2, 8, 4, 2, 4, 4),    # kv heads 2 over 4 ranks: each replicated twice
    (1, 12, 6, 6, 2, 3),
    (1, 8, 4, 1, 3, 4),    # one kv head on every rank
    (2, 6, 2, 2, 2, 1),
    (1, 16, 8, 2, 2, 4),   # 2 query heads per rank sharing one kv head
]


def run_ulysses_forward(q, k, v, p, scale, causal):
    hq = q.shape[2]
    rq, rk, rv = (all_to_all([ulysses_pack(x, p) for x in shards(t, p)]) for t in (q, k, v))
    o_send, lse_parts = [], []
    for j in range(p):
        o, lse = attention_forward(*(ulysses_sequence_view(r[j]) for r in (rq, rk, rv)),
                                   scale, causal)
        o_send.append(to_send(o, p))
        lse_parts.append(lse)
    o_recv = all_to_all(o_send)
    return [ulysses_unpack(o_recv[r], hq) for r in range(p)], lse_parts


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_ulysses_attention_equals_full(case, causal):
    b, n, hq, hkv, d, p = case
    q, k, v = rnd(1, b, n, hq, d), rnd(2, b, n, hkv, d), rnd(3, b, n, hkv, d)
    scale = 0.4
    o_full, lse_full = attention_forward(q, k, v, scale, causal)
    outs, lses = run_ulysses_forward(q, k, v, p, scale, causal)
    nl = n // p
    for r in range(p):
        np.testing.assert_allclose(outs[r], o_full[:, r * nl:(r + 1) * nl], rtol=0, atol=1e-12)
    hl = hq // p
    for j in range(p):
        np.testing.assert_allclose(lses[j], lse_full[:, j * hl:(j + 1) * hl], rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_ulysses_backward_equals_full(case):
    b, n, hq, hkv, d, p = case
    q, k, v, do = (rnd(4, b, n, hq, d), rnd(5, b, n, hkv, d), rnd(6, b, n, hkv, d),
                   rnd(7, b, n, hq, d))
    scale, causal = 0.4, True
    dq_f, dk_f, dv_f = attention_backward(q, k, v, do, scale, causal)
    rq, rk, rv, rdo = (all_to_all([ulysses_pack(x, p) for x in shards(t, p)])
                       for t in (q, k, v, do))
    sends = {"dq": [], "dk": [], "dv": []}
    for j in range(p):
        grads = attention_backward(*(ulysses_sequence_view(r[j]) for r in (rq, rk, rv, rdo)),
                                   scale, causal)
        for name, g in zip(("dq", "dk", "dv"), grads):
            sends[name].append(to_send(g, p))
    nl = n // p
    for name, full, heads in (("dq", dq_f, hq), ("dk", dk_f, hkv), ("dv", dv_f, hkv)):
        recv = all_to_all(sends[name])
        for r in range(p):
            np.testing.assert_allclose(ulysses_unpack(recv[r], heads),
                                       full[:, r * nl:(r + 1) * nl], rtol=0, atol=1e-11)


def test_unpack_rejects_mismatched_buffer():
    with pytest.raises(ValueError):
        ulysses_unpack(np.zeros((4, 2, 1, 2, 3)), 4)  # 4 heads over 4 ranks is Hl = 1
