"""GPU parity of the attention backward (dQ, dK, dV) against the fp64 oracle."""
import numpy as np
import pytest

from attention_fab_forward_amd.inputs import WORKLOADS, attention_inputs, random_array
from oracle import (attention_backward, attention_backward_keys, attention_backward_rows,
                    attention_forward)
from fab_testutil import (assert_close, assert_lse, dk_floor_keys, dq_floor_rows, grad_floors,
                          to_device, to_host)

pytestmark = pytest.mark.gpu


def run(x, dtype, causal, scale):
    import attention_fab_forward_amd as fab
    q, k, v, do = (to_device(x[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fab.forward(q, k, v, "softmax", causal, scale)
    dq, dk, dv = fab.backward(q, k, v, o, lse, do, "softmax", causal, scale)
    return (to_host(o), lse.cpu().numpy().astype(np.float64), to_host(dq), to_host(dk),
            to_host(dv))


def check(x, dtype, causal, scale):
    o, lse, dq, dk, dv = run(x, dtype, causal, scale)
    ro, rl = attention_forward(x["q"], x["k"], x["v"], scale, causal)
    rq, rk, rv = attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    fq, fk = grad_floors(x, scale, causal, ro)
    errs = [assert_close("O", o, ro, dtype), assert_close("dQ", dq, rq, dtype, floor=fq),
            assert_close("dK", dk, rk, dtype, floor=fk), assert_close("dV", dv, rv, dtype)]
    assert_lse(lse, rl, dtype)
    print("errors O/dQ/dK/dV:", " ".join(f"{e:.2e}" for e in errs))


def test_fp32_single_head_n256_d64():
    w = WORKLOADS["attn_f32_h1_n256_d64"]
    check(attention_inputs(w), "f32", False, w.scale())


@pytest.mark.parametrize("n", [256, 1000, 4096])
def test_bf16_causal_h32_d128_reduced(n):
    """All 32 heads at reduced n, every element against the oracle (n = 4096
    is the largest reduced size the plan for full-tensor parity names)."""
    w = WORKLOADS["attn_causal_bf16_h32_n32768_d128"]
    check(attention_inputs(w, seq=n), "bf16", True, w.scale())


@pytest.mark.parametrize("n", [4096, 16384])
def test_bf16_rank_share_reduced(n):
    """The rank share's 4 heads, full tensors up to n = 16384."""
    w = WORKLOADS["attn_causal_bf16_h4_n131072_d128"]
    check(attention_inputs(w, seq=n), "bf16", True, w.scale())


@pytest.mark.parametrize("n", [1024, 4096, 16384])
def test_bf16_causal_gqa_reduced(n):
    w = WORKLOADS["attn_causal_bf16_gqa2_n1048576_d128"]
    check(attention_inputs(w, seq=n), "bf16", True, w.scale())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,hq,hkv", [(1, 2, 1), (17, 2, 2), (65, 4, 2), (129, 3, 1),
                                      (200, 2, 1)])
def test_bf16_small_and_ragged(d, causal, n, hq, hkv):
    x = {"q": random_array(61, (1, n, hq, d), 1.0, "bf16"),
         "k": random_array(62, (1, n, hkv, d), 1.0, "bf16"),
         "v": random_array(63, (1, n, hkv, d), 1.0, "bf16"),
         "do": random_array(64, (1, n, hq, d), 1.0, "bf16")}
    check(x, "bf16", causal, float(np.float32(d ** -0.5)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 40, 300])
def test_fp32_small_and_ragged(d, causal, n):
    x = {"q": random_array(71, (2, n, 4, d)), "k": random_array(72, (2, n, 2, d)),
         "v": random_array(73, (2, n, 2, d)), "do": random_array(74, (2, n, 4, d))}
    check(x, "f32", causal, float(np.float32(d ** -0.5)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rectangular_noncausal(dtype):
    x = {"q": random_array(81, (2, 300, 4, 128), 1.0, dtype),
         "k": random_array(82, (2, 777, 2, 128), 1.0, dtype),
         "v": random_array(83, (2, 777, 2, 128), 1.0, dtype),
         "do": random_array(84, (2, 300, 4, 128), 1.0, dtype)}
    check(x, dtype, False, 0.07)


def identities(q, k, v, o, do, dq, dk, dv, group, scale):
    """Exact identities of the softmax block, checked on device outputs.

    sum_j dV_j = sum over the group's heads and rows of dO (rows of P sum to 1);
    sum_j dK_j = 0 (rows of dS sum to 0); <dV, V> = <dO, O>;
    <dQ, Q> = <dK, K> (invariance under Q -> aQ, K -> K/a).

    Tolerance: each side is a sum over rows whose rounding errors are
    independent, so rows within the per-row gate give a sum within 1e-2 of
    the root-sum-square of the rows' terms (per d column for the vector
    identities, per row's |inner product| for the scalar ones), not of their
    plain sum; at n = 2^20 that is about 1000 times tighter.  sum_j dK_j also
    carries D's rounding: it equals scale sum_i (sum_j dS_ij) Q_i, and an error
    e_i in D_i moves sum_j dS_ij by -e_i, so its budget adds the D term the
    per-row gate allows, 1e-2 scale w_i |Q_i| with w_i = sum_d |dO_id O_id|,
    combined over the query rows (and heads of the group) the same way.  In
    <dQ, Q> - <dK, K> D's contribution is the same on both sides and cancels.
    """
    b, n, hkv, d = k.shape
    rss = lambda *xs: np.sqrt(sum(np.sum(np.square(x), axis=1) for x in xs))
    grouped = lambda x: x.reshape(b, -1, hkv, group, x.shape[-1])
    do_g = grouped(do).sum(axis=3)
    err = np.abs(dv.sum(axis=1) - do_g.sum(axis=1))
    bound = 1e-2 * rss(dv, do_g)
    print(f"  sum dV - sum dO: max {float(np.max(err / bound)):.2f} of the bound")
    assert np.all(err <= bound), "sum dV != sum dO"
    w = np.abs(do * o).sum(axis=-1, keepdims=True)  # [b, m, hq, 1]
    wq = grouped(w * np.abs(q))                      # [b, m, hkv, group, d]
    d_term = scale * np.sqrt(np.sum(np.square(wq), axis=(1, 3)))
    err = np.abs(dk.sum(axis=1))
    bound = 1e-2 * (rss(dk) + d_term)
    print(f"  sum dK: max {float(np.max(err / bound)):.2f} of the bound "
          f"(without the D term: {float(np.max(err / (1e-2 * rss(dk)))):.2f})")
    assert np.all(err <= bound), "sum dK != 0"
    row_dot = lambda x, y: np.abs(x * y).sum(axis=-1).ravel()
    for (x1, y1), (x2, y2), name in (((dv, v), (do, o), "<dV,V> = <dO,O>"),
                                      ((dq, q), (dk, k), "<dQ,Q> = <dK,K>")):
        a, bb = np.sum(x1 * y1), np.sum(x2 * y2)
        bound = 1e-2 * np.sqrt(np.sum(row_dot(x1, y1) ** 2) + np.sum(row_dot(x2, y2) ** 2))
        print(f"  {name}: {abs(a - bb) / bound:.2f} of the bound")
        assert abs(a - bb) <= bound, (name, a, bb)


def sampled(n, seed, count=16):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, 127, 128, n // 2, n - 65, n - 64, n - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, n, count)]))


@pytest.mark.parametrize("key", ["attn_causal_bf16_h32_n32768_d128",
                                 "attn_causal_bf16_h4_n131072_d128",
                                 "attn_causal_bf16_gqa2_n1048576_d128"])
def test_full_size_sampled_and_identities(key):
    """Full-size backward (the benchmarked launch): exact oracle rows of dQ,
    exact late-key rows of dK / dV, and the identities over every row."""
    w = WORKLOADS[key]
    x = attention_inputs(w)
    o, lse, dq, dk, dv = run(x, "bf16", True, w.scale())
    identities(x["q"], x["k"], x["v"], o, x["do"], dq, dk, dv, w.heads_q // w.heads_kv,
               w.scale())
    n = w.seq
    rows = sampled(n, w.number)
    keys = np.unique(np.concatenate([[n - 256, n - 129, n - 128, n - 2, n - 1],
                                     np.random.default_rng(w.number).integers(n - 256, n, 8)]))
    for h in sorted({0, w.heads_q - 1}):
        rq = attention_backward_rows(x["q"], x["k"], x["v"], x["do"], w.scale(), True, 0, h, rows)
        fq = dq_floor_rows(x, w.scale(), True, 0, h, rows)
        assert_close(f"dQ head {h}", dq[0, rows, h], rq, "bf16", floor=fq)
    for g in sorted({0, w.heads_kv - 1}):
        rk, rv = attention_backward_keys(x["q"], x["k"], x["v"], x["do"], w.scale(), True, 0, g,
                                         keys)
        fk = dk_floor_keys(x, w.scale(), True, 0, g, keys)
        assert_close(f"dK head {g}", dk[0, keys, g], rk, "bf16", floor=fk)
        assert_close(f"dV head {g}", dv[0, keys, g], rv, "bf16")


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_strided_views_backward(dtype, d, causal):
    """Q, K, V as views of one fused [b, n, h, 3, d] projection (row stride
    3 h d, unlike O and dO, packed at h d), and a grouped-query case whose K and
    V have different row strides (K contiguous, V a view of a [b, n, hkv, 2, d]
    tensor): the kernel variants for unequal strides.  Gradients take the
    layouts of their primal views."""
    import attention_fab_forward_amd as fab
    b, n, h = 2, 300, 3
    big = random_array(101, (b, n, h, 3, d), 1.0, dtype)
    do = random_array(102, (b, n, h, d), 1.0, dtype)
    t = to_device(big, dtype)
    q, k, v = t[:, :, :, 0], t[:, :, :, 1], t[:, :, :, 2]
    assert q.stride(1) == 3 * h * d
    sc = float(np.float32(d ** -0.5))
    o, lse = fab.forward(q, k, v, "softmax", causal, sc)
    dq, dk, dv = fab.backward(q, k, v, o, lse, to_device(do, dtype), "softmax", causal, sc)
    assert dq.stride() == q.stride() and dk.stride() == k.stride()
    xs = {"q": big[:, :, :, 0], "k": big[:, :, :, 1], "v": big[:, :, :, 2], "do": do}
    rq, rk, rv = attention_backward(xs["q"], xs["k"], xs["v"], do, sc, causal)
    fq, fk = grad_floors(xs, sc, causal)
    assert_close("dQ", to_host(dq), rq, dtype, floor=fq)
    assert_close("dK", to_host(dk), rk, dtype, floor=fk)
    assert_close("dV", to_host(dv), rv, dtype)

    hq, hkv = 4, 2
    qg = random_array(103, (b, n, hq, d), 1.0, dtype)
    kg = random_array(104, (b, n, hkv, d), 1.0, dtype)
    kvbig = random_array(105, (b, n, hkv, 2, d), 1.0, dtype)
    vg = kvbig[:, :, :, 1]
    dog = random_array(106, (b, n, hq, d), 1.0, dtype)
    vt = to_device(kvbig, dtype)[:, :, :, 1]
    qt, kt = to_device(qg, dtype), to_device(kg, dtype)
    assert vt.stride(1) != kt.stride(1)
    o, lse = fab.forward(qt, kt, vt, "softmax", causal, sc)
    dq, dk, dv = fab.backward(qt, kt, vt, o, lse, to_device(dog, dtype), "softmax", causal, sc)
    assert dv.stride() == vt.stride()
    rq, rk, rv = attention_backward(qg, kg, vg, dog, sc, causal)
    fq, fk = grad_floors({"q": qg, "k": kg, "v": vg, "do": dog}, sc, causal)
    assert_close("dQ (GQA, V strided)", to_host(dq), rq, dtype, floor=fq)
    assert_close("dK (GQA, V strided)", to_host(dk), rk, dtype, floor=fk)
    assert_close("dV (GQA, V strided)", to_host(dv), rv, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_peaked_scores_backward(dtype, causal):
    """Queries and keys drawn with sigma 3 at d = 128: scores with a standard
    deviation near 9, so most rows put nearly all their weight on a few keys
    and the running maximum moves by large steps.  The backward recomputes P
    from the saved LSE; every gradient row still meets the bar."""
    b, n, h, d = 1, 300, 2, 128
    x = {"q": random_array(111, (b, n, h, d), 3.0, dtype),
         "k": random_array(112, (b, n, h, d), 3.0, dtype),
         "v": random_array(113, (b, n, h, d), 1.0, dtype),
         "do": random_array(114, (b, n, h, d), 1.0, dtype)}
    check(x, dtype, causal, float(np.float32(d ** -0.5)))


def test_backward_is_deterministic():
    """No atomics anywhere in the backward: two calls on the same inputs give
    bitwise-identical dQ, dK and dV (grouped-query heads, causal)."""
    import attention_fab_forward_amd as fab
    import torch
    x = attention_inputs(WORKLOADS["attn_causal_bf16_gqa2_n1048576_d128"], seq=2048)
    q, k, v, do = (to_device(x[t], "bf16") for t in ("q", "k", "v", "do"))
    o, lse = fab.forward(q, k, v, "softmax", True)
    first = fab.backward(q, k, v, o, lse, do, "softmax", True)
    second = fab.backward(q, k, v, o, lse, do, "softmax", True)
    for name, a, c in zip(("dQ", "dK", "dV"), first, second):
        assert torch.equal(a, c), name
