"""GPU parity of attention forward + backward on a seeded sweep of shapes:
batch, ragged and rectangular m x n, grouped kv heads, both head dims and
dtypes, causal masks with global offsets (rows that see no key included)."""
import numpy as np
import pytest

from attention_fab_forward_amd.inputs import random_array
from oracle import attention_backward, attention_forward
from fab_testutil import assert_close, assert_lse, grad_floors, to_device, to_host

pytestmark = pytest.mark.gpu


def cases(count=96, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        dtype = "bf16" if i % 3 else "f32"
        d = int(rng.choice([64, 128]))
        b = int(rng.integers(1, 3))
        hkv = int(rng.integers(1, 4))
        group = int(rng.choice([1, 2, 4]))
        m = int(rng.integers(1, 1200))
        n = int(rng.integers(1, 1200))
        causal = bool(rng.integers(0, 2))
        qo = ko = 0
        if causal:
            qo, ko = (int(x) for x in rng.integers(-300, 300, 2))
        out.append((i, dtype, d, b, hkv * group, hkv, m, n, causal, qo, ko))
    return out


@pytest.mark.parametrize("i,dtype,d,b,hq,hkv,m,n,causal,qo,ko", cases())
def test_random_shape(i, dtype, d, b, hq, hkv, m, n, causal, qo, ko):
    import attention_fab_forward_amd as fab
    x = {"q": random_array(1000 + 4 * i, (b, m, hq, d), 1.0, dtype),
         "k": random_array(1001 + 4 * i, (b, n, hkv, d), 1.0, dtype),
         "v": random_array(1002 + 4 * i, (b, n, hkv, d), 1.0, dtype),
         "do": random_array(1003 + 4 * i, (b, m, hq, d), 1.0, dtype)}
    sc = float(np.float32(d ** -0.5))
    q, k, v, do = (to_device(x[t], dtype) for t in ("q", "k", "v", "do"))
    o, lse = fab.forward(q, k, v, "softmax", causal, sc, q_offset=qo, k_offset=ko)
    dq, dk, dv = fab.backward(q, k, v, o, lse, do, "softmax", causal, sc, q_offset=qo,
                              k_offset=ko)
    ro, rl = attention_forward(x["q"], x["k"], x["v"], sc, causal, q_offset=qo, k_offset=ko)
    rq, rk, rv = attention_backward(x["q"], x["k"], x["v"], x["do"], sc, causal,
                                    q_offset=qo, k_offset=ko)
    fq, fk = grad_floors(x, sc, causal, ro, qo, ko)
    assert_close("O", to_host(o), ro, dtype)
    lse_h = lse.cpu().numpy().astype(np.float64)
    finite = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse_h), finite), "rows without keys must get LSE = -inf"
    assert_lse(lse_h[finite], rl[finite], dtype)
    assert_close("dQ", to_host(dq), rq, dtype, floor=fq)
    assert_close("dK", to_host(dk), rk, dtype, floor=fk)
    assert_close("dV", to_host(dv), rv, dtype)
