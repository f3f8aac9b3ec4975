"""GPU parity of attention over a slice of the sequence (causal positions set
by q_offset / k_offset) and of the merge of results over disjoint key ranges,
against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

from attention_fab_forward_amd.inputs import random_array
from oracle import attention_backward, attention_forward, attention_merge
from fab_testutil import LSE_TOL, assert_close, grad_floors, to_device, to_host

pytestmark = pytest.mark.gpu

# (m, n, q_offset, k_offset): queries at global positions q_offset + i, keys at
# k_offset + j
CASES = [
    (256, 256, 0, 0),      # the plain causal mask
    (200, 300, 100, 0),    # a query slice at the end of the keys (m != n)
    (300, 200, 0, 100),    # keys start after the first 100 queries: empty rows
    (129, 65, 64, 0),      # ragged tiles on both axes
    (100, 100, 0, 150),    # no row sees a key
    (100, 100, 500, 0),    # every row sees every key
]


def inputs(seed, m, n, d, dtype, hq=4, hkv=2):
    return (random_array(seed, (1, m, hq, d), 1.0, dtype), random_array(seed + 1, (1, n, hkv, d), 1.0, dtype),
            random_array(seed + 2, (1, n, hkv, d), 1.0, dtype), random_array(seed + 3, (1, m, hq, d), 1.0, dtype))


def check_lse(got, ref, dtype):
    got = np.asarray(got, np.float64)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref)), "rows without keys must give -inf"
    fin = np.isfinite(ref)
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= LSE_TOL[dtype], f"lse: abs error {err:.3e}"
    return err


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("m,n,q_offset,k_offset", CASES)
def test_offset_forward_backward(dtype, d, m, n, q_offset, k_offset):
    import attention_fab_forward_amd as fab
    q, k, v, do = inputs(100 + m + n + q_offset, m, n, d, dtype)
    scale = float(np.float32(d ** -0.5))
    tq, tk, tv, tdo = (to_device(x, dtype) for x in (q, k, v, do))
    o, lse = fab.forward(tq, tk, tv, "softmax", True, scale, q_offset, k_offset)
    ro, rl = attention_forward(q, k, v, scale, True, q_offset=q_offset, k_offset=k_offset)
    print(f"case m={m} n={n} q_off={q_offset} k_off={k_offset} {dtype} d={d}")
    assert_close("O", to_host(o), ro, dtype)
    check_lse(lse.cpu().numpy(), rl, dtype)
    dq, dk, dv = fab.backward(tq, tk, tv, o, lse, tdo, "softmax", True, scale, q_offset, k_offset)
    rdq, rdk, rdv = attention_backward(q, k, v, do, scale, True, q_offset=q_offset,
                                       k_offset=k_offset)
    fq, fk = grad_floors({"q": q, "k": k, "v": v, "do": do}, scale, True, ro, q_offset, k_offset)
    for name, g, r, fl in (("dQ", dq, rdq, fq), ("dK", dk, rdk, fk), ("dV", dv, rdv, None)):
        assert_close(name, to_host(g), r, dtype, floor=fl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("causal", [True, False])
def test_key_split_merge_and_range_backward(dtype, causal):
    """Keys split into three ranges, each computed with its k_offset, merged
    pairwise on the GPU (the last merge in place) = the full result; the
    backward per range with the merged O, LSE gives dK, dV of the range and
    dQ contributions that sum to the full dQ."""
    import torch
    import attention_fab_forward_amd as fab
    d, n = (128, 640) if dtype == "bf16" else (64, 320)
    q, k, v, do = inputs(7, n, n, d, dtype)
    scale = float(np.float32(d ** -0.5))
    tq, tk, tv, tdo = (to_device(x, dtype) for x in (q, k, v, do))
    bounds = [0, 3 * n // 10, 7 * n // 10, n]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        ka, va = tk[:, a:b].contiguous(), tv[:, a:b].contiguous()
        parts.append(fab.forward(tq, ka, va, "softmax", causal, scale, 0, a))
    o12, l12 = fab.merge(parts[1][0], parts[1][1], parts[2][0], parts[2][1])
    o, lse = fab.merge(parts[0][0], parts[0][1], o12, l12, out=parts[0])  # in place
    assert o.data_ptr() == parts[0][0].data_ptr()
    ro, rl = attention_forward(q, k, v, scale, causal)
    assert_close("O merged", to_host(o), ro, dtype)
    check_lse(lse.cpu().numpy(), rl, dtype)
    # the merge kernel against the merge formula on the same two GPU parts
    mo, ml = attention_merge(to_host(parts[1][0]), parts[1][1].cpu().numpy(),
                             to_host(parts[2][0]), parts[2][1].cpu().numpy())
    assert_close("O merge formula", to_host(o12), mo, dtype)
    check_lse(l12.cpu().numpy(), ml, dtype)

    rdq, rdk, rdv = attention_backward(q, k, v, do, scale, causal)
    fq, fk = grad_floors({"q": q, "k": k, "v": v, "do": do}, scale, causal, ro)
    dq_sum = torch.zeros_like(tq, dtype=torch.float32)
    for (a, b) in zip(bounds[:-1], bounds[1:]):
        ka, va = tk[:, a:b].contiguous(), tv[:, a:b].contiguous()
        dq, dk, dv = fab.backward(tq, ka, va, o, lse, tdo, "softmax", causal, scale, 0, a)
        dq_sum += dq.float()
        assert_close(f"dK[{a}:{b}]", to_host(dk), rdk[:, a:b], dtype, floor=fk[:, a:b])
        assert_close(f"dV[{a}:{b}]", to_host(dv), rdv[:, a:b], dtype)
    assert_close("dQ (sum of ranges)", to_host(dq_sum), rdq, dtype, floor=fq)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_merge_direct(dtype, d):
    """fab_merge on random parts (batch 2, 3 heads, ragged rows; some rows with
    one or both LSE = -inf) against the merge formula."""
    import attention_fab_forward_amd as fab
    b, m, hq = 2, 77, 3
    oa = random_array(900 + d, (b, m, hq, d), 1.0, dtype)
    ob = random_array(901 + d, (b, m, hq, d), 1.0, dtype)
    la = 3.0 * np.random.default_rng(902).standard_normal((b, hq, m)).astype(np.float32)
    lb = 3.0 * np.random.default_rng(903).standard_normal((b, hq, m)).astype(np.float32)
    la[0, 1, :5] = -np.inf
    lb[1, 2, 3:9] = -np.inf
    la[1, 2, 5:7] = -np.inf          # rows 5, 6 of (1, 2): both sides empty
    import torch
    o, lse = fab.merge(to_device(oa, dtype), torch.from_numpy(la).cuda(),
                       to_device(ob, dtype), torch.from_numpy(lb).cuda())
    ro, rl = attention_merge(oa, la, ob, lb)
    assert_close("O merge", to_host(o), ro, dtype)
    check_lse(lse.cpu().numpy(), rl, dtype)
    assert np.all(to_host(o)[1, 5:7, 2] == 0.0)
