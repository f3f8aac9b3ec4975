"""GPU parity of the fp32 matrix-core attention kernels (forward and
backward) against the fp64 oracle at the fp32 bound (1e-5 per row): the
kernel family forced on small, ragged, grouped-query, rectangular, offset and
strided problems, and chosen by the library for the large ones it serves."""
import numpy as np
import pytest

from attention_fab_forward_amd import _binding as B
from attention_fab_forward_amd.inputs import random_array
from oracle import attention_backward, attention_forward
from fab_testutil import assert_close, assert_lse, grad_floors, to_device, to_host

pytestmark = pytest.mark.gpu

MFMA = B.VARIANT_F32_MFMA


def run_check(x, causal, scale, variant=MFMA, q_offset=0, k_offset=0, expect_mfma=True):
    import attention_fab_forward_amd as fab
    q, k, v, do = (to_device(x[t], "f32") for t in ("q", "k", "v", "do"))
    plan = B.attention_plan(q, k, v, causal, scale, q_offset, k_offset, variant=variant)
    assert ("fp32 MFMA" in plan.describe()) == expect_mfma, plan.describe()
    o, lse = fab.forward(q, k, v, "softmax", causal, scale, q_offset, k_offset, variant=variant)
    dq, dk, dv = fab.backward(q, k, v, o, lse, do, "softmax", causal, scale, q_offset, k_offset,
                              variant=variant)
    ro, rl = attention_forward(x["q"], x["k"], x["v"], scale, causal, q_offset=q_offset,
                               k_offset=k_offset)
    rq, rk, rv = attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal,
                                    q_offset=q_offset, k_offset=k_offset)
    fq, fk = grad_floors(x, scale, causal, ro, q_offset, k_offset)
    assert_close("O", to_host(o), ro, "f32")
    assert_lse(lse.cpu().numpy().astype(np.float64), rl, "f32")
    assert_close("dQ", to_host(dq), rq, "f32", floor=fq)
    assert_close("dK", to_host(dk), rk, "f32", floor=fk)
    assert_close("dV", to_host(dv), rv, "f32")


def inputs(seed, b, m, n, hq, hkv, d):
    return {"q": random_array(seed, (b, m, hq, d)), "k": random_array(seed + 1, (b, n, hkv, d)),
            "v": random_array(seed + 2, (b, n, hkv, d)), "do": random_array(seed + 3, (b, m, hq, d))}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 33, 300])
def test_small_and_ragged(d, causal, n):
    run_check(inputs(3100 + n, 2, n, n, 4, 2, d), causal, float(np.float32(d ** -0.5)))


@pytest.mark.parametrize("causal", [False, True])
def test_rectangular(causal):
    run_check(inputs(3200, 2, 300, 777, 4, 2, 128), causal, 0.07)


@pytest.mark.parametrize("m,n,q_offset,k_offset", [(200, 300, 100, 0), (300, 200, 0, 100),
                                                   (129, 65, 64, 0), (100, 100, 0, 150)])
def test_offsets(m, n, q_offset, k_offset):
    run_check(inputs(3300 + m + n, 1, m, n, 2, 1, 64), True, 0.125, q_offset=q_offset,
              k_offset=k_offset)


@pytest.mark.parametrize("d", [64, 128])
def test_strided_views(d):
    """Q, K, V as views of one fused [b, n, h, 3, d] projection."""
    import attention_fab_forward_amd as fab
    b, n, h = 2, 200, 3
    big = random_array(3400 + d, (b, n, h, 3, d))
    do = random_array(3401 + d, (b, n, h, d))
    t = to_device(big, "f32")
    q, k, v = t[:, :, :, 0], t[:, :, :, 1], t[:, :, :, 2]
    sc = float(np.float32(d ** -0.5))
    o, lse = fab.forward(q, k, v, "softmax", True, sc, variant=MFMA)
    dq, dk, dv = fab.backward(q, k, v, o, lse, to_device(do, "f32"), "softmax", True, sc,
                              variant=MFMA)
    x = {"q": big[:, :, :, 0], "k": big[:, :, :, 1], "v": big[:, :, :, 2], "do": do}
    ro, _ = attention_forward(x["q"], x["k"], x["v"], sc, True)
    rq, rk, rv = attention_backward(x["q"], x["k"], x["v"], do, sc, True)
    fq, fk = grad_floors(x, sc, True, ro)
    assert_close("O", to_host(o), ro, "f32")
    assert_close("dQ", to_host(dq), rq, "f32", floor=fq)
    assert_close("dK", to_host(dk), rk, "f32", floor=fk)
    assert_close("dV", to_host(dv), rv, "f32")


@pytest.mark.parametrize("n,hq,hkv,d,causal", [(1024, 8, 8, 64, False), (2048, 4, 2, 128, True),
                                               (4096, 2, 1, 64, False),
                                               (8192, 1, 1, 128, True)])
def test_large_chosen_by_size(n, hq, hkv, d, causal):
    """Sizes the library runs on the matrix cores by itself (32 blocks of 64
    queries at d = 128, 64 at d = 64, and 2^22 unmasked pairs), every element
    against the oracle."""
    run_check(inputs(3500 + n + d, 1, n, n, hq, hkv, d), causal, float(np.float32(d ** -0.5)),
              variant=B.VARIANT_AUTO)


def test_forced_fma_family_still_runs_large():
    """The plain-FMA family can still be asked for at a size where the library
    would choose the matrix cores."""
    run_check(inputs(3600, 1, 1024, 1024, 8, 4, 64), False, 0.125, variant=B.VARIANT_F32_FMA,
              expect_mfma=False)




@pytest.mark.parametrize("a", [1.0, 4.0])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_rising_along_the_keys(a, causal):
    """The matrix-core forward on scores that rise along the keys up to 0 at
    each row's last visible key: raw score a (j - i) causal, a (j - n + 1)
    otherwise, from two nonzero columns holding small integers times a power
    of two, so every product and sum is exact in fp32.  With scale 1/sqrt(128)
    that is about 8 (a = 1) or 33 (a = 4) log2 units per 64 keys: the
    exponentials run against a reference that trails the row maximum, and the
    LSE stays small.  O and the LSE meet the fp32 bound."""
    import attention_fab_forward_amd as fab
    b, n, h, d = 1, 1024, 2, 128
    scale = float(np.float32(d ** -0.5))
    rows = np.arange(n, dtype=np.float32) if causal else np.full(n, n - 1.0, np.float32)
    q = np.zeros((b, n, h, d), np.float32)
    k = np.zeros((b, n, h, d), np.float32)
    q[..., 0] = a
    q[..., 1] = (-a * rows)[None, :, None]
    k[..., 0] = np.arange(n, dtype=np.float32)[None, :, None]
    k[..., 1] = 1.0
    x = {"q": q, "k": k, "v": random_array(131, (b, n, h, d))}
    qt, kt, vt = (to_device(x[t], "f32") for t in ("q", "k", "v"))
    o, lse = fab.forward(qt, kt, vt, "softmax", causal, scale, variant=MFMA)
    ro, rl = attention_forward(x["q"], x["k"], x["v"], scale, causal)
    assert_close("O", to_host(o), ro, "f32")
    assert_lse(lse.cpu().numpy().astype(np.float64), rl, "f32")
