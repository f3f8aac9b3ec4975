"""GPU parity of the fused GeLU MLP (forward and backward) against the fp64 oracle."""
import numpy as np
import pytest

from attention_fab_forward_amd.inputs import WORKLOADS, mlp_inputs, random_array
from oracle import mlp_backward, mlp_forward
from fab_testutil import assert_close, to_device, to_host

pytestmark = pytest.mark.gpu


def run(x, scale):
    import attention_fab_forward_amd as fab
    a, bt, c, do = (to_device(x[n], "bf16") for n in ("a", "bt", "c", "do"))
    o, lse = fab.forward(a, bt, c, "gelu", False, scale)
    assert lse is None
    da, dbt, dc = fab.backward(a, bt, c, None, None, do, "gelu", False, scale)
    return to_host(o), to_host(da), to_host(dbt), to_host(dc)


def check(x, scale):
    o, da, dbt, dc = run(x, scale)
    ro = mlp_forward(x["a"], x["bt"], x["c"], scale)
    ra, rb, rc = mlp_backward(x["a"], x["bt"], x["c"], x["do"], scale)
    errs = [assert_close("O", o, ro, "bf16"), assert_close("dA", da, ra, "bf16"),
            assert_close("dBt", dbt, rb, "bf16"), assert_close("dC", dc, rc, "bf16")]
    print("errors O/dA/dBt/dC:", " ".join(f"{e:.2e}" for e in errs))


def test_full_size_m4096_k1024_n4096_p1024():
    w = WORKLOADS["mlp_gelu_m4096_k1024_n4096_p1024"]
    check(mlp_inputs(w), w.scale())


@pytest.mark.parametrize("m,n,k,p", [(1, 1, 128, 128), (100, 33, 128, 256), (300, 200, 256, 128),
                                     (64, 1000, 512, 512), (257, 96, 1024, 128),
                                     (33, 70, 128, 1024)])
@pytest.mark.parametrize("sigma", [0.02, 0.15])
def test_ragged_shapes(m, n, k, p, sigma):
    x = {"a": random_array(91, (m, k), sigma, "bf16"), "bt": random_array(92, (n, k), sigma, "bf16"),
         "c": random_array(93, (n, p), sigma, "bf16"), "do": random_array(94, (m, p), 1.0, "bf16")}
    check(x, 1.0)


def test_scale_and_strided_rows():
    import torch
    import attention_fab_forward_amd as fab
    m, n, k, p = 130, 70, 256, 128
    big_a = random_array(95, (m, k + 64), 0.1, "bf16")
    x = {"a": big_a[:, :k], "bt": random_array(96, (n, k), 0.1, "bf16"),
         "c": random_array(97, (n, p), 0.1, "bf16"), "do": random_array(98, (m, p), 1.0, "bf16")}
    a = to_device(big_a, "bf16")[:, :k]
    assert not a.is_contiguous()
    bt, c, do = (to_device(x[n_], "bf16") for n_ in ("bt", "c", "do"))
    o, _ = fab.forward(a, bt, c, "gelu", False, 0.7)
    da, dbt, dc = fab.backward(a, bt, c, None, None, do, "gelu", False, 0.7)
    assert da.stride() == a.stride()
    ra, rb, rc = mlp_backward(x["a"], x["bt"], x["c"], x["do"], 0.7)
    assert_close("O", to_host(o), mlp_forward(x["a"], x["bt"], x["c"], 0.7), "bf16")
    assert_close("dA", to_host(da), ra, "bf16")
    assert_close("dBt", to_host(dbt), rb, "bf16")
    assert_close("dC", to_host(dc), rc, "bf16")
    del torch


def test_zero_weights_special_case():
    """Bt = 0 gives O = 0, dA = 0, dC = 0 and dBt = scale/2 (dO C^T)^T A exactly
    up to rounding."""
    import attention_fab_forward_amd as fab
    m, n, k, p = 96, 64, 128, 128
    a = random_array(99, (m, k), 0.5, "bf16")
    c = random_array(100, (n, p), 0.5, "bf16")
    do = random_array(101, (m, p), 1.0, "bf16")
    bt = np.zeros((n, k), np.float32)
    ta, tb, tc, tdo = (to_device(v, "bf16") for v in (a, bt, c, do))
    o, _ = fab.forward(ta, tb, tc, "gelu", False, 0.9)
    da, dbt, dc = fab.backward(ta, tb, tc, None, None, tdo, "gelu", False, 0.9)
    assert float(o.abs().max()) == 0 and float(da.abs().max()) == 0 and float(dc.abs().max()) == 0
    ref = 0.5 * 0.9 * (do.astype(np.float64) @ c.T.astype(np.float64)).T @ a.astype(np.float64)
    assert_close("dBt", to_host(dbt), ref, "bf16")


@pytest.mark.parametrize("k", [128, 256, 512, 1024])
@pytest.mark.parametrize("p", [128, 256, 512, 1024])
def test_every_supported_width_pair(k, p):
    """Each (k, p) pair the library instantiates, at small ragged m and n."""
    m, n = 77, 45
    x = {"a": random_array(111, (m, k), 0.1, "bf16"), "bt": random_array(112, (n, k), 0.1, "bf16"),
         "c": random_array(113, (n, p), 0.1, "bf16"), "do": random_array(114, (m, p), 1.0, "bf16")}
    check(x, 1.0)


@pytest.mark.parametrize("k,p", [(64, 128), (128, 64), (192, 320), (320, 192), (64, 64),
                                 (448, 960), (960, 576), (1024, 64)])
def test_widths_between_the_compiled_ones(k, p):
    """k and p multiples of 64 that the kernels run zero-padded to the next
    compiled width (128, 256, 512, 1024): the padding must not leak into any
    output or gradient."""
    m, n = 130, 97
    x = {"a": random_array(121, (m, k), 0.1, "bf16"), "bt": random_array(122, (n, k), 0.1, "bf16"),
         "c": random_array(123, (n, p), 0.1, "bf16"), "do": random_array(124, (m, p), 1.0, "bf16")}
    check(x, 1.0)


def mlp_cases(count=24, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        k = int(rng.choice([128, 256, 512, 1024]))
        p = int(rng.choice([128, 256, 512, 1024]))
        m = int(rng.integers(1, 1500))
        n = int(rng.integers(1, 1500))
        sigma = float(rng.choice([0.02, 0.1, 0.3]))
        scale = float(np.float32(rng.uniform(0.25, 2.0)))
        out.append((i, m, n, k, p, sigma, scale))
    return out


@pytest.mark.parametrize("i,m,n,k,p,sigma,scale", mlp_cases())
def test_random_shape(i, m, n, k, p, sigma, scale):
    x = {"a": random_array(2000 + 4 * i, (m, k), sigma, "bf16"),
         "bt": random_array(2001 + 4 * i, (n, k), sigma, "bf16"),
         "c": random_array(2002 + 4 * i, (n, p), sigma, "bf16"),
         "do": random_array(2003 + 4 * i, (m, p), 1.0, "bf16")}
    check(x, scale)


def test_forward_and_backward_are_deterministic():
    """The split partial sums are added by a fixed-order reduction (no
    atomics): two calls on the same inputs give bitwise-identical O, dA, dBt
    and dC at the full size."""
    import attention_fab_forward_amd as fab
    import torch
    x = mlp_inputs(WORKLOADS["mlp_gelu_m4096_k1024_n4096_p1024"])
    a, bt, c, do = (to_device(x[n], "bf16") for n in ("a", "bt", "c", "do"))
    outs = []
    for _ in range(2):
        o, _lse = fab.forward(a, bt, c, "gelu", False, 1.0)
        outs.append((o,) + tuple(fab.backward(a, bt, c, None, None, do, "gelu", False, 1.0)))
    for name, u, w in zip(("O", "dA", "dBt", "dC"), outs[0], outs[1]):
        assert torch.equal(u, w), name
