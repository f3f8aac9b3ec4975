"""GPU parity of the attention forward against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

from attention_fab_forward_amd.inputs import WORKLOADS, attention_inputs, random_array
from oracle import attention_forward, attention_forward_rows
from fab_testutil import assert_close, assert_lse, to_device, to_host

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, dtype, causal, scale):
    import attention_fab_forward_amd as fab
    o, lse = fab.forward(to_device(q, dtype), to_device(k, dtype), to_device(v, dtype),
                         "softmax", causal, scale)
    return to_host(o), lse.cpu().numpy().astype(np.float64)


def check_fwd(x, dtype, causal, scale):
    o, lse = run_fwd(x["q"], x["k"], x["v"], dtype, causal, scale)
    ro, rl = attention_forward(x["q"], x["k"], x["v"], scale, causal)
    e = assert_close("O", o, ro, dtype)
    le = assert_lse(lse, rl, dtype)
    print(f"O err {e:.2e} lse err {le:.2e}")


def test_fp32_single_head_n256_d64():
    w = WORKLOADS["attn_f32_h1_n256_d64"]
    x = attention_inputs(w, with_grad=False)
    check_fwd(x, "f32", False, w.scale())


@pytest.mark.parametrize("n", [256, 1024, 1000])
def test_bf16_causal_h32_d128_reduced(n):
    w = WORKLOADS["attn_causal_bf16_h32_n32768_d128"]
    x = attention_inputs(w, seq=n, with_grad=False)
    check_fwd(x, "bf16", True, w.scale())


@pytest.mark.parametrize("n", [1024, 4096])
def test_bf16_causal_gqa_reduced(n):
    w = WORKLOADS["attn_causal_bf16_gqa2_n1048576_d128"]
    x = attention_inputs(w, seq=n, with_grad=False)
    check_fwd(x, "bf16", True, w.scale())


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 17, 63, 64, 65, 129, 200])
def test_bf16_small_and_ragged(d, causal, n):
    q = random_array(11, (1, n, 2, d), 1.0, "bf16")
    k = random_array(12, (1, n, 2, d), 1.0, "bf16")
    v = random_array(13, (1, n, 2, d), 1.0, "bf16")
    check_fwd({"q": q, "k": k, "v": v}, "bf16", causal, float(np.float32(d ** -0.5)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 33, 300])
def test_fp32_small_and_ragged(d, causal, n):
    q = random_array(21, (2, n, 3, d))
    k = random_array(22, (2, n, 1, d))
    v = random_array(23, (2, n, 1, d))
    check_fwd({"q": q, "k": k, "v": v}, "f32", causal, float(np.float32(d ** -0.5)))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rectangular_noncausal(dtype):
    q = random_array(31, (2, 300, 4, 128), 1.0, dtype)
    k = random_array(32, (2, 777, 2, 128), 1.0, dtype)
    v = random_array(33, (2, 777, 2, 128), 1.0, dtype)
    check_fwd({"q": q, "k": k, "v": v}, dtype, False, 0.07)


def test_strided_views():
    import torch
    import attention_fab_forward_amd as fab
    n, d = 333, 128
    big = random_array(41, (1, n, 3, 3, d), 1.0, "bf16")  # [b, n, h, {q,k,v}, d]
    t = to_device(big, "bf16")
    q, k, v = t[:, :, :, 0], t[:, :, :, 1], t[:, :, :, 2]
    assert not q.is_contiguous()
    o, lse = fab.forward(q, k, v, "softmax", True, 0.1)
    ro, rl = attention_forward(big[:, :, :, 0], big[:, :, :, 1], big[:, :, :, 2], 0.1, True)
    assert_close("O", to_host(o), ro, "bf16")
    assert_lse(lse.cpu().numpy(), rl, "bf16")
    del torch


def test_large_scores_stay_finite():
    q = random_array(51, (1, 256, 2, 128), 30.0, "bf16")
    k = random_array(52, (1, 256, 2, 128), 30.0, "bf16")
    v = random_array(53, (1, 256, 2, 128), 1.0, "bf16")
    check_fwd({"q": q, "k": k, "v": v}, "bf16", True, 0.0883883461356163)


@pytest.mark.parametrize("growth", [12.0, 40.0])
@pytest.mark.parametrize("causal", [False, True])
def test_scores_rising_along_the_keys(growth, causal):
    """Every row's scores rise steadily along the keys, by `growth` (in log2
    units) per 64-key block, up to a few hundred: each block's exponentials
    are taken against a reference that trails the row maximum, so in-block
    probabilities reach about 2^growth before the reference catches up (at
    12 it mostly stays put; at 40 a block's sum passes 2^32 and the reference
    moves at nearly every block).  O and the LSE still match the plain
    definition."""
    from attention_fab_forward_amd.inputs import round_to_bf16
    b, n, h, d = 1, 1024, 2, 128
    scale = float(np.float32(d ** -0.5))
    # score of key j in log2 units: 0.5 d c_j scale log2(e)
    per_key = growth / 64 / (0.5 * d * scale * 1.4426950408889634)
    c = round_to_bf16((np.arange(n) * per_key).astype(np.float32))
    q = np.full((b, n, h, d), 0.5, np.float32)
    k = np.ascontiguousarray(np.broadcast_to(c[None, :, None, None], (b, n, h, d)), np.float32)
    v = random_array(121, (b, n, h, d), 1.0, "bf16")
    check_fwd({"q": q, "k": k, "v": v}, "bf16", causal, scale)


def test_forward_is_deterministic():
    import attention_fab_forward_amd as fab
    x = attention_inputs(WORKLOADS["attn_causal_bf16_h32_n32768_d128"], seq=2048,
                         heads_q=8, heads_kv=8, with_grad=False)
    q, k, v = (to_device(x[n], "bf16") for n in "qkv")
    o1, l1 = fab.forward(q, k, v, "softmax", True)
    o2, l2 = fab.forward(q, k, v, "softmax", True)
    import torch
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


SAMPLE_ROWS = 24


def sampled_rows(n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 127, 128, 129, n // 2, n - 129, n - 128, n - 2, n - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, n, SAMPLE_ROWS)]))


@pytest.mark.parametrize("key", ["attn_causal_bf16_h32_n32768_d128",
                                 "attn_causal_bf16_h4_n131072_d128",
                                 "attn_causal_bf16_gqa2_n1048576_d128"])
def test_full_size_sampled_rows(key):
    """Full-size forward (the benchmarked launch), checked on sampled rows."""
    w = WORKLOADS[key]
    x = attention_inputs(w, with_grad=False)
    o, lse = run_fwd(x["q"], x["k"], x["v"], "bf16", True, w.scale())
    rows = sampled_rows(w.seq, w.number)
    heads = sorted({0, w.heads_q - 1, w.heads_q // 2})
    for h in heads:
        ro, rl = attention_forward_rows(x["q"], x["k"], x["v"], w.scale(), True, 0, h, rows)
        assert_close(f"O head {h}", o[0, rows, h], ro, "bf16")
        assert_lse(lse[0, h, rows], rl, "bf16")
