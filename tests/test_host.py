"""CPU tests of host-side pieces: the benchmark's contract and work counts,
and the product path failing loudly without the HIP library."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("fab_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_attention_work_counts():
    """Unmasked (query, key) pairs and flops of the attention workloads:
    n(n+1)/2 pairs per head when causal, n^2 otherwise; 4 d flops per pair
    forward, 10 d backward (five products, one recomputation of S)."""
    from attention_fab_forward_amd.inputs import WORKLOADS
    b = load_bench()
    expect = {  # fwd flops, bwd flops
        "attn_f32_h1_n256_d64": (16_777_216, 41_943_040),
        "attn_causal_bf16_h32_n32768_d128": (8_796_361_457_664, 21_990_903_644_160),
        "attn_causal_bf16_h4_n131072_d128": (17_592_320_262_144, 43_980_800_655_360),
        "attn_causal_bf16_gqa2_n1048576_d128": (562_950_490_292_224, 1_407_376_225_730_560),
        "attn_causal_f32_h8_n4096_d128": (34_368_126_976, 85_920_317_440),
    }
    for key, (fwd, bwd) in expect.items():
        f, g, unit = b.attention_flops(WORKLOADS[key])
        assert (f, g) == (fwd, bwd), key
        w = WORKLOADS[key]
        assert unit * 4 * w.d == fwd
    kf = b.kernel_flops(WORKLOADS["attn_causal_bf16_h32_n32768_d128"])
    # the dK/dV and dQ kernels together carry the backward's algorithmic flops
    assert kf["attn_bwd_dkdv_bf16"] + kf["attn_bwd_dq_bf16"] == 21_990_903_644_160


def test_measured_counters_only_for_matching_sources():
    """Counter summaries are attached to the bench line only while the kernel
    sources they were taken from are unchanged (hash in the summary)."""
    b = load_bench()
    assert b.measured_traffic("no_such_kernel") is None
    assert b.measured_mfma("no_such_kernel") is None
    m = b.measured_mfma("attn_bwd_dkdv_bf16")
    if m is not None:
        assert 0.0 < m["mfma_busy"] < 1.0 and 1.0 < m["clock_ghz"] < 2.5
        assert abs(m["bf16_flops_executed"] / 17_592_722_915_328 - 1.0) < 0.01


def test_product_path_fails_loudly_without_library():
    code = ("import attention_fab_forward_amd as fab\n"
            "try:\n"
            "    fab.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised', e)\n")
    env = dict(os.environ, FAB_LIBRARY=os.path.join(ROOT, "no_such_dir", "libfab.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised" in r.stdout and "not built" in r.stdout


def test_binding_rejects_mismatched_shapes_before_any_launch():
    """Shape disagreements between the operands raise in the binding (on the
    host, before device checks), so no kernel can index past a tensor."""
    import pytest
    import torch
    import attention_fab_forward_amd as fab
    from attention_fab_forward_amd import _binding as B
    e = lambda *sh: torch.empty(sh, dtype=torch.bfloat16)
    q, k, v = e(2, 64, 4, 128), e(2, 80, 2, 128), e(2, 80, 2, 128)
    assert B.attention_shapes(q, k, v) == (2, 64, 4, 2, 80, 128, 128)
    bad = {
        "batch": (q, e(1, 80, 2, 128), v),
        "v rows": (q, k, e(2, 79, 2, 128)),
        "v heads": (q, k, e(2, 80, 1, 128)),
        "k dim": (q, e(2, 80, 2, 64), v),
        "groups": (e(2, 64, 3, 128), k, v),
        "rank": (e(64, 4, 128), k, v),
    }
    for name, (a_, b_, c_) in bad.items():
        with pytest.raises(ValueError):
            fab.forward(a_, b_, c_, "softmax", True)
    o, do = e(2, 64, 4, 128), e(2, 64, 4, 128)
    lse = torch.empty(2, 4, 64)
    B.attention_grad_shapes(q, k, v, o, lse, do)
    for args in ((q, k, v, e(2, 64, 4, 64), lse, do), (q, k, v, o, lse, e(2, 63, 4, 128)),
                 (q, k, v, o, torch.empty(2, 64, 4), do), (q, e(2, 80, 2, 64), v, o, lse, do)):
        with pytest.raises(ValueError):
            fab.backward(*args, "softmax", True)
    a, bt, c = e(128, 256), e(512, 256), e(512, 128)
    assert B.mlp_shapes(a, bt, c, e(128, 128)) == (128, 256, 512, 128)
    for args in ((a, e(512, 128), c), (a, bt, e(256, 128)), (e(128, 256, 1), bt, c)):
        with pytest.raises(ValueError):
            fab.forward(*args, "gelu")
    with pytest.raises(ValueError):
        fab.backward(a, bt, c, None, None, e(128, 256), "gelu")
    with pytest.raises(ValueError):
        fab.backward(a, bt, e(511, 128), None, None, e(128, 128), "gelu")


def test_binding_layout_distinctness():
    """The binding's one-to-one layout test agrees with the library's rule:
    expanded (broadcast) tensors overlap, views of a fused projection do not."""
    import torch
    from attention_fab_forward_amd import _binding as B
    k = torch.empty(1, 16, 1, 8)
    assert B._distinct(k)
    assert not B._distinct(k.expand(1, 16, 4, 8))
    big = torch.empty(2, 16, 3, 3, 8)
    assert B._distinct(big[:, :, :, 1])
    assert not B._distinct(torch.empty(16, 8).as_strided((16, 8), (4, 1)))
    assert B._distinct(torch.empty(1, 1, 1, 8).expand(1, 1, 1, 8))
