"""GPU tests of the measurement entry points: per-kernel event timing on a
plan and the exponential-rate probe."""
import ctypes

import pytest

from attention_fab_forward_amd.inputs import random_array
from fab_testutil import to_device

pytestmark = pytest.mark.gpu


def attention_plan_and_buffers(dtype, d, causal):
    import torch
    from attention_fab_forward_amd import _binding as B
    q = to_device(random_array(121, (1, 300, 4, d), 1.0, dtype), dtype)
    k = to_device(random_array(122, (1, 300, 2, d), 1.0, dtype), dtype)
    v = to_device(random_array(123, (1, 300, 2, d), 1.0, dtype), dtype)
    do = to_device(random_array(124, (1, 300, 4, d), 1.0, dtype), dtype)
    plan = B.attention_plan(q, k, v, causal, d ** -0.5)
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 300), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(plan.bwd_workspace, 1), dtype=torch.uint8, device=q.device)
    P, s = B._ptr, B._stream()

    def step():
        plan.forward_raw(P(q), P(k), P(v), P(o), P(lse), P(ws), plan.fwd_workspace, s)
        plan.backward_raw(P(q), P(k), P(v), P(o), P(lse), P(do), P(dq), P(dk), P(dv), P(ws),
                          plan.bwd_workspace, s)
    return plan, step


@pytest.mark.parametrize("dtype,d,kernels", [
    ("bf16", 128, {"attn_fwd_bf16", "attn_bwd_prep", "attn_bwd_dkdv_bf16", "attn_bwd_dq_bf16"}),
    ("f32", 64, {"attn_fwd_f32", "attn_bwd_f32"}),
])
def test_per_kernel_timing(dtype, d, kernels):
    plan, step = attention_plan_and_buffers(dtype, d, True)
    step()
    assert plan.kernel_times() == {}  # timing off: nothing recorded
    plan.set_timing(True)
    plan.reset_kernel_times()
    for _ in range(3):
        step()
    t = plan.kernel_times()
    assert set(t) == kernels
    for name, (count, total_ms) in t.items():
        assert count == 3, name
        assert 0.0 < total_ms < 1000.0, name
    plan.reset_kernel_times()
    assert all(c == 0 for c, _ in plan.kernel_times().values())
    plan.set_timing(False)
    assert plan.kernel_times() == {}


def test_exp_probe_runs_and_counts():
    import torch
    from attention_fab_forward_amd import _binding as B
    L = B.lib()
    blocks, iters = 64, 256
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    count = ctypes.c_int64()
    B.check(L.fab_exp_probe(blocks, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.byref(count),
                            B._stream()))
    torch.cuda.synchronize()
    chains = count.value // (blocks * 256 * iters)
    assert count.value == blocks * 256 * iters * chains and chains >= 1
    # every lane wrote the sum of its chains, each of which stays in (0, 1)
    assert bool(((sink > 0) & (sink < chains)).all())
