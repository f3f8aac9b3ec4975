"""GPU test of fab_backward_noalloc, the backward entry point that allocates
nothing (its workspace is the library's static per-GPU scratch), for callers
that cannot allocate device memory: through the
C ABI, two calls in a row -- the second on a smaller problem, so it runs on a
scratch that still holds the first call's values -- each against fab_backward
with a caller workspace on the same inputs (the same kernels, so the results
must be bitwise equal), and the attention case also against the oracle."""
import numpy as np
import pytest
import torch

from attention_fab_forward_amd import _binding as B
from attention_fab_forward_amd.inputs import random_array
from oracle import attention_backward
from fab_testutil import assert_close, grad_floors, to_device, to_host

pytestmark = pytest.mark.gpu


def _stream():
    return B.ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _attention_case(seed, b, n, hq, hkv, d, causal):
    """Gradients from both entry points (plus the inputs) for one problem."""
    import attention_fab_forward_amd as fab
    x = {t: random_array(seed + i, (b, n, hq if t in ("q", "do") else hkv, d), 1.0, "bf16")
         for i, t in enumerate(("q", "k", "v", "do"))}
    q, k, v, do = (to_device(x[t], "bf16") for t in ("q", "k", "v", "do"))
    scale = float(np.float32(d ** -0.5))
    o, lse = fab.forward(q, k, v, "softmax", causal, scale)
    plan = B.attention_plan(q, k, v, causal, scale, o=o)
    P = B._ptr
    # caller workspace full of 0xff bytes: the result must not depend on its contents
    ws = torch.full((max(plan.bwd_workspace, 1),), 255, dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(t) for t in (q, k, v)]
    plan.backward_raw(P(q), P(k), P(v), P(o), P(lse), P(do), *(P(t) for t in ref), P(ws),
                      plan.bwd_workspace, _stream())
    got = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    plan.backward_noalloc_raw(P(q), P(k), P(v), P(o), P(lse), P(do), *(P(t) for t in got),
                              _stream())
    torch.cuda.synchronize()
    return x, scale, ref, got


def _check_attention(x, scale, causal, ref, got, label):
    print(f"{label}: noalloc vs workspace entry point", flush=True)
    for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(r, g), f"{label} {name}: fab_backward_noalloc differs from fab_backward"
    rq, rk, rv = attention_backward(x["q"], x["k"], x["v"], x["do"], scale, causal)
    fq, fk = grad_floors(x, scale, causal)
    assert_close(f"{label} dQ", to_host(got[0]), rq, "bf16", floor=fq)
    assert_close(f"{label} dK", to_host(got[1]), rk, "bf16", floor=fk)
    assert_close(f"{label} dV", to_host(got[2]), rv, "bf16")


def test_noalloc_attention_two_calls_second_smaller():
    big = (901, 2, 1000, 8, 2, 128, True)
    small = (911, 1, 300, 4, 4, 64, False)
    for label, case in (("first call (b 2, n 1000, 8/2 heads, d 128, causal)", big),
                        ("second call (b 1, n 300, 4 heads, d 64, full)", small)):
        x, scale, ref, got = _attention_case(*case)
        _check_attention(x, scale, case[-1], ref, got, label)


def test_noalloc_mlp_then_attention():
    """The GeLU MLP (whose backward workspace holds packed operands and
    partial sums) through the same scratch, then a smaller attention call."""
    import attention_fab_forward_amd as fab
    m, k, n, p = 256, 256, 512, 128
    x = {"a": random_array(921, (m, k), 0.5, "bf16"), "bt": random_array(922, (n, k), 0.1, "bf16"),
         "c": random_array(923, (n, p), 0.1, "bf16"), "do": random_array(924, (m, p), 1.0, "bf16")}
    a, bt, c, do = (to_device(x[t], "bf16") for t in ("a", "bt", "c", "do"))
    plan = B.mlp_plan(a, bt, c, 1.0)
    assert plan.bwd_workspace <= 32 << 20
    P = B._ptr
    ws = torch.full((plan.bwd_workspace,), 255, dtype=torch.uint8, device="cuda")
    ref = [torch.empty_like(t) for t in (a, bt, c)]
    plan.backward_raw(P(a), P(bt), P(c), None, None, P(do), *(P(t) for t in ref), P(ws),
                      plan.bwd_workspace, _stream())
    got = [torch.full_like(t, float("nan")) for t in (a, bt, c)]
    plan.backward_noalloc_raw(P(a), P(bt), P(c), None, None, P(do), *(P(t) for t in got),
                              _stream())
    torch.cuda.synchronize()
    print("mlp: noalloc vs workspace entry point", flush=True)
    for name, r, g in zip(("dA", "dBt", "dC"), ref, got):
        assert torch.equal(r, g), f"mlp {name}: fab_backward_noalloc differs from fab_backward"
    del fab
    case = (931, 1, 200, 2, 1, 128, True)
    xa, scale, ref, got = _attention_case(*case)
    _check_attention(xa, scale, True, ref, got, "attention after the MLP (b 1, n 200, 2/1 heads)")


def test_noalloc_refuses_oversized_problem():
    """A problem whose workspace exceeds the static scratch is refused with
    FAB_ERR_WORKSPACE_TOO_SMALL before anything is launched."""
    prob = B.make_problem(B.SOFTMAX, B.BF16, 1, 64, 64, 1 << 17, 1 << 17, 128, 128, 0.088, True)
    plan = B.Plan(prob)
    good = B.ctypes.c_void_p(0x10000)
    st = B.lib().fab_backward_noalloc(plan._ptr, *([good] * 9), _stream())
    assert B.STATUS[st] == "FAB_ERR_WORKSPACE_TOO_SMALL"
