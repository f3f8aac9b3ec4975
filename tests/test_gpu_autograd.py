"""GPU parity of the autograd wrappers (attention, GeLU MLP and the chained
attention + MLP block) against the oracle's gradients, and of what they keep
between the passes: Q, K, V, O, LSE for attention, only the inputs for the
MLP (its intermediate is recomputed)."""
import numpy as np
import pytest

from attention_fab_forward_amd.inputs import random_array
from oracle import attention_backward, attention_forward, mlp_backward, mlp_forward
from fab_testutil import assert_close, grad_floors, to_device, to_host

pytestmark = pytest.mark.gpu


def leaf(x, dtype):
    return to_device(x, dtype).requires_grad_(True)


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 64, False),
                                            ("f32", 64, True)])
def test_attention_function_grads(dtype, d, causal):
    from attention_fab_forward_amd import autograd as AG
    b, n, hq, hkv = 2, 160, 4, 2
    q = random_array(8100, (b, n, hq, d), 1.0, dtype)
    k = random_array(8101, (b, n, hkv, d), 1.0, dtype)
    v = random_array(8102, (b, n, hkv, d), 1.0, dtype)
    do = random_array(8103, (b, n, hq, d), 1.0, dtype)
    scale = float(np.float32(d ** -0.5))
    tq, tk, tv = leaf(q, dtype), leaf(k, dtype), leaf(v, dtype)
    o = AG.attention(tq, tk, tv, causal, scale)
    o.backward(to_device(do, dtype))
    ro, _ = attention_forward(q, k, v, scale, causal)
    rdq, rdk, rdv = attention_backward(q, k, v, do, scale, causal)
    assert_close("O", to_host(o.detach()), ro, dtype)
    fq, fk = grad_floors({"q": q, "k": k, "v": v, "do": do}, scale, causal, ro)
    for name, t, r, fl in (("dQ", tq, rdq, fq), ("dK", tk, rdk, fk), ("dV", tv, rdv, None)):
        assert_close(name, to_host(t.grad), r, dtype, floor=fl)


def test_gelu_mlp_function_grads():
    from attention_fab_forward_amd import autograd as AG
    m, k, n, p = 200, 256, 300, 128
    a = random_array(8200, (m, k), 0.5, "bf16")
    bt = random_array(8201, (n, k), 0.1, "bf16")
    c = random_array(8202, (n, p), 0.1, "bf16")
    do = random_array(8203, (m, p), 1.0, "bf16")
    ta, tb, tc = leaf(a, "bf16"), leaf(bt, "bf16"), leaf(c, "bf16")
    o = AG.gelu_mlp(ta, tb, tc, 0.7)
    o.backward(to_device(do, "bf16"))
    assert_close("O", to_host(o.detach()), mlp_forward(a, bt, c, 0.7), "bf16")
    for name, t, r in zip(("dA", "dBt", "dC"), (ta, tb, tc), mlp_backward(a, bt, c, do, 0.7)):
        assert_close(name, to_host(t.grad), r, "bf16")


def test_block_grads_match_chained_oracle():
    """Attention then MLP on its rows: gradients through the module equal the
    chain rule applied to the oracle's attention and MLP gradients."""
    import torch
    from attention_fab_forward_amd import autograd as AG
    b, n, hq, d, ffn, out = 1, 192, 2, 64, 256, 128
    q = random_array(8300, (b, n, hq, d), 1.0, "bf16")
    k = random_array(8301, (b, n, hq, d), 1.0, "bf16")
    v = random_array(8302, (b, n, hq, d), 1.0, "bf16")
    dy = random_array(8303, (b, n, out), 1.0, "bf16")
    blk = AG.AttentionMlpBlock(hq * d, ffn, out, seed=3)
    w1 = blk.w1.detach().float().cpu().numpy().astype(np.float64)
    w2 = blk.w2.detach().float().cpu().numpy().astype(np.float64)
    tq, tk, tv = leaf(q, "bf16"), leaf(k, "bf16"), leaf(v, "bf16")
    y = blk(tq, tk, tv, causal=True)
    y.backward(to_device(dy, "bf16"))
    scale = d ** -0.5
    ro, _ = attention_forward(q, k, v, scale, True)
    a = ro.reshape(b * n, hq * d)
    assert_close("y", to_host(y.detach()).reshape(b * n, out), mlp_forward(a, w1, w2), "bf16")
    da, dw1, dw2 = mlp_backward(a, w1, w2, dy.reshape(b * n, out).astype(np.float64))
    rdq, rdk, rdv = attention_backward(q, k, v, da.reshape(b, n, hq, d), scale, True)
    assert_close("dW1", to_host(blk.w1.grad), dw1, "bf16")
    assert_close("dW2", to_host(blk.w2.grad), dw2, "bf16")
    fq, fk = grad_floors({"q": q, "k": k, "v": v, "do": da.reshape(b, n, hq, d)}, scale, True, ro)
    for name, t, r, fl in (("dQ", tq, rdq, fq), ("dK", tk, rdk, fk), ("dV", tv, rdv, None)):
        assert_close(name, to_host(t.grad), r, "bf16", floor=fl)
    assert isinstance(y, torch.Tensor)


def test_saved_activations_are_inputs_output_and_lse():
    import torch
    from attention_fab_forward_amd import autograd as AG
    b, n, hq, d, ffn, out = 1, 256, 4, 128, 512, 256
    mk = lambda *sh: torch.randn(sh, device="cuda").to(torch.bfloat16).requires_grad_(True)
    q, k, v = mk(b, n, hq, d), mk(b, n, hq, d), mk(b, n, hq, d)
    blk = AG.AttentionMlpBlock(hq * d, ffn, out)
    _, saved = AG.saved_activation_bytes(blk, q, k, v, exclude=(blk.w1, blk.w2))
    tensor_bytes = b * n * hq * d * 2
    # Q, K, V, O (the MLP's A is a view of O) and the fp32 LSE; no n x n or
    # n x ffn tensor
    assert saved == 4 * tensor_bytes + b * hq * n * 4
    a = mk(b * n, hq * d)
    _, saved_mlp = AG.saved_activation_bytes(AG.gelu_mlp, a, blk.w1, blk.w2,
                                             exclude=(blk.w1, blk.w2))
    assert saved_mlp == b * n * hq * d * 2
