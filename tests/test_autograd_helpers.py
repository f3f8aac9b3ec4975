"""CPU checks of the activation-memory counter used by the benchmark: it sums
distinct storages that autograd saves, once per storage, minus exclusions."""
import torch

from attention_fab_forward_amd.autograd import saved_activation_bytes


def test_counts_each_saved_storage_once():
    x = torch.randn(8, 16, requires_grad=True)
    w = torch.randn(16, 4, requires_grad=True)
    # x @ w saves x and w; (x @ w).exp() saves its output; x.view() shares x
    out, nbytes = saved_activation_bytes(lambda: (x.view(8, 16) @ w).exp() + (x @ w))
    assert nbytes == x.numel() * 4 + w.numel() * 4 + 8 * 4 * 4
    _, without_w = saved_activation_bytes(lambda: x @ w, exclude=(w,))
    assert without_w == x.numel() * 4
    assert out.shape == (8, 4)


def test_nothing_saved_without_grad():
    x = torch.randn(4, 4)
    _, nbytes = saved_activation_bytes(lambda: (x @ x).exp())
    assert nbytes == 0
