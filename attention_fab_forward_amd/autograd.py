"""torch.autograd wrappers over the C ABI, saving only what the recompute
backward needs.

Attention saves (Q, K, V, O, LSE): the n x n probabilities are rebuilt tile by
tile in the backward.  The GeLU MLP saves only its inputs (A, Bt, C): the
m x n pre-activation H and G = GeLU(H) are recomputed in the backward instead
of being kept between the passes -- the sequence-aware activation
checkpointing of "AutoSP" (section 2.B: rematerialise the linear / MLP
activations, whose share of the work shrinks as the sequence grows, while
attention keeps only its output).

AttentionMlpBlock chains the two: attention over (q, k, v), then the MLP on
the attention output's rows, y = GeLU(scale O W1^T) W2 with O viewed as
[b n, hq d].  Its activation memory between the passes is Q, K, V, O, LSE;
`saved_activation_bytes` measures it (and that of any other callable) from
the tensors autograd actually keeps.

All compute runs in libfab.so; these are argument marshalling only.
"""
import torch

from . import _binding as B


class FabAttentionFn(torch.autograd.Function):
    """O = softmax(scale Q K^T [+ causal mask]) V; saves Q, K, V, O, LSE."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = B.forward(q, k, v, "softmax", causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = B.backward(q, k, v, o, lse, do.contiguous(), "softmax", ctx.causal,
                                ctx.scale)
        return dq, dk, dv, None, None


class FabGeluMlpFn(torch.autograd.Function):
    """O = GeLU(scale A Bt^T) C; saves A, Bt, C only (H is recomputed)."""

    @staticmethod
    def forward(ctx, a, bt, c, scale):
        o, _ = B.forward(a, bt, c, "gelu", scale=scale)
        ctx.save_for_backward(a, bt, c)
        ctx.scale = scale
        return o

    @staticmethod
    def backward(ctx, do):
        a, bt, c = ctx.saved_tensors
        da, dbt, dc = B.backward(a, bt, c, None, None, do.contiguous(), "gelu",
                                 scale=ctx.scale)
        return da, dbt, dc, None


def attention(q, k, v, causal=False, scale=None):
    """q [b, m, hq, d], k / v [b, n, hkv, d] (bf16 or fp32, d in {64, 128})."""
    if scale is None:
        scale = 1.0 / float(q.shape[3]) ** 0.5
    return FabAttentionFn.apply(q, k, v, bool(causal), float(scale))


def gelu_mlp(a, bt, c, scale=1.0):
    """a [m, k], bt [n, k], c [n, p] bf16; k and p multiples of 64, <= 1024."""
    return FabGeluMlpFn.apply(a, bt, c, float(scale))


class AttentionMlpBlock(torch.nn.Module):
    """Attention followed by the GeLU MLP on its output rows.

    w1: [ffn, hq d] (the nn.Linear weight of the first product, i.e. Bt),
    w2: [ffn, out] (C).  hq d and out must be multiples of 64, at most 1024.
    """

    def __init__(self, hidden, ffn, out, device="cuda", dtype=torch.bfloat16, seed=0):
        super().__init__()
        gen = torch.Generator(device="cpu")
        gen.manual_seed(seed)
        w1 = torch.randn((ffn, hidden), generator=gen) * hidden ** -0.5
        w2 = torch.randn((ffn, out), generator=gen) * ffn ** -0.5
        self.w1 = torch.nn.Parameter(w1.to(device=device, dtype=dtype))
        self.w2 = torch.nn.Parameter(w2.to(device=device, dtype=dtype))

    def forward(self, q, k, v, causal=True):
        b, n, hq, d = q.shape
        o = attention(q, k, v, causal)
        return gelu_mlp(o.reshape(b * n, hq * d), self.w1, self.w2).reshape(b, n, -1)


def saved_activation_bytes(fn, *args, exclude=()):
    """Runs fn(*args) under autograd and returns (output, bytes of the
    distinct tensor storages autograd saves for the backward), leaving out
    the storages of `exclude` (e.g. parameters)."""
    skip = {t.untyped_storage().data_ptr() for t in exclude}
    seen = {}

    def pack(t):
        st = t.untyped_storage()
        if st.data_ptr() not in skip:
            seen[st.data_ptr()] = st.nbytes()
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        out = fn(*args)
    return out, sum(seen.values())
