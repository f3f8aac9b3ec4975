"""GPU parity of the Ulysses exchange layout kernels (fab_ulysses_pack /
fab_ulysses_unpack) against the oracle, and of attention and its gradients
computed the Ulysses way: p ranks simulated on one GPU, the all-to-all done
as a plain tensor exchange between their buffers, attention run in place on
each rank's receive buffer through the C ABI."""
import numpy as np
import pytest

from attention_fab_forward_amd.inputs import random_array
from oracle import (all_to_all, attention_backward, attention_forward, ulysses_pack,
                    ulysses_unpack)
from fab_testutil import LSE_TOL, assert_close, grad_floors, to_device, to_host

pytestmark = pytest.mark.gpu

LAYOUTS = [  # b, n_local, heads, d, ranks, dtype
    (1, 64, 8, 128, 4, "bf16"),
    (2, 37, 8, 64, 8, "bf16"),    # one head per rank, ragged token count
    (1, 1, 4, 128, 4, "bf16"),    # a single token per rank
    (2, 16, 2, 128, 8, "bf16"),   # 2 heads over 8 ranks: each sent to 4 ranks
    (1, 33, 4, 64, 1, "bf16"),    # one rank: a reordering of the same tokens
    (3, 5, 6, 64, 3, "f32"),
    (2, 7, 3, 32, 3, "f32"),
    (1, 129, 32, 128, 8, "bf16"),
]


def exchange(sends):
    """The all-to-all with equal splits between simulated ranks."""
    import torch
    p = len(sends)
    return [torch.stack([sends[s][j] for s in range(p)]).contiguous() for j in range(p)]


@pytest.mark.parametrize("b,nl,h,d,p,dtype", LAYOUTS)
def test_pack_bit_exact(b, nl, h, d, p, dtype):
    import attention_fab_forward_amd as fab
    x = random_array(7000 + nl + h, (b, nl, h, d), 1.0, dtype)
    print(f"pack b={b} n_local={nl} H={h} d={d} p={p} {dtype}", flush=True)
    got = to_host(fab.ulysses_pack(to_device(x, dtype), p))
    np.testing.assert_array_equal(got, ulysses_pack(x.astype(np.float64), p))


def test_pack_strided_input():
    import attention_fab_forward_amd as fab
    b, nl, h, d, p = 2, 24, 8, 128, 4
    qkv = random_array(7100, (b, nl, 3, h, d), 1.0, "bf16")
    t = to_device(qkv, "bf16")[:, :, 1]  # the K part of a fused projection: strided rows
    assert not t.is_contiguous()
    got = to_host(fab.ulysses_pack(t, p))
    np.testing.assert_array_equal(got, ulysses_pack(qkv[:, :, 1].astype(np.float64), p))


@pytest.mark.parametrize("b,nl,h,d,p,dtype", LAYOUTS)
def test_unpack(b, nl, h, d, p, dtype):
    import torch
    import attention_fab_forward_amd as fab
    hl = h // p if h >= p else 1
    recv = random_array(7200 + nl + h, (p, nl, b, hl, d), 1.0, dtype)
    print(f"unpack b={b} n_local={nl} H={h} d={d} p={p} {dtype}", flush=True)
    # unpack into a strided view of a larger tensor; the rest must stay untouched
    big = torch.full((b, nl, 2, h, d), 7.0, dtype=torch.bfloat16 if dtype == "bf16"
                     else torch.float32, device="cuda")
    out = fab.ulysses_unpack(to_device(recv, dtype), h, out=big[:, :, 0])
    ref = ulysses_unpack(recv.astype(np.float64), h)
    got = to_host(out)
    assert np.all(to_host(big[:, :, 1]) == 7.0)
    if p <= h:  # one holder per head: a copy
        np.testing.assert_array_equal(got, ref)
    else:       # replicas summed in fp32 and rounded once
        rtol = 2.0 ** -7 if dtype == "bf16" else 1e-6
        assert np.all(np.abs(got - ref) <= rtol * np.abs(ref) + 1e-30), \
            float(np.max(np.abs(got - ref)))


FLOWS = [  # b, n, hq, hkv, d, p
    (1, 512, 8, 8, 128, 4),
    (2, 256, 8, 2, 64, 4),     # key/value heads 2 over 4 ranks: replicated
    (1, 384, 4, 1, 128, 4),    # one key/value head on every rank
    (1, 320, 8, 4, 128, 2),
]


def ulysses_flow(fab, q, k, v, p, scale, causal, do=None):
    """Forward (and backward when do is given) through pack / exchange /
    attention on the receive buffers / exchange / unpack."""
    import torch
    b, n, hq, d = q.shape
    hkv = k.shape[2]
    nl = n // p

    def shard_exchange(t):
        return exchange([fab.ulysses_pack(t[:, j * nl:(j + 1) * nl], p) for j in range(p)])

    rq, rk, rv = shard_exchange(q), shard_exchange(k), shard_exchange(v)
    hlq = rq[0].shape[3]
    o_send, lse_parts = [], []
    for j in range(p):
        obuf = torch.empty((p, nl, b, hlq, d), dtype=q.dtype, device=q.device)
        lse = torch.empty((b, hlq, n), dtype=torch.float32, device=q.device)
        fab.forward(*(fab.ulysses_sequence_view(r[j]) for r in (rq, rk, rv)), "softmax", causal,
                    scale, out=(fab.ulysses_sequence_view(obuf), lse))
        o_send.append(obuf)
        lse_parts.append(lse)
    o_recv = exchange(o_send)
    o = torch.cat([fab.ulysses_unpack(o_recv[r], hq) for r in range(p)], dim=1)
    if do is None:
        return o, lse_parts, None
    rdo = shard_exchange(do)
    sends = {"dq": [], "dk": [], "dv": []}
    for j in range(p):
        grads = fab.backward(*(fab.ulysses_sequence_view(r[j]) for r in (rq, rk, rv)),
                             fab.ulysses_sequence_view(o_send[j]), lse_parts[j],
                             fab.ulysses_sequence_view(rdo[j]), "softmax", causal, scale)
        for name, g in zip(("dq", "dk", "dv"), grads):
            # gradients take the receive buffers' layout: [n, b, Hl, d] in memory
            sends[name].append(g.permute(1, 0, 2, 3).contiguous().view(p, nl, b, g.shape[2], d))
    out = {}
    for name, heads in (("dq", hq), ("dk", hkv), ("dv", hkv)):
        recv = exchange(sends[name])
        out[name] = torch.cat([fab.ulysses_unpack(recv[r], heads) for r in range(p)], dim=1)
    return o, lse_parts, out


@pytest.mark.parametrize("b,n,hq,hkv,d,p", FLOWS)
def test_ulysses_attention_forward(b, n, hq, hkv, d, p):
    import attention_fab_forward_amd as fab
    dtype, causal = "bf16", True
    q = random_array(7300 + n, (b, n, hq, d), 1.0, dtype)
    k = random_array(7301 + n, (b, n, hkv, d), 1.0, dtype)
    v = random_array(7302 + n, (b, n, hkv, d), 1.0, dtype)
    scale = float(np.float32(d ** -0.5))
    print(f"ulysses forward b={b} n={n} hq={hq} hkv={hkv} d={d} p={p}", flush=True)
    o, lses, _ = ulysses_flow(fab, *(to_device(x, dtype) for x in (q, k, v)), p, scale, causal)
    ro, rl = attention_forward(q, k, v, scale, causal)
    assert_close("O (Ulysses)", to_host(o), ro, dtype)
    hl = hq // p
    for j in range(p):
        err = np.max(np.abs(lses[j].cpu().numpy() - rl[:, j * hl:(j + 1) * hl]))
        assert err <= LSE_TOL[dtype], f"lse of rank {j}: {err:.3e}"


@pytest.mark.parametrize("b,n,hq,hkv,d,p", FLOWS)
def test_ulysses_attention_backward(b, n, hq, hkv, d, p):
    import attention_fab_forward_amd as fab
    dtype, causal = "bf16", True
    q = random_array(7400 + n, (b, n, hq, d), 1.0, dtype)
    k = random_array(7401 + n, (b, n, hkv, d), 1.0, dtype)
    v = random_array(7402 + n, (b, n, hkv, d), 1.0, dtype)
    do = random_array(7403 + n, (b, n, hq, d), 1.0, dtype)
    scale = float(np.float32(d ** -0.5))
    print(f"ulysses backward b={b} n={n} hq={hq} hkv={hkv} d={d} p={p}", flush=True)
    _, _, g = ulysses_flow(fab, *(to_device(x, dtype) for x in (q, k, v)), p, scale, causal,
                           do=to_device(do, dtype))
    rdq, rdk, rdv = attention_backward(q, k, v, do, scale, causal)
    fq, fk = grad_floors({"q": q, "k": k, "v": v, "do": do}, scale, causal)
    assert_close("dQ (Ulysses)", to_host(g["dq"]), rdq, dtype, floor=fq)
    assert_close("dK (Ulysses)", to_host(g["dk"]), rdk, dtype, floor=fk)
    assert_close("dV (Ulysses)", to_host(g["dv"]), rdv, dtype)


def test_full_size_rank_share_bit_exact():
    """The size the benchmark times (x 1 x 16384 x 32 x 128 bf16, 8 ranks: one
    rank of the 4-head, 131072-token share): every element of pack and of
    unpack against the oracle."""
    import attention_fab_forward_amd as fab
    b, nl, h, d, p = 1, 16384, 32, 128, 8
    x = random_array(7500, (b, nl, h, d), 1.0, "bf16")
    print(f"full-size pack / unpack b={b} n_local={nl} H={h} d={d} p={p}", flush=True)
    send = fab.ulysses_pack(to_device(x, "bf16"), p)
    ref = ulysses_pack(x, p)
    assert np.array_equal(send.float().cpu().numpy(), ref)
    back = fab.ulysses_unpack(send, h)
    assert np.array_equal(back.float().cpu().numpy(), ulysses_unpack(ref, h))
