#!/usr/bin/env python3
"""Benchmark of the fused two-matmul block O = f(A.B).C on one MI355X.

Step = one forward + backward pass of causal softmax attention, bf16,
batch 1, 32 heads, n = 32768, d = 128 (scale 1/sqrt(128)), on seeded synthetic
N(0, 1) inputs already resident in device memory.  Throughput is algorithmic
TFLOP/s: forward 4*d flops and backward 10*d flops (its five products, one
recomputation of S included) per unmasked (query, key) pair, n(n+1)/2 pairs
per head.

The headline step is timed over K steps with events between steps only; a
second pass over K steps records HIP events around every kernel on the launch
stream (the per-kernel durations the roofline entry uses).  Also reported on
the same line: the GPU clock before and after (amd-smi), peak device memory
versus sequence length for the long-context grouped-query geometry (with the
HIP free-memory delta as a cross-check), the other workloads on their seeded
inputs, a GeLU-MLP measurement with the 256 MB last-level cache flushed
between repetitions, and the CPU oracle timed on bounded samples of the
workloads, with the time a full run would take extrapolated from them.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk, dense bf16 MFMA
HBM_PEAK_GBS = 8000.0
F32_MATRIX_PEAK_TFLOPS = 157.3  # dense fp32 MFMA
WORKLOAD = "attn_causal_bf16_h32_n32768_d128"
MLP_WORKLOAD = "mlp_gelu_m4096_k1024_n4096_p1024"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attention_flops(w):
    pairs = w.seq * (w.seq + 1) // 2 if w.causal else w.seq * w.seq
    unit = pairs * w.heads_q * w.batch
    return 4 * w.d * unit, 10 * w.d * unit, unit


def device_inputs(w, torch):
    from attention_fab_forward_amd.inputs import attention_inputs
    x = attention_inputs(w)
    dev = {}
    for name in ("q", "k", "v", "do"):
        dev[name] = torch.from_numpy(x[name]).to(torch.bfloat16).cuda()
    return x, dev


def time_attention(w, steps, warmup, torch, fab_binding):
    x, t = device_inputs(w, torch)
    plan = fab_binding.attention_plan(t["q"], t["k"], t["v"], True, w.scale())
    log(f"plan: {plan.describe()}")
    b, n, hq, d = t["q"].shape
    o = torch.empty_like(t["q"])
    lse = torch.empty((b, hq, n), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["k"]), torch.empty_like(t["v"])
    ws = torch.empty(max(plan.bwd_workspace, plan.fwd_workspace, 1), dtype=torch.uint8,
                     device="cuda")
    P = fab_binding._ptr
    stream = torch.cuda.current_stream()
    sp = fab_binding.ctypes.c_void_p(stream.cuda_stream)

    def fwd():
        plan.forward_raw(P(t["q"]), P(t["k"]), P(t["v"]), P(o), P(lse), P(ws), plan.fwd_workspace,
                         sp)

    def bwd():
        plan.backward_raw(P(t["q"]), P(t["k"]), P(t["v"]), P(o), P(lse), P(t["do"]), P(dq),
                          P(dk), P(dv), P(ws), plan.bwd_workspace, sp)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # main timed region: K full steps, an event between steps (per-step spread)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fwd()
        bwd()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = ev[0].elapsed_time(ev[-1]) / steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))

    # second timed region: the same K steps with a HIP event pair around every
    # kernel (on the launch stream), for the per-kernel durations
    plan.set_timing(True)
    plan.reset_kernel_times()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fwd()
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    kernels = plan.kernel_times()
    plan.set_timing(False)
    step_ms_kernel_pass = e0.elapsed_time(e1) / steps

    def spread(fn):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(stream)
        for i in range(steps):
            fn()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        d = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        return evs[0].elapsed_time(evs[-1]) / steps, d

    fwd_ms, fwd_d = spread(fwd)  # forward alone (timing off)
    bwd_ms, bwd_d = spread(bwd)  # backward alone, on the fixed forward outputs
    stats = lambda d: {"median": d[len(d) // 2], "min": d[0], "max": d[-1]}
    return {"step_ms": step_ms, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms, "wall_s": wall,
            "kernels": kernels, "inputs": x, "step_ms_kernel_pass": step_ms_kernel_pass,
            "spread_ms": {"step": stats(per_step), "fwd": stats(fwd_d), "bwd": stats(bwd_d)}}


def time_workload(key, reps, torch, fab, back_to_back=False):
    """Forward and backward time of another attention configuration on its
    seeded inputs (the same PCG64 draws the tests and the oracle use).

    Outputs and workspace are allocated once; each repetition enqueues the
    plan's raw forward and backward calls between events (device time; the
    reported figures are the medians over `reps`, with min and max); a second
    pass records HIP events around every kernel (kernel durations alone).
    back_to_back (latency-bound workloads of microseconds): the reps are
    enqueued back to back between two events instead, so the host's enqueue
    time between calls is hidden, and the figures are means."""
    from attention_fab_forward_amd import _binding as B
    from attention_fab_forward_amd.inputs import WORKLOADS, attention_inputs
    w = WORKLOADS[key]
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = attention_inputs(w)
    q, k, v, do = (torch.from_numpy(x[t]).to(dt).cuda() for t in ("q", "k", "v", "do"))
    del x
    plan = B.attention_plan(q, k, v, w.causal, w.scale())
    o, lse = torch.empty_like(q), torch.empty((w.batch, w.heads_q, w.seq), dtype=torch.float32,
                                              device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(plan.bwd_workspace, plan.fwd_workspace, 1), dtype=torch.uint8,
                     device="cuda")
    P = B._ptr
    stream = torch.cuda.current_stream()
    sp = B.ctypes.c_void_p(stream.cuda_stream)

    def fwd():
        plan.forward_raw(P(q), P(k), P(v), P(o), P(lse), P(ws), plan.fwd_workspace, sp)

    def bwd():
        plan.backward_raw(P(q), P(k), P(v), P(o), P(lse), P(do), P(dq), P(dk), P(dv), P(ws),
                          plan.bwd_workspace, sp)

    fwd()
    bwd()
    torch.cuda.synchronize()
    fms, bms = [], []
    for _ in range(1 if back_to_back else reps):
        if back_to_back:
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            for _ in range(reps):
                fwd()
            e[1].record(stream)
            for _ in range(reps):
                bwd()
            e[2].record(stream)
            torch.cuda.synchronize()
            fms.append(e[0].elapsed_time(e[1]) / reps)
            bms.append(e[1].elapsed_time(e[2]) / reps)
            break
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
        torch.cuda.synchronize()
        fms.append(e[0].elapsed_time(e[1]))
        bms.append(e[1].elapsed_time(e[2]))
    fms.sort()
    bms.sort()
    fm, bm = fms[len(fms) // 2], bms[len(bms) // 2]
    plan.set_timing(True)
    plan.reset_kernel_times()
    for _ in range(reps):
        fwd()
        bwd()
    kernels = {name: tot / cnt for name, (cnt, tot) in plan.kernel_times().items()}
    plan.set_timing(False)
    fwd_fl, bwd_fl, _ = attention_flops(w)
    family = plan.describe()
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    extra = {}
    if w.dtype == "f32":
        extra = {"fwd_pct_f32_matrix_peak": 100.0 * fwd_fl / fm / 1e9 / F32_MATRIX_PEAK_TFLOPS,
                 "fwd_bwd_pct_f32_matrix_peak":
                     100.0 * (fwd_fl + bwd_fl) / (fm + bm) / 1e9 / F32_MATRIX_PEAK_TFLOPS}
    return {**extra, "plan": family, "fwd_ms": fm, "bwd_ms": bm, "fwd_us": 1e3 * fm,
            "bwd_us": 1e3 * bm,
            "fwd_ms_min_max": [fms[0], fms[-1]], "bwd_ms_min_max": [bms[0], bms[-1]],
            "dtype": w.dtype, "fwd_tflops": fwd_fl / fm / 1e9,
            "fwd_bwd_tflops": (fwd_fl + bwd_fl) / (fm + bm) / 1e9,
            "fwd_bwd_pct_bf16_peak": 100.0 * (fwd_fl + bwd_fl) / (fm + bm) / 1e9 / BF16_PEAK_TFLOPS,
            "kernels_avg_ms": kernels, "reps": reps,
            "timing": ("device time per call, calls enqueued back to back between two events "
                       "(mean)" if back_to_back else
                       "device time per call (events around each call), median of reps"),
            "inputs": "seeded PCG64 draws (the workload's own seeds), rounded to the dtype"}


def kernel_flops(w):
    """Algorithmic flops each attention kernel carries per launch."""
    _, _, unit = attention_flops(w)
    d = w.d
    return {
        "attn_fwd_bf16": 4 * d * unit,        # S = QK^T and O = PV
        "attn_bwd_dkdv_bf16": 8 * d * unit,   # S (recompute), dP, dV, dK
        "attn_bwd_dq_bf16": 2 * d * unit,     # dQ (its S, dP recomputes are extra work)
        "attn_bwd_prep": 0,
    }


def kernel_bytes(w):
    """Algorithmic HBM bytes of the memory-bound preprocessing kernel."""
    rows = w.batch * w.heads_q * w.seq
    # reads O and dO (bf16) and the LSE; writes -D and LSE * log2(e) (fp32)
    return {"attn_bwd_prep": rows * w.d * 2 * 2 + rows * 4 * 3}


# rocprofv3 names and source files of the kernels bench.py reports
ROCPROF_NAMES = {
    "attn_fwd_bf16": ("attn_fwd_bf16_kernel<128, true>", "attn_fwd.hip"),
    "attn_bwd_dkdv_bf16": ("attn_dkdv_bf16_kernel<128, true>", "attn_bwd.hip"),
    "attn_bwd_dq_bf16": ("attn_dq_bf16_kernel<128, true, 1, true>", "attn_bwd.hip"),
    "attn_bwd_prep": ("attn_bwd_prep_bf16_kernel<128>", "attn_bwd.hip"),
    "mlp_fwd": ("mlp_fwd_kernel<1024, 1024>", "mlp.hip"),
    "mlp_bwd_da": ("mlp_bwd_da_kernel<1024, 1024>", "mlp.hip"),
    "mlp_bwd_dbt": ("mlp_bwd_dbt_kernel<1024, 1024>", "mlp.hip"),
    "mlp_bwd_dc": ("mlp_bwd_dc_kernel<1024, 1024>", "mlp.hip"),
}


def source_hash(src):
    """sha256[:16] over a kernel's source file and the shared device headers."""
    import hashlib
    csrc = os.path.join(ROOT, "attention_fab_forward_amd", "csrc")
    h = hashlib.sha256()
    for name in (src, "fab_device.h", "fab_internal.h"):
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary of the
    workload (default: the benchmarked one), or None when that summary is
    missing or was taken from different kernel sources."""
    if kernel not in ROCPROF_NAMES:
        return None
    rname, src = ROCPROF_NAMES[kernel]
    path = os.path.join(ROOT, "profiles", f"{workload or WORKLOAD}.hbm_counters.txt")
    if not os.path.exists(path):
        return None
    want = f"{src}:{source_hash(src)}"
    with open(path) as fh:
        for line in fh:
            if line.startswith(rname) and line.rstrip().endswith(want):
                return float(line.split()[-2])
    return None


def measured_mfma(kernel):
    """MFMA counters of a kernel from the committed rocprofv3 summary (median
    dispatch): share of SIMD cycles its MFMA unit was busy, the GPU-active
    clock, and executed bf16 MFMA flops per dispatch; None when the summary is
    missing or was taken from different kernel sources."""
    if kernel not in ROCPROF_NAMES:
        return None
    rname, src = ROCPROF_NAMES[kernel]
    path = os.path.join(ROOT, "profiles", "attn_mlp_bf16.mfma_counters.txt")
    if not os.path.exists(path):
        return None
    want = f"{src}:{source_hash(src)}"
    with open(path) as fh:
        for line in fh:
            if line.startswith(rname) and line.rstrip().endswith(want):
                f = line[len(rname):].split()
                # columns: dispatches, avg_ms, bf16_flops, clock_ghz, mfma_busy, mfma_util, ...
                return {"mfma_busy": float(f[4]) / 100.0, "clock_ghz": float(f[3]),
                        "bf16_flops_executed": float(f[2])}
    return None


def peak_hbm_sweep(torch, fab, exps=range(12, 21), hq=2, hkv=1):
    """Peak device memory of forward + backward versus n, causal bf16, d = 128
    (default: the long-context geometry, 2 query heads and 1 kv head).  The
    library allocates nothing, so torch's peak counter sees every byte."""
    out = []
    for e in exps:
        n = 1 << e
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        free0 = torch.cuda.mem_get_info()[0]  # hipMemGetInfo
        q = torch.randn(1, n, hq, 128, device="cuda", dtype=torch.bfloat16)
        k = torch.randn(1, n, hkv, 128, device="cuda", dtype=torch.bfloat16)
        v = torch.randn(1, n, hkv, 128, device="cuda", dtype=torch.bfloat16)
        do = torch.randn_like(q)
        o, lse = fab.forward(q, k, v, "softmax", True)
        fwd_peak = torch.cuda.max_memory_allocated() - base
        grads = fab.backward(q, k, v, o, lse, do, "softmax", True)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        # device memory that left the free pool over the call (torch's
        # reserved blocks, rounded up to its allocation granules): at least
        # the peak, and no more than a granule per tensor above it
        used = free0 - torch.cuda.mem_get_info()[0]
        out.append({"n": n, "fwd_peak_bytes": int(fwd_peak), "fwd_bwd_peak_bytes": int(peak),
                    "hip_free_delta_bytes": int(used)})
        del q, k, v, do, o, lse, grads
    ns = [r["n"] for r in out]
    ys = [r["fwd_bwd_peak_bytes"] for r in out]
    # least-squares a + b n and the largest relative residual
    mn = sum(ns) / len(ns)
    my = sum(ys) / len(ys)
    b = sum((x - mn) * (y - my) for x, y in zip(ns, ys)) / sum((x - mn) ** 2 for x in ns)
    a = my - b * mn
    resid = max(abs(y - (a + b * x)) / y for x, y in zip(ns, ys))
    ratios = [ys[i + 1] / ys[i] for i in range(len(ys) - 1)]
    hip = [r["hip_free_delta_bytes"] / r["fwd_bwd_peak_bytes"] for r in out]
    return {"geometry": f"causal, {hq} query heads / {hkv} kv heads, d=128, bf16, fwd+bwd",
            "points": out, "bytes_per_token": b, "max_rel_residual_linear_fit": resid,
            "doubling_ratios": ratios,
            "hip_free_delta_over_peak": {"min": min(hip), "max": max(hip)}}


def time_merge(w, reps, torch, fab):
    """HBM rate of the merge of two partial results (fab_merge) at the size of
    the benchmarked attention output: reads two O and two LSE, writes one of
    each."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    shape = (w.batch, w.seq, w.heads_q, w.d)
    oa = torch.randn(shape, device="cuda", generator=gen).to(torch.bfloat16)
    ob = torch.randn(shape, device="cuda", generator=gen).to(torch.bfloat16)
    la = torch.randn((w.batch, w.heads_q, w.seq), device="cuda", generator=gen)
    lb = torch.randn((w.batch, w.heads_q, w.seq), device="cuda", generator=gen)
    oo, lo = torch.empty_like(oa), torch.empty_like(la)
    fab.merge(oa, la, ob, lb, out=(oo, lo))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fab.merge(oa, la, ob, lb, out=(oo, lo))
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = 3 * oa.numel() * 2 + 3 * la.numel() * 4
    return {"ms": ms, "bytes": nbytes, "gbs": nbytes / ms / 1e6,
            "frac_hbm_peak": nbytes / ms / 1e6 / HBM_PEAK_GBS,
            "shape": f"O {list(shape)} bf16, LSE {[w.batch, w.heads_q, w.seq]} fp32"}


def exp_bound(torch, fab_binding, pairs_fwd):
    """Secondary bound of the softmax: the rate of exp2(fma(x, a, b)) (one per
    probability) from the library's probe, timed with events on torch's
    stream, and the time the benchmarked step's exponentials would take at
    that rate (forward: one per unmasked pair and head; backward: two, the dK/dV
    and dQ kernels each rebuilding P)."""
    blocks, iters = 2048, 2048
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    fab_binding.exp_probe(blocks, iters, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    count = 0
    for _ in range(5):
        count += fab_binding.exp_probe(blocks, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    rate = count / (e0.elapsed_time(e1) / 1e3)
    return {"exp_per_s": rate, "exp_bound_ms_fwd": pairs_fwd / rate * 1e3,
            "exp_bound_ms_fwd_bwd": 3 * pairs_fwd / rate * 1e3,
            "probe": f"{blocks} x 256 lanes x {iters} steps x 8 chains of exp2(fma)"}


def time_ulysses(w, reps, torch, fab, ranks=8):
    """HBM rate of the two layout kernels around the Ulysses exchanges, for a
    rank of a `ranks`-way group whose share after the exchange is the
    benchmarked attention workload: pack reads this rank's n / ranks tokens
    of all heads and writes the send buffer; unpack reads the return
    buffer and writes the tokens back (each byte read once, written once)."""
    heads = w.heads_q * ranks
    nl = w.seq // ranks
    gen = torch.Generator(device="cuda")
    gen.manual_seed(78)
    x = torch.randn((w.batch, nl, heads, w.d), device="cuda", generator=gen).to(torch.bfloat16)
    send = fab.ulysses_pack(x, ranks)
    back = torch.empty_like(x)
    out = {}
    for name, fn in (("pack", lambda: fab.ulysses_pack(x, ranks, out=send)),
                     ("unpack", lambda: fab.ulysses_unpack(send, heads, out=back))):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = 2 * x.numel() * 2
        out[name] = {"ms": ms, "bytes": nbytes, "gbs": nbytes / ms / 1e6,
                     "frac_hbm_peak": nbytes / ms / 1e6 / HBM_PEAK_GBS}
    out["shape"] = (f"x {[w.batch, nl, heads, w.d]} bf16 over {ranks} ranks "
                    f"(exchange buffer {list(send.shape)})")
    return out


def eager_attention_mlp(torch, q, k, v, w1t, w2, causal, scale, part="both", a_in=None):
    """The same attention + GeLU MLP block composed from plain PyTorch ops,
    used only to count the activations autograd keeps when nothing is
    recomputed (scores, probabilities, H, GeLU(H)).  Forward only; every
    batched bf16 product gets contiguous operands, the softmax runs in fp32.
    part: "attention" (returns O), "mlp" (applies the MLP to a_in) or "both"."""
    import torch.nn.functional as F
    if part in ("attention", "both"):
        b, n, hq, d = q.shape
        qh = q.permute(0, 2, 1, 3).contiguous()
        kt = k.permute(0, 2, 3, 1).contiguous()
        vh = v.permute(0, 2, 1, 3).contiguous()
        sc = torch.matmul(qh, kt).float() * scale
        if causal:
            mask = torch.triu(torch.ones(n, n, dtype=torch.bool, device=q.device), 1)
            sc = sc.masked_fill(mask, float("-inf"))
        pr = torch.softmax(sc, dim=-1).to(q.dtype)
        o = torch.matmul(pr, vh).permute(0, 2, 1, 3)
        if part == "attention":
            return o
        a_in = o.reshape(b * n, hq * d)
    return torch.matmul(F.gelu(torch.matmul(a_in, w1t)), w2)


def activation_memory(torch, fab_pkg):
    """Bytes autograd keeps between forward and backward for the attention +
    GeLU MLP block (attention over 8 heads of d = 128 on 4096 tokens, then
    the MLP 1024 -> 4096 -> 1024 on its rows), the fused kernels' path vs the
    plain composition; weights are not counted."""
    from attention_fab_forward_amd import autograd as AG
    b, n, hq, d, ffn, out = 1, 4096, 8, 128, 4096, 1024
    gen = torch.Generator(device="cuda")
    gen.manual_seed(79)
    mk = lambda *sh: (torch.randn(sh, device="cuda", generator=gen) * 0.5).to(
        torch.bfloat16).requires_grad_(True)
    q, k, v = mk(b, n, hq, d), mk(b, n, hq, d), mk(b, n, hq, d)
    blk = AG.AttentionMlpBlock(hq * d, ffn, out)
    w1t = blk.w1.detach().t().contiguous().requires_grad_(True)
    w2 = blk.w2.detach().clone().requires_grad_(True)
    scale = d ** -0.5
    a = mk(b * n, hq * d)
    params = (blk.w1, blk.w2, w1t, w2)
    res = {}
    _, res["fab_attention"] = AG.saved_activation_bytes(AG.attention, q, k, v, True, scale)
    _, res["fab_mlp"] = AG.saved_activation_bytes(AG.gelu_mlp, a, blk.w1, blk.w2,
                                                  exclude=params)
    _, res["fab_block"] = AG.saved_activation_bytes(blk, q, k, v, exclude=params)
    _, res["eager_attention"] = AG.saved_activation_bytes(
        lambda: eager_attention_mlp(torch, q, k, v, w1t, w2, True, scale, "attention"))
    _, res["eager_mlp"] = AG.saved_activation_bytes(
        lambda: eager_attention_mlp(torch, q, k, v, w1t, w2, True, scale, "mlp", a),
        exclude=params)
    _, res["eager_block"] = AG.saved_activation_bytes(
        lambda: eager_attention_mlp(torch, q, k, v, w1t, w2, True, scale), exclude=params)
    torch.cuda.synchronize()
    res["ratio_attention"] = res["eager_attention"] / res["fab_attention"]
    res["ratio_mlp"] = res["eager_mlp"] / res["fab_mlp"]
    res["ratio_block"] = res["eager_block"] / res["fab_block"]
    res["shape"] = (f"b {b} n {n} heads {hq} d {d} causal bf16; MLP {hq * d} -> {ffn} -> {out}")
    return res


def time_mlp(steps, warmup, torch, fab_binding):
    from attention_fab_forward_amd.inputs import WORKLOADS, mlp_inputs
    w = WORKLOADS[MLP_WORKLOAD]
    x = mlp_inputs(w)
    t = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    plan = fab_binding.mlp_plan(t["a"], t["bt"], t["c"], 1.0)
    m, k = t["a"].shape
    n, p = t["bt"].shape[0], t["c"].shape[1]
    o = torch.empty((m, p), dtype=torch.bfloat16, device="cuda")
    da, dbt, dc = torch.empty_like(t["a"]), torch.empty_like(t["bt"]), torch.empty_like(t["c"])
    ws = torch.empty(max(plan.fwd_workspace, plan.bwd_workspace, 1), dtype=torch.uint8,
                     device="cuda")
    P = fab_binding._ptr
    stream = torch.cuda.current_stream()
    sp = fab_binding.ctypes.c_void_p(stream.cuda_stream)
    fwd = lambda: plan.forward_raw(P(t["a"]), P(t["bt"]), P(t["c"]), P(o), None, P(ws),
                                   plan.fwd_workspace, sp)
    bwd = lambda: plan.backward_raw(P(t["a"]), P(t["bt"]), P(t["c"]), None, None, P(t["do"]),
                                    P(da), P(dbt), P(dc), P(ws), plan.bwd_workspace, sp)
    # 512 MiB written between repetitions: the 32 MiB of operands (and the
    # workspace) cannot stay in the 256 MB last-level cache from one
    # repetition to the next, so each is timed from HBM
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    fms, sms = [], []
    for _ in range(steps):
        flush.fill_(1)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        fwd()
        e[1].record(stream)
        bwd()
        e[2].record(stream)
        torch.cuda.synchronize()
        fms.append(e[0].elapsed_time(e[1]))
        sms.append(e[0].elapsed_time(e[2]))
    fms.sort()
    sms.sort()
    fwd_ms, step_ms = fms[len(fms) // 2], sms[len(sms) // 2]
    # per-kernel durations: a separate pass with events around every kernel
    plan.set_timing(True)
    plan.reset_kernel_times()
    for _ in range(steps):
        flush.fill_(1)
        fwd()
        bwd()
    torch.cuda.synchronize()
    kernels = plan.kernel_times()
    plan.set_timing(False)
    del flush
    gemm = 2 * m * k * n
    fwd_fl, bwd_fl = 2 * gemm, 5 * gemm
    fwd_tf, step_tf = fwd_fl / fwd_ms / 1e9, (fwd_fl + bwd_fl) / step_ms / 1e9
    return {"workload": MLP_WORKLOAD, "fwd_ms": fwd_ms, "fwd_bwd_ms": step_ms,
            "fwd_ms_min_max": [fms[0], fms[-1]], "fwd_bwd_ms_min_max": [sms[0], sms[-1]],
            "fwd_tflops": fwd_tf, "fwd_bwd_tflops": step_tf,
            "fwd_pct_bf16_peak": 100.0 * fwd_tf / BF16_PEAK_TFLOPS,
            "fwd_bwd_pct_bf16_peak": 100.0 * step_tf / BF16_PEAK_TFLOPS,
            "timing": ("events around each repetition's forward and forward + backward "
                       "(median of reps), 512 MiB written between repetitions"),
            "kernels_avg_ms": {k_: v[1] / v[0] for k_, v in kernels.items()},
            "mfma_counters": {k_: measured_mfma(k_) for k_ in kernels if measured_mfma(k_)},
            "hbm_traffic_bytes": {k_: measured_traffic(k_, MLP_WORKLOAD) for k_ in kernels
                                  if measured_traffic(k_, MLP_WORKLOAD)}}


def oracle_rows_timed(w, x, seconds=None, rows_per_head=None, chunk=32, seed=0):
    """The oracle, unchanged, on a sample of query rows of a workload: chunks
    of `chunk` consecutive rows (forward rows and their backward work) at
    seeded, uniformly random positions over all heads, run by a pool of host
    threads (one BLAS thread each) until `seconds` have passed, or
    `rows_per_head` rows of every head.  The oracle materialises full-width
    rows, so every row costs the same and the full run's time is the sample's
    time times (all rows / sampled rows)."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    scale, n = w.scale(), w.seq
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    rng = np.random.default_rng(1000 * w.number + seed)
    starts = np.arange(0, n - chunk + 1, chunk)
    if rows_per_head is None:
        order = [(h, int(r)) for h in range(w.heads_q) for r in starts]
        order = [order[i] for i in rng.permutation(len(order))]
    else:
        order = [(h, int(r)) for h in range(w.heads_q)
                 for r in np.sort(rng.choice(starts, rows_per_head // chunk, replace=False))]

    def work(item):
        h, r0 = item
        rows = np.arange(r0, r0 + chunk)
        oracle.attention_forward_rows(q, k, v, scale, True, 0, h, rows)
        oracle.attention_backward_rows(q, k, v, do, scale, True, 0, h, rows)
        return rows

    done = []
    t0 = time.perf_counter()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        with ThreadPoolExecutor(max_workers=cores) as ex:
            pos = 0
            while pos < len(order) and (seconds is None or time.perf_counter() - t0 < seconds):
                batch = order[pos:pos + cores]
                pos += len(batch)
                done.extend(ex.map(work, batch))
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    elapsed = time.perf_counter() - t0
    rows = np.concatenate(done)
    flops = float(np.sum(14.0 * w.d * (rows + 1)))  # causal: row i has i + 1 keys
    frac = len(rows) / (n * w.heads_q)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": elapsed, "rows": int(len(rows)), "sample_fraction": frac,
            "extrapolated": True, "extrapolation_factor": 1.0 / frac,
            "extrapolated_full_seconds": elapsed / frac}


def cpu_baseline(w, x, seconds, step_ms):
    """The oracle on a bounded sample of the benchmarked workload (rows at
    uniformly random positions over all heads, `seconds` of host time), with
    the full run's time extrapolated from it."""
    r = oracle_rows_timed(w, x, seconds=seconds)
    r["sample"] = (f"{r['rows']} query rows ({r['sample_fraction']:.2%} of the rows) of "
                   f"{WORKLOAD} in 32-row chunks at seeded uniformly random positions over all "
                   "heads: forward rows plus their backward work (fp64 numpy, full-width rows); "
                   "value = algorithmic fwd+bwd flops of those rows / wall time; the full run's "
                   f"time is extrapolated (x{r['extrapolation_factor']:.1f})")
    r["gpu_step_ms"] = step_ms
    r["extrapolated_oracle_over_gpu"] = r["extrapolated_full_seconds"] * 1e3 / step_ms
    return r


def gpu_clock(tag):
    """Current GPU clocks from amd-smi (None where the tool or field is
    missing); the raw JSON is kept, trimmed, for inspection.  Skipped under
    rocprofv3 (its variables are in the environment): the tool's child would
    carry the profiler's library into a second program."""
    import subprocess
    if any(k.startswith("ROCPROF") for k in os.environ):
        return {"when": tag, "tool": None, "gfx_mhz": None,
                "fields": "not read: running under rocprofv3"}
    for cmd in (["amd-smi", "metric", "-g", "0", "--clock", "--json"],
                ["rocm-smi", "--showclocks", "--json"]):
        try:
            out = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except Exception as e:  # noqa: BLE001 - a missing tool is a result, not an error
            last = f"{cmd[0]}: {e}"
            continue
        if out.returncode != 0:
            last = f"{cmd[0]}: rc {out.returncode} {out.stderr.strip()[:200]}"
            continue
        try:
            data = json.loads(out.stdout)
        except ValueError:
            last = f"{cmd[0]}: unparsable output"
            continue
        found = {}

        def walk(node, path):
            if isinstance(node, dict):
                for key, val in node.items():
                    walk(val, f"{path}.{key}" if path else str(key))
            elif isinstance(node, list):
                for i, val in enumerate(node):
                    walk(val, f"{path}[{i}]")
            elif "gfx" in path.lower() or "sclk" in path.lower():
                found[path] = node

        walk(data, "")
        # current clock of each graphics engine (one per XCD), in MHz
        mhz = [v for k_, v in found.items() if k_.endswith(".clk.value") or k_.endswith("sclk")]
        return {"when": tag, "tool": cmd[0], "gfx_mhz": mhz if mhz else None,
                "fields": None if mhz else dict(list(found.items())[:24])}
    return {"when": tag, "tool": None, "error": last}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip every measurement besides the benchmarked workload")
    ap.add_argument("--extras", default="all",
                    help="comma list of extra measurements: sweep, workloads, f32, merge, ulysses, "
                         "activation, mlp (default all)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run a plain device copy of this many MiB "
                         "three times (reference reading for hardware byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this build has "
              "no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_fab_forward_amd as fab
    from attention_fab_forward_amd import _binding as fab_binding
    from attention_fab_forward_amd.inputs import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fab.lib()

    clocks = [gpu_clock("before")]
    w = WORKLOADS[WORKLOAD]
    fwd_fl, bwd_fl, unit = attention_flops(w)
    log(f"workload {WORKLOAD}: {unit} unmasked pairs, fwd {fwd_fl:.3e} flop, bwd {bwd_fl:.3e} flop")
    r = time_attention(w, args.steps, args.warmup, torch, fab_binding)
    clocks.append(gpu_clock("after the timed steps"))
    step_ms, fwd_ms = r["step_ms"], r["fwd_ms"]
    value = (fwd_fl + bwd_fl) / step_ms / 1e9
    kflops = kernel_flops(w)
    kbytes = kernel_bytes(w)
    kern = {}
    for name, (cnt, tot) in r["kernels"].items():
        avg = tot / cnt
        entry = {"launches": cnt, "avg_ms": avg}
        if kflops.get(name):
            entry["tflops"] = kflops[name] / avg / 1e9
        if kbytes.get(name):
            entry["gbs"] = kbytes[name] / avg / 1e6
        kern[name] = entry
    dom = max(kern, key=lambda k_: kern[k_]["avg_ms"] * kern[k_]["launches"])
    if kflops.get(dom):
        ach = kflops[dom] / kern[dom]["avg_ms"] / 1e9
        roof = {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / BF16_PEAK_TFLOPS, "traffic": measured_traffic(dom), "kernel": dom,
                "flops_per_launch": kflops[dom], "avg_launch_ms": kern[dom]["avg_ms"],
                "mfma_counters": measured_mfma(dom)}
    else:
        ach = kbytes[dom] / kern[dom]["avg_ms"] / 1e6
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(dom), "kernel": dom}
    log(f"step {step_ms:.3f} ms ({value:.1f} TFLOP/s), fwd {fwd_ms:.3f} ms; kernels: "
        + ", ".join(f"{k_} {v['avg_ms']:.3f} ms" for k_, v in kern.items()))
    secondary = exp_bound(torch, fab_binding, unit)
    secondary["exp_bound_frac_of_step"] = secondary["exp_bound_ms_fwd_bwd"] / step_ms
    log(f"exp2(fma) rate {secondary['exp_per_s']:.3e}/s -> exp-bound {secondary['exp_bound_ms_fwd_bwd']:.3f} ms "
        f"of the {step_ms:.3f} ms step")

    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB copied 3 times")
        del src, dst

    extras = {}
    want = set() if args.no_extras else (
        {"sweep", "workloads", "merge", "ulysses", "activation", "mlp"} if args.extras == "all"
        else set(args.extras.split(",")))
    if "sweep" in want:
        log("peak-memory sweep ...")
        extras["peak_hbm_vs_seq"] = peak_hbm_sweep(torch, fab)
        # the sequence-parallel rank share's geometry (4 heads), up to its
        # full n = 2^17
        extras["peak_hbm_vs_seq_rank_share"] = peak_hbm_sweep(torch, fab, range(12, 18), 4, 4)
    if "workloads" in want or "f32" in want:
        log("other workloads ...")
        # (repetitions, back to back); the fp32 ones alone with --extras f32
        reps = {
            # latency-bound (microseconds of work): reported in us
            "attn_f32_h1_n256_d64": (200, True),
            "attn_causal_f32_h8_n4096_d128": (10, False),
            "attn_causal_bf16_h4_n131072_d128": (5, False),
            "attn_causal_bf16_gqa2_n1048576_d128": (3, False),
        }
        extras["workloads"] = {
            key: time_workload(key, r_, torch, fab, back_to_back=b2b)
            for key, (r_, b2b) in reps.items() if "workloads" in want or "_f32_" in key}
    if "merge" in want:
        log("merge ...")
        extras["merge"] = time_merge(w, 20, torch, fab)
    if "ulysses" in want:
        log("ulysses layout ...")
        extras["ulysses_layout"] = time_ulysses(
            WORKLOADS["attn_causal_bf16_h4_n131072_d128"], 20, torch, fab)
    if "activation" in want:
        log("activation memory ...")
        extras["activation_memory"] = activation_memory(torch, fab)
    if "mlp" in want:
        log("mlp ...")
        extras["mlp"] = time_mlp(max(3, args.steps), args.warmup, torch, fab_binding)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline ({args.cpu_seconds:.0f} s) ...")
        cpu = cpu_baseline(w, r["inputs"], args.cpu_seconds, step_ms)
        if "workloads" in want:
            # the two long-sequence workloads: 256 rows per head, extrapolated
            from attention_fab_forward_amd.inputs import attention_inputs
            samples = {}
            for key in ("attn_causal_bf16_h4_n131072_d128", "attn_causal_bf16_gqa2_n1048576_d128"):
                log(f"cpu oracle sample of {key} ...")
                wk = WORKLOADS[key]
                res = oracle_rows_timed(wk, attention_inputs(wk), rows_per_head=256)
                res["sample"] = (f"256 query rows per head ({res['sample_fraction']:.3%} of the "
                                 "rows) in 32-row chunks at seeded uniformly random positions; "
                                 "full run extrapolated")
                gpu = extras["workloads"][key]
                res["extrapolated_oracle_over_gpu"] = (res["extrapolated_full_seconds"] * 1e3
                                                       / (gpu["fwd_ms"] + gpu["bwd_ms"]))
                samples[key] = res
            cpu["other_workloads"] = samples

    line = {
        "metric": "f(AB)C fwd / fwd+bwd TFLOP/s and % bf16 MFMA peak; peak HBM vs seq len",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {"workload": WORKLOAD, "batch": w.batch, "heads_q": w.heads_q,
                   "heads_kv": w.heads_kv, "seq_len": w.seq, "head_dim": w.d, "mask": "causal",
                   "step": "forward + backward", "parallelism": "single GPU"},
        "pct_bf16_peak": 100.0 * value / BF16_PEAK_TFLOPS,
        "fwd_tflops": fwd_fl / fwd_ms / 1e9,
        "fwd_pct_bf16_peak": 100.0 * fwd_fl / fwd_ms / 1e9 / BF16_PEAK_TFLOPS,
        "fwd_ms": fwd_ms,
        "bwd_ms": r["bwd_ms"],
        "spread_ms": r["spread_ms"],
        "step_ms_with_kernel_events": r["step_ms_kernel_pass"],
        "gpu_clock": clocks,
        "kernels": kern,
        "roofline": roof,
        "cpu_baseline": cpu,
        "secondary_bound": secondary,
    }
    line.update(extras)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
