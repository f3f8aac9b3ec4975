"""Seeded synthetic inputs for the fused f(A.B).C block.

Shared by the tests, the smoke check and the benchmark; it holds none of the
method's arithmetic, only random draws and the rounding of those draws to the
input dtype.  Every tensor comes from numpy's PCG64 generator seeded with
1000 * c + t, where c is the workload number below and t is 1 for A/Q, 2 for
B/K, 3 for C/V and 4 for dO.  Values are drawn as float32 normals, scaled by
sigma, then (for bf16 workloads) rounded to the nearest bf16 value, ties to
even; the result is returned as float32 arrays that hold bf16 values exactly,
so the oracle (which widens them to float64) and the device (which narrows
them to bf16 without loss) see the same numbers.
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, value scale and mask."""
    key: str
    number: int          # c in the seed formula
    f: str               # "softmax" or "gelu"
    dtype: str           # "bf16" or "f32"
    causal: bool
    sigma: float
    batch: int = 1
    heads_q: int = 1
    heads_kv: int = 1
    seq: int = 0         # attention: n_q = n_k = seq
    d: int = 0           # attention head dim
    mlp: tuple = field(default=(0, 0, 0, 0))  # (m, k, n, p) for the MLP

    def scale(self):
        """Scale applied inside f, as the float32 value the device receives."""
        if self.f == "gelu":
            return 1.0
        return float(np.float32(1.0 / np.sqrt(np.float32(self.d))))


WORKLOADS = {
    # single-head fp32 attention, n = 256, d = 64, no mask
    "attn_f32_h1_n256_d64": Workload("attn_f32_h1_n256_d64", 1, "softmax", "f32",
                                     False, 1.0, 1, 1, 1, 256, 64),
    # GeLU MLP, A 4096x1024, B 1024x4096, C 4096x1024, entries N(0, 0.02^2)
    "mlp_gelu_m4096_k1024_n4096_p1024": Workload(
        "mlp_gelu_m4096_k1024_n4096_p1024", 2, "gelu", "bf16", False, 0.02,
        mlp=(4096, 1024, 4096, 1024)),
    # causal multi-head attention, 32 heads, n = 32768, d = 128
    "attn_causal_bf16_h32_n32768_d128": Workload(
        "attn_causal_bf16_h32_n32768_d128", 3, "softmax", "bf16", True, 1.0,
        1, 32, 32, 32768, 128),
    # one sequence-parallel rank's share: 4 of 32 heads, full n = 131072
    "attn_causal_bf16_h4_n131072_d128": Workload(
        "attn_causal_bf16_h4_n131072_d128", 4, "softmax", "bf16", True, 1.0,
        1, 4, 4, 131072, 128),
    # long context, grouped-query: 2 query heads share 1 kv head, n = 2^20
    "attn_causal_bf16_gqa2_n1048576_d128": Workload(
        "attn_causal_bf16_gqa2_n1048576_d128", 5, "softmax", "bf16", True, 1.0,
        1, 2, 1, 1 << 20, 128),
    # fp32 causal attention large enough for the fp32 matrix cores:
    # 8 heads, n = 4096, d = 128
    "attn_causal_f32_h8_n4096_d128": Workload(
        "attn_causal_f32_h8_n4096_d128", 6, "softmax", "f32", True, 1.0,
        1, 8, 8, 4096, 128),
}


def normal_f32(seed, shape, sigma=1.0):
    """float32 normals from PCG64(seed), multiplied by sigma in float32."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def round_to_bf16(x):
    """Round float32 values to the nearest bf16 value (ties to even).

    Returns float32 arrays whose low 16 bits are zero.  Inputs are finite.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32)


def draw(seed, shape, sigma, dtype):
    x = normal_f32(seed, shape, sigma)
    return round_to_bf16(x) if dtype == "bf16" else x


def attention_inputs(w, seq=None, heads_q=None, heads_kv=None, batch=None,
                     with_grad=True):
    """Q, K, V (and dO) in [batch, seq, heads, d] order as float32 arrays.

    seq / heads override the workload's sizes for reduced-size parity runs;
    the seeds stay the workload's own.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    n = w.seq if seq is None else seq
    hq = w.heads_q if heads_q is None else heads_q
    hkv = w.heads_kv if heads_kv is None else heads_kv
    b = w.batch if batch is None else batch
    base = 1000 * w.number
    out = {
        "q": draw(base + 1, (b, n, hq, w.d), w.sigma, w.dtype),
        "k": draw(base + 2, (b, n, hkv, w.d), w.sigma, w.dtype),
        "v": draw(base + 3, (b, n, hkv, w.d), w.sigma, w.dtype),
    }
    if with_grad:
        out["do"] = draw(base + 4, (b, n, hq, w.d), 1.0, w.dtype)
    return out


def mlp_inputs(w, m=None, with_grad=True):
    """A [m, k], Bt [n, k] (B drawn as [k, n] then transposed), C [n, p], dO."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    mm, k, n, p = w.mlp
    if m is not None:
        mm = m
    base = 1000 * w.number
    b = draw(base + 2, (k, n), w.sigma, w.dtype)
    out = {
        "a": draw(base + 1, (mm, k), w.sigma, w.dtype),
        "bt": np.ascontiguousarray(b.T),
        "c": draw(base + 3, (n, p), w.sigma, w.dtype),
    }
    if with_grad:
        out["do"] = draw(base + 4, (mm, p), 1.0, w.dtype)
    return out


def random_array(seed, shape, sigma=1.0, dtype="f32"):
    """Generic seeded draw for tests that need extra shapes."""
    return draw(seed, shape, sigma, dtype)
