"""CPU tests of the C ABI: the library loads, exports every declared symbol and
validates problems and arguments without touching a device."""
import ctypes
import os
import re

import pytest

from attention_fab_forward_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "fab.h")) as fh:
        text = fh.read()
    return set(re.findall(r"\b(fab_[a-z_]+)\s*\(", text))


def test_exports_every_declared_symbol():
    L = B.lib()
    names = declared_functions()
    assert names == set(B.EXPORTS)
    for name in names:
        assert hasattr(L, name), name


def test_abi_version_and_struct_size():
    L = B.lib()
    assert L.fab_abi_version() == B.ABI_VERSION
    assert L.fab_abi_version() == 3
    assert L.fab_problem_size() == ctypes.sizeof(B.FabProblem) == 192
    assert ctypes.sizeof(B.FabUlyssesLayout) == 72


def attn(**kw):
    base = dict(f=B.SOFTMAX, dtype=B.BF16, batch=1, heads_a=4, heads_bc=2, m=256, n=256,
                k=128, p=128, scale=0.088, causal=True)
    base.update(kw)
    return B.make_problem(**base)


def status_of(prob):
    try:
        B.Plan(prob)
    except B.FabError as e:
        return e.name
    return "FAB_OK"


@pytest.mark.parametrize("kw,expect", [
    ({}, "FAB_OK"),
    ({"dtype": B.F32, "k": 64, "p": 64}, "FAB_OK"),
    ({"causal": False, "m": 100, "n": 300}, "FAB_OK"),
    ({"heads_a": 3}, "FAB_ERR_BAD_SHAPE"),
    ({"m": 0}, "FAB_ERR_BAD_SHAPE"),
    ({"batch": 0}, "FAB_ERR_BAD_SHAPE"),
    ({"m": 100, "n": 300}, "FAB_OK"),  # causal with m != n: offsets place the rows
    ({"m": 100, "n": 300, "q_offset": 200}, "FAB_OK"),
    ({"k_offset": -5, "q_offset": 7}, "FAB_OK"),
    ({"q_offset": 1 << 41}, "FAB_ERR_BAD_SHAPE"),
    # grids of 2^31 workgroups or more are refused at plan time
    ({"batch": 1 << 10, "heads_a": 1 << 10, "heads_bc": 1 << 10, "m": 1 << 13, "n": 1 << 13},
     "FAB_ERR_UNSUPPORTED"),
    ({"batch": 1 << 10, "heads_a": 1 << 10, "heads_bc": 1 << 10, "m": (1 << 13) - 1,
      "n": (1 << 13) - 1}, "FAB_OK"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "q_offset": 3},
     "FAB_ERR_UNSUPPORTED"),
    ({"k": 96, "p": 96}, "FAB_ERR_UNSUPPORTED"),
    ({"k": 128, "p": 64}, "FAB_ERR_UNSUPPORTED"),
    ({"scale": 0.0}, "FAB_ERR_UNSUPPORTED"),
    ({"scale": float("nan")}, "FAB_ERR_BAD_SHAPE"),
    ({"abi_version": 99}, "FAB_ERR_ABI_VERSION"),
    ({"f": 7}, "FAB_ERR_UNSUPPORTED"),
    ({"dtype": 5}, "FAB_ERR_UNSUPPORTED"),
    ({"strides": {"a_stride": (256 * 4 * 128, 128, 4 * 128 + 4)}}, "FAB_ERR_ALIGNMENT"),
    ({"strides": {"a_stride": (256 * 4 * 128, 128, 64)}}, "FAB_ERR_BAD_SHAPE"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": True}, "FAB_ERR_UNSUPPORTED"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "dtype": B.F32},
     "FAB_ERR_UNSUPPORTED"),
    # GeLU widths: multiples of 64 from 64 to 1024
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "k": 1024, "p": 256},
     "FAB_OK"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "k": 384, "p": 128},
     "FAB_OK"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "k": 64, "p": 960},
     "FAB_OK"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "k": 96, "p": 128},
     "FAB_ERR_UNSUPPORTED"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "k": 128, "p": 32},
     "FAB_ERR_UNSUPPORTED"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "k": 2048, "p": 128},
     "FAB_ERR_UNSUPPORTED"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "k": 128, "p": 1088},
     "FAB_ERR_UNSUPPORTED"),
    # an output whose heads (or batch entries) share memory is refused
    ({"strides": {"o_stride": (256 * 4 * 128, 0, 4 * 128)}}, "FAB_ERR_BAD_SHAPE"),
    ({"batch": 2, "strides": {"o_stride": (0, 128, 4 * 128)}}, "FAB_ERR_BAD_SHAPE"),
    ({"strides": {"o_stride": (256 * 4 * 128, 64, 4 * 128)}}, "FAB_ERR_BAD_SHAPE"),
    # inputs broadcast over heads plan fine (the forward only reads them)
    ({"strides": {"bt_stride": (256 * 128, 0, 128), "c_stride": (256 * 128, 0, 128)}},
     "FAB_OK"),
    # an exchange-buffer layout {batch Hl d, head d, row b Hl d} is one-to-one
    ({"batch": 3, "strides": {"o_stride": (4 * 128, 128, 3 * 4 * 128)}}, "FAB_OK"),
    # fp32 kernel family: fp32 softmax only, known values only
    ({"dtype": B.F32, "variant": B.VARIANT_F32_MFMA}, "FAB_OK"),
    ({"dtype": B.F32, "variant": B.VARIANT_F32_FMA}, "FAB_OK"),
    ({"variant": B.VARIANT_F32_MFMA}, "FAB_ERR_UNSUPPORTED"),
    ({"dtype": B.F32, "variant": 3}, "FAB_ERR_BAD_SHAPE"),
    ({"dtype": B.F32, "variant": -1}, "FAB_ERR_BAD_SHAPE"),
    ({"f": B.GELU_ERF, "heads_a": 1, "heads_bc": 1, "causal": False, "variant": 1},
     "FAB_ERR_UNSUPPORTED"),
    # row strides the kernels' 32-bit copy offsets cannot address
    ({"strides": {"a_stride": (1 << 30, 1 << 24, 1 << 25)}}, "FAB_ERR_UNSUPPORTED"),
])
def test_plan_validation(kw, expect):
    assert status_of(attn(**kw)) == expect


def test_plan_workspace_and_describe():
    p = B.Plan(attn())
    assert p.fwd_workspace == 0
    assert p.bwd_workspace >= 4 * 256 * 4
    assert "attention bf16 d=128 causal" in p.describe()
    # the fp32 FMA backward forms D inside its kernel: no workspace
    small = B.Plan(attn(dtype=B.F32, k=64, p=64))
    assert small.bwd_workspace == 0 and "fp32 FMA" in small.describe()
    # the fp32 matrix-core backward keeps -D and LSE log2(e) per row (8 bytes)
    forced = B.Plan(attn(dtype=B.F32, k=64, p=64, variant=B.VARIANT_F32_MFMA))
    assert "fp32 MFMA" in forced.describe() and forced.bwd_workspace >= 4 * 256 * 8


@pytest.mark.parametrize("m,heads,d,causal,mfma", [
    (256, 1, 128, False, False),     # 4 blocks of 64 queries: plain FMA
    (1024, 1, 128, False, False),    # 16 blocks of 64 queries
    (2048, 1, 128, False, True),     # 32 blocks at d = 128, 2^22 pairs: matrix cores
    (1024, 8, 128, False, True),     # 128 blocks, 2^23 pairs
    (8192, 1, 128, True, True),      # 128 blocks, 2^25 causal pairs
    (512, 16, 128, True, False),     # 128 blocks but 2^21 causal pairs
    (2048, 1, 64, False, False),     # 32 blocks: d = 64 needs 64
    (4096, 1, 64, False, True),      # 64 blocks at d = 64, 2^24 pairs
])
def test_fp32_kernel_family_by_size(m, heads, d, causal, mfma):
    p = B.Plan(attn(dtype=B.F32, heads_a=heads, heads_bc=heads, m=m, n=m, k=d, p=d, causal=causal))
    assert ("fp32 MFMA" in p.describe()) == mfma, p.describe()


def test_null_and_alignment_errors_before_any_launch():
    L = B.lib()
    p = B.Plan(attn())
    vp = ctypes.c_void_p
    good = vp(0x10000)
    st = L.fab_forward(p._ptr, None, good, good, good, good, None, 0, None)
    assert B.STATUS[st] == "FAB_ERR_NULL_ARG"
    assert "null" in L.fab_last_error().decode()
    st = L.fab_forward(p._ptr, vp(0x10008), good, good, good, good, None, 0, None)
    assert B.STATUS[st] == "FAB_ERR_ALIGNMENT"
    st = L.fab_forward(p._ptr, good, good, good, good, None, None, 0, None)
    assert B.STATUS[st] == "FAB_ERR_NULL_ARG"
    st = L.fab_backward(p._ptr, good, good, good, good, good, good, good, good, good, good,
                        p.bwd_workspace - 1, None)
    assert B.STATUS[st] == "FAB_ERR_WORKSPACE_TOO_SMALL"
    st = L.fab_backward(p._ptr, good, good, good, good, good, good, good, good, good, None,
                        p.bwd_workspace, None)
    assert B.STATUS[st] == "FAB_ERR_NULL_ARG"
    st = L.fab_plan(None, None, None, None)
    assert B.STATUS[st] == "FAB_ERR_NULL_ARG"


def test_status_strings():
    L = B.lib()
    for code in B.STATUS:
        assert L.fab_status_string(code)
    assert L.fab_status_string(0) == b"ok"


def test_merge_argument_errors_before_any_launch():
    L = B.lib()
    p = B.Plan(attn())
    vp = ctypes.c_void_p
    good = vp(0x10000)
    st = L.fab_merge(p._ptr, good, good, None, good, good, good, None)
    assert B.STATUS[st] == "FAB_ERR_NULL_ARG"
    st = L.fab_merge(p._ptr, vp(0x10008), good, good, good, good, good, None)
    assert B.STATUS[st] == "FAB_ERR_ALIGNMENT"
    st = L.fab_merge(p._ptr, good, vp(0x10002), good, good, good, good, None)
    assert B.STATUS[st] == "FAB_ERR_ALIGNMENT"
    g = B.Plan(attn(f=B.GELU_ERF, heads_a=1, heads_bc=1, causal=False, m=128, n=128, k=128,
                    p=128, scale=1.0))
    st = L.fab_merge(g._ptr, good, good, good, good, good, good, None)
    assert B.STATUS[st] == "FAB_ERR_UNSUPPORTED"


def ulysses_status(lay):
    L = B.lib()
    hl, elems = ctypes.c_int64(-1), ctypes.c_int64(-1)
    st = L.fab_ulysses_sizes(ctypes.byref(lay), ctypes.byref(hl), ctypes.byref(elems))
    return B.STATUS[st], hl.value, elems.value


@pytest.mark.parametrize("b,nl,heads,d,p,hl", [
    (1, 4096, 32, 128, 8, 4), (2, 100, 8, 64, 8, 1), (1, 16, 2, 128, 8, 1), (3, 7, 6, 64, 3, 2),
    (1, 1, 1, 8, 1, 1)])
def test_ulysses_sizes(b, nl, heads, d, p, hl):
    import torch
    st, got_hl, elems = ulysses_status(B._ulysses_layout(torch.bfloat16, b, nl, heads, d, p))
    assert (st, got_hl, elems) == ("FAB_OK", hl, p * nl * b * hl * d)


@pytest.mark.parametrize("change,expect", [
    ({"heads": 6, "ranks": 4}, "FAB_ERR_BAD_SHAPE"),
    ({"ranks": 0}, "FAB_ERR_BAD_SHAPE"),
    ({"n_local": 0}, "FAB_ERR_BAD_SHAPE"),
    ({"head_dim": 12}, "FAB_ERR_ALIGNMENT"),          # 24 bytes per bf16 row
    ({"abi_version": 2}, "FAB_ERR_ABI_VERSION"),
    ({"dtype": 7}, "FAB_ERR_UNSUPPORTED"),
    ({"x_stride": (4096, 128, -1)}, "FAB_ERR_BAD_SHAPE"),
    ({"x_stride": (4096, 132, 512)}, "FAB_ERR_ALIGNMENT"),
    ({"x_stride": (4096, 128, 64)}, "FAB_ERR_BAD_SHAPE"),  # row shorter than a head row
    ({"n_local": 1 << 28}, "FAB_ERR_UNSUPPORTED"),     # beyond 2^31 16-byte chunks
])
def test_ulysses_layout_validation(change, expect):
    import torch
    lay = B._ulysses_layout(torch.bfloat16, 1, 64, 8, 128, 4)
    for k, v in change.items():
        if k == "x_stride":
            lay.x_stride[:] = list(v)
        else:
            setattr(lay, k, v)
    assert ulysses_status(lay)[0] == expect


def test_ulysses_argument_errors_before_any_launch():
    import torch
    L = B.lib()
    vp = ctypes.c_void_p
    good = vp(0x10000)
    lay = B._ulysses_layout(torch.bfloat16, 1, 64, 8, 128, 4)
    for fn in (L.fab_ulysses_pack, L.fab_ulysses_unpack):
        assert B.STATUS[fn(None, good, good, None)] == "FAB_ERR_NULL_ARG"
        assert B.STATUS[fn(ctypes.byref(lay), None, good, None)] == "FAB_ERR_NULL_ARG"
        assert B.STATUS[fn(ctypes.byref(lay), good, None, None)] == "FAB_ERR_NULL_ARG"
        assert B.STATUS[fn(ctypes.byref(lay), vp(0x10008), good, None)] == "FAB_ERR_ALIGNMENT"
        assert B.STATUS[fn(ctypes.byref(lay), good, vp(0x10004), None)] == "FAB_ERR_ALIGNMENT"
        bad = B._ulysses_layout(torch.bfloat16, 1, 64, 6, 128, 4)
        assert B.STATUS[fn(ctypes.byref(bad), good, good, None)] == "FAB_ERR_BAD_SHAPE"


def test_exp_probe_count_and_argument_errors():
    L = B.lib()
    count = ctypes.c_int64(-1)
    # count only: a NULL sink launches nothing
    assert B.STATUS[L.fab_exp_probe(10, 100, None, ctypes.byref(count), None)] == "FAB_OK"
    assert count.value == 10 * 256 * 100 * 8
    assert B.STATUS[L.fab_exp_probe(0, 100, None, None, None)] == "FAB_ERR_BAD_SHAPE"
    assert B.STATUS[L.fab_exp_probe(10, 0, None, None, None)] == "FAB_ERR_BAD_SHAPE"
    assert B.STATUS[L.fab_exp_probe(10, 100, ctypes.c_void_p(0x10002), None, None)] == \
        "FAB_ERR_ALIGNMENT"


def test_backward_refuses_gradient_layouts_that_overlap():
    """A K broadcast over heads (zero head stride) is a valid forward input, but
    its gradient cannot be written in that layout: both backward entry points
    refuse before any launch."""
    L = B.lib()
    good = ctypes.c_void_p(0x10000)
    p = B.Plan(attn(strides={"bt_stride": (256 * 128, 0, 128)}))
    st = L.fab_backward(p._ptr, good, good, good, good, good, good, good, good, good, good,
                        p.bwd_workspace, None)
    assert B.STATUS[st] == "FAB_ERR_BAD_SHAPE"
    assert "Bt" in L.fab_last_error().decode()
    st = L.fab_backward_noalloc(p._ptr, good, good, good, good, good, good, good, good, good, None)
    assert B.STATUS[st] == "FAB_ERR_BAD_SHAPE"


def test_backward_noalloc_argument_errors_before_any_launch():
    L = B.lib()
    vp = ctypes.c_void_p
    good = vp(0x10000)
    p = B.Plan(attn())
    fn = L.fab_backward_noalloc
    assert B.STATUS[fn(None, good, good, good, good, good, good, good, good, good, None)] == \
        "FAB_ERR_NULL_ARG"
    assert B.STATUS[fn(p._ptr, good, None, good, good, good, good, good, good, good, None)] == \
        "FAB_ERR_NULL_ARG"
    assert B.STATUS[fn(p._ptr, good, good, good, None, good, good, good, good, good, None)] == \
        "FAB_ERR_NULL_ARG"
    assert B.STATUS[fn(p._ptr, vp(0x10008), good, good, good, good, good, good, good, good,
                       None)] == "FAB_ERR_ALIGNMENT"
    # 64 heads x 2^17 rows x 8 bytes of workspace = 64 MiB > the 32 MiB static scratch
    big = B.Plan(attn(heads_a=64, heads_bc=64, m=1 << 17, n=1 << 17))
    assert big.bwd_workspace > 32 << 20
    st = fn(big._ptr, good, good, good, good, good, good, good, good, good, None)
    assert B.STATUS[st] == "FAB_ERR_WORKSPACE_TOO_SMALL"
    assert "32" in L.fab_last_error().decode() or str(32 << 20) in L.fab_last_error().decode()
