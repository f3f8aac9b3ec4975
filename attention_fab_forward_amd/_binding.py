"""ctypes binding of libfab.so: argument marshalling only.

Every computation runs in the library's HIP kernels; this module builds the
problem descriptor, allocates outputs and workspace with torch on the input's
device, and passes raw pointers plus torch's current HIP stream.  If the
library is missing it raises: there is no fallback path.
"""
import ctypes
import os
import threading

import torch

LIB_PATH = os.environ.get("FAB_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libfab.so")
ABI_VERSION = 3

SOFTMAX, GELU_ERF = 0, 1
# fp32 softmax kernel family (fab_variant): the library chooses, plain FMA, matrix cores
VARIANT_AUTO, VARIANT_F32_FMA, VARIANT_F32_MFMA = 0, 1, 2
MASK_NONE, MASK_CAUSAL = 0, 1
BF16, F32 = 0, 1

STATUS = {
    0: "FAB_OK", 1: "FAB_ERR_NULL_ARG", 2: "FAB_ERR_BAD_SHAPE", 3: "FAB_ERR_UNSUPPORTED",
    4: "FAB_ERR_ALIGNMENT", 5: "FAB_ERR_WORKSPACE_TOO_SMALL", 6: "FAB_ERR_ABI_VERSION",
    7: "FAB_ERR_HIP",
}

# every symbol include/fab.h declares
EXPORTS = ("fab_plan", "fab_forward", "fab_backward", "fab_plan_destroy",
           "fab_status_string", "fab_last_error", "fab_abi_version",
           "fab_problem_size", "fab_plan_describe", "fab_plan_set_timing",
           "fab_plan_kernel_times", "fab_plan_reset_kernel_times", "fab_merge",
           "fab_ulysses_sizes", "fab_ulysses_pack", "fab_ulysses_unpack", "fab_exp_probe",
           "fab_backward_noalloc")


class FabProblem(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("f", ctypes.c_int32), ("mask", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("batch", ctypes.c_int64), ("heads_a", ctypes.c_int64),
        ("heads_bc", ctypes.c_int64), ("m", ctypes.c_int64), ("n", ctypes.c_int64),
        ("k", ctypes.c_int64), ("p", ctypes.c_int64), ("scale", ctypes.c_float),
        ("variant", ctypes.c_int32), ("a_stride", ctypes.c_int64 * 3),
        ("bt_stride", ctypes.c_int64 * 3), ("c_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3), ("q_offset", ctypes.c_int64),
        ("k_offset", ctypes.c_int64),
    ]


class FabUlyssesLayout(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32), ("dtype", ctypes.c_int32), ("batch", ctypes.c_int64),
        ("n_local", ctypes.c_int64), ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("ranks", ctypes.c_int64), ("x_stride", ctypes.c_int64 * 3),
    ]


class FabError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {message}")


_lib = None
_lock = threading.Lock()


def lib():
    """Load libfab.so once and check its ABI; raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m attention_fab_forward_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.fab_plan.argtypes = [ctypes.POINTER(FabProblem), ctypes.POINTER(vp),
                               ctypes.POINTER(sz), ctypes.POINTER(sz)]
        L.fab_plan.restype = ctypes.c_int
        L.fab_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fab_forward.restype = ctypes.c_int
        L.fab_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.fab_backward.restype = ctypes.c_int
        L.fab_backward_noalloc.argtypes = [vp] * 11
        L.fab_backward_noalloc.restype = ctypes.c_int
        L.fab_plan_destroy.argtypes = [vp]
        L.fab_plan_destroy.restype = None
        L.fab_status_string.argtypes = [ctypes.c_int]
        L.fab_status_string.restype = ctypes.c_char_p
        L.fab_last_error.argtypes = []
        L.fab_last_error.restype = ctypes.c_char_p
        L.fab_abi_version.argtypes = []
        L.fab_abi_version.restype = ctypes.c_int32
        L.fab_problem_size.argtypes = []
        L.fab_problem_size.restype = ctypes.c_size_t
        L.fab_plan_describe.argtypes = [vp, ctypes.c_char_p, sz]
        L.fab_plan_describe.restype = ctypes.c_size_t
        L.fab_plan_set_timing.argtypes = [vp, ctypes.c_int]
        L.fab_plan_set_timing.restype = ctypes.c_int
        L.fab_plan_kernel_times.argtypes = [vp, ctypes.POINTER(ctypes.c_char_p),
                                            ctypes.POINTER(ctypes.c_int),
                                            ctypes.POINTER(ctypes.c_double), ctypes.c_int]
        L.fab_plan_kernel_times.restype = ctypes.c_int
        L.fab_plan_reset_kernel_times.argtypes = [vp]
        L.fab_plan_reset_kernel_times.restype = ctypes.c_int
        L.fab_merge.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.fab_merge.restype = ctypes.c_int
        lp = ctypes.POINTER(FabUlyssesLayout)
        L.fab_ulysses_sizes.argtypes = [lp, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_int64)]
        L.fab_ulysses_sizes.restype = ctypes.c_int
        L.fab_ulysses_pack.argtypes = [lp, vp, vp, vp]
        L.fab_ulysses_pack.restype = ctypes.c_int
        L.fab_ulysses_unpack.argtypes = [lp, vp, vp, vp]
        L.fab_ulysses_unpack.restype = ctypes.c_int
        L.fab_exp_probe.argtypes = [ctypes.c_int, ctypes.c_int, vp, ctypes.POINTER(ctypes.c_int64), vp]
        L.fab_exp_probe.restype = ctypes.c_int
        if L.fab_abi_version() != ABI_VERSION:
            raise RuntimeError(f"libfab.so ABI {L.fab_abi_version()} != binding {ABI_VERSION}")
        if L.fab_problem_size() != ctypes.sizeof(FabProblem):
            raise RuntimeError("fab_problem layout differs between library and binding")
        _lib = L
    return _lib


def check(status):
    if status != 0:
        raise FabError(status, lib().fab_last_error().decode())


def make_problem(f, dtype, batch, heads_a, heads_bc, m, n, k, p, scale, causal=False,
                 strides=None, abi_version=ABI_VERSION, q_offset=0, k_offset=0, variant=0):
    prob = FabProblem()
    prob.abi_version = abi_version
    prob.variant = variant
    prob.f, prob.dtype = f, dtype
    prob.mask = MASK_CAUSAL if causal else MASK_NONE
    prob.batch, prob.heads_a, prob.heads_bc = batch, heads_a, heads_bc
    prob.m, prob.n, prob.k, prob.p = m, n, k, p
    prob.scale = scale
    prob.q_offset, prob.k_offset = q_offset, k_offset
    if strides:
        for name in ("a_stride", "bt_stride", "c_stride", "o_stride"):
            if name in strides:
                getattr(prob, name)[:] = list(strides[name])
    return prob


class Plan:
    """A validated problem; wraps fab_plan / fab_forward / fab_backward."""

    def __init__(self, prob):
        self.prob = prob
        self._ptr = ctypes.c_void_p()
        fw, bw = ctypes.c_size_t(), ctypes.c_size_t()
        check(lib().fab_plan(ctypes.byref(prob), ctypes.byref(self._ptr), ctypes.byref(fw),
                             ctypes.byref(bw)))
        self.fwd_workspace = fw.value
        self.bwd_workspace = bw.value

    def describe(self):
        buf = ctypes.create_string_buffer(512)
        lib().fab_plan_describe(self._ptr, buf, 512)
        return buf.value.decode()

    def set_timing(self, enable=True):
        check(lib().fab_plan_set_timing(self._ptr, 1 if enable else 0))

    def reset_kernel_times(self):
        check(lib().fab_plan_reset_kernel_times(self._ptr))

    def kernel_times(self):
        """{kernel name: (launches, total ms)} since the last reset (waits for them)."""
        cap = 32
        names = (ctypes.c_char_p * cap)()
        counts = (ctypes.c_int * cap)()
        totals = (ctypes.c_double * cap)()
        k = lib().fab_plan_kernel_times(self._ptr, names, counts, totals, cap)
        if k < 0:
            raise FabError(7, lib().fab_last_error().decode())
        return {names[i].decode(): (counts[i], totals[i]) for i in range(min(k, cap))}

    def forward_raw(self, a, bt, c, o, lse, ws, ws_bytes, stream):
        check(lib().fab_forward(self._ptr, a, bt, c, o, lse, ws, ws_bytes, stream))

    def backward_raw(self, a, bt, c, o, lse, do, da, dbt, dc, ws, ws_bytes, stream):
        check(lib().fab_backward(self._ptr, a, bt, c, o, lse, do, da, dbt, dc, ws, ws_bytes,
                                 stream))

    def backward_noalloc_raw(self, a, bt, c, o, lse, do, da, dbt, dc, stream):
        """fab_backward_noalloc: the backward with the library's static scratch
        in place of a workspace."""
        check(lib().fab_backward_noalloc(self._ptr, a, bt, c, o, lse, do, da, dbt, dc, stream))

    def merge_raw(self, oa, la, ob, lb, oo, lo, stream):
        check(lib().fab_merge(self._ptr, oa, la, ob, lb, oo, lo, stream))

    def __del__(self):
        ptr = getattr(self, "_ptr", None)
        if ptr and _lib is not None:
            _lib.fab_plan_destroy(ptr)


_plans = {}


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check_tensor(name, t, ndim, device, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be on the same GPU as the others ({device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name} needs a contiguous last dimension")


def _strides4(t):
    return (t.stride(0), t.stride(2), t.stride(1))


def _distinct(t):
    """True when no two elements of t share an address (the library's test:
    sorted by stride, each dimension of size > 1 steps past the span of the
    smaller ones)."""
    span = 0
    for stride, size in sorted((st, sz) for st, sz in zip(t.stride(), t.shape) if sz > 1):
        if stride <= span:
            return False
        span += (size - 1) * stride
    return True


def _shape(t, name, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def attention_shapes(q, k, v):
    """(b, m, hq, hkv, n, d, dv) of Q [b, m, hq, d], K [b, n, hkv, d],
    V [b, n, hkv, dv]; ValueError when K and V do not fit Q."""
    b, m, hq, d = _shape(q, "q", 4)
    bk, n, hkv, dk = _shape(k, "k", 4)
    bv, nv, hv, dv = _shape(v, "v", 4)
    if bk != b or bv != b:
        raise ValueError(f"q, k, v batch sizes differ: {b}, {bk}, {bv}")
    if (nv, hv) != (n, hkv):
        raise ValueError(f"v {tuple(v.shape)} must have k's sequence length and heads "
                         f"({n}, {hkv})")
    if dk != d:
        raise ValueError(f"k's head dim {dk} differs from q's {d}")
    if hkv < 1 or hq % hkv:
        raise ValueError(f"query heads {hq} are not a multiple of kv heads {hkv}")
    return b, m, hq, hkv, n, d, dv


def attention_grad_shapes(q, k, v, o, lse, do):
    """attention_shapes, plus O and dO [b, m, hq, dv] and LSE [b, hq, m]."""
    b, m, hq, hkv, n, d, dv = attention_shapes(q, k, v)
    want = (b, m, hq, dv)
    if _shape(o, "o", 4) != want:
        raise ValueError(f"o has shape {tuple(o.shape)}, expected {want}")
    if _shape(do, "do", 4) != want:
        raise ValueError(f"do has shape {tuple(do.shape)}, expected {want}")
    if _shape(lse, "lse", 3) != (b, hq, m):
        raise ValueError(f"lse has shape {tuple(lse.shape)}, expected {(b, hq, m)}")
    return b, m, hq, hkv, n, d, dv


def mlp_shapes(a, bt, c, do=None):
    """(m, k, n, p) of A [m, k], Bt [n, k], C [n, p] (and dO [m, p])."""
    m, k = _shape(a, "a", 2)
    n, kb = _shape(bt, "bt", 2)
    nc, p = _shape(c, "c", 2)
    if kb != k:
        raise ValueError(f"bt [n, k] has k = {kb}, a has k = {k}")
    if nc != n:
        raise ValueError(f"c [n, p] has n = {nc}, bt has n = {n}")
    if do is not None and _shape(do, "do", 2) != (m, p):
        raise ValueError(f"do has shape {tuple(do.shape)}, expected {(m, p)}")
    return m, k, n, p


def _get_plan(key, build):
    plan = _plans.get(key)
    if plan is None:
        plan = Plan(build())
        _plans[key] = plan
    return plan


def attention_plan(q, k, v, causal, scale, q_offset=0, k_offset=0, o=None, variant=0):
    """Plan for these tensors' shapes and strides; O packed [b, m, hq, d]
    unless `o` gives its layout.  variant: fp32 kernel family (VARIANT_*)."""
    b, m, hq, d = q.shape
    n, hkv = k.shape[1], k.shape[2]
    o_stride = (_strides4(o) if o is not None
                else (m * hq * v.shape[3], v.shape[3], hq * v.shape[3]))
    strides = {"a_stride": _strides4(q), "bt_stride": _strides4(k), "c_stride": _strides4(v),
               "o_stride": o_stride}
    key = ("softmax", q.dtype, b, hq, hkv, m, n, d, v.shape[3], float(scale), bool(causal),
           tuple(sorted(strides.items())), int(q_offset), int(k_offset), int(variant))
    return _get_plan(key, lambda: make_problem(SOFTMAX, _dtype_code(q), b, hq, hkv, m, n, d,
                                               v.shape[3], scale, causal, strides,
                                               q_offset=q_offset, k_offset=k_offset,
                                               variant=variant))


def mlp_plan(a, bt, c, scale):
    m, k = a.shape
    n, p = bt.shape[0], c.shape[1]
    strides = {"a_stride": (m * a.stride(0), 0, a.stride(0)),
               "bt_stride": (n * bt.stride(0), 0, bt.stride(0)),
               "c_stride": (n * c.stride(0), 0, c.stride(0)),
               "o_stride": (m * p, 0, p)}
    key = ("gelu", a.dtype, m, n, k, p, float(scale), tuple(sorted(strides.items())))
    return _get_plan(key, lambda: make_problem(GELU_ERF, _dtype_code(a), 1, 1, 1, m, n, k, p,
                                               scale, False, strides))


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def forward(a, bt, c, f="softmax", causal=False, scale=None, q_offset=0, k_offset=0,
            out=None, variant=0):
    """O = f(scale * A Bt^T) C on the GPU.

    softmax: a = Q [b, m, hq, d], bt = K [b, n, hkv, d], c = V [b, n, hkv, d];
    returns (O [b, m, hq, d], LSE float32 [b, hq, m]).  Default scale 1/sqrt(d).
    causal: key j is visible to query i iff k_offset + j <= q_offset + i; rows
    that see no key get O = 0, LSE = -inf.  out=(o, lse) writes there; o may
    have any layout with a contiguous last dimension (e.g. an exchange buffer).
    gelu: a [m, k], bt [n, k], c [n, p]; returns (O [m, p], None).  Default scale 1.
    variant (fp32 softmax only): VARIANT_F32_FMA or VARIANT_F32_MFMA picks the
    kernel family; 0 lets the library choose by size.
    """
    dev, dt = a.device, a.dtype
    if f == "softmax":
        attention_shapes(a, bt, c)
        for name, t in (("q", a), ("k", bt), ("v", c)):
            _check_tensor(name, t, 4, dev, dt)
        if scale is None:
            scale = 1.0 / float(a.shape[3]) ** 0.5
        b, m, hq, _ = a.shape
        if out is not None:
            o, lse = out
            _check_tensor("out o", o, 4, dev, dt)
            if tuple(o.shape) != (b, m, hq, c.shape[3]):
                raise ValueError(f"out o has shape {tuple(o.shape)}, expected "
                                 f"{(b, m, hq, c.shape[3])}")
            if (lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != dev
                    or tuple(lse.shape) != (b, hq, m)):
                raise ValueError(f"out lse must be contiguous float32 {(b, hq, m)} on {dev}")
        else:
            o = torch.empty((b, m, hq, c.shape[3]), dtype=dt, device=dev)
            lse = torch.empty((b, hq, m), dtype=torch.float32, device=dev)
        plan = attention_plan(a, bt, c, causal, scale, q_offset, k_offset, o, variant)
    elif f == "gelu":
        if causal:
            raise ValueError("GeLU takes no causal mask")
        if out is not None:
            raise ValueError("out= is for softmax only")
        mlp_shapes(a, bt, c)
        for name, t in (("a", a), ("bt", bt), ("c", c)):
            _check_tensor(name, t, 2, dev, dt)
        scale = 1.0 if scale is None else scale
        plan = mlp_plan(a, bt, c, scale)
        o = torch.empty((a.shape[0], c.shape[1]), dtype=dt, device=dev)
        lse = None
    else:
        raise ValueError(f"unknown f {f!r}")
    ws = torch.empty(max(plan.fwd_workspace, 1), dtype=torch.uint8, device=dev)
    plan.forward_raw(_ptr(a), _ptr(bt), _ptr(c), _ptr(o), _ptr(lse), _ptr(ws),
                     plan.fwd_workspace, _stream())
    return o, lse


def backward(a, bt, c, o, lse, do, f="softmax", causal=False, scale=None, q_offset=0,
             k_offset=0, variant=0):
    """Gradients (dA, dBt, dC) of <dO, O> for the forward above.  Over a key
    range (offsets) pass the merged O and LSE of all keys: dA is then the
    range's contribution to dQ.  O may have any layout (dO must share it);
    the gradients take the layouts of A, Bt and C.  A primal whose layout
    maps two elements to one address (say K expanded over heads) is replaced
    by a packed copy first, and its gradient comes back packed."""
    dev, dt = a.device, a.dtype
    if f == "softmax":
        if lse is None:
            raise ValueError("lse must be the contiguous float32 tensor from forward()")
        attention_grad_shapes(a, bt, c, o, lse, do)
        for name, t in (("q", a), ("k", bt), ("v", c), ("o", o), ("do", do)):
            _check_tensor(name, t, 4, dev, dt)
        if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != dev:
            raise ValueError("lse must be the contiguous float32 tensor from forward()")
        if do.stride() != o.stride():
            raise ValueError("dO must have the layout of O")
        if scale is None:
            scale = 1.0 / float(a.shape[3]) ** 0.5
        a, bt, c = (t if _distinct(t) else t.contiguous() for t in (a, bt, c))
        plan = attention_plan(a, bt, c, causal, scale, q_offset, k_offset, o, variant)
    elif f == "gelu":
        mlp_shapes(a, bt, c, do)
        for name, t in (("a", a), ("bt", bt), ("c", c), ("do", do)):
            _check_tensor(name, t, 2, dev, dt)
        scale = 1.0 if scale is None else scale
        plan = mlp_plan(a, bt, c, scale)
        o = lse = None
    else:
        raise ValueError(f"unknown f {f!r}")
    da, dbt, dc = (torch.empty_strided(t.shape, t.stride(), dtype=dt, device=dev)
                   for t in (a, bt, c))
    ws = torch.empty(max(plan.bwd_workspace, 1), dtype=torch.uint8, device=dev)
    plan.backward_raw(_ptr(a), _ptr(bt), _ptr(c), _ptr(o), _ptr(lse), _ptr(do), _ptr(da),
                      _ptr(dbt), _ptr(dc), _ptr(ws), plan.bwd_workspace, _stream())
    return da, dbt, dc


def merge(o_a, lse_a, o_b, lse_b, out=None):
    """Merge two softmax results over disjoint key sets of the same queries
    (fab_merge).  o_* [b, m, hq, d] packed, lse_* float32 [b, hq, m].  Returns
    (O, LSE); out=(o, lse) writes there (may be (o_a, lse_a))."""
    dev, dt = o_a.device, o_a.dtype
    for name, t in (("o_a", o_a), ("o_b", o_b)):
        _check_tensor(name, t, 4, dev, dt)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be packed [b, m, hq, d]")
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != dev:
            raise ValueError(f"{name} must be a contiguous float32 tensor on {dev}")
    b, m, hq, d = o_a.shape
    if o_b.shape != o_a.shape or lse_a.shape != (b, hq, m) or lse_b.shape != (b, hq, m):
        raise ValueError("shape mismatch between the two parts")
    if out is not None:
        o, lse = out
        if (not isinstance(o, torch.Tensor) or o.shape != o_a.shape or o.dtype != dt
                or o.device != dev or not o.is_contiguous()):
            raise ValueError(f"out o must be a packed {dt} tensor of shape {tuple(o_a.shape)} "
                             f"on {dev}")
        if (not isinstance(lse, torch.Tensor) or lse.shape != (b, hq, m)
                or lse.dtype != torch.float32 or lse.device != dev or not lse.is_contiguous()):
            raise ValueError(f"out lse must be a contiguous float32 tensor of shape "
                             f"{(b, hq, m)} on {dev}")
    else:
        o, lse = torch.empty_like(o_a), torch.empty_like(lse_a)
    key = ("merge", dt, b, hq, m, d)
    plan = _get_plan(key, lambda: make_problem(SOFTMAX, _dtype_code(o_a), b, hq, hq, m, m, d, d,
                                               1.0, False, None))
    plan.merge_raw(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse), _stream())
    return o, lse


# ---------------------------------------------------------------------------
# Ulysses exchange layout (fab_ulysses_pack / fab_ulysses_unpack)
# ---------------------------------------------------------------------------

def _ulysses_layout(dtype, b, n_local, heads, d, ranks, x_stride=(0, 0, 0)):
    lay = FabUlyssesLayout()
    lay.abi_version = ABI_VERSION
    lay.dtype = _dtype_code(torch.empty(0, dtype=dtype))
    lay.batch, lay.n_local, lay.heads, lay.head_dim, lay.ranks = b, n_local, heads, d, ranks
    lay.x_stride[:] = list(x_stride)
    return lay


def ulysses_sizes(b, n_local, heads, d, ranks, dtype=torch.bfloat16):
    """(heads per rank Hl, elements of one exchange buffer); host only."""
    lay = _ulysses_layout(dtype, b, n_local, heads, d, ranks)
    hl, elems = ctypes.c_int64(), ctypes.c_int64()
    check(lib().fab_ulysses_sizes(ctypes.byref(lay), ctypes.byref(hl), ctypes.byref(elems)))
    return hl.value, elems.value


def ulysses_pack(x, ranks, out=None):
    """Send buffer [p, n_local, b, Hl, d] (block j for rank j) from this rank's
    tokens x [b, n_local, H, d] (any strides, contiguous last dimension)."""
    _check_tensor("x", x, 4, x.device, x.dtype)
    b, nl, heads, d = x.shape
    lay = _ulysses_layout(x.dtype, b, nl, heads, d, ranks, _strides4(x))
    hl, _ = ulysses_sizes(b, nl, heads, d, ranks, x.dtype)
    shape = (ranks, nl, b, hl, d)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif tuple(out.shape) != shape or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError(f"out must be a contiguous {x.dtype} tensor of shape {shape}")
    check(lib().fab_ulysses_pack(ctypes.byref(lay), _ptr(x), _ptr(out), _stream()))
    return out


def ulysses_unpack(recv, heads, out=None):
    """x [b, n_local, H, d] from the return exchange's receive buffer
    [p, n_local, b, Hl, d]; a head held by several ranks gets their sum.
    out: a tensor of that shape, any strides with a contiguous last dimension."""
    if not recv.is_contiguous() or recv.dim() != 5:
        raise ValueError("recv must be a contiguous [p, n_local, b, Hl, d] tensor")
    p, nl, b, hl, d = recv.shape
    if out is None:
        out = torch.empty((b, nl, heads, d), dtype=recv.dtype, device=recv.device)
    _check_tensor("out", out, 4, recv.device, recv.dtype)
    if tuple(out.shape) != (b, nl, heads, d):
        raise ValueError(f"out must have shape {(b, nl, heads, d)}")
    lay = _ulysses_layout(recv.dtype, b, nl, heads, d, p, _strides4(out))
    if ulysses_sizes(b, nl, heads, d, p, recv.dtype)[0] != hl:
        raise ValueError("recv's head count does not match heads / ranks")
    check(lib().fab_ulysses_unpack(ctypes.byref(lay), _ptr(recv), _ptr(out), _stream()))
    return out


def ulysses_sequence_view(recv):
    """A receive buffer [p, n_local, b, Hl, d] of the first exchange seen as
    [b, n, Hl, d] (no copy): the layout attention reads and writes in place."""
    p, nl, b, hl, d = recv.shape
    return recv.view(p * nl, b, hl, d).permute(1, 0, 2, 3)


def exp_probe(blocks, iters, sink):
    """Enqueue the exp2(fma) rate probe (fab_exp_probe) on torch's current
    stream; sink: float32 CUDA tensor of at least blocks * 256 elements.
    Returns the number of exponentials enqueued."""
    if sink.dtype != torch.float32 or sink.numel() < blocks * 256 or sink.device.type != "cuda":
        raise ValueError("sink must be a float32 CUDA tensor of blocks * 256 elements")
    count = ctypes.c_int64()
    check(lib().fab_exp_probe(blocks, iters, _ptr(sink), ctypes.byref(count), _stream()))
    return count.value
