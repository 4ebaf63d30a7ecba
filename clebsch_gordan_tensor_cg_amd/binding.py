"""Thin Python binding of the cgtp C ABI (include/cgtp.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch supplies device memory and the current stream.  torch is
imported before the library is loaded so that both share one HIP runtime
(they resolve the same libamdhip64.so.7 soname).  If the library has not
been built this module raises at load time; nothing falls back to the CPU.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading libcgtp.so)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcgtp.so")

CGTP_UVU, CGTP_UVW = 0, 1
DTYPES = {"f32": 0, "f64": 1, "bf16": 2}
TORCH_DTYPES = {"f32": torch.float32, "f64": torch.float64, "bf16": torch.bfloat16}
CGTP_SHARED_WEIGHTS = 1
CGTP_PLAN_NO_LOAD = 2
CGTP_BF16_WEIGHTS = 4

_ERRORS = {-1: "INVALID_ARGUMENT", -2: "UNSUPPORTED", -3: "COMPILE", -4: "HIP", -5: "GRAPH"}


class CgtpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"cgtp error {code} ({_ERRORS.get(code, '?')}): {msg}")
        self.code = code


class _Path(ctypes.Structure):
    _fields_ = [("i_in1", ctypes.c_int32), ("i_in2", ctypes.c_int32), ("i_out", ctypes.c_int32)]


class _Dims(ctypes.Structure):
    _fields_ = [("dim_in1", ctypes.c_int64), ("dim_in2", ctypes.c_int64), ("dim_out", ctypes.c_int64),
                ("weight_numel", ctypes.c_int64), ("n_paths", ctypes.c_int32),
                ("lmax_in2", ctypes.c_int32), ("n_kernels", ctypes.c_int32), ("cached", ctypes.c_int32)]


EXPORTS = [
    "cgtp_plan", "cgtp_plan_info", "cgtp_plan_paths", "cgtp_plan_coupling", "cgtp_plan_source",
    "cgtp_plan_destroy", "cgtp_workspace_bytes", "cgtp_forward", "cgtp_tp_backward", "cgtp_conv_forward",
    "cgtp_conv_forward_vec", "cgtp_conv_forward_radial", "cgtp_backward", "cgtp_conv_backward_vec",
    "cgtp_conv_forward_backward", "cgtp_conv_forward_backward_vec", "cgtp_double_backward",
    "cgtp_sparse_attention", "cgtp_sparse_attention_rows", "cgtp_sparse_attention_layout_bytes",
    "cgtp_sparse_attention_prepare", "cgtp_csr_workspace_bytes", "cgtp_build_csr", "cgtp_build_csr_order",
    "cgtp_build_csr_order_noalloc", "cgtp_build_csr_transpose_canonical",
    "cgtp_validate_csr", "cgtp_node_order_workspace_bytes", "cgtp_node_order", "cgtp_sh", "cgtp_sh_vjp_forces",
    "cgtp_force_loss_sh_cotangent", "cgtp_timing_enable", "cgtp_timing_collect", "cgtp_stream_probe",
    "cgtp_last_error", "cgtp_version",
]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m clebsch_gordan_tensor_cg_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                 ctypes.c_size_t)
        sig = {
            "cgtp_plan": [ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, vp, i32, i32, i32, u32, vp],
            "cgtp_plan_info": [vp, vp],
            "cgtp_plan_paths": [vp, vp, i32],
            "cgtp_plan_coupling": [vp, i32, vp, i64],
            "cgtp_plan_source": [vp, vp, i64, vp],
            "cgtp_workspace_bytes": [vp, i64, i64, vp],
            "cgtp_forward": [vp, vp, vp, vp, i64, vp, vp, sz, vp],
            "cgtp_tp_backward": [vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, sz, vp],
            "cgtp_conv_forward": [vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, sz, vp],
            "cgtp_backward": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, sz, vp],
            "cgtp_double_backward": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
                                     vp, vp, vp, vp, vp, sz, vp],
            "cgtp_node_order_workspace_bytes": [i64, vp],
            "cgtp_conv_forward_radial": [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, sz, vp],
            "cgtp_sparse_attention": [i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, i64, i64, vp, sz, vp, vp],
            "cgtp_sparse_attention_rows": [i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, i64, i64, i64, vp, vp],
            "cgtp_sparse_attention_layout_bytes": [i64, i64, vp],
            "cgtp_sparse_attention_prepare": [vp, vp, i64, i64, i64, vp, sz, vp],
            "cgtp_conv_forward_vec": [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, sz, vp],
            "cgtp_conv_backward_vec": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, sz,
                                       vp],
            "cgtp_conv_forward_backward": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp, sz, vp],
            "cgtp_conv_forward_backward_vec": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, vp,
                                               vp, sz, vp],
            "cgtp_node_order": [vp, i64, vp, vp, sz, vp],
            "cgtp_csr_workspace_bytes": [i64, i64, vp],
            "cgtp_build_csr": [vp, vp, i64, i64, vp, vp, vp, vp, vp, sz, vp],
            "cgtp_build_csr_order": [vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, sz, vp],
            "cgtp_build_csr_order_noalloc": [vp, vp, i64, i64, vp, vp, vp, vp, vp, vp],
            "cgtp_build_csr_transpose_canonical": [vp, vp, i64, i64, vp, vp, vp],
            "cgtp_validate_csr": [vp, i64, i64, vp, i64, vp, vp],
            "cgtp_sh": [i32, i32, vp, vp, i64, vp, vp],
            "cgtp_sh_vjp_forces": [i32, i32, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, sz, vp],
            "cgtp_force_loss_sh_cotangent": [i32, i32, vp, vp, vp, vp, vp, i64, vp, vp],
            "cgtp_timing_enable": [i32],
            "cgtp_timing_collect": [vp, vp, i32, vp],
            "cgtp_stream_probe": [i32, vp, vp, sz, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.cgtp_plan_destroy.argtypes = [vp]
        L.cgtp_plan_destroy.restype = None
        L.cgtp_last_error.restype = ctypes.c_char_p
        L.cgtp_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise CgtpError(rc, lib().cgtp_last_error().decode())


def _ptr(t):
    # a plain int: ctypes converts it for c_void_p arguments
    return None if t is None else t.data_ptr()


_I32 = torch.int32


class _Args:
    """Argument checks of the marshalling layer, done before any call into
    the library: every tensor on the same CUDA device, contiguous, with the
    exact shape and dtype the call's contract states.  Shapes and dtypes
    are checked first (so that host tensors can exercise them), the device
    last.  Index values (src in range, monotone row_ptr) are not read here:
    cgtp_validate_csr checks untrusted graphs on the device."""

    def __init__(self, call: str):
        self.call = call
        self.seen = []

    def __call__(self, name, t, shape, dtype, optional=True):
        if t is None:
            if not optional:
                raise ValueError(f"{self.call}: {name} is required")
            return None
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.call}: {name} must be a torch.Tensor")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{self.call}: {name}: expected {dtype}, got {t.dtype}")
        # (torch.Size compares equal to a tuple of ints: the common case costs
        # one comparison; the slow path normalises numpy integers)
        if shape is not None and t.shape != shape:
            want = tuple(int(v) for v in shape)
            if tuple(t.shape) != want:
                raise ValueError(f"{self.call}: {name}: expected shape {want}, got {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{self.call}: {name} must be contiguous")
        self.seen.append((name, t))
        return t

    def device(self):
        """All checked tensors on one CUDA device; returns its index.
        (get_device() is an int, -1 on the host: cheaper than building a
        torch.device per tensor, which matters for launch-bound calls.)"""
        dev = None
        for name, t in self.seen:
            d = t.get_device()
            if d < 0:
                raise ValueError(f"{self.call}: {name} is on {t.device}; cgtp runs on the GPU only")
            if dev is None:
                dev = d
            elif d != dev:
                raise ValueError(f"{self.call}: {name} is on {t.device}, other tensors on cuda:{dev}")
        return dev


def _feat(plan):
    return plan.torch_dtype


def _vec_dtype(plan):
    return torch.float64 if plan.dtype == "f64" else torch.float32


def _wshape(plan, n):
    return (plan.weight_numel,) if plan.shared_weights else (n, plan.weight_numel)


def _graph_args(A, plan, N, E, src, dst_row_ptr, node_order, src_row_ptr=None, src_perm=None):
    A("src", src, (E,), _I32, optional=False)
    A("dst_row_ptr", dst_row_ptr, (N + 1,), _I32, optional=False)
    A("node_order", node_order, (N,), _I32)
    A("src_row_ptr", src_row_ptr, (N + 1,), _I32)
    A("src_perm", src_perm, (E,), _I32)


def _vec_args(A, plan, E, vec, vec_perm):
    A("vec_perm", vec_perm, (E,), _I32)
    if vec is None:
        raise ValueError(f"{A.call}: vec is required")
    rows = vec.shape[0] if vec.dim() == 2 else -1
    if vec_perm is None and rows != E:
        raise ValueError(f"{A.call}: vec: expected shape ({E}, 3) without vec_perm, got {tuple(vec.shape)}")
    A("vec", vec, (rows, 3), _vec_dtype(plan))


def _out(A, name, t, shape, dtype, dev_like, want: bool):
    """Caller-given output (checked) or a new one when wanted."""
    if t is not None:
        return A(name, t, shape, dtype)
    if not want:
        return None
    return torch.empty(*shape, dtype=dtype, device=dev_like.device)


def _ws(plan, N, E, ws, dev_like):
    need = cgtp_workspace_bytes(plan, N, E)
    if ws is None:
        return workspace(need, dev_like.device)
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous 1-D uint8 tensor")
    if ws.device != dev_like.device:
        raise ValueError(f"workspace is on {ws.device}, inputs on {dev_like.device}")
    return ws


def _stream(stream=None, like=None):
    """Stream handle: the given stream, else torch's current stream on the
    tensors' device (host tensors: the NULL stream, for argument checks)."""
    if stream is None and like is not None:
        d = like.get_device()
        if d < 0:
            return None
        if _raw_stream is not None:   # torch's cheap accessor for the current stream
            return _raw_stream(d)
        return torch.cuda.current_stream(d).cuda_stream
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


# ---------------------------------------------------------------------------
# plans
# ---------------------------------------------------------------------------
class Plan:
    def __init__(self, irreps_in1: str, irreps_in2: str, irreps_out: str, paths=None, mode: str = "uvu",
                 dtype: str = "f32", shared_weights: bool = False, no_load: bool = False,
                 bf16_weights: bool = False, radial_hidden: int = 0):
        self.dtype = dtype
        self.mode = mode
        self.shared_weights = shared_weights
        self.bf16_weights = bf16_weights
        self.radial_hidden = radial_hidden
        arr, n = None, 0
        if paths:
            n = len(paths)
            arr = (_Path * n)(*[_Path(*p) for p in paths])
        flags = ((CGTP_SHARED_WEIGHTS if shared_weights else 0) | (CGTP_PLAN_NO_LOAD if no_load else 0) |
                 (CGTP_BF16_WEIGHTS if bf16_weights else 0) | (int(radial_hidden) << 16))
        h = ctypes.c_void_p()
        _check(lib().cgtp_plan(irreps_in1.encode(), irreps_in2.encode(), irreps_out.encode(),
                               ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None, n,
                               {"uvu": CGTP_UVU, "uvw": CGTP_UVW}[mode], DTYPES[dtype], flags,
                               ctypes.byref(h)))
        self.handle = h
        d = _Dims()
        _check(lib().cgtp_plan_info(h, ctypes.byref(d)))
        self.dim_in1, self.dim_in2, self.dim_out = d.dim_in1, d.dim_in2, d.dim_out
        self.weight_numel, self.n_paths, self.lmax_in2 = d.weight_numel, d.n_paths, d.lmax_in2
        self.n_kernels, self.cached = d.n_kernels, bool(d.cached)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.cgtp_plan_destroy(h)
            self.handle = None

    @property
    def torch_dtype(self):
        return TORCH_DTYPES[self.dtype]

    @property
    def weight_dtype(self):
        return torch.bfloat16 if self.bf16_weights else TORCH_DTYPES[self.dtype]

    @property
    def out_dtype(self):
        return torch.float64 if self.dtype == "f64" else torch.float32

    def paths(self):
        arr = (_Path * self.n_paths)()
        _check(lib().cgtp_plan_paths(self.handle, ctypes.cast(arr, ctypes.c_void_p), self.n_paths))
        return [(p.i_in1, p.i_in2, p.i_out) for p in arr]

    def coupling(self, p: int, shape):
        import numpy as np
        R = np.empty(shape, dtype=np.float64)
        _check(lib().cgtp_plan_coupling(self.handle, p, R.ctypes.data_as(ctypes.c_void_p), R.size))
        return R

    def source(self) -> str:
        n = ctypes.c_int64()
        _check(lib().cgtp_plan_source(self.handle, None, 0, ctypes.byref(n)))
        buf = ctypes.create_string_buffer(n.value + 1)
        _check(lib().cgtp_plan_source(self.handle, buf, n.value + 1, None))
        return buf.value.decode()


def cgtp_plan(irreps_in1, irreps_in2, irreps_out, paths=None, mode="uvu", dtype="f32",
              shared_weights=False, no_load=False, bf16_weights=False) -> Plan:
    return Plan(irreps_in1, irreps_in2, irreps_out, paths, mode, dtype, shared_weights, no_load, bf16_weights)


# ---------------------------------------------------------------------------
# execution
# ---------------------------------------------------------------------------
def cgtp_workspace_bytes(plan: Plan, n_items: int, n_edges: int = 0) -> int:
    """Workspace bytes that serve every execution call of the plan on at most
    n_items items and n_edges edges."""
    b = ctypes.c_size_t()
    _check(lib().cgtp_workspace_bytes(plan.handle, n_items, n_edges, ctypes.byref(b)))
    return b.value


def workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte-aligned (or better) blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _fwd_ws(plan, N, ws, like):
    # uvu forwards take no workspace (and skip the size query)
    if plan.mode == "uvu" and ws is None:
        return None, 0
    ws = _ws(plan, N, 0, ws, like)
    return ws, ws.numel()


def cgtp_forward(plan: Plan, x, y, w, out=None, ws=None, stream=None):
    A = _Args("cgtp_forward")
    B = x.shape[0]
    A("x", x, (B, plan.dim_in1), _feat(plan), optional=False)
    A("y", y, (B, plan.dim_in2), _feat(plan), optional=False)
    A("w", w, _wshape(plan, B), plan.weight_dtype, optional=False)
    out = _out(A, "out", out, (B, plan.dim_out), plan.out_dtype, x, True)
    A.device()
    ws, nws = _fwd_ws(plan, B, ws, x)
    _check(lib().cgtp_forward(plan.handle, _ptr(x), _ptr(y), _ptr(w), B, _ptr(out), _ptr(ws), nws,
                              _stream(stream, x)))
    return out


def cgtp_tp_backward(plan: Plan, x, y, w, g_out, need=("x", "y", "w"), ws=None, out=None, stream=None):
    """Backward of cgtp_forward; returns (g_x, g_y, g_w), None where not
    requested."""
    A = _Args("cgtp_tp_backward")
    B = x.shape[0]
    A("x", x, (B, plan.dim_in1), _feat(plan), optional=False)
    A("y", y, (B, plan.dim_in2), _feat(plan), optional=False)
    A("w", w, _wshape(plan, B), plan.weight_dtype, optional=False)
    A("g_out", g_out, (B, plan.dim_out), plan.out_dtype, optional=False)
    o = out if out is not None else (None, None, None)
    od = plan.out_dtype
    g_x = _out(A, "g_x", o[0], (B, plan.dim_in1), od, x, out is None and "x" in need)
    g_y = _out(A, "g_y", o[1], (B, plan.dim_in2), od, x, out is None and "y" in need)
    g_w = _out(A, "g_w", o[2], (B, plan.weight_numel), od, x, out is None and "w" in need)
    A.device()
    ws = _ws(plan, B, 0, ws, x)
    _check(lib().cgtp_tp_backward(plan.handle, _ptr(x), _ptr(y), _ptr(w), B, _ptr(g_out), _ptr(g_x), _ptr(g_y),
                                  _ptr(g_w), _ptr(ws), ws.numel(), _stream(stream, x)))
    return g_x, g_y, g_w


def cgtp_conv_forward(plan: Plan, x, sh, w, src, dst_row_ptr, out=None, ws=None, stream=None, node_order=None):
    A = _Args("cgtp_conv_forward")
    N, E = x.shape[0], src.shape[0]
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    A("sh", sh, (E, plan.dim_in2), _feat(plan), optional=False)
    A("w", w, _wshape(plan, E), plan.weight_dtype, optional=False)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order)
    out = _out(A, "out", out, (N, plan.dim_out), plan.out_dtype, x, True)
    A.device()
    ws, nws = _fwd_ws(plan, N, ws, x)
    _check(lib().cgtp_conv_forward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(src), _ptr(dst_row_ptr),
                                   _ptr(node_order), N, E, _ptr(out), _ptr(ws), nws, _stream(stream, x)))
    return out


def cgtp_conv_forward_vec(plan: Plan, x, vec, vec_perm, w, src, dst_row_ptr, out=None, ws=None, stream=None,
                          node_order=None):
    """Convolution with the SH computed in the kernel from the edge vectors."""
    A = _Args("cgtp_conv_forward_vec")
    N, E = x.shape[0], src.shape[0]
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    _vec_args(A, plan, E, vec, vec_perm)
    A("w", w, _wshape(plan, E), plan.weight_dtype, optional=False)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order)
    out = _out(A, "out", out, (N, plan.dim_out), plan.out_dtype, x, True)
    A.device()
    ws, nws = _fwd_ws(plan, N, ws, x)
    _check(lib().cgtp_conv_forward_vec(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(w), _ptr(src),
                                       _ptr(dst_row_ptr), _ptr(node_order), N, E, _ptr(out), _ptr(ws), nws,
                                       _stream(stream, x)))
    return out


def cgtp_conv_forward_radial(plan: Plan, x, vec, vec_perm, radial, w, src, dst_row_ptr, out=None, ws=None,
                             stream=None, node_order=None):
    """uvw convolution with per-edge weights from the radial network:
    radial float32 [2][H], w bf16 [H+1][weight_numel]."""
    A = _Args("cgtp_conv_forward_radial")
    N, E, H = x.shape[0], src.shape[0], plan.radial_hidden
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    _vec_args(A, plan, E, vec, vec_perm)
    A("radial", radial, (2, H), torch.float32, optional=False)
    A("w", w, (H + 1, plan.weight_numel), plan.weight_dtype, optional=False)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order)
    out = _out(A, "out", out, (N, plan.dim_out), torch.float32, x, True)
    A.device()
    ws, nws = _fwd_ws(plan, N, ws, x)
    _check(lib().cgtp_conv_forward_radial(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(radial), _ptr(w),
                                          _ptr(src), _ptr(dst_row_ptr), _ptr(node_order), N, E, _ptr(out), _ptr(ws),
                                          nws, _stream(stream, x)))
    return out


def _bwd_outs(A, plan, N, E, out, need, like, names=("x", "sh", "w")):
    o = out if out is not None else (None,) * len(names)
    od = plan.out_dtype
    shapes = {"x": (N, plan.dim_in1), "sh": (E, plan.dim_in2), "w": (E, plan.weight_numel), "F": (N, 3)}
    return [_out(A, ("g_" + nm) if nm != "F" else "F", t, shapes[nm], od, like, out is None and nm in need)
            for nm, t in zip(names, o)]


def cgtp_backward(plan: Plan, x, sh, w, src, dst_row_ptr, src_row_ptr, src_perm, g_out, need=("x", "sh", "w"),
                  ws=None, out=None, stream=None, node_order=None):
    """Gradient of the convolution; returns (g_x, g_sh, g_w), None where not
    requested."""
    A = _Args("cgtp_backward")
    N, E = x.shape[0], src.shape[0]
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    A("sh", sh, (E, plan.dim_in2), _feat(plan), optional=False)
    A("w", w, _wshape(plan, E), plan.weight_dtype, optional=False)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order, src_row_ptr, src_perm)
    A("g_out", g_out, (N, plan.dim_out), plan.out_dtype, optional=False)
    g_x, g_sh, g_w = _bwd_outs(A, plan, N, E, out, need, x)
    A.device()
    ws = _ws(plan, N, E, ws, x)
    _check(lib().cgtp_backward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(src), _ptr(dst_row_ptr),
                               _ptr(node_order), _ptr(src_row_ptr), _ptr(src_perm), _ptr(g_out), N, E, _ptr(g_x),
                               _ptr(g_sh), _ptr(g_w), _ptr(ws), ws.numel(), _stream(stream, x)))
    return g_x, g_sh, g_w


def cgtp_conv_backward_vec(plan: Plan, x, vec, vec_perm, w, src, dst_row_ptr, src_row_ptr, src_perm, g_out,
                           need=("x", "w", "F"), ws=None, out=None, stream=None, node_order=None):
    """Backward with in-kernel SH; returns (g_x, g_sh, g_w, F), None where not
    requested."""
    A = _Args("cgtp_conv_backward_vec")
    N, E = x.shape[0], src.shape[0]
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    _vec_args(A, plan, E, vec, vec_perm)
    A("w", w, _wshape(plan, E), plan.weight_dtype, optional=False)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order, src_row_ptr, src_perm)
    A("g_out", g_out, (N, plan.dim_out), plan.out_dtype, optional=False)
    g_x, g_sh, g_w, F = _bwd_outs(A, plan, N, E, out, need, x, ("x", "sh", "w", "F"))
    A.device()
    ws = _ws(plan, N, E, ws, x)
    _check(lib().cgtp_conv_backward_vec(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(w), _ptr(src),
                                        _ptr(dst_row_ptr), _ptr(node_order), _ptr(src_row_ptr), _ptr(src_perm),
                                        _ptr(g_out), N, E, _ptr(g_x), _ptr(g_sh), _ptr(g_w), _ptr(F), _ptr(ws),
                                        ws.numel(), _stream(stream, x)))
    return g_x, g_sh, g_w, F


def cgtp_conv_forward_backward(plan: Plan, x, sh, w, src, dst_row_ptr, src_row_ptr, src_perm, g_out,
                               need=("x", "sh", "w"), ws=None, out=None, stream=None, node_order=None):
    """Forward and backward in one pass (g_out must not depend on out);
    returns (out, g_x, g_sh, g_w), None where not requested."""
    A = _Args("cgtp_conv_forward_backward")
    N, E = x.shape[0], src.shape[0]
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    A("sh", sh, (E, plan.dim_in2), _feat(plan), optional=False)
    A("w", w, _wshape(plan, E), plan.weight_dtype, optional=False)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order, src_row_ptr, src_perm)
    A("g_out", g_out, (N, plan.dim_out), plan.out_dtype, optional=False)
    o = _out(A, "out", out[0] if out is not None else None, (N, plan.dim_out), plan.out_dtype, x, True)
    g_x, g_sh, g_w = _bwd_outs(A, plan, N, E, out[1:] if out is not None else None, need, x)
    A.device()
    ws = _ws(plan, N, E, ws, x)
    _check(lib().cgtp_conv_forward_backward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(src), _ptr(dst_row_ptr),
                                            _ptr(node_order), _ptr(src_row_ptr), _ptr(src_perm), _ptr(g_out), N, E,
                                            _ptr(o), _ptr(g_x), _ptr(g_sh), _ptr(g_w), _ptr(ws), ws.numel(),
                                            _stream(stream, x)))
    return o, g_x, g_sh, g_w


def cgtp_conv_forward_backward_vec(plan: Plan, x, vec, vec_perm, w, src, dst_row_ptr, src_row_ptr, src_perm, g_out,
                                   need=("x", "w", "F"), ws=None, out=None, stream=None, node_order=None):
    """Forward and backward in one pass with in-kernel SH; returns
    (out, g_x, g_sh, g_w, F), None where not requested."""
    A = _Args("cgtp_conv_forward_backward_vec")
    N, E = x.shape[0], src.shape[0]
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    _vec_args(A, plan, E, vec, vec_perm)
    A("w", w, _wshape(plan, E), plan.weight_dtype, optional=False)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order, src_row_ptr, src_perm)
    A("g_out", g_out, (N, plan.dim_out), plan.out_dtype, optional=False)
    o = _out(A, "out", out[0] if out is not None else None, (N, plan.dim_out), plan.out_dtype, x, True)
    g_x, g_sh, g_w, F = _bwd_outs(A, plan, N, E, out[1:] if out is not None else None, need, x,
                                  ("x", "sh", "w", "F"))
    A.device()
    ws = _ws(plan, N, E, ws, x)
    _check(lib().cgtp_conv_forward_backward_vec(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(w), _ptr(src),
                                                _ptr(dst_row_ptr), _ptr(node_order), _ptr(src_row_ptr),
                                                _ptr(src_perm), _ptr(g_out), N, E, _ptr(o), _ptr(g_x), _ptr(g_sh),
                                                _ptr(g_w), _ptr(F), _ptr(ws), ws.numel(), _stream(stream, x)))
    return o, g_x, g_sh, g_w, F


def cgtp_double_backward(plan: Plan, x, sh, w, g_out, gg_x, gg_sh, gg_w, src, dst_row_ptr, src_row_ptr, src_perm,
                         need=("g_out", "x", "sh", "w"), ws=None, out=None, stream=None, node_order=None):
    """Second derivatives for cotangents (gg_x, gg_sh, gg_w) on the backward's
    outputs; returns (d_g_out, d_x, d_sh, d_w), None where not requested."""
    A = _Args("cgtp_double_backward")
    N, E = x.shape[0], src.shape[0]
    A("x", x, (N, plan.dim_in1), _feat(plan), optional=False)
    A("sh", sh, (E, plan.dim_in2), _feat(plan), optional=gg_x is None and gg_w is None)
    A("w", w, _wshape(plan, E), plan.weight_dtype, optional=False)
    A("g_out", g_out, (N, plan.dim_out), plan.out_dtype, optional=False)
    A("gg_x", gg_x, (N, plan.dim_in1), _feat(plan))
    A("gg_sh", gg_sh, (E, plan.dim_in2), _feat(plan))
    A("gg_w", gg_w, _wshape(plan, E), plan.weight_dtype)
    _graph_args(A, plan, N, E, src, dst_row_ptr, node_order, src_row_ptr, src_perm)
    o = out if out is not None else (None,) * 4
    od = plan.out_dtype
    shapes = [(N, plan.dim_out), (N, plan.dim_in1), (E, plan.dim_in2), (E, plan.weight_numel)]
    d = [_out(A, "d_" + nm, t, sh_, od, x, out is None and nm in need)
         for nm, t, sh_ in zip(("g_out", "x", "sh", "w"), o, shapes)]
    A.device()
    ws = _ws(plan, N, E, ws, x)
    _check(lib().cgtp_double_backward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(g_out), _ptr(gg_x),
                                      _ptr(gg_sh), _ptr(gg_w), _ptr(src), _ptr(dst_row_ptr), _ptr(node_order),
                                      _ptr(src_row_ptr), _ptr(src_perm), N, E, _ptr(d[0]), _ptr(d[1]), _ptr(d[2]),
                                      _ptr(d[3]), _ptr(ws), ws.numel(), _stream(stream, x)))
    return tuple(d)


def cgtp_node_order(row_ptr, ws=None, out=None, stream=None):
    """Rows of a CSR by decreasing length (processing order for the
    convolution calls)."""
    A = _Args("cgtp_node_order")
    n = row_ptr.shape[0] - 1
    A("row_ptr", row_ptr, (n + 1,), _I32, optional=False)
    order = _out(A, "out", out, (n,), _I32, row_ptr, True)
    A.device()
    b = ctypes.c_size_t()
    _check(lib().cgtp_node_order_workspace_bytes(n, ctypes.byref(b)))
    if ws is None:
        ws = workspace(b.value, row_ptr.device)
    _check(lib().cgtp_node_order(_ptr(row_ptr), n, _ptr(order), _ptr(ws), ws.numel(), _stream(stream, row_ptr)))
    return order


def cgtp_sparse_attention_prepare(col, row_ptr, n_cols: int, out=None, stream=None):
    """Compacted window layout of a CSR graph for cgtp_sparse_attention."""
    A = _Args("cgtp_sparse_attention_prepare")
    n_rows, E = row_ptr.shape[0] - 1, col.shape[0]
    A("col", col, (E,), _I32, optional=False)
    A("row_ptr", row_ptr, (n_rows + 1,), _I32, optional=False)
    A.device()
    b = ctypes.c_size_t()
    _check(lib().cgtp_sparse_attention_layout_bytes(n_rows, E, ctypes.byref(b)))
    layout = workspace(b.value, row_ptr.device) if out is None else out
    if layout.numel() < b.value or layout.device != row_ptr.device:
        raise ValueError(f"cgtp_sparse_attention_prepare: layout needs {b.value} bytes on {row_ptr.device}")
    _check(lib().cgtp_sparse_attention_prepare(_ptr(col), _ptr(row_ptr), n_rows, n_cols, E, _ptr(layout),
                                               layout.numel(), _stream(stream, row_ptr)))
    return layout


def _attn_args(A, q, k, v, row_ptr, out):
    n_rows = row_ptr.shape[0] - 1
    H, D = q.shape[1], q.shape[2]
    A("q", q, (n_rows, H, D), torch.bfloat16, optional=False)
    A("k", k, (k.shape[0], H, D), torch.bfloat16, optional=False)
    A("v", v, (k.shape[0], H, D), torch.bfloat16, optional=False)
    A("row_ptr", row_ptr, (n_rows + 1,), _I32, optional=False)
    return n_rows, H, D, _out(A, "out", out, (n_rows, H, D), torch.float32, q, True)


def cgtp_sparse_attention(q, k, v, row_ptr, n_edges: int, layout, scale=None, out=None, stream=None):
    """Graph sparse attention per head: q [n_rows][H][D], k and v
    [n_cols][H][D] (bf16) over a graph prepared by
    cgtp_sparse_attention_prepare; returns float32 [n_rows][H][D]."""
    A = _Args("cgtp_sparse_attention")
    n_rows, H, D, out = _attn_args(A, q, k, v, row_ptr, out)
    A("layout", layout, (layout.shape[0],), torch.uint8, optional=False)
    A.device()
    if scale is None:
        scale = 1.0 / D ** 0.5
    _check(lib().cgtp_sparse_attention(DTYPES["bf16"], H, D, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                       n_rows, n_edges, _ptr(layout), layout.numel(), _ptr(out), _stream(stream, q)))
    return out


def cgtp_sparse_attention_rows(q, k, v, col, row_ptr, scale=None, out=None, stream=None):
    """The same attention in row form, straight from the CSR (col, row_ptr):
    q [n_rows][H][D], k and v [n_cols][H][D] (bf16); returns float32
    [n_rows][H][D]."""
    A = _Args("cgtp_sparse_attention_rows")
    n_rows, H, D, out = _attn_args(A, q, k, v, row_ptr, out)
    A("col", col, (col.shape[0],), _I32, optional=False)
    A.device()
    if scale is None:
        scale = 1.0 / D ** 0.5
    _check(lib().cgtp_sparse_attention_rows(DTYPES["bf16"], H, D, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(col),
                                            _ptr(row_ptr), n_rows, k.shape[0], col.shape[0], _ptr(out),
                                            _stream(stream, q)))
    return out


def cgtp_csr_workspace_bytes(n_edges: int, n_keys: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().cgtp_csr_workspace_bytes(n_edges, n_keys, ctypes.byref(b)))
    return b.value


def _csr_outputs(A, key, n_keys, val, sorted_key, ws, out):
    E = key.shape[0]
    A("key", key, (E,), _I32, optional=False)
    A("val", val, (E,), _I32)
    o = out if out is not None else (None, None, None, None)
    perm = _out(A, "perm", o[0], (E,), _I32, key, True)
    row_ptr = _out(A, "row_ptr", o[1], (n_keys + 1,), _I32, key, True)
    sk = _out(A, "sorted_key", o[2], (E,), _I32, key, out is None and sorted_key)
    sv = _out(A, "sorted_val", o[3], (E,), _I32, key, out is None and val is not None)
    A.device()
    if ws is None:
        ws = workspace(cgtp_csr_workspace_bytes(E, n_keys), key.device)
    return E, perm, row_ptr, sk, sv, ws


def cgtp_build_csr(key, n_keys: int, val=None, sorted_key: bool = True, ws=None, out=None, stream=None):
    """Returns (perm, row_ptr, sorted_key or None, sorted_val or None)."""
    A = _Args("cgtp_build_csr")
    E, perm, row_ptr, sk, sv, ws = _csr_outputs(A, key, n_keys, val, sorted_key, ws, out)
    _check(lib().cgtp_build_csr(_ptr(key), _ptr(val), E, n_keys, _ptr(perm), _ptr(row_ptr), _ptr(sk), _ptr(sv),
                                _ptr(ws), ws.numel(), _stream(stream, key)))
    return perm, row_ptr, sk, sv


def cgtp_build_csr_order(key, n_keys: int, val=None, sorted_key: bool = True, ws=None, out=None, order=None,
                         stream=None):
    """cgtp_build_csr plus the longest-first node order (cgtp_node_order's)
    from the same launches.  Returns (perm, row_ptr, sorted_key or None,
    sorted_val or None, order)."""
    A = _Args("cgtp_build_csr_order")
    order = _out(A, "order", order, (n_keys,), _I32, key, True)
    E, perm, row_ptr, sk, sv, ws = _csr_outputs(A, key, n_keys, val, sorted_key, ws, out)
    _check(lib().cgtp_build_csr_order(_ptr(key), _ptr(val), E, n_keys, _ptr(perm), _ptr(row_ptr), _ptr(sk),
                                      _ptr(sv), _ptr(order), _ptr(ws), ws.numel(), _stream(stream, key)))
    return perm, row_ptr, sk, sv, order


def cgtp_build_csr_transpose_canonical(src, perm, n_keys: int, out=None, stream=None):
    """Transpose CSR (by source) of a canonical edge list (sorted by source,
    ties by destination) from its destination CSR's perm; the same arrays
    cgtp_build_csr gives for the destination-sorted sources.  Returns
    (src_perm, src_row_ptr)."""
    A = _Args("cgtp_build_csr_transpose_canonical")
    E = src.shape[0]
    A("src", src, (E,), _I32, optional=False)
    A("perm", perm, (E,), _I32, optional=False)
    o = out if out is not None else (None, None)
    src_perm = _out(A, "src_perm", o[0], (E,), _I32, src, True)
    src_row_ptr = _out(A, "src_row_ptr", o[1], (n_keys + 1,), _I32, src, True)
    A.device()
    _check(lib().cgtp_build_csr_transpose_canonical(_ptr(src), _ptr(perm), E, n_keys, _ptr(src_perm),
                                                    _ptr(src_row_ptr), _stream(stream, src)))
    return src_perm, src_row_ptr


def cgtp_build_csr_order_noalloc(key, n_keys: int, val=None, sorted_key: bool = True, out=None, order=None,
                                 stream=None):
    """cgtp_build_csr_order with the library's fixed device scratch instead
    of a workspace (for callers that cannot allocate; calls on one GPU must
    not overlap).  Returns (perm, row_ptr, sorted_key or None, sorted_val or
    None, order or None); order is written only when given."""
    A = _Args("cgtp_build_csr_order_noalloc")
    E = key.shape[0]
    A("key", key, (E,), _I32, optional=False)
    A("val", val, (E,), _I32)
    o = out if out is not None else (None, None, None, None)
    perm = _out(A, "perm", o[0], (E,), _I32, key, True)
    row_ptr = _out(A, "row_ptr", o[1], (n_keys + 1,), _I32, key, True)
    sk = _out(A, "sorted_key", o[2], (E,), _I32, key, out is None and sorted_key)
    sv = _out(A, "sorted_val", o[3], (E,), _I32, key, out is None and val is not None)
    A("order", order, (n_keys,), _I32)
    A.device()
    _check(lib().cgtp_build_csr_order_noalloc(_ptr(key), _ptr(val), E, n_keys, _ptr(perm), _ptr(row_ptr), _ptr(sk),
                                              _ptr(sv), _ptr(order), _stream(stream, key)))
    return perm, row_ptr, sk, sv, order


def cgtp_validate_csr(row_ptr, n_edges: int, idx=None, n_idx_range: int = 0, stream=None) -> bool:
    A = _Args("cgtp_validate_csr")
    A("row_ptr", row_ptr, (row_ptr.shape[0],), _I32, optional=False)
    A("idx", idx, (n_edges,), _I32)
    A.device()
    ws = workspace(256, row_ptr.device)
    rc = lib().cgtp_validate_csr(_ptr(row_ptr), row_ptr.shape[0] - 1, n_edges, _ptr(idx), n_idx_range,
                                 _ptr(ws), _stream(stream, row_ptr))
    if rc == -5:
        return False
    _check(rc)
    return True


def _sh_vec(A, vec, perm, n, dtype):
    A("perm", perm, (n,), _I32)
    rows = vec.shape[0] if vec.dim() == 2 else -1
    if perm is None and rows != n:
        raise ValueError(f"{A.call}: vec: expected shape ({n}, 3) without perm, got {tuple(vec.shape)}")
    A("vec", vec, (rows, 3), torch.float64 if dtype == "f64" else torch.float32, optional=False)


def cgtp_sh(lmax: int, vec, perm=None, dtype: str = "f32", out=None, stream=None):
    """Real SH rows of degrees 0..lmax of the edge vectors vec[perm[t]]."""
    A = _Args("cgtp_sh")
    n = perm.shape[0] if perm is not None else vec.shape[0]
    _sh_vec(A, vec, perm, n, dtype)
    out = _out(A, "out", out, (n, (lmax + 1) ** 2), TORCH_DTYPES[dtype], vec, True)
    A.device()
    _check(lib().cgtp_sh(lmax, DTYPES[dtype], _ptr(vec), _ptr(perm), n, _ptr(out), _stream(stream, vec)))
    return out


def cgtp_sh_vjp_forces(lmax: int, vec, perm, g_sh, dst_row_ptr, src_row_ptr, src_perm, dtype: str = "f32",
                       need=("F",), ws=None, out=None, stream=None):
    """Per-edge SH vector-Jacobian products g_vec = J^T g_sh and the atom
    forces they imply; returns (g_vec, F), None where not requested
    (need: "vec", "F")."""
    A = _Args("cgtp_sh_vjp_forces")
    E = g_sh.shape[0]
    N = dst_row_ptr.shape[0] - 1 if dst_row_ptr is not None else 0
    td = TORCH_DTYPES[dtype]
    _sh_vec(A, vec, perm, E, dtype)
    A("g_sh", g_sh, (E, (lmax + 1) ** 2), td, optional=False)
    want_F = (out is None and "F" in need) or (out is not None and out[1] is not None)
    A("dst_row_ptr", dst_row_ptr, (N + 1,), _I32, optional=not want_F)
    A("src_row_ptr", src_row_ptr, (N + 1,), _I32, optional=not want_F)
    A("src_perm", src_perm, (E,), _I32, optional=not want_F)
    o = out if out is not None else (None, None)
    g_vec = _out(A, "g_vec", o[0], (E, 3), td, g_sh, out is None and "vec" in need)
    F = _out(A, "F", o[1], (N, 3), td, g_sh, out is None and "F" in need)
    A.device()
    nb = 0 if g_vec is not None else E * 3 * (8 if dtype == "f64" else 4)
    if ws is None and nb:
        ws = workspace(nb, g_sh.device)
    _check(lib().cgtp_sh_vjp_forces(lmax, DTYPES[dtype], _ptr(vec), _ptr(perm), _ptr(g_sh), _ptr(dst_row_ptr),
                                    _ptr(src_row_ptr), _ptr(src_perm), N, E, _ptr(g_vec), _ptr(F), _ptr(ws),
                                    ws.numel() if ws is not None else 0, _stream(stream, g_sh)))
    return g_vec, F


def cgtp_force_loss_sh_cotangent(lmax: int, vec, perm, src, dst, F, dtype: str = "f32", out=None,
                                 stream=None):
    A = _Args("cgtp_force_loss_sh_cotangent")
    E = src.shape[0]
    td = TORCH_DTYPES[dtype]
    _sh_vec(A, vec, perm, E, dtype)
    A("src", src, (E,), _I32, optional=False)
    A("dst", dst, (E,), _I32, optional=False)
    A("F", F, (F.shape[0], 3), td, optional=False)
    out = _out(A, "out", out, (E, (lmax + 1) ** 2), td, F, True)
    A.device()
    _check(lib().cgtp_force_loss_sh_cotangent(lmax, DTYPES[dtype], _ptr(vec), _ptr(perm), _ptr(src), _ptr(dst),
                                              _ptr(F), E, _ptr(out), _stream(stream, F)))
    return out


def cgtp_timing_enable(enable: bool = True):
    _check(lib().cgtp_timing_enable(1 if enable else 0))


def cgtp_timing_collect(cap: int = 1 << 16):
    """[(kernel name, ms)] of the launches recorded since the last collect."""
    names = ctypes.create_string_buffer(64 * cap)
    ms = (ctypes.c_float * cap)()
    n = ctypes.c_int32()
    _check(lib().cgtp_timing_collect(ctypes.cast(names, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p), cap,
                                     ctypes.byref(n)))
    raw = names.raw
    return [(raw[64 * i:64 * i + 64].split(b"\0", 1)[0].decode(), float(ms[i])) for i in range(n.value)]


STREAM_PROBE_KINDS = {"read": 0, "write": 1, "copy": 2}


def cgtp_stream_probe(kind: str, src, dst, stream=None):
    """One streaming launch over dst (and src): kind "read" reads src (dst
    receives at most 4 bytes), "write" writes dst, "copy" copies src into
    dst.  Both CUDA tensors of one device, byte sizes equal (read: src's
    size) and a multiple of 16."""
    if kind not in STREAM_PROBE_KINDS:
        raise ValueError(f"kind must be one of {sorted(STREAM_PROBE_KINDS)}")
    ts = [t for t in (src, dst) if t is not None]
    if dst is None or (kind != "write" and src is None):
        raise ValueError("stream probe needs dst (and src unless kind is 'write')")
    for t in ts:
        if not t.is_cuda or not t.is_contiguous() or t.device != dst.device:
            raise ValueError("stream probe buffers must be contiguous CUDA tensors on one device")
    nbytes = (src if kind != "write" else dst).numel() * (src if kind != "write" else dst).element_size()
    if kind == "copy" and dst.numel() * dst.element_size() != nbytes:
        raise ValueError("copy: src and dst sizes differ")
    _check(lib().cgtp_stream_probe(STREAM_PROBE_KINDS[kind], _ptr(src), _ptr(dst), nbytes, _stream(stream, dst)))


def version() -> str:
    return lib().cgtp_version().decode()


# ---------------------------------------------------------------------------
# ahead-of-time compilation of the standard workloads' kernels
# ---------------------------------------------------------------------------
def standard_plan_args():
    from . import workloads as W
    out = []
    for name in ("c1", "c2", "c3", "c5"):
        c = W.config(name)
        out.append(dict(irreps_in1=c.irreps_in1, irreps_in2=c.irreps_in2, irreps_out=c.irreps_out,
                        paths=c.paths, mode=c.mode, dtype=c.dtype, shared_weights=c.shared_weights))
    out.append(dict(out[1], bf16_weights=True))   # the 4096-atom box with bf16 weight storage
    return out


def precompile_standard_plans():
    for kw in standard_plan_args():
        Plan(**kw, no_load=True)
