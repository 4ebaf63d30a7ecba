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
    "cgtp_plan_destroy", "cgtp_forward_workspace_bytes", "cgtp_forward", "cgtp_conv_forward",
    "cgtp_conv_workspace_bytes", "cgtp_conv_forward_vec", "cgtp_conv_backward_vec", "cgtp_conv_forward_radial", "cgtp_sparse_attention", "cgtp_sparse_attention_rows",
    "cgtp_conv_forward_backward", "cgtp_conv_forward_backward_vec",
    "cgtp_sparse_attention_layout_bytes", "cgtp_sparse_attention_prepare",
    "cgtp_conv_backward", "cgtp_conv_double_backward", "cgtp_csr_workspace_bytes", "cgtp_build_csr",
    "cgtp_build_csr_order",
    "cgtp_validate_csr", "cgtp_node_order_workspace_bytes", "cgtp_node_order", "cgtp_spherical_harmonics", "cgtp_forces_workspace_bytes", "cgtp_sh_forces",
    "cgtp_force_loss_sh_cotangent", "cgtp_timing_enable", "cgtp_timing_collect", "cgtp_last_error",
    "cgtp_version",
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
            "cgtp_forward_workspace_bytes": [vp, i64, vp],
            "cgtp_forward": [vp, vp, vp, vp, i64, vp, vp, sz, vp],
            "cgtp_conv_forward": [vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, sz, vp],
            "cgtp_conv_workspace_bytes": [vp, i64, i64, vp],
            "cgtp_conv_backward": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, sz, vp],
            "cgtp_conv_double_backward": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64,
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
            "cgtp_validate_csr": [vp, i64, i64, vp, i64, vp, vp],
            "cgtp_spherical_harmonics": [i32, i32, vp, vp, i64, vp, vp],
            "cgtp_forces_workspace_bytes": [i64, i32, vp],
            "cgtp_sh_forces": [i32, i32, vp, vp, vp, vp, vp, vp, i64, i64, vp, vp, sz, vp],
            "cgtp_force_loss_sh_cotangent": [i32, i32, vp, vp, vp, vp, vp, i64, vp, vp],
            "cgtp_timing_enable": [i32],
            "cgtp_timing_collect": [vp, vp, i32, vp],
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
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to cgtp must be contiguous")
    return t.data_ptr()


def _want(plan, **tensors):
    """Argument check of the marshalling layer: feature-like tensors in the
    plan's storage type, weight-like tensors in its weight storage type,
    index tensors int32 (None entries are skipped)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if name in ("w", "gg_w"):
            want = plan.weight_dtype
        elif name in ("src", "dst", "dst_row_ptr", "src_row_ptr", "src_perm", "vec_perm", "node_order"):
            want = torch.int32
        elif name == "vec":
            want = torch.float64 if plan.dtype == "f64" else torch.float32
        else:
            want = plan.torch_dtype
        if t.dtype != want:
            raise TypeError(f"{name}: expected {want}, got {t.dtype}")


def _stream(stream=None, like=None):
    """Stream handle: the given stream, else torch's current stream on the
    tensors' device (host tensors: the NULL stream, for argument checks)."""
    if stream is None and like is not None:
        if not like.is_cuda:
            return None
        if _raw_stream is not None:   # torch's cheap accessor for the current stream
            return _raw_stream(like.device.index)
        return torch.cuda.current_stream(like.device).cuda_stream
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
def cgtp_forward_workspace_bytes(plan: Plan, n_items: int) -> int:
    if plan.mode == "uvu":
        return 0   # uvu forwards take no workspace
    b = ctypes.c_size_t()
    _check(lib().cgtp_forward_workspace_bytes(plan.handle, n_items, ctypes.byref(b)))
    return b.value


def cgtp_forward(plan: Plan, x, y, w, out=None, ws=None, stream=None):
    _want(plan, x=x, y=y, w=w)
    B = x.shape[0]
    if out is None:
        out = torch.empty(B, plan.dim_out, dtype=plan.out_dtype, device=x.device)
    nb = cgtp_forward_workspace_bytes(plan, B)
    if ws is None and nb:
        ws = workspace(nb, x.device)
    _check(lib().cgtp_forward(plan.handle, _ptr(x), _ptr(y), _ptr(w), B, _ptr(out), _ptr(ws),
                              ws.numel() if ws is not None else 0, _stream(stream, x)))
    return out


def cgtp_conv_forward(plan: Plan, x, sh, w, src, dst_row_ptr, out=None, ws=None, stream=None, node_order=None):
    _want(plan, x=x, sh=sh, w=w, src=src, dst_row_ptr=dst_row_ptr, node_order=node_order)
    N, E = x.shape[0], src.shape[0]
    if out is None:
        out = torch.empty(N, plan.dim_out, dtype=plan.out_dtype, device=x.device)
    nb = cgtp_forward_workspace_bytes(plan, N)
    if ws is None and nb:
        ws = workspace(nb, x.device)
    _check(lib().cgtp_conv_forward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(src), _ptr(dst_row_ptr),
                                   _ptr(node_order), N, E, _ptr(out), _ptr(ws), ws.numel() if ws is not None else 0,
                                   _stream(stream, x)))
    return out


def cgtp_conv_forward_vec(plan: Plan, x, vec, vec_perm, w, src, dst_row_ptr, out=None, ws=None, stream=None,
                          node_order=None):
    """Convolution with the SH computed in the kernel from the edge vectors."""
    _want(plan, x=x, vec=vec, vec_perm=vec_perm, w=w, src=src, dst_row_ptr=dst_row_ptr, node_order=node_order)
    N, E = x.shape[0], src.shape[0]
    if out is None:
        out = torch.empty(N, plan.dim_out, dtype=plan.out_dtype, device=x.device)
    nb = cgtp_forward_workspace_bytes(plan, N)
    if ws is None and nb:
        ws = workspace(nb, x.device)
    _check(lib().cgtp_conv_forward_vec(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(w), _ptr(src),
                                       _ptr(dst_row_ptr), _ptr(node_order), N, E, _ptr(out), _ptr(ws),
                                       ws.numel() if ws is not None else 0, _stream(stream, x)))
    return out


def cgtp_conv_forward_radial(plan: Plan, x, vec, vec_perm, radial, w, src, dst_row_ptr, out=None, ws=None,
                             stream=None, node_order=None):
    """uvw convolution with per-edge weights from the radial network:
    radial float32 [2][H], w bf16 [H+1][weight_numel]."""
    _want(plan, x=x, vec=vec, vec_perm=vec_perm, w=w, src=src, dst_row_ptr=dst_row_ptr, node_order=node_order)
    if radial.dtype != torch.float32:
        raise TypeError(f"radial: expected torch.float32, got {radial.dtype}")
    N, E = x.shape[0], src.shape[0]
    if out is None:
        out = torch.empty(N, plan.dim_out, dtype=torch.float32, device=x.device)
    nb = cgtp_forward_workspace_bytes(plan, N)
    if ws is None and nb:
        ws = workspace(nb, x.device)
    _check(lib().cgtp_conv_forward_radial(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(radial), _ptr(w),
                                          _ptr(src), _ptr(dst_row_ptr), _ptr(node_order), N, E, _ptr(out), _ptr(ws),
                                          ws.numel() if ws is not None else 0, _stream(stream, x)))
    return out


def cgtp_conv_backward_vec(plan: Plan, x, vec, vec_perm, w, src, dst_row_ptr, src_row_ptr, src_perm, g_out,
                           need=("x", "w", "F"), ws=None, out=None, stream=None, node_order=None):
    """Backward with in-kernel SH; returns (g_x, g_sh, g_w, F), None where not
    requested."""
    _want(plan, x=x, vec=vec, vec_perm=vec_perm, w=w, src=src, dst_row_ptr=dst_row_ptr, src_row_ptr=src_row_ptr,
          src_perm=src_perm, g_out=g_out, node_order=node_order)
    N, E = x.shape[0], src.shape[0]
    dev = x.device
    od = plan.out_dtype
    if out is None:
        g_x = torch.empty(N, plan.dim_in1, dtype=od, device=dev) if "x" in need else None
        g_sh = torch.empty(E, plan.dim_in2, dtype=od, device=dev) if "sh" in need else None
        g_w = torch.empty(E, plan.weight_numel, dtype=od, device=dev) if "w" in need else None
        F = torch.empty(N, 3, dtype=od, device=dev) if "F" in need else None
    else:
        g_x, g_sh, g_w, F = out
    if ws is None:
        ws = workspace(cgtp_conv_workspace_bytes(plan, N, E), dev)
    _check(lib().cgtp_conv_backward_vec(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(w), _ptr(src),
                                        _ptr(dst_row_ptr), _ptr(node_order), _ptr(src_row_ptr), _ptr(src_perm),
                                        _ptr(g_out), N, E, _ptr(g_x), _ptr(g_sh), _ptr(g_w), _ptr(F), _ptr(ws),
                                        ws.numel(), _stream(stream, x)))
    return g_x, g_sh, g_w, F


def cgtp_conv_forward_backward(plan: Plan, x, sh, w, src, dst_row_ptr, src_row_ptr, src_perm, g_out,
                               need=("x", "sh", "w"), ws=None, out=None, stream=None, node_order=None):
    """Forward and backward in one pass (g_out must not depend on out);
    returns (out, g_x, g_sh, g_w), None where not requested."""
    _want(plan, x=x, sh=sh, w=w, src=src, dst_row_ptr=dst_row_ptr, src_row_ptr=src_row_ptr, src_perm=src_perm,
          g_out=g_out, node_order=node_order)
    N, E = x.shape[0], src.shape[0]
    dev = x.device
    od = plan.out_dtype
    if out is None:
        o = torch.empty(N, plan.dim_out, dtype=od, device=dev)
        g_x = torch.empty(N, plan.dim_in1, dtype=od, device=dev) if "x" in need else None
        g_sh = torch.empty(E, plan.dim_in2, dtype=od, device=dev) if "sh" in need else None
        g_w = torch.empty(E, plan.weight_numel, dtype=od, device=dev) if "w" in need else None
    else:
        o, g_x, g_sh, g_w = out
    if ws is None:
        ws = workspace(cgtp_conv_workspace_bytes(plan, N, E), dev)
    _check(lib().cgtp_conv_forward_backward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(src), _ptr(dst_row_ptr),
                                            _ptr(node_order), _ptr(src_row_ptr), _ptr(src_perm), _ptr(g_out), N, E,
                                            _ptr(o), _ptr(g_x), _ptr(g_sh), _ptr(g_w), _ptr(ws), ws.numel(),
                                            _stream(stream, x)))
    return o, g_x, g_sh, g_w


def cgtp_conv_forward_backward_vec(plan: Plan, x, vec, vec_perm, w, src, dst_row_ptr, src_row_ptr, src_perm, g_out,
                                   need=("x", "w", "F"), ws=None, out=None, stream=None, node_order=None):
    """Forward and backward in one pass with in-kernel SH; returns
    (out, g_x, g_sh, g_w, F), None where not requested."""
    _want(plan, x=x, vec=vec, vec_perm=vec_perm, w=w, src=src, dst_row_ptr=dst_row_ptr, src_row_ptr=src_row_ptr,
          src_perm=src_perm, g_out=g_out, node_order=node_order)
    N, E = x.shape[0], src.shape[0]
    dev = x.device
    od = plan.out_dtype
    if out is None:
        o = torch.empty(N, plan.dim_out, dtype=od, device=dev)
        g_x = torch.empty(N, plan.dim_in1, dtype=od, device=dev) if "x" in need else None
        g_sh = torch.empty(E, plan.dim_in2, dtype=od, device=dev) if "sh" in need else None
        g_w = torch.empty(E, plan.weight_numel, dtype=od, device=dev) if "w" in need else None
        F = torch.empty(N, 3, dtype=od, device=dev) if "F" in need else None
    else:
        o, g_x, g_sh, g_w, F = out
    if ws is None:
        ws = workspace(cgtp_conv_workspace_bytes(plan, N, E), dev)
    _check(lib().cgtp_conv_forward_backward_vec(plan.handle, _ptr(x), _ptr(vec), _ptr(vec_perm), _ptr(w), _ptr(src),
                                                _ptr(dst_row_ptr), _ptr(node_order), _ptr(src_row_ptr),
                                                _ptr(src_perm), _ptr(g_out), N, E, _ptr(o), _ptr(g_x), _ptr(g_sh),
                                                _ptr(g_w), _ptr(F), _ptr(ws), ws.numel(), _stream(stream, x)))
    return o, g_x, g_sh, g_w, F


def cgtp_conv_workspace_bytes(plan: Plan, n_nodes: int, n_edges: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().cgtp_conv_workspace_bytes(plan.handle, n_nodes, n_edges, ctypes.byref(b)))
    return b.value


def workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte-aligned (or better) blocks
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def cgtp_conv_backward(plan: Plan, x, sh, w, src, dst, dst_row_ptr, src_row_ptr, src_perm, g_out,
                       need=("x", "sh", "w"), ws=None, out=None, stream=None, node_order=None):
    _want(plan, x=x, sh=sh, w=w, src=src, dst=dst, dst_row_ptr=dst_row_ptr, src_row_ptr=src_row_ptr,
          src_perm=src_perm, g_out=g_out, node_order=node_order)
    N, E = x.shape[0], src.shape[0]
    dev = x.device
    od = plan.out_dtype
    g_x, g_sh, g_w = out if out is not None else (None, None, None)
    if out is None:
        g_x = torch.empty(N, plan.dim_in1, dtype=od, device=dev) if "x" in need else None
        g_sh = torch.empty(E, plan.dim_in2, dtype=od, device=dev) if "sh" in need else None
        g_w = torch.empty(E, plan.weight_numel, dtype=od, device=dev) if "w" in need else None
    nb = cgtp_conv_workspace_bytes(plan, N, E)
    if ws is None:
        ws = workspace(nb, dev)
    _check(lib().cgtp_conv_backward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(src), _ptr(dst),
                                    _ptr(dst_row_ptr), _ptr(node_order), _ptr(src_row_ptr), _ptr(src_perm),
                                    _ptr(g_out), N, E, _ptr(g_x), _ptr(g_sh), _ptr(g_w), _ptr(ws), ws.numel(),
                                    _stream(stream, x)))
    return g_x, g_sh, g_w


def cgtp_conv_double_backward(plan: Plan, x, sh, w, src, dst, dst_row_ptr, src_row_ptr, src_perm, g_out,
                              gg_x=None, gg_sh=None, gg_w=None, need=("g_out", "x", "sh", "w"), ws=None,
                              out=None, stream=None, node_order=None):
    _want(plan, x=x, sh=sh, w=w, src=src, dst=dst, dst_row_ptr=dst_row_ptr, src_row_ptr=src_row_ptr,
          src_perm=src_perm, g_out=g_out, gg_x=gg_x, gg_sh=gg_sh, gg_w=gg_w, node_order=node_order)
    N, E = x.shape[0], src.shape[0]
    dev = x.device
    od = plan.out_dtype
    if out is None:
        d_g = torch.empty(N, plan.dim_out, dtype=od, device=dev) if "g_out" in need else None
        d_x = torch.empty(N, plan.dim_in1, dtype=od, device=dev) if "x" in need else None
        d_sh = torch.empty(E, plan.dim_in2, dtype=od, device=dev) if "sh" in need else None
        d_w = torch.empty(E, plan.weight_numel, dtype=od, device=dev) if "w" in need else None
    else:
        d_g, d_x, d_sh, d_w = out
    nb = cgtp_conv_workspace_bytes(plan, N, E)
    if ws is None:
        ws = workspace(nb, dev)
    _check(lib().cgtp_conv_double_backward(plan.handle, _ptr(x), _ptr(sh), _ptr(w), _ptr(src), _ptr(dst),
                                           _ptr(dst_row_ptr), _ptr(node_order), _ptr(src_row_ptr),
                                           _ptr(src_perm), _ptr(g_out), _ptr(gg_x), _ptr(gg_sh), _ptr(gg_w), N, E, _ptr(d_g), _ptr(d_x),
                                           _ptr(d_sh), _ptr(d_w), _ptr(ws), ws.numel(), _stream(stream, x)))
    return d_g, d_x, d_sh, d_w


def cgtp_node_order(row_ptr, ws=None, out=None, stream=None):
    """Rows of a CSR by decreasing length (processing order for the
    convolution calls)."""
    n = row_ptr.shape[0] - 1
    order = torch.empty(n, dtype=torch.int32, device=row_ptr.device) if out is None else out
    b = ctypes.c_size_t()
    _check(lib().cgtp_node_order_workspace_bytes(n, ctypes.byref(b)))
    if ws is None:
        ws = workspace(b.value, row_ptr.device)
    _check(lib().cgtp_node_order(_ptr(row_ptr), n, _ptr(order), _ptr(ws), ws.numel(), _stream(stream, row_ptr)))
    return order


def cgtp_sparse_attention_prepare(col, row_ptr, n_cols: int, out=None, stream=None):
    """Compacted window layout of a CSR graph for cgtp_sparse_attention."""
    n_rows = row_ptr.shape[0] - 1
    b = ctypes.c_size_t()
    _check(lib().cgtp_sparse_attention_layout_bytes(n_rows, col.shape[0], ctypes.byref(b)))
    layout = workspace(b.value, row_ptr.device) if out is None else out
    _check(lib().cgtp_sparse_attention_prepare(_ptr(col), _ptr(row_ptr), n_rows, n_cols, col.shape[0], _ptr(layout),
                                               layout.numel(), _stream(stream, row_ptr)))
    return layout


def cgtp_sparse_attention(q, k, v, row_ptr, n_edges: int, layout, scale=None, out=None, stream=None):
    """Graph sparse attention per head: q [n_rows][H][D], k and v
    [n_cols][H][D] (bf16) over a graph prepared by
    cgtp_sparse_attention_prepare; returns float32 [n_rows][H][D]."""
    n_rows = row_ptr.shape[0] - 1
    H, D = q.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / D ** 0.5
    if out is None:
        out = torch.empty(n_rows, H, D, dtype=torch.float32, device=q.device)
    _check(lib().cgtp_sparse_attention(DTYPES["bf16"], H, D, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                       n_rows, n_edges, _ptr(layout), layout.numel(), _ptr(out), _stream(stream, q)))
    return out


def cgtp_sparse_attention_rows(q, k, v, col, row_ptr, scale=None, out=None, stream=None):
    """The same attention in row form, straight from the CSR (col, row_ptr):
    q [n_rows][H][D], k and v [n_cols][H][D] (bf16); returns float32
    [n_rows][H][D]."""
    n_rows = row_ptr.shape[0] - 1
    H, D = q.shape[1], q.shape[2]
    if scale is None:
        scale = 1.0 / D ** 0.5
    if out is None:
        out = torch.empty(n_rows, H, D, dtype=torch.float32, device=q.device)
    _check(lib().cgtp_sparse_attention_rows(DTYPES["bf16"], H, D, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(col),
                                            _ptr(row_ptr), n_rows, k.shape[0], col.shape[0], _ptr(out),
                                            _stream(stream, q)))
    return out


def cgtp_csr_workspace_bytes(n_edges: int, n_keys: int) -> int:
    b = ctypes.c_size_t()
    _check(lib().cgtp_csr_workspace_bytes(n_edges, n_keys, ctypes.byref(b)))
    return b.value


def _csr_outputs(key, n_keys, val, sorted_key, ws, out):
    E = key.shape[0]
    dev = key.device
    if out is None:
        perm = torch.empty(E, dtype=torch.int32, device=dev)
        row_ptr = torch.empty(n_keys + 1, dtype=torch.int32, device=dev)
        sk = torch.empty(E, dtype=torch.int32, device=dev) if sorted_key else None
        sv = torch.empty(E, dtype=torch.int32, device=dev) if val is not None else None
    else:
        perm, row_ptr, sk, sv = out
    if ws is None:
        ws = workspace(cgtp_csr_workspace_bytes(E, n_keys), dev)
    return E, perm, row_ptr, sk, sv, ws


def cgtp_build_csr(key, n_keys: int, val=None, sorted_key: bool = True, ws=None, out=None, stream=None):
    """Returns (perm, row_ptr, sorted_key or None, sorted_val or None)."""
    E, perm, row_ptr, sk, sv, ws = _csr_outputs(key, n_keys, val, sorted_key, ws, out)
    _check(lib().cgtp_build_csr(_ptr(key), _ptr(val), E, n_keys, _ptr(perm), _ptr(row_ptr), _ptr(sk), _ptr(sv),
                                _ptr(ws), ws.numel(), _stream(stream, key)))
    return perm, row_ptr, sk, sv


def cgtp_build_csr_order(key, n_keys: int, val=None, sorted_key: bool = True, ws=None, out=None, order=None,
                         stream=None):
    """cgtp_build_csr plus the longest-first node order (cgtp_node_order's)
    from the same launches.  Returns (perm, row_ptr, sorted_key or None,
    sorted_val or None, order)."""
    E, perm, row_ptr, sk, sv, ws = _csr_outputs(key, n_keys, val, sorted_key, ws, out)
    if order is None:
        order = torch.empty(n_keys, dtype=torch.int32, device=key.device)
    _check(lib().cgtp_build_csr_order(_ptr(key), _ptr(val), E, n_keys, _ptr(perm), _ptr(row_ptr), _ptr(sk),
                                      _ptr(sv), _ptr(order), _ptr(ws), ws.numel(), _stream(stream, key)))
    return perm, row_ptr, sk, sv, order


def cgtp_validate_csr(row_ptr, n_edges: int, idx=None, n_idx_range: int = 0, stream=None) -> bool:
    ws = workspace(256, row_ptr.device)
    rc = lib().cgtp_validate_csr(_ptr(row_ptr), row_ptr.shape[0] - 1, n_edges, _ptr(idx), n_idx_range,
                                 _ptr(ws), _stream(stream, row_ptr))
    if rc == -5:
        return False
    _check(rc)
    return True


def cgtp_spherical_harmonics(lmax: int, vec, perm=None, dtype: str = "f32", out=None, stream=None):
    n = perm.shape[0] if perm is not None else vec.shape[0]
    if out is None:
        out = torch.empty(n, (lmax + 1) ** 2, dtype=TORCH_DTYPES[dtype], device=vec.device)
    _check(lib().cgtp_spherical_harmonics(lmax, DTYPES[dtype], _ptr(vec), _ptr(perm), n, _ptr(out),
                                          _stream(stream, vec)))
    return out


def cgtp_forces_workspace_bytes(n_edges: int, dtype: str) -> int:
    b = ctypes.c_size_t()
    _check(lib().cgtp_forces_workspace_bytes(n_edges, DTYPES[dtype], ctypes.byref(b)))
    return b.value


def cgtp_sh_forces(lmax: int, vec, perm, g_sh, dst_row_ptr, src_row_ptr, src_perm, dtype: str = "f32",
                   ws=None, out=None, stream=None):
    N, E = dst_row_ptr.shape[0] - 1, g_sh.shape[0]
    if out is None:
        out = torch.empty(N, 3, dtype=TORCH_DTYPES[dtype], device=g_sh.device)
    if ws is None:
        ws = workspace(cgtp_forces_workspace_bytes(E, dtype), g_sh.device)
    _check(lib().cgtp_sh_forces(lmax, DTYPES[dtype], _ptr(vec), _ptr(perm), _ptr(g_sh), _ptr(dst_row_ptr),
                                _ptr(src_row_ptr), _ptr(src_perm), N, E, _ptr(out), _ptr(ws), ws.numel(),
                                _stream(stream, g_sh)))
    return out


def cgtp_force_loss_sh_cotangent(lmax: int, vec, perm, src, dst, F, dtype: str = "f32", out=None,
                                 stream=None):
    E = src.shape[0]
    if out is None:
        out = torch.empty(E, (lmax + 1) ** 2, dtype=TORCH_DTYPES[dtype], device=F.device)
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
