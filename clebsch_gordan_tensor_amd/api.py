"""Thin Python binding of libe3hip.so (include/e3hip.h), via ctypes.

Argument marshalling only: every step of the convolution runs in the HIP
kernels of the library.  Tensors are torch tensors on the GPU (torch is used
for device memory and streams); the calls are asynchronous on the current
torch stream.  The library must have been built (``__graft_entry__.build()``
or ``python -m clebsch_gordan_tensor_amd.build``); a missing library raises.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

from . import synth

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libe3hip.so")
_lib = None

E3_F32, E3_BF16 = 0, 1
E3_Y_GIVEN = 1
E3_OUT_PER_PATH = 2
E3_CHECK = 4
E3_ERR_GRAPH = -5


class E3Error(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"e3hip status {status}: {msg}")
        self.status = status


class _Irrep(C.Structure):
    _fields_ = [("mul", C.c_int32), ("l", C.c_int32), ("parity", C.c_int32)]


class _Irreps(C.Structure):
    _fields_ = [("n", C.c_int32), ("v", C.POINTER(_Irrep))]


class _Desc(C.Structure):
    _fields_ = [("x", _Irreps), ("y", _Irreps), ("out", _Irreps), ("flags", C.c_int32)]


EXPORTS = ["e3_num_paths", "e3_path_info", "e3_supported", "e3_cg_block",
           "e3_spherical_harmonics", "e3_spherical_harmonics_backward", "e3_tp_forward",
           "e3_tp_backward", "e3_conv_forward", "e3_conv_workspace_size",
           "e3_conv_prepare_transpose", "e3_conv_backward", "e3_edge_grad_to_nodes",
           "e3_linear_num_weights", "e3_linear", "e3_linear_workspace_size",
           "e3_linear_backward", "e3_conv_double_backward_scratch_size",
           "e3_conv_double_backward", "e3_radial_mlp", "e3_conv_forward_radial",
           "e3_radial_mlp_backward_workspace_size", "e3_radial_mlp_backward",
           "e3_generic_plan_size", "e3_generic_plan_build", "e3_tp_forward_generic",
           "e3_tp_forward_gemm", "e3_conv_forward_gemm",
           "e3_tp_backward_generic", "e3_conv_forward_generic", "e3_conv_backward_generic",
           "e3_conv_double_backward_generic", "e3_check_graph", "e3_check_graph_host", "e3_conv_backward_noalloc",
           "e3_tp_backward_gemm", "e3_conv_backward_gemm",
           "e3_radial_hidden_size", "e3_radial_hidden", "e3_conv_forward_radial_hidden",
           "e3_radial_mlp_hidden", "e3_conv_backward_radial_scratch_size",
           "e3_conv_backward_radial_hidden",
           "e3_release_all",
           "e3_last_error"]
E3_GEN_FORWARD, E3_GEN_DX, E3_GEN_DW, E3_GEN_DY, E3_GEN_GEMM = 0, 1, 2, 3, 4
E3_GEN_GEMM_DX, E3_GEN_GEMM_DW, E3_GEN_GEMM_DY = 5, 6, 7


class _CRadial(C.Structure):
    _fields_ = [("cutoff", C.c_float), ("n_basis", C.c_int32), ("hidden", C.c_int32),
                ("W1", C.c_void_p), ("W2", C.c_void_p)]


def lib():
    """Open libe3hip.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = C.CDLL(_LIB_PATH)
    vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    dp = C.POINTER(_Desc)
    L.e3_num_paths.argtypes = [dp, C.POINTER(i32)]
    L.e3_path_info.argtypes = [dp, i32, C.POINTER(i32), C.POINTER(i32), C.POINTER(i32)]
    L.e3_supported.argtypes = [dp, C.c_int]
    L.e3_supported.restype = i32
    L.e3_cg_block.argtypes = [i32, i32, i32, C.POINTER(C.c_double)]
    L.e3_spherical_harmonics.argtypes = [i32, i64, vp, vp, vp]
    L.e3_spherical_harmonics_backward.argtypes = [i32, i64, vp, vp, vp, vp]
    L.e3_tp_forward.argtypes = [dp, i64, vp, vp, vp, vp, C.c_int, vp]
    L.e3_tp_backward.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, vp, C.c_int, vp]
    L.e3_edge_grad_to_nodes.argtypes = [i32, i32, vp, vp, vp, sz, vp, vp, vp]
    ip = C.POINTER(_Irreps)
    L.e3_linear_num_weights.argtypes = [ip, ip, C.POINTER(i32)]
    L.e3_linear.argtypes = [ip, ip, i64, vp, vp, vp, C.c_int, vp]
    L.e3_linear_workspace_size.argtypes = [ip, ip, C.POINTER(sz)]
    L.e3_radial_mlp.argtypes = [C.POINTER(_CRadial), i32, i32, vp, vp, vp]
    L.e3_conv_forward_radial.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, vp,
                                         C.POINTER(_CRadial), vp, vp]
    L.e3_radial_hidden_size.argtypes = [i32, C.POINTER(sz)]
    L.e3_radial_hidden.argtypes = [C.POINTER(_CRadial), i32, vp, vp, sz, vp]
    L.e3_radial_mlp_hidden.argtypes = [C.POINTER(_CRadial), i32, i32, vp, sz, vp, vp]
    L.e3_conv_forward_radial_hidden.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, vp,
                                                C.POINTER(_CRadial), vp, sz, vp, vp]
    L.e3_conv_backward_radial_scratch_size.argtypes = [dp, i32, C.POINTER(sz)]
    L.e3_conv_backward_radial_hidden.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, vp,
                                                 C.POINTER(_CRadial), vp, sz, vp, vp, vp, vp, vp,
                                                 sz, vp]
    L.e3_generic_plan_size.argtypes = [dp, i32, C.POINTER(sz)]
    L.e3_generic_plan_build.argtypes = [dp, i32, vp, sz]
    L.e3_tp_backward_generic.argtypes = [dp, i64, vp, sz, vp, sz, vp, sz, vp, vp, vp, vp, vp, vp,
                                         vp, C.c_int, vp]
    L.e3_tp_forward_generic.argtypes = [dp, i64, vp, sz, vp, vp, vp, vp, C.c_int, vp]
    L.e3_tp_forward_gemm.argtypes = [dp, i64, vp, sz, vp, vp, vp, vp, vp]
    L.e3_conv_forward_gemm.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, vp, vp, vp, vp]
    L.e3_conv_forward_generic.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, sz, vp, vp, vp, vp,
                                          C.c_int, vp]
    L.e3_conv_backward_generic.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, sz, vp, sz, vp, sz,
                                           vp, vp, vp, vp, vp, vp, vp, C.c_int, vp]
    L.e3_conv_double_backward_generic.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, sz, vp, sz,
                                                  vp, sz, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  vp, vp, vp, vp, sz, C.c_int, vp]
    L.e3_radial_mlp_backward_workspace_size.argtypes = [C.POINTER(_CRadial), i32, i32,
                                                        C.POINTER(sz)]
    L.e3_radial_mlp_backward.argtypes = [C.POINTER(_CRadial), i32, i32, vp, vp, vp, vp, vp, vp,
                                         sz, vp]
    L.e3_conv_double_backward_scratch_size.argtypes = [dp, i32, i32, C.c_int, C.POINTER(sz)]
    L.e3_conv_double_backward.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp,
                                          vp, vp, vp, vp, vp, vp, sz, C.c_int, vp]
    L.e3_linear_backward.argtypes = [ip, ip, i64, vp, vp, vp, vp, vp, vp, sz, C.c_int, vp]
    L.e3_conv_forward.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, vp, vp, vp, C.c_int, vp]
    L.e3_conv_workspace_size.argtypes = [i32, i32, C.POINTER(sz)]
    L.e3_conv_prepare_transpose.argtypes = [i32, i32, vp, vp, vp, vp, sz, vp]
    L.e3_conv_backward.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp,
                                   C.c_int, vp]
    L.e3_check_graph.argtypes = [i32, i32, vp, vp, vp]
    L.e3_tp_backward_gemm.argtypes = [dp, i64, vp, sz, vp, sz, vp, sz, vp, vp, vp, vp, vp, vp, vp,
                                      vp]
    L.e3_conv_backward_gemm.argtypes = [dp, i32, i32, vp, vp, vp, sz, vp, sz, vp, sz, vp, sz, vp,
                                        vp, vp, vp, vp, vp, vp, vp]
    L.e3_conv_backward_noalloc.argtypes = [dp, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           C.c_int, vp]
    L.e3_check_graph_host.argtypes = [i32, i32, vp, vp]
    L.e3_release_all.argtypes = []
    L.e3_last_error.restype = C.c_char_p
    for name in EXPORTS:
        if name not in ("e3_last_error", "e3_supported", "e3_release_all"):
            getattr(L, name).restype = C.c_int
    L.e3_release_all.restype = None
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise E3Error(status, lib().e3_last_error().decode())


@dataclass
class Desc:
    """Irreps of x, y (multiplicity 1) and the output, as lists of (l, parity),
    with C channels on x and the output."""
    x: list
    y: list
    out: list
    channels: int
    flags: int = 0

    @classmethod
    def from_strings(cls, x: str, y: str, out: str, flags: int = 0):
        C_, xi = synth.parse_irreps(x)
        _, yi = synth.parse_irreps(y)
        C2, oi = synth.parse_irreps(out)
        if C2 != C_:
            raise ValueError("x and out need the same multiplicity")
        return cls(xi, yi, oi, C_, flags)

    def with_flags(self, flags):
        return Desc(self.x, self.y, self.out, self.channels, flags)

    @property
    def dx(self):
        return synth.dim(self.x)

    @property
    def dy(self):
        return synth.dim(self.y)

    @property
    def dout(self):
        if self.flags & E3_OUT_PER_PATH:  # one output block per path, as the library lists them
            return sum(2 * self.out[path_info(self, i)[2]][0] + 1
                       for i in range(num_paths(self)))
        return synth.dim(self.out)

    def c(self):
        """ctypes struct (kept alive together with its arrays)."""
        def arr(ir, mul):
            a = (_Irrep * max(1, len(ir)))()
            for i, (l, p) in enumerate(ir):
                a[i] = _Irrep(mul, l, p)
            return a
        ax, ay, ao = arr(self.x, self.channels), arr(self.y, 1), arr(self.out, self.channels)
        d = _Desc(_Irreps(len(self.x), ax), _Irreps(len(self.y), ay),
                  _Irreps(len(self.out), ao), self.flags)
        d._keep = (ax, ay, ao)
        return d


def _dtype_code(t):
    import torch
    if t.dtype == torch.float32:
        return E3_F32
    if t.dtype == torch.bfloat16:
        return E3_BF16
    raise TypeError(f"unsupported storage dtype {t.dtype}")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _need(t, name, shape=None, dtype=None):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def check_graph(rowptr, sender, stream=None):
    """Host-side check of a CSR graph on the GPU (e3_check_graph): raises
    E3Error (status E3_ERR_GRAPH) naming the first violation.  Synchronises
    the stream."""
    import torch
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    _check(lib().e3_check_graph(rowptr.shape[0] - 1, sender.shape[0], _ptr(rowptr), _ptr(sender),
                                _stream(stream)))


def check_graph_host(rowptr, sender):
    """e3_check_graph on host (numpy int32) arrays: raises E3Error
    (status E3_ERR_GRAPH) naming the first violation."""
    import numpy as np
    rp = np.ascontiguousarray(rowptr, dtype=np.int32)
    sn = np.ascontiguousarray(sender, dtype=np.int32)
    _check(lib().e3_check_graph_host(rp.shape[0] - 1, sn.shape[0], rp.ctypes.data_as(C.c_void_p),
                                     sn.ctypes.data_as(C.c_void_p)))


def release_all():
    """Frees the library's host-side plan cache (e3_release_all)."""
    lib().e3_release_all()


def num_paths(desc: Desc) -> int:
    n = C.c_int32()
    _check(lib().e3_num_paths(C.byref(desc.c()), C.byref(n)))
    return n.value


def path_info(desc: Desc, i: int):
    a, b, c = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib().e3_path_info(C.byref(desc.c()), i, C.byref(a), C.byref(b), C.byref(c)))
    return a.value, b.value, c.value


def supported(desc: Desc, dtype_code: int = E3_F32) -> bool:
    return bool(lib().e3_supported(C.byref(desc.c()), dtype_code))


def cg_block(l1: int, l2: int, L: int):
    import numpy as np
    out = np.zeros((2 * L + 1) * (2 * l1 + 1) * (2 * l2 + 1))
    _check(lib().e3_cg_block(l1, l2, L, out.ctypes.data_as(C.POINTER(C.c_double))))
    return out.reshape(2 * L + 1, 2 * l1 + 1, 2 * l2 + 1)


def spherical_harmonics(lmax: int, vec, out=None, stream=None):
    import torch
    _need(vec, "vec", dtype=torch.float32)
    n = vec.shape[0]
    if out is None:
        out = torch.empty((n, (lmax + 1) ** 2), device=vec.device, dtype=torch.float32)
    _need(out, "out", shape=(n, (lmax + 1) ** 2), dtype=torch.float32)
    _check(lib().e3_spherical_harmonics(lmax, n, _ptr(vec), _ptr(out), _stream(stream)))
    return out


def spherical_harmonics_backward(lmax: int, vec, dY, out=None, stream=None):
    """dvec [n][3] = J^T dY, J the Jacobian of the harmonics of vec [n][3]."""
    import torch
    _need(vec, "vec", dtype=torch.float32)
    n = vec.shape[0]
    _need(vec, "vec", shape=(n, 3))
    _need(dY, "dY", shape=(n, (lmax + 1) ** 2), dtype=torch.float32)
    if out is None:
        out = torch.empty((n, 3), device=vec.device, dtype=torch.float32)
    _need(out, "out", shape=(n, 3), dtype=torch.float32)
    _check(lib().e3_spherical_harmonics_backward(lmax, n, _ptr(vec), _ptr(dY), _ptr(out),
                                                 _stream(stream)))
    return out


def tp_backward(desc: Desc, x, y, w, dz, dx=None, dw=None, dy=None, stream=None):
    """(dx, dw, dy) of z = tp_forward(x, y, w) for the cotangent dz."""
    import torch
    B = x.shape[0]
    P = num_paths(desc)
    _need(x, "x", shape=(B, desc.dx, desc.channels))
    _need(y, "y", shape=(B, desc.dy), dtype=torch.float32)
    _need(w, "w", shape=(B, P, desc.channels), dtype=x.dtype)
    _need(dz, "dz", shape=(B, desc.dout, desc.channels), dtype=x.dtype)
    dev, dt = x.device, x.dtype
    if dx is None:
        dx = torch.empty((B, desc.dx, desc.channels), device=dev, dtype=dt)
    if dw is None:
        dw = torch.empty((B, P, desc.channels), device=dev, dtype=dt)
    if dy is None:
        dy = torch.empty((B, desc.dy), device=dev, dtype=torch.float32)
    _need(dx, "dx", shape=(B, desc.dx, desc.channels), dtype=dt)
    _need(dw, "dw", shape=(B, P, desc.channels), dtype=dt)
    _need(dy, "dy", shape=(B, desc.dy), dtype=torch.float32)
    _check(lib().e3_tp_backward(C.byref(desc.c()), B, _ptr(x), _ptr(y), _ptr(w), _ptr(dz),
                                _ptr(dx), _ptr(dw), _ptr(dy), _dtype_code(x), _stream(stream)))
    return dx, dw, dy


def tp_forward(desc: Desc, x, y, w, out=None, stream=None):
    import torch
    B = x.shape[0]
    P = num_paths(desc)
    _need(x, "x", shape=(B, desc.dx, desc.channels))
    _need(y, "y", shape=(B, desc.dy), dtype=torch.float32)
    _need(w, "w", shape=(B, P, desc.channels), dtype=x.dtype)
    if out is None:
        out = torch.empty((B, desc.dout, desc.channels), device=x.device, dtype=x.dtype)
    _need(out, "out", shape=(B, desc.dout, desc.channels), dtype=x.dtype)
    _check(lib().e3_tp_forward(C.byref(desc.c()), B, _ptr(x), _ptr(y), _ptr(w), _ptr(out),
                               _dtype_code(x), _stream(stream)))
    return out


def conv_forward(desc: Desc, rowptr, sender, edge_vec_or_Y, x, w, out=None, workspace=None,
                 stream=None):
    """m = conv(x, Y(edge_vec), w).  workspace (optional) is the prepared
    per-graph index; with it receivers are visited in its locality order."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    ycols = desc.dy if desc.flags & E3_Y_GIVEN else 3
    _need(edge_vec_or_Y, "edge_vec_or_Y", shape=(E, ycols), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels))
    _need(w, "w", shape=(E, P, desc.channels), dtype=x.dtype)
    if out is None:
        out = torch.empty((N, desc.dout, desc.channels), device=x.device, dtype=x.dtype)
    _need(out, "out", shape=(N, desc.dout, desc.channels), dtype=x.dtype)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().e3_conv_forward(C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender),
                                 _ptr(workspace), wsb, _ptr(edge_vec_or_Y), _ptr(x), _ptr(w),
                                 _ptr(out), _dtype_code(x), _stream(stream)))
    return out


def workspace_size(n_nodes: int, n_edges: int) -> int:
    b = C.c_size_t()
    _check(lib().e3_conv_workspace_size(n_nodes, n_edges, C.byref(b)))
    return b.value


def conv_prepare_transpose(rowptr, sender, workspace=None, edge_vec=None, stream=None):
    """Build the per-graph index (sender-ordered edge list and node locality
    order); returns the workspace (uint8 tensor).  edge_vec (optional, [E][3]
    float32) lets the order follow rebuilt positions."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    nb = workspace_size(N, E)
    if workspace is None:
        workspace = torch.empty(nb, device=rowptr.device, dtype=torch.uint8)
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    if edge_vec is not None:
        _need(edge_vec, "edge_vec", shape=(E, 3), dtype=torch.float32)
    _check(lib().e3_conv_prepare_transpose(N, E, _ptr(rowptr), _ptr(sender), _ptr(edge_vec),
                                           _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(stream)))
    return workspace


def conv_backward(desc: Desc, rowptr, sender, workspace, edge_vec_or_Y, x, w, dm,
                  dx=None, dw=None, dY=None, stream=None):
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    ycols = desc.dy if desc.flags & E3_Y_GIVEN else 3
    _need(edge_vec_or_Y, "edge_vec_or_Y", shape=(E, ycols), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels))
    _need(w, "w", shape=(E, P, desc.channels), dtype=x.dtype)
    _need(dm, "dm", shape=(N, desc.dout, desc.channels), dtype=x.dtype)
    dev, dt = x.device, x.dtype
    if dx is None:
        dx = torch.empty((N, desc.dx, desc.channels), device=dev, dtype=dt)
    if dw is None:
        dw = torch.empty((E, P, desc.channels), device=dev, dtype=dt)
    if dY is None:
        dY = torch.empty((E, desc.dy), device=dev, dtype=torch.float32)
    _need(dx, "dx", shape=(N, desc.dx, desc.channels), dtype=dt)
    _need(dw, "dw", shape=(E, P, desc.channels), dtype=dt)
    _need(dY, "dY", shape=(E, desc.dy), dtype=torch.float32)
    _check(lib().e3_conv_backward(C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _ptr(edge_vec_or_Y), _ptr(x), _ptr(w), _ptr(dm), _ptr(dx),
                                  _ptr(dw), _ptr(dY), _dtype_code(x), _stream(stream)))
    return dx, dw, dY


def conv_backward_noalloc(desc: Desc, rowptr, sender, edge_vec_or_Y, x, w, dm, dx=None, dw=None,
                          dY=None, stream=None):
    """The backward with its per-graph index built inside the call in the
    library's fixed device scratch (e3_conv_backward_noalloc); the library
    allocates nothing (this wrapper allocates the outputs it is not given)."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    ycols = desc.dy if desc.flags & E3_Y_GIVEN else 3
    _need(edge_vec_or_Y, "edge_vec_or_Y", shape=(E, ycols), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels))
    _need(w, "w", shape=(E, P, desc.channels), dtype=x.dtype)
    _need(dm, "dm", shape=(N, desc.dout, desc.channels), dtype=x.dtype)
    dev, dt = x.device, x.dtype
    if dx is None:
        dx = torch.empty((N, desc.dx, desc.channels), device=dev, dtype=dt)
    if dw is None:
        dw = torch.empty((E, P, desc.channels), device=dev, dtype=dt)
    if dY is None:
        dY = torch.empty((E, desc.dy), device=dev, dtype=torch.float32)
    _need(dx, "dx", shape=(N, desc.dx, desc.channels), dtype=dt)
    _need(dw, "dw", shape=(E, P, desc.channels), dtype=dt)
    _need(dY, "dY", shape=(E, desc.dy), dtype=torch.float32)
    _check(lib().e3_conv_backward_noalloc(C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender),
                                          _ptr(edge_vec_or_Y), _ptr(x), _ptr(w), _ptr(dm),
                                          _ptr(dx), _ptr(dw), _ptr(dY), _dtype_code(x),
                                          _stream(stream)))
    return dx, dw, dY


def edge_grad_to_nodes(rowptr, sender, workspace, edge_grad, out=None, stream=None):
    """node_grad [N][3]: sum of edge_grad over each node's in-edges minus the
    sum over its out-edges (r_e = pos[recv] - pos[sender]); forces are its
    negative.  workspace: from conv_prepare_transpose on the same graph."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    _need(edge_grad, "edge_grad", shape=(E, 3), dtype=torch.float32)
    if out is None:
        out = torch.empty((N, 3), device=rowptr.device, dtype=torch.float32)
    _need(out, "out", shape=(N, 3), dtype=torch.float32)
    _check(lib().e3_edge_grad_to_nodes(N, E, _ptr(rowptr), _ptr(sender), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _ptr(edge_grad), _ptr(out), _stream(stream)))
    return out


def _irreps_struct(irreps, mul):
    a = (_Irrep * max(1, len(irreps)))()
    for i, (l, p) in enumerate(irreps):
        a[i] = _Irrep(mul, l, p)
    st = _Irreps(len(irreps), a)
    st._keep = a
    return st


def linear_num_weights(in_irreps, out_irreps) -> int:
    """Number of [Cin][Cout] weight matrices of the per-irrep channel mixing."""
    n = C.c_int32()
    a, b = _irreps_struct(in_irreps, 8), _irreps_struct(out_irreps, 32)
    _check(lib().e3_linear_num_weights(C.byref(a), C.byref(b), C.byref(n)))
    return n.value


def linear(in_irreps, out_irreps, x, W, out=None, stream=None):
    """y [rows][dout][Cout] = per-irrep channel mixing of x [rows][din][Cin]
    with W [n_pairs][Cin][Cout] (float32); in/out irreps as lists of (l, parity)."""
    import torch
    rows, din, cin = x.shape
    n_pairs, cin_w, cout = W.shape
    if cin_w != cin:
        raise ValueError("W and x disagree on Cin")
    if din != synth.dim(in_irreps):
        raise ValueError("x does not match the input irreps")
    _need(x, "x")
    _need(W, "W", dtype=torch.float32)
    dout = synth.dim(out_irreps)
    if out is None:
        out = torch.empty((rows, dout, cout), device=x.device, dtype=x.dtype)
    _need(out, "out", shape=(rows, dout, cout), dtype=x.dtype)
    a, b = _irreps_struct(in_irreps, cin), _irreps_struct(out_irreps, cout)
    if n_pairs != linear_num_weights(in_irreps, out_irreps):
        raise ValueError("W has the wrong number of matrices")
    _check(lib().e3_linear(C.byref(a), C.byref(b), rows, _ptr(x), _ptr(W), _ptr(out),
                           _dtype_code(x), _stream(stream)))
    return out


def linear_backward(in_irreps, out_irreps, x, W, dy, dx=None, dW=None, workspace=None,
                    stream=None):
    """(dx, dW) of linear() for the cotangent dy."""
    import torch
    rows, din, cin = x.shape
    n_pairs, _, cout = W.shape
    _need(x, "x")
    _need(W, "W", dtype=torch.float32)
    _need(dy, "dy", shape=(rows, synth.dim(out_irreps), cout), dtype=x.dtype)
    a, b = _irreps_struct(in_irreps, cin), _irreps_struct(out_irreps, cout)
    nb = C.c_size_t()
    _check(lib().e3_linear_workspace_size(C.byref(a), C.byref(b), C.byref(nb)))
    if workspace is None:
        workspace = torch.empty(nb.value, device=x.device, dtype=torch.uint8)
    if dx is None:
        dx = torch.empty_like(x)
    if dW is None:
        dW = torch.empty_like(W)
    _need(dx, "dx", shape=tuple(x.shape), dtype=x.dtype)
    _need(dW, "dW", shape=tuple(W.shape), dtype=torch.float32)
    _check(lib().e3_linear_backward(C.byref(a), C.byref(b), rows, _ptr(x), _ptr(W), _ptr(dy),
                                    _ptr(dx), _ptr(dW), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _dtype_code(x), _stream(stream)))
    return dx, dW


def conv_double_backward(desc: Desc, rowptr, sender, workspace, Y, x, w, dm, ddx, ddY, ddw,
                         scratch=None, stream=None):
    """(dx2, dY2, dw2, ddm): the double backward of the convolution for the
    variations (ddx, ddY, ddw) of the backward's outputs; desc needs
    E3_Y_GIVEN and Y the given harmonics."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    dt = x.dtype
    _need(Y, "Y", shape=(E, desc.dy), dtype=torch.float32)
    _need(ddY, "ddY", shape=(E, desc.dy), dtype=torch.float32)
    for t, n, shp in ((x, "x", (N, desc.dx, desc.channels)), (ddx, "ddx", (N, desc.dx, desc.channels)),
                      (w, "w", (E, P, desc.channels)), (ddw, "ddw", (E, P, desc.channels)),
                      (dm, "dm", (N, desc.dout, desc.channels))):
        _need(t, n, shape=shp, dtype=dt)
    nb = C.c_size_t()
    _check(lib().e3_conv_double_backward_scratch_size(C.byref(desc.c()), N, E, _dtype_code(x),
                                                      C.byref(nb)))
    if scratch is None:
        scratch = torch.empty(nb.value, device=x.device, dtype=torch.uint8)
    dx2, dw2 = torch.empty_like(x), torch.empty_like(w)
    dY2 = torch.empty_like(Y)
    ddm = torch.empty_like(dm)
    _check(lib().e3_conv_double_backward(
        C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(Y), _ptr(x), _ptr(w), _ptr(dm),
        _ptr(ddx), _ptr(ddY), _ptr(ddw), _ptr(dx2), _ptr(dY2), _ptr(dw2), _ptr(ddm),
        _ptr(scratch), scratch.numel() * scratch.element_size(), _dtype_code(x), _stream(stream)))
    return dx2, dY2, dw2, ddm


def _radial(cutoff, W1, W2):
    import torch
    _need(W1, "W1", dtype=torch.float32)
    _need(W2, "W2", dtype=torch.float32)
    if W1.dim() != 2 or W2.dim() != 2 or W1.shape[1] != W2.shape[0]:
        raise ValueError("W1 [n_basis][hidden] and W2 [hidden][n_cols] expected")
    return _CRadial(float(cutoff), W1.shape[0], W1.shape[1], W1.data_ptr(), W2.data_ptr())


def radial_mlp(edge_vec, cutoff, W1, W2, out=None, stream=None):
    """w[E][n_cols] = silu(B(|r|) W1) W2 with the 8-function Bessel basis."""
    import torch
    E = edge_vec.shape[0]
    _need(edge_vec, "edge_vec", shape=(E, 3), dtype=torch.float32)
    r = _radial(cutoff, W1, W2)
    n_cols = W2.shape[1]
    if out is None:
        out = torch.empty((E, n_cols), device=edge_vec.device, dtype=torch.float32)
    _need(out, "out", shape=(E, n_cols), dtype=torch.float32)
    _check(lib().e3_radial_mlp(C.byref(r), E, n_cols, _ptr(edge_vec), _ptr(out), _stream(stream)))
    return out


def conv_forward_radial(desc: Desc, rowptr, sender, edge_vec, x, cutoff, W1, W2, out=None,
                        workspace=None, stream=None):
    """m = conv(x, Y(edge_vec), w) with w = radial_mlp(edge_vec) computed inside
    the kernel (never stored); W2 is [64][P*C]."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    _need(edge_vec, "edge_vec", shape=(E, 3), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels), dtype=torch.float32)
    r = _radial(cutoff, W1, W2)
    if W2.shape[1] != num_paths(desc) * desc.channels:
        raise ValueError("W2 must have P*C columns")
    if out is None:
        out = torch.empty((N, desc.dout, desc.channels), device=x.device, dtype=torch.float32)
    _need(out, "out", shape=(N, desc.dout, desc.channels), dtype=torch.float32)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().e3_conv_forward_radial(C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender),
                                        _ptr(workspace), wsb, _ptr(edge_vec), _ptr(x), C.byref(r),
                                        _ptr(out), _stream(stream)))
    return out


def radial_hidden(edge_vec, cutoff, W1, W2, out=None, stream=None):
    """The radial MLP's hidden layer of every edge in the packed operand form
    conv_forward_radial_hidden reads (uint8 [E * 256])."""
    import torch
    E = edge_vec.shape[0]
    _need(edge_vec, "edge_vec", shape=(E, 3), dtype=torch.float32)
    r = _radial(cutoff, W1, W2)
    n = C.c_size_t()
    _check(lib().e3_radial_hidden_size(E, C.byref(n)))
    if out is None:
        out = torch.empty(n.value, device=edge_vec.device, dtype=torch.uint8)
    nb = out.numel() * out.element_size()
    _check(lib().e3_radial_hidden(C.byref(r), E, _ptr(edge_vec), _ptr(out), nb, _stream(stream)))
    return out


def radial_mlp_hidden(hidden, n_edges, cutoff, W1, W2, out=None, stream=None):
    """radial_mlp with the hidden layer from radial_hidden."""
    import torch
    r = _radial(cutoff, W1, W2)
    n_cols = W2.shape[1]
    if out is None:
        out = torch.empty((n_edges, n_cols), device=hidden.device, dtype=torch.float32)
    _need(out, "out", shape=(n_edges, n_cols), dtype=torch.float32)
    hb = hidden.numel() * hidden.element_size()
    _check(lib().e3_radial_mlp_hidden(C.byref(r), n_edges, n_cols, _ptr(hidden), hb, _ptr(out),
                                      _stream(stream)))
    return out


def conv_forward_radial_hidden(desc: Desc, rowptr, sender, edge_vec, x, cutoff, W1, W2, hidden,
                               out=None, workspace=None, stream=None):
    """conv_forward_radial with the hidden layer from radial_hidden."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    _need(edge_vec, "edge_vec", shape=(E, 3), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels), dtype=torch.float32)
    r = _radial(cutoff, W1, W2)
    if W2.shape[1] != num_paths(desc) * desc.channels:
        raise ValueError("W2 must have P*C columns")
    if out is None:
        out = torch.empty((N, desc.dout, desc.channels), device=x.device, dtype=torch.float32)
    _need(out, "out", shape=(N, desc.dout, desc.channels), dtype=torch.float32)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    hb = hidden.numel() * hidden.element_size()
    _check(lib().e3_conv_forward_radial_hidden(C.byref(desc.c()), N, E, _ptr(rowptr),
                                               _ptr(sender), _ptr(workspace), wsb, _ptr(edge_vec),
                                               _ptr(x), C.byref(r), _ptr(hidden), hb, _ptr(out),
                                               _stream(stream)))
    return out


def conv_backward_radial_scratch_bytes(desc: Desc, n_edges):
    """Device scratch bytes conv_backward_radial_hidden needs."""
    nb = C.c_size_t()
    _check(lib().e3_conv_backward_radial_scratch_size(C.byref(desc.c()), n_edges, C.byref(nb)))
    return max(nb.value, 16)


def conv_backward_radial_hidden(desc: Desc, rowptr, sender, workspace, edge_vec, x, cutoff, W1,
                                W2, hidden, dm, dx=None, dw=None, dY=None, scratch=None,
                                stream=None):
    """(dx, dw, dY) of the fused radial forward: conv_backward with w formed
    from the hidden layer (radial_hidden of the same edge vectors)."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    _need(edge_vec, "edge_vec", shape=(E, 3), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels), dtype=torch.float32)
    _need(dm, "dm", shape=(N, desc.dout, desc.channels), dtype=torch.float32)
    r = _radial(cutoff, W1, W2)
    if W2.shape[1] != P * desc.channels:
        raise ValueError("W2 must have P*C columns")
    dev = x.device
    if dx is None:
        dx = torch.empty((N, desc.dx, desc.channels), device=dev, dtype=torch.float32)
    if dw is None:
        dw = torch.empty((E, P, desc.channels), device=dev, dtype=torch.float32)
    if dY is None:
        dY = torch.empty((E, desc.dy), device=dev, dtype=torch.float32)
    _need(dx, "dx", shape=(N, desc.dx, desc.channels), dtype=torch.float32)
    _need(dw, "dw", shape=(E, P, desc.channels), dtype=torch.float32)
    _need(dY, "dY", shape=(E, desc.dy), dtype=torch.float32)
    if scratch is None:
        scratch = torch.empty(conv_backward_radial_scratch_bytes(desc, E), device=dev,
                              dtype=torch.uint8)
    _check(lib().e3_conv_backward_radial_hidden(
        C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(edge_vec), _ptr(x), C.byref(r),
        _ptr(hidden), hidden.numel() * hidden.element_size(), _ptr(dm), _ptr(dx), _ptr(dw),
        _ptr(dY), _ptr(scratch), scratch.numel() * scratch.element_size(), _stream(stream)))
    return dx, dw, dY


def radial_mlp_backward_workspace_bytes(W1, W2, n_edges, n_cols):
    """Device workspace bytes radial_mlp_backward needs for n_edges x n_cols."""
    r = _radial(5.0, W1, W2)
    nb = C.c_size_t()
    _check(lib().e3_radial_mlp_backward_workspace_size(C.byref(r), n_edges, n_cols, C.byref(nb)))
    return nb.value


def radial_mlp_backward(edge_vec, cutoff, W1, W2, dw, workspace=None, stream=None):
    """(dW1, dW2, dvec) for the cotangent dw [E][n_cols] of radial_mlp; dvec is
    the edge-vector gradient through |r| only."""
    import torch
    E, n_cols = dw.shape
    _need(edge_vec, "edge_vec", shape=(E, 3), dtype=torch.float32)
    _need(dw, "dw", shape=(E, n_cols), dtype=torch.float32)
    r = _radial(cutoff, W1, W2)
    nb = C.c_size_t()
    _check(lib().e3_radial_mlp_backward_workspace_size(C.byref(r), E, n_cols, C.byref(nb)))
    if workspace is None:
        workspace = torch.empty(nb.value, device=dw.device, dtype=torch.uint8)
    dW1, dW2 = torch.empty_like(W1), torch.empty_like(W2)
    dvec = torch.empty_like(edge_vec)
    _check(lib().e3_radial_mlp_backward(
        C.byref(r), E, n_cols, _ptr(edge_vec), _ptr(dw), _ptr(dW1), _ptr(dW2), _ptr(dvec),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return dW1, dW2, dvec


_GENERIC_PLANS = {}


def generic_plan(desc: Desc, device, table=0):
    """Coefficient table `table` (E3_GEN_FORWARD, E3_GEN_DX, E3_GEN_DW,
    E3_GEN_DY) of the generic tensor product for desc: built on the host by the library, copied
    to device memory once per descriptor."""
    import numpy as np
    import torch
    key = (repr(desc.x), repr(desc.y), repr(desc.out), desc.channels, desc.flags, str(device),
           table)
    if key not in _GENERIC_PLANS:
        nb = C.c_size_t()
        _check(lib().e3_generic_plan_size(C.byref(desc.c()), table, C.byref(nb)))
        host = np.zeros(nb.value // 4, dtype=np.int32)
        _check(lib().e3_generic_plan_build(C.byref(desc.c()), table, host.ctypes.data, nb.value))
        _GENERIC_PLANS[key] = torch.from_numpy(host).to(device)
    return _GENERIC_PLANS[key]


def tp_forward_generic(desc: Desc, x, y, w, out=None, stream=None):
    """z = tensor product of x and y weighted by w (as tp_forward) through the
    coefficient-table kernel: any signature with degrees up to 7 (at most 63
    components per operand)."""
    import torch
    B = x.shape[0]
    P = num_paths(desc)
    _need(x, "x", shape=(B, desc.dx, desc.channels))
    _need(y, "y", shape=(B, desc.dy), dtype=torch.float32)
    _need(w, "w", shape=(B, P, desc.channels), dtype=x.dtype)
    if out is None:
        out = torch.empty((B, desc.dout, desc.channels), device=x.device, dtype=x.dtype)
    _need(out, "out", shape=(B, desc.dout, desc.channels), dtype=x.dtype)
    plan = generic_plan(desc, x.device)
    _check(lib().e3_tp_forward_generic(C.byref(desc.c()), B, _ptr(plan), plan.numel() * 4, _ptr(x),
                                       _ptr(y), _ptr(w), _ptr(out), _dtype_code(x),
                                       _stream(stream)))
    return out


def tp_forward_gemm(desc: Desc, x, y, w, out=None, stream=None):
    """z = tensor product of x and y weighted by w (as tp_forward_generic) as
    one dense product per output block on the fp32 matrix cores (float32,
    C % 16 == 0, degrees up to 7)."""
    import torch
    B = x.shape[0]
    P = num_paths(desc)
    _need(x, "x", shape=(B, desc.dx, desc.channels), dtype=torch.float32)
    _need(y, "y", shape=(B, desc.dy), dtype=torch.float32)
    _need(w, "w", shape=(B, P, desc.channels), dtype=torch.float32)
    if out is None:
        out = torch.empty((B, desc.dout, desc.channels), device=x.device, dtype=torch.float32)
    _need(out, "out", shape=(B, desc.dout, desc.channels), dtype=torch.float32)
    plan = generic_plan(desc, x.device, E3_GEN_GEMM)
    _check(lib().e3_tp_forward_gemm(C.byref(desc.c()), B, _ptr(plan), plan.numel() * 4, _ptr(x),
                                    _ptr(y), _ptr(w), _ptr(out), _stream(stream)))
    return out


def conv_forward_gemm(desc: Desc, rowptr, sender, edge_vec_or_Y, x, w, out=None, stream=None):
    """m = the convolution (as conv_forward_generic) as dense products per
    receiver and output block on the fp32 matrix cores; edge_vec_or_Y is the
    edge vectors [E][3] or, with E3_Y_GIVEN, the harmonics [E][dy]."""
    import torch
    N, E = rowptr.numel() - 1, sender.numel()
    P = num_paths(desc)
    Y = edge_vec_or_Y
    _need(x, "x", shape=(N, desc.dx, desc.channels), dtype=torch.float32)
    _need(Y, "edge_vec_or_Y", shape=(E, desc.dy if desc.flags & E3_Y_GIVEN else 3),
          dtype=torch.float32)
    _need(w, "w", shape=(E, P, desc.channels), dtype=torch.float32)
    if out is None:
        out = torch.empty((N, desc.dout, desc.channels), device=x.device, dtype=torch.float32)
    _need(out, "out", shape=(N, desc.dout, desc.channels), dtype=torch.float32)
    plan = generic_plan(desc, x.device, E3_GEN_GEMM)
    _check(lib().e3_conv_forward_gemm(C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender),
                                      _ptr(plan), plan.numel() * 4, _ptr(Y), _ptr(x), _ptr(w),
                                      _ptr(out), _stream(stream)))
    return out


def tp_backward_gemm(desc: Desc, x, y, w, dz, dx=None, dw=None, dy=None, stream=None):
    """(dx, dw, dy) of tp_forward_gemm for the cotangent dz, as dense products
    on the fp32 matrix cores (tables E3_GEN_GEMM_DX, _DW, _DY)."""
    import torch
    B = x.shape[0]
    P = num_paths(desc)
    f32 = torch.float32
    _need(x, "x", shape=(B, desc.dx, desc.channels), dtype=f32)
    _need(y, "y", shape=(B, desc.dy), dtype=f32)
    _need(w, "w", shape=(B, P, desc.channels), dtype=f32)
    _need(dz, "dz", shape=(B, desc.dout, desc.channels), dtype=f32)
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w) if dw is None else dw
    dy = torch.empty_like(y) if dy is None else dy
    for t, n, ref in ((dx, "dx", x), (dw, "dw", w), (dy, "dy", y)):
        _need(t, n, shape=tuple(ref.shape), dtype=f32)
    px, pw, py = (generic_plan(desc, x.device, t)
                  for t in (E3_GEN_GEMM_DX, E3_GEN_GEMM_DW, E3_GEN_GEMM_DY))
    _check(lib().e3_tp_backward_gemm(C.byref(desc.c()), B, _ptr(px), px.numel() * 4, _ptr(pw),
                                     pw.numel() * 4, _ptr(py), py.numel() * 4, _ptr(x), _ptr(y),
                                     _ptr(w), _ptr(dz), _ptr(dx), _ptr(dw), _ptr(dy),
                                     _stream(stream)))
    return dx, dw, dy


def conv_backward_gemm(desc: Desc, rowptr, sender, workspace, Y, x, w, dm, dx=None, dw=None,
                       dY=None, stream=None):
    """(dx, dw, dY) of conv_forward_gemm with given harmonics (desc needs
    E3_Y_GIVEN), as dense products on the fp32 matrix cores; workspace from
    conv_prepare_transpose on the same graph."""
    import torch
    N, E = rowptr.numel() - 1, sender.numel()
    P = num_paths(desc)
    f32 = torch.float32
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    _need(Y, "Y", shape=(E, desc.dy), dtype=f32)
    _need(x, "x", shape=(N, desc.dx, desc.channels), dtype=f32)
    _need(w, "w", shape=(E, P, desc.channels), dtype=f32)
    _need(dm, "dm", shape=(N, desc.dout, desc.channels), dtype=f32)
    dx = torch.empty_like(x) if dx is None else dx
    dw = torch.empty_like(w) if dw is None else dw
    dY = torch.empty_like(Y) if dY is None else dY
    px, pw, py = (generic_plan(desc, x.device, t)
                  for t in (E3_GEN_GEMM_DX, E3_GEN_GEMM_DW, E3_GEN_GEMM_DY))
    _check(lib().e3_conv_backward_gemm(C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender),
                                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _ptr(px), px.numel() * 4, _ptr(pw), pw.numel() * 4,
                                       _ptr(py), py.numel() * 4, _ptr(Y), _ptr(x), _ptr(w),
                                       _ptr(dm), _ptr(dx), _ptr(dw), _ptr(dY), _stream(stream)))
    return dx, dw, dY


def tp_backward_generic(desc: Desc, x, y, w, dz, stream=None):
    """(dx, dw, dy) of tp_forward_generic for the cotangent dz."""
    import torch
    B = x.shape[0]
    P = num_paths(desc)
    _need(x, "x", shape=(B, desc.dx, desc.channels))
    _need(y, "y", shape=(B, desc.dy), dtype=torch.float32)
    _need(w, "w", shape=(B, P, desc.channels), dtype=x.dtype)
    _need(dz, "dz", shape=(B, desc.dout, desc.channels), dtype=x.dtype)
    px, pw, py = (generic_plan(desc, x.device, t) for t in (E3_GEN_DX, E3_GEN_DW, E3_GEN_DY))
    dx, dw = torch.empty_like(x), torch.empty_like(w)
    dy = torch.empty((B, desc.dy), device=x.device, dtype=torch.float32)
    _check(lib().e3_tp_backward_generic(
        C.byref(desc.c()), B, _ptr(px), px.numel() * 4, _ptr(pw), pw.numel() * 4, _ptr(py),
        py.numel() * 4, _ptr(x), _ptr(y), _ptr(w), _ptr(dz), _ptr(dx), _ptr(dw), _ptr(dy),
        _dtype_code(x), _stream(stream)))
    return dx, dw, dy


def conv_forward_generic(desc: Desc, rowptr, sender, edge_vec_or_Y, x, w, out=None,
                         workspace=None, stream=None):
    """m = conv(x, Y(edge_vec), w) (as conv_forward) through the
    coefficient-table kernels: any signature with degrees up to 7 (at most 63
    components per operand; harmonics from edge vectors to degree 6)."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    ycols = desc.dy if desc.flags & E3_Y_GIVEN else 3
    _need(edge_vec_or_Y, "edge_vec_or_Y", shape=(E, ycols), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels))
    _need(w, "w", shape=(E, P, desc.channels), dtype=x.dtype)
    if out is None:
        out = torch.empty((N, desc.dout, desc.channels), device=x.device, dtype=x.dtype)
    _need(out, "out", shape=(N, desc.dout, desc.channels), dtype=x.dtype)
    plan = generic_plan(desc, x.device, E3_GEN_FORWARD)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().e3_conv_forward_generic(
        C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender), _ptr(workspace), wsb, _ptr(plan),
        plan.numel() * 4, _ptr(edge_vec_or_Y), _ptr(x), _ptr(w), _ptr(out), _dtype_code(x),
        _stream(stream)))
    return out


def conv_backward_generic(desc: Desc, rowptr, sender, workspace, edge_vec_or_Y, x, w, dm,
                          dx=None, dw=None, dY=None, stream=None):
    """(dx, dw, dY) of conv_forward_generic for the cotangent dm; workspace
    from conv_prepare_transpose on the same graph."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    _need(rowptr, "rowptr", dtype=torch.int32)
    _need(sender, "sender", dtype=torch.int32)
    ycols = desc.dy if desc.flags & E3_Y_GIVEN else 3
    _need(edge_vec_or_Y, "edge_vec_or_Y", shape=(E, ycols), dtype=torch.float32)
    _need(x, "x", shape=(N, desc.dx, desc.channels))
    _need(w, "w", shape=(E, P, desc.channels), dtype=x.dtype)
    _need(dm, "dm", shape=(N, desc.dout, desc.channels), dtype=x.dtype)
    dev, dt = x.device, x.dtype
    if dx is None:
        dx = torch.empty((N, desc.dx, desc.channels), device=dev, dtype=dt)
    if dw is None:
        dw = torch.empty((E, P, desc.channels), device=dev, dtype=dt)
    if dY is None:
        dY = torch.empty((E, desc.dy), device=dev, dtype=torch.float32)
    _need(dx, "dx", shape=(N, desc.dx, desc.channels), dtype=dt)
    _need(dw, "dw", shape=(E, P, desc.channels), dtype=dt)
    _need(dY, "dY", shape=(E, desc.dy), dtype=torch.float32)
    px, pw, py = (generic_plan(desc, x.device, t) for t in (E3_GEN_DX, E3_GEN_DW, E3_GEN_DY))
    _check(lib().e3_conv_backward_generic(
        C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(px), px.numel() * 4, _ptr(pw),
        pw.numel() * 4, _ptr(py), py.numel() * 4, _ptr(edge_vec_or_Y), _ptr(x), _ptr(w), _ptr(dm),
        _ptr(dx), _ptr(dw), _ptr(dY), _dtype_code(x), _stream(stream)))
    return dx, dw, dY


def conv_double_backward_generic(desc: Desc, rowptr, sender, workspace, Y, x, w, dm, ddx, ddY,
                                 ddw, scratch=None, stream=None):
    """(dx2, dY2, dw2, ddm) as conv_double_backward through the coefficient
    tables (degrees up to 7); desc needs E3_Y_GIVEN."""
    import torch
    N, E = rowptr.shape[0] - 1, sender.shape[0]
    P = num_paths(desc)
    dt = x.dtype
    _need(Y, "Y", shape=(E, desc.dy), dtype=torch.float32)
    _need(ddY, "ddY", shape=(E, desc.dy), dtype=torch.float32)
    for t, n, shp in ((x, "x", (N, desc.dx, desc.channels)), (ddx, "ddx", (N, desc.dx, desc.channels)),
                      (w, "w", (E, P, desc.channels)), (ddw, "ddw", (E, P, desc.channels)),
                      (dm, "dm", (N, desc.dout, desc.channels))):
        _need(t, n, shape=shp, dtype=dt)
    nb = C.c_size_t()
    _check(lib().e3_conv_double_backward_scratch_size(C.byref(desc.c()), N, E, _dtype_code(x),
                                                      C.byref(nb)))
    if scratch is None:
        scratch = torch.empty(nb.value, device=x.device, dtype=torch.uint8)
    pf, px, pw, py = (generic_plan(desc, x.device, t)
                      for t in (E3_GEN_FORWARD, E3_GEN_DX, E3_GEN_DW, E3_GEN_DY))
    dx2, dw2 = torch.empty_like(x), torch.empty_like(w)
    dY2 = torch.empty_like(Y)
    ddm = torch.empty_like(dm)
    _check(lib().e3_conv_double_backward_generic(
        C.byref(desc.c()), N, E, _ptr(rowptr), _ptr(sender), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(pf), pf.numel() * 4, _ptr(px),
        px.numel() * 4, _ptr(pw), pw.numel() * 4, _ptr(py), py.numel() * 4, _ptr(Y), _ptr(x),
        _ptr(w), _ptr(dm), _ptr(ddx), _ptr(ddY), _ptr(ddw), _ptr(dx2), _ptr(dY2), _ptr(dw2),
        _ptr(ddm), _ptr(scratch), scratch.numel() * scratch.element_size(), _dtype_code(x),
        _stream(stream)))
    return dx2, dY2, dw2, ddm
