"""Python binding of ``libw4gemm.so`` (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module only checks
Python-side types, allocates outputs with torch (device memory and streams are torch's) and
forwards plain pointers and sizes through the C ABI declared in ``include/w4gemm.h``.  There
is no fallback: if the library is missing or fails to load, importing the compute functions
raises.

torch is imported before the library is loaded so that the HIP runtime torch already mapped
(``libamdhip64.so.7``) is the one the library binds to: one runtime, so torch's device
pointers and streams are valid handles for the library.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4gemm.so")

OP_LINEAR, OP_SWIGLU, OP_ADD = 0, 1, 2
GROUP = 64

_STATUS = {0: "W4_OK", -1: "W4_ERR_INVALID_ARG", -2: "W4_ERR_UNSUPPORTED", -3: "W4_ERR_MISALIGNED",
           -4: "W4_ERR_ALIAS", -5: "W4_ERR_DOMAIN", -6: "W4_ERR_DEVICE", -7: "W4_ERR_LAUNCH",
           -8: "W4_ERR_SCRATCH"}
SCRATCH_BYTES = 32 << 20  # W4_SCRATCH_BYTES: static scratch of the allocation-free call

GROUPS = (32, 64, 128)

EXPORTS = (
    "w4_packed_bytes", "w4_packed_sz_bytes", "w4_repack", "w4_repack_pair", "w4_linear",
    "w4_linear_swiglu", "w4_linear_add", "w4_route_for", "w4_linear_route", "w4_route_count",
    "w4_route_name", "w4_route_domain", "w4_status_str", "w4_layout_version", "w4_linear_grouped",
    "w4_bf16_workspace_bytes", "w4_linear_bf16", "w4_linear_swiglu_bf16", "w4_linear_add_bf16",
    "w4_linear_route_bf16", "w4_linear_bf16_noalloc", "w4_graph_set_create", "w4_graph_set_begin",
    "w4_graph_set_end", "w4_graph_set_launch", "w4_graph_set_has", "w4_graph_set_destroy",
    "w4_a8_workspace_bytes", "w4_quantize_a8", "w4_linear_a8", "w4_linear_swiglu_a8", "w4_linear_add_a8",
)


class _Parent(ctypes.Structure):
    # mirrors w4_parent in include/w4gemm.h
    _fields_ = [("w", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("N", ctypes.c_int), ("bits", ctypes.c_int), ("out", ctypes.c_void_p)]


class W4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({status_str(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libw4gemm.so once (after torch); raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m w4_groupwise_gemm_amd.build`")
    import torch  # noqa: F401  -- map torch's HIP runtime first
    L = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.w4_packed_bytes.argtypes = [i, i, i, i]
    L.w4_packed_bytes.restype = sz
    L.w4_packed_sz_bytes.argtypes = [i, i, i]
    L.w4_packed_sz_bytes.restype = sz
    L.w4_repack.argtypes = [vp, vp, vp, vp, i, i, i, i, vp, vp, vp]
    L.w4_repack.restype = i
    L.w4_repack_pair.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, vp, vp]
    L.w4_repack_pair.restype = i
    L.w4_linear.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp]
    L.w4_linear.restype = i
    L.w4_linear_swiglu.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp]
    L.w4_linear_swiglu.restype = i
    L.w4_linear_add.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp]
    L.w4_linear_add.restype = i
    L.w4_route_for.argtypes = [i, i, i, i, i]
    L.w4_route_for.restype = i
    L.w4_linear_route.argtypes = [i, i, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp]
    L.w4_linear_route.restype = i
    L.w4_route_count.argtypes = []
    L.w4_route_count.restype = i
    L.w4_route_name.argtypes = [i]
    L.w4_route_name.restype = ctypes.c_char_p
    L.w4_route_domain.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
    L.w4_route_domain.restype = i
    L.w4_status_str.argtypes = [i]
    L.w4_status_str.restype = ctypes.c_char_p
    L.w4_layout_version.argtypes = []
    L.w4_linear_grouped.argtypes = [vp, ctypes.POINTER(_Parent), i, i, i, i, vp]
    L.w4_linear_grouped.restype = i
    L.w4_layout_version.restype = i
    L.w4_bf16_workspace_bytes.argtypes = [i, i]
    L.w4_bf16_workspace_bytes.restype = sz
    L.w4_linear_bf16.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
    L.w4_linear_bf16.restype = i
    L.w4_linear_swiglu_bf16.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
    L.w4_linear_swiglu_bf16.restype = i
    L.w4_linear_add_bf16.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
    L.w4_linear_add_bf16.restype = i
    L.w4_linear_route_bf16.argtypes = [i, i, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
    L.w4_linear_route_bf16.restype = i
    L.w4_linear_bf16_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp]
    L.w4_linear_bf16_noalloc.restype = i
    L.w4_graph_set_create.argtypes = []
    L.w4_graph_set_create.restype = vp
    for name in ("w4_graph_set_begin", "w4_graph_set_end", "w4_graph_set_launch"):
        getattr(L, name).argtypes = [vp, i, vp]
        getattr(L, name).restype = i
    L.w4_graph_set_has.argtypes = [vp, i]
    L.w4_graph_set_has.restype = i
    L.w4_graph_set_destroy.argtypes = [vp]
    L.w4_graph_set_destroy.restype = None
    L.w4_a8_workspace_bytes.argtypes = [i, i]
    L.w4_a8_workspace_bytes.restype = sz
    L.w4_quantize_a8.argtypes = [vp, i, i, vp, sz, vp]
    L.w4_quantize_a8.restype = i
    L.w4_linear_a8.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
    L.w4_linear_a8.restype = i
    L.w4_linear_swiglu_a8.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
    L.w4_linear_swiglu_a8.restype = i
    L.w4_linear_add_a8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, sz, vp]
    L.w4_linear_add_a8.restype = i
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().w4_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise W4Error(status, where)


# ------------------------------------------------------------------ host-side repacking

def packed_bytes(N: int, K: int, bits: int, group: int = GROUP) -> int:
    return int(lib().w4_packed_bytes(N, K, bits, group))


def packed_sz_bytes(N: int, K: int, group: int = GROUP) -> int:
    return int(lib().w4_packed_sz_bytes(N, K, group))


def bf16_workspace_bytes(T: int, K: int) -> int:
    return int(lib().w4_bf16_workspace_bytes(T, K))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _host(a, dtype) -> Optional[np.ndarray]:
    """Contiguous host array of ``dtype``; same-size dtypes (fp16 -> uint16) are viewed."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        if a.dtype.itemsize != np.dtype(dtype).itemsize:
            raise TypeError(f"expected {np.dtype(dtype)}-sized elements, got {a.dtype}")
        a = a.view(dtype)
    return a


def repack(lo, hi, scales, zeros, bits: int, group: int = GROUP) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Canonical host arrays -> packed (codes uint8, scales uint16, zeros uint16) host arrays."""
    lo = _host(lo, np.uint8)
    hi = _host(hi, np.uint8)
    s = _host(scales, np.uint16)
    z = _host(zeros, np.uint16)
    N, K = lo.shape[0], lo.shape[1] * 2
    nw, nsz = packed_bytes(N, K, bits, group), packed_sz_bytes(N, K, group)
    if nw == 0 or nsz == 0:
        raise W4Error(-1, "repack")
    w = np.empty(nw, dtype=np.uint8)
    so = np.empty(nsz // 2, dtype=np.uint16)
    zo = np.empty(nsz // 2, dtype=np.uint16)
    _check(lib().w4_repack(_ptr(lo), _ptr(hi), _ptr(s), _ptr(z), N, K, bits, group,
                           _ptr(w), _ptr(so), _ptr(zo)), "w4_repack")
    return w, so, zo


def repack_pair(gate, up, bits: int, group: int = GROUP) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """gate/up = (lo, hi, scales, zeros) canonical host tuples -> interleaved pair layout."""
    g = [_host(gate[0], np.uint8), _host(gate[1], np.uint8), _host(gate[2], np.uint16),
         _host(gate[3], np.uint16)]
    u = [_host(up[0], np.uint8), _host(up[1], np.uint8), _host(up[2], np.uint16),
         _host(up[3], np.uint16)]
    N, K = g[0].shape[0], g[0].shape[1] * 2
    nw, nsz = packed_bytes(2 * N, K, bits, group), packed_sz_bytes(2 * N, K, group)
    if nw == 0 or nsz == 0:
        raise W4Error(-1, "repack_pair")
    w = np.empty(nw, dtype=np.uint8)
    so = np.empty(nsz // 2, dtype=np.uint16)
    zo = np.empty(nsz // 2, dtype=np.uint16)
    _check(lib().w4_repack_pair(*[_ptr(a) for a in g], *[_ptr(a) for a in u], N, K, bits, group,
                                _ptr(w), _ptr(so), _ptr(zo)), "w4_repack_pair")
    return w, so, zo


# ------------------------------------------------------------------ device weights + compute

@dataclasses.dataclass
class PackedWeight:
    """Packed weights resident on a device (torch tensors own the memory)."""
    w: "object"        # torch.uint8 [bytes]
    scales: "object"   # torch.int16 [elements] (fp16 bit patterns)
    zeros: "object"    # torch.int16
    N: int             # output width (of each of gate/up for a pair)
    K: int
    bits: int
    pair: bool = False
    group: int = GROUP  # columns per scale / zero-point group (32, 64 or 128)

    @property
    def nbytes_stream(self) -> int:
        """Bytes one call streams: packed codes + scales + zeros (padding included)."""
        return self.w.numel() + 2 * self.scales.numel() + 2 * self.zeros.numel()


def to_device(packed: Tuple[np.ndarray, np.ndarray, np.ndarray], N: int, K: int, bits: int,
              pair: bool = False, device="cuda", group: int = GROUP) -> PackedWeight:
    import torch
    w, s, z = packed
    return PackedWeight(torch.from_numpy(w).to(device),
                        torch.from_numpy(s.view(np.int16)).to(device),
                        torch.from_numpy(z.view(np.int16)).to(device), N, K, bits, pair, group)


def pack_weight(lo, hi, scales, zeros, bits: int, device="cuda", group: int = GROUP) -> PackedWeight:
    lo = np.asarray(lo)
    return to_device(repack(lo, hi, scales, zeros, bits, group), lo.shape[0], lo.shape[1] * 2, bits,
                     False, device, group)


def pack_pair(gate, up, bits: int, device="cuda", group: int = GROUP) -> PackedWeight:
    lo = np.asarray(gate[0])
    return to_device(repack_pair(gate, up, bits, group), lo.shape[0], lo.shape[1] * 2, bits, True,
                     device, group)


def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check_tensor(t, name: str, shape, dtype, device) -> None:
    """Raise ValueError unless t is a contiguous tensor of `dtype` and `shape` on `device`.

    The library receives bare pointers, so everything it cannot check (the device a pointer
    belongs to, the element type, the extent) is checked here, before any launch."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_x(x, K: int, dtype=None):
    import torch
    dtype = torch.float16 if dtype is None else dtype
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("x must be a CUDA tensor of shape [T, K]")
    if x.dim() != 2:
        raise ValueError(f"x must be a CUDA {dtype} tensor of shape [T, K]")
    _check_tensor(x, "x", (x.shape[0], K), dtype, x.device)


def _check_weight(pw: "PackedWeight", device) -> None:
    """The packed tensors must live on the activations' device and hold what the shape needs."""
    import torch
    rows = 2 * pw.N if pw.pair else pw.N
    nw, nsz = packed_bytes(rows, pw.K, pw.bits, pw.group), packed_sz_bytes(rows, pw.K, pw.group)
    _check_tensor(pw.w, "packed codes", (nw,), torch.uint8, device)
    _check_tensor(pw.scales, "packed scales", (nsz // 2,), torch.int16, device)
    _check_tensor(pw.zeros, "packed zero-points", (nsz // 2,), torch.int16, device)


def _check_residual(residual, T: int, N: int, like) -> None:
    # the residual and the output have the activations' dtype (float16 or bfloat16)
    _check_tensor(residual, "residual", (T, N), like.dtype, like.device)


def _out(out, T: int, N: int, like):
    import torch
    if out is None:
        return torch.empty((T, N), dtype=like.dtype, device=like.device)
    _check_tensor(out, "out", (T, N), like.dtype, like.device)
    return out


def linear(x, pw: PackedWeight, out=None, stream=None):
    """out[T, N] = x . dequant(W)^T (fp16) via ``w4_linear``."""
    if pw.pair:
        raise ValueError("a gate/up pair runs through linear_swiglu")
    _check_x(x, pw.K)
    _check_weight(pw, x.device)
    T = x.shape[0]
    out = _out(out, T, pw.N, x)
    _check(lib().w4_linear(_dptr(x), _dptr(pw.w), _dptr(pw.scales), _dptr(pw.zeros), T, pw.N,
                           pw.K, pw.bits, pw.group, _dptr(out), _stream(stream)), "w4_linear")
    return out


def linear_swiglu(x, pw: PackedWeight, out=None, stream=None):
    """out[T, N] = silu(x . Wg^T) * (x . Wu^T) via ``w4_linear_swiglu`` (pw from pack_pair)."""
    if not pw.pair:
        raise ValueError("linear_swiglu needs a gate/up pair from pack_pair")
    _check_x(x, pw.K)
    _check_weight(pw, x.device)
    T = x.shape[0]
    out = _out(out, T, pw.N, x)
    _check(lib().w4_linear_swiglu(_dptr(x), _dptr(pw.w), _dptr(pw.scales), _dptr(pw.zeros), T,
                                  pw.N, pw.K, pw.bits, pw.group, _dptr(out), _stream(stream)),
           "w4_linear_swiglu")
    return out


def linear_add(x, pw: PackedWeight, residual, out=None, stream=None):
    """out[T, N] = x . dequant(W)^T + residual via ``w4_linear_add`` (out may be residual)."""
    if pw.pair:
        raise ValueError("a gate/up pair runs through linear_swiglu")
    _check_x(x, pw.K)
    _check_weight(pw, x.device)
    T = x.shape[0]
    _check_residual(residual, T, pw.N, x)
    out = _out(out, T, pw.N, x)
    _check(lib().w4_linear_add(_dptr(x), _dptr(pw.w), _dptr(pw.scales), _dptr(pw.zeros),
                               _dptr(residual), T, pw.N, pw.K, pw.bits, pw.group, _dptr(out),
                               _stream(stream)), "w4_linear_add")
    return out


def linear_grouped(x, pws, outs=None, stream=None):
    """[x . dequant(W_p)^T for each packed matrix p] via ``w4_linear_grouped`` (1 to 4 matrices,
    4- or 5-bit, same K, not SwiGLU pairs): one launch for T <= 64 and K <= 5120."""
    pws = list(pws)
    if not 1 <= len(pws) <= 4 or any(pw.pair for pw in pws) or len({(pw.K, pw.group) for pw in pws}) != 1:
        raise ValueError("linear_grouped takes 1 to 4 single matrices with one K and group size")
    K = pws[0].K
    _check_x(x, K)
    for pw in pws:
        _check_weight(pw, x.device)
    T = x.shape[0]
    outs = [None] * len(pws) if outs is None else list(outs)
    if len(outs) != len(pws):
        raise ValueError("one output per matrix")
    outs = [_out(o, T, pw.N, x) for o, pw in zip(outs, pws)]
    arr = (_Parent * len(pws))(*[_Parent(_dptr(pw.w), _dptr(pw.scales), _dptr(pw.zeros), pw.N, pw.bits,
                                         _dptr(o)) for pw, o in zip(pws, outs)])
    _check(lib().w4_linear_grouped(_dptr(x), arr, len(pws), T, K, pws[0].group, _stream(stream)),
           "w4_linear_grouped")
    return outs


def linear_route(route_id: int, op: int, x, pw: PackedWeight, residual=None, out=None,
                 stream=None):
    """Run one specific route (benches and per-route parity tests)."""
    _check_x(x, pw.K)
    _check_weight(pw, x.device)
    if op == OP_SWIGLU and not pw.pair:
        raise ValueError("the SwiGLU op needs a gate/up pair from pack_pair")
    if op != OP_SWIGLU and pw.pair:
        raise ValueError("a gate/up pair runs the SwiGLU op only")
    T = x.shape[0]
    if op == OP_ADD:
        _check_residual(residual, T, pw.N, x)
    else:
        residual = None
    out = _out(out, T, pw.N, x)
    _check(lib().w4_linear_route(route_id, op, _dptr(x), _dptr(pw.w), _dptr(pw.scales),
                                 _dptr(pw.zeros), _dptr(residual), T, pw.N, pw.K, pw.bits, pw.group,
                                 _dptr(out), _stream(stream)), "w4_linear_route")
    return out


# ------------------------------------------------------------------ bf16 activations

def _workspace(workspace, T: int, K: int, like):
    import torch
    nbytes = bf16_workspace_bytes(T, K)
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=like.device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != like.device or \
            not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a contiguous tensor of >= {nbytes} bytes on {like.device}")
    return workspace


def _bf16_call(route_id: int, op: int, x, pw: PackedWeight, residual, out, workspace, stream):
    import torch
    if (op == OP_SWIGLU) != pw.pair:
        raise ValueError("the SwiGLU op takes a gate/up pair from pack_pair; the others a single matrix")
    _check_x(x, pw.K, torch.bfloat16)
    _check_weight(pw, x.device)
    T = x.shape[0]
    if op == OP_ADD:
        _check_residual(residual, T, pw.N, x)
    else:
        residual = None
    out = _out(out, T, pw.N, x)
    ws = _workspace(workspace, T, pw.K, x)
    nbytes = ws.numel() * ws.element_size()
    args = (_dptr(x), _dptr(pw.w), _dptr(pw.scales), _dptr(pw.zeros))
    L = lib()
    if route_id >= 0:
        st = L.w4_linear_route_bf16(route_id, op, *args, _dptr(residual), T, pw.N, pw.K, pw.bits,
                                    pw.group, _dptr(out), _dptr(ws), nbytes, _stream(stream))
    elif op == OP_SWIGLU:
        st = L.w4_linear_swiglu_bf16(*args, T, pw.N, pw.K, pw.bits, pw.group, _dptr(out), _dptr(ws),
                                     nbytes, _stream(stream))
    elif op == OP_ADD:
        st = L.w4_linear_add_bf16(*args, _dptr(residual), T, pw.N, pw.K, pw.bits, pw.group, _dptr(out),
                                  _dptr(ws), nbytes, _stream(stream))
    else:
        st = L.w4_linear_bf16(*args, T, pw.N, pw.K, pw.bits, pw.group, _dptr(out), _dptr(ws), nbytes,
                              _stream(stream))
    _check(st, "w4_linear*_bf16")
    return out


def linear_bf16(x, pw: PackedWeight, out=None, workspace=None, stream=None):
    """out[T, N] = x . dequant(W)^T with bf16 x and out, via ``w4_linear_bf16``.  workspace: a
    device byte tensor of >= bf16_workspace_bytes(T, K) bytes (allocated here if None)."""
    return _bf16_call(-1, OP_LINEAR, x, pw, None, out, workspace, stream)


def linear_bf16_noalloc(x, pw: PackedWeight, out, stream=None):
    """As linear_bf16, through ``w4_linear_bf16_noalloc``: the library's static device scratch
    instead of a workspace (for callers that cannot allocate; `out` must be given).  Calls on
    one device share that scratch, so they must not overlap."""
    import torch
    if pw.pair:
        raise ValueError("a gate/up pair runs through linear_swiglu_bf16")
    _check_x(x, pw.K, torch.bfloat16)
    _check_weight(pw, x.device)
    T = x.shape[0]
    _check_tensor(out, "out", (T, pw.N), torch.bfloat16, x.device)
    _check(lib().w4_linear_bf16_noalloc(_dptr(x), _dptr(pw.w), _dptr(pw.scales), _dptr(pw.zeros), T,
                                        pw.N, pw.K, pw.bits, pw.group, _dptr(out), _stream(stream)),
           "w4_linear_bf16_noalloc")
    return out


def linear_swiglu_bf16(x, pw: PackedWeight, out=None, workspace=None, stream=None):
    return _bf16_call(-1, OP_SWIGLU, x, pw, None, out, workspace, stream)


def linear_add_bf16(x, pw: PackedWeight, residual, out=None, workspace=None, stream=None):
    return _bf16_call(-1, OP_ADD, x, pw, residual, out, workspace, stream)


def linear_route_bf16(route_id: int, op: int, x, pw: PackedWeight, residual=None, out=None,
                      workspace=None, stream=None):
    """Run one specific route with bf16 activations (per-route parity tests)."""
    if route_id < 0:
        raise ValueError("route id must be >= 0")
    return _bf16_call(route_id, op, x, pw, residual, out, workspace, stream)


# ------------------------------------------------------------------ A8 prefill route (lossy)

def a8_workspace_bytes(T: int, K: int) -> int:
    return int(lib().w4_a8_workspace_bytes(T, K))


def _a8_workspace(workspace, T: int, K: int, device):
    import torch
    nbytes = a8_workspace_bytes(T, K)
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or \
            not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must be a contiguous tensor of >= {nbytes} bytes on {device}")
    return workspace


def quantize_a8(x, workspace=None, stream=None):
    """Quantise x (fp16 [T, K]) into the A8 workspace (int8 codes + scales per 64 columns); the
    workspace can then serve several A8 calls with x=None."""
    _check_x(x, x.shape[1] if x.dim() == 2 else -1)
    T, K = x.shape
    ws = _a8_workspace(workspace, T, K, x.device)
    _check(lib().w4_quantize_a8(_dptr(x), T, K, _dptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "w4_quantize_a8")
    return ws


def _a8_call(op: int, x, pw: PackedWeight, residual, out, workspace, stream, T=None):
    """x: fp16 [T, K], or None with a workspace that quantize_a8 filled (then T is given)."""
    import torch
    if (op == OP_SWIGLU) != pw.pair:
        raise ValueError("the SwiGLU op takes a gate/up pair from pack_pair; the others a single matrix")
    if x is not None:
        _check_x(x, pw.K)
        T, dev = x.shape[0], x.device
    else:
        if workspace is None or T is None:
            raise ValueError("without x, give the quantised workspace and T")
        dev = workspace.device
    _check_weight(pw, dev)
    like = torch.empty(0, dtype=torch.float16, device=dev)
    if op == OP_ADD:
        _check_tensor(residual, "residual", (T, pw.N), torch.float16, dev)
    else:
        residual = None
    if out is None:
        out = torch.empty((T, pw.N), dtype=torch.float16, device=dev)
    _check_tensor(out, "out", (T, pw.N), like.dtype, dev)
    ws = _a8_workspace(workspace, T, pw.K, dev)
    nb = ws.numel() * ws.element_size()
    args = (_dptr(x), _dptr(pw.w), _dptr(pw.scales), _dptr(pw.zeros))
    L = lib()
    if op == OP_SWIGLU:
        st = L.w4_linear_swiglu_a8(*args, T, pw.N, pw.K, pw.bits, pw.group, _dptr(out), _dptr(ws), nb,
                                   _stream(stream))
    elif op == OP_ADD:
        st = L.w4_linear_add_a8(*args, _dptr(residual), T, pw.N, pw.K, pw.bits, pw.group, _dptr(out),
                                _dptr(ws), nb, _stream(stream))
    else:
        st = L.w4_linear_a8(*args, T, pw.N, pw.K, pw.bits, pw.group, _dptr(out), _dptr(ws), nb,
                            _stream(stream))
    _check(st, "w4_linear*_a8")
    return out


def linear_a8(x, pw: PackedWeight, out=None, workspace=None, stream=None, T=None):
    """A8 route (lossy, int8 activations per 64 columns): out = x . dequant(W)^T."""
    return _a8_call(OP_LINEAR, x, pw, None, out, workspace, stream, T)


def linear_swiglu_a8(x, pw: PackedWeight, out=None, workspace=None, stream=None, T=None):
    return _a8_call(OP_SWIGLU, x, pw, None, out, workspace, stream, T)


def linear_add_a8(x, pw: PackedWeight, residual, out=None, workspace=None, stream=None, T=None):
    return _a8_call(OP_ADD, x, pw, residual, out, workspace, stream, T)


# ------------------------------------------------------------------ per-verify-width graphs

class VerifyGraphs:
    """One recorded graph per token width, over ``w4_graph_set_*``.

    ``run(T, step)``: the first time a width is seen, ``step(T)`` is called once with the
    stream captured (it enqueues that width's library calls on ``stream``: every call of this
    library is capturable), and the instantiated graph is kept; every call then replays it in
    one launch.  The tensors ``step`` uses must outlive the set and keep their addresses; their
    contents are read at replay time.  The stream must not be the null stream."""

    def __init__(self, stream=None):
        import torch
        self._stream = torch.cuda.Stream() if stream is None else stream
        self._set = lib().w4_graph_set_create()
        if not self._set:
            raise MemoryError("w4_graph_set_create")

    @property
    def stream(self):
        return self._stream

    def recorded(self, T: int) -> bool:
        return bool(lib().w4_graph_set_has(self._set, T))

    def record(self, T: int, step) -> None:
        import torch
        h = self._stream.cuda_stream
        torch.cuda.current_stream().synchronize()
        with torch.cuda.stream(self._stream):
            _check(lib().w4_graph_set_begin(self._set, T, h), "w4_graph_set_begin")
            try:
                step(T)
            finally:
                st = lib().w4_graph_set_end(self._set, T, h)
            _check(st, "w4_graph_set_end")

    def run(self, T: int, step=None) -> None:
        """Replay the width-T graph on the set's stream (recording it first if needed)."""
        if not self.recorded(T):
            if step is None:
                raise KeyError(f"no graph recorded for width {T}")
            self.record(T, step)
        _check(lib().w4_graph_set_launch(self._set, T, self._stream.cuda_stream), "w4_graph_set_launch")

    def close(self) -> None:
        if self._set:
            lib().w4_graph_set_destroy(self._set)
            self._set = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover -- interpreter shutdown
            pass


def route_for(op: int, bits: int, T: int, N: int, K: int) -> int:
    return int(lib().w4_route_for(op, bits, T, N, K))


def route_count() -> int:
    return int(lib().w4_route_count())


def route_name(route_id: int) -> Optional[str]:
    r = lib().w4_route_name(route_id)
    return None if r is None else r.decode()


def route_domain(route_id: int) -> Tuple[int, int]:
    lo, hi = ctypes.c_int(), ctypes.c_int()
    _check(lib().w4_route_domain(route_id, ctypes.byref(lo), ctypes.byref(hi)), "w4_route_domain")
    return lo.value, hi.value


def layout_version() -> int:
    return int(lib().w4_layout_version())
