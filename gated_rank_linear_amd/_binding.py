"""ctypes binding for libgsi (include/gsi.h): argument marshalling only.

Each `gsi_*` function here has the name of the C entry point it calls and takes torch tensors
(device memory) in place of raw pointers; every computation happens in the HIP library. PyTorch
provides device memory and the current stream, nothing else. If the library has not been built,
importing this module raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
import sys

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GSI_LIB") or os.path.join(_HERE, "_lib", "libgsi.so")

GSI_F32, GSI_F16, GSI_BF16 = 0, 1, 2
GSI_SITE_GATED, GSI_SITE_STATIC, GSI_SITE_DENSE = 0, 1, 2
GSI_OK = 0
STATUS_NAMES = {0: "GSI_OK", -1: "GSI_ERR_NULL", -2: "GSI_ERR_SHAPE", -3: "GSI_ERR_DTYPE", -4: "GSI_ERR_EPS",
                -5: "GSI_ERR_WORKSPACE", -6: "GSI_ERR_ALIGN", -7: "GSI_ERR_DEVICE", -8: "GSI_ERR_HIP",
                -9: "GSI_ERR_TIMEOUT"}

_DTYPES = {torch.float32: GSI_F32, torch.float16: GSI_F16, torch.bfloat16: GSI_BF16}

_vp, _sz, _int, _float = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float

# (name, restype, argtypes) exactly as declared in include/gsi.h
SIGNATURES = [
    ("gsi_status_string", ctypes.c_char_p, [_int]),
    ("gsi_device_check", _int, []),
    ("gsi_layer_aux_bytes", _sz, [_int, _int, _int, _int]),
    ("gsi_layer_create_workspace_bytes", _sz, [_int, _int, _int, _int]),
    ("gsi_layer_create", _int, [ctypes.POINTER(_vp), _int, _int, _int, _int, _vp, _vp, _vp, _vp, _sz, _vp, _sz,
                                _vp]),
    ("gsi_layer_create_dense", _int, [ctypes.POINTER(_vp), _int, _int, _int, _vp, _vp, _sz, _vp]),
    ("gsi_layer_destroy", _int, [_vp]),
    ("gsi_workspace_bytes", _sz, [_int, _int, _int, _int, _int]),
    ("gsi_forward", _int, [_vp, _vp, _int, _float, _vp, _vp, _vp, _vp, _sz, _vp]),
    ("gsi_stack_create", _int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), _int]),
    ("gsi_stack_create_modes", _int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_int), _int]),
    ("gsi_stack_destroy", _int, [_vp]),
    ("gsi_stack_workspace_bytes", _sz, [_vp, _int]),
    ("gsi_stack_decode", _int, [_vp, _vp, _int, _int, _float, _vp, _vp, _vp, _vp, _sz, _vp]),
    ("gsi_workspace_status", _int, [_vp, _sz, ctypes.POINTER(_int), _vp]),
    ("gsi_stack_decode_noalloc", _int, [_vp, _vp, _int, _int, _float, _vp, _vp, _vp, _vp]),
    ("gsi_calibrate_workspace_bytes", _sz, [_int, _int, _int]),
    ("gsi_calibrate", _int, [_int, _int, _int, _vp, _vp, _int, _vp, _vp, _sz, _vp]),
    ("gsi_block_step_workspace_bytes", _sz, [_vp, _vp, _int]),
    ("gsi_block_step", _int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _float, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _sz, _vp]),
    ("gsi_decode_step", _int, [_int, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                               ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _int, _int, _float, _vp,
                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    ("gsi_decode_step_devpos", _int, [_int, ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                      ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, _int, _int,
                                      _float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
]


class GsiError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = lib.gsi_status_string(code).decode() if lib is not None else ""
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({msg})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libgsi is not built ({LIB_PATH} missing); run `python -m gated_rank_linear_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    for name, res, args in SIGNATURES:
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _check(rc: int, where: str):
    if rc != GSI_OK:
        raise GsiError(rc, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("libgsi takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libgsi takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    return _DTYPES[dt]


class Layer:
    """Host handle of a created layer; keeps the borrowed tensors alive."""

    def __init__(self, handle: int, dtype: int, d_out: int, d: int, k: int, keep: tuple):
        self.handle = handle
        self.dtype, self.d_out, self.d, self.k = dtype, d_out, d, k
        self._keep = keep

    def destroy(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and lib is not None:
            lib.gsi_layer_destroy(h)

    def __del__(self):
        self.destroy()   # host memory only: safe at any time


class Stack:
    """Host handle of a stack. destroy() frees its device table; call it before the process
    ends. At interpreter shutdown the table is left to the process exit (the HIP runtime may
    already be gone then)."""

    def __init__(self, handle: int, layers: list):
        self.handle = handle
        self.layers = layers

    def destroy(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and lib is not None:
            _check(lib.gsi_stack_destroy(h), "gsi_stack_destroy")

    def __del__(self):
        if sys.is_finalizing():
            self.handle = None
            return
        try:
            self.destroy()
        except GsiError:
            pass


def gsi_device_check() -> int:
    return lib.gsi_device_check()


def gsi_layer_aux_bytes(dtype: int, d_out: int, d: int, k: int) -> int:
    return lib.gsi_layer_aux_bytes(dtype, d_out, d, k)


def gsi_workspace_bytes(dtype: int, d_out: int, d: int, k: int, T_max: int) -> int:
    return lib.gsi_workspace_bytes(dtype, d_out, d, k, T_max)


def gsi_layer_create_workspace_bytes(dtype: int, d_out: int, d: int, k: int) -> int:
    return lib.gsi_layer_create_workspace_bytes(dtype, d_out, d, k)


def gsi_layer_create(W: torch.Tensor, V: torch.Tensor, M: torch.Tensor, aux: torch.Tensor,
                     ws: torch.Tensor | None = None, stream=None) -> Layer:
    d_out, d = W.shape
    k = V.shape[1]
    dt = dtype_code(W.dtype)
    h = _vp()
    rc = lib.gsi_layer_create(ctypes.byref(h), dt, d_out, d, k, _ptr(W), _ptr(V), _ptr(M), _ptr(aux),
                              aux.numel() * aux.element_size(), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gsi_layer_create")
    return Layer(h.value, dt, d_out, d, k, (W, M, aux))


def gsi_forward(layer: Layer, x: torch.Tensor, eps: float, y: torch.Tensor, gate: torch.Tensor,
                rho: torch.Tensor | None, ws: torch.Tensor, stream=None) -> None:
    T = x.shape[0] if x.dim() == 2 else 1
    rc = lib.gsi_forward(layer.handle, _ptr(x), T, float(eps), _ptr(y), _ptr(gate), _ptr(rho), _ptr(ws),
                         ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gsi_forward")


def gsi_layer_create_dense(W: torch.Tensor, aux: torch.Tensor, stream=None) -> Layer:
    d_out, d = W.shape
    dt = dtype_code(W.dtype)
    h = _vp()
    rc = lib.gsi_layer_create_dense(ctypes.byref(h), dt, d_out, d, _ptr(W), _ptr(aux),
                                    aux.numel() * aux.element_size(), _stream(stream))
    _check(rc, "gsi_layer_create_dense")
    return Layer(h.value, dt, d_out, d, 0, (W, None, aux))


def gsi_stack_create(layers: list) -> Stack:
    arr = (_vp * len(layers))(*[L.handle for L in layers])
    h = _vp()
    _check(lib.gsi_stack_create(ctypes.byref(h), arr, len(layers)), "gsi_stack_create")
    return Stack(h.value, list(layers))


def gsi_stack_create_modes(layers: list, modes) -> Stack:
    """A stack whose site i runs in modes[i] (GSI_SITE_GATED / GSI_SITE_STATIC / GSI_SITE_DENSE)."""
    arr = (_vp * len(layers))(*[L.handle for L in layers])
    md = (_int * len(layers))(*[int(m) for m in modes])
    h = _vp()
    _check(lib.gsi_stack_create_modes(ctypes.byref(h), arr, md, len(layers)), "gsi_stack_create_modes")
    return Stack(h.value, list(layers))


def gsi_stack_workspace_bytes(stack: Stack, T_step: int) -> int:
    return lib.gsi_stack_workspace_bytes(stack.handle, T_step)


def gsi_stack_decode(stack: Stack, X: torch.Tensor, n_steps: int, T_step: int, eps: float, Y: torch.Tensor,
                     gates: torch.Tensor, rho: torch.Tensor | None, ws: torch.Tensor, stream=None) -> None:
    rc = lib.gsi_stack_decode(stack.handle, _ptr(X), n_steps, T_step, float(eps), _ptr(Y), _ptr(gates), _ptr(rho),
                              _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gsi_stack_decode")


def gsi_workspace_status(ws: torch.Tensor, stream=None) -> int:
    out = _int(0)
    rc = lib.gsi_workspace_status(_ptr(ws), ws.numel() * ws.element_size(), ctypes.byref(out), _stream(stream))
    _check(rc, "gsi_workspace_status")
    return out.value


def gsi_calibrate_workspace_bytes(n: int, d: int, k: int) -> int:
    return lib.gsi_calibrate_workspace_bytes(n, d, k)


def gsi_calibrate(A: torch.Tensor, Q0t: torch.Tensor, n_iter: int, Qt: torch.Tensor, ws: torch.Tensor,
                  stream=None) -> None:
    """Subspace iteration with DGKS Gram-Schmidt on the GPU: A [n, d] float32, Q0t and Qt [k, d]."""
    n, d = A.shape
    k = Q0t.shape[0]
    rc = lib.gsi_calibrate(n, d, k, _ptr(A), _ptr(Q0t), int(n_iter), _ptr(Qt), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gsi_calibrate")


def gsi_block_step_workspace_bytes(A: Stack, B: Stack, n_heads: int) -> int:
    return lib.gsi_block_step_workspace_bytes(A.handle, B.handle, int(n_heads))


def gsi_block_step(A: Stack, B: Stack, gamma: torch.Tensor, beta: torch.Tensor, x: torch.Tensor,
                   k_cache: torch.Tensor, v_cache: torch.Tensor, pos: int, n_heads: int, eps: float,
                   xa: torch.Tensor, ya: torch.Tensor, xb: torch.Tensor, yb: torch.Tensor, gates: torch.Tensor,
                   rho: torch.Tensor | None, ws: torch.Tensor, stream=None) -> None:
    """One decode-step block: LayerNorm, stack A [QKV, fc_in], attention over the caches (row pos
    written), GELU, stack B [out, fc_out], x += y_out + y_mlp (x updated in place)."""
    rc = lib.gsi_block_step(A.handle, B.handle, _ptr(gamma), _ptr(beta), _ptr(x), _ptr(k_cache), _ptr(v_cache),
                            int(pos), int(n_heads), float(eps), _ptr(xa), _ptr(ya), _ptr(xb), _ptr(yb), _ptr(gates),
                            _ptr(rho), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gsi_block_step")


def gsi_decode_step(A: list, B: list, gamma: list, beta: list, k_cache: list, v_cache: list, pos: int,
                    n_heads: int, eps: float, x: torch.Tensor, xa: torch.Tensor, ya: torch.Tensor, xb: torch.Tensor,
                    yb: torch.Tensor, gates: torch.Tensor, rho: torch.Tensor | None, ws: torch.Tensor,
                    stream=None) -> None:
    """A whole decode step: gsi_block_step for every block in order on the token row x (per-block
    lists of stacks, LayerNorm parameters and caches; gates [n_blocks * 4])."""
    n = len(A)
    if not (len(B) == len(gamma) == len(beta) == len(k_cache) == len(v_cache) == n):
        raise ValueError("per-block lists differ in length")
    arr = lambda vals: (_vp * n)(*vals)
    rc = lib.gsi_decode_step(n, arr([s.handle for s in A]), arr([s.handle for s in B]), arr([_ptr(t) for t in gamma]),
                             arr([_ptr(t) for t in beta]), arr([_ptr(t) for t in k_cache]),
                             arr([_ptr(t) for t in v_cache]), int(pos), int(n_heads), float(eps), _ptr(x), _ptr(xa),
                             _ptr(ya), _ptr(xb), _ptr(yb), _ptr(gates), _ptr(rho), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gsi_decode_step")


def gsi_decode_step_devpos(A: list, B: list, gamma: list, beta: list, k_cache: list, v_cache: list,
                           pos: torch.Tensor, n_heads: int, eps: float, x: torch.Tensor, xa: torch.Tensor,
                           ya: torch.Tensor, xb: torch.Tensor, yb: torch.Tensor, gates: torch.Tensor,
                           rho: torch.Tensor | None, ws: torch.Tensor, stream=None) -> None:
    """gsi_decode_step at the position held by the device int32 tensor `pos` (advanced by one by the
    step itself), so that a captured graph of one call replays token after token."""
    n = len(A)
    if not (len(B) == len(gamma) == len(beta) == len(k_cache) == len(v_cache) == n):
        raise ValueError("per-block lists differ in length")
    if pos.dtype != torch.int32 or pos.numel() != 1:
        raise ValueError("pos must be one int32 element")
    arr = lambda vals: (_vp * n)(*vals)
    rc = lib.gsi_decode_step_devpos(n, arr([s.handle for s in A]), arr([s.handle for s in B]),
                                    arr([_ptr(t) for t in gamma]), arr([_ptr(t) for t in beta]),
                                    arr([_ptr(t) for t in k_cache]), arr([_ptr(t) for t in v_cache]), _ptr(pos),
                                    int(k_cache[0].shape[0]), int(n_heads), float(eps), _ptr(x), _ptr(xa), _ptr(ya),
                                    _ptr(xb), _ptr(yb), _ptr(gates), _ptr(rho), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "gsi_decode_step_devpos")


# ------------------------------------------------------------------------------------------------
# Allocation conveniences (device memory through torch; all compute stays in libgsi)
# ------------------------------------------------------------------------------------------------
def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Zero-filled workspace (libgsi requires zeros before first use)."""
    return torch.zeros((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


def create_layer(W: torch.Tensor, V: torch.Tensor, stream=None, ws: torch.Tensor | None = None,
                 split: bool = True) -> Layer:
    """Allocate M and aux on W's device and run gsi_layer_create. The create workspace is `ws`
    when given, else (split=True) a temporary one from torch's caching allocator, released when
    the call returns (the allocator keeps the block for later work on the same stream), or none
    (split=False: the single-pass kernels)."""
    d_out, d = W.shape
    k = V.shape[1]
    dt = dtype_code(W.dtype)
    nb = gsi_layer_aux_bytes(dt, d_out, d, k)
    if nb == 0:
        _check(-2, "gsi_layer_aux_bytes")
    M = torch.empty((d_out, k), dtype=W.dtype, device=W.device)
    aux = torch.empty(nb, dtype=torch.uint8, device=W.device)
    if ws is None and split:
        wb = gsi_layer_create_workspace_bytes(dt, d_out, d, k)
        ws = torch.empty(wb, dtype=torch.uint8, device=W.device) if wb else None
    return gsi_layer_create(W, V, M, aux, ws, stream)


def create_dense_layer(W: torch.Tensor, stream=None) -> Layer:
    """Allocate aux on W's device and run gsi_layer_create_dense (y = W x for every token)."""
    d_out, d = W.shape
    nb = gsi_layer_aux_bytes(dtype_code(W.dtype), d_out, d, 0)
    if nb == 0:
        _check(-2, "gsi_layer_aux_bytes")
    aux = torch.empty(nb, dtype=torch.uint8, device=W.device)
    return gsi_layer_create_dense(W, aux, stream)


def layer_image(layer: Layer) -> torch.Tensor:
    """The cached image M of a layer made by create_layer."""
    return layer._keep[1]
