"""The C ABI loads, exports every symbol include/gsi.h declares, and rejects invalid arguments
before touching the device (these calls run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

g = pytest.importorskip("gated_rank_linear_amd")
lib = g.lib
vp = ctypes.c_void_p


def _declared():
    src = open(os.path.join(ROOT, "include", "gsi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gsi_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 12
    bound = {n for n, _, _ in g.SIGNATURES}
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
        assert n in bound, f"{n} has no binding"



def test_library_carries_no_phase_stamps():
    # the wall-clock stamps of the batch-1 kernel exist only in the separate stamp build
    if os.path.basename(g.LIB_PATH) != "libgsi.so":
        pytest.skip("a non-default library is loaded")
    with pytest.raises(AttributeError):
        lib.gsi_phase_stamps


def test_decode_step_devpos_rejects_before_device():
    """The device-position step checks its pointer and cache length before anything is enqueued."""
    p = vp(256)
    arr = (vp * 1)(None)
    f = ctypes.c_float(0.1)
    args = lambda pos, rows: (1, arr, arr, arr, arr, arr, arr, pos, rows, 16, f, p, p, p, p, p, p, None, p, 1 << 20, None)
    assert lib.gsi_decode_step_devpos(*args(None, 8)) == -1            # no position
    assert lib.gsi_decode_step_devpos(*args(vp(256), 0)) == -2         # empty cache
    assert lib.gsi_decode_step_devpos(*args(vp(256), (1 << 24) + 1)) == -2
    assert lib.gsi_decode_step_devpos(*args(vp(258), 8)) == -2         # misaligned int
    assert lib.gsi_decode_step_devpos(*args(vp(256), 8)) == -1         # null stacks

def test_status_strings():
    for code in range(0, -10, -1):
        s = lib.gsi_status_string(code)
        assert s and len(s) > 1
    assert lib.gsi_status_string(12345) == b"unknown status"


@pytest.mark.parametrize("dtype,d_out,d,k,ok", [
    (2, 12288, 4096, 256, True), (2, 4096, 16384, 256, True), (0, 768, 768, 64, True), (1, 2304, 768, 256, True),
    (2, 4096, 4096, 512, True), (3, 16, 16, 8, False), (2, 0, 16, 8, False), (2, 16, 12, 8, False),
    (2, 16, 16, 24, False), (2, 16, 16, 32, False), (2, 16, 4096, 1024, False), (2, 16, 16, 4, False),
    (2, 262144, 16, 8, True), (2, 262145, 16, 8, False), (0, 262144, 512, 512, True), (0, 262145, 512, 512, False),
])
def test_aux_and_workspace_sizes(dtype, d_out, d, k, ok):
    a = lib.gsi_layer_aux_bytes(dtype, d_out, d, k)
    w = lib.gsi_workspace_bytes(dtype, d_out, d, k, 64)
    if ok:
        es = 4 if dtype == 0 else 2
        assert a >= k * d * es + k * k * 4
        assert w >= 64 * k * 4
    else:
        assert a == 0 and w == 0


def test_layer_create_validation_before_device():
    h = vp()
    p = vp(256)  # never dereferenced: validation fails first
    assert lib.gsi_layer_create(None, 2, 16, 16, 8, p, p, p, p, 1 << 20, None, 0, None) == -1
    assert lib.gsi_layer_create(ctypes.byref(h), 2, 16, 16, 8, None, p, p, p, 1 << 20, None, 0, None) == -1
    assert h.value is None
    assert lib.gsi_layer_create(ctypes.byref(h), 7, 16, 16, 8, p, p, p, p, 1 << 20, None, 0, None) == -3
    assert lib.gsi_layer_create(ctypes.byref(h), 2, 16, 16, 24, p, p, p, p, 1 << 20, None, 0, None) == -2
    assert lib.gsi_layer_create(ctypes.byref(h), 2, 16, 16, 8, vp(257), p, p, p, 1 << 20, None, 0, None) == -6
    assert lib.gsi_layer_create(ctypes.byref(h), 2, 16, 16, 8, p, p, p, p, 16, None, 0, None) == -5
    assert lib.gsi_layer_create(ctypes.byref(h), 2, 16, 16, 8, p, p, p, p, 1 << 20, vp(264), 1 << 20, None) == -6
    # a create workspace smaller than asked for
    need = lib.gsi_layer_create_workspace_bytes(2, 4096, 4096, 256)
    assert lib.gsi_layer_create(ctypes.byref(h), 2, 4096, 4096, 256, p, p, p, p, 1 << 30, p, need - 256, None) == -5
    assert lib.gsi_layer_create_dense(ctypes.byref(h), 2, 16, 12, p, p, 1 << 20, None) == -2
    assert lib.gsi_layer_create_dense(ctypes.byref(h), 2, 16, 16, None, p, 1 << 20, None) == -1
    assert lib.gsi_layer_create_dense(ctypes.byref(h), 2, 16, 16, p, p, 16, None) == -5


@pytest.mark.parametrize("dtype,d_out,d,k,splits_m", [
    (2, 4096, 4096, 256, 8), (2, 4096, 16384, 256, 8), (2, 12288, 4096, 256, 2), (2, 16384, 4096, 256, 2),
    (1, 2304, 768, 256, 0), (0, 768, 768, 64, 0), (2, 4096, 4096, 512, 4), (2, 1000, 2048, 256, 4),
])
def test_create_workspace_sizes(dtype, d_out, d, k, splits_m):
    """The create workspace holds the K-split partial sums of M = W V (float32, splits x d_out x
    k) when the shape takes the split path, and of V^T V - I otherwise (0 for float32)."""
    w = lib.gsi_layer_create_workspace_bytes(dtype, d_out, d, k)
    if splits_m:
        assert w >= splits_m * d_out * k * 4
    if dtype == 0:
        assert w == 0
    assert lib.gsi_layer_create_workspace_bytes(dtype, d_out, d, 24) == 0


def test_forward_and_stack_validation_before_device():
    p = vp(256)
    assert lib.gsi_forward(None, p, 1, ctypes.c_float(0.1), p, p, None, p, 1 << 20, None) == -1
    assert lib.gsi_stack_create(None, None, 0) == -1
    h = vp()
    assert lib.gsi_stack_create(ctypes.byref(h), None, 1) == -1
    arr = (vp * 1)(None)
    assert lib.gsi_stack_create(ctypes.byref(h), arr, 1) == -1
    assert lib.gsi_stack_create(ctypes.byref(h), arr, 0) == -2
    assert lib.gsi_stack_create_modes(ctypes.byref(h), arr, None, 0) == -2
    assert lib.gsi_stack_create_modes(ctypes.byref(h), None, None, 1) == -1
    assert lib.gsi_stack_decode(None, p, 1, 1, ctypes.c_float(0.1), p, p, None, p, 1 << 20, None) == -1
    assert lib.gsi_stack_workspace_bytes(None, 1) == 0
    assert lib.gsi_workspace_status(None, 0, None, None) == -1
    assert lib.gsi_layer_destroy(None) == 0 and lib.gsi_stack_destroy(None) == 0


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        g._binding._ptr(torch.zeros(4))


@pytest.mark.parametrize("n,d,k,ok", [
    (2048, 4096, 256, True), (512, 16384, 512, True), (64, 64, 8, True), (2048, 4096, 4, False),
    (2048, 4096, 1024, False), (2048, 32768, 256, False), (2048, 4100, 256, False), (100, 4096, 256, False),
    (2044, 4096, 256, False), ((1 << 20) + 8, 64, 8, False),
])
def test_calibrate_workspace_sizes(n, d, k, ok):
    w = lib.gsi_calibrate_workspace_bytes(n, d, k)
    if ok:
        assert w >= 4 * (d * n + k * n + k * d)
    else:
        assert w == 0


def test_calibrate_rejects_before_the_device():
    n, d, k = 64, 64, 8
    ws = lib.gsi_calibrate_workspace_bytes(n, d, k)
    A, Q0, Q, W = 1 << 20, 2 << 20, 3 << 20, 4 << 20   # never dereferenced: every call fails first
    assert lib.gsi_calibrate(n, d, k, A, Q0, 0, Q, W, ws, None) == -2          # n_iter < 1
    assert lib.gsi_calibrate(n, d, k, A, Q0, 65, Q, W, ws, None) == -2         # n_iter > 64
    assert lib.gsi_calibrate(n, d, k, None, Q0, 1, Q, W, ws, None) == -1
    assert lib.gsi_calibrate(n, d, k, A + 4, Q0, 1, Q, W, ws, None) == -6
    assert lib.gsi_calibrate(n, d, k, A, Q0, 1, Q, W, ws - 1, None) == -5
    assert lib.gsi_calibrate(n, d, k, A, Q0, 1, A + 256, W, ws, None) == -2    # result overlaps A
    assert lib.gsi_calibrate(n, d, k, A, Q0, 1, Q0 + 16, W, ws, None) == -2    # partial overlap with Q0
    assert lib.gsi_calibrate(n, d, k, A, Q0, 1, W, W, ws, None) == -2          # result overlaps workspace


@pytest.mark.parametrize("eps", [-0.1, -1e-30, float("nan"), float("-inf")])
def test_eps_rejected_before_device(eps):
    """eps < 0 or NaN is GSI_ERR_EPS for both the layer and the stack entry points, and is
    detected before the handle or any buffer is read (the handles here are never dereferenced)."""
    p = vp(256)
    fake = vp(4096)
    assert lib.gsi_forward(fake, p, 1, ctypes.c_float(eps), p, p, None, p, 1 << 20, None) == -4
    assert lib.gsi_stack_decode(fake, p, 1, 1, ctypes.c_float(eps), p, p, None, p, 1 << 20, None) == -4
    assert lib.gsi_stack_decode(fake, p, 1, 64, ctypes.c_float(eps), p, p, None, p, 1 << 20, None) == -4


def test_noalloc_rejects_before_device():
    """The no-allocation decode validates like gsi_stack_decode and refuses the batched path's
    sizes (T_step >= 16) before touching the stack handle or the device."""
    p = vp(256)
    fake = vp(4096)
    f = ctypes.c_float
    assert lib.gsi_stack_decode_noalloc(None, p, 1, 1, f(0.1), p, p, None, None) == -1
    assert lib.gsi_stack_decode_noalloc(fake, p, -1, 1, f(0.1), p, p, None, None) == -2
    assert lib.gsi_stack_decode_noalloc(fake, p, 1, 0, f(0.1), p, p, None, None) == -2
    assert lib.gsi_stack_decode_noalloc(fake, p, 1, 1, f(float("nan")), p, p, None, None) == -4
    assert lib.gsi_stack_decode_noalloc(fake, p, 1, 16, f(0.1), p, p, None, None) == -5
    assert lib.gsi_stack_decode_noalloc(fake, p, 1, 64, f(0.1), p, p, None, None) == -5
    assert lib.gsi_stack_decode_noalloc(fake, p, 0, 1, f(0.1), p, p, None, None) == 0
