"""GPU parity of the calibration (subspace iteration with DGKS Gram-Schmidt, depth cascade)
against the fp64 oracle on the same float32 inputs.

Tolerance (float32 arithmetic against fp64): the products are float32 sums of n or d terms
(relative error ~ sqrt(len) * 2^-24 ~ 4e-6 at 4096) and Gram-Schmidt amplifies it by at most the
conditioning of A^T A Q (<= (s_max / s_min)^2 = 4 plus noise for these inputs), so the basis
(stored by rows) must match within 1e-4 relative Frobenius per layer, with rows orthonormal to
1e-5 and the spans within 1e-4 (largest principal sine).
"""
import numpy as np
import pytest
import torch

from oracle import gsi_calibration as cal
from synth.calibration import CalibrationChain, activations, cold_start, planted_bases
from tests.gpu_util import say

pytestmark = pytest.mark.gpu
TOL_REL = 1e-4


@pytest.fixture(scope="module")
def g():
    import gated_rank_linear_amd as g
    assert g.gsi_device_check() == 0
    return g


def _gpu_calibrate(g, A, Q0t, n_iter, out=None):
    n, d = A.shape
    k = Q0t.shape[0]
    ws = torch.empty(g.gsi_calibrate_workspace_bytes(n, d, k), dtype=torch.uint8, device="cuda")
    Qt = torch.empty((k, d), dtype=torch.float32, device="cuda") if out is None else out
    g.gsi_calibrate(A, Q0t, n_iter, Qt, ws)
    torch.cuda.synchronize()
    return Qt


def _compare(Qt_gpu, Q_orc, label):
    Qg = Qt_gpu.detach().cpu().double().numpy().T           # d x k
    rel = np.linalg.norm(Qg - Q_orc) / np.linalg.norm(Q_orc)
    orth = np.max(np.abs(Qg.T @ Qg - np.eye(Qg.shape[1])))
    sin = cal.principal_sines(Q_orc, Qg)[0]
    say(f"  {label}: rel {rel:.2e}, orthonormality {orth:.2e}, largest sine {sin:.2e}")
    assert rel <= TOL_REL and orth <= 1e-5 and sin <= TOL_REL, label
    return rel


def test_cascade_small_chain(g):
    """Three layers of a 25-degree chain (n = 512, d = 1024, k = 64): cold start with 4 steps for
    layer 0, then 2 warm steps per layer from the previous basis, on the GPU and in the oracle."""
    c = CalibrationChain(cid=2, n_layers=3, n=512, d=1024, k=64)
    say("case: calibration cascade, 3 layers, n=512 d=1024 k=64")
    P = planted_bases(c)
    As = [activations(c, l, P[l]) for l in range(c.n_layers)]
    Om = cold_start(c)
    ref = cal.calibrate_cascade(As, Om.numpy().T, 4, 2)
    Q = Om.cuda()
    for l, A in enumerate(As):
        Q = _gpu_calibrate(g, A.cuda(), Q, 4 if l == 0 else 2)
        _compare(Q, ref[l], f"layer {l}")


@pytest.mark.parametrize("n,d,k,iters", [(200, 136, 24, 3), (64, 64, 8, 1), (1000, 520, 40, 2), (96, 264, 72, 5),
                                         (304, 2040, 40, 2), (256, 8192, 72, 1), (128, 6152, 20, 2)])
def test_ragged_shapes(g, n, d, k, iters):
    """Sizes off every tile (rows, columns and K tails of the products; k not a power of two);
    every width class of the in-panel Gram-Schmidt (1, 2, 4, 8 and 16 elements of a row per
    thread: panels of 16, 16, 16, 8 and 4 rows), the ragged last panel included."""
    rng = np.random.default_rng(n + d + k)
    B = np.linalg.qr(rng.standard_normal((d, k)))[0]
    A = (rng.standard_normal((n, k)) * np.linspace(6, 3, k)) @ B.T + 0.3 * rng.standard_normal((n, d))
    A32 = torch.from_numpy(A.astype(np.float32))
    Q0 = torch.from_numpy(rng.standard_normal((k, d)).astype(np.float32))
    say(f"case: calibration ragged n={n} d={d} k={k} iters={iters}")
    ref = cal.subspace_iteration(A32.numpy(), Q0.numpy().T, iters)
    _compare(_gpu_calibrate(g, A32.cuda(), Q0.cuda(), iters), ref, "ragged")


@pytest.mark.parametrize("n,d,k,iters", [(2048, 4096, 256, 2), (1024, 16384, 512, 1)])
def test_full_widths(g, n, d, k, iters):
    """The GPT-J-shaped calibration size (d = 4096, k = 256, 2048 tokens) and the widest input
    (d = 16384, the fc_out width, at the largest rank k = 512), compared in full."""
    c = CalibrationChain(cid=3, n_layers=1, n=n, d=d, k=k)
    say(f"case: calibration full width n={n} d={d} k={k} iters={iters}")
    P = planted_bases(c)
    A = activations(c, 0, P[0])
    Om = cold_start(c)
    ref = cal.subspace_iteration(A.numpy(), Om.numpy().T, iters)
    _compare(_gpu_calibrate(g, A.cuda(), Om.cuda(), iters), ref, f"d={d}")


def test_in_place_and_reproducible(g):
    """Qt == Q0t gives the same bits as a separate output; two runs give identical bits."""
    c = CalibrationChain(cid=4, n_layers=1, n=256, d=512, k=32)
    P = planted_bases(c)
    A = activations(c, 0, P[0]).cuda()
    Om = cold_start(c).cuda()
    say("case: calibration in place and reproducible")
    a = _gpu_calibrate(g, A, Om, 3)
    b = _gpu_calibrate(g, A, Om, 3)
    q = Om.clone()
    _gpu_calibrate(g, A, q, 3, out=q)
    assert torch.equal(a, b) and torch.equal(a, q)


def test_reorthogonalisation_on_ill_conditioned_rows(g):
    """With A = I (A^T A = I exactly in float32) one call orthonormalises Q0 itself. Q0's rows
    are B S R (B orthonormal, S = diag from 1 to 1e-4, R a random rotation): condition number
    1e4, so one Gram-Schmidt pass loses orthogonality (|Q Q^T - I| ~ u cond^2 ~ 0.2 in float32,
    checked on the CPU) while the DGKS second projection keeps it at float32 rounding. The span
    of every leading block of rows matches the oracle's within u times that block's condition
    number (at most 1e4 here, so <= 1e-3)."""
    d, k = 256, 48
    rng = np.random.default_rng(5)
    B = np.linalg.qr(rng.standard_normal((d, k)))[0]
    R = np.linalg.qr(rng.standard_normal((k, k)))[0]
    Q0 = torch.from_numpy((B @ np.diag(np.geomspace(1.0, 1e-4, k)) @ R).T.astype(np.float32).copy())
    A = torch.eye(d, dtype=torch.float32)
    say("case: calibration DGKS on ill-conditioned rows (A = I)")
    Qt = _gpu_calibrate(g, A.cuda(), Q0.cuda(), 1)
    Qg = Qt.double().cpu().numpy().T
    orth = np.max(np.abs(Qg.T @ Qg - np.eye(k)))
    say(f"  orthonormality {orth:.2e}")
    assert orth <= 1e-5
    ref, twice = cal.dgks_orthonormalize(Q0.double().numpy().T)
    assert twice.sum() > k // 2
    for j in (4, 16, 32, 48):
        sin = cal.principal_sines(ref[:, :j], Qg[:, :j])[0]
        say(f"  leading {j} rows: largest sine {sin:.2e}")
        assert sin <= (1e-5 if j == 4 else 1e-3), j


def test_cascade_at_the_measured_size(g):
    """The cascade as the benchmark times it (GPT-J-shaped chain: 2048 tokens x 4096, k = 256,
    layer 0 from the Gaussian start with 8 steps, then 2 warm steps per layer), on its first four
    layers, against the oracle."""
    from synth.calibration import GPTJ_CALIBRATION as c
    say("case: calibration cascade at the measured size, 4 layers, n=2048 d=4096 k=256")
    P = planted_bases(c, 4)
    As = [activations(c, l, P[l]) for l in range(4)]
    Om = cold_start(c)
    ref = cal.calibrate_cascade(As, Om.numpy().T, 8, 2)
    Q = Om.cuda()
    for l, A in enumerate(As):
        Q = _gpu_calibrate(g, A.cuda(), Q, 8 if l == 0 else 2)
        _compare(Q, ref[l], f"layer {l}")
