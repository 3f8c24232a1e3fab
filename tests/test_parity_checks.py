"""The comparison the GPU parity tests apply must reject plausible kernel mistakes (CPU only).

A mistaken kernel output is built on the host from the fp64 oracle's own intermediate values and
handed to the same `compare_site` the GPU tests use.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gsi_oracle as orc
from tests.gpu_util import TOL, compare_site, rel_l2


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16).double().numpy()


@pytest.fixture(scope="module")
def gptj_out_site():
    """Block 0's attention-output site of the GPT-J-shaped batch-1 workload (4096 -> 4096, k = 256,
    eps = 0.10, 512 tokens of which one is slow)."""
    cfg = synth.get(3)
    si = synth.site_inputs(cfg, 0, 1)
    W = synth.site_weight(cfg, 0, 1)
    ref = orc.forward(W, si.V, si.X, cfg.eps)
    M = orc.precompute_image(W, si.V)
    return cfg, ref, M


def test_correct_output_passes(gptj_out_site):
    _, ref, _ = gptj_out_site
    err, worst = compare_site(_bf16(ref["y"]), ref["gate"], ref, TOL["bf16"], where="exact")
    assert worst < 5e-3


def test_slow_token_answered_by_fast_path_is_rejected(gptj_out_site):
    """A kernel that returned M g for the slow token too: the site-wide error stays under the
    tolerance (one token in 512), so only the per-token and slow-token checks can see it."""
    _, ref, M = gptj_out_site
    slow = ref["gate"] == orc.SLOW
    assert slow.sum() == 1
    y_bad = _bf16(ref["g"] @ M.T)
    assert rel_l2(y_bad, ref["y"]) <= TOL["bf16"], "the site-wide check alone would pass"
    bad_tok = np.linalg.norm(y_bad[slow] - ref["y"][slow]) / np.linalg.norm(ref["y"][slow])
    assert bad_tok > 5 * TOL["bf16"]
    with pytest.raises(AssertionError, match="token|slow"):
        compare_site(y_bad, ref["gate"], ref, TOL["bf16"], where="slow-as-fast")


def test_flipped_gate_bit_is_rejected(gptj_out_site):
    _, ref, _ = gptj_out_site
    gate = ref["gate"].copy()
    gate[3] ^= 1
    with pytest.raises(AssertionError, match="gate bits"):
        compare_site(_bf16(ref["y"]), gate, ref, TOL["bf16"], where="flipped gate")


def test_one_token_from_the_wrong_row_is_rejected(gptj_out_site):
    _, ref, _ = gptj_out_site
    y_bad = _bf16(ref["y"])
    y_bad[100] = y_bad[101]
    with pytest.raises(AssertionError, match="token 100|rel L2"):
        compare_site(y_bad, ref["gate"], ref, TOL["bf16"], where="wrong row")
