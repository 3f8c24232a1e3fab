"""GPU parity of the batch-1 decode kernel at the ranks of the operating-point sweep.

One GPT-J-shaped block (QKV 4096->12288, out 4096->4096, fc_in 4096->16384, fc_out 16384->4096,
bf16) at k = 64, 128 and 512 (k = 256 is covered by the full-stack tests), 48 tokens per site of
which 6 are slow: gate bits against the fp64 oracle bit for bit, y within 2e-2 relative L2 per
site. At k = 512 the fc_out slice of V_k fills a whole LDS region, so the M rows and the
(V^T V - I) rows of that site are read from HBM instead: that path is covered here.
"""
import dataclasses

import pytest

from synth.configs import SlowPlan, sweep_config
from tests.gpu_util import Built, check_site, decode, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import gated_rank_linear_amd as g
    assert g.gsi_device_check() == 0
    return g


@pytest.mark.parametrize("k", [64, 128, 512])
def test_sweep_rank_one_block(g, k):
    cfg = dataclasses.replace(sweep_config(k), n_blocks=1, n_steps=48, slow=SlowPlan("fixed", count=6))
    say(f"case: sweep rank k={k}, one GPT-J-shaped block, 48 tokens, batch 1")
    built = Built(cfg, blocks=[0], keep_w_for="all")
    Y, gates, _, _ = decode(built, cfg.eps)
    Ys = built.split_outputs(Y)
    worst = 0.0
    for i in range(len(built.sites)):
        worst = max(worst, check_site(built, i, Ys[i], gates[:, i], cfg.eps, with_y=True))
    assert int(gates.sum()) == 6 * len(built.sites)
    say(f"  gates exact, worst y rel L2 {worst:.2e}")
