"""Plain, slow, fp64 CPU oracle of one batch-1 decode step of a GPT-J-shaped stack whose linear
maps are GSI sites, with an unchanged plain attention between them.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or execute this module:
it is used by the tests and by the benchmark's CPU-baseline timing leg. It shares no code with the
HIP library and imports nothing from it; the GSI sites themselves are gsi_oracle.forward.

Source: the technical summary "Gated Subspace Inference for transformer acceleration" (cited as
[GSI §n]) runs every linear map of GPT-2, GPT-J and OPT as a GSI site and leaves attention as it
is [GSI §3 item 4, §5 last bullet]; it does not describe the rest of the block. Readings taken
here (each listed in the design notes):
  * the block is GPT-J's parallel form: one LayerNorm a = LN(x) feeds both the attention branch
    (QKV site, attention, out site) and the MLP branch (fc_in site, GELU, fc_out site), and
    x' = x + y_out + y_mlp;
  * LayerNorm: (x - mean) / sqrt(var + 1e-5) * gamma + beta, var the mean squared deviation;
  * GELU in its tanh form, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)));
  * plain softmax attention per head over the cached positions 0 .. pos, scores scaled by
    1/sqrt(head dim), no positional rotation (none is on the pages), no bias terms;
  * the QKV site's output is [q | k | v], each d wide; k and v of the new token join the cache at
    position pos before attention.
All arithmetic is float64 on stored (upcast) values; numpy's matmul, exp and tanh are the library
primitives used as steps. Pins: tests/step_pins.py (run by tests/test_step_pins.py).
"""
from __future__ import annotations

import numpy as np

from oracle import gsi_oracle as orc

LN_EPS = 1e-5


def layer_norm(x, gamma, beta, eps_ln: float = LN_EPS) -> np.ndarray:
    """LayerNorm of each row of x (... x d): centred, divided by the root of the mean squared
    deviation plus eps_ln, then scaled by gamma and shifted by beta."""
    x = orc.as_f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    dev = x - mu
    var = (dev * dev).mean(axis=-1, keepdims=True)
    return dev / np.sqrt(var + eps_ln) * orc.as_f64(gamma) + orc.as_f64(beta)


def gelu_tanh(z) -> np.ndarray:
    """GELU in its tanh form, elementwise."""
    z = orc.as_f64(z)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (z + 0.044715 * z ** 3)))


def attention_decode(q, K, V, n_heads: int) -> np.ndarray:
    """One query row q (d) against the cached keys K and values V (L x d), per head h (columns
    h dh .. h dh + dh - 1, dh = d / n_heads): scores s_j = <q_h, K_jh> / sqrt(dh), weights
    p = softmax(s) over the L positions, output o_h = sum_j p_j V_jh."""
    q = orc.as_f64(q).reshape(-1)
    K = np.atleast_2d(orc.as_f64(K))
    V = np.atleast_2d(orc.as_f64(V))
    d = q.shape[0]
    if d % n_heads or K.shape[1] != d or V.shape != K.shape:
        raise ValueError("shapes do not chain")
    dh = d // n_heads
    o = np.empty(d)
    for h in range(n_heads):
        c = slice(h * dh, (h + 1) * dh)
        s = K[:, c] @ q[c] / np.sqrt(dh)
        p = np.exp(s - s.max())
        p /= p.sum()
        o[c] = p @ V[:, c]
    return o


def _site(pair, x, eps):
    """gsi_oracle.forward on one site given as (W, V) or (W, V, M) with M = W V precomputed."""
    return orc.forward(pair[0], pair[1], x[None], eps, M=pair[2] if len(pair) > 2 else None)


def decode_block(x, blk: dict, K_cache, V_cache, pos: int, eps: float, n_heads: int) -> dict:
    """One block for one token. blk holds the block's weights and bases: gamma, beta, and per site
    ("qkv", "out", "fc_in", "fc_out") (W, V) or (W, V, M) with M = W V already formed [GSI §2.1]
    (the out site's input is the attention output, the fc_out site's the GELU of the fc_in output).
    K_cache / V_cache (>= pos + 1 rows x d) hold the earlier positions; rows pos are overwritten
    with this token's k and v (in float64). Returns every intermediate: a, qkv, f, o, u, y_out,
    y_mlp, x_next, and the four sites' gates and ratios in the order QKV, out, fc_in, fc_out."""
    x = orc.as_f64(x).reshape(-1)
    d = x.shape[0]
    a = layer_norm(x, blk["gamma"], blk["beta"])
    r_qkv = _site(blk["qkv"], a, eps)
    r_fc = _site(blk["fc_in"], a, eps)
    qkv = r_qkv["y"][0]
    q, k, v = qkv[:d], qkv[d:2 * d], qkv[2 * d:3 * d]
    K_cache[pos] = k
    V_cache[pos] = v
    o = attention_decode(q, K_cache[:pos + 1], V_cache[:pos + 1], n_heads)
    u = gelu_tanh(r_fc["y"][0])
    r_out = _site(blk["out"], o, eps)
    r_mlp = _site(blk["fc_out"], u, eps)
    x_next = x + r_out["y"][0] + r_mlp["y"][0]
    return {"a": a, "qkv": qkv, "f": r_fc["y"][0], "o": o, "u": u, "y_out": r_out["y"][0],
            "y_mlp": r_mlp["y"][0], "x_next": x_next,
            "gates": np.array([r_qkv["gate"][0], r_out["gate"][0], r_fc["gate"][0], r_mlp["gate"][0]], np.uint8),
            "rho": np.array([r_qkv["rho"][0], r_out["rho"][0], r_fc["rho"][0], r_mlp["rho"][0]])}
