"""The decode-step oracle against library routines, closed forms and invariants, and planted
mistakes in a copy of it that some pin must reject (CPU only)."""
import numpy as np
import pytest

from oracle import gsi_step as step
from tests import step_pins

_real = {n: getattr(step, n) for n in ("layer_norm", "gelu_tanh", "attention_decode", "decode_block")}


@pytest.mark.parametrize("pin", step_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(step)


def m_ln_no_centre(x, gamma, beta, eps_ln=1e-5):
    x = np.asarray(x, dtype=np.float64)
    var = x.var(axis=-1, keepdims=True)
    return x / np.sqrt(var + eps_ln) * gamma + beta


def m_ln_std_not_var(x, gamma, beta, eps_ln=1e-5):
    x = np.asarray(x, dtype=np.float64)
    dev = x - x.mean(axis=-1, keepdims=True)
    return dev / (dev.std(axis=-1, keepdims=True) + eps_ln) ** 2 * gamma + beta


def m_ln_no_shift(x, gamma, beta, eps_ln=1e-5):
    return _real["layer_norm"](x, gamma, np.zeros_like(np.asarray(beta, dtype=np.float64)), eps_ln)


def m_gelu_erf(z):
    import math
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.vectorize(math.erf)(z / math.sqrt(2.0)))


def m_gelu_no_cube(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * z))


def m_attn_no_scale(q, K, V, n_heads):
    dh = np.asarray(q).reshape(-1).shape[0] // n_heads
    return _real["attention_decode"](np.asarray(q, dtype=np.float64) * np.sqrt(dh), K, V, n_heads)


def m_attn_one_head(q, K, V, n_heads):
    return _real["attention_decode"](q, K, V, 1)


def m_attn_last_position_dropped(q, K, V, n_heads):
    K = np.atleast_2d(K)
    V = np.atleast_2d(V)
    return _real["attention_decode"](q, K[:-1] if K.shape[0] > 1 else K, V[:-1] if V.shape[0] > 1 else V, n_heads)


def m_block_no_mlp(x, blk, K_cache, V_cache, pos, eps, n_heads):
    r = _real["decode_block"](x, blk, K_cache, V_cache, pos, eps, n_heads)
    r["x_next"] = r["x_next"] - r["y_mlp"]
    return r


def m_block_serial(x, blk, K_cache, V_cache, pos, eps, n_heads):
    """the MLP branch fed from x + y_out instead of the shared LayerNorm (a serial block)"""
    r = _real["decode_block"](x, blk, K_cache, V_cache, pos, eps, n_heads)
    from oracle import gsi_oracle as orc
    a2 = _real["layer_norm"](np.asarray(x, np.float64) + r["y_out"], blk["gamma"], blk["beta"])
    f = orc.forward(blk["fc_in"][0], blk["fc_in"][1], a2[None], eps)["y"][0]
    y = orc.forward(blk["fc_out"][0], blk["fc_out"][1], _real["gelu_tanh"](f)[None], eps)["y"][0]
    r["x_next"] = np.asarray(x, np.float64) + r["y_out"] + y
    return r


MUTANTS = [("layer_norm", m_ln_no_centre), ("layer_norm", m_ln_std_not_var), ("layer_norm", m_ln_no_shift),
           ("gelu_tanh", m_gelu_erf), ("gelu_tanh", m_gelu_no_cube), ("attention_decode", m_attn_no_scale),
           ("attention_decode", m_attn_one_head), ("attention_decode", m_attn_last_position_dropped),
           ("decode_block", m_block_no_mlp), ("decode_block", m_block_serial)]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=lambda m: getattr(m, "__name__", str(m)))
def test_mutant_rejected(monkeypatch, name, mutant):
    monkeypatch.setattr(step, name, mutant)
    caught = []
    for pin in step_pins.ALL_PINS:
        try:
            pin(step)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects {mutant.__name__}"


@pytest.mark.parametrize("eps", [0.05, 0.2, 1.5])
def test_shared_input_site_equals_its_two_sites(eps):
    """Two maps of one input on one basis (QKV and fc_in of a parallel block) run as one site with
    their rows stacked give, in the oracle, the two sites' outputs side by side and the same gate
    and ratio: the residual norm and the gate depend on the input and the basis only. At eps 1.5
    every token is fast, at 0.05 most are slow, at 0.2 both occur."""
    from oracle import gsi_oracle as orc
    rng = np.random.default_rng(30)
    d, k, n = 64, 8, 40
    Q, R = np.linalg.qr(rng.standard_normal((d, k + 24)))
    V, C = Q[:, :k], Q[:, k:]
    W1 = rng.standard_normal((3 * 16, d))
    W2 = rng.standard_normal((24, d))
    rho = rng.uniform(0.02, 0.4, n)
    z = rng.standard_normal((n, k))
    w = rng.standard_normal((n, C.shape[1]))
    s = rho * np.linalg.norm(z, axis=1) / (np.linalg.norm(w, axis=1) * np.sqrt(1 - rho ** 2))
    X = z @ V.T + (s[:, None] * w) @ C.T
    both = orc.forward(np.vstack([W1, W2]), V, X, eps)
    r1, r2 = orc.forward(W1, V, X, eps), orc.forward(W2, V, X, eps)
    assert np.array_equal(both["gate"], r1["gate"]) and np.array_equal(both["gate"], r2["gate"])
    np.testing.assert_allclose(both["rho"], r1["rho"], rtol=1e-12, atol=0)
    np.testing.assert_allclose(both["y"], np.hstack([r1["y"], r2["y"]]), rtol=1e-12, atol=1e-12)
    if eps == 0.2:
        assert 0 < both["gate"].sum() < n
