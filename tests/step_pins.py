"""Pins of the decode-step oracle (oracle/gsi_step.py) against library routines, closed forms and
invariants; each pin takes the module under test so that planted mistakes can be run through them.

  S1 layer_norm equals torch.nn.functional.layer_norm (float64).
  S2 layer_norm is unchanged by x -> c x + b 1 (c > 0) with unit gain and zero shift, and its rows
     then have mean 0 and mean square var / (var + eps).
  S3 gelu_tanh equals torch.nn.functional.gelu(approximate="tanh"); gelu(0) = 0 and
     gelu(z) - gelu(-z) = z exactly (tanh is odd).
  S4 attention_decode equals torch.nn.functional.scaled_dot_product_attention per head (float64).
  S5 attention special cases: one position gives o = v; equal keys give the mean of the values;
     one key far ahead of the others gives that position's value.
  S6 decode_block at eps = 0 (every site slow, y = W x) equals a dense GPT-J-shaped block written
     with torch's LayerNorm, linear maps, GELU and attention; the new k and v are in the cache.
  S7 decode_block at eps > 1 (every site fast, y = M g = W V V^T x) equals the same dense block on
     the weights W V V^T.
"""
import numpy as np
import torch
import torch.nn.functional as F


def _rng(seed):
    return np.random.default_rng(seed)


def s1_layer_norm_library(step):
    rng = _rng(1)
    for d in (8, 77, 768):
        x = rng.standard_normal((5, d)) * 3 + 1.5
        g = rng.standard_normal(d)
        b = rng.standard_normal(d)
        ref = F.layer_norm(torch.from_numpy(x), (d,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-5).numpy()
        assert np.allclose(step.layer_norm(x, g, b), ref, rtol=1e-12, atol=1e-12)


def s2_layer_norm_invariance(step):
    rng = _rng(2)
    d = 64
    x = rng.standard_normal((3, d))
    one, zero = np.ones(d), np.zeros(d)
    y = step.layer_norm(x, one, zero)
    # the shift cancels in the centring; the scale changes only eps's weight (var ~ 1 here, so
    # by ~eps / 2 relative)
    y2 = step.layer_norm(1e3 * x + 7.25, one, zero)
    assert np.allclose(y, y2, rtol=1e-4, atol=1e-4)
    var = x.var(axis=1)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((y * y).mean(axis=1), var / (var + 1e-5), rtol=1e-12)


def s3_gelu(step):
    z = np.linspace(-6, 6, 241)
    ref = F.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    assert np.allclose(step.gelu_tanh(z), ref, rtol=1e-13, atol=1e-15)
    assert step.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert np.allclose(step.gelu_tanh(z) - step.gelu_tanh(-z), z, rtol=0, atol=1e-14)


def s4_attention_library(step):
    rng = _rng(4)
    for d, H, L in ((64, 2, 1), (96, 3, 17), (256, 4, 40)):
        q = rng.standard_normal(d)
        K = rng.standard_normal((L, d))
        V = rng.standard_normal((L, d))
        dh = d // H
        qt = torch.from_numpy(q).view(1, H, 1, dh)
        Kt = torch.from_numpy(K).view(L, H, dh).permute(1, 0, 2).unsqueeze(0)
        Vt = torch.from_numpy(V).view(L, H, dh).permute(1, 0, 2).unsqueeze(0)
        ref = F.scaled_dot_product_attention(qt, Kt, Vt).reshape(d).numpy()
        assert np.allclose(step.attention_decode(q, K, V, H), ref, rtol=1e-12, atol=1e-12)


def s5_attention_special(step):
    rng = _rng(5)
    d, H = 32, 2
    q = rng.standard_normal(d)
    v = rng.standard_normal((1, d))
    assert np.allclose(step.attention_decode(q, rng.standard_normal((1, d)), v, H), v[0], rtol=1e-14)
    K = np.tile(rng.standard_normal(d), (6, 1))
    V = rng.standard_normal((6, d))
    assert np.allclose(step.attention_decode(q, K, V, H), V.mean(axis=0), rtol=1e-12)
    K = rng.standard_normal((5, d)) * 1e-3
    K[3] = 200.0 * np.sign(q)  # every head's score for position 3 is far ahead
    assert np.allclose(step.attention_decode(q, K, V[:5], H), V[3], rtol=1e-9, atol=1e-9)


def _dense_block_torch(x, blk, Kc, Vc, pos, H, weights):
    """The block with dense maps, from torch routines (float64)."""
    d = x.shape[0]
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    a = F.layer_norm(t(x), (d,), t(blk["gamma"]), t(blk["beta"]), eps=1e-5)
    qkv = F.linear(a, t(weights["qkv"]))
    q, k, v = qkv[:d], qkv[d:2 * d], qkv[2 * d:]
    K = t(Kc[:pos + 1]).clone()
    V = t(Vc[:pos + 1]).clone()
    K[pos] = k
    V[pos] = v
    dh = d // H
    o = F.scaled_dot_product_attention(q.view(1, H, 1, dh), K.view(pos + 1, H, dh).permute(1, 0, 2).unsqueeze(0),
                                       V.view(pos + 1, H, dh).permute(1, 0, 2).unsqueeze(0)).reshape(d)
    u = F.gelu(F.linear(a, t(weights["fc_in"])), approximate="tanh")
    return (t(x) + F.linear(o, t(weights["out"])) + F.linear(u, t(weights["fc_out"]))).numpy(), k.numpy(), v.numpy()


def _toy_block(seed, d=48, H=3, k=8, pos=4):
    rng = _rng(seed)
    blk = {"gamma": 1 + 0.1 * rng.standard_normal(d), "beta": 0.1 * rng.standard_normal(d)}
    shapes = {"qkv": (3 * d, d), "out": (d, d), "fc_in": (4 * d, d), "fc_out": (d, 4 * d)}
    for name, (do, di) in shapes.items():
        W = rng.standard_normal((do, di)) / np.sqrt(di)
        Q, R = np.linalg.qr(rng.standard_normal((di, k)))
        blk[name] = (W, Q * np.sign(np.diag(R)))
    Kc = rng.standard_normal((pos + 1, d))
    Vc = rng.standard_normal((pos + 1, d))
    x = rng.standard_normal(d)
    return blk, Kc, Vc, x, H, pos


def s6_block_all_slow(step):
    blk, Kc, Vc, x, H, pos = _toy_block(6)
    weights = {n: blk[n][0] for n in ("qkv", "out", "fc_in", "fc_out")}
    ref, k, v = _dense_block_torch(x, blk, Kc, Vc, pos, H, weights)
    K2, V2 = Kc.copy(), Vc.copy()
    r = step.decode_block(x, blk, K2, V2, pos, 0.0, H)
    assert np.all(r["gates"] == 1)
    assert np.allclose(r["x_next"], ref, rtol=1e-11, atol=1e-11)
    assert np.allclose(K2[pos], k, rtol=1e-12) and np.allclose(V2[pos], v, rtol=1e-12)


def s7_block_all_fast(step):
    blk, Kc, Vc, x, H, pos = _toy_block(7)
    weights = {n: blk[n][0] @ blk[n][1] @ blk[n][1].T for n in ("qkv", "out", "fc_in", "fc_out")}
    ref, _, _ = _dense_block_torch(x, blk, Kc, Vc, pos, H, weights)
    r = step.decode_block(x, blk, Kc.copy(), Vc.copy(), pos, 1.5, H)
    assert np.all(r["gates"] == 0)
    assert np.allclose(r["x_next"], ref, rtol=1e-10, atol=1e-10)


ALL_PINS = [s1_layer_norm_library, s2_layer_norm_invariance, s3_gelu, s4_attention_library, s5_attention_special,
            s6_block_all_slow, s7_block_all_fast]
