"""Pins of the training oracle (dropout forward, backward) against facts outside it.

[DSV2 page] ``MultiHeadLatentAttention`` (dropout on the attention weights, default 0.1) and
[MLA page] ``MLAAttention`` (the same in a trainable module).  References: the published
SplitMix64 outputs (tests/golden/splitmix64_reference.txt), the inference oracle (itself
pinned in test_oracle.py) at p = 0, a closed form for the first causal row, the binomial
spread of the keep fraction, and central finite differences of the forward for every
gradient.
"""
import os

import numpy as np
import pytest

import mla_synth as S
from oracle import mla_oracle as O
from oracle import train_oracle as T

TINY = S.CONFIGS["tiny_fp32"]
SMALL_DEC = S.CONFIGS["dsv2_prefill"].replace(name="dsv2_train_small", d_model=48, n_heads=3, d_nope=8,
                                              d_rope=4, r_kv=6, r_q=10, dtype="f32", batch=1, seq=11)


def _weights(cfg, seed=5, scale=0.7):
    r = np.random.default_rng(seed)
    return {k: r.standard_normal(s) * scale for k, s in cfg.weight_shapes().items()}


GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_reference.txt")


def _reference_outputs():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                vals = [int(v) for v in line.split()]
                rows.append((vals[0], vals[1:]))
    return rows


@pytest.mark.parametrize("state,outs", _reference_outputs(), ids=lambda v: str(v)[:12])
def test_splitmix64_matches_reference_outputs(state, outs):
    """Counter n of the oracle's generator is output n + 1 of SplitMix64 from the seed."""
    got = T.splitmix64(np.uint64(state), np.arange(len(outs), dtype=np.uint64))
    assert [int(v) for v in got] == outs


def test_splitmix64_vectorised_equals_scalar():
    n = np.arange(50, dtype=np.uint64) * np.uint64(977)
    words = T.splitmix64(np.uint64(11), n)
    for t in (0, 17, 49):
        assert int(words[t]) == int(T.splitmix64(np.uint64(11), n[t]))


@pytest.mark.parametrize("p", [0.1, 0.3, 0.5])
def test_keep_fraction_is_binomial(p):
    n_q, n_k = 200, 500
    keep = T.dropout_keep(1234, 0, 4, 2, n_q, n_k, p)
    n = keep.size
    assert abs(keep.mean() - (1 - p)) <= 5 * np.sqrt(p * (1 - p) / n)
    assert T.dropout_keep(1234, 0, 4, 2, n_q, n_k, 0.0).all()
    # different heads / sequences / seeds draw different masks
    assert (keep != T.dropout_keep(1234, 0, 4, 3, n_q, n_k, p)).mean() > 0.1
    assert (keep != T.dropout_keep(1234, 1, 4, 2, n_q, n_k, p)).mean() > 0.1
    assert (keep != T.dropout_keep(1235, 0, 4, 2, n_q, n_k, p)).mean() > 0.1


def test_keep_mask_element_addressing():
    """Element (i, j) of head h of sequence b uses bits 16 (j % 4) .. + 15 of output n + 1 of
    SplitMix64 from the seed, n = (b H + h) 2^38 + i 2^18 + j // 4 (the state advanced with
    Python integers here)."""
    p, seed, b, H, h = 0.4, 99, 1, 3, 2
    keep = T.dropout_keep(seed, b, H, h, 6, 13, p)
    thr = T.keep_threshold(p)
    assert thr == int(0.4 * 65536)
    gamma, mask = 0x9E3779B97F4A7C15, (1 << 64) - 1
    for i, j in np.ndindex(*keep.shape):
        n = ((b * H + h) << 38) + (i << 18) + (j // 4)
        w = int(T.splitmix64(np.uint64((seed + n * gamma) & mask), np.uint64(0)))
        assert keep[i, j] == (((w >> (16 * (j % 4))) & 0xFFFF) >= thr)


@pytest.mark.parametrize("cfg", [TINY, SMALL_DEC], ids=lambda c: c.name)
def test_no_dropout_is_the_inference_forward(cfg):
    W = _weights(cfg)
    x = np.random.default_rng(1).standard_normal((cfg.seq, cfg.d_model))
    d = O.Dims.from_cfg(cfg)
    y, _ = T.train_forward(x, W, d, 0.0, 7, 0)
    np.testing.assert_allclose(y, O.forward(x, W, d), atol=1e-12)


def test_first_row_closed_form_with_dropout():
    """Row 0 attends only to itself: its weight is 1, dropped or scaled to 1 / (1 - p), so
    y_0 = W_o [v_0,h keep_h(0, 0) / (1 - p)]_h."""
    cfg = SMALL_DEC
    W = _weights(cfg)
    x = np.random.default_rng(2).standard_normal((cfg.seq, cfg.d_model))
    d = O.Dims.from_cfg(cfg)
    p, seed, b = 0.5, 31, 3
    y, sv = T.train_forward(x, W, d, p, seed, b)
    v0 = (W["w_uv"] @ (W["w_dkv"] @ x[0])).reshape(cfg.n_heads, cfg.d_nope)
    ks = [T.dropout_keep(seed, b, cfg.n_heads, h, 1, 1, p)[0, 0] for h in range(cfg.n_heads)]
    assert any(ks) and not all(ks)               # this seed drops some heads' first weight
    o0 = np.concatenate([v0[h] * ks[h] / (1 - p) for h in range(cfg.n_heads)])
    np.testing.assert_allclose(y[0], W["w_o"] @ o0, atol=1e-12)


def test_lse_matches_softmax_rows():
    cfg = SMALL_DEC
    W = _weights(cfg)
    x = np.random.default_rng(3).standard_normal((cfg.seq, cfg.d_model))
    d = O.Dims.from_cfg(cfg)
    _, sv = T.train_forward(x, W, d, 0.2, 1, 0)
    lse = T.lse_log2(sv, d)
    q, k = sv["q"], sv["k"]
    for h in range(cfg.n_heads):
        s = d.scale() * (q[:, h] @ k[:, h].T)
        for i in range(cfg.seq):
            np.testing.assert_allclose(np.exp2(lse[h, i]), np.exp(s[i, :i + 1]).sum(), rtol=1e-12)


@pytest.mark.parametrize("cfg,p", [(TINY, 0.3), (SMALL_DEC, 0.25), (SMALL_DEC, 0.0)], ids=["tiny", "small", "small_p0"])
def test_gradients_match_finite_differences(cfg, p):
    """For f = sum(dy * y) with the dropout mask fixed by the seed, each gradient's inner
    product with a random direction equals the central difference of f along it."""
    W = _weights(cfg)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((cfg.seq, cfg.d_model))
    d = O.Dims.from_cfg(cfg)
    seed, b = 77, 1
    y, sv = T.train_forward(x, W, d, p, seed, b)
    dy = rng.standard_normal(y.shape)
    g = T.train_backward(dy, W, d, p, sv)

    def f(xx, WW):
        return float(np.sum(dy * T.train_forward(xx, WW, d, p, seed, b)[0]))

    eps = 1e-5
    for name in ["x"] + sorted(W):
        base = x if name == "x" else W[name]
        delta = rng.standard_normal(base.shape)
        if name == "x":
            fp, fm = f(x + eps * delta, W), f(x - eps * delta, W)
        else:
            fp = f(x, {**W, name: W[name] + eps * delta})
            fm = f(x, {**W, name: W[name] - eps * delta})
        fd = (fp - fm) / (2 * eps)
        an = float(np.sum(g[name] * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)
        assert g[name].shape == base.shape
