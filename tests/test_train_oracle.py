"""Pins of the training oracle (dropout forward, backward) against facts outside it.

[DSV2 page] ``MultiHeadLatentAttention`` (dropout on the attention weights, default 0.1) and
[MLA page] ``MLAAttention`` (the same in a trainable module).  References: numpy's Philox
bit generator (Philox4x64-10), the inference oracle (itself pinned in test_oracle.py) at
p = 0, a closed form for the first causal row, the binomial spread of the keep fraction,
and central finite differences of the forward for every gradient.
"""
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


@pytest.mark.parametrize("key,ctr", [((0, 0), (0, 0, 0, 0)), ((123, 456), (7, 8, 9, 10)),
                                     ((2**64 - 1, 2**63 + 5), (2**64 - 2, 1, 2**40 + 3, 99))])
def test_philox_matches_numpy(key, ctr):
    """numpy.random.Philox is Philox4x64-10; it increments its counter before each block, so
    its first four raw outputs from counter c are the block at c + 1."""
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(ctr, dtype=np.uint64))
    raw = bg.random_raw(8)
    c = list(ctr)
    for blk in range(2):
        for w in range(4):                       # 256-bit counter increment with carry
            c[w] = (c[w] + 1) % 2**64
            if c[w]:
                break
        got = T.philox4x64(*[np.uint64(v) for v in c], key[0], key[1])
        assert [int(w) for w in got] == [int(w) for w in raw[4 * blk:4 * blk + 4]]


def test_philox_vectorised_equals_scalar():
    c0 = np.arange(50, dtype=np.uint64) * np.uint64(977)
    words = T.philox4x64(c0, np.uint64(3), np.uint64(5), np.uint64(0), 11, 0)
    for t in (0, 17, 49):
        one = T.philox4x64(c0[t], np.uint64(3), np.uint64(5), np.uint64(0), 11, 0)
        assert all(int(words[w][t]) == int(one[w]) for w in range(4))


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
    """Element (i, j) uses word j % 4 of the block at counter (j // 4, i, b H + h, 0)."""
    p, seed, b, H, h = 0.4, 99, 1, 3, 2
    keep = T.dropout_keep(seed, b, H, h, 6, 13, p)
    thr = T.keep_threshold(p)
    for i, j in [(0, 0), (5, 12), (3, 7), (2, 4)]:
        w = T.philox4x64(np.uint64(j // 4), np.uint64(i), np.uint64(b * H + h), np.uint64(0), seed, 0)[j % 4]
        assert keep[i, j] == (int(w) >> 32 >= thr)


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
