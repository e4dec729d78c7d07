"""Pins of the CCA / CCGQA oracle against facts that do not come from the oracle itself.

[CCA page] frankenstein-transformer docs, ``latent/cca_attn``: ``_apply_causal_convs``,
``CCAAttention.forward``, ``CCGQAAttention.forward``.  Independent references: torch's
conv1d and scaled_dot_product_attention in fp64, numpy's convolve, closed forms for special
weights, and invariants the page's definition implies (causality, invariance of the
normalised queries and keys to the scale of the projections, the GQA reduction when every
query head has its own key head, the first causal row).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import mla_synth as S
from oracle import cca_oracle as C
from oracle import mla_oracle as O

torch.set_default_dtype(torch.float64)

TINY_CCA = S.CCA_CONFIGS["cca_tiny_fp32"]
TINY_GQA = S.CCA_CONFIGS["ccgqa_tiny_fp32"]


def _weights(cfg, seed=3, scale=0.6):
    r = np.random.default_rng(seed)
    return {k: r.standard_normal(s) * scale for k, s in cfg.weight_shapes().items()}


def _x(cfg, seed=4, S_=None):
    return np.random.default_rng(seed).standard_normal((S_ or cfg.seq, cfg.d_model))


# ---------------------------------------------------------------------------
# The causal convolutions ([CCA page] _apply_causal_convs)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("k", [1, 3, 4])
def test_depthwise_conv_matches_torch_conv1d(k):
    r = np.random.default_rng(k)
    S_, Cn = 11, 6
    u, w = r.standard_normal((S_, Cn)), r.standard_normal((Cn, k))
    want = F.conv1d(F.pad(torch.from_numpy(u.T[None]), (k - 1, 0)), torch.from_numpy(w[:, None, :]),
                    groups=Cn)[0].numpy().T
    np.testing.assert_allclose(C.causal_conv_depthwise(u, w), want, atol=1e-13)


def test_depthwise_conv_matches_numpy_convolve():
    """Per channel a causal FIR filter: out = (u * flip(w))[:S] (numpy's full convolution)."""
    r = np.random.default_rng(9)
    u, w = r.standard_normal((13, 3)), r.standard_normal((3, 4))
    got = C.causal_conv_depthwise(u, w)
    for c in range(3):
        np.testing.assert_allclose(got[:, c], np.convolve(u[:, c], w[c, ::-1])[:13], atol=1e-13)


@pytest.mark.parametrize("groups,k", [(2, 3), (4, 1), (3, 2)])
def test_grouped_conv_matches_torch_conv1d(groups, k):
    r = np.random.default_rng(groups + 10 * k)
    S_, Cn = 10, 12
    u, w = r.standard_normal((S_, Cn)), r.standard_normal((Cn, Cn // groups, k))
    want = F.conv1d(F.pad(torch.from_numpy(u.T[None]), (k - 1, 0)), torch.from_numpy(w),
                    groups=groups)[0].numpy().T
    np.testing.assert_allclose(C.causal_conv_grouped(u, w, groups), want, atol=1e-13)


def test_conv_impulse_response_closed_form():
    """A unit impulse at step t0 in channel c comes out as the flipped filter: output step
    t0 + m carries w[c, k - 1 - m] for m < k and nothing earlier (causality)."""
    k, S_, Cn = 4, 12, 2
    w = np.arange(1.0, 1.0 + Cn * k).reshape(Cn, k)
    u = np.zeros((S_, Cn))
    u[5, 1] = 1.0
    out = C.causal_conv_depthwise(u, w)
    assert np.all(out[:5] == 0) and np.all(out[:, 0] == 0)
    np.testing.assert_array_equal(out[5:9, 1], w[1, ::-1])
    assert np.all(out[9:] == 0)


# ---------------------------------------------------------------------------
# Layer-level invariants and reductions
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [TINY_CCA, TINY_GQA], ids=lambda c: c.name)
def test_causality(cfg):
    """Decoder mode: y_t does not depend on x_{t'} for t' > t (convolutions, value shift
    and attention are all causal)."""
    W, x = _weights(cfg), _x(cfg)
    y = C.forward(x, W, cfg)
    for t in (0, 3, 7):
        x2 = x.copy()
        x2[t + 1:] += np.random.default_rng(t).standard_normal(x2[t + 1:].shape) * 3
        y2 = C.forward(x2, W, cfg)
        np.testing.assert_allclose(y2[:t + 1], y[:t + 1], atol=1e-12)
        assert np.max(np.abs(y2[t + 1:] - y[t + 1:])) > 1e-6


@pytest.mark.parametrize("cfg", [TINY_CCA, TINY_GQA], ids=lambda c: c.name)
@pytest.mark.parametrize("which", ["w_qk", "conv_seq", "conv_ch"])
def test_qk_normalisation_removes_projection_scale(cfg, which):
    """The queries and keys are linear in w_qk and in each convolution's filter (the
    q-k-mean included), and the L2 normalisation divides any positive scale out: scaling
    one of them by 7 leaves the layer unchanged."""
    W, x = _weights(cfg), _x(cfg)
    W2 = dict(W)
    W2[which] = W[which] * 7.0
    if which != "w_qk":
        # q-k-mean adds unconvolved terms: scale them too so q and k stay proportional
        W2 = {**W2, "w_qk": W["w_qk"]}
        cfg = cfg.replace(qk_mean=False)
    np.testing.assert_allclose(C.forward(x, W2, cfg), C.forward(x, W, cfg), rtol=1e-10, atol=1e-12)


def test_ccgqa_with_one_query_head_per_key_head_is_cca():
    """[CCA page] CCGQA with as many key / value heads as query heads (group size 1) is
    CCA: the grouped q-k-mean, the head replication and the convolution groups reduce."""
    cfg = TINY_CCA
    W, x = _weights(cfg), _x(cfg)
    np.testing.assert_allclose(C.ccgqa_forward(x, W, cfg), C.cca_forward(x, W, cfg), atol=1e-12)


def test_ccgqa_equals_cca_with_replicated_key_heads_without_convolutions():
    """Without convolutions and q-k-mean, CCGQA is CCA whose key and value heads are
    copies of the group's key / value head (the same key / value rows per group)."""
    g = TINY_GQA.replace(num_conv_layers=0, qk_mean=False)
    Wg, x = _weights(g), _x(g)
    Hq, Hkv, dh = g.n_heads, g.n_kv_heads, g.head_dim
    gs = Hq // Hkv
    Lq = Hq * dh
    c = g.replace(n_kv_heads=Hq)
    wk = Wg["w_qk"][Lq:].reshape(Hkv, dh, -1)
    wv = Wg["w_v"].reshape(2, Hkv // 2, dh, -1)       # value shift: [current; previous] halves
    # CCA value heads: its first half sees the current token, the second half the previous
    # token; replicate each CCGQA key / value head gs times in head order
    wv_rep = np.repeat(wv.reshape(Hkv, dh, -1), gs, axis=0)
    half = Hq // 2
    assert np.all(np.arange(Hq)[:half] // gs < Hkv // 2)   # the halves line up for these dims
    Wc = {"w_qk": np.concatenate([Wg["w_qk"][:Lq], np.repeat(wk, gs, axis=0).reshape(Hq * dh, -1)]),
          "w_v": wv_rep.reshape(Hq * dh, -1), "conv_seq": np.zeros((2 * Lq, g.conv_kernel_seq)),
          "conv_ch": np.zeros((2 * Lq, dh, g.conv_kernel_ch)), "w_o": Wg["w_o"]}
    np.testing.assert_allclose(C.ccgqa_forward(x, Wg, g), C.cca_forward(x, Wc, c), atol=1e-12)


@pytest.mark.parametrize("cfg", [TINY_CCA, TINY_GQA], ids=lambda c: c.name)
def test_qk_mean_closed_form_with_identity_convolutions(cfg):
    """With filters that pass their input through (last tap 1), the convolved q, k equal
    the projections, and q-k-mean gives q = 1.5 q_pre + 0.5 k_pre(group) and
    k = 1.5 k_pre + 0.5 mean over the group of q_pre."""
    W, x = _weights(cfg), _x(cfg)
    cp = (cfg.n_heads + cfg.n_kv_heads) * cfg.head_dim
    W["conv_seq"] = np.zeros((cp, cfg.conv_kernel_seq))
    W["conv_seq"][:, -1] = 1.0
    W["conv_ch"] = np.zeros((cp, cfg.head_dim, cfg.conv_kernel_ch))
    for o in range(cp):
        W["conv_ch"][o, o % cfg.head_dim, -1] = 1.0
    Hq, Hkv, dh = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    gs = Hq // Hkv
    P = x @ W["w_qk"].T
    qp = P[:, :Hq * dh].reshape(-1, Hq, dh)
    kp = P[:, Hq * dh:].reshape(-1, Hkv, dh)
    q, k = (C.ccgqa_qk if Hkv != Hq else C.cca_qk)(x, W, cfg)
    for h in range(Hq):
        np.testing.assert_allclose(q[:, h], 1.5 * qp[:, h] + 0.5 * kp[:, h // gs], atol=1e-12)
    for j in range(Hkv):
        np.testing.assert_allclose(k[:, j], 1.5 * kp[:, j] + 0.5 * qp[:, j * gs:(j + 1) * gs].mean(axis=1),
                                   atol=1e-12)


@pytest.mark.parametrize("cfg", [TINY_CCA, TINY_GQA], ids=lambda c: c.name)
def test_first_row_closed_form(cfg):
    """Row 0 attends only to itself (softmax over one key is 1), and with value shift the
    previous-token half of the value heads is zero there (x_{-1} = 0):
    y_0 = W_o [v_{kv(h)}]_h with v = [x_0 W_v1^T ; 0]."""
    W, x = _weights(cfg), _x(cfg)
    Hq, Hkv, dh = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    half = Hkv * dh // 2
    v0 = np.concatenate([W["w_v"][:half] @ x[0], np.zeros(half)]).reshape(Hkv, dh)
    o0 = np.concatenate([v0[h // (Hq // Hkv)] for h in range(Hq)])
    np.testing.assert_allclose(C.forward(x, W, cfg)[0], W["w_o"] @ o0, atol=1e-12)


def test_value_shift_off_first_row():
    cfg = TINY_CCA.replace(value_shift=False)
    W, x = _weights(cfg), _x(cfg)
    np.testing.assert_allclose(C.forward(x, W, cfg)[0], W["w_o"] @ (W["w_v"] @ x[0]), atol=1e-12)


@pytest.mark.parametrize("beta", [-0.7, 0.0, 1.3])
def test_key_temperature_is_a_score_scale(beta):
    """k scaled by exp(beta) after normalisation multiplies every score by exp(beta):
    the same as beta = 0 with the softmax scale d_h^{-1/2} exp(beta)."""
    cfg = TINY_GQA.replace(beta=beta)
    W, x = _weights(cfg), _x(cfg)
    want = C.forward(x, W, cfg.replace(beta=0.0), scale=cfg.head_dim ** -0.5 * math.exp(beta))
    np.testing.assert_allclose(C.forward(x, W, cfg), want, atol=1e-12)


def test_attention_core_matches_torch_sdpa():
    """Without convolutions, q-k-mean and value shift, the whole CCGQA layer against torch
    in fp64: normalised projections, half-split RoPE as complex multiplication, and
    scaled_dot_product_attention with a causal mask."""
    cfg = TINY_GQA.replace(num_conv_layers=0, qk_mean=False, value_shift=False, beta=0.4)
    W, x = _weights(cfg), _x(cfg)
    Hq, Hkv, dh = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    gs = Hq // Hkv
    S_ = x.shape[0]
    tx = torch.from_numpy(x)
    P = tx @ torch.from_numpy(W["w_qk"]).T
    q = P[:, :Hq * dh].reshape(S_, Hq, dh)
    k = P[:, Hq * dh:].reshape(S_, Hkv, dh).repeat_interleave(gs, dim=1)
    v = (tx @ torch.from_numpy(W["w_v"]).T).reshape(S_, Hkv, dh).repeat_interleave(gs, dim=1)
    q = q / q.norm(dim=-1, keepdim=True) * math.sqrt(dh)
    k = k / k.norm(dim=-1, keepdim=True) * math.sqrt(dh) * math.exp(cfg.beta)

    def rope(a):       # half-split pairs as complex numbers, rotated by exp(i t theta_j)
        half = dh // 2
        th = 10000.0 ** (-torch.arange(half, dtype=torch.float64) * 2 / dh)
        z = torch.complex(a[..., :half], a[..., half:]) * torch.polar(torch.ones(S_, 1, half),
                                                                       torch.arange(S_)[:, None, None] * th)
        return torch.cat([z.real, z.imag], dim=-1)

    q, k = rope(q), rope(k)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), is_causal=True,
                                       scale=dh ** -0.5).transpose(0, 1)
    want = o.reshape(S_, -1) @ torch.from_numpy(W["w_o"]).T
    np.testing.assert_allclose(C.forward(x, W, cfg), want.numpy(), atol=1e-12)


def test_page_defaults_in_workloads():
    """The two large workloads use the page's defaults: CCA latent E/4 (C = 4); CCGQA query
    latent E/2 (C1 = 2), key / value latent E/8 (C2 = 8), a quarter of the heads as key
    heads; two convolutions with kernels 4 and 3."""
    a, g = S.CCA_CONFIGS["cca"], S.CCA_CONFIGS["ccgqa"]
    assert a.q_latent == a.d_model // 4 and a.n_kv_heads == a.n_heads
    assert g.q_latent == g.d_model // 2 and g.kv_latent == g.d_model // 8 and g.n_kv_heads == g.n_heads // 4
    for c in (a, g):
        assert (c.num_conv_layers, c.conv_kernel_seq, c.conv_kernel_ch) == (2, 4, 3)
        assert c.qk_mean and c.value_shift and c.head_dim % 2 == 0
