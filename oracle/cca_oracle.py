"""fp64 CPU oracle for compressed convolutional attention (CCA, CCGQA) -- TEST INFRASTRUCTURE.

Only the test suite and bench.py's CPU-baseline leg may import this module.  The GPU
library never calls it and shares no code with it: it is a plain, slow numpy-fp64
statement of what the CCA page defines, used to check the GPU kernels element by element.

Page followed (cited by title and section):
  [CCA page]  frankenstein-transformer docs, module ``latent/cca_attn``:
              ``_apply_causal_convs``, ``CCAAttention.forward`` and
              ``CCGQAAttention.forward`` (queries, keys and values down-projected into a
              compressed latent; attention runs inside the latent; a single output
              up-projection).

What the layer computes, in the page's order, for one sequence x [S, E]:
  1. packed down-projection P = x W_qk^T, split into the query part (Hq heads of d_h)
     and the key part (Hkv heads of d_h); the pre-convolution parts are kept;
  2. causal convolutions of P along the sequence: a depth-wise one (kernel k_seq), then a
     grouped one whose groups are the heads (kernel k_ch), each left-padded with zeros;
  3. q-k-mean: the mean of the pre-convolution query and key added to the convolved ones
     (CCGQA: each query head pairs with its key head; a key head takes the group mean);
  4. values x W_v^T, or with value shift [x_t W_v1^T ; x_{t-1} W_v2^T] (x_{-1} = 0),
     concatenated along the channels and then split into heads;
  5. q and k scaled to L2 norm sqrt(d_h) per head (norm clamped at 1e-6), k also by
     exp(beta) (the learnable key temperature);
  6. half-split RoPE in the latent at positions 0..S-1;
  7. causal softmax attention with scale d_h^{-1/2} (the page's decoder mode), query head
     h using key / value head h // (Hq / Hkv);
  8. y = concat_h(o_h) W_o^T.

Readings of points the page leaves open (also listed in the repository's design notes):
  * Value shift: the page's code concatenates the current-token and previous-token
    projections along the channels and then views the result as heads, so the first half
    of the value heads see the current token and the second half the previous one (its
    requirement of an even head count fits this); the module docstring's "half of each
    head's values" is not what the code does.  The code is followed.
  * w_v stacks the current-token rows above the previous-token rows ([2 x Hkv d_h / 2][E]).
  * Decoder mode (causal); inference: no dropout.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from . import mla_oracle as _mla

F64 = np.float64


def causal_conv_depthwise(u: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Depth-wise causal convolution along the sequence.

    [CCA page] ``_apply_causal_convs`` (the first convolution: one filter per channel,
    zero left padding of k - 1 steps): channel c at step t is
    sum_j w[c, j] * u[t - (k - 1) + j, c], with u = 0 before step 0.
    u [S, C], w [C, k] -> [S, C].
    """
    u = np.asarray(u, dtype=F64)
    w = np.asarray(w, dtype=F64)
    S, C = u.shape
    k = w.shape[1]
    padded = np.concatenate([np.zeros((k - 1, C)), u], axis=0)
    out = np.zeros((S, C))
    for j in range(k):
        out += w[:, j][None, :] * padded[j:j + S]
    return out


def causal_conv_grouped(u: np.ndarray, w: np.ndarray, groups: int) -> np.ndarray:
    """Grouped causal convolution along the sequence.

    [CCA page] ``_apply_causal_convs`` (the second convolution; its groups are the heads,
    so each output channel mixes the channels of its own head over k steps): for output
    channel o of group g = o // (C / groups),
    out[t, o] = sum_{c < C/groups} sum_j w[o, c, j] * u[t - (k - 1) + j, g C/groups + c].
    u [S, C], w [C, C / groups, k] -> [S, C].
    """
    u = np.asarray(u, dtype=F64)
    w = np.asarray(w, dtype=F64)
    S, C = u.shape
    cg = C // groups
    k = w.shape[2]
    padded = np.concatenate([np.zeros((k - 1, C)), u], axis=0)
    out = np.zeros((S, C))
    for g in range(groups):
        sl = slice(g * cg, (g + 1) * cg)
        for j in range(k):
            out[:, sl] += padded[j:j + S, sl] @ w[sl, :, j].T
    return out


def apply_causal_convs(P: np.ndarray, W: Dict[str, np.ndarray], cfg, groups: int) -> np.ndarray:
    """[CCA page] ``_apply_causal_convs``: none, the depth-wise one, or both in order."""
    out = np.asarray(P, dtype=F64)
    if cfg.num_conv_layers >= 1:
        out = causal_conv_depthwise(out, W["conv_seq"])
    if cfg.num_conv_layers >= 2:
        out = causal_conv_grouped(out, W["conv_ch"], groups)
    return out


def _values(x: np.ndarray, W: Dict[str, np.ndarray], cfg) -> np.ndarray:
    """[CCA page] ``forward`` value projection (step 4 above) -> [S, Hkv, d_h]."""
    x = np.asarray(x, dtype=F64)
    wv = np.asarray(W["w_v"], dtype=F64)
    S = x.shape[0]
    if cfg.value_shift:
        half = wv.shape[0] // 2
        x_prev = np.concatenate([np.zeros((1, x.shape[1])), x[:-1]], axis=0)
        v = np.concatenate([x @ wv[:half].T, x_prev @ wv[half:].T], axis=1)
    else:
        v = x @ wv.T
    return v.reshape(S, cfg.n_kv_heads, cfg.head_dim)


def _normalise(a: np.ndarray, dh: int, gain: float = 1.0) -> np.ndarray:
    """[CCA page] ``forward`` QK L2-norm: each head vector scaled to length sqrt(d_h)
    (its norm clamped below at 1e-6), times `gain`."""
    n = np.maximum(np.linalg.norm(a, axis=-1, keepdims=True), 1e-6)
    return a * (math.sqrt(dh) / n) * gain


def cca_qk(x: np.ndarray, W: Dict[str, np.ndarray], cfg):
    """[CCA page] ``CCAAttention.forward`` steps 1-3: q, k [S, H, d_h] after the
    convolutions and the q-k-mean, before the normalisation (Hq = Hkv = H)."""
    H, dh = cfg.n_heads, cfg.head_dim
    L = H * dh
    S = x.shape[0]
    P = np.asarray(x, dtype=F64) @ np.asarray(W["w_qk"], dtype=F64).T
    q_pre, k_pre = P[:, :L].reshape(S, H, dh), P[:, L:].reshape(S, H, dh)
    Pc = apply_causal_convs(P, W, cfg, groups=2 * H)
    q, k = Pc[:, :L].reshape(S, H, dh), Pc[:, L:].reshape(S, H, dh)
    if cfg.qk_mean:
        m = 0.5 * (q_pre + k_pre)
        q, k = q + m, k + m
    return q, k


def cca_forward(x: np.ndarray, W: Dict[str, np.ndarray], cfg, scale: Optional[float] = None) -> np.ndarray:
    """[CCA page] ``CCAAttention.forward`` in decoder mode: x [S, E] -> y [S, E].
    `scale` overrides the softmax scale d_h^{-1/2} (the parity pins use it)."""
    if cfg.n_kv_heads != cfg.n_heads:
        raise ValueError("CCA has as many key / value heads as query heads")
    dh = cfg.head_dim
    S = x.shape[0]
    pos = np.arange(S)
    q, k = cca_qk(x, W, cfg)
    v = _values(x, W, cfg)
    q = _normalise(q, dh)
    k = _normalise(k, dh, math.exp(cfg.beta))
    q = _mla.rope_halfsplit(q, pos, cfg.rope_base)
    k = _mla.rope_halfsplit(k, pos, cfg.rope_base)
    o = _mla.causal_attention(q, k, v, dh ** -0.5 if scale is None else scale, pos, pos)
    return o.reshape(S, -1) @ np.asarray(W["w_o"], dtype=F64).T


def ccgqa_qk(x: np.ndarray, W: Dict[str, np.ndarray], cfg):
    """[CCA page] ``CCGQAAttention.forward`` steps 1-3: q [S, Hq, d_h] and k [S, Hkv, d_h]
    after the convolutions (groups: the Hq + Hkv heads) and the grouped q-k-mean."""
    Hq, Hkv, dh = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    gs = Hq // Hkv
    Lq = Hq * dh
    S = x.shape[0]
    P = np.asarray(x, dtype=F64) @ np.asarray(W["w_qk"], dtype=F64).T
    q_pre, k_pre = P[:, :Lq].reshape(S, Hq, dh), P[:, Lq:].reshape(S, Hkv, dh)
    Pc = apply_causal_convs(P, W, cfg, groups=Hq + Hkv)
    q, k = Pc[:, :Lq].reshape(S, Hq, dh), Pc[:, Lq:].reshape(S, Hkv, dh)
    if cfg.qk_mean:
        # each query head pairs with the key head of its group; a key head takes the mean
        # of its group's pairs
        m_q = 0.5 * (q_pre + np.repeat(k_pre, gs, axis=1))
        m_k = m_q.reshape(S, Hkv, gs, dh).mean(axis=2)
        q, k = q + m_q, k + m_k
    return q, k


def ccgqa_forward(x: np.ndarray, W: Dict[str, np.ndarray], cfg, scale: Optional[float] = None) -> np.ndarray:
    """[CCA page] ``CCGQAAttention.forward`` in decoder mode: x [S, E] -> y [S, E];
    query head h attends with key / value head h // (Hq / Hkv)."""
    Hq, Hkv, dh = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    gs = Hq // Hkv
    S = x.shape[0]
    pos = np.arange(S)
    q, k = ccgqa_qk(x, W, cfg)
    v = _values(x, W, cfg)
    k, v = np.repeat(k, gs, axis=1), np.repeat(v, gs, axis=1)
    q = _normalise(q, dh)
    k = _normalise(k, dh, math.exp(cfg.beta))
    q = _mla.rope_halfsplit(q, pos, cfg.rope_base)
    k = _mla.rope_halfsplit(k, pos, cfg.rope_base)
    o = _mla.causal_attention(q, k, v, dh ** -0.5 if scale is None else scale, pos, pos)
    return o.reshape(S, -1) @ np.asarray(W["w_o"], dtype=F64).T


def forward(x: np.ndarray, W: Dict[str, np.ndarray], cfg, scale: Optional[float] = None) -> np.ndarray:
    """The page's layer for a workload: CCA when it has as many key heads as query heads,
    CCGQA otherwise."""
    if cfg.n_kv_heads == cfg.n_heads:
        return cca_forward(x, W, cfg, scale)
    return ccgqa_forward(x, W, cfg, scale)
