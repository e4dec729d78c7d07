"""fp64 CPU oracle for multi-head latent attention (MLA) -- TEST INFRASTRUCTURE.

Only the test suite, the package's smoke() entry and bench.py's CPU-baseline leg
may import this module.  The GPU library never calls it, and it shares no code
with the GPU path: it is a plain, slow, obviously correct numpy-fp64 transcription
of what the pages define, used to check the GPU kernels element by element.

Pages followed (cited by title and section throughout):
  [MLA page]   frankenstein-transformer docs, module ``latent/mla_attn``:
               ``_apply_rope`` and ``MLAAttention.forward`` (latent MLA with RoPE on
               the decompressed queries and keys, half-split pairing).
  [MLRA page]  frankenstein-transformer docs, module ``latent/mlra_attn``:
               ``MLRAAttention.forward`` (latent split into L latent heads with
               per-block up-projections, no RoPE).
  [DSV2 page]  bird-of-paradise/deepseek-mla ``src/mla.py``: ``precompute_freqs_cis``,
               ``apply_rotary_emb`` and ``MultiHeadLatentAttention.forward`` (query
               latent, decoupled RoPE key shared by all heads, latent + RoPE-key cache).
  [gist]       RohanAwhad's ``mla.py`` gist "Multi-Head Latent Attention": shapes of
               the decoupled form at tiny dimensions.

Readings of points the pages leave open (each is also listed with its reason in the
design notes of the repository):
  * The decoupled RoPE key is rotated once at its absolute token position and cached
    after rotation (the gist marks the rotated key as the cached quantity).
  * Per-head attention over sequence positions (the gist's product over heads is a
    shape slip); causal masking keys j <= query i; no dropout, no biases.
  * Softmax scale: decoupled 1/sqrt(d_nope + d_rope) (DSV2 page ``scaler``, gist),
    otherwise 1/sqrt(d_head) (MLA and MLRA pages ``scale``).
  * Weights are [out x in] (torch.nn.Linear layout); MLRA up-projections are L dense
    blocks [sub_out x sub_rank]; query head h uses latent block g = h // (H / L).

Parity pins: every function below is checked by tests/test_oracle.py against facts
that do not come from this file: closed forms (RoPE frequencies and rotations, the
two-key softmax, the first causal row), library routines (torch's
scaled_dot_product_attention and complex multiplication in fp64), exact reductions
(MLA with identity up-projections is multi-head attention; MLRA with L blocks is MLA
with a block-diagonal up-projection), invariants (norm preservation, relative
position, causality, row sums, identical latents) and the gist's printed shapes.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

F64 = np.float64

FAMILY_DECOUPLED = "decoupled"
FAMILY_FULLROPE = "fullrope"
FAMILY_MLRA = "mlra"


# ---------------------------------------------------------------------------
# Rotary position embedding
# ---------------------------------------------------------------------------
def rope_inv_freq(dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_j = base^(-2j/dim), j = 0 .. dim/2-1.

    [MLA page] ``_apply_rope``: inverse frequencies 1/base^(2j/dim);
    [DSV2 page] ``precompute_freqs_cis``: the same frequencies for the rotary dim.
    """
    if dim % 2:
        raise ValueError("rotary dimension must be even")
    j = np.arange(dim // 2, dtype=F64)
    return 1.0 / (float(base) ** (2.0 * j / dim))


def rope_interleaved(v: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate consecutive pairs (v[2j], v[2j+1]) by angle pos * theta_j.

    [DSV2 page] ``apply_rotary_emb``: the last dimension is viewed as complex numbers
    v[2j] + i v[2j+1] and multiplied by exp(i * pos * theta_j).  ``v`` has shape
    [n, ..., dim] and ``pos`` has shape [n] (absolute token positions).
    """
    v = np.asarray(v, dtype=F64)
    dim = v.shape[-1]
    ang = np.asarray(pos, dtype=F64)[:, None] * rope_inv_freq(dim, base)[None, :]
    ang = ang.reshape((ang.shape[0],) + (1,) * (v.ndim - 2) + (dim // 2,))
    c, s = np.cos(ang), np.sin(ang)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def rope_halfsplit(v: np.ndarray, pos: np.ndarray, base: float = 10000.0) -> np.ndarray:
    """Rotate the pairs (v[j], v[j + dim/2]) by angle pos * theta_j.

    [MLA page] ``_apply_rope``: coordinate j of the first half and coordinate j of the
    second half form one plane, rotated by the angle of frequency j.  Written here as the
    complex number z_j = v[j] + i v[j + dim/2] multiplied by the unit phasor
    exp(i pos theta_j); the real parts go back to the first half, the imaginary parts to
    the second.  Shapes as in rope_interleaved.
    """
    v = np.asarray(v, dtype=F64)
    dim = v.shape[-1]
    half = dim // 2
    ang = np.asarray(pos, dtype=F64)[:, None] * rope_inv_freq(dim, base)[None, :]
    ang = ang.reshape((ang.shape[0],) + (1,) * (v.ndim - 2) + (half,))
    z = (v[..., :half] + 1j * v[..., half:]) * np.exp(1j * ang)
    out = np.empty_like(v)
    out[..., :half] = z.real
    out[..., half:] = z.imag
    return out


# ---------------------------------------------------------------------------
# Softmax attention
# ---------------------------------------------------------------------------
def softmax_last(s: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis, with the row maximum subtracted; exp(-inf)=0.

    [DSV2 page] ``forward``: softmax over the key axis of the score matrix.
    """
    s = np.asarray(s, dtype=F64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                     q_pos: np.ndarray, k_pos: np.ndarray) -> np.ndarray:
    """Per-head softmax(scale * q k^T) v with keys restricted to k_pos <= q_pos.

    q [nq, H, dq], k [nk, H, dq], v [nk, H, dv] -> [nq, H, dv].
    [MLA page] ``forward`` (decoder mode: strictly-upper-triangular mask -> -inf);
    [DSV2 page] ``forward`` cached path (query at position p sees keys < p + 1).
    """
    q = np.asarray(q, dtype=F64)
    k = np.asarray(k, dtype=F64)
    v = np.asarray(v, dtype=F64)
    allowed = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]      # [nq, nk]
    out = np.empty((q.shape[0], q.shape[1], v.shape[2]), dtype=F64)
    for h in range(q.shape[1]):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        s = np.where(allowed, s, -np.inf)
        out[:, h, :] = softmax_last(s) @ v[:, h, :]
    return out


# ---------------------------------------------------------------------------
# Dimensions
# ---------------------------------------------------------------------------
class Dims:
    """Plain container for the layer's dimensions (no defaults are invented here)."""

    def __init__(self, family: str, d_model: int, n_heads: int, d_nope: int, d_rope: int,
                 r_kv: int, r_q: int, n_latent_heads: int = 1, rope_base: float = 10000.0,
                 softmax_scale: Optional[float] = None):
        self.family = family
        self.d_model = d_model
        self.n_heads = n_heads
        self.d_nope = d_nope
        self.d_v = d_nope
        self.d_rope = d_rope
        self.r_kv = r_kv
        self.r_q = r_q
        self.n_latent_heads = n_latent_heads
        self.rope_base = rope_base
        self.softmax_scale = softmax_scale

    @classmethod
    def from_cfg(cls, cfg) -> "Dims":
        return cls(cfg.family, cfg.d_model, cfg.n_heads, cfg.d_nope, cfg.d_rope, cfg.r_kv,
                   cfg.r_q, cfg.n_latent_heads, cfg.rope_base)

    def scale(self) -> float:
        if self.softmax_scale is not None:
            return float(self.softmax_scale)
        if self.family == FAMILY_DECOUPLED:
            # [DSV2 page] ``__init__``: scaler = 1/sqrt(d_head + d_rotate); [gist] same.
            return 1.0 / math.sqrt(self.d_nope + self.d_rope)
        # [MLA page] / [MLRA page] ``__init__``: scale = head_dim ** -0.5.
        return 1.0 / math.sqrt(self.d_nope)


def _w(W: Dict[str, np.ndarray], name: str) -> np.ndarray:
    return np.asarray(W[name], dtype=F64)


# ---------------------------------------------------------------------------
# Latent (the only cached quantity) and the explicit keys / values
# ---------------------------------------------------------------------------
def latent_rows(x: np.ndarray, W: Dict[str, np.ndarray], d: Dims, pos: np.ndarray):
    """Cache contents for tokens x [n, d_model] at absolute positions pos [n].

    Returns (c [n, r_kv], k_rope [n, d_rope] or None).
    c = W_DKV x: [MLA page] ``forward`` (dkv_proj), [DSV2 page] ``forward`` (DKV_proj,
    the cached latent).  k_rope = RoPE(W_KR x, pos) with interleaved pairs: [DSV2 page]
    ``forward`` (RK_proj) and ``apply_rotary_emb``; rotated at the absolute position
    and cached after rotation ([gist]: the rotated key is the cached one).
    """
    x = np.asarray(x, dtype=F64)
    c = x @ _w(W, "w_dkv").T
    kr = None
    if d.family == FAMILY_DECOUPLED and d.d_rope > 0:
        kr = rope_interleaved(x @ _w(W, "w_kr").T, pos, d.rope_base)
    return c, kr


def _keys_values(c: np.ndarray, kr: Optional[np.ndarray], W, d: Dims, pos: np.ndarray):
    """Explicit per-head keys [n, H, dq] and values [n, H, dv] from the latent."""
    n, H, dn = c.shape[0], d.n_heads, d.d_nope
    if d.family == FAMILY_MLRA:
        # [MLRA page] ``forward``: c is viewed as L chunks; chunk g goes through its own
        # up-projection; the L outputs are concatenated and reshaped to (H, head_dim).
        L = d.n_latent_heads
        sr = d.r_kv // L
        wuk, wuv = _w(W, "w_uk"), _w(W, "w_uv")
        kp = [c[:, g * sr:(g + 1) * sr] @ wuk[g].T for g in range(L)]
        vp = [c[:, g * sr:(g + 1) * sr] @ wuv[g].T for g in range(L)]
        k = np.concatenate(kp, axis=1).reshape(n, H, dn)
        v = np.concatenate(vp, axis=1).reshape(n, H, dn)
        return k, v
    k = (c @ _w(W, "w_uk").T).reshape(n, H, dn)            # UK_proj / uk_proj
    v = (c @ _w(W, "w_uv").T).reshape(n, H, d.d_v)          # UV_proj / uv_proj
    if d.family == FAMILY_FULLROPE:
        # [MLA page] ``forward``: RoPE on the decompressed keys, positions 0..S-1.
        k = rope_halfsplit(k, pos, d.rope_base)
    elif d.family == FAMILY_DECOUPLED and d.d_rope > 0:
        # [DSV2 page] ``forward``: k_R is shared by all heads (expand over heads) and
        # concatenated after the decompressed key.
        k = np.concatenate([k, np.broadcast_to(kr[:, None, :], (n, H, d.d_rope))], axis=-1)
    return k, v


def _queries(x: np.ndarray, W, d: Dims, pos: np.ndarray) -> np.ndarray:
    """Per-head queries [n, H, dq]."""
    x = np.asarray(x, dtype=F64)
    n, H, dn = x.shape[0], d.n_heads, d.d_nope
    if d.family == FAMILY_DECOUPLED:
        # [DSV2 page] ``forward``: C_Q = DQ_proj(x); Q = UQ_proj(C_Q);
        # Q_rotate = RQ_proj(C_Q), rotated per head; q = [q_C ; q_R].
        if d.r_q > 0:
            cq = x @ _w(W, "w_dq").T
            qc = (cq @ _w(W, "w_uq").T).reshape(n, H, dn)
            src = cq
        else:
            qc = (x @ _w(W, "w_q").T).reshape(n, H, dn)
            src = x
        if d.d_rope > 0:
            qr = (src @ _w(W, "w_qr").T).reshape(n, H, d.d_rope)
            qr = rope_interleaved(qr, pos, d.rope_base)
            return np.concatenate([qc, qr], axis=-1)
        return qc
    q = (x @ _w(W, "w_q").T).reshape(n, H, dn)               # q_proj
    if d.family == FAMILY_FULLROPE:
        q = rope_halfsplit(q, pos, d.rope_base)               # RoPE on the decompressed q
    return q                                                  # MLRA: no RoPE


def _output(o: np.ndarray, W) -> np.ndarray:
    """y = W_O [o_1; ...; o_H]: heads concatenated, then the output projection."""
    return o.reshape(o.shape[0], -1) @ _w(W, "w_o").T


# ---------------------------------------------------------------------------
# Forward passes (explicit K/V up-projection)
# ---------------------------------------------------------------------------
def forward(x: np.ndarray, W: Dict[str, np.ndarray], d: Dims,
            q_rows: Optional[Sequence[int]] = None, start_pos: int = 0) -> np.ndarray:
    """Causal self-attention layer over one sequence, explicit form.

    x [S, d_model] holds the tokens at absolute positions start_pos .. start_pos+S-1;
    returns y [len(q_rows), d_model] for the requested rows (default: all).
    Keys and values are up-projected explicitly from the latent of every token.
    """
    x = np.asarray(x, dtype=F64)
    S = x.shape[0]
    pos = np.arange(start_pos, start_pos + S)
    rows = np.arange(S) if q_rows is None else np.asarray(q_rows, dtype=np.int64)
    c, kr = latent_rows(x, W, d, pos)
    k, v = _keys_values(c, kr, W, d, pos)
    q = _queries(x[rows], W, d, pos[rows])
    o = causal_attention(q, k, v, d.scale(), pos[rows], pos)
    return _output(o, W)


def forward_from_cache(x_new: np.ndarray, c_cache: np.ndarray, kr_cache: Optional[np.ndarray],
                       W: Dict[str, np.ndarray], d: Dims, start_pos: int) -> np.ndarray:
    """Tokens x_new at positions start_pos.. attending over cached latents + their own.

    [DSV2 page] ``forward`` with use_cache: the new latents are written at rows
    start_pos .. start_pos+T-1, the cache is read up to start_pos+T and up-projected
    explicitly; query i sees keys at positions <= start_pos + i.
    """
    x_new = np.asarray(x_new, dtype=F64)
    T = x_new.shape[0]
    pos_new = np.arange(start_pos, start_pos + T)
    c_new, kr_new = latent_rows(x_new, W, d, pos_new)
    c = np.concatenate([np.asarray(c_cache, dtype=F64)[:start_pos], c_new], axis=0)
    kr = None
    if kr_new is not None:
        kr = np.concatenate([np.asarray(kr_cache, dtype=F64)[:start_pos], kr_new], axis=0)
    pos = np.arange(start_pos + T)
    k, v = _keys_values(c, kr, W, d, pos)
    q = _queries(x_new, W, d, pos_new)
    o = causal_attention(q, k, v, d.scale(), pos_new, pos)
    return _output(o, W)


def decode(x_seq: np.ndarray, W: Dict[str, np.ndarray], d: Dims) -> np.ndarray:
    """Output of the last token of x_seq [ctx+1, d_model] (one decode step).

    The new token sits at position ctx and attends to all ctx+1 latents, itself
    included; it equals the last row of the causal forward pass.
    """
    S = np.asarray(x_seq).shape[0]
    return forward(x_seq, W, d, q_rows=[S - 1])[0]


def latent_attention(q_lat: np.ndarray, q_rope: Optional[np.ndarray], lat: np.ndarray,
                     kr: Optional[np.ndarray], scale: float) -> np.ndarray:
    """Attention of one query per head over latent rows, without up-projection.

    q_lat [H, r] and q_rope [H, d_rope] (or None) against latent rows lat [n, r] and
    rotated keys kr [n, d_rope]: s_j = scale (q_lat . lat_j + q_rope . kr_j); returns
    z [H, r] = sum_j softmax_j(s) lat_j.  All n rows are visible (the query is the last
    token, so causality admits every cached row).
    """
    q_lat = np.asarray(q_lat, dtype=F64)
    lat = np.asarray(lat, dtype=F64)
    s = scale * (q_lat @ lat.T)                                # [H, n]
    if q_rope is not None:
        s = s + scale * (np.asarray(q_rope, dtype=F64) @ np.asarray(kr, dtype=F64).T)
    return softmax_last(s) @ lat


def absorbed_decode(x_seq: np.ndarray, W: Dict[str, np.ndarray], d: Dims) -> np.ndarray:
    """The same decode step computed over the latent itself (W_UK folded into the
    query, W_UV applied after the attention-weighted latent sum).

    Not on the pages; it follows from associativity applied to the explicit form:
    q_C . (W_UK,h c) = (W_UK,h^T q_C) . c  and  sum_j p_j W_UV,h c_j = W_UV,h sum_j p_j c_j.
    Only defined where RoPE does not touch the decompressed key (decoupled, MLRA).
    """
    if d.family == FAMILY_FULLROPE:
        raise ValueError("RoPE on the decompressed key does not commute with absorption")
    x_seq = np.asarray(x_seq, dtype=F64)
    S = x_seq.shape[0]
    pos = np.arange(S)
    c, kr = latent_rows(x_seq, W, d, pos)
    q = _queries(x_seq[S - 1:], W, d, pos[S - 1:])[0]        # [H, dq]
    H, dn = d.n_heads, d.d_nope
    o = np.empty((H, d.d_v), dtype=F64)
    for h in range(H):
        wuk, wuv, lat = head_up_projections(W, d, h, c)
        q_lat = (wuk.T @ q[h, :dn])[None]
        q_rope = q[h, dn:][None] if kr is not None else None
        z = latent_attention(q_lat, q_rope, lat, kr, d.scale())[0]
        o[h] = wuv @ z
    return _output(o[None], W)[0]


def head_up_projections(W: Dict[str, np.ndarray], d: Dims, h: int, c: np.ndarray):
    """(W_UK rows of head h [dn, rb], W_UV rows of head h [dv, rb], latent block [n, rb]).

    MLA: rows h*dn .. of the full up-projections and the whole latent.  MLRA: the rows of
    head h inside its block g = h // (H/L) and latent columns g*rb .. (g+1)*rb.
    """
    dn = d.d_nope
    if d.family == FAMILY_MLRA:
        L = d.n_latent_heads
        hpg, sr = d.n_heads // L, d.r_kv // L
        g, hi = h // hpg, h % hpg
        return (_w(W, "w_uk")[g][hi * dn:(hi + 1) * dn], _w(W, "w_uv")[g][hi * dn:(hi + 1) * dn],
                np.asarray(c, dtype=F64)[:, g * sr:(g + 1) * sr])
    return (_w(W, "w_uk")[h * dn:(h + 1) * dn], _w(W, "w_uv")[h * dn:(h + 1) * dn],
            np.asarray(c, dtype=F64))


def queries(x: np.ndarray, W: Dict[str, np.ndarray], d: Dims, pos: np.ndarray) -> np.ndarray:
    """Per-head queries [n, H, d_nope + d_rope] of tokens x at positions pos."""
    return _queries(x, W, d, np.asarray(pos))


def keys_values(c: np.ndarray, kr: Optional[np.ndarray], W: Dict[str, np.ndarray], d: Dims,
                pos: np.ndarray):
    """Explicit per-head keys [n, H, dq] and values [n, H, dv] from latent rows."""
    return _keys_values(np.asarray(c, dtype=F64), None if kr is None else np.asarray(kr, dtype=F64),
                        W, d, np.asarray(pos))


def prefill_batch(xs: Sequence[np.ndarray], W, d: Dims) -> np.ndarray:
    """forward() over a batch of equal-length sequences -> [B, S, d_model]."""
    return np.stack([forward(x, W, d) for x in xs])


__all__ = [
    "rope_inv_freq", "rope_interleaved", "rope_halfsplit", "softmax_last",
    "causal_attention", "Dims", "latent_rows", "forward", "forward_from_cache",
    "decode", "absorbed_decode", "prefill_batch", "latent_attention", "head_up_projections",
    "queries", "keys_values",
    "FAMILY_DECOUPLED", "FAMILY_FULLROPE", "FAMILY_MLRA",
]
