"""fp64 CPU oracle for training the MLA layer: dropout forward and backward -- TEST INFRASTRUCTURE.

Only the test suite and bench.py's CPU-baseline leg may import this module; the GPU library
shares no code with it.

Pages followed (cited by title and section):
  [DSV2 page]  bird-of-paradise/deepseek-mla ``src/mla.py``: ``MultiHeadLatentAttention``
               (``__init__`` takes a dropout probability, default 0.1; ``forward`` applies
               dropout to the attention weights after the softmax and before the product
               with the values).
  [MLA page]   frankenstein-transformer docs, ``latent/mla_attn``: ``MLAAttention`` (the same
               dropout on the attention weights of a trainable module).
The layer is the decoupled-RoPE family of mla_oracle (query latent, rotary key shared by
the heads); its forward is mla_oracle.forward with the attention weights P replaced by
P * keep / (1 - p).

Dropout draws come from SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used as a counter-based generator.  One 64-bit draw
serves four consecutive keys, 16 bits each: for attention weight (sequence b, head h,
query i, key j)
    n = (b H + h) 2^38 + i 2^18 + floor(j / 4)
    r = mix64(seed + (n + 1) gamma)            (the (n+1)-th output of SplitMix64 from state seed)
    u = bits 16 (j mod 4) .. 16 (j mod 4) + 15 of r
    keep  <=>  u >= floor(p 2^16)
with gamma = 0x9E3779B97F4A7C15 and mix64 the generator's output function, so any group
of four keys can be drawn on its own, in any order, on either side.  (The pages name no
generator; the keep probability is 1 - floor(p 2^16) / 2^16, within 2^-16 of 1 - p.)

The backward is the chain rule through that forward, written out step by step (reverse
order of the forward).  With o = Pd v and Pd = P keep / (1 - p):
    dPd = do v^T,  dv = Pd^T do,  dP = dPd keep / (1 - p),
    ds = P (dP - rowsum(P dP)),  dq = tau ds k,  dk = tau ds^T q
and rowsum(P dP) = rowsum(do o) (the dropout factors cancel).  The rotations are orthogonal,
so their backward is the rotation by the negative angle.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import mla_oracle as O

F64 = np.float64
U64 = np.uint64
SM_GAMMA = U64(0x9E3779B97F4A7C15)                               # state increment
SM_MUL = (U64(0xBF58476D1CE4E5B9), U64(0x94D049BB133111EB))      # output-function multipliers


def splitmix64(state, n):
    """Output n + 1 of SplitMix64 started at `state` (arrays broadcast): the state advanced
    n + 1 times by gamma, then the output function: two xor-shift-multiply steps and a final
    xor-shift, all modulo 2^64."""
    with np.errstate(over="ignore"):
        z = np.asarray(state, dtype=U64) + (np.asarray(n, dtype=U64) + U64(1)) * SM_GAMMA
        z = (z ^ (z >> U64(30))) * SM_MUL[0]
        z = (z ^ (z >> U64(27))) * SM_MUL[1]
        return z ^ (z >> U64(31))


def element_counter(b: int, H: int, h: int, i, j):
    """Counter of the draw of attention weight (b, h, i, j): (b H + h) 2^38 + i 2^18 + j // 4
    (S <= 2^20, B H <= 2^24)."""
    return ((U64(b * H + h) << U64(38)) + (np.asarray(i, dtype=U64) << U64(18))
            + (np.asarray(j, dtype=U64) >> U64(2)))


def keep_threshold(p: float) -> int:
    """A weight is kept when its 16-bit field of the draw is >= floor(p 2^16)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(p * 65536.0))


def dropout_keep(seed: int, b: int, H: int, h: int, n_q: int, n_k: int, p: float) -> np.ndarray:
    """Keep mask [n_q, n_k] of head h of sequence b (queries 0..n_q-1, keys 0..n_k-1)."""
    if keep_threshold(p) == 0:
        return np.ones((n_q, n_k), dtype=bool)          # every draw passes a zero threshold
    i, j = np.arange(n_q)[:, None], np.arange(n_k)[None, :]
    r = splitmix64(U64(seed), element_counter(b, H, h, i, j))
    field = (r >> (U64(16) * (np.asarray(j, dtype=U64) & U64(3)))) & U64(0xFFFF)
    return field >= U64(keep_threshold(p))


def _check_family(d: O.Dims):
    if d.family != O.FAMILY_DECOUPLED or d.r_q <= 0 or d.d_rope <= 0:
        raise ValueError("training oracle: decoupled-RoPE family with a query latent")


def train_forward(x: np.ndarray, W: Dict[str, np.ndarray], d: O.Dims, p: float, seed: int, b: int):
    """[DSV2 page] ``MultiHeadLatentAttention.forward`` with dropout p on the attention weights,
    for sequence b of the batch (its index enters the dropout counter).  Returns (y, saved)."""
    _check_family(d)
    x = np.asarray(x, dtype=F64)
    S, H, dn, dr = x.shape[0], d.n_heads, d.d_nope, d.d_rope
    pos = np.arange(S)
    Wf = {k: np.asarray(v, dtype=F64) for k, v in W.items()}
    cq = x @ Wf["w_dq"].T
    q_c = (cq @ Wf["w_uq"].T).reshape(S, H, dn)
    q_r = O.rope_interleaved((cq @ Wf["w_qr"].T).reshape(S, H, dr), pos, d.rope_base)
    c = x @ Wf["w_dkv"].T
    k_r = O.rope_interleaved(x @ Wf["w_kr"].T, pos, d.rope_base)
    k_c = (c @ Wf["w_uk"].T).reshape(S, H, dn)
    v = (c @ Wf["w_uv"].T).reshape(S, H, dn)
    q = np.concatenate([q_c, q_r], axis=-1)
    k = np.concatenate([k_c, np.broadcast_to(k_r[:, None, :], (S, H, dr))], axis=-1)
    o = np.zeros((S, H, dn))
    for h in range(H):
        P, keep = _weights_of_head(q, k, d, p, seed, b, h)
        o[:, h] = (P * keep / (1.0 - p)) @ v[:, h]
    y = o.reshape(S, H * dn) @ Wf["w_o"].T
    saved = dict(x=x, cq=cq, c=c, q=q, k=k, v=v, o=o, pos=pos, seed=seed, b=b)
    return y, saved


def _weights_of_head(q, k, d: O.Dims, p: float, seed: int, b: int, h: int):
    """Causal softmax weights P [S, S] of head h and their dropout keep mask."""
    S, H = q.shape[0], q.shape[1]
    pos = np.arange(S)
    s = np.where(pos[None, :] <= pos[:, None], d.scale() * (q[:, h] @ k[:, h].T), -np.inf)
    return O.softmax_last(s), dropout_keep(seed, b, H, h, S, S, p)


def train_backward(dy: np.ndarray, W: Dict[str, np.ndarray], d: O.Dims, p: float, saved) -> Dict[str, np.ndarray]:
    """Gradients of sum(dy * y) for the forward above: dx and one entry per weight."""
    Wf = {k: np.asarray(v, dtype=F64) for k, v in W.items()}
    dy = np.asarray(dy, dtype=F64)
    x, cq, c, q, k, v, o, pos = (saved[n] for n in ("x", "cq", "c", "q", "k", "v", "o", "pos"))
    S, H, dn, dr = x.shape[0], d.n_heads, d.d_nope, d.d_rope
    tau = d.scale()
    g: Dict[str, np.ndarray] = {}
    # output projection y = o_cat W_o^T
    o_cat = o.reshape(S, H * dn)
    g["w_o"] = dy.T @ o_cat
    do = (dy @ Wf["w_o"]).reshape(S, H, dn)
    # attention, head by head
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(H):
        P, keep = _weights_of_head(q, k, d, p, saved["seed"], saved["b"], h)   # recomputed per head
        Pd = P * keep / (1.0 - p)
        dPd = do[:, h] @ v[:, h].T
        dv[:, h] = Pd.T @ do[:, h]
        dP = dPd * keep / (1.0 - p)
        ds = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
        dq[:, h] = tau * (ds @ k[:, h])
        dk[:, h] = tau * (ds.T @ q[:, h])
    # split of q and k into their decompressed and rotary parts
    dq_c, dq_r = dq[..., :dn], dq[..., dn:]
    dk_c, dk_r = dk[..., :dn], dk[..., dn:].sum(axis=1)       # k_R is shared by the heads
    dq_r0 = O.rope_interleaved(dq_r, -pos, d.rope_base)        # rotation by the negative angle
    dk_r0 = O.rope_interleaved(dk_r, -pos, d.rope_base)
    dq_c, dq_r0 = dq_c.reshape(S, H * dn), dq_r0.reshape(S, H * dr)
    dk_c, dv = dk_c.reshape(S, H * dn), dv.reshape(S, H * dn)
    # query path
    g["w_uq"] = dq_c.T @ cq
    g["w_qr"] = dq_r0.T @ cq
    dcq = dq_c @ Wf["w_uq"] + dq_r0 @ Wf["w_qr"]
    g["w_dq"] = dcq.T @ x
    # key / value path
    g["w_uk"] = dk_c.T @ c
    g["w_uv"] = dv.T @ c
    dc = dk_c @ Wf["w_uk"] + dv @ Wf["w_uv"]
    g["w_dkv"] = dc.T @ x
    g["w_kr"] = dk_r0.T @ x
    g["x"] = dcq @ Wf["w_dq"] + dc @ Wf["w_dkv"] + dk_r0 @ Wf["w_kr"]
    return g


def lse_log2(saved, d: O.Dims) -> np.ndarray:
    """log2 of each softmax row's normaliser sum_j exp(s_ij) (scores in natural units), [H, S]:
    the per-row statistic a flash forward keeps for its backward."""
    q, k, pos = saved["q"], saved["k"], saved["pos"]
    S, H = q.shape[0], q.shape[1]
    out = np.zeros((H, S))
    causal = pos[None, :] <= pos[:, None]
    for h in range(H):
        s = np.where(causal, d.scale() * (q[:, h] @ k[:, h].T), -np.inf)
        m = s.max(axis=1)
        out[h] = (m + np.log(np.exp(s - m[:, None]).sum(axis=1))) / np.log(2.0)
    return out
