"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the page passage or the mathematical fact it relies on.  Library
routines used as independent references: torch's scaled_dot_product_attention,
torch.nn.MultiheadAttention and complex multiplication (all in fp64 on the CPU).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import mla_synth as S
from oracle import mla_oracle as O

torch.set_default_dtype(torch.float64)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_weights(dims: O.Dims, seed=0, scale=0.5):
    cfg = S.MLAConfig("t", dims.family, "prefill", 1, 1, dims.d_model, dims.n_heads,
                      dims.d_nope, dims.d_rope, dims.r_kv, dims.r_q, dims.n_latent_heads,
                      dtype="f32")
    r = _rng(seed)
    return {k: r.standard_normal(s) * scale for k, s in cfg.weight_shapes().items()}


# ---------------------------------------------------------------------------
# RoPE: closed forms ([MLA page] _apply_rope; [DSV2 page] precompute_freqs_cis,
# apply_rotary_emb) and the rotation's algebraic properties
# ---------------------------------------------------------------------------
def test_inv_freq_closed_form():
    np.testing.assert_allclose(O.rope_inv_freq(4, 10000.0), [1.0, 0.01], rtol=1e-15)
    th = O.rope_inv_freq(64, 10000.0)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[1], 10000.0 ** (-2 / 64), rtol=1e-15)
    np.testing.assert_allclose(th[31], 10000.0 ** (-62 / 64), rtol=1e-14)
    with pytest.raises(ValueError):
        O.rope_inv_freq(5)


@pytest.mark.parametrize("t", [0, 1, 3, 7, 4096])
def test_rope_unit_vectors_closed_form(t):
    e = np.eye(4)[None]                      # four unit vectors at one position
    a, b = float(t), 0.01 * t
    got = O.rope_interleaved(e, np.array([t]))[0]
    want = np.array([[math.cos(a), math.sin(a), 0, 0],
                     [-math.sin(a), math.cos(a), 0, 0],
                     [0, 0, math.cos(b), math.sin(b)],
                     [0, 0, -math.sin(b), math.cos(b)]])
    np.testing.assert_allclose(got, want, atol=1e-12)
    got = O.rope_halfsplit(e, np.array([t]))[0]
    want = np.array([[math.cos(a), 0, math.sin(a), 0],
                     [0, math.cos(b), 0, math.sin(b)],
                     [-math.sin(a), 0, math.cos(a), 0],
                     [0, -math.sin(b), 0, math.cos(b)]])
    np.testing.assert_allclose(got, want, atol=1e-12)


def _torch_rope_complex(v, pos, base, pairing):
    """Rotation as complex multiplication by exp(i pos theta) (independent route)."""
    v = torch.as_tensor(v)
    dim = v.shape[-1]
    theta = base ** (-torch.arange(0, dim, 2, dtype=torch.float64) / dim)
    ang = torch.as_tensor(pos, dtype=torch.float64)[:, None] * theta[None, :]
    ang = ang.reshape((ang.shape[0],) + (1,) * (v.dim() - 2) + (dim // 2,))
    rot = torch.polar(torch.ones_like(ang), ang)
    if pairing == "interleaved":
        z = torch.view_as_complex(v.reshape(*v.shape[:-1], dim // 2, 2).contiguous())
        return torch.view_as_real(z * rot).flatten(-2)
    z = torch.complex(v[..., : dim // 2], v[..., dim // 2:])
    w = z * rot
    return torch.cat([w.real, w.imag], dim=-1)


@pytest.mark.parametrize("pairing", ["interleaved", "halfsplit"])
def test_rope_matches_complex_multiplication(pairing):
    v = _rng(1).standard_normal((7, 3, 64))
    pos = np.array([0, 1, 2, 100, 2047, 4095, 16384])
    f = O.rope_interleaved if pairing == "interleaved" else O.rope_halfsplit
    got = f(v, pos, 10000.0)
    want = _torch_rope_complex(v, pos, 10000.0, pairing).numpy()
    np.testing.assert_allclose(got, want, atol=1e-12)


@pytest.mark.parametrize("f", [O.rope_interleaved, O.rope_halfsplit])
def test_rope_identity_norm_and_relative_position(f):
    r = _rng(2)
    q, k = r.standard_normal((1, 64)), r.standard_normal((1, 64))
    np.testing.assert_array_equal(f(q, np.array([0])), q)
    for p in [1, 17, 4096]:
        np.testing.assert_allclose(np.linalg.norm(f(q, np.array([p]))), np.linalg.norm(q), rtol=1e-13)
    for m, n, delta in [(5, 2, 100), (0, 9, 7), (4096, 1, 3000)]:
        d0 = (f(q, np.array([m])) @ f(k, np.array([n])).T).item()
        d1 = (f(q, np.array([m + delta])) @ f(k, np.array([n + delta])).T).item()
        d2 = (q @ f(k, np.array([n - m])).T).item()
        assert abs(d0 - d1) < 1e-10 and abs(d0 - d2) < 1e-10


def test_halfsplit_is_a_permuted_interleaved_rotation():
    v = _rng(3).standard_normal((5, 2, 16))
    pos = np.arange(5) * 11
    perm = np.stack([np.arange(8), np.arange(8) + 8], axis=1).reshape(-1)  # half -> pairs
    inv = np.argsort(perm)
    got = O.rope_interleaved(v[..., perm], pos)[..., inv]
    np.testing.assert_allclose(got, O.rope_halfsplit(v, pos), atol=1e-13)


# ---------------------------------------------------------------------------
# Softmax ([DSV2 page] forward: softmax over keys)
# ---------------------------------------------------------------------------
def test_softmax_closed_form_and_invariants():
    a, b = 0.3, -1.7
    np.testing.assert_allclose(O.softmax_last(np.array([a, b])),
                               [1 / (1 + math.exp(b - a)), 1 / (1 + math.exp(a - b))], rtol=1e-15)
    s = _rng(4).standard_normal((6, 9)) * 30
    p = O.softmax_last(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(O.softmax_last(s + 123.0), p, rtol=1e-12)
    p = O.softmax_last(np.array([0.5, -np.inf, 1.0]))
    assert p[1] == 0.0 and abs(p.sum() - 1) < 1e-15


# ---------------------------------------------------------------------------
# Attention core vs torch's scaled_dot_product_attention (fp64 CPU)
# ---------------------------------------------------------------------------
def test_causal_attention_matches_sdpa():
    r = _rng(5)
    n, H, dq, dv = 9, 3, 5, 4
    q, k, v = r.standard_normal((n, H, dq)), r.standard_normal((n, H, dq)), r.standard_normal((n, H, dv))
    pos = np.arange(n)
    got = O.causal_attention(q, k, v, 0.37, pos, pos)
    t = lambda a: torch.as_tensor(a).transpose(0, 1)[None]
    want = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True, scale=0.37)
    np.testing.assert_allclose(got, want[0].transpose(0, 1).numpy(), atol=1e-13)
    # queries at positions 5..8 over keys 0..8 (a continued chunk): explicit mask
    got = O.causal_attention(q[5:], k, v, 0.37, pos[5:], pos)
    mask = torch.as_tensor(pos[None, :] <= pos[5:, None])
    want = F.scaled_dot_product_attention(t(q[5:]), t(k), t(v), attn_mask=mask, scale=0.37)
    np.testing.assert_allclose(got, want[0].transpose(0, 1).numpy(), atol=1e-13)
    # rows sum to one: with all-ones values every output is exactly one
    ones = O.causal_attention(q, k, np.ones((n, H, 2)), 0.37, pos, pos)
    np.testing.assert_allclose(ones, 1.0, rtol=1e-14)


# ---------------------------------------------------------------------------
# Whole layers against independent library compositions
# ---------------------------------------------------------------------------
def _mha_reference(x, wq, wk, wv, wo, H):
    """Textbook causal multi-head attention through torch.nn.MultiheadAttention."""
    dm = wq.shape[1]
    m = torch.nn.MultiheadAttention(dm, H, bias=False, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.cat([torch.as_tensor(wq), torch.as_tensor(wk), torch.as_tensor(wv)]))
        m.out_proj.weight.copy_(torch.as_tensor(wo))
    S_ = x.shape[0]
    mask = torch.triu(torch.ones(S_, S_, dtype=torch.bool), diagonal=1)
    y, _ = m(*(torch.as_tensor(x)[None],) * 3, attn_mask=mask, need_weights=False)
    return y[0].detach().numpy()


def test_mla_with_identity_upprojections_is_mha():
    """r_kv = 2*H*d with W_DKV = [W_K; W_V], W_UK = [I 0], W_UV = [0 I] is exactly MHA."""
    H, d, dm, Sq = 3, 4, 12, 10
    r = _rng(6)
    wq, wk, wv, wo = (r.standard_normal((dm, dm)) * 0.4 for _ in range(4))
    dims = O.Dims(O.FAMILY_DECOUPLED, dm, H, d, 0, 2 * H * d, 0)
    eye, zero = np.eye(H * d), np.zeros((H * d, H * d))
    W = {"w_q": wq, "w_dkv": np.concatenate([wk, wv]), "w_uk": np.concatenate([eye, zero], 1),
         "w_uv": np.concatenate([zero, eye], 1), "w_o": wo}
    x = r.standard_normal((Sq, dm))
    np.testing.assert_allclose(O.forward(x, W, dims), _mha_reference(x, wq, wk, wv, wo, H), atol=1e-12)


def test_mla_without_rope_is_mha_with_product_weights():
    """No RoPE: keys W_UK W_DKV x, queries W_UQ W_DQ x -> MHA with product weights."""
    H, d, dm, Sq = 2, 6, 12, 7
    dims = O.Dims(O.FAMILY_DECOUPLED, dm, H, d, 0, 5, 4)
    W = _rand_weights(dims, seed=7)
    x = _rng(8).standard_normal((Sq, dm))
    want = _mha_reference(x, W["w_uq"] @ W["w_dq"], W["w_uk"] @ W["w_dkv"], W["w_uv"] @ W["w_dkv"],
                          W["w_o"], H)
    np.testing.assert_allclose(O.forward(x, W, dims), want, atol=1e-12)


def test_mlra_is_mha_with_blockdiagonal_products():
    """[MLRA page] forward: chunk g of the latent feeds block g of the heads."""
    import scipy.linalg
    H, d, L, r_, dm, Sq = 4, 3, 2, 6, 12, 9
    dims = O.Dims(O.FAMILY_MLRA, dm, H, d, 0, r_, 0, n_latent_heads=L)
    W = _rand_weights(dims, seed=9)
    uk = scipy.linalg.block_diag(*W["w_uk"])            # [H*d, r]
    uv = scipy.linalg.block_diag(*W["w_uv"])
    x = _rng(10).standard_normal((Sq, dm))
    want = _mha_reference(x, W["w_q"], uk @ W["w_dkv"], uv @ W["w_dkv"], W["w_o"], H)
    np.testing.assert_allclose(O.forward(x, W, dims), want, atol=1e-12)
    # L = 1 is plain MLA with W_Q
    dims1 = O.Dims(O.FAMILY_MLRA, dm, H, d, 0, r_, 0, n_latent_heads=1)
    W1 = dict(W, w_uk=uk[None], w_uv=uv[None])
    dimsd = O.Dims(O.FAMILY_DECOUPLED, dm, H, d, 0, r_, 0)
    Wd = dict(W, w_uk=uk, w_uv=uv)
    np.testing.assert_allclose(O.forward(x, W1, dims1), O.forward(x, Wd, dimsd), atol=1e-13)
    np.testing.assert_allclose(O.forward(x, W, dims), O.forward(x, Wd, dimsd), atol=1e-13)


def _torch_decoupled(x, W, dims, start=0):
    """Decoupled MLA composed from torch primitives (linear, complex RoPE, SDPA)."""
    t = lambda a: torch.as_tensor(a)
    x = t(x)
    n, H, dn, dr = x.shape[0], dims.n_heads, dims.d_nope, dims.d_rope
    pos = np.arange(start, start + n)
    cq = F.linear(x, t(W["w_dq"]))
    qc = F.linear(cq, t(W["w_uq"])).view(n, H, dn)
    qr = _torch_rope_complex(F.linear(cq, t(W["w_qr"])).view(n, H, dr), pos, dims.rope_base, "interleaved")
    c = F.linear(x, t(W["w_dkv"]))
    kr = _torch_rope_complex(F.linear(x, t(W["w_kr"])), pos, dims.rope_base, "interleaved")
    kc = F.linear(c, t(W["w_uk"])).view(n, H, dn)
    v = F.linear(c, t(W["w_uv"])).view(n, H, dn)
    q = torch.cat([qc, qr], -1).transpose(0, 1)
    k = torch.cat([kc, kr[:, None, :].expand(n, H, dr)], -1).transpose(0, 1)
    o = F.scaled_dot_product_attention(q, k, v.transpose(0, 1), is_causal=True,
                                       scale=1 / math.sqrt(dn + dr))
    return F.linear(o.transpose(0, 1).reshape(n, H * dn), t(W["w_o"])).numpy()


def test_decoupled_matches_torch_composition():
    dims = O.Dims(O.FAMILY_DECOUPLED, 10, 3, 6, 4, 5, 7)
    W = _rand_weights(dims, seed=11)
    x = _rng(12).standard_normal((11, 10))
    np.testing.assert_allclose(O.forward(x, W, dims), _torch_decoupled(x, W, dims), atol=1e-12)
    # the rotary part matters: dropping the rotated key changes the output
    W0 = dict(W, w_kr=np.zeros_like(W["w_kr"]))
    assert np.max(np.abs(O.forward(x, W0, dims) - O.forward(x, W, dims))) > 1e-3


def test_fullrope_matches_torch_composition():
    H, d, dm, r_, n = 2, 8, 16, 6, 9
    dims = O.Dims(O.FAMILY_FULLROPE, dm, H, d, 0, r_, 0)
    W = _rand_weights(dims, seed=13)
    x = _rng(14).standard_normal((n, dm))
    t = lambda a: torch.as_tensor(a)
    pos = np.arange(n)
    q = _torch_rope_complex(F.linear(t(x), t(W["w_q"])).view(n, H, d), pos, 10000.0, "halfsplit")
    c = F.linear(t(x), t(W["w_dkv"]))
    k = _torch_rope_complex(F.linear(c, t(W["w_uk"])).view(n, H, d), pos, 10000.0, "halfsplit")
    v = F.linear(c, t(W["w_uv"])).view(n, H, d)
    o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1),
                                       is_causal=True, scale=d ** -0.5)
    want = F.linear(o.transpose(0, 1).reshape(n, H * d), t(W["w_o"])).numpy()
    np.testing.assert_allclose(O.forward(x, W, dims), want, atol=1e-12)


# ---------------------------------------------------------------------------
# Invariants of the method
# ---------------------------------------------------------------------------
FAMILY_DIMS = [
    O.Dims(O.FAMILY_DECOUPLED, 8, 4, 8, 4, 2, 2),                     # the gist's tiny dims
    O.Dims(O.FAMILY_DECOUPLED, 12, 2, 6, 4, 5, 0),                    # direct W_Q, W_QR on x
    O.Dims(O.FAMILY_FULLROPE, 16, 2, 8, 0, 6, 0),
    O.Dims(O.FAMILY_MLRA, 12, 4, 3, 0, 8, 0, n_latent_heads=2),
]


@pytest.mark.parametrize("dims", FAMILY_DIMS, ids=lambda d: d.family + str(d.r_q))
def test_relative_position_shift_invariance(dims):
    """Scores depend on position differences only: shifting every position is a no-op."""
    W = _rand_weights(dims, seed=15)
    x = _rng(16).standard_normal((8, dims.d_model))
    np.testing.assert_allclose(O.forward(x, W, dims, start_pos=1000), O.forward(x, W, dims), atol=1e-11)


@pytest.mark.parametrize("dims", FAMILY_DIMS, ids=lambda d: d.family + str(d.r_q))
def test_causality(dims):
    W = _rand_weights(dims, seed=17)
    x = _rng(18).standard_normal((10, dims.d_model))
    y = O.forward(x, W, dims)
    x2 = x.copy()
    x2[6:] += _rng(19).standard_normal(x2[6:].shape) * 5
    y2 = O.forward(x2, W, dims)
    np.testing.assert_array_equal(y2[:6], y[:6])
    assert np.max(np.abs(y2[6:] - y[6:])) > 1e-3


def _value_only_output(c_row, W, dims):
    """W_O [W_UV,h c]_h: the output when every attention row puts all weight on
    latents equal to c_row."""
    H, dn = dims.n_heads, dims.d_nope
    if dims.family == O.FAMILY_MLRA:
        L = dims.n_latent_heads
        sr = dims.r_kv // L
        o = np.concatenate([W["w_uv"][g] @ c_row[g * sr:(g + 1) * sr] for g in range(L)])
    else:
        o = W["w_uv"] @ c_row
    return W["w_o"] @ o


@pytest.mark.parametrize("dims", FAMILY_DIMS, ids=lambda d: d.family + str(d.r_q))
def test_first_row_and_identical_latents_closed_form(dims):
    W = _rand_weights(dims, seed=20)
    x = _rng(21).standard_normal((7, dims.d_model))
    c0 = x[0] @ W["w_dkv"].T
    # causal row 0 sees only itself: y_0 = W_O [W_UV,h c_0]_h whatever the queries
    np.testing.assert_allclose(O.forward(x, W, dims)[0], _value_only_output(c0, W, dims), atol=1e-12)
    # identical tokens -> identical latents and values -> every row has the same closed form
    xs = np.repeat(x[:1], 7, axis=0)
    y = O.forward(xs, W, dims)
    np.testing.assert_allclose(y, np.broadcast_to(_value_only_output(c0, W, dims), y.shape), atol=1e-12)


@pytest.mark.parametrize("dims", [d for d in FAMILY_DIMS if d.family != O.FAMILY_FULLROPE],
                         ids=lambda d: d.family + str(d.r_q))
def test_absorbed_equals_explicit(dims):
    W = _rand_weights(dims, seed=22)
    x = _rng(23).standard_normal((9, dims.d_model))
    np.testing.assert_allclose(O.absorbed_decode(x, W, dims), O.decode(x, W, dims), atol=1e-12)


def test_absorbed_rejects_fullrope():
    with pytest.raises(ValueError):
        O.absorbed_decode(np.zeros((2, 16)), {}, FAMILY_DIMS[2])


@pytest.mark.parametrize("dims", FAMILY_DIMS, ids=lambda d: d.family + str(d.r_q))
def test_decode_and_cached_chunks_equal_prefill_rows(dims):
    W = _rand_weights(dims, seed=24)
    x = _rng(25).standard_normal((9, dims.d_model))
    y = O.forward(x, W, dims)
    for t in range(9):
        np.testing.assert_allclose(O.decode(x[:t + 1], W, dims), y[t], atol=1e-12)
    c, kr = O.latent_rows(x, W, dims, np.arange(9))
    for start in [1, 4, 8]:
        got = O.forward_from_cache(x[start:], c, kr, W, dims, start)
        np.testing.assert_allclose(got, y[start:], atol=1e-12)


def test_cache_rows_are_rotated_at_absolute_positions():
    dims = FAMILY_DIMS[0]
    W = _rand_weights(dims, seed=26)
    x = _rng(27).standard_normal((5, 8))
    pos = np.array([0, 3, 4, 100, 4095])
    c, kr = O.latent_rows(x, W, dims, pos)
    np.testing.assert_allclose(c, x @ W["w_dkv"].T, atol=1e-14)
    want = _torch_rope_complex(x @ W["w_kr"].T, pos, 10000.0, "interleaved").numpy()
    np.testing.assert_allclose(kr, want, atol=1e-12)


def test_two_token_closed_form():
    """Row 1 of a 2-token sequence: logistic weights over the two values."""
    dims = O.Dims(O.FAMILY_DECOUPLED, 3, 1, 2, 0, 2, 0)
    W = {"w_q": np.array([[1.0, 0, 0], [0, 1, 0]]), "w_dkv": np.array([[1.0, 0, 0], [0, 0, 1]]),
         "w_uk": np.eye(2), "w_uv": np.array([[2.0, 0], [0, -1]]), "w_o": np.array([[1.0, 0], [0, 1], [1, 1]])}
    x = np.array([[1.0, 2.0, 3.0], [0.5, -1.0, 2.0]])
    tau = 1 / math.sqrt(2)
    # q1 = (0.5, -1); k0 = (1, 3); k1 = (0.5, 2); s0 = tau*(-2.5), s1 = tau*(-1.75)
    p1 = 1 / (1 + math.exp(tau * (-2.5) - tau * (-1.75)))
    v0, v1 = np.array([2.0, -3.0]), np.array([1.0, -2.0])
    o = (1 - p1) * v0 + p1 * v1
    np.testing.assert_allclose(O.forward(x, W, dims)[1], [o[0], o[1], o[0] + o[1]], rtol=1e-14)


def test_scalar_loop_brute_force():
    """Independent pure-Python loops (no numpy linear algebra) on the gist's dims."""
    dims = FAMILY_DIMS[0]
    W = _rand_weights(dims, seed=28)
    x = _rng(29).standard_normal((5, 8))
    H, dn, dr, r_, rq, dm = 4, 8, 4, 2, 2, 8

    def mv(w, v):
        return [sum(w[i][j] * v[j] for j in range(len(v))) for i in range(len(w))]

    def rot(v, p):
        out = list(v)
        for j in range(len(v) // 2):
            a = p * 10000.0 ** (-2.0 * j / len(v))
            out[2 * j] = v[2 * j] * math.cos(a) - v[2 * j + 1] * math.sin(a)
            out[2 * j + 1] = v[2 * j] * math.sin(a) + v[2 * j + 1] * math.cos(a)
        return out

    Wl = {k: v.tolist() for k, v in W.items()}
    xs = x.tolist()
    lat = [mv(Wl["w_dkv"], xs[t]) for t in range(5)]
    kr = [rot(mv(Wl["w_kr"], xs[t]), t) for t in range(5)]
    kall = [mv(Wl["w_uk"], lat[t]) for t in range(5)]
    vall = [mv(Wl["w_uv"], lat[t]) for t in range(5)]
    y = []
    for i in range(5):
        cq = mv(Wl["w_dq"], xs[i])
        qc = mv(Wl["w_uq"], cq)
        qr = mv(Wl["w_qr"], cq)
        o = []
        for h in range(H):
            qh = qc[h * dn:(h + 1) * dn] + rot(qr[h * dr:(h + 1) * dr], i)
            sc = []
            for j in range(i + 1):
                kh = kall[j][h * dn:(h + 1) * dn] + kr[j]
                sc.append(sum(a * b for a, b in zip(qh, kh)) / math.sqrt(dn + dr))
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            o += [sum(e[j] / z * vall[j][h * dn + dd] for j in range(i + 1)) for dd in range(dn)]
        y.append(mv(Wl["w_o"], o))
    np.testing.assert_allclose(O.forward(x, W, dims), np.array(y), atol=1e-12)


def test_gist_shapes_golden():
    shapes = {}
    with open(os.path.join(GOLDEN, "gist_tiny_shapes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split(":")
            shapes[k.strip()] = tuple(int(s) for s in v.split(","))
    cfg = S.CONFIGS["tiny_fp32"]
    B, Sq = cfg.batch, cfg.seq
    ws = cfg.weight_shapes()
    gist_name = {"w_dq": "w_dq", "w_uq": "w_uq", "w_qr": "w_rq", "w_dkv": "w_dkv", "w_uk": "w_uk",
                 "w_kr": "w_rk", "w_uv": "w_uv", "w_o": "w_out"}
    for ours, theirs in gist_name.items():
        assert ws[ours] == shapes[theirs][::-1], ours
    prob = S.make_problem(cfg)
    dims = O.Dims.from_cfg(cfg)
    x = np.stack([prob.x(b, Sq) for b in range(B)])
    assert x.shape == shapes["x"]
    pos = np.arange(Sq)
    q = np.stack([O._queries(x[b], prob.weights, dims, pos) for b in range(B)])
    assert q.shape == shapes["q"]
    lat = [O.latent_rows(x[b], prob.weights, dims, pos) for b in range(B)]
    assert np.stack([c for c, _ in lat]).shape == shapes["dkvc"]
    kv = [O._keys_values(c, kr, prob.weights, dims, pos) for c, kr in lat]
    assert np.stack([k for k, _ in kv]).shape == shapes["k"]
    assert np.stack([v for _, v in kv]).shape == shapes["v"]
    y = O.prefill_batch(list(x), prob.weights, dims)
    assert y.shape == shapes["out"]


# ---------------------------------------------------------------------------
# The seeded input module
# ---------------------------------------------------------------------------
def test_round_bf16_matches_torch_conversion():
    r = _rng(30)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 65504.0, 1e-30], np.float32)])
    want = torch.as_tensor(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(S.round_bf16(a), want)
    bits = S.bf16_bits(S.round_bf16(a))
    np.testing.assert_array_equal(bits, torch.as_tensor(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_synthetic_inputs_are_seeded_and_scaled():
    cfg = S.CONFIGS["small_lm"]
    p1, p2 = S.make_problem(cfg), S.make_problem(cfg)
    for k in p1.weights:
        np.testing.assert_array_equal(p1.weights[k], p2.weights[k])
        fan_in = p1.weights[k].shape[-1]
        assert abs(p1.weights[k].std() * math.sqrt(fan_in) - 1) < 0.02
    x = S.make_x(cfg, 3, 64)
    np.testing.assert_array_equal(S.make_x(cfg, 3, 16), x[:16])     # prefix-stable
    np.testing.assert_array_equal(S.round_bf16(x), x)                # bf16-representable
    m = S.make_problem(S.CONFIGS["mlra_decode"])
    assert m.ctx_lens.min() >= 512 and m.ctx_lens.max() <= 16384 and len(m.ctx_lens) == 128
    assert m.weights["w_uk"].shape == (4, 512, 128)


def test_activations_are_independent_of_the_weights():
    """No sequence's activation stream may replay the weight stream (numpy's SeedSequence
    zero-pads its entropy, so a key [seed, 0] would equal [seed])."""
    cfg = S.CONFIGS["mlra_decode"].replace(dtype="f32")
    w0 = np.random.Generator(np.random.PCG64(cfg.seed)).standard_normal(4096, dtype=np.float32)
    for b in (0, 1, 2):
        x = S.make_x(cfg, b, 2).reshape(-1)
        assert not np.allclose(x, w0[:x.size])
        assert abs(np.corrcoef(x, w0[:x.size])[0, 1]) < 0.1
    # latents of sequence 0 stay at the N(0, 1) scale (a replayed weight row would give
    # c_i = sqrt(d_model) |W_DKV,i|^2 ~ 45 for the rows that align with W_DKV)
    p = S.make_problem(cfg)
    x = S.make_x(cfg, 0, 2600)
    c = x @ p.weights["w_dkv"].T
    assert np.abs(c).max() < 8.0


def test_mlra_output_is_the_sum_over_latent_heads():
    """MLRA page: head h reads latent block h // (H/L) only, and W_O is linear in the heads'
    outputs, so each latent head with its H/L query heads is an L = 1 layer of rank r/L and
    the layer's output is the sum of theirs (decode of the same token, fp64)."""
    import latent_heads as LH
    cfg = S.CONFIGS["mlra_decode"].replace(d_model=96, n_heads=8, d_nope=16, r_kv=32, n_latent_heads=4,
                                           batch=2, ctx_lo=0, ctx_hi=0, dtype="f32")
    prob = S.make_problem(cfg)
    x = S.make_x(cfg, 0, 7)
    y = O.decode(x, prob.weights, O.Dims.from_cfg(cfg))
    parts = []
    for g in range(cfg.n_latent_heads):
        pg = LH.block_problem(prob, g)
        parts.append(O.decode(x, pg.weights, O.Dims.from_cfg(pg.cfg)))
    np.testing.assert_allclose(np.sum(parts, axis=0), y, rtol=1e-10, atol=1e-12)
    # and each part is a real share of the output, not the whole of it
    assert all(np.linalg.norm(p) < 0.9 * np.linalg.norm(y) for p in parts)
