"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The whole call runs at full size (every sequence, every head, the full context); the
fp64 oracle then recomputes sampled outputs one by one: whole sequences for decode,
sampled query rows for prefill.  Tolerances as elsewhere: bf16-in / fp32-accumulate
rel-L2 <= 1e-2 and max-abs <= 3e-2 per compared output row.
"""
import numpy as np
import pytest

import mla_synth as S
from oracle import mla_oracle as O

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


def _fill_with_last(gu, lay, ckv, kr, lens):
    """Cache rows 0..lens[b]-1 from the seeded inputs; returns each sequence's next token."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = lay.cfg
    nt = S.host_threads()
    last = np.zeros((len(lens), cfg.d_model), np.float32)
    for i0 in range(0, len(lens), nt):
        idx = list(range(i0, min(len(lens), i0 + nt)))
        with ThreadPoolExecutor(nt) as ex:
            xs = list(ex.map(lambda b: S.make_x(cfg, b, int(lens[b]) + 1), idx))
        for b, x in zip(idx, xs):
            last[b] = x[-1]
            if lens[b] > 0:
                lay.append(gu.to_dev(x[:-1], cfg)[None], [0], lay.cache_view(ckv, kr, b, 1))
        del xs
    torch.cuda.synchronize()
    return last


@pytest.mark.parametrize("name,sample", [("dsv2_decode", [0, 37, 63]), ("mlra_decode", [0, 77, 127])])
def test_decode_full(gu, name, sample):
    cfg = S.CONFIGS[name]
    gu.say(f"[decode-full] {name} B={cfg.batch} sample={sample}")
    lay = gu.Layer(cfg)
    ctx = [int(c) for c in lay.prob.ctx_lens]
    B = cfg.batch
    max_ctx = max(ctx)
    ckv, kr = lay.new_cache(B, max_ctx + 8, fill=3.0)
    last = _fill_with_last(gu, lay, ckv, kr, ctx)
    gu.say(f"  cache filled: {sum(ctx)} tokens, max ctx {max_ctx}")
    y = gu.to_host(lay.decode(gu.to_dev(last, cfg), ctx, lay.cache_view(ckv, kr, 0, B)))
    assert np.all(np.isfinite(y))
    d = O.Dims.from_cfg(cfg)
    for b in sample:
        seq = S.make_x(cfg, b, ctx[b] + 1)
        c, _ = O.latent_rows(seq[-1:], lay.prob.weights, d, np.array([ctx[b]]))
        gu.assert_close(gu.to_host(ckv[b, ctx[b]]), c[0], cfg.dtype, f"appended row b={b}")
        gu.assert_close(y[b], O.decode(seq, lay.prob.weights, d), cfg.dtype, f"y b={b} ctx={ctx[b]}")


@pytest.mark.parametrize("B,sample", [(20, None), (40, [0, 1, 19, 31, 32, 33, 38, 39])])
def test_decode_full_dims_short_contexts(gu, B, sample):
    """The DeepSeek-V2 decode dimensions (d_model 5120, 128 heads, r_q 1536) with 20 and 40
    sequences of short ragged contexts: the few-row projections with one (20 rows) and two
    (40 rows, the second block ragged) 32-row activation blocks, the vectorised output stage
    (rotary pairs, cache rows); every sampled sequence's output and appended cache row
    against the oracle."""
    cfg = S.CONFIGS["dsv2_decode"].replace(name=f"dsv2_decode_b{B}", batch=B, ctx_lo=16, ctx_hi=64)
    sample = list(range(B)) if sample is None else sample
    gu.say(f"[decode-full-dims] {cfg.name} B={B} sample={len(sample)} sequences")
    lay = gu.Layer(cfg)
    ctx = [int(c) for c in lay.prob.ctx_lens]
    ckv, kr = lay.new_cache(B, max(ctx) + 8, fill=3.0)
    last = _fill_with_last(gu, lay, ckv, kr, ctx)
    y = gu.to_host(lay.decode(gu.to_dev(last, cfg), ctx, lay.cache_view(ckv, kr, 0, B)))
    assert np.all(np.isfinite(y))
    d = O.Dims.from_cfg(cfg)
    for b in sample:
        seq = S.make_x(cfg, b, ctx[b] + 1)
        c, _ = O.latent_rows(seq[-1:], lay.prob.weights, d, np.array([ctx[b]]))
        gu.assert_close(gu.to_host(ckv[b, ctx[b]]), c[0], cfg.dtype, f"appended row b={b}")
        gu.assert_close(y[b], O.decode(seq, lay.prob.weights, d), cfg.dtype, f"y b={b} ctx={ctx[b]}")


def test_decode_latent_head_full(gu):
    """One MLRA latent head on its own (rank 128, its 4 query heads) over the full MLRA
    contexts: the token-split decode kernel with 4096-token splits, four partial rows each."""
    import latent_heads as LH
    full = S.make_problem(S.CONFIGS["mlra_decode"])
    pg = LH.block_problem(full, 2)
    cfg = pg.cfg
    sample = [0, 77, 127]
    gu.say(f"[decode-full] {cfg.name} B={cfg.batch} sample={sample}")
    lay = gu.Layer(cfg, pg)
    ctx = [int(c) for c in pg.ctx_lens]
    B = cfg.batch
    max_ctx = max(ctx)
    ckv, kr = lay.new_cache(B, max_ctx + 8, fill=3.0)
    last = _fill_with_last(gu, lay, ckv, kr, ctx)
    y = gu.to_host(lay.decode(gu.to_dev(last, cfg), ctx, lay.cache_view(ckv, kr, 0, B)))
    assert np.all(np.isfinite(y))
    d = O.Dims.from_cfg(cfg)
    for b in sample:
        seq = S.make_x(cfg, b, ctx[b] + 1)
        gu.assert_close(y[b], O.decode(seq, pg.weights, d), cfg.dtype, f"y b={b} ctx={ctx[b]}")


@pytest.mark.parametrize("name", ["dsv2_decode", "mlra_decode"])
def test_decode_attention_full(gu, name):
    """mla_decode_attention at full size over the cache the library filled, with absorbed
    queries made by the oracle; the oracle attends over the same (bf16) cache rows.  Every
    sequence (every split work item of the launch) is compared: all heads of one latent
    block at once, as the queries of one oracle call."""
    import head_latent_attention_dkv_amd as M
    cfg = S.CONFIGS[name]
    gu.say(f"[decode-attention-full] {name} B={cfg.batch} every sequence")
    lay = gu.Layer(cfg)
    W = lay.prob.weights
    ctx = [int(c) for c in lay.prob.ctx_lens]
    B, H, L, dn = cfg.batch, cfg.n_heads, cfg.n_latent_heads, cfg.d_nope
    rb = cfg.r_kv // L
    max_ctx = max(ctx)
    ckv, kr = lay.new_cache(B, max_ctx + 8, fill=3.0)
    last = _fill_with_last(gu, lay, ckv, kr, ctx)
    # the new tokens' latents at row ctx[b] (one append of B rows)
    lay.append(gu.to_dev(last, cfg)[:, None], ctx, lay.cache_view(ckv, kr, 0, B))
    d = O.Dims.from_cfg(cfg)
    q_lat = np.zeros((B, H, rb), np.float32)
    q_rope = np.zeros((B, H, cfg.d_rope), np.float32) if cfg.d_rope else None
    zero_lat = np.zeros((1, cfg.r_kv))
    wuk = [O.head_up_projections(W, d, h, zero_lat)[0] for h in range(H)]
    for b in range(B):
        q = O.queries(last[b][None], W, d, np.array([ctx[b]]))[0]
        for h in range(H):
            q_lat[b, h] = wuk[h].T @ q[h, :dn]
            if q_rope is not None:
                q_rope[b, h] = q[h, dn:]
    q_lat = S.round_bf16(q_lat)
    if q_rope is not None:
        q_rope = S.round_bf16(q_rope)
    z = torch.empty((B, H, rb), dtype=gu.tdtype(cfg), device="cuda")
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    ws, nbytes = lay.workspace(M.MLA_OP_DECODE_ATTENTION, B, max_ctx)
    M.mla_decode_attention(lay.dims, gu.to_dev(q_lat, cfg), None if q_rope is None else gu.to_dev(q_rope, cfg),
                           B, cl, max_ctx, lay.cache_view(ckv, kr, 0, B), z, ws, nbytes)
    z_h = gu.to_host(z)
    hpb = H // L
    for b in range(B):
        n = ctx[b] + 1
        c_rows = gu.to_host(ckv[b, :n])
        if b in (0, B - 1):
            c_new, _ = O.latent_rows(last[b][None], W, d, np.array([ctx[b]]))
            gu.assert_close(c_rows[-1], c_new[0], cfg.dtype, f"appended row b={b}")
        kr_rows = gu.to_host(kr[b, :n]) if kr is not None else None
        want = np.zeros((H, rb))
        for g in range(L):
            hs = slice(g * hpb, (g + 1) * hpb)
            want[hs] = O.latent_attention(q_lat[b, hs], None if q_rope is None else q_rope[b, hs],
                                          c_rows[:, g * rb:(g + 1) * rb], kr_rows, d.scale())
        gu.assert_close(z_h[b], want, cfg.dtype, f"z b={b} ctx={ctx[b]}")


# DeepSeek-V2 prefill: one row in each of the sixteen 256-query tiles of every sequence (the
# flash kernel's block map differs per tile), at varying offsets inside the tile, plus both
# ends of the sequence.
DSV2_PREFILL_ROWS = sorted({0, 4095} | {256 * t + (37 * t + 1) % 256 for t in range(16)})


@pytest.mark.parametrize("name,sample_b,rows", [
    ("dsv2_prefill", [0, 1, 2, 3], DSV2_PREFILL_ROWS),
    ("small_lm", [0, 5], None),
])
def test_prefill_full(gu, name, sample_b, rows):
    cfg = S.CONFIGS[name]
    gu.say(f"[prefill-full] {name} B={cfg.batch} S={cfg.seq}")
    lay = gu.Layer(cfg)
    B, S_ = cfg.batch, cfg.seq
    xs = S.make_x_batch(cfg, [S_] * B, threads=S.host_threads())
    x = gu.to_dev(np.stack(xs), cfg)
    ckv, kr = lay.new_cache(B, S_, fill=3.0)
    y = gu.to_host(lay.prefill(x, lay.cache_view(ckv, kr, 0, B)))
    assert np.all(np.isfinite(y))
    d = O.Dims.from_cfg(cfg)
    for b in sample_b:
        want = O.forward(xs[b], lay.prob.weights, d, q_rows=rows)
        got = y[b] if rows is None else y[b][rows]
        for i in range(want.shape[0]):
            r = i if rows is None else rows[i]
            if rows is None and i % 128 != 0 and i != S_ - 1:
                continue
            gu.assert_close(got[i], want[i], cfg.dtype, f"y b={b} row={r}")
        gu.assert_close(got, want, cfg.dtype, f"y b={b} sampled rows together")
        c, _ = O.latent_rows(xs[b][:64], lay.prob.weights, d, np.arange(64))
        gu.assert_close(gu.to_host(ckv[b, :64]), c, cfg.dtype, f"cache rows 0..63 b={b}")


def test_prefill_chunk_full(gu):
    """Continued prefill at the DeepSeek-V2 prefill shape: 3072 cached tokens, 1024 new."""
    cfg = S.CONFIGS["dsv2_prefill"]
    B, start, T = cfg.batch, 3072, 1024
    gu.say(f"[prefill-chunk-full] B={B} start={start} T={T}")
    lay = gu.Layer(cfg)
    ckv, kr = lay.new_cache(B, start + T, fill=3.0)
    lay.fill_cache(ckv, kr, [start] * B, threads=S.host_threads())
    xs = S.make_x_batch(cfg, [start + T] * B, threads=S.host_threads())
    x = gu.to_dev(np.stack([xb[start:] for xb in xs]), cfg)
    y = gu.to_host(lay.prefill_chunk(x, start, lay.cache_view(ckv, kr, 0, B)))
    assert np.all(np.isfinite(y))
    d = O.Dims.from_cfg(cfg)
    # a row at a boundary of each of the sixteen 64-row groups of the new tokens
    rows = [64 * g + (63 if g % 2 else 0) for g in range(16)]
    for b in range(B):
        want = O.forward(xs[b], lay.prob.weights, d, q_rows=[start + r for r in rows])
        got = y[b][rows]
        for i, r in enumerate(rows):
            gu.assert_close(got[i], want[i], cfg.dtype, f"y b={b} row={start + r}")
        gu.assert_close(got, want, cfg.dtype, f"y b={b} sampled rows together")
