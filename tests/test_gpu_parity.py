"""GPU parity of the HIP kernels against the fp64 oracle, through the C ABI.

Sizes are small enough for the oracle to finish in seconds but span several tiles and a
ragged tail (query tiles of 128, key tiles of 64, decode tiles of 32 tokens and context
splits).  Tolerances: fp32 rel-L2 <= 1e-5; bf16-in / fp32-accumulate rel-L2 <= 1e-2 and
max-abs <= 3e-2 (whole tensor).
"""
import numpy as np
import pytest

import latent_heads as LH
import mla_synth as S
from oracle import mla_oracle as O

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

SENTINEL = 3.0   # canary value of untouched cache rows (exact in bf16)

# Scaled cases of the five workloads (same families and per-head shapes).
TINY = S.CONFIGS["tiny_fp32"]
SMALL = S.CONFIGS["small_lm"].replace(batch=2, seq=200)
DSV2 = S.CONFIGS["dsv2_decode"].replace(d_model=512, batch=3, seq=1000)   # reduced d_model
DSV2_P = S.CONFIGS["dsv2_prefill"].replace(d_model=512, batch=2, seq=300)
MLRA = S.CONFIGS["mlra_decode"].replace(d_model=512, batch=4, ctx_lo=0, ctx_hi=0)
# Shapes of the flash prefill path (sequence a multiple of 64 key rows; 320 = one full and
# one partial 256-query tile, five key tiles).
DSV2_PF = S.CONFIGS["dsv2_prefill"].replace(name="dsv2_prefill_s320", d_model=512, batch=2, seq=320)
SMALL_PF = S.CONFIGS["small_lm"].replace(name="small_lm_s320", batch=2, seq=320)
# 576 = two full 256-query tiles and a partial one: an odd number of query tiles per head
# (even counts are walked in pairs of a short and a long tile, odd ones one tile at a time).
DSV2_PF3 = S.CONFIGS["dsv2_prefill"].replace(name="dsv2_prefill_s576", d_model=512, batch=2, seq=576)
MLRA_PF = S.CONFIGS["mlra_decode"].replace(name="mlra_prefill_s384", mode="prefill", d_model=512, batch=2,
                                           seq=384, ctx_lo=0, ctx_hi=0)
# Few-row products (B*S <= 128 rows) of the full-RoPE family: the query and key rotations
# run in the output stage of the few-row GEMM, whose tile must hold whole half-split heads.
SMALL_FEW = S.CONFIGS["small_lm"].replace(name="small_lm_b1_s64", batch=1, seq=64)
TINY_BF16_MLRA = S.MLAConfig("mlra_tiny", S.FAMILY_MLRA, "decode", 2, 40, d_model=64, n_heads=8,
                             d_nope=16, d_rope=0, r_kv=32, r_q=0, n_latent_heads=4, seed=77)


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


_layers = {}


def layer(gu, cfg):
    key = cfg
    if key not in _layers:
        _layers[key] = gu.Layer(cfg)
    return _layers[key]


def _dims(cfg):
    return O.Dims.from_cfg(cfg)


# ---------------------------------------------------------------------------
# mla_cache_append: fused down-projection + RoPE + cache write
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [TINY, SMALL, DSV2, MLRA], ids=lambda c: c.name)
def test_cache_append(gu, cfg):
    gu.say(f"[append] {cfg.name} seed={cfg.seed}")
    lay = layer(gu, cfg)
    B, T, max_seq = 3, 37, 96
    starts = [0, 5, 59]
    ckv, kr = lay.new_cache(B, max_seq, fill=SENTINEL)
    xs = [S.make_x(cfg, b, starts[b] + T)[starts[b]:] for b in range(B)]
    x = gu.to_dev(np.stack(xs), cfg)
    lay.append(x, starts, lay.cache_view(ckv, kr, 0, B))
    torch.cuda.synchronize()
    ckv_h, kr_h = gu.to_host(ckv), (gu.to_host(kr) if kr is not None else None)
    d = _dims(cfg)
    for b in range(B):
        pos = np.arange(starts[b], starts[b] + T)
        c, krr = O.latent_rows(xs[b], lay.prob.weights, d, pos)
        gu.assert_close(ckv_h[b, pos], c, cfg.dtype, f"latent rows b={b}")
        if krr is not None:
            gu.assert_close(kr_h[b, pos], krr, cfg.dtype, f"rotary key rows b={b}")
        outside = np.ones(max_seq, bool)
        outside[pos] = False
        assert np.all(ckv_h[b, outside] == SENTINEL), "rows outside the append changed"
        if kr_h is not None:
            assert np.all(kr_h[b, outside] == SENTINEL)


# ---------------------------------------------------------------------------
# mla_prefill: causal prefill, explicit K/V up-projection
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [TINY, SMALL, DSV2_P, MLRA.replace(name="mlra_prefill_s150", mode="prefill", batch=2,
                                                                  seq=150),
                                 DSV2_PF, SMALL_PF, MLRA_PF, SMALL_FEW],
                         ids=lambda c: c.name)
@pytest.mark.parametrize("with_cache", [False, True])
def test_prefill(gu, cfg, with_cache):
    gu.say(f"[prefill] {cfg.name} B={cfg.batch} S={cfg.seq} cache={with_cache}")
    lay = layer(gu, cfg)
    B, S_ = cfg.batch, cfg.seq
    xs = [S.make_x(cfg, b, S_) for b in range(B)]
    x = gu.to_dev(np.stack(xs), cfg)
    cache = None
    if with_cache:
        ckv, kr = lay.new_cache(B, S_ + 5, fill=SENTINEL)
        cache = lay.cache_view(ckv, kr, 0, B)
    y = gu.to_host(lay.prefill(x, cache))
    d = _dims(cfg)
    for b in range(B):
        want = O.forward(xs[b], lay.prob.weights, d)
        gu.assert_close(y[b], want, cfg.dtype, f"y b={b}")
    if with_cache:
        ckv_h = gu.to_host(ckv)
        for b in range(B):
            c, _ = O.latent_rows(xs[b], lay.prob.weights, d, np.arange(S_))
            gu.assert_close(ckv_h[b, :S_], c, cfg.dtype, f"cache b={b}")
            assert np.all(ckv_h[b, S_:] == SENTINEL)


# ---------------------------------------------------------------------------
# mla_prefill_chunk: continued prefill over an existing latent cache
# ---------------------------------------------------------------------------
CHUNK_CASES = [
    (DSV2_PF, 128, 192),     # flash path: key offset and key count multiples of 64
    (SMALL_PF, 64, 256),     # flash path, full-RoPE family (keys rotated after up-projection)
    (MLRA_PF, 192, 128),     # flash path, latent blocks
    (DSV2_P, 37, 50),        # generic path (offset not a multiple of 64), ragged tiles
    (DSV2_PF, 0, 320),       # start 0: the same as mla_prefill with a cache
    (TINY, 5, 3),            # fp32 workload
    (SMALL, 100, 1),         # full-RoPE family, one new token per sequence (2 rows)
    (SMALL, 64, 64),         # full-RoPE family, 128 new rows: few-row products with rotation
]


@pytest.mark.parametrize("cfg,start,T", CHUNK_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_prefill_chunk(gu, cfg, start, T):
    gu.say(f"[prefill-chunk] {cfg.name} start={start} T={T}")
    lay = layer(gu, cfg)
    B = cfg.batch
    max_seq = start + T + 7
    ckv, kr = lay.new_cache(B, max_seq, fill=SENTINEL)
    lay.fill_cache(ckv, kr, [start] * B)
    xs = [S.make_x(cfg, b, start + T) for b in range(B)]
    x = gu.to_dev(np.stack([xb[start:] for xb in xs]), cfg)
    y = gu.to_host(lay.prefill_chunk(x, start, lay.cache_view(ckv, kr, 0, B)))
    d = _dims(cfg)
    ckv_h = gu.to_host(ckv)
    for b in range(B):
        want = O.forward(xs[b], lay.prob.weights, d, q_rows=np.arange(start, start + T))
        gu.assert_close(y[b], want, cfg.dtype, f"y b={b}")
        c, _ = O.latent_rows(xs[b][start:], lay.prob.weights, d, np.arange(start, start + T))
        gu.assert_close(ckv_h[b, start:start + T], c, cfg.dtype, f"appended rows b={b}")
        assert np.all(ckv_h[b, start + T:] == SENTINEL), "rows after the chunk changed"


def test_prefill_chunk_capacity(gu):
    import head_latent_attention_dkv_amd as M
    cfg = DSV2_PF
    lay = layer(gu, cfg)
    ckv, kr = lay.new_cache(1, 100)
    x = gu.to_dev(np.stack([S.make_x(cfg, 0, 64)]), cfg)
    with pytest.raises(M.MLAError) as e:
        lay.prefill_chunk(x, 40, lay.cache_view(ckv, kr, 0, 1))     # 40 + 64 > 100 rows
    assert e.value.status == M.MLA_ERR_CAPACITY


# ---------------------------------------------------------------------------
# mla_decode: absorbed decode over the latent cache
# ---------------------------------------------------------------------------
DECODE_CASES = [
    (DSV2, [37, 300, 1000]),          # one, several and many 32-token tiles; several splits
    # 37 sequences: the fused combine's second group of 32 holds 5, the merged down-projection
    # runs on 37 rows; short ragged contexts keep the oracle quick
    (DSV2, [int(c) for c in np.random.default_rng(37).integers(0, 70, size=37)]),
    (MLRA, [5, 100, 700, 1500]),      # ragged, 4 latent heads
    (TINY_BF16_MLRA, [0, 39]),        # empty context (attends to itself only)
    (TINY.replace(mode="decode"), [0, 7]),
]


@pytest.mark.parametrize("cfg,ctx", DECODE_CASES, ids=lambda v: getattr(v, "name", str(v)))
def test_decode(gu, cfg, ctx):
    gu.say(f"[decode] {cfg.name} ctx={ctx}")
    lay = layer(gu, cfg)
    B = len(ctx)
    max_seq = max(ctx) + 9
    ckv, kr = lay.new_cache(B, max_seq, fill=SENTINEL)
    lay.fill_cache(ckv, kr, ctx)
    seqs = [S.make_x(cfg, b, ctx[b] + 1) for b in range(B)]
    x = gu.to_dev(np.stack([s[-1] for s in seqs]), cfg)
    y = gu.to_host(lay.decode(x, ctx, lay.cache_view(ckv, kr, 0, B)))
    d = _dims(cfg)
    ckv_h = gu.to_host(ckv)
    for b in range(B):
        gu.assert_close(y[b], O.decode(seqs[b], lay.prob.weights, d), cfg.dtype, f"y b={b} ctx={ctx[b]}")
        c, _ = O.latent_rows(seqs[b][-1:], lay.prob.weights, d, np.array([ctx[b]]))
        gu.assert_close(ckv_h[b, ctx[b]], c[0], cfg.dtype, f"appended row b={b}")
        assert np.all(ckv_h[b, ctx[b] + 1:] == SENTINEL)


def test_decode_many_sequences(gu):
    """150 sequences: above the few-row path's 128 rows, so the decode step's projections run
    on the general GEMM kernels, and the fused combine's fifth group of 32 holds 22.  All
    outputs finite; sampled sequences (both sides of every group edge) against the oracle."""
    cfg = DSV2
    ctx = [int(c) for c in np.random.default_rng(150).integers(0, 24, size=150)]
    sample = [0, 31, 32, 127, 128, 129, 140, 149]
    gu.say(f"[decode] {cfg.name} B={len(ctx)} sample={sample}")
    lay = layer(gu, cfg)
    B = len(ctx)
    ckv, kr = lay.new_cache(B, max(ctx) + 9, fill=SENTINEL)
    lay.fill_cache(ckv, kr, ctx)
    last = np.stack([S.make_x(cfg, b, ctx[b] + 1)[-1] for b in range(B)])
    y = gu.to_host(lay.decode(gu.to_dev(last, cfg), ctx, lay.cache_view(ckv, kr, 0, B)))
    assert np.all(np.isfinite(y))
    d = _dims(cfg)
    for b in sample:
        gu.assert_close(y[b], O.decode(S.make_x(cfg, b, ctx[b] + 1), lay.prob.weights, d), cfg.dtype,
                        f"y b={b} ctx={ctx[b]}")


def test_decode_every_position_tiny(gu):
    """fp32: decoding token t after a cache of t tokens equals prefill row t, for all t."""
    cfg = TINY
    lay = layer(gu, cfg)
    d = _dims(cfg)
    Sq = cfg.seq
    xs = [S.make_x(cfg, b, Sq) for b in range(cfg.batch)]
    want = [O.forward(xs[b], lay.prob.weights, d) for b in range(cfg.batch)]
    ckv, kr = lay.new_cache(cfg.batch, Sq + 1, fill=SENTINEL)
    for t in range(Sq):
        gu.say(f"[decode-every] t={t}")
        x = gu.to_dev(np.stack([xs[b][t] for b in range(cfg.batch)]), cfg)
        y = gu.to_host(lay.decode(x, [t] * cfg.batch, lay.cache_view(ckv, kr, 0, cfg.batch)))
        for b in range(cfg.batch):
            gu.assert_close(y[b], want[b][t], cfg.dtype, f"row t={t} b={b}")


def test_decode_is_deterministic(gu):
    cfg, ctx = DSV2, [37, 300, 1000]
    lay = layer(gu, cfg)
    B = len(ctx)
    ckv, kr = lay.new_cache(B, max(ctx) + 1)
    lay.fill_cache(ckv, kr, ctx)
    x = gu.to_dev(np.stack([S.make_x(cfg, b, ctx[b] + 1)[-1] for b in range(B)]), cfg)
    cs = lay.cache_view(ckv, kr, 0, B)
    y1 = lay.decode(x, ctx, cs).clone()
    y2 = lay.decode(x, ctx, cs).clone()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("cfg,ctx", [(DSV2, [37, 300, 1000]), (MLRA, [5, 1030]),
                                     (LH.block_cfg(MLRA), [0, 129, 1030])],
                         ids=["dsv2", "mlra", "mlra_latent_head"])
def test_decode_graph_replay(gu, cfg, ctx):
    """mla_decode captured into a HIP graph: the call makes no allocation, fill or host
    synchronisation, so the captured kernels replay it.  Every replay, with eager work and a
    synchronisation between replays, equals the eager call bit for bit, and leaves the same
    cache."""
    import head_latent_attention_dkv_amd as M
    gu.say(f"[decode graph] {cfg.name} ctx={ctx}")
    lay = layer(gu, cfg)
    B = len(ctx)
    ckv, kr = lay.new_cache(B, max(ctx) + 1)
    lay.fill_cache(ckv, kr, ctx)
    x = gu.to_dev(np.stack([S.make_x(cfg, b, ctx[b] + 1)[-1] for b in range(B)]), cfg)
    cs = lay.cache_view(ckv, kr, 0, B)
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    mc = max(ctx)
    ws, n = lay.workspace(M.MLA_OP_DECODE, B, mc)
    y = torch.empty((B, cfg.d_model), dtype=torch.float32, device="cuda")

    def call():
        M.mla_decode(lay.dims, lay.ws_struct, x, B, cl, mc, cs, y, ws, n)

    call()
    torch.cuda.synchronize()
    want, ckv_want = y.clone(), ckv.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        y.fill_(float("nan"))
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {i}"
        assert torch.equal(ckv, ckv_want), f"cache after replay {i}"
    del g


# ---------------------------------------------------------------------------
# Staged entry points with oracle-made inputs
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,ctx", [(DSV2, [40, 513, 999]), (MLRA, [5, 1030]),
                                     (LH.block_cfg(MLRA), [0, 5, 127, 128, 129, 1030])],
                         ids=["dsv2", "mlra", "mlra_latent_head"])
def test_decode_attention_entry(gu, cfg, ctx):
    """mla_decode_attention on latent rows and absorbed queries made by the oracle."""
    _decode_attention_case(gu, cfg, ctx)


# Cache strides (rows per sequence) around the point where a row's byte offset inside its
# sequence stops fitting 32 bits for the fast kernels: the latent-head kernel's 256-byte
# rows (2^23) and the 128-byte rotary rows of the DSV2 kernel (2^25).  Only the first rows
# of each sequence are filled; the rows just past each context hold large values that any
# read beyond the context would turn into a mismatch.
@pytest.mark.parametrize("cfg,max_seq", [(LH.block_cfg(MLRA), 2**23 - 64), (LH.block_cfg(MLRA), 2**23 + 64),
                                         (DSV2, 2**25 + 64)],
                         ids=["latent_head_below", "latent_head_above", "dsv2_above"])
def test_decode_attention_long_cache_stride(gu, cfg, max_seq):
    cache_bytes = 2 * max_seq * (cfg.r_kv + cfg.d_rope) * 2
    free, _ = torch.cuda.mem_get_info()
    if free < cache_bytes + (4 << 30):
        pytest.skip(f"needs {cache_bytes >> 30} GiB of free device memory")
    try:
        _decode_attention_case(gu, cfg, [300, 77], max_seq=max_seq)
    finally:
        torch.cuda.empty_cache()


def _decode_attention_case(gu, cfg, ctx, max_seq=None):
    import head_latent_attention_dkv_amd as M
    gu.say(f"[decode_attention] {cfg.name} ctx={ctx} max_seq={max_seq}")
    lay = layer(gu, cfg)
    d = _dims(cfg)
    B, H, L = len(ctx), cfg.n_heads, cfg.n_latent_heads
    rb = cfg.r_kv // L
    n_host = max(ctx) + 1
    max_seq = max_seq or n_host
    ckv_h = np.zeros((B, n_host, cfg.r_kv), np.float32)
    kr_h = np.zeros((B, n_host, cfg.d_rope), np.float32) if cfg.d_rope else None
    q_lat = np.zeros((B, H, rb), np.float32)
    q_rope = np.zeros((B, H, cfg.d_rope), np.float32) if cfg.d_rope else None
    want = np.zeros((B, H, rb))
    rng = np.random.default_rng(5)
    for b in range(B):
        n = ctx[b] + 1
        xs = S.make_x(cfg, b, n)
        c, kr = O.latent_rows(xs, lay.prob.weights, d, np.arange(n))
        ckv_h[b, :n] = S.round_bf16(c.astype(np.float32))
        if kr is not None:
            kr_h[b, :n] = S.round_bf16(kr.astype(np.float32))
        q_lat[b] = S.round_bf16(rng.standard_normal((H, rb)).astype(np.float32) * 4)
        if q_rope is not None:
            q_rope[b] = S.round_bf16(rng.standard_normal((H, cfg.d_rope)).astype(np.float32) * 4)
        for h in range(H):
            g = h // (H // L)
            lat = ckv_h[b, :n, g * rb:(g + 1) * rb]
            want[b, h] = O.latent_attention(q_lat[b, h][None], None if q_rope is None else q_rope[b, h][None],
                                            lat, None if kr_h is None else kr_h[b, :n], d.scale())[0]
    if max_seq == n_host:
        ckv, kr = gu.to_dev(ckv_h, cfg), (gu.to_dev(kr_h, cfg) if kr_h is not None else None)
    else:
        tail = min(64, max_seq - n_host)
        ckv = torch.empty((B, max_seq, cfg.r_kv), dtype=gu.tdtype(cfg), device="cuda")
        kr = torch.empty((B, max_seq, cfg.d_rope), dtype=gu.tdtype(cfg), device="cuda") if cfg.d_rope else None
        for b in range(B):
            n = ctx[b] + 1
            ckv[b, :n].copy_(gu.to_dev(ckv_h[b, :n], cfg))
            ckv[b, n:n + tail].fill_(SENTINEL * 1e4)
            if kr is not None:
                kr[b, :n].copy_(gu.to_dev(kr_h[b, :n], cfg))
                kr[b, n:n + tail].fill_(SENTINEL * 1e4)
    z = torch.empty((B, H, rb), dtype=gu.tdtype(cfg), device="cuda")
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    ws, nbytes = lay.workspace(M.MLA_OP_DECODE_ATTENTION, B, max(ctx))
    M.mla_decode_attention(lay.dims, gu.to_dev(q_lat, cfg), None if q_rope is None else gu.to_dev(q_rope, cfg),
                           B, cl, max(ctx), M.cache_struct(ckv, kr, B, max_seq), z, ws, nbytes)
    gu.assert_close(gu.to_host(z), want, cfg.dtype, "z")


@pytest.mark.parametrize("cfg", [DSV2_P, SMALL, DSV2_PF, SMALL_PF, DSV2_PF3], ids=lambda c: c.name)
def test_prefill_attention_entry(gu, cfg):
    """mla_prefill_attention on oracle queries and oracle latent rows."""
    import head_latent_attention_dkv_amd as M
    gu.say(f"[prefill_attention] {cfg.name}")
    lay = layer(gu, cfg)
    d = _dims(cfg)
    B, S_, H = cfg.batch, cfg.seq, cfg.n_heads
    dq = cfg.d_nope + cfg.d_rope
    ckv_h = np.zeros((B, S_, cfg.r_kv), np.float32)
    kr_h = np.zeros((B, S_, cfg.d_rope), np.float32) if cfg.d_rope else None
    q_h = np.zeros((B, S_, H, dq), np.float32)
    want = np.zeros((B, S_, H, cfg.d_v))
    pos = np.arange(S_)
    for b in range(B):
        xs = S.make_x(cfg, b, S_)
        c, kr = O.latent_rows(xs, lay.prob.weights, d, pos)
        ckv_h[b] = S.round_bf16(c.astype(np.float32))
        if kr is not None:
            kr_h[b] = S.round_bf16(kr.astype(np.float32))
        q_h[b] = S.round_bf16(O.queries(xs, lay.prob.weights, d, pos).astype(np.float32))
        k, v = O.keys_values(ckv_h[b], None if kr_h is None else kr_h[b], lay.prob.weights, d, pos)
        want[b] = O.causal_attention(q_h[b], k, v, d.scale(), pos, pos)
    ckv, kr = gu.to_dev(ckv_h, cfg), (gu.to_dev(kr_h, cfg) if kr_h is not None else None)
    o = torch.empty((B, S_, H, cfg.d_v), dtype=gu.tdtype(cfg), device="cuda")
    ws, nbytes = lay.workspace(M.MLA_OP_PREFILL_ATTENTION, B, S_)
    M.mla_prefill_attention(lay.dims, lay.ws_struct, gu.to_dev(q_h, cfg), B, S_, M.cache_struct(ckv, kr, B, S_),
                            o, ws, nbytes)
    gu.assert_close(gu.to_host(o), want, cfg.dtype, "o")


@pytest.mark.parametrize("spike_at", [[3, 450, 990], [0, 700, 31]], ids=["late", "early"])
def test_decode_attention_score_spikes(gu, spike_at):
    """Scores that jump far above the first tile's maximum (exercises the exact-maximum
    re-stream): one cache row per sequence is aligned with the absorbed query."""
    import head_latent_attention_dkv_amd as M
    cfg = DSV2
    lay = layer(gu, cfg)
    d = _dims(cfg)
    ctx = [40, 513, 999]
    B, H, rb = len(ctx), cfg.n_heads, cfg.r_kv
    max_seq = max(ctx) + 1
    rng = np.random.default_rng(11)
    u = S.round_bf16(rng.standard_normal(rb).astype(np.float32))
    ckv_h = S.round_bf16(rng.standard_normal((B, max_seq, rb)).astype(np.float32))
    kr_h = S.round_bf16(rng.standard_normal((B, max_seq, cfg.d_rope)).astype(np.float32))
    for b in range(B):
        ckv_h[b, spike_at[b]] = S.round_bf16(2.0 * u)
    q_lat = np.broadcast_to(u, (B, H, rb)).astype(np.float32).copy()
    q_rope = S.round_bf16(rng.standard_normal((B, H, cfg.d_rope)).astype(np.float32))
    want = np.zeros((B, H, rb))
    for b in range(B):
        n = ctx[b] + 1
        for h in range(H):
            want[b, h] = O.latent_attention(q_lat[b, h][None], q_rope[b, h][None], ckv_h[b, :n], kr_h[b, :n],
                                            d.scale())[0]
    ckv, kr = gu.to_dev(ckv_h, cfg), gu.to_dev(kr_h, cfg)
    z = torch.empty((B, H, rb), dtype=gu.tdtype(cfg), device="cuda")
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    ws, nbytes = lay.workspace(M.MLA_OP_DECODE_ATTENTION, B, max(ctx))
    M.mla_decode_attention(lay.dims, gu.to_dev(q_lat, cfg), gu.to_dev(q_rope, cfg), B, cl, max(ctx),
                           M.cache_struct(ckv, kr, B, max_seq), z, ws, nbytes)
    gu.assert_close(gu.to_host(z), want, cfg.dtype, f"z spikes at {spike_at}")


@pytest.mark.parametrize("spike", [False, True], ids=["plain", "spikes"])
def test_decode_attention_many_tiles_per_split(gu, spike):
    """64 sequences (few splits per sequence, so each split spans many 32-token tiles and
    every LDS stage is reused) with mixed context lengths; random bf16 cache rows and
    queries.  With spikes, one row per sequence aligned with the query far into the
    context forces the exact-maximum re-stream over many tiles.  Sampled sequences are
    compared with the oracle."""
    import head_latent_attention_dkv_amd as M
    cfg = DSV2
    lay = layer(gu, cfg)
    d = _dims(cfg)
    rng = np.random.default_rng(21 + int(spike))
    B, H, rb = 64, cfg.n_heads, cfg.r_kv
    ctx = [int(c) for c in rng.integers(100, 900, B)]
    ctx[5] = 0
    ctx[6] = 31
    ctx[7] = 899
    gu.say(f"[decode_attention many tiles] spike={spike} ctx[:8]={ctx[:8]}")
    max_seq = max(ctx) + 1
    ckv_h = S.round_bf16(rng.standard_normal((B, max_seq, rb)).astype(np.float32))
    kr_h = S.round_bf16(rng.standard_normal((B, max_seq, cfg.d_rope)).astype(np.float32))
    q_lat = S.round_bf16(rng.standard_normal((B, H, rb)).astype(np.float32))
    q_rope = S.round_bf16(rng.standard_normal((B, H, cfg.d_rope)).astype(np.float32))
    if spike:
        for b in range(B):
            at = (ctx[b] * 3) // 4
            ckv_h[b, at] = S.round_bf16(2.0 * q_lat[b, b % H])
    ckv, kr = gu.to_dev(ckv_h, cfg), gu.to_dev(kr_h, cfg)
    z = torch.empty((B, H, rb), dtype=gu.tdtype(cfg), device="cuda")
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    ws, nbytes = lay.workspace(M.MLA_OP_DECODE_ATTENTION, B, max(ctx))
    M.mla_decode_attention(lay.dims, gu.to_dev(q_lat, cfg), gu.to_dev(q_rope, cfg), B, cl, max(ctx),
                           M.cache_struct(ckv, kr, B, max_seq), z, ws, nbytes)
    z_h = gu.to_host(z)
    for b in [0, 5, 6, 7, 40, 63]:
        n = ctx[b] + 1
        want = np.zeros((H, rb))
        for h in range(H):
            want[h] = O.latent_attention(q_lat[b, h][None], q_rope[b, h][None], ckv_h[b, :n], kr_h[b, :n],
                                         d.scale())[0]
        gu.assert_close(z_h[b], want, cfg.dtype, f"z b={b} ctx={ctx[b]}")


def test_prefill_attention_exact_max_restream(gu):
    """Scores that rise far above the first key tile's maximum (the flash kernel's fixed
    softmax reference): the first 32 latent and rotary-key rows are zero (score 0 for every
    query) and the queries are scaled by 20, so later keys exceed the reference by more than
    the kernel's 64 log2-unit gap and the workgroup re-streams with the exact maximum.  The
    oracle attends over the bf16-rounded explicit keys and values (the kernel's stored K/V)."""
    import head_latent_attention_dkv_amd as M
    cfg = DSV2_PF
    gu.say(f"[prefill_attention restream] {cfg.name}")
    lay = layer(gu, cfg)
    d = _dims(cfg)
    B, S_, H = cfg.batch, cfg.seq, cfg.n_heads
    dq = cfg.d_nope + cfg.d_rope
    pos = np.arange(S_)
    ckv_h = np.zeros((B, S_, cfg.r_kv), np.float32)
    kr_h = np.zeros((B, S_, cfg.d_rope), np.float32)
    q_h = np.zeros((B, S_, H, dq), np.float32)
    want = np.zeros((B, S_, H, cfg.d_v))
    for b in range(B):
        xs = S.make_x(cfg, b, S_)
        c, kr = O.latent_rows(xs, lay.prob.weights, d, pos)
        c[:32] = 0.0
        kr[:32] = 0.0
        ckv_h[b] = S.round_bf16(c.astype(np.float32))
        kr_h[b] = S.round_bf16(kr.astype(np.float32))
        q_h[b] = S.round_bf16((20.0 * O.queries(xs, lay.prob.weights, d, pos)).astype(np.float32))
        k, v = O.keys_values(ckv_h[b], kr_h[b], lay.prob.weights, d, pos)
        k, v = S.round_bf16(k.astype(np.float32)), S.round_bf16(v.astype(np.float32))
        want[b] = O.causal_attention(q_h[b], k, v, d.scale(), pos, pos)
    o = torch.empty((B, S_, H, cfg.d_v), dtype=gu.tdtype(cfg), device="cuda")
    ws, nbytes = lay.workspace(M.MLA_OP_PREFILL_ATTENTION, B, S_)
    M.mla_prefill_attention(lay.dims, lay.ws_struct, gu.to_dev(q_h, cfg), B, S_,
                            M.cache_struct(gu.to_dev(ckv_h, cfg), gu.to_dev(kr_h, cfg), B, S_), o, ws, nbytes)
    gu.assert_close(gu.to_host(o), want, cfg.dtype, "o with far-above-reference scores")


# ---------------------------------------------------------------------------
# One MLRA latent head on its own (L = 1, rank 128, its H/L query heads): the token-split
# decode kernel.  Every latent head against the oracle run on it alone, and the sum over
# the latent heads against the oracle's whole layer (the MLRA page's partition of the
# latent: the sum a latent-head-parallel decode would all-reduce).
# ---------------------------------------------------------------------------
def test_decode_latent_heads_sum(gu):
    cfg = MLRA
    prob = S.make_problem(cfg)
    ctx = [5, 300, 1500, 129, 128, 0, 33]   # ragged; 128-token tile edges; empty context
    gu.say(f"[decode latent heads] {cfg.name} ctx={ctx}")
    B = len(ctx)
    seqs = [S.make_x(cfg, b, ctx[b] + 1) for b in range(B)]
    ys = []
    for g in range(cfg.n_latent_heads):
        pg = LH.block_problem(prob, g)
        lay = gu.Layer(pg.cfg, pg)
        x = gu.to_dev(np.stack([sq[-1] for sq in seqs]), pg.cfg)
        ckv, kr = lay.new_cache(B, max(ctx) + 9, fill=SENTINEL)
        lay.fill_cache(ckv, kr, ctx)
        y = gu.to_host(lay.decode(x, ctx, lay.cache_view(ckv, kr, 0, B)))
        dg = _dims(pg.cfg)
        for b in range(B):
            gu.assert_close(y[b], O.decode(seqs[b], pg.weights, dg), cfg.dtype, f"latent head {g} b={b}")
        ys.append(y)
    d = _dims(cfg)
    ysum = np.sum(ys, axis=0)
    for b in range(B):
        gu.assert_close(ysum[b], O.decode(seqs[b], prob.weights, d), cfg.dtype, f"sum over latent heads b={b}")
