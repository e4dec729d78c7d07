"""GPU parity of the training path (dropout forward, backward) against the fp64 oracle.

[DSV2 page] ``MultiHeadLatentAttention`` with dropout on the attention weights, trained:
mla_train_forward and mla_train_backward through the C ABI against oracle/train_oracle.py
(gradients of sum(dy * y), summed over the batch for the weights).  Tolerances: fp32 rel-L2
<= 1e-5; bf16 (bf16 operands, fp32 accumulation) rel-L2 <= 1e-2 per array, and max-abs <=
3e-2 times the array's largest reference magnitude (the outputs' 3e-2 bound, scaled to each
gradient's size).
"""
import numpy as np
import pytest

import mla_synth as S
from oracle import mla_oracle as O
from oracle import train_oracle as T

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TINY = S.CONFIGS["tiny_fp32"]
# DeepSeek-V2 per-head shapes at a reduced width and head count; 600 tokens: three query blocks
# of the backward (256, 256, 88) and ragged key tiles
DSV2_T = S.CONFIGS["dsv2_prefill"].replace(name="dsv2_train", d_model=256, n_heads=16, r_q=384, batch=2, seq=600)
# whole 64-token tiles: the flash forward and the flash backward kernels (key blocks of 128 with
# a ragged last block of 64; three heads: (sequence, head) groups not a multiple of 8)
DSV2_F = DSV2_T.replace(name="dsv2_train_flash", seq=320)
DSV2_F3 = DSV2_T.replace(name="dsv2_train_flash_h3", n_heads=3, d_model=192, seq=192)
# one 64-token tile and a single sequence; a longer sequence (eight key blocks of 128)
DSV2_F1 = DSV2_T.replace(name="dsv2_train_flash_s64", batch=1, seq=64)
DSV2_FL = DSV2_T.replace(name="dsv2_train_flash_s1024", batch=1, n_heads=4, d_model=256, seq=1024)


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


def _close(gu, got, want, dtype, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    r = gu.rel_l2(got, want)
    m = float(np.max(np.abs(got - want)))
    scale = float(np.max(np.abs(want)))
    gu.say(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e} (max |ref| {scale:.3e})")
    assert np.all(np.isfinite(got)), what
    if dtype == "f32":
        assert r <= 1e-5, f"{what}: rel_l2 {r:.3e}"
    else:
        assert r <= 1e-2, f"{what}: rel_l2 {r:.3e}"
        assert m <= 3e-2 * scale, f"{what}: max_abs {m:.3e} > 3e-2 * {scale:.3e}"


def _train(gu, cfg, p, seed, xs, dys):
    import head_latent_attention_dkv_amd as M
    lay = gu.Layer(cfg)
    B, S_ = len(xs), xs[0].shape[0]
    x = gu.to_dev(np.stack(xs), cfg)
    dy = torch.from_numpy(np.stack(dys).astype(np.float32)).cuda()
    y = torch.empty((B, S_, cfg.d_model), dtype=torch.float32, device="cuda")
    ns = M.mla_train_saved_bytes(lay.dims, B, S_)
    nw = M.mla_train_workspace_bytes(lay.dims, B, S_)
    assert ns > 0 and nw > 0
    saved = torch.empty(ns, dtype=torch.uint8, device="cuda")
    ws = torch.empty(nw, dtype=torch.uint8, device="cuda")
    M.mla_train_forward(lay.dims, lay.ws_struct, x, B, S_, p, seed, y, saved, ns)
    shapes = {"dx": (B, S_, cfg.d_model)}
    shapes.update({"d" + k: v.shape for k, v in lay.prob.weights.items()})
    g = {k: torch.full(s, float("nan"), dtype=torch.float32, device="cuda") for k, s in shapes.items()}
    M.mla_train_backward(lay.dims, lay.ws_struct, x, B, S_, p, seed, dy, saved, ns, M.grads_struct(g), ws, nw)
    torch.cuda.synchronize()
    return gu.to_host(y), {k: gu.to_host(v) for k, v in g.items()}, lay.prob.weights


def _oracle(cfg, W, p, seed, xs, dys):
    p = float(np.float32(p))       # the library takes p as a float32 (keep threshold floor(p 2^16))
    d = O.Dims.from_cfg(cfg)
    ys, gs = [], {}
    for b, (x, dy) in enumerate(zip(xs, dys)):
        y, sv = T.train_forward(x, W, d, p, seed, b)
        g = T.train_backward(dy, W, d, p, sv)
        ys.append(y)
        gs.setdefault("dx", []).append(g["x"])
        for k in W:
            gs["d" + k] = gs.get("d" + k, 0) + g[k]
    gs["dx"] = np.stack(gs["dx"])
    return np.stack(ys), gs


@pytest.mark.parametrize("cfg,p,seed", [(TINY, 0.3, 42), (TINY, 0.0, 1), (DSV2_T, 0.1, 7), (DSV2_T, 0.5, 9),
                                        (DSV2_F, 0.1, 7), (DSV2_F, 0.5, 9), (DSV2_F, 0.0, 2), (DSV2_F3, 0.25, 3),
                                        (DSV2_F1, 0.9, 5), (DSV2_FL, 0.2, 13)],
                         ids=["tiny_p0.3", "tiny_p0", "dsv2_p0.1", "dsv2_p0.5", "flash_p0.1", "flash_p0.5",
                              "flash_p0", "flash_h3_p0.25", "flash_s64_p0.9", "flash_s1024_p0.2"])
def test_train_forward_backward(gu, cfg, p, seed):
    gu.say(f"[train] {cfg.name} p={p} seed={seed} B={cfg.batch} S={cfg.seq}")
    rng = np.random.default_rng(seed)
    xs = [S.make_x(cfg, b, cfg.seq) for b in range(cfg.batch)]
    dys = [rng.standard_normal((cfg.seq, cfg.d_model)).astype(np.float32) for _ in range(cfg.batch)]
    y, g, W = _train(gu, cfg, p, seed, xs, dys)
    y_want, g_want = _oracle(cfg, W, p, seed, xs, dys)
    _close(gu, y, y_want, cfg.dtype, "y")
    for k in sorted(g_want):
        _close(gu, g[k], g_want[k], cfg.dtype, k)


def test_train_forward_without_dropout_is_prefill(gu):
    """p = 0: the training forward returns mla_prefill's output (the same projections and the
    generic attention kernel in place of the flash one: equal within rounding)."""
    cfg = DSV2_T
    lay = gu.Layer(cfg)
    xs = [S.make_x(cfg, b, cfg.seq) for b in range(cfg.batch)]
    y_pre = gu.to_host(lay.prefill(gu.to_dev(np.stack(xs), cfg)))
    y_tr, _, _ = _train(gu, cfg, 0.0, 3, xs, [np.zeros((cfg.seq, cfg.d_model), np.float32)] * cfg.batch)
    gu.assert_close(y_tr, y_pre, cfg.dtype, "train forward p=0 vs prefill")


def test_train_dropout_changes_with_seed(gu):
    cfg = TINY
    xs = [S.make_x(cfg, b, cfg.seq) for b in range(cfg.batch)]
    dys = [np.ones((cfg.seq, cfg.d_model), np.float32)] * cfg.batch
    y1, _, _ = _train(gu, cfg, 0.5, 10, xs, dys)
    y2, _, _ = _train(gu, cfg, 0.5, 10, xs, dys)
    y3, _, _ = _train(gu, cfg, 0.5, 11, xs, dys)
    assert np.array_equal(y1, y2)
    assert not np.allclose(y1, y3)


def test_train_full_shape(gu):
    """The DeepSeek-V2 prefill shape (d_model 5120, 128 heads, r_q 1536, r_kv 512, S=4096) for
    two sequences without dropout (the oracle draws no masks): sixteen query blocks per
    (sequence, head); every gradient against the oracle."""
    cfg = S.CONFIGS["dsv2_prefill"].replace(batch=2)
    gu.say(f"[train-full] {cfg.name} B={cfg.batch} S={cfg.seq}")
    rng = np.random.default_rng(5)
    xs = S.make_x_batch(cfg, [cfg.seq] * cfg.batch, threads=S.host_threads())
    dys = [rng.standard_normal((cfg.seq, cfg.d_model)).astype(np.float32) for _ in range(cfg.batch)]
    y, g, W = _train(gu, cfg, 0.0, 1, xs, dys)
    y_want, g_want = _oracle(cfg, W, 0.0, 1, xs, dys)
    _close(gu, y, y_want, cfg.dtype, "y")
    for k in sorted(g_want):
        _close(gu, g[k], g_want[k], cfg.dtype, k)
