"""mla_decode_attention_noalloc (no workspace argument; the library's per-GPU scratch array)
against mla_decode_attention (caller-owned workspace) on the same inputs: two calls in a row,
the second smaller, for the DeepSeek-V2 decode shape and the MLRA shape.  The two entry points
run the same kernels with the same split plan, so their outputs must be identical; each is
also within the bf16 tolerance of the other (rel-L2 <= 1e-2, max-abs <= 3e-2)."""
import numpy as np
import pytest

import mla_synth as S

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DSV2 = S.CONFIGS["dsv2_decode"].replace(d_model=512)
MLRA = S.CONFIGS["mlra_decode"].replace(d_model=512)


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


def _inputs(gu, cfg, ctx, seed):
    rng = np.random.default_rng(seed)
    B, H, L = len(ctx), cfg.n_heads, cfg.n_latent_heads
    rb = cfg.r_kv // L
    max_seq = max(ctx) + 3
    dev = lambda a: gu.to_dev(S.round_bf16(a.astype(np.float32)), cfg)
    ckv = dev(rng.standard_normal((B, max_seq, cfg.r_kv)))
    kr = dev(rng.standard_normal((B, max_seq, cfg.d_rope))) if cfg.d_rope else None
    q_lat = dev(rng.standard_normal((B, H, rb)) * 0.5)
    q_rope = dev(rng.standard_normal((B, H, cfg.d_rope)) * 0.5) if cfg.d_rope else None
    return ckv, kr, q_lat, q_rope, max_seq


@pytest.mark.parametrize("cfg,calls", [
    (DSV2, [[40, 513, 999, 2047], [5, 300]]),
    (MLRA, [[5, 1030, 4000], [0, 77]]),
], ids=["dsv2", "mlra"])
def test_noalloc_matches_workspace_entry(gu, cfg, calls):
    import head_latent_attention_dkv_amd as M
    dims = M.dims_from_cfg(cfg)
    H, rb = cfg.n_heads, cfg.r_kv // cfg.n_latent_heads
    for i, ctx in enumerate(calls):
        gu.say(f"[noalloc] {cfg.name} call {i} ctx={ctx}")
        B = len(ctx)
        ckv, kr, q_lat, q_rope, max_seq = _inputs(gu, cfg, ctx, 100 + i)
        cache = M.cache_struct(ckv, kr, B, max_seq)
        cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
        n = M.mla_workspace_bytes(dims, M.MLA_OP_DECODE_ATTENTION, B, max(ctx))
        assert 0 < n <= M.mla_decode_attention_noalloc_max_bytes()
        ws = torch.empty(n, dtype=torch.uint8, device="cuda")
        z_ref = torch.full((B, H, rb), float("nan"), dtype=gu.tdtype(cfg), device="cuda")
        z = torch.full((B, H, rb), float("nan"), dtype=gu.tdtype(cfg), device="cuda")
        M.mla_decode_attention(dims, q_lat, q_rope, B, cl, max(ctx), cache, z_ref, ws, n)
        M.mla_decode_attention_noalloc(dims, q_lat, q_rope, B, cl, max(ctx), cache, z)
        torch.cuda.synchronize()
        gu.assert_close(gu.to_host(z), gu.to_host(z_ref), cfg.dtype, f"noalloc vs workspace, call {i}")
        assert torch.equal(z, z_ref), f"call {i}: outputs differ"


def test_noalloc_rejects_shapes_beyond_its_scratch(gu):
    import head_latent_attention_dkv_amd as M
    cfg = S.CONFIGS["dsv2_decode"]
    dims = M.dims_from_cfg(cfg)
    B, max_ctx = 512, 100
    assert M.mla_workspace_bytes(dims, M.MLA_OP_DECODE_ATTENTION, B, max_ctx) > M.mla_decode_attention_noalloc_max_bytes()
    one = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    cl = torch.zeros(B, dtype=torch.int32, device="cuda")
    cache = M.cache_struct(one, one, B, max_ctx + 1)
    with pytest.raises(M.MLAError) as e:
        M.mla_decode_attention_noalloc(dims, one, one, B, cl, max_ctx, cache, one)
    assert e.value.status == M.MLA_ERR_WORKSPACE
