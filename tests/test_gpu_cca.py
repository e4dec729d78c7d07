"""GPU parity of compressed convolutional attention (CCA / CCGQA) against the fp64 oracle.

[CCA page] frankenstein-transformer docs, ``latent/cca_attn``: ``CCAAttention.forward`` and
``CCGQAAttention.forward`` in decoder mode.  The library's mla_cca_prefill runs on seeded
inputs; the oracle (oracle/cca_oracle.py) recomputes whole sequences.  Sequences of whole 64-token
tiles run attention on the flash prefill kernel, others on the generic one.  Tolerances as for
the MLA workloads: fp32 rel-L2 <= 1e-5; bf16-in / fp32-accumulate rel-L2 <= 1e-2 and
max-abs <= 3e-2 per sequence.  Sizes span several 16-token preparation blocks, 128-query
attention tiles and 64-key tiles with ragged tails.
"""
import numpy as np
import pytest

import mla_synth as S
from oracle import cca_oracle as C

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TINY_CCA = S.CCA_CONFIGS["cca_tiny_fp32"]
TINY_GQA = S.CCA_CONFIGS["ccgqa_tiny_fp32"]
# reduced-width bf16 cases of both workloads (same head widths and group sizes)
CCA_S = S.CCA_CONFIGS["cca"].replace(name="cca_e256_s300", batch=2, seq=300, d_model=256, n_heads=8, n_kv_heads=8)
GQA_S = S.CCA_CONFIGS["ccgqa"].replace(name="ccgqa_e256_s300", batch=2, seq=300, d_model=512, n_heads=8,
                                       n_kv_heads=2)


@pytest.fixture(scope="module")
def gu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gpu_util
    return gpu_util


def _run(gu, cfg, xs):
    import head_latent_attention_dkv_amd as M
    prob = S.make_cca_problem(cfg)
    dims = M.cca_dims_from_cfg(cfg)
    assert M.mla_cca_validate(dims) == M.MLA_OK
    w = {k: gu.to_dev(v, cfg) for k, v in prob.weights.items()}
    B, S_ = len(xs), xs[0].shape[0]
    x = gu.to_dev(np.stack(xs), cfg)
    y = torch.empty((B, S_, cfg.d_model), dtype=torch.float32, device="cuda")
    n = M.mla_cca_workspace_bytes(dims, B, S_)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    M.mla_cca_prefill(dims, M.cca_weights_struct(w, cfg.beta), x, B, S_, y, ws, n)
    return gu.to_host(y), prob


VARIANTS = [
    (TINY_CCA, {}), (TINY_GQA, {}),
    (TINY_GQA, dict(num_conv_layers=1)), (TINY_GQA, dict(num_conv_layers=0, qk_mean=False)),
    (TINY_CCA, dict(value_shift=False, beta=-0.5)),
    (CCA_S, {}), (GQA_S, {}),
    (GQA_S, dict(num_conv_layers=1, qk_mean=False)), (CCA_S, dict(value_shift=False, num_conv_layers=0)),
    (GQA_S.replace(name="ccgqa_dh32", head_dim=32), {}),
    (CCA_S.replace(name="cca_s1", seq=1), {}),
    # whole 64-token tiles: attention on the flash prefill kernel (heads of 32 features padded
    # to 64; 64 and 128 as they are), a partial second 256-query tile
    (CCA_S.replace(name="cca_s320", seq=320), {}),
    (GQA_S.replace(name="ccgqa_s320", seq=320), {}),
    (GQA_S.replace(name="ccgqa_dh128_s256", head_dim=128, seq=256), {}),
    (GQA_S.replace(name="ccgqa_dh32_s64", head_dim=32, seq=64), dict(num_conv_layers=1, value_shift=False)),
    # the longest convolution kernels the library takes, and odd ones (MFMA channel convolution)
    (CCA_S.replace(name="cca_k8_s128", seq=128), dict(conv_kernel_seq=8, conv_kernel_ch=8)),
    (GQA_S.replace(name="ccgqa_k2k5_s192", seq=192), dict(conv_kernel_seq=2, conv_kernel_ch=5)),
]


@pytest.mark.parametrize("cfg,kw", VARIANTS, ids=lambda v: v.name if hasattr(v, "name") else
                         ",".join(f"{k}={w}" for k, w in v.items()) or "page-defaults")
def test_cca_prefill(gu, cfg, kw):
    cfg = cfg.replace(**kw)
    gu.say(f"[cca] {cfg.name} {kw} B={cfg.batch} S={cfg.seq}")
    xs = [S.make_x(cfg, b, cfg.seq) for b in range(cfg.batch)]
    y, prob = _run(gu, cfg, xs)
    for b in range(cfg.batch):
        gu.assert_close(y[b], C.forward(xs[b], prob.weights, cfg), cfg.dtype, f"y b={b}")


@pytest.mark.parametrize("seq", [300, 320], ids=["generic", "flash"])
def test_cca_prefill_is_causal(gu, seq):
    """Perturbing the last tokens leaves every earlier output row unchanged (bitwise: the
    earlier rows' arithmetic does not read the later tokens)."""
    cfg = GQA_S.replace(seq=seq)
    xs = [S.make_x(cfg, b, cfg.seq) for b in range(cfg.batch)]
    y1, _ = _run(gu, cfg, xs)
    xs2 = [x.copy() for x in xs]
    for x in xs2:
        x[250:] = S.round_bf16(x[250:] * -2.0 + 1.0)
    y2, _ = _run(gu, cfg, xs2)
    assert np.array_equal(y1[:, :250], y2[:, :250])
    assert not np.allclose(y1[:, 250:], y2[:, 250:])


@pytest.mark.parametrize("name", ["cca", "ccgqa"])
def test_cca_prefill_full(gu, name):
    """The page-default workloads at full size (B=4, S=2048); the oracle recomputes the first
    and the last sequence whole."""
    cfg = S.CCA_CONFIGS[name]
    gu.say(f"[cca-full] {name} B={cfg.batch} S={cfg.seq}")
    xs = S.make_x_batch(cfg, [cfg.seq] * cfg.batch, threads=S.host_threads())
    y, prob = _run(gu, cfg, xs)
    assert np.all(np.isfinite(y))
    for b in (0, cfg.batch - 1):
        gu.assert_close(y[b], C.forward(xs[b], prob.weights, cfg), cfg.dtype, f"y b={b}")
