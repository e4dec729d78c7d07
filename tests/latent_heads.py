"""One MLRA latent head as a workload of its own (test infrastructure).

The MLRA page splits the latent into L latent heads; head h reads latent block
g = h // (H/L) only.  Latent head g with its H/L query heads is therefore an MLRA layer
with L = 1 and rank r/L: the rows of W_Q for its heads, the rows of W_DKV for its block,
its dense W_UK / W_UV blocks, and the columns of W_O for its heads.  The output
projection is linear in the concatenated head outputs, so the layer's output is the sum
over g of these per-head-block outputs (the sum a latent-head-parallel decode would
all-reduce).
"""
import numpy as np

import mla_synth as S


def block_cfg(cfg: S.MLAConfig) -> S.MLAConfig:
    L = cfg.n_latent_heads
    return cfg.replace(name=f"{cfg.name}_lhead", n_heads=cfg.n_heads // L, r_kv=cfg.r_kv // L,
                       n_latent_heads=1)


def block_problem(prob: S.Problem, g: int) -> S.Problem:
    cfg = prob.cfg
    assert cfg.family == S.FAMILY_MLRA
    L, H, dn = cfg.n_latent_heads, cfg.n_heads, cfg.d_nope
    hb, rb = H // L, cfg.r_kv // L
    w = prob.weights
    wg = {
        "w_q": np.ascontiguousarray(w["w_q"][g * hb * dn:(g + 1) * hb * dn]),
        "w_dkv": np.ascontiguousarray(w["w_dkv"][g * rb:(g + 1) * rb]),
        "w_uk": np.ascontiguousarray(w["w_uk"][g:g + 1]),
        "w_uv": np.ascontiguousarray(w["w_uv"][g:g + 1]),
        "w_o": np.ascontiguousarray(w["w_o"][:, g * hb * dn:(g + 1) * hb * dn]),
    }
    return S.Problem(block_cfg(cfg), wg, prob.ctx_lens)
