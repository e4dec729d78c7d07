"""Seeded synthetic inputs for the MLA workloads.

This module is shared by the fp64 oracle side (tests, bench CPU baseline) and the
GPU side (tests, bench, smoke).  It holds workload shapes, seeded random draws and
bf16 rounding of those draws -- and none of the attention method's arithmetic.

Recipe (every workload):
  * rng = numpy Generator(PCG64(seed)).
  * Weights are drawn first, in the fixed order
        W_DQ, W_UQ, W_QR, W_Q, W_DKV, W_KR, W_UK, W_UV, W_O
    (matrices a family does not have are skipped), each entry N(0, 1/fan_in)
    where fan_in is the matrix's number of input features.  Layout is
    [out_features x in_features], row-major (torch.nn.Linear's weight layout).
    For the partitioned-latent family the key/value up-projections are L dense
    blocks [sub_out x sub_rank] stored back to back (shape [L, sub_out, sub_rank]),
    fan_in = sub_rank; all W_UK blocks are drawn before all W_UV blocks.
  * Ragged context lengths (if any) are drawn next from the same rng:
        rng.integers(lo, hi, batch, endpoint=True).
  * Token activations of sequence b come from a child generator
    PCG64([seed, b + 1]) as x[t, :] ~ N(0, 1), t = 0, 1, ... so that any sequence can
    be regenerated on its own (the oracle streams sequence by sequence).  The key is
    b + 1, not b: numpy's SeedSequence zero-pads its entropy, so [seed, 0] would replay
    the weight stream PCG64(seed) and sequence 0 would be scaled copies of weight rows.
  * bf16 workloads round x and every weight to bf16 with round-to-nearest-even
    before either side sees them; both sides consume the identical values.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

FAMILY_DECOUPLED = "decoupled"   # query latent + decoupled RoPE key shared by heads
FAMILY_FULLROPE = "fullrope"     # RoPE (half-split pairs) on the decompressed q and k
FAMILY_MLRA = "mlra"             # latent split into L disjoint latent heads, no RoPE

WEIGHT_ORDER = ("w_dq", "w_uq", "w_qr", "w_q", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")


@dataclasses.dataclass(frozen=True)
class MLAConfig:
    name: str
    family: str
    mode: str                  # "prefill" or "decode"
    batch: int
    seq: int                   # prefill: S; decode: cached context length (fixed case)
    d_model: int
    n_heads: int
    d_nope: int                # per-head q/k width without the rotary part (= d_v)
    d_rope: int                # decoupled rotary width (0 if none)
    r_kv: int                  # latent rank (total over all latent heads)
    r_q: int                   # query latent rank (0: direct W_Q)
    n_latent_heads: int = 1
    dtype: str = "bf16"        # "f32" or "bf16"
    rope_base: float = 10000.0
    seed: int = 0
    ctx_lo: int = 0            # ragged decode contexts: uniform integers in [ctx_lo, ctx_hi]
    ctx_hi: int = 0

    @property
    def d_v(self) -> int:
        return self.d_nope

    @property
    def ragged(self) -> bool:
        return self.ctx_hi > 0

    def replace(self, **kw) -> "MLAConfig":
        return dataclasses.replace(self, **kw)

    def weight_shapes(self) -> Dict[str, tuple]:
        H, dn, dr, r, rq, dm = (self.n_heads, self.d_nope, self.d_rope, self.r_kv,
                                self.r_q, self.d_model)
        s: Dict[str, tuple] = {}
        if self.family == FAMILY_DECOUPLED:
            if rq > 0:
                s["w_dq"] = (rq, dm)
                s["w_uq"] = (H * dn, rq)
                if dr > 0:
                    s["w_qr"] = (H * dr, rq)
            else:
                if dr > 0:
                    s["w_qr"] = (H * dr, dm)
                s["w_q"] = (H * dn, dm)
            s["w_dkv"] = (r, dm)
            if dr > 0:
                s["w_kr"] = (dr, dm)
            s["w_uk"] = (H * dn, r)
            s["w_uv"] = (H * dn, r)
        elif self.family == FAMILY_FULLROPE:
            s["w_q"] = (H * dn, dm)
            s["w_dkv"] = (r, dm)
            s["w_uk"] = (H * dn, r)
            s["w_uv"] = (H * dn, r)
        elif self.family == FAMILY_MLRA:
            L = self.n_latent_heads
            s["w_q"] = (H * dn, dm)
            s["w_dkv"] = (r, dm)
            s["w_uk"] = (L, H * dn // L, r // L)
            s["w_uv"] = (L, H * dn // L, r // L)
        else:
            raise ValueError(f"unknown family {self.family}")
        s["w_o"] = (dm, H * dn)
        return s


# The five workloads: shapes and value distributions of the pages' models.
CONFIGS: Dict[str, MLAConfig] = {
    # Tiny decoupled-RoPE MLA at the gist's dimensions, fp32, causal prefill.
    "tiny_fp32": MLAConfig("tiny_fp32", FAMILY_DECOUPLED, "prefill", batch=2, seq=8,
                           d_model=8, n_heads=4, d_nope=8, d_rope=4, r_kv=2, r_q=2,
                           dtype="f32", seed=1001),
    # Small-LM MLA, RoPE on the decompressed q/k, causal prefill.
    "small_lm": MLAConfig("small_lm", FAMILY_FULLROPE, "prefill", batch=8, seq=1024,
                          d_model=512, n_heads=8, d_nope=64, d_rope=0, r_kv=256, r_q=0,
                          seed=1002),
    # DeepSeek-V2-shaped single-layer decode over a 4096-token latent + k_R cache.
    "dsv2_decode": MLAConfig("dsv2_decode", FAMILY_DECOUPLED, "decode", batch=64, seq=4096,
                             d_model=5120, n_heads=128, d_nope=128, d_rope=64, r_kv=512,
                             r_q=1536, seed=1003),
    # DeepSeek-V2-shaped single-layer causal prefill.
    "dsv2_prefill": MLAConfig("dsv2_prefill", FAMILY_DECOUPLED, "prefill", batch=4, seq=4096,
                              d_model=5120, n_heads=128, d_nope=128, d_rope=64, r_kv=512,
                              r_q=1536, seed=1004),
    # Partitioned-latent (MLRA) decode, 4 latent heads of rank 128, ragged contexts.
    "mlra_decode": MLAConfig("mlra_decode", FAMILY_MLRA, "decode", batch=128, seq=16384,
                             d_model=2048, n_heads=16, d_nope=128, d_rope=0, r_kv=512,
                             r_q=0, n_latent_heads=4, seed=1005, ctx_lo=512, ctx_hi=16384),
}


# ---------------------------------------------------------------------------
# bf16 rounding of the draws (input preparation, not method arithmetic)
# ---------------------------------------------------------------------------
def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Problem:
    cfg: MLAConfig
    weights: Dict[str, np.ndarray]      # float32 arrays (bf16-representable for bf16 cfgs)
    ctx_lens: np.ndarray                # decode: tokens already cached per sequence

    def x(self, b: int, n_tokens: int) -> np.ndarray:
        return make_x(self.cfg, b, n_tokens)


def make_problem(cfg: MLAConfig) -> Problem:
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    shapes = cfg.weight_shapes()
    weights: Dict[str, np.ndarray] = {}
    for name in WEIGHT_ORDER:
        if name not in shapes:
            continue
        shp = shapes[name]
        fan_in = shp[-1]
        w = rng.standard_normal(shp, dtype=np.float32)
        w *= np.float32(1.0 / np.sqrt(fan_in))
        weights[name] = _finish(w, cfg.dtype)
    if cfg.ragged:
        ctx = rng.integers(cfg.ctx_lo, cfg.ctx_hi, cfg.batch, endpoint=True).astype(np.int64)
    else:
        ctx = np.full(cfg.batch, cfg.seq, dtype=np.int64)
    return Problem(cfg, weights, ctx)


def make_x(cfg: MLAConfig, b: int, n_tokens: int) -> np.ndarray:
    """Activations of sequence b, tokens 0..n_tokens-1 (prefixes are stable)."""
    rng = np.random.Generator(np.random.PCG64([cfg.seed, b + 1]))
    return _finish(rng.standard_normal((n_tokens, cfg.d_model), dtype=np.float32), cfg.dtype)


def make_x_batch(cfg: MLAConfig, lens: Sequence[int], threads: int = 8) -> List[np.ndarray]:
    """Activations for several sequences, generated in parallel threads."""
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda bl: make_x(cfg, bl[0], int(bl[1])), enumerate(lens)))


# ---------------------------------------------------------------------------
# Compressed convolutional attention (CCA / CCGQA) workloads
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class CCAConfig:
    """Shapes of the CCA page's layers.  CCA is the case n_kv_heads == n_heads.

    Weights (drawn in this order, each N(0, 1/fan_in), [out x in] row-major):
      w_qk     [(Hq + Hkv) dh][E]      packed q / k down-projection
      w_v      [Hkv dh][E]             value projection; with value_shift its first
                                       Hkv dh / 2 rows are the current-token projection
                                       and the rest the previous-token projection
      conv_seq [(Hq + Hkv) dh][k_seq]  depth-wise sequence convolution (fan_in k_seq)
      conv_ch  [(Hq + Hkv) dh][dh][k_ch] head-wise grouped convolution (fan_in dh k_ch)
      w_o      [E][Hq dh]              output up-projection
    Activations as for MLAConfig (child generator PCG64([seed, b + 1])).  The key
    temperature beta is a fixed value of the workload (the page initialises it to 0).
    """
    name: str
    batch: int
    seq: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    num_conv_layers: int = 2
    conv_kernel_seq: int = 4
    conv_kernel_ch: int = 3
    qk_mean: bool = True
    value_shift: bool = True
    beta: float = 0.25
    dtype: str = "bf16"
    rope_base: float = 10000.0
    seed: int = 0

    def replace(self, **kw) -> "CCAConfig":
        return dataclasses.replace(self, **kw)

    @property
    def q_latent(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_latent(self) -> int:
        return self.n_kv_heads * self.head_dim

    def weight_shapes(self) -> Dict[str, tuple]:
        cp = self.q_latent + self.kv_latent
        return {"w_qk": (cp, self.d_model), "w_v": (self.kv_latent, self.d_model),
                "conv_seq": (cp, self.conv_kernel_seq),
                "conv_ch": (cp, self.head_dim, self.conv_kernel_ch),
                "w_o": (self.d_model, self.q_latent)}


CCA_WEIGHT_ORDER = ("w_qk", "w_v", "conv_seq", "conv_ch", "w_o")

# Workloads at the page's defaults: CCA with compression C = 4 (latent E/4) and CCGQA with
# C1 = 2, C2 = 8 and a quarter of the heads as KV heads; two convolutions (k_seq 4, k_ch 3),
# q-k-mean and value shift on.
CCA_CONFIGS: Dict[str, CCAConfig] = {
    "cca_tiny_fp32": CCAConfig("cca_tiny_fp32", batch=2, seq=9, d_model=16, n_heads=4, n_kv_heads=4,
                               head_dim=4, dtype="f32", beta=0.3, seed=1011),
    "ccgqa_tiny_fp32": CCAConfig("ccgqa_tiny_fp32", batch=2, seq=9, d_model=16, n_heads=4, n_kv_heads=2,
                                 head_dim=4, dtype="f32", beta=0.3, seed=1012),
    "cca": CCAConfig("cca", batch=4, seq=2048, d_model=2048, n_heads=16, n_kv_heads=16, head_dim=32,
                     seed=1013),
    "ccgqa": CCAConfig("ccgqa", batch=4, seq=2048, d_model=2048, n_heads=16, n_kv_heads=4, head_dim=64,
                       seed=1014),
}


@dataclasses.dataclass
class CCAProblem:
    cfg: CCAConfig
    weights: Dict[str, np.ndarray]


def make_cca_problem(cfg: CCAConfig) -> CCAProblem:
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    weights: Dict[str, np.ndarray] = {}
    for name, shp in zip(CCA_WEIGHT_ORDER, (cfg.weight_shapes()[n] for n in CCA_WEIGHT_ORDER)):
        fan_in = int(np.prod(shp[1:]))
        w = rng.standard_normal(shp, dtype=np.float32)
        w *= np.float32(1.0 / np.sqrt(fan_in))
        weights[name] = _finish(w, cfg.dtype)
    return CCAProblem(cfg, weights)


def scaled(cfg: MLAConfig, **kw) -> MLAConfig:
    """Same family and structure at other sizes (for quick parity cases)."""
    return cfg.replace(**kw)


def host_threads() -> int:
    import os
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


__all__ = [
    "MLAConfig", "CONFIGS", "Problem", "make_problem", "make_x", "make_x_batch",
    "round_bf16", "bf16_bits", "scaled", "host_threads", "WEIGHT_ORDER",
    "FAMILY_DECOUPLED", "FAMILY_FULLROPE", "FAMILY_MLRA",
    "CCAConfig", "CCA_CONFIGS", "CCAProblem", "make_cca_problem", "CCA_WEIGHT_ORDER",
]
