"""GPU-side test helpers: device copies of the seeded inputs and calls through the C ABI.

Numbers compared against the oracle come only from the library's kernels; torch is used
for allocation, host<->device copies and the stream.
"""
from __future__ import annotations

import sys
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import head_latent_attention_dkv_amd as M
import mla_synth as S

RTOL_F32 = 1e-5            # rel-L2 bound for the fp32 workload
RTOL_BF16 = 1e-2           # rel-L2 bound for bf16-in / fp32-accumulate workloads
ATOL_BF16 = 3e-2           # max-abs bound for bf16 workloads


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def assert_close(got, want, dtype: str, what: str):
    r, m = rel_l2(got, want), max_abs(got, want)
    say(f"  {what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert np.all(np.isfinite(np.asarray(got))), f"{what}: non-finite values"
    if dtype == "f32":
        assert r <= RTOL_F32, f"{what}: rel_l2 {r:.3e} > {RTOL_F32}"
    else:
        assert r <= RTOL_BF16, f"{what}: rel_l2 {r:.3e} > {RTOL_BF16}"
        assert m <= ATOL_BF16, f"{what}: max_abs {m:.3e} > {ATOL_BF16}"


def tdtype(cfg) -> torch.dtype:
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, cfg) -> torch.Tensor:
    """float32 host values (bf16-representable for bf16 workloads) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda").to(tdtype(cfg)).contiguous()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class Layer:
    """Device weights + workspace management for one workload."""

    def __init__(self, cfg, prob: Optional[S.Problem] = None):
        self.cfg = cfg
        self.prob = prob if prob is not None else S.make_problem(cfg)
        self.dims = M.dims_from_cfg(cfg)
        assert M.mla_validate(self.dims) == M.MLA_OK
        self.w = {k: to_dev(v, cfg) for k, v in self.prob.weights.items()}
        self.ws_struct = M.weights_struct(self.w)
        self._ws: Dict[int, torch.Tensor] = {}

    def workspace(self, op: int, B: int, S_: int):
        n = M.mla_workspace_bytes(self.dims, op, B, S_)
        key = op
        t = self._ws.get(key)
        if t is None or t.numel() < n:
            t = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
            self._ws[key] = t
        return t, n

    def new_cache(self, max_batch: int, max_seq: int, fill: float = 0.0):
        cfg = self.cfg
        ckv = torch.full((max_batch, max_seq, cfg.r_kv), fill, dtype=tdtype(cfg), device="cuda")
        kr = None
        if cfg.d_rope > 0:
            kr = torch.full((max_batch, max_seq, cfg.d_rope), fill, dtype=tdtype(cfg), device="cuda")
        return ckv, kr

    @staticmethod
    def cache_view(ckv, kr, b0: int, nb: int):
        """mla_cache over sequences b0 .. b0+nb-1 of a larger cache."""
        return M.cache_struct(ckv[b0:b0 + nb], kr[b0:b0 + nb] if kr is not None else None, nb, ckv.shape[1])

    def append(self, x: torch.Tensor, start_pos: Sequence[int], cache_struct) -> None:
        B, T = x.shape[0], x.shape[1]
        sp = torch.tensor(list(start_pos), dtype=torch.int32, device="cuda")
        M.mla_cache_append(self.dims, self.ws_struct, x, B, T, sp, int(max(start_pos)), cache_struct)

    def fill_cache(self, ckv, kr, lens: Sequence[int], threads: int = 8, b0: int = 0) -> None:
        """Write the latents of tokens 0..lens[b]-1 of sequences b0+b (seeded inputs)."""
        from concurrent.futures import ThreadPoolExecutor
        for i0 in range(0, len(lens), threads):
            idx = [i for i in range(i0, min(len(lens), i0 + threads)) if lens[i] > 0]
            with ThreadPoolExecutor(threads) as ex:
                xs = list(ex.map(lambda i: S.make_x(self.cfg, b0 + i, int(lens[i])), idx))
            for i, xh in zip(idx, xs):
                x = to_dev(xh, self.cfg)[None]
                self.append(x, [0], self.cache_view(ckv, kr, b0 + i, 1))

    def prefill(self, x: torch.Tensor, cache_struct=None) -> torch.Tensor:
        B, S_ = x.shape[0], x.shape[1]
        y = torch.empty((B, S_, self.cfg.d_model), dtype=torch.float32, device="cuda")
        ws, n = self.workspace(M.MLA_OP_PREFILL, B, S_)
        M.mla_prefill(self.dims, self.ws_struct, x, B, S_, cache_struct, y, ws, n)
        return y

    def prefill_chunk(self, x: torch.Tensor, start_pos: int, cache_struct) -> torch.Tensor:
        """Continued prefill of x [B][T] at positions start_pos.. over the cached rows below."""
        B, T = x.shape[0], x.shape[1]
        y = torch.empty((B, T, self.cfg.d_model), dtype=torch.float32, device="cuda")
        ws, n = self.workspace(M.MLA_OP_PREFILL_CHUNK, B, start_pos + T)
        M.mla_prefill_chunk(self.dims, self.ws_struct, x, B, T, int(start_pos), cache_struct, y, ws, n)
        return y

    def decode(self, x: torch.Tensor, ctx_len: Sequence[int], cache_struct) -> torch.Tensor:
        B = x.shape[0]
        y = torch.empty((B, self.cfg.d_model), dtype=torch.float32, device="cuda")
        cl = torch.tensor(list(ctx_len), dtype=torch.int32, device="cuda")
        mc = int(max(ctx_len))
        ws, n = self.workspace(M.MLA_OP_DECODE, B, mc)
        M.mla_decode(self.dims, self.ws_struct, x, B, cl, mc, cache_struct, y, ws, n)
        return y
