"""Benchmark of the MLA hot path on one MI355X.

One "step" is one whole mla_decode call of the DeepSeek-V2-shaped decode workload
(B=64 sequences, 4096 cached tokens + 1 new token each, H=128, latent 512 + rotary 64,
query latent 1536, d_model 5120, absorbed form): append, query path, absorbed query,
split-context latent attention, the combine fused with W_UV, and W_O.  `value` is the latent-cache
bytes that step streams (sum over sequences of (ctx+1) * (512+64) * 2 B = 302.06 MB)
divided by the measured step time.  The latent cache rotates between two copies
(604 MB > the 256 MB Infinity Cache) so that every step reads it from HBM.  All inputs
are resident in device memory before the timed region; HIP events on the library's
stream bracket the timed steps, with a device synchronisation on both sides.

The JSON line also carries:
  * roofline -- the step's dominant unit, mla_decode_attention (split-context attention
    kernel + combine kernel), timed live with HIP events, against 8 TB/s HBM; `traffic`
    is the HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE counters scaled by
    a copy kernel of known size (profiles/dsv2_decode_attention_traffic.json, used only
    while the kernel sources match the digest stored with it);
  * decode_step -- the whole call against HBM including the 298 MB of weights it reads;
  * prefill -- the DeepSeek-V2-shaped causal prefill (B=4, S=4096): whole mla_prefill and
    the attention core unit mla_prefill_attention against the 2.5 PFLOP/s bf16 MFMA peak;
  * mlra_decode -- the MLRA decode (B=128, ragged contexts, 4 latent heads of rank 128);
  * mlra_latent_head_decode -- one of those latent heads on its own (rank 128, its 4 query
    heads, the same contexts): what one GPU of a latent-head-parallel decode runs;
  * small_lm_prefill -- the small-LM prefill (B=8, S=1024);
  * cpu_baseline -- the fp64 CPU oracle timed on the host on a bounded sample of the
    decode workload (whole sequences, ~15 s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only PART]
       python bench.py --summarize DIR     (profile summaries from rocprofv3 output)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import mla_synth as S  # noqa: E402

METRIC = "MLA decode latent-cache GB/s + prefill TFLOP/s (1 MI355X, % roofline)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PROFILES = os.path.join(ROOT, "profiles")


_PROBLEMS = {}


def problem(cfg):
    """Seeded weights of a workload, drawn once per process (the draw takes seconds at d_model 5120)."""
    if cfg not in _PROBLEMS:
        _PROBLEMS[cfg] = S.make_problem(cfg)
    return _PROBLEMS[cfg]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_threads():
    return S.host_threads()


# ---------------------------------------------------------------------------
# Device setup helpers (allocation and copies only; all compute is in libmla)
# ---------------------------------------------------------------------------
class Dev:
    def __init__(self, cfg):
        import torch
        import head_latent_attention_dkv_amd as M
        self.torch, self.M = torch, M
        self.cfg = cfg
        self.prob = problem(cfg)
        self.dims = M.dims_from_cfg(cfg)
        self.dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.w = {k: self.up(v) for k, v in self.prob.weights.items()}
        self.wst = M.weights_struct(self.w)

    def up(self, a):
        t = self.torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
        return t.to("cuda").to(self.dt).contiguous()

    def workspace(self, op, B, S_):
        n = self.M.mla_workspace_bytes(self.dims, op, B, S_)
        return self.torch.empty(max(n, 256), dtype=self.torch.uint8, device="cuda"), n

    def new_cache(self, B, max_seq):
        cfg, torch = self.cfg, self.torch
        ckv = torch.zeros((B, max_seq, cfg.r_kv), dtype=self.dt, device="cuda")
        kr = torch.zeros((B, max_seq, cfg.d_rope), dtype=self.dt, device="cuda") if cfg.d_rope else None
        return ckv, kr

    def fill(self, ckv, kr, lens, keep_last=True):
        """Cache rows 0..lens[b]-1 from the seeded inputs; returns the new-token rows."""
        from concurrent.futures import ThreadPoolExecutor
        torch, M = self.torch, self.M
        nt = host_threads()
        last = np.zeros((len(lens), self.cfg.d_model), np.float32)
        for i0 in range(0, len(lens), nt):
            idx = list(range(i0, min(len(lens), i0 + nt)))
            with ThreadPoolExecutor(nt) as ex:
                xs = list(ex.map(lambda b: S.make_x(self.cfg, b, int(lens[b]) + 1), idx))
            for b, x in zip(idx, xs):
                last[b] = x[-1]
                n = int(lens[b])
                if n == 0:
                    continue
                xd = self.up(x[:n])[None]
                sp = torch.zeros(1, dtype=torch.int32, device="cuda")
                cs = M.cache_struct(ckv[b:b + 1], kr[b:b + 1] if kr is not None else None, 1, ckv.shape[1])
                M.mla_cache_append(self.dims, self.wst, xd, 1, n, sp, 0, cs)
            del xs
        torch.cuda.synchronize()
        return last


# Per-call spread (a second loop with an event after every call).  Off for `--only` runs,
# whose rocprofv3 traces then hold back-to-back calls only, as the timed loop runs them.
PER_CALL_STATS = True


# Untimed calls before every timed loop run for at least this long (after the `warmup` calls),
# so that the loop starts at the clock the GPU holds under that load: a loop of a few short
# calls right after a phase of other work otherwise times part of the clock ramp.
MIN_WARM_S = 0.1


def timed(torch, fn, steps, warmup, stats=None):
    """Average ms per call of fn(i) over `steps` calls after `warmup` calls (and at least
    MIN_WARM_S seconds of untimed calls).

    HIP events on the current stream (the stream the library launches on) bracket the
    timed calls, with a device synchronisation on both sides; nothing else is enqueued
    between the calls (an event record between calls adds a few microseconds of its own).
    When `stats` is a dict, a second loop of `steps` calls with an event after each call
    gives the per-call median / p10 / p90 that go into it.
    """
    if steps <= 0:
        return float("nan")
    i = 0
    for i in range(warmup):
        fn(i)
    i = warmup
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < MIN_WARM_S:
        for _ in range(4):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for j in range(steps):
        fn(i + j)
    e1.record()
    torch.cuda.synchronize()
    i += steps
    ms = e0.elapsed_time(e1) / steps
    if stats is not None and PER_CALL_STATS:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for j in range(steps):
            fn(i + j)
            ev[j + 1].record()
        torch.cuda.synchronize()
        per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
        stats.update({"median_ms": float(np.median(per)), "p10_ms": float(np.percentile(per, 10)),
                      "p90_ms": float(np.percentile(per, 90))})
    return ms


# Sources of each measured kernel unit (a stored counter measurement is valid only for them).
UNIT_SOURCES = {
    "dsv2_decode_attention": ("decode_fast.hip", "decode.hip", "lds_dma.h", "common.h", "internal.h"),
    "dsv2_prefill_attention": ("prefill_fast.hip", "prefill.hip", "gemm.hip", "gemm_big.hip", "gemm_epilogue.h",
                               "lds_dma.h", "common.h", "internal.h"),
    "mlra_decode_attention": ("decode_fast.hip", "decode.hip", "lds_dma.h", "common.h", "internal.h"),
    "mlra_latent_head_decode_attention": ("decode_fast.hip", "decode.hip", "lds_dma.h", "common.h", "internal.h"),
}


def src_digest(*files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "head_latent_attention_dkv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(name, digest):
    """HBM bytes per launch measured by rocprofv3 counters for kernel unit `name`, if the
    stored measurement was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{name}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("src_digest") != digest:
        return None
    return rec.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------
# one MLRA latent head (L = 1, rank r/L, H/L query heads) as a workload of its own
MLRA_LATENT_HEAD = S.CONFIGS["mlra_decode"].replace(name="mlra_latent_head", n_heads=4, r_kv=128, n_latent_heads=1)


def bench_decode(cfg, steps, warmup, copies=2, attention_steps=None, ctx_from=None):
    torch = __import__("torch")
    d = Dev(cfg)
    M = d.M
    B = cfg.batch
    ctx = [int(c) for c in (problem(ctx_from).ctx_lens if ctx_from is not None else d.prob.ctx_lens)]
    max_ctx = max(ctx)
    max_seq = max_ctx + 8
    log(f"[bench] {cfg.name}: filling latent cache ({sum(ctx)} tokens)")
    caches = [d.new_cache(B, max_seq)]
    last = d.fill(*caches[0], ctx)
    for _ in range(copies - 1):
        caches.append(tuple(t.clone() if t is not None else None for t in caches[0]))
    cstructs = [M.cache_struct(ck, kr, B, max_seq) for ck, kr in caches]
    x = d.up(last)
    cl = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    y = torch.empty((B, cfg.d_model), dtype=torch.float32, device="cuda")
    ws, nws = d.workspace(M.MLA_OP_DECODE, B, max_ctx)
    cache_bytes = sum((c + 1) * (cfg.r_kv + cfg.d_rope) for c in ctx) * 2
    weight_bytes = sum(v.size for v in d.prob.weights.values()) * 2

    def step(i):
        M.mla_decode(d.dims, d.wst, x, B, cl, max_ctx, cstructs[i % copies], y, ws, nws)

    # dominant kernel unit: split-context latent attention + combine (timed first, as its
    # rocprofv3 summary times it: right after the cache fill)
    H, L = cfg.n_heads, cfg.n_latent_heads
    rb = cfg.r_kv // L
    g = torch.Generator(device="cpu").manual_seed(cfg.seed)
    q_lat = (torch.randn((B, H, rb), generator=g) * 0.6).to(d.dt).cuda()
    q_rope = (torch.randn((B, H, cfg.d_rope), generator=g) * 0.6).to(d.dt).cuda() if cfg.d_rope else None
    z = torch.empty((B, H, rb), dtype=d.dt, device="cuda")
    wsa, nwsa = d.workspace(M.MLA_OP_DECODE_ATTENTION, B, max_ctx)

    def att(i):
        M.mla_decode_attention(d.dims, q_lat, q_rope, B, cl, max_ctx, cstructs[i % copies], z, wsa, nwsa)

    log(f"[bench] {cfg.name}: timing mla_decode_attention")
    st_att = {}
    ms_att = timed(torch, att, attention_steps or steps, warmup, st_att)
    log(f"[bench] {cfg.name}: timing mla_decode")
    st_call = {}
    ms = timed(torch, step, steps, warmup, st_call)

    # the same step replayed from HIP graphs (one per cache copy): the launches of the
    # step's kernels are recorded once
    ms_graph, st_graph = float("nan"), {}
    if steps > 0:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for i in range(copies):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(i)
            graphs.append(gr)
        log(f"[bench] {cfg.name}: timing mla_decode replayed from a graph")
        ms_graph = timed(torch, lambda i: graphs[i % copies].replay(), steps, warmup, st_graph)
        del graphs

    res = {
        "call_stats": st_call, "attention_stats": st_att, "ms_per_call_graph": ms_graph, "graph_stats": st_graph,
        "workload": cfg.name, "batch": B, "ctx_total": int(sum(ctx)), "max_ctx": max_ctx,
        "ms_per_call": ms, "cache_bytes": int(cache_bytes), "weight_bytes": int(weight_bytes),
        "cache_GBps_call": cache_bytes / ms / 1e6,
        "call_GBps_incl_weights": (cache_bytes + weight_bytes) / ms / 1e6,
        "attention_ms": ms_att, "attention_GBps": cache_bytes / ms_att / 1e6,
    }
    del caches, cstructs
    torch.cuda.empty_cache()
    return res, d


def bench_prefill(cfg, steps, warmup, parts=("call", "attention", "chunk")):
    torch = __import__("torch")
    d = Dev(cfg)
    M = d.M
    B, S_ = cfg.batch, cfg.seq
    log(f"[bench] {cfg.name}: inputs")
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(host_threads()) as ex:
        xs = list(ex.map(lambda b: S.make_x(cfg, b, S_), range(B)))
    x = d.up(np.stack(xs))
    del xs
    ckv, kr = d.new_cache(B, S_)
    cs = M.cache_struct(ckv, kr, B, S_)
    y = torch.empty((B, S_, cfg.d_model), dtype=torch.float32, device="cuda")
    ws, nws = d.workspace(M.MLA_OP_PREFILL, B, S_)

    def call(i):
        M.mla_prefill(d.dims, d.wst, x, B, S_, cs, y, ws, nws)

    # the latent cache must hold the workload's rows (a zero cache gives all-zero keys and
    # values, whose products draw less power and run at a higher clock)
    call(0)
    torch.cuda.synchronize()
    H, dn, dr, dv = cfg.n_heads, cfg.d_nope, cfg.d_rope, cfg.d_v
    g = torch.Generator(device="cpu").manual_seed(cfg.seed)
    q = torch.randn((B, S_, H, dn + dr), generator=g).to(d.dt).cuda()
    o = torch.empty((B, S_, H, dv), dtype=d.dt, device="cuda")
    wsa, nwsa = d.workspace(M.MLA_OP_PREFILL_ATTENTION, B, S_)

    def att(i):
        M.mla_prefill_attention(d.dims, d.wst, q, B, S_, cs, o, wsa, nwsa)

    # the attention unit is timed first, on its own (as its rocprofv3 summary times it): a
    # loop of whole-layer calls before it leaves the clock lower for a while
    log(f"[bench] {cfg.name}: timing mla_prefill_attention")
    st_att = {}
    ms_att = timed(torch, att, steps, warmup, st_att)
    st_call = {}
    ms = float("nan")
    if "call" in parts:
        log(f"[bench] {cfg.name}: timing mla_prefill")
        ms = timed(torch, call, steps, warmup, st_call)
    core = 2.0 * B * H * (S_ * (S_ + 1) / 2) * (dn + dr + dv)
    kvup = 2.0 * B * S_ * cfg.r_kv * H * (dn + dv) / cfg.n_latent_heads
    w = d.prob.weights
    proj = 2.0 * B * S_ * sum(v.size for k, v in w.items() if k not in ("w_uk", "w_uv"))
    layer = core + kvup + proj
    res = {
        "call_stats": st_call, "attention_stats": st_att,
        "workload": cfg.name, "batch": B, "seq": S_, "ms_per_call": ms,
        "layer_flop": layer, "layer_TFLOPs": layer / ms / 1e9,
        "attention_ms": ms_att, "attention_flop": core + kvup,
        "attention_TFLOPs": (core + kvup) / ms_att / 1e9,
    }
    # continued prefill: the last quarter of each sequence over the cached first three
    # quarters (the cache already holds every row; the call rewrites rows start.. with the
    # same values)
    start, T = (3 * S_ // 4) // 64 * 64, S_ - (3 * S_ // 4) // 64 * 64
    if 0 < start < S_ and "chunk" in parts:
        xc = x[:, start:].contiguous()
        yc = torch.empty((B, T, cfg.d_model), dtype=torch.float32, device="cuda")
        wsc, nwsc = d.workspace(M.MLA_OP_PREFILL_CHUNK, B, S_)

        def chunk(i):
            M.mla_prefill_chunk(d.dims, d.wst, xc, B, T, start, cs, yc, wsc, nwsc)

        log(f"[bench] {cfg.name}: timing mla_prefill_chunk (start {start}, {T} new tokens)")
        st_chunk = {}
        ms_chunk = timed(torch, chunk, steps, warmup, st_chunk)
        core_c = 2.0 * B * H * ((S_ * (S_ + 1) - start * (start + 1)) / 2) * (dn + dr + dv)
        proj_c = 2.0 * B * T * sum(v.size for k, v in w.items() if k not in ("w_uk", "w_uv"))
        flop_c = core_c + kvup + proj_c
        res["chunk"] = {"start": start, "new_tokens": T, "ms_per_call": ms_chunk, "stats": st_chunk,
                        "flop": flop_c, "TFLOPs": flop_c / ms_chunk / 1e9,
                        "new_tokens_per_s": B * T / ms_chunk * 1e3}
    return res


def bench_cca(cfg, steps, warmup):
    """mla_cca_prefill on the page-default CCA / CCGQA workload (B=4, S=2048)."""
    torch = __import__("torch")
    import head_latent_attention_dkv_amd as M
    prob = S.make_cca_problem(cfg)
    dims = M.cca_dims_from_cfg(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    w = {k: torch.from_numpy(np.ascontiguousarray(v, np.float32)).to("cuda").to(dt) for k, v in prob.weights.items()}
    wst = M.cca_weights_struct(w, cfg.beta)
    B, S_ = cfg.batch, cfg.seq
    xs = S.make_x_batch(cfg, [S_] * B, threads=host_threads())
    x = torch.from_numpy(np.stack(xs)).to("cuda").to(dt)
    y = torch.empty((B, S_, cfg.d_model), dtype=torch.float32, device="cuda")
    n = M.mla_cca_workspace_bytes(dims, B, S_)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")

    def call(i):
        M.mla_cca_prefill(dims, wst, x, B, S_, y, ws, n)

    log(f"[bench] {cfg.name}: timing mla_cca_prefill")
    st = {}
    ms = timed(torch, call, steps, warmup, st)
    Hq, Hkv, dh, E = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_model
    rows = B * S_
    proj = 2.0 * rows * E * (Hq * dh + 2 * Hkv * dh) + 2.0 * rows * Hq * dh * E
    conv = 2.0 * rows * (Hq + Hkv) * dh * (cfg.conv_kernel_seq + dh * cfg.conv_kernel_ch)
    core = 2.0 * B * Hq * (S_ * (S_ + 1) / 2) * (2 * dh)
    flop = proj + conv + core
    return {"workload": cfg.name, "ms_per_call": ms, "timing": st, "flop": flop, "TFLOPs": flop / ms / 1e9,
            "frac_of_mfma_peak": flop / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, "attention_core_flop": core,
            "tokens_per_s": rows / (ms * 1e-3)}


def bench_train(cfg, steps, warmup, p=0.1, seed=1234):
    """One training step of the DeepSeek-V2-shaped layer: mla_train_forward (dropout p on the
    attention weights) then mla_train_backward for dy ~ N(0, 1)."""
    torch = __import__("torch")
    d = Dev(cfg)
    M = d.M
    B, S_ = cfg.batch, cfg.seq
    xs = S.make_x_batch(cfg, [S_] * B, threads=host_threads())
    x = d.up(np.stack(xs))
    del xs
    g = torch.Generator(device="cpu").manual_seed(cfg.seed)
    dy = torch.randn((B, S_, cfg.d_model), generator=g).cuda()
    y = torch.empty((B, S_, cfg.d_model), dtype=torch.float32, device="cuda")
    ns, nw = M.mla_train_saved_bytes(d.dims, B, S_), M.mla_train_workspace_bytes(d.dims, B, S_)
    saved = torch.empty(ns, dtype=torch.uint8, device="cuda")
    ws = torch.empty(nw, dtype=torch.uint8, device="cuda")
    grads = {"dx": torch.empty((B, S_, cfg.d_model), dtype=torch.float32, device="cuda")}
    grads.update({"d" + k: torch.empty(v.shape, dtype=torch.float32, device="cuda") for k, v in d.prob.weights.items()})
    gst = M.grads_struct(grads)

    def fwd(i):
        M.mla_train_forward(d.dims, d.wst, x, B, S_, p, seed, y, saved, ns)

    def bwd(i):
        M.mla_train_backward(d.dims, d.wst, x, B, S_, p, seed, dy, saved, ns, gst, ws, nw)

    log(f"[bench] {cfg.name}: timing mla_train_forward / mla_train_backward (p={p})")
    st_f, st_b = {}, {}
    ms_f = timed(torch, fwd, steps, warmup, st_f)
    ms_b = timed(torch, bwd, steps, warmup, st_b)
    w = d.prob.weights
    H, dn, dr, dv = cfg.n_heads, cfg.d_nope, cfg.d_rope, cfg.d_v
    core = 2.0 * B * H * (S_ * (S_ + 1) / 2) * (dn + dr + dv)
    proj = 2.0 * B * S_ * sum(v.size for v in w.values())
    fwd_flop = core + proj
    bwd_flop = 2.0 * fwd_flop          # two products per forward product (input and weight gradients)
    return {"workload": f"{cfg.name} training step (dropout p={p}), B={B}, S={S_}", "fwd_ms": ms_f, "bwd_ms": ms_b,
            "fwd_timing": st_f, "bwd_timing": st_b, "fwd_flop": fwd_flop, "bwd_flop": bwd_flop,
            "fwd_TFLOPs": fwd_flop / ms_f / 1e9, "bwd_TFLOPs": bwd_flop / ms_b / 1e9,
            "step_TFLOPs": (fwd_flop + bwd_flop) / (ms_f + ms_b) / 1e9,
            "frac_of_mfma_peak": (fwd_flop + bwd_flop) / (ms_f + ms_b) / 1e9 / MFMA_BF16_PEAK_TFLOPS,
            "saved_bytes": ns, "workspace_bytes": nw,
            "tokens_per_s": B * S_ / ((ms_f + ms_b) * 1e-3)}


def cpu_baseline(cfg, budget_s=15.0, max_seqs=64):
    """fp64 oracle on a bounded sample of the decode workload (whole sequences)."""
    from oracle import mla_oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 0) for i in info if i.get("user_api") == "blas"] or [0])
    except Exception:  # pragma: no cover
        cores = 0
    prob = problem(cfg)
    d = O.Dims.from_cfg(cfg)
    done, t_tot, nbytes = 0, 0.0, 0
    while done < max_seqs and (t_tot < budget_s or done == 0):
        b = done
        n = int(prob.ctx_lens[b]) + 1
        x = S.make_x(cfg, b, n)
        t0 = time.perf_counter()
        O.decode(x, prob.weights, d)
        t_tot += time.perf_counter() - t0
        nbytes += n * (cfg.r_kv + cfg.d_rope) * 2
        done += 1
    return {"value": nbytes / t_tot / 1e9, "unit": "GB/s", "cores": int(cores or host_threads()),
            "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences of {cfg.name} (fp64 numpy decode step with "
                      f"explicit K/V up-projection), {t_tot:.1f} s; value = their latent-cache bytes / time"}


def cpu_baseline_prefill(cfg, budget_s=12.0, rows_per_seq=256):
    """fp64 oracle on a bounded sample of the prefill workload: for each sampled sequence,
    its whole explicit K/V up-projection and the causal attention of `rows_per_seq` query rows
    spread over the sequence (the oracle's forward restricted to those rows).  The value counts
    the same algorithmic flops as the GPU attention unit for that sample."""
    from oracle import mla_oracle as O
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([i.get("num_threads", 0) for i in info if i.get("user_api") == "blas"] or [0])
    except Exception:  # pragma: no cover
        cores = 0
    prob = problem(cfg)
    d = O.Dims.from_cfg(cfg)
    S_, H = cfg.seq, cfg.n_heads
    dq, dv = cfg.d_nope + cfg.d_rope, cfg.d_v
    rows = np.linspace(0, S_ - 1, rows_per_seq).round().astype(int)
    kvup = 2.0 * S_ * cfg.r_kv * H * (cfg.d_nope + dv) / cfg.n_latent_heads
    core = float(sum(2.0 * H * (r + 1) * (dq + dv) for r in rows))
    done, t_tot = 0, 0.0
    while done < cfg.batch and (t_tot < budget_s or done == 0):
        x = S.make_x(cfg, done, S_)
        t0 = time.perf_counter()
        O.forward(x, prob.weights, d, q_rows=rows)
        t_tot += time.perf_counter() - t0
        done += 1
    flop = done * (kvup + core)
    return {"value": flop / t_tot / 1e12, "unit": "TFLOP/s", "cores": int(cores or host_threads()),
            "kind": "oracle",
            "sample": f"{done} of {cfg.batch} sequences of {cfg.name}: explicit K/V up-projection of all "
                      f"{S_} rows + causal attention of {rows_per_seq} query rows each (fp64 numpy), "
                      f"{t_tot:.1f} s; value = that sample's attention-unit flops / time"}


# Units the profile summaries cover: the `bench.py --only` mode that runs the unit alone,
# the kernels one call launches (name fragments, in launch order), the algorithmic work of one
# call and its peak, and the summary file.
PROFILE_UNITS = {
    "decode_attention": dict(title="mla_decode_attention, DeepSeek-V2 decode (B=64, 4096 cached + 1, H=128, "
                                   "latent 512 + rotary 64)", kernels=("decode_h128_kernel", "combine_uv_kernel"),
                             work=lambda: S.CONFIGS["dsv2_decode"], bound="hbm", file="dsv2_decode_attention"),
    "mlra_attention": dict(title="mla_decode_attention, MLRA decode (B=128, contexts U[512, 16384], 4 latent "
                                 "heads x rank 128)", kernels=("decode_fast_kernel", "combine_kernel"),
                           work=lambda: S.CONFIGS["mlra_decode"], bound="hbm", file="mlra_decode_attention"),
    "lh_attention": dict(title="mla_decode_attention, one MLRA latent head (rank 128, 4 query heads, the MLRA "
                               "contexts)", kernels=("decode_fast_kernel", "combine_kernel"),
                         work=lambda: MLRA_LATENT_HEAD, bound="hbm", file="mlra_latent_head_decode_attention"),
    "prefill_attention": dict(title="mla_prefill_attention, DeepSeek-V2 prefill (B=4, S=4096, H=128): K/V "
                                    "up-projection + flash causal attention",
                              kernels=("gemm_kv_kernel", "prefill_flash"),
                              work=lambda: S.CONFIGS["dsv2_prefill"], bound="mfma", file="dsv2_prefill_attention"),
}


def unit_work(unit):
    """Algorithmic bytes (decode) or flops (prefill) of one call of a profiled unit."""
    cfg = PROFILE_UNITS[unit]["work"]()
    if PROFILE_UNITS[unit]["bound"] == "hbm":
        ctx = problem(S.CONFIGS["mlra_decode"]).ctx_lens if unit == "lh_attention" else problem(cfg).ctx_lens
        return float(sum((int(c) + 1) * (cfg.r_kv + cfg.d_rope) * 2 for c in ctx))
    B, S_, H = cfg.batch, cfg.seq, cfg.n_heads
    core = 2.0 * B * H * (S_ * (S_ + 1) / 2) * (cfg.d_nope + cfg.d_rope + cfg.d_v)
    return core + 2.0 * B * S_ * cfg.r_kv * H * (cfg.d_nope + cfg.d_v) / cfg.n_latent_heads


def summarize_profiles(d):
    """Turn rocprofv3 CSV output under directory d into the committed summaries (profiles/).

    For each unit U of PROFILE_UNITS (run alone by `bench.py --only U`):
      d/U_trace   --kernel-trace --stats
      d/U_fetch   --pmc FETCH_SIZE            d/U_write  --pmc WRITE_SIZE
      d/U_mfma    --pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
    and d/copy_fetch, d/copy_write (the same counters on `bench.py --only copy`, a 1 GiB copy)
    for the bytes-per-counter scale.  d/decode_trace (`bench.py --only decode`) gives the
    kernels of one whole decode step.  Writes profiles/<file>_kernels.md per unit and
    profiles/<file>_traffic.json (read by the bench while the kernel sources match).
    """
    import csv
    import glob

    def rows(sub, pattern):
        out = []
        for f in glob.glob(os.path.join(d, sub, "**", pattern), recursive=True):
            with open(f) as fh:
                out.extend(csv.DictReader(fh))
        return out

    demangled = {}

    def short(name):
        if name.startswith("_Z"):
            # mangled names of this library's kernels (binutils' c++filt does not know the
            # bfloat16 code DF16b): namespace prefixes, the kernel name, its element type
            if name not in demangled:
                m = re.match(r"_ZN(?:3mla)?(?:12_GLOBAL__N_1)?(\d+)", name)
                out = name
                if m:
                    n = int(m.group(1))
                    base = name[m.end():m.end() + n]
                    rest = name[m.end() + n:]
                    typ = {"IDF16b": "<bf16>", "If": "<float>"}
                    out = base + next((t for k, t in typ.items() if rest.startswith(k)), "")
                demangled[name] = out
            name = demangled[name]
        name = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("mla::", "")
        name = re.sub(r"\(.*$", "", name).replace("__hip_bfloat16", "bf16")
        return name[:90]

    def grid_of(r):
        wg = max(1, int(r.get("Workgroup_Size_X") or 1))
        return f"{int(r.get('Grid_Size_X') or 0) // wg}x{int(r.get('Grid_Size_Y') or 1)}x{int(r.get('Grid_Size_Z') or 1)}"

    def dur(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3

    def kernel_table(trace, limit=None):
        """Per (kernel, grid) launch counts and durations, longest total first."""
        per = {}
        for r in trace:
            per.setdefault((short(r["Kernel_Name"]), grid_of(r)), []).append(dur(r))
        out = ["| kernel | grid (workgroups) | launches | total ms | avg µs | min µs | max µs |",
               "|---|---|---|---|---|---|---|"]
        for (k, g), v in sorted(per.items(), key=lambda kv: -sum(kv[1]))[:limit]:
            out.append(f"| {k} | {g} | {len(v)} | {sum(v) / 1e3:.2f} | {np.mean(v):.1f} | {np.min(v):.1f} | "
                       f"{np.max(v):.1f} |")
        return out, per

    def per_dispatch(sub, counters):
        """{dispatch id: (kernel name, {counter: value summed over the device})}"""
        out = {}
        for r in rows(sub, "*counter_collection.csv"):
            if r.get("Counter_Name") not in counters:
                continue
            key = r.get("Dispatch_Id")
            name, vals = out.setdefault(key, (r.get("Kernel_Name", ""), {}))
            vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return out

    def copy_kib(sub, counter):
        xs = [v[counter] for n, v in per_dispatch(sub, {counter}).values()
              if ("copy" in n.lower() or "elementwise" in n.lower()) and v.get(counter, 0) > 1e5]
        return float(np.median(xs)) if xs else None

    n_copy = 1 << 30
    cf, cw = copy_kib("copy_fetch", "FETCH_SIZE"), copy_kib("copy_write", "WRITE_SIZE")
    fscale = n_copy / (cf * 1024.0) if cf else None
    wscale = n_copy / (cw * 1024.0) if cw else None
    cmd = ("rocprofv3 {opt} --output-format csv -d <dir>/{sub} -o run -- python3 bench.py --only {unit} "
           "--steps {steps} --warmup 2")
    for unit, spec in PROFILE_UNITS.items():
        trace = rows(f"{unit}_trace", "*kernel_trace.csv")
        if not trace:
            continue
        trace.sort(key=lambda r: int(r["Start_Timestamp"]))
        first, last = spec["kernels"][0], spec["kernels"][-1]
        # calls: a dispatch of the first kernel opens a call, the next dispatch of the last kernel
        # closes it.  The bench times a loop of back-to-back calls with events, so its time per
        # call is the steady-state period between the starts of consecutive calls (kernels plus
        # the launch gaps between them); the first call after the set-up is left out.
        calls = []
        i = 0
        while i < len(trace):
            if first in trace[i]["Kernel_Name"] or first in short(trace[i]["Kernel_Name"]):
                j = i + 1
                while j < len(trace) and last not in short(trace[j]["Kernel_Name"]) \
                        and first not in short(trace[j]["Kernel_Name"]):
                    j += 1
                if j < len(trace) and last in short(trace[j]["Kernel_Name"]):
                    calls.append(trace[i:j + 1])
                    i = j + 1
                    continue
            i += 1
        if len(calls) < 3:
            continue
        starts = [int(c[0]["Start_Timestamp"]) for c in calls]
        periods = np.diff(starts)[1:] / 1e3
        spans = [(int(c[-1]["End_Timestamp"]) - int(c[0]["Start_Timestamp"])) / 1e3 for c in calls[1:]]
        table, per_kernel = kernel_table([r for c in calls[1:] for r in c])
        work = unit_work(unit)
        period = float(np.median(periods))
        peak = HBM_PEAK_GBS if spec["bound"] == "hbm" else MFMA_BF16_PEAK_TFLOPS
        div = 1e3 if spec["bound"] == "hbm" else 1e6
        achieved = work / period / div
        unit_s = "GB/s" if spec["bound"] == "hbm" else "TFLOP/s"
        kern_sum = sum(float(np.mean(v)) for v in per_kernel.values())
        lines = [f"# Kernel times and counters: {spec['title']}", "",
                 "Commands (from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first, then "
                 "`python3 bench.py --summarize <dir>`):", "", "```",
                 cmd.format(opt="--kernel-trace --stats", sub=f"{unit}_trace", unit=unit, steps=20),
                 cmd.format(opt="--pmc FETCH_SIZE", sub=f"{unit}_fetch", unit=unit, steps=3),
                 cmd.format(opt="--pmc WRITE_SIZE", sub=f"{unit}_write", unit=unit, steps=3),
                 cmd.format(opt="--pmc MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE", sub=f"{unit}_mfma",
                            unit=unit, steps=3),
                 cmd.format(opt="--pmc FETCH_SIZE", sub="copy_fetch", unit="copy", steps=3),
                 cmd.format(opt="--pmc WRITE_SIZE", sub="copy_write", unit="copy", steps=3),
                 "```", "",
                 f"One call = {' + '.join(spec['kernels'])}.  {len(calls) - 1} back-to-back calls traced (the first, "
                 "after the set-up, left out).", ""] + table + [
                 "", f"- sum of the kernels' average times: **{kern_sum:.1f} µs**",
                 f"- per-call period (start of a call to the start of the next; what the bench's events time over "
                 f"a loop of calls): median **{period:.1f} µs** (min {np.min(periods):.1f}, max {np.max(periods):.1f})",
                 f"- per-call span (first kernel's start to last kernel's end): median {np.median(spans):.1f} µs",
                 f"- algorithmic work per call: {work / 1e6:.2f} MB" if spec["bound"] == "hbm" else
                 f"- algorithmic work per call: {work / 1e12:.4f} TFLOP",
                 f"- achieved over the period: **{achieved:.1f} {unit_s}**, fraction of the {peak:.0f} {unit_s} peak "
                 f"= **{achieved / peak:.3f}** (over the kernel sum: {work / kern_sum / div / peak:.3f})", ""]
        rec = {"unit": spec["title"], "src_digest": src_digest(*UNIT_SOURCES[spec["file"]]),
               "period_us": period, "kernel_sum_us": kern_sum, "work_per_call": work,
               "frac_over_period": achieved / peak}
        fet = per_dispatch(f"{unit}_fetch", {"FETCH_SIZE"})
        wri = per_dispatch(f"{unit}_write", {"WRITE_SIZE"})
        if fet and wri and fscale and wscale:
            tot_r = tot_w = 0.0
            lines += ["HBM traffic per call (median per dispatch; FETCH_SIZE scaled by "
                      f"{fscale:.3f} and WRITE_SIZE by {wscale:.3f}, the factors that make a 1 GiB device copy read "
                      "and write 1 GiB):", ""]
            for kf in spec["kernels"]:
                fr = [v["FETCH_SIZE"] for n, v in fet.values() if kf in n]
                wr = [v["WRITE_SIZE"] for n, v in wri.values() if kf in n]
                if fr and wr:
                    rb, wb = float(np.median(fr)) * 1024 * fscale, float(np.median(wr)) * 1024 * wscale
                    tot_r += rb
                    tot_w += wb
                    lines.append(f"- {kf}: read {rb / 1e6:.1f} MB, write {wb / 1e6:.1f} MB")
            lines += [f"- unit total: **{(tot_r + tot_w) / 1e6:.1f} MB** per call"
                      + (f" against {work / 1e6:.1f} MB algorithmic ({(tot_r + tot_w) / work:.2f}x)"
                         if spec["bound"] == "hbm" else ""), ""]
            rec.update({"fetch_scale": fscale, "write_scale": wscale, "hbm_read_bytes_per_launch": tot_r,
                        "hbm_write_bytes_per_launch": tot_w, "hbm_bytes_per_launch": tot_r + tot_w})
        mf = per_dispatch(f"{unit}_mfma", {"MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_BUSY_CYCLES"})
        if mf:
            lines += ["MFMA utilisation (median per dispatch; MfmaUtil = sum of SQ_VALU_MFMA_BUSY_CYCLES over the "
                      "SIMDs / (GRBM_GUI_ACTIVE x SIMD count); clock = GRBM_GUI_ACTIVE summed over the 8 XCDs / 8 / "
                      "the kernel's average time above):", "",
                      "| kernel | MfmaUtil % | SQ_VALU_MFMA_BUSY_CYCLES | GRBM_GUI_ACTIVE | clock GHz |", "|---|---|---|---|---|"]
            for kf in spec["kernels"]:
                vs = [v for n, v in mf.values() if kf in n]
                if not vs:
                    continue
                med = {c: float(np.median([v.get(c, np.nan) for v in vs])) for c in
                       ("MfmaUtil", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")}
                t_us = np.mean([np.mean(v) for (k, g), v in per_kernel.items() if kf in k] or [np.nan])
                # (kernels under 50 µs: the counter window's own overhead dominates, no clock shown)
                clk = med["GRBM_GUI_ACTIVE"] / 8 / (t_us * 1e-6) / 1e9 if t_us >= 50 else float("nan")
                lines.append(f"| {kf} | {med['MfmaUtil']:.1f} | {med['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | "
                             f"{med['GRBM_GUI_ACTIVE']:.4g} | " + (f"{clk:.2f} |" if clk == clk else "— |"))
                rec.setdefault("mfma_util_pct", {})[kf] = med["MfmaUtil"]
            lines.append("")
        lines.append(f"Kernel sources digest: {rec['src_digest']}")
        with open(os.path.join(PROFILES, f"{spec['file']}_kernels.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        with open(os.path.join(PROFILES, f"{spec['file']}_traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
        print(f"{unit}: period {period:.1f} us, frac {achieved / peak:.3f}")

    # the kernels of one whole decode step (bench.py --only decode)
    trace = rows("decode_trace", "*kernel_trace.csv")
    if trace:
        trace.sort(key=lambda r: int(r["Start_Timestamp"]))
        names = [short(r["Kernel_Name"]) for r in trace]
        # a step ends with the output projection (plus its split reduce) after the fused combine
        ends = []
        for c, n in enumerate(names):
            if n.startswith("combine_uv_kernel") and "false" not in n and c + 1 < len(names):
                j = c + 1
                if j + 1 < len(names) and names[j + 1].startswith("split_reduce"):
                    j += 1
                ends.append(j)
        lines = ["# Kernel times: one mla_decode step, DeepSeek-V2 decode (B=64, 4096 cached tokens, H=128, "
                 "d_model 5120)", "",
                 "Command (from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "", "```",
                 "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/decode_trace -o run -- python3 bench.py "
                 "--only decode --steps 20 --warmup 5", "python3 bench.py --summarize <dir>", "```", ""]
        steps = [(ends[k] + 1, ends[k + 1]) for k in range(len(ends) - 1)]
        if steps:
            n_k = int(np.median([b - a + 1 for a, b in steps]))
            steps = [(a, b) for a, b in steps if b - a + 1 == n_k]
        if len(steps) >= 3:
            a0, b0 = steps[-1]
            lines += [f"{len(steps)} steps of {n_k} kernels traced (eager calls and graph replays); median per "
                      "kernel:", "", "| kernel | grid (workgroups) | median µs |", "|---|---|---|"]
            tot = 0.0
            for pos in range(n_k):
                us = float(np.median([dur(trace[a + pos]) for a, b in steps]))
                tot += us
                lines.append(f"| {short(trace[a0 + pos]['Kernel_Name'])} | {grid_of(trace[a0 + pos])} | {us:.1f} |")
            spans = [(int(trace[b]["End_Timestamp"]) - int(trace[a]["Start_Timestamp"])) / 1e3 for a, b in steps]
            per = [(int(trace[steps[k + 1][0]]["Start_Timestamp"]) - int(trace[steps[k][0]]["Start_Timestamp"])) / 1e3
                   for k in range(len(steps) - 1)]
            per = [x for x in per if x < 2 * np.median(spans)]          # back-to-back steps only
            lines += [f"| **sum** | | **{tot:.1f}** |", "",
                      f"- step span (first kernel's start to last kernel's end): median {np.median(spans):.1f} µs",
                      f"- step period (start of a step to the start of the next, back-to-back steps): median "
                      f"**{np.median(per):.1f} µs**; latent cache 302.06 MB per period: "
                      f"{302.06e6 / np.median(per) / 1e3:.1f} GB/s", ""]
        with open(os.path.join(PROFILES, "dsv2_decode_step_kernels.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")

    # kernels of the CCA / CCGQA prefill and of the training step (bench.py --only cca / train)
    for sub, title, fname, steps in (
            ("cca_trace", "mla_cca_prefill, CCA and CCGQA at the page defaults (B=4, S=2048, E=2048, 16 query heads; "
                          "CCA 16 key/value heads of 32, CCGQA 4 of 64)", "cca_prefill_kernels.md", 3),
            ("train_trace", "mla_train_forward + mla_train_backward, DeepSeek-V2 prefill shape (B=4, S=4096), "
                            "dropout 0.1", "dsv2_train_step_kernels.md", 3)):
        trace = rows(sub, "*kernel_trace.csv")
        if not trace:
            continue
        unit = sub.split("_")[0]
        table, _ = kernel_table([r for r in trace if not short(r["Kernel_Name"]).startswith(("at::", "__amd"))])
        lines = [f"# Kernel times: {title}", "", "Command (from the repository root on one MI355X; "
                 "`cd /tmp && export TMPDIR=/tmp` first):", "", "```",
                 f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/{sub} -o run -- python3 bench.py "
                 f"--only {unit} --steps {steps} --warmup 1", "python3 bench.py --summarize <dir>", "```", "",
                 "Library kernels of every call in the run (warm-up included), per grid shape:", ""] + table
        with open(os.path.join(PROFILES, fname), "w") as fh:
            fh.write("\n".join(lines) + "\n")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    choices=["all", "decode", "decode_attention", "prefill", "prefill_attention", "mlra",
                             "mlra_attention", "lh_attention", "small", "cca", "train", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize", metavar="DIR", help="write profile summaries from rocprofv3 output in DIR")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize)
        return
    if args.only != "all":
        # profiled runs: the trace holds the timed loop's back-to-back calls and few others
        global PER_CALL_STATS, MIN_WARM_S
        PER_CALL_STATS = False
        MIN_WARM_S = 0.0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: there is no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import head_latent_attention_dkv_amd as M
    M.lib()
    torch.cuda.set_device(0)

    if args.only == "copy":
        # plain device copy of a known size (counter calibration for HBM traffic)
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        ms = timed(torch, lambda i: b.copy_(a), args.steps, args.warmup)
        print(json.dumps({"copy_bytes": n, "ms": ms, "GBps_read_plus_write": 2 * n / ms / 1e6}))
        return
    if args.only == "decode_attention":
        r, _ = bench_decode(S.CONFIGS["dsv2_decode"], 0, 0, attention_steps=args.steps)
        print(json.dumps(r))
        return
    if args.only == "prefill_attention":
        print(json.dumps(bench_prefill(S.CONFIGS["dsv2_prefill"], args.steps, args.warmup, parts=("attention",))))
        return
    if args.only == "mlra_attention":
        r, _ = bench_decode(S.CONFIGS["mlra_decode"], 0, 0, copies=1, attention_steps=args.steps)
        print(json.dumps(r))
        return
    if args.only == "lh_attention":
        r, _ = bench_decode(MLRA_LATENT_HEAD, 0, 0, copies=2, attention_steps=args.steps,
                            ctx_from=S.CONFIGS["mlra_decode"])
        print(json.dumps(r))
        return
    if args.only == "cca":
        print(json.dumps({n: bench_cca(S.CCA_CONFIGS[n], args.steps, args.warmup) for n in ("cca", "ccgqa")}))
        return
    if args.only == "train":
        print(json.dumps(bench_train(S.CONFIGS["dsv2_prefill"], args.steps, args.warmup)))
        return

    out = {}
    if args.only in ("all", "decode"):
        dec, _ = bench_decode(S.CONFIGS["dsv2_decode"], args.steps, args.warmup)
        out["decode"] = dec
    if args.only in ("all", "prefill"):
        out["prefill"] = bench_prefill(S.CONFIGS["dsv2_prefill"], max(10, args.steps // 2), max(1, args.warmup // 2))
    if args.only in ("all", "mlra"):
        out["mlra"], _ = bench_decode(S.CONFIGS["mlra_decode"], args.steps, args.warmup, copies=1)
        # one latent head's cache is 288 MB: two copies (576 MB) exceed the 256 MB Infinity Cache
        out["mlra_lh"], _ = bench_decode(MLRA_LATENT_HEAD, args.steps, args.warmup, copies=2,
                                         ctx_from=S.CONFIGS["mlra_decode"])
    if args.only in ("all", "small"):
        out["small"] = bench_prefill(S.CONFIGS["small_lm"], args.steps, args.warmup)
    if args.only == "all":
        out["cca"] = {n: bench_cca(S.CCA_CONFIGS[n], max(3, args.steps // 4), max(1, args.warmup // 2))
                      for n in ("cca", "ccgqa")}
        out["train"] = bench_train(S.CONFIGS["dsv2_prefill"], max(2, args.steps // 8), 1)
    if args.only != "all":
        print(json.dumps(out))
        return

    dec = out["decode"]
    cfg3 = S.CONFIGS["dsv2_decode"]
    line = {
        "metric": METRIC,
        "value": dec["cache_GBps_call"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_call"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) activations and N(0,1/fan_in) weights, bf16-rounded; "
                "latent cache filled by the library from the seeded activations",
        "config": {
            "workload": "DeepSeek-V2-shaped single-layer MLA decode, absorbed form: one mla_decode call "
                        "(append, query path, absorbed query, split-context latent attention + combine, "
                        "W_UV, W_O) for 64 sequences of 4096 cached tokens + 1 new token",
            "batch": cfg3.batch, "cached_tokens": cfg3.seq, "n_heads": cfg3.n_heads, "d_nope": cfg3.d_nope,
            "d_rope": cfg3.d_rope, "r_kv": cfg3.r_kv, "r_q": cfg3.r_q, "d_model": cfg3.d_model,
            "value_definition": "latent-cache bytes streamed per step (302.06 MB) / step time",
            "cache_copies": 2,
        },
        "roofline": {
            "kernel": "mla_decode_attention unit: split-context latent attention kernel + combine kernel "
                      "(the step's dominant kernels)",
            "bound": "hbm",
            "achieved": dec["attention_GBps"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": dec["attention_GBps"] / HBM_PEAK_GBS,
            "traffic": traffic_from_profiles("dsv2_decode_attention", src_digest(*UNIT_SOURCES["dsv2_decode_attention"])),
            "algorithmic_bytes_per_launch": dec["cache_bytes"],
            "ms_per_launch": dec["attention_ms"],
            "timing": dec["attention_stats"],
        },
        "decode_step": {"ms": dec["ms_per_call"], "timing": dec["call_stats"],
                        "GBps_incl_weights": dec["call_GBps_incl_weights"], "weight_bytes": dec["weight_bytes"],
                        "cache_bytes": dec["cache_bytes"],
                        "frac_of_hbm_incl_weights": dec["call_GBps_incl_weights"] / HBM_PEAK_GBS,
                        "tokens_per_s": cfg3.batch / (dec["ms_per_call"] * 1e-3),
                        "graph_replay": {"ms": dec["ms_per_call_graph"], "timing": dec["graph_stats"],
                                         "cache_GBps": dec["cache_bytes"] / dec["ms_per_call_graph"] / 1e6}},
    }
    pre = out["prefill"]
    line["prefill"] = {
        "workload": "DeepSeek-V2-shaped MLA causal prefill B=4, S=4096 (dims as decode)",
        "ms_per_call": pre["ms_per_call"], "timing": pre["call_stats"], "layer_TFLOPs": pre["layer_TFLOPs"],
        "tokens_per_s": 4 * 4096 / (pre["ms_per_call"] * 1e-3),
        "roofline": {"kernel": "mla_prefill_attention (explicit K/V up-projection + flash causal attention)",
                     "bound": "mfma", "achieved": pre["attention_TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": pre["attention_TFLOPs"] / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic_from_profiles("dsv2_prefill_attention",
                                                      src_digest(*UNIT_SOURCES["dsv2_prefill_attention"])),
                     "algorithmic_flop_per_launch": pre["attention_flop"], "ms_per_launch": pre["attention_ms"],
                     "timing": pre["attention_stats"]},
    }
    if "chunk" in pre:
        ch = pre["chunk"]
        line["prefill_chunk"] = {
            "workload": f"DeepSeek-V2-shaped continued prefill B=4: {ch['new_tokens']} new tokens over "
                        f"{ch['start']} cached (mla_prefill_chunk)",
            "ms_per_call": ch["ms_per_call"], "timing": ch["stats"], "TFLOPs": ch["TFLOPs"],
            "frac_of_mfma_peak": ch["TFLOPs"] / MFMA_BF16_PEAK_TFLOPS, "new_tokens_per_s": ch["new_tokens_per_s"],
            "algorithmic_flop_per_call": ch["flop"]}
    ml = out["mlra"]
    line["mlra_decode"] = {
        "workload": "MLRA decode B=128, ctx ~ U[512,16384], 4 latent heads x rank 128, H=16, d_model=2048",
        "ms_per_call": ml["ms_per_call"], "cache_GBps_call": ml["cache_GBps_call"], "cache_bytes": ml["cache_bytes"],
        "roofline": {"kernel": "mla_decode_attention unit (split kernel + combine)", "bound": "hbm",
                     "achieved": ml["attention_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": ml["attention_GBps"] / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles("mlra_decode_attention",
                                                      src_digest(*UNIT_SOURCES["mlra_decode_attention"])),
                     "algorithmic_bytes_per_launch": ml["cache_bytes"], "ms_per_launch": ml["attention_ms"]},
    }
    lh = out["mlra_lh"]
    line["mlra_latent_head_decode"] = {
        "workload": "one MLRA latent head: rank 128, its 4 query heads, d_model=2048, B=128, the contexts of "
                    "mlra_decode (token-split decode kernel)",
        "ms_per_call": lh["ms_per_call"], "cache_GBps_call": lh["cache_GBps_call"], "cache_bytes": lh["cache_bytes"],
        "roofline": {"kernel": "mla_decode_attention unit (token-split kernel + combine)", "bound": "hbm",
                     "achieved": lh["attention_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": lh["attention_GBps"] / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles("mlra_latent_head_decode_attention",
                                                      src_digest(*UNIT_SOURCES["mlra_latent_head_decode_attention"])),
                     "algorithmic_bytes_per_launch": lh["cache_bytes"], "ms_per_launch": lh["attention_ms"]},
    }
    sm = out["small"]
    line["small_lm_prefill"] = {"workload": "small-LM MLA prefill B=8, S=1024, d_model=512, H=8, r_kv=256",
                                "ms_per_call": sm["ms_per_call"], "layer_TFLOPs": sm["layer_TFLOPs"],
                                "attention_TFLOPs": sm["attention_TFLOPs"]}
    line["cca_prefill"] = {n: {**r, "roofline": {"bound": "mfma", "achieved": r["TFLOPs"], "peak": MFMA_BF16_PEAK_TFLOPS,
                                                 "unit": "TFLOP/s", "frac": r["frac_of_mfma_peak"]}}
                           for n, r in out["cca"].items()}
    tr = out["train"]
    line["train_step"] = {**tr, "roofline": {"bound": "mfma", "achieved": tr["step_TFLOPs"],
                                             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                             "frac": tr["frac_of_mfma_peak"]}}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(S.CONFIGS["dsv2_decode"])
        log("[bench] cpu baseline of the prefill unit (oracle)")
        line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(S.CONFIGS["dsv2_prefill"])
    print(json.dumps(line))


if __name__ == "__main__":
    main()
