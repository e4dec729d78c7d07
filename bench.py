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


def timed(torch, fn, steps, warmup, stats=None):
    """Average ms per call of fn(i) over `steps` calls after `warmup` calls.

    HIP events on the current stream (the stream the library launches on) bracket the
    timed calls, with a device synchronisation on both sides; an event between calls gives
    each call's duration, whose median / p10 / p90 go into `stats` when it is a dict.
    """
    if steps <= 0:
        return float("nan")
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn(warmup + i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    if stats is not None:
        stats.update({"median_ms": float(np.median(per)), "p10_ms": float(np.percentile(per, 10)),
                      "p90_ms": float(np.percentile(per, 90))})
    return ev[0].elapsed_time(ev[steps]) / steps


# Sources of each measured kernel unit (a stored counter measurement is valid only for them).
UNIT_SOURCES = {
    "dsv2_decode_attention": ("decode_fast.hip", "decode.hip", "lds_dma.h", "common.h", "internal.h"),
    "dsv2_prefill_attention": ("prefill_fast.hip", "prefill.hip", "gemm.hip", "gemm_big.hip", "gemm_epilogue.h",
                               "lds_dma.h", "common.h", "internal.h"),
    "mlra_decode_attention": ("decode_fast.hip", "decode.hip", "lds_dma.h", "common.h", "internal.h"),
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

    # dominant kernel unit: split-context latent attention + combine
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


def bench_prefill(cfg, steps, warmup):
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

    log(f"[bench] {cfg.name}: timing mla_prefill")
    st_call = {}
    ms = timed(torch, call, steps, warmup, st_call)
    H, dn, dr, dv = cfg.n_heads, cfg.d_nope, cfg.d_rope, cfg.d_v
    g = torch.Generator(device="cpu").manual_seed(cfg.seed)
    q = torch.randn((B, S_, H, dn + dr), generator=g).to(d.dt).cuda()
    o = torch.empty((B, S_, H, dv), dtype=d.dt, device="cuda")
    wsa, nwsa = d.workspace(M.MLA_OP_PREFILL_ATTENTION, B, S_)

    def att(i):
        M.mla_prefill_attention(d.dims, d.wst, q, B, S_, cs, o, wsa, nwsa)

    log(f"[bench] {cfg.name}: timing mla_prefill_attention")
    st_att = {}
    ms_att = timed(torch, att, steps, warmup, st_att)
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
    if 0 < start < S_:
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


def cpu_baseline_prefill(cfg, budget_s=12.0, rows_per_seq=32):
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


def summarize_profiles(d):
    """Turn rocprofv3 CSV output under directory d into the committed summaries.

    d/stats/*kernel_stats.csv        (--kernel-trace --stats of `bench.py --only decode`)
    d/fetch/*counter_collection.csv  (--pmc FETCH_SIZE of `bench.py --only decode_attention`)
    d/write/*counter_collection.csv  (--pmc WRITE_SIZE of the same)
    d/copy_fetch, d/copy_write       (the same counters on `bench.py --only copy`)
    Writes profiles/dsv2_decode_attention_traffic.json (bytes per launch of the unit,
    scaled by the copy kernel's bytes-per-counter-KiB) for the current kernel sources.
    """
    import csv
    import glob

    def rows(sub, pattern):
        out = []
        for f in glob.glob(os.path.join(d, sub, "**", pattern), recursive=True):
            with open(f) as fh:
                out.extend(csv.DictReader(fh))
        return out

    def per_dispatch(sub, counter, match):
        vals = {}
        for r in rows(sub, "*counter_collection.csv"):
            name = r.get("Kernel_Name", "")
            if r.get("Counter_Name") != counter or not match(name):
                continue
            key = (name, r.get("Dispatch_Id"))
            vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
        return vals

    def unit_kib(sub, counter):
        v = per_dispatch(sub, counter, lambda n: "decode_h128_kernel" in n or "combine_kernel" in n
                         or "combine_uv_kernel" in n)
        by = {}
        for (name, _), x in v.items():
            by.setdefault("combine" if "combine" in name else "split", []).append(x)
        return {k: float(np.median(x)) for k, x in by.items()}

    def copy_kib(sub, counter):
        v = per_dispatch(sub, counter, lambda n: "copy" in n.lower() or "elementwise" in n.lower())
        xs = [x for x in v.values() if x > 1e5]
        return float(np.median(xs)) if xs else None

    n_copy = 1 << 30
    cf, cw = copy_kib("copy_fetch", "FETCH_SIZE"), copy_kib("copy_write", "WRITE_SIZE")
    uf, uw = unit_kib("fetch", "FETCH_SIZE"), unit_kib("write", "WRITE_SIZE")
    rec = {"unit": "mla_decode_attention: split kernel + combine kernel, DeepSeek-V2 decode shape",
           "copy_bytes": n_copy, "copy_fetch_kib": cf, "copy_write_kib": cw,
           "fetch_kib": uf, "write_kib": uw}
    if cf and cw and uf and uw:
        ff, fw = n_copy / (cf * 1024.0), n_copy / (cw * 1024.0)
        rec["fetch_scale"], rec["write_scale"] = ff, fw
        rec["hbm_read_bytes_per_launch"] = sum(uf.values()) * 1024.0 * ff
        rec["hbm_write_bytes_per_launch"] = sum(uw.values()) * 1024.0 * fw
        rec["hbm_bytes_per_launch"] = rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    rec["src_digest"] = src_digest(*UNIT_SOURCES["dsv2_decode_attention"])
    out = os.path.join(PROFILES, "dsv2_decode_attention_traffic.json")
    with open(out, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))

    # kernel-time summary of `bench.py --only decode`
    def short(name):
        name = name.replace("mla::(anonymous namespace)::", "").replace("(mla::GemmParams)", "")
        name = name.replace("(mla::DecodeParams)", "").replace("void ", "")
        if name.startswith("_ZN3mla"):
            m = re.match(r"_ZN3mla12_GLOBAL__N_114combine_kernelI(DF16b|f)Li(\d+)E", name)
            if m:
                return f"combine_kernel<{'bf16' if m.group(1) == 'DF16b' else 'float'},{m.group(2)}>"
            name = {"_ZN3mla12_GLOBAL__N_111gemm_kernelIDF16bLi64ELi64EEEvNS_10GemmParamsE": "gemm_kernel<bf16,64,64>",
                    "_ZN3mla12_GLOBAL__N_111gemm_kernelIDF16bLi128ELi128EEEvNS_10GemmParamsE":
                        "gemm_kernel<bf16,128,128>"}.get(name, name)
        name = re.sub(r"\(.*$", "", name)             # argument list
        return name[:70]

    lines = ["# Kernel times: DeepSeek-V2-shaped decode step (B=64, 4096 cached tokens, H=128)", "",
             "Commands (run from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "",
             "```",
             "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/stats -o run -- "
             "python3 bench.py --only decode --steps 20 --warmup 5",
             "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/fetch -o run -- "
             "python3 bench.py --only decode_attention --steps 3",
             "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/write -o run -- "
             "python3 bench.py --only decode_attention --steps 3",
             "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir>/copy_fetch -o run -- "
             "python3 bench.py --only copy --steps 3 --warmup 1",
             "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir>/copy_write -o run -- "
             "python3 bench.py --only copy --steps 3 --warmup 1",
             "python3 bench.py --summarize <dir>",
             "```", ""]
    trace = rows("stats", "*kernel_trace.csv")
    if trace:
        trace.sort(key=lambda r: int(r["Start_Timestamp"]))
        # one timed mla_decode step.  Launch order inside the call: W_DQ (+reduce), queries
        # (+reduce), latent (+reduce), absorbed query, attention, the combine fused with W_UV,
        # W_O (+reduce); the first timing loop runs whole calls, so a step ends after the W_O
        # product that follows the fused combine, and starts after the previous step's end.
        names = [short(r["Kernel_Name"]) for r in trace]

        def step_end(c):
            j = c + 1                                   # W_O
            if j + 1 < len(names) and names[j + 1] == "split_reduce_kernel":
                j += 1
            return j

        combines = [i for i, n in enumerate(names) if n.startswith("combine_uv_kernel") and "false" not in n]
        ends = [step_end(c) for c in combines if c + 1 < len(names) and names[c + 1].startswith("skinny")]
        step = (ends[-2] + 1, ends[-1]) if len(ends) >= 2 else None
        if step:
            lines += ["One timed mla_decode step (kernel trace):", "",
                      "| kernel | blocks (grid x) | µs |", "|---|---|---|"]
            tot = 0.0
            for r in trace[step[0]:step[1] + 1]:
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                tot += us
                blocks = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]) if "Grid_Size_X" in r else r.get("Grid_Size")
                lines.append(f"| {short(r['Kernel_Name'])} | {blocks} | {us:.1f} |")
            lines += [f"| **sum** | | **{tot:.1f}** |", ""]
    stats = rows("stats", "*kernel_stats.csv")
    if stats:
        lines += ["rocprofv3 --stats (whole command, including the cache fill's append GEMMs):", "",
                  "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
        for r in stats[:14]:
            lines.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                         f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        lines.append("")
    lines += ["HBM traffic of the mla_decode_attention unit (median per dispatch; FETCH_SIZE scaled by "
              f"{rec.get('fetch_scale', float('nan')):.3f}, WRITE_SIZE by {rec.get('write_scale', float('nan')):.3f}, "
              "the factors that make a 1 GiB device copy read and write 1 GiB):", "",
              f"- split kernel: read {uf.get('split', 0) * 1024 * rec.get('fetch_scale', 0) / 1e6:.1f} MB, "
              f"write {uw.get('split', 0) * 1024 * rec.get('write_scale', 0) / 1e6:.1f} MB",
              f"- combine kernel: read {uf.get('combine', 0) * 1024 * rec.get('fetch_scale', 0) / 1e6:.1f} MB, "
              f"write {uw.get('combine', 0) * 1024 * rec.get('write_scale', 0) / 1e6:.1f} MB",
              f"- unit total: {rec.get('hbm_bytes_per_launch', 0) / 1e6:.1f} MB per launch vs 302.1 MB algorithmic "
              "(latent + rotary cache)", "",
              f"Kernel sources digest: {rec['src_digest']}", ""]
    with open(os.path.join(PROFILES, "dsv2_decode_step_kernels.md"), "w") as fh:
        fh.write("\n".join(lines))

    # kernel times of `bench.py --only prefill_attention` (d/prefill_stats)
    pstats = rows("prefill_stats", "*kernel_stats.csv")
    if pstats:
        pl = ["# Kernel times: DeepSeek-V2-shaped prefill attention (B=4, S=4096, H=128, d_nope=128, "
              "d_rope=64, r_kv=512)", "",
              "Command (run from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "",
              "```",
              "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/prefill_stats -o run -- "
              "python3 bench.py --only prefill_attention --steps 8 --warmup 2",
              "python3 bench.py --summarize <dir>",
              "```", "",
              "mla_prefill_attention = K/V up-projection GEMM (gemm_big_kernel, writes head-major K and "
              "token-permuted V^T) + flash causal attention (prefill_flash_kernel).", "",
              "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
        for r in pstats[:8]:
            pl.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                      f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        pl += ["", f"Kernel sources digest: {src_digest(*UNIT_SOURCES['dsv2_prefill_attention'])}", ""]
        with open(os.path.join(PROFILES, "dsv2_prefill_attention_kernels.md"), "w") as fh:
            fh.write("\n".join(pl))

    # kernel times of `bench.py --only mlra` (d/mlra_stats)
    mstats = rows("mlra_stats", "*kernel_stats.csv")
    if mstats:
        ml = ["# Kernel times: MLRA decode (B=128, contexts U[512, 16384], 4 latent blocks x rank 128, "
              "H=16, d_model=2048) and one of its latent heads on its own (rank 128, 4 query heads)", "",
              "Command (run from the repository root on one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "",
              "```",
              "rocprofv3 --kernel-trace --stats --output-format csv -d <dir>/mlra_stats -o run -- "
              "python3 bench.py --only mlra --steps 20 --warmup 5",
              "python3 bench.py --summarize <dir>",
              "```", "",
              "mla_decode_attention = split kernel (decode_fast_kernel; `true` = the token-split form of the "
              "latent-head workload) + combine kernel; the calls also run the few-row projections and the "
              "cache append.", "",
              "| kernel | calls | avg µs | min µs | max µs |", "|---|---|---|---|---|"]
        for r in mstats[:14]:
            ml.append(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                      f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
        ml += ["", f"Kernel sources digest: {src_digest(*UNIT_SOURCES['mlra_decode_attention'])}", ""]
        with open(os.path.join(PROFILES, "mlra_decode_attention_kernels.md"), "w") as fh:
            fh.write("\n".join(ml))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="all",
                    choices=["all", "decode", "decode_attention", "prefill", "prefill_attention", "mlra",
                             "small", "copy"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize", metavar="DIR", help="write profile summaries from rocprofv3 output in DIR")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize)
        return
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
        print(json.dumps(bench_prefill(S.CONFIGS["dsv2_prefill"], args.steps, args.warmup)))
        return

    out = {}
    if args.only in ("all", "decode"):
        dec, _ = bench_decode(S.CONFIGS["dsv2_decode"], args.steps, args.warmup)
        out["decode"] = dec
    if args.only in ("all", "prefill"):
        out["prefill"] = bench_prefill(S.CONFIGS["dsv2_prefill"], max(3, args.steps // 4), max(1, args.warmup // 2))
    if args.only in ("all", "mlra"):
        out["mlra"], _ = bench_decode(S.CONFIGS["mlra_decode"], args.steps, args.warmup, copies=1)
        # one latent head's cache is 288 MB: two copies (576 MB) exceed the 256 MB Infinity Cache
        out["mlra_lh"], _ = bench_decode(MLRA_LATENT_HEAD, args.steps, args.warmup, copies=2,
                                         ctx_from=S.CONFIGS["mlra_decode"])
    if args.only in ("all", "small"):
        out["small"] = bench_prefill(S.CONFIGS["small_lm"], args.steps, args.warmup)
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
                     "algorithmic_bytes_per_launch": lh["cache_bytes"], "ms_per_launch": lh["attention_ms"]},
    }
    sm = out["small"]
    line["small_lm_prefill"] = {"workload": "small-LM MLA prefill B=8, S=1024, d_model=512, H=8, r_kv=256",
                                "ms_per_call": sm["ms_per_call"], "layer_TFLOPs": sm["layer_TFLOPs"],
                                "attention_TFLOPs": sm["attention_TFLOPs"]}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(S.CONFIGS["dsv2_decode"])
        log("[bench] cpu baseline of the prefill unit (oracle)")
        line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(S.CONFIGS["dsv2_prefill"])
    print(json.dumps(line))


if __name__ == "__main__":
    main()
