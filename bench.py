#!/usr/bin/env python3
"""Throughput of the hybrid-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  Its headline (`value`) is the Pro-like long-context
decode: batch 4 at a 1,048,576-token context, 128 query heads, one KV head,
d = 128, fp8 e4m3 compressed K / V with one fp32 scale per 64-entry page,
bf16 indexer keys, top-1024 CSA layer plus HCA layer, window 128.  One step
is one hsa_decode_step of the CSA layer followed by one of the HCA layer for
the 4 requests: ring / tail upkeep, the lightning indexer over all 262,113
visible compressed blocks of every request, the top-k, the gather attention
(window + selected entries, CSA; window + all 8,192 entries, HCA) and the
split merges.  `value` = requests / step time (decode tokens/s of the layer
pair); `--steps` steps are timed exactly, captured in one HIP graph that
cycles over 8 independent cache copies (3.3 GB, so the 256 MB Infinity
Cache cannot hold them), after `--warmup` eager steps and one untimed replay.

`workloads` in the same line carries the other three throughput workloads,
each with its own roofline and oracle baseline:
  csa_decode_128k      batch 32 x 131,072 tokens, 64 heads, top-512, bf16;
  hybrid_prefill_128k  131,072 tokens, 64 heads, a CSA (top-512) and an HCA
                       layer; the timed pass includes block compression of
                       both layers (hsa_kv_compress), the indexer, top-k and
                       both attentions;
  ragged_serving       16 requests, log-uniform 8K..1M tokens, shuffled
                       64-entry pages, 256 decode steps of a CSA (top-1024)
                       and an HCA layer, blocks appended as tokens stream in.

Every `roofline` names the dominant kernel, its algorithmic bytes (or flops)
per launch, its average launch duration measured live with HIP events handed
to that kernel's own dispatch, the fraction of MI355X's peak (8 TB/s HBM,
2.5 PFLOP/s dense bf16 MFMA) and -- while the kernel's source is unchanged --
the HBM bytes per launch from committed rocprofv3 counter summaries.
`cpu_baseline` is the oracle (float64 NumPy) on a bounded sample of the same
workload, run on a process pool over this host's cores.

Counter tools (no GPU): --traffic-summary and --mfma-summary turn rocprofv3
--pmc CSV files into the summaries under profiles/.
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s at 128K-1M ctx + prefill Ktok/s; % of HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
COPIES = 8
RAGGED_COPIES = 4
MAX_CPU_WORKERS = 16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


# ----------------------------------------------------------------------------- decode state

def build_decode_state(w, layer, L, T, gen, copies, fp8=False, shuffle=False, draft=1,
                       kmix=False, index_fp4=False):
    """Caches of w.B requests holding tokens 0..L-1, rings up to L-1, and the
    new token's inputs (position L), in `copies` independent copies.  fp8 K / V
    caches carry the stash appending to them needs.
    index_fp4: the indexer keys are stored fp4 (the indexer computes in FP4),
    and step["kic_bf16"] holds the same keys in bf16 (for the selection recall).
    draft > 1: the step's inputs are [B][draft][...] (tokens L .. L+draft-1);
    rings hold n_win + draft - 1 tokens and the indexer tail m + draft - 1.
    kmix: the K caches hold mixed entries (RoPE channels bf16, the rest fp8)."""
    import torch
    B, m, n_win = w.B, w.m(layer), w.n_win
    z = gen.pool_logits(w, layer)
    alpha = {k: T.pooling_weights(torch.from_numpy(z["z" + k]).cuda())
             for k in (["k", "v", "i"] if layer == "csa" else ["k", "v"])}
    n_ent = L // m + 2
    ppr = -(-n_ent // 64)
    perm = torch.from_numpy(gen.page_permutation(w, layer, B * ppr)) if shuffle else None
    stash = fp8 or kmix
    kc = T.PagedCache.allocate(B, n_ent, 128, fp8=fp8, page_order=perm, mixed=kmix, stash=stash)
    vc = T.PagedCache.allocate(B, n_ent, 128, fp8=fp8 or kmix, page_order=perm, stash=stash)
    kic = (T.PagedCache.allocate(B, n_ent, 64, fp4=index_fp4, page_order=perm)
           if layer == "csa" else None)
    kic16 = (T.PagedCache.allocate(B, n_ent, 64, page_order=perm)
             if layer == "csa" and index_fp4 else None)
    cap = n_win + draft - 1
    ring_k = torch.zeros((B, cap, 128), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    tail = (torch.zeros((B, m + draft - 1, 64), dtype=torch.bfloat16, device="cuda")
            if layer == "csa" else None)
    inp = {"Q": [], "k_new": [], "v_new": [], "qI": [], "kI_new": [], "w": []}
    for r in range(B):
        d = gen.decode_request(w, layer, r, L=L, extra_tokens=draft, n_queries=draft)
        nb = L // m
        T.kv_compress(T.Tokens(bf(d["k"][:L])[None].contiguous()), kc, r, 0, nb, m, alpha["k"])
        T.kv_compress(T.Tokens(bf(d["v"][:L])[None].contiguous()), vc, r, 0, nb, m, alpha["v"])
        if layer == "csa":
            T.kv_compress(T.Tokens(bf(d["ki"][:L])[None].contiguous()), kic, r, 0, nb, m, alpha["i"])
            if kic16 is not None:
                T.kv_compress(T.Tokens(bf(d["ki"][:L])[None].contiguous()), kic16, r, 0, nb, m,
                              alpha["i"])
            t0 = nb * m
            if t0 < L:
                tail[r, torch.arange(t0, L) % tail.shape[1]] = bf(d["ki"][t0:L])
            inp["qI"].append(d["qi"][0] if draft == 1 else d["qi"][:draft])
            inp["kI_new"].append(d["ki"][L] if draft == 1 else d["ki"][L:L + draft])
            inp["w"].append(d["w"][0] if draft == 1 else d["w"][:draft])
        lo = max(0, L - n_win)
        ring_k[r, torch.arange(lo, L) % cap] = bf(d["k"][lo:L])
        ring_v[r, torch.arange(lo, L) % cap] = bf(d["v"][lo:L])
        inp["Q"].append(d["q"][0] if draft == 1 else d["q"][:draft])
        inp["k_new"].append(d["k"][L] if draft == 1 else d["k"][L:L + draft])
        inp["v_new"].append(d["v"][L] if draft == 1 else d["v"][L:L + draft])
        del d
        torch.cuda.synchronize()
    step = {"Q": bf(np.stack(inp["Q"])), "k_new": bf(np.stack(inp["k_new"])),
            "v_new": bf(np.stack(inp["v_new"]))}
    if layer == "csa":
        step.update(qI=bf(np.stack(inp["qI"])), kI_new=bf(np.stack(inp["kI_new"])),
                    w=torch.from_numpy(np.stack(inp["w"])).cuda())
    step["pos"] = torch.full((B,), L, dtype=torch.int64, device="cuda")
    if kic16 is not None:
        step["kic_bf16"] = kic16

    def clone_cache(c):
        if c is None:
            return None
        return T.PagedCache(c.data.clone(), c.page_table, c.n_entries.clone(),
                            None if c.scale is None else c.scale.clone(), c.mixed, c.fp4,
                            None if c.stash is None else c.stash.clone())

    layers = []
    for i in range(copies):
        same = i == 0
        kw = dict(kind=T.LAYER_CSA if layer == "csa" else T.LAYER_HCA, H=w.H, n_win=n_win, m=m,
                  alpha_k=alpha["k"], alpha_v=alpha["v"],
                  ring_k=T.Tokens(ring_k if same else ring_k.clone()),
                  ring_v=T.Tokens(ring_v if same else ring_v.clone()),
                  kc=kc if same else clone_cache(kc), vc=vc if same else clone_cache(vc))
        if layer == "csa":
            kw.update(topk=w.k_csa, alpha_i=alpha["i"],
                      tail_i=T.Tokens(tail if same else tail.clone()),
                      kic=kic if same else clone_cache(kic))
        layers.append(T.Layer(**kw))
    torch.cuda.synchronize()
    return layers, step


class StepCall:
    """Pre-marshalled hsa_decode_step arguments: the stream is the caller's
    current stream at call time, so the call can be captured in a graph."""

    def __init__(self, T, layer, step, L_max, O, ws=None):
        import torch
        self.T = T
        self.lc = layer.c()
        B = step["pos"].shape[0]
        nb = T.lib().hsa_decode_step_workspace_bytes(C.byref(self.lc), B, L_max)
        self.ws = ws if ws is not None and ws.numel() >= nb else \
            torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        p = lambda t: None if t is None else C.c_void_p(t.data_ptr())
        self.args = (C.byref(self.lc), B, p(step["pos"]), L_max, p(step["Q"]), p(step["k_new"]),
                     p(step["v_new"]), p(step.get("qI")), p(step.get("kI_new")), p(step.get("w")),
                     p(O), None, None, C.c_void_p(self.ws.data_ptr()), self.ws.numel())
        self.fn = T.lib().hsa_decode_step

    def __call__(self):
        import torch
        st = self.fn(*self.args, C.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            self.T._check(st, "decode_step")


class DraftCall(StepCall):
    """Pre-marshalled hsa_decode_draft arguments (n_tok tokens per request)."""

    def __init__(self, T, layer, step, L_max, O, n_tok):
        import torch
        self.T = T
        self.lc = layer.c()
        B = step["pos"].shape[0]
        nb = T.lib().hsa_decode_draft_workspace_bytes(C.byref(self.lc), B, n_tok, L_max)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        p = lambda t: None if t is None else C.c_void_p(t.data_ptr())
        self.args = (C.byref(self.lc), B, n_tok, p(step["pos"]), L_max, p(step["Q"]),
                     p(step["k_new"]), p(step["v_new"]), p(step.get("qI")), p(step.get("kI_new")),
                     p(step.get("w")), p(O), None, None, C.c_void_p(self.ws.data_ptr()),
                     self.ws.numel())
        self.fn = T.lib().hsa_decode_draft


class Seq:
    """Several calls made as one step."""

    def __init__(self, *calls):
        self.calls = calls

    def __call__(self):
        for c in self.calls:
            c()


def time_steps(steps_cycle, K, W):
    """W eager warmup steps, then exactly K steps (cycling over steps_cycle)
    captured in one HIP graph: one untimed replay, one timed replay.
    Returns ms per step."""
    import torch
    n = len(steps_cycle)
    for i in range(W):
        steps_cycle[i % n]()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(K):
                steps_cycle[i % n]()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    del g
    return ms


def kernel_avg_ms(T, kid, fn, n, warm=4):
    """Average duration of one kernel over n eager calls of fn(i): HIP events
    on the kernel's own stream, handed by the library to the kernel's dispatch
    (HSA_K_INDEXER_SCAN, _GEMM, _ATTN) or recorded around its launches (_SEL,
    _COMPRESS).  Returns (ms per launch, launches)."""
    import torch
    # a few untimed calls first (warm > 0: calls that may repeat): the first
    # eager calls after a graph replay or a different workload run slower than
    # the steady state
    for i in range(min(n, warm)):
        fn(i)
    torch.cuda.synchronize()
    T.kernel_timing_read(kid)
    T.kernel_timing(kid, True)
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    T.kernel_timing(kid, False)
    ms, cnt = T.kernel_timing_read(kid)
    return ms / max(cnt, 1), cnt


def kernel_table(T, fn, n):
    """Average ms per launch of every timed kernel class over n calls of fn(i)."""
    out = {}
    for name, kid in (("indexer_scan", T.K_INDEXER_SCAN), ("indexer_gemm", T.K_INDEXER_GEMM),
                      ("selection", T.K_INDEXER_SEL), ("attention", T.K_ATTN),
                      ("compress", T.K_COMPRESS)):
        ms, cnt = kernel_avg_ms(T, kid, fn, n)
        if cnt:
            out[name] = {"ms_per_launch": round(ms, 5), "launches_per_step": round(cnt / n, 2)}
    return out


# ----------------------------------------------------------------------------- counters

def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_hybrid_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_sources(kernel):
    if kernel.startswith("idx_"):
        return ("indexer.hip", "common.h", "update.h")
    if kernel.startswith("compress"):
        return ("compress.hip", "common.h", "update.h")
    return ("attention.hip", "common.h")


def committed_counter(kind, kernel, workload, key):
    """A figure from a committed rocprofv3 counter summary
    (profiles/<kind>_<kernel>_<workload>.json), if it was taken on the current
    kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kind}_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash(*kernel_sources(kernel)):
        return None
    return t.get(key)


def _pmc_rows(path, counter, kernel_regex, reduce="sum", grid=None):
    """Per-dispatch values of one rocprofv3 counter for the kernels whose name
    matches kernel_regex (and, if given, whose grid size is `grid` threads),
    summed, or the maximum, over the counter's instances."""
    import csv
    import re
    rx = re.compile(kernel_regex)
    per = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter or not rx.search(row.get("Kernel_Name", "")):
                continue
            if grid is not None and int(row.get("Grid_Size", -1)) != grid:
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            v = float(row["Counter_Value"])
            per[key] = max(per.get(key, 0.0), v) if reduce == "max" else per.get(key, 0.0) + v
    return per


def _pmc_per_dispatch(path, counter, kernel_regex, reduce="sum", grid=None):
    """Mean per dispatch of one rocprofv3 counter over the kernels whose name
    matches kernel_regex (a --pmc run written with --output-format csv)."""
    per = _pmc_rows(path, counter, kernel_regex, reduce, grid)
    if not per:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {kernel_regex!r}")
    return sum(per.values()) / len(per), len(per)


def traffic_summary(args):
    """HBM-side bytes per launch of a kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for an elementwise copy of a known 1 GiB
    (bench.py --calibrate-copy).  Writes profiles/traffic_<kernel>_<workload>.json."""
    kernel, workload, fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.traffic_summary
    fk, nf = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE", kernel, grid=args.grid)
    wk, nw = _pmc_per_dispatch(write_csv, "WRITE_SIZE", kernel, grid=args.grid)
    cf, _ = _pmc_per_dispatch(cfetch_csv, "FETCH_SIZE", "elementwise")
    cw, _ = _pmc_per_dispatch(cwrite_csv, "WRITE_SIZE", "elementwise")
    kib = float(1 << 20)   # the copy reads and writes 1 GiB
    f_scale, w_scale = kib / cf, kib / cw
    name = kernel.split("<")[0]
    tag = name + (f"_{args.label}" if args.label else "")
    out = {"kernel": kernel, "workload": workload, "grid_threads": args.grid,
           "source_hash": source_hash(*kernel_sources(name)),
           "fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wk, 1),
           "dispatches": [nf, nw],
           "copy_calibration": {"fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                                "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "bytes_per_launch": int(round((fk * f_scale + wk * w_scale) * 1024))}
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def mfma_summary(args):
    """MFMA utilisation of a kernel from one rocprofv3 --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_INSTS_VALU_MFMA_MOPS_F16 and GRBM_GUI_ACTIVE.  As read on this part:
    GRBM_GUI_ACTIVE comes as one value per dispatch, the sum over the 8 XCDs
    (value / 8 = the kernel's active cycles: ~2.1 GHz times its duration under
    the profiler); SQ_VALU_MFMA_BUSY_CYCLES sums 16 cycles per 16x16x32 MFMA
    over all 1,024 SIMDs, so busy = BUSY / (active x 1,024); the MOPS counters
    count MFMA flops / 512 (x 512 reproduces the algorithmic flops of the score
    GEMM exactly), compared with the algorithmic flops per launch given on the
    command line.  Writes profiles/mfma_<kernel>_<workload>.json."""
    kernel, workload, csv_path, alg_flops = args.mfma_summary
    alg = float(alg_flops)
    g = args.grid   # one launch shape (the CSA prefill attention has two)
    busy, n = _pmc_per_dispatch(csv_path, "SQ_VALU_MFMA_BUSY_CYCLES", kernel, grid=g)
    bf16, _ = _pmc_per_dispatch(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_BF16", kernel, grid=g)
    f16, _ = _pmc_per_dispatch(csv_path, "SQ_INSTS_VALU_MFMA_MOPS_F16", kernel, grid=g)
    grbm, _ = _pmc_per_dispatch(csv_path, "GRBM_GUI_ACTIVE", kernel, grid=g)
    active = grbm / 8
    simds = 256 * 4
    executed = (bf16 + f16) * 512
    name = kernel.split("<")[0]
    out = {"kernel": kernel, "workload": workload, "grid_threads": g,
           "source_hash": source_hash(*kernel_sources(name)), "dispatches": n,
           "mfma_busy_cycles_per_simd": round(busy / simds, 1),
           "active_cycles": round(active, 1),
           "mfma_busy_frac": round(busy / (active * simds), 4),
           "mfma_flops_executed": executed, "algorithmic_flops": alg,
           "executed_over_algorithmic": round(executed / alg, 3)}
    path = os.path.join(ROOT, "profiles", f"mfma_{name}_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def roofline_hbm(kernel, workload, alg_bytes, ms, launches):
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": committed_counter("traffic", kernel, workload, "bytes_per_launch"),
            "algorithmic_bytes_per_launch": int(alg_bytes), "avg_launch_ms": round(ms, 5),
            "launches_timed": launches}


def roofline_mfma(kernel, workload, alg_flops, ms, launches):
    tf = alg_flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "traffic": committed_counter("traffic", kernel, workload, "bytes_per_launch"),
            "mfma_busy_frac": committed_counter("mfma", kernel, workload, "mfma_busy_frac"),
            "algorithmic_flops_per_launch": float(alg_flops), "avg_launch_ms": round(ms, 5),
            "launches_timed": launches}


def nvis(t, m, n_win):
    s = max(0, t - n_win + 1)
    return min(-(-s // m), (t + 1) // m)


# ----------------------------------------------------------------------------- oracle baselines

_CPU = {}   # inputs of the running baseline: set before the pool forks, read by its workers
_PREFILL_INPUTS = {}   # the 128K prefill's generated inputs, kept for its oracle baseline


def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_pool_run(task, budget_s):
    """Run task(i) for i = 0, 1, 2, ... on a fork-based process pool (at most
    16 workers, one BLAS thread each) until budget_s has passed.  Returns
    (tasks done, seconds, workers)."""
    import multiprocessing as mp
    workers = max(1, min(MAX_CPU_WORKERS, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("fork")
    done, nxt = 0, 0
    t0 = time.time()
    t_end = t0
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        pending = []
        while True:
            while len(pending) < 2 * workers and (time.time() - t0 < budget_s or nxt == 0):
                pending.append(pool.apply_async(task, (nxt,)))
                nxt += 1
            if not pending:
                break
            pending.pop(0).get()
            done += 1
            t_end = time.time()
    return done, t_end - t0, workers


def _baseline(value, unit, done, dt, workers, sample):
    return {"value": value, "unit": unit, "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(), "host_cpus_visible": len(os.sched_getaffinity(0)),
            "sample": f"{sample}; {done} tasks in {dt:.1f}s on {workers} worker processes "
                      f"(one BLAS thread each), float64"}


def _task_csa_decode(i):
    from oracle import hybrid as orc
    w = _CPU["w"]
    d, c = _CPU["sample"][i % len(_CPU["sample"])]
    orc.csa_query(w.L, d["q"][0], d["qi"][0], d["w"][0], d["k"], d["v"], c["kc"], c["vc"], c["kic"],
                  w.m_csa, w.n_win, w.k_csa)


def cpu_baseline_csa_decode(w, budget_s):
    """The oracle's decode query (indexer over every visible block, top-k,
    attention) on 4 of the requests; caches compressed outside the timing."""
    from oracle import hybrid as orc
    from synth import gen
    z = gen.pool_logits(w, "csa")
    sample = []
    for r in range(4):
        d = gen.decode_request(w, "csa", r)
        L = w.L
        sample.append((d, dict(kc=orc.compress(d["k"][:L], z["zk"], w.m_csa),
                               vc=orc.compress(d["v"][:L], z["zv"], w.m_csa),
                               kic=orc.compress(d["ki"][:L], z["zi"], w.m_csa))))
    _CPU.clear()
    _CPU.update(w=w, sample=sample)
    done, dt, workers = cpu_pool_run(_task_csa_decode, budget_s)
    _CPU.clear()
    return _baseline(done / dt, "tok/s", done, dt, workers,
                     f"decode queries of 4 of the {w.B} requests at context {w.L} (indexer over "
                     f"{nvis(w.L, w.m_csa, w.n_win)} blocks, top-{w.k_csa}, attention over "
                     f"{w.n_win + w.k_csa} entries)")


def _task_pro_decode(i):
    from oracle import hybrid as orc
    w, dc, dh, cc, ch = (_CPU[k] for k in ("w", "dc", "dh", "cc", "ch"))
    L = w.L
    orc.csa_query(L, dc["q"][0], dc["qi"][0], dc["w"][0], dc["k"], dc["v"], cc["kc"], cc["vc"],
                  cc["kic"], w.m_csa, w.n_win, w.k_csa)
    orc.hca_query(L, dh["q"][0], dh["k"], dh["v"], ch["kc"], ch["vc"], w.m_hca, w.n_win)


def cpu_baseline_pro_decode(w, budget_s):
    """The oracle's step (indexer, top-k, CSA attention, HCA attention) for one
    request at the 1M context; fp8 caches compressed outside the timing."""
    from oracle import hybrid as orc
    from synth import gen
    L = w.L
    dc = gen.decode_request(w, "csa", 0)
    dh = gen.decode_request(w, "hca", 0)
    zc, zh = gen.pool_logits(w, "csa"), gen.pool_logits(w, "hca")
    cc = dict(kc=orc.compress(dc["k"][:L], zc["zk"], w.m_csa, "fp8"),
              vc=orc.compress(dc["v"][:L], zc["zv"], w.m_csa, "fp8"),
              kic=orc.compress(dc["ki"][:L], zc["zi"], w.m_csa))
    ch = dict(kc=orc.compress(dh["k"][:L], zh["zk"], w.m_hca, "fp8"),
              vc=orc.compress(dh["v"][:L], zh["zv"], w.m_hca, "fp8"))
    _CPU.clear()
    _CPU.update(w=w, dc=dc, dh=dh, cc=cc, ch=ch)
    done, dt, workers = cpu_pool_run(_task_pro_decode, budget_s)
    _CPU.clear()
    return _baseline(done / dt, "tok/s", done, dt, workers,
                     f"decode steps of one request at context {L} (CSA top-{w.k_csa} over "
                     f"{nvis(L, w.m_csa, w.n_win)} blocks + HCA over {nvis(L, w.m_hca, w.n_win)} "
                     f"entries, fp8 caches)")


def _task_prefill(i):
    from oracle import hybrid as orc
    w, inc, inh, cc, ch, rows = (_CPU[k] for k in ("w", "inc", "inh", "cc", "ch", "rows"))
    t = rows[i % len(rows)]
    orc.prefill_rows(inc, "csa", [t], w.m_csa, w.n_win, topk=w.k_csa, caches=cc)
    orc.prefill_rows(inh, "hca", [t], w.m_hca, w.n_win, caches=ch)


def cpu_baseline_prefill(w, budget_s):
    """The oracle's 128K prefill: both layers' compression timed once (in this
    process), and the CSA + HCA outputs of query rows drawn uniformly over all
    131,072 positions on the pool; Ktok/s of the layer pair = 1 / (compression
    time per token + time per row on the pool)."""
    from oracle import hybrid as orc
    from synth import gen
    inc = _PREFILL_INPUTS.pop("csa", None) or gen.prefill_layer(w, "csa")
    inh = _PREFILL_INPUTS.pop("hca", None) or gen.prefill_layer(w, "hca")
    t0 = time.time()
    cc, ch = orc.layer_caches(inc, "csa", w.m_csa), orc.layer_caches(inh, "hca", w.m_hca)
    t_comp = time.time() - t0
    rows = gen.rng(w.seed, "cpu.rows").integers(0, w.T, 4096).tolist()
    _CPU.clear()
    _CPU.update(w=w, inc=inc, inh=inh, cc=cc, ch=ch, rows=rows)
    done, dt, workers = cpu_pool_run(_task_prefill, budget_s)
    _CPU.clear()
    per_tok = t_comp / w.T + dt / done
    return _baseline(1.0 / per_tok / 1e3, "Ktok/s", done, dt, workers,
                     f"compression of both layers' {w.T} tokens timed once ({t_comp:.1f}s, one "
                     f"process) plus CSA + HCA outputs of query rows drawn uniformly over the "
                     f"{w.T} positions")


def _task_ragged(i):
    from oracle import hybrid as orc
    w, reqs, Ls, cs, ch = (_CPU[k] for k in ("w", "reqs", "Ls", "cs", "ch"))
    j = i % len(reqs)
    s = (i // len(reqs)) % w.steps
    dc, dh = reqs[j]
    t = Ls[j] + s
    orc.csa_query(t, dc["q"][s], dc["qi"][s], dc["w"][s], dc["k"], dc["v"], cs[j]["kc"], cs[j]["vc"],
                  cs[j]["kic"], w.m_csa, w.n_win, w.k_csa)
    orc.hca_query(t, dh["q"][s], dh["k"], dh["v"], ch[j]["kc"], ch[j]["vc"], w.m_hca, w.n_win)


def cpu_baseline_ragged(w, budget_s):
    """The oracle's decode step (CSA + HCA) of 4 of the 16 ragged requests
    (seeded choice) at successive steps; caches compressed outside the timing.
    The rate is scaled to the whole batch by the sampled requests' share of the
    batch's tokens (the oracle's cost of a request-step grows with its
    context)."""
    from oracle import hybrid as orc
    from synth import gen
    Ls = [int(x) for x in gen.ragged_lengths(w)]
    pick = sorted(gen.rng(w.seed, "cpu.ragged").choice(len(Ls), 4, replace=False).tolist())
    zc, zh = gen.pool_logits(w, "csa"), gen.pool_logits(w, "hca")
    reqs, cs, ch = [], [], []
    for r in pick:
        dc = gen.decode_request(w, "csa", r, L=Ls[r], extra_tokens=w.steps, n_queries=w.steps)
        dh = gen.decode_request(w, "hca", r, L=Ls[r], extra_tokens=w.steps, n_queries=w.steps)
        n = Ls[r] + w.steps
        reqs.append((dc, dh))
        cs.append(dict(kc=orc.compress(dc["k"][:n], zc["zk"], w.m_csa),
                       vc=orc.compress(dc["v"][:n], zc["zv"], w.m_csa),
                       kic=orc.compress(dc["ki"][:n], zc["zi"], w.m_csa)))
        ch.append(dict(kc=orc.compress(dh["k"][:n], zh["zk"], w.m_hca),
                       vc=orc.compress(dh["v"][:n], zh["zv"], w.m_hca)))
    _CPU.clear()
    _CPU.update(w=w, reqs=reqs, Ls=[Ls[r] for r in pick], cs=cs, ch=ch)
    done, dt, workers = cpu_pool_run(_task_ragged, budget_s)
    _CPU.clear()
    # a request-step's cost grows with its context: the batch's average
    # request-step costs 1 / (share * 16 / 4) of the sample's
    share = sum(Ls[r] for r in pick) / sum(Ls)
    rate = done / dt * (len(Ls) / len(pick)) * share
    return _baseline(rate, "tok/s", done, dt, workers,
                     f"decode steps (CSA top-{w.k_csa} + HCA) of requests {pick} of the ragged "
                     f"batch (contexts {[Ls[r] for r in pick]}), scaled to the batch by their "
                     f"{share:.3f} share of its tokens")


# ----------------------------------------------------------------------------- workloads

def bench_pro_decode(args, w, K, W):
    """Headline: the 1M-token Pro decode, a CSA and an HCA hsa_decode_step per
    step (fp8 K / V caches with their stashes; bf16, fp8 or fp4 indexer keys)."""
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    L = w.L
    kmix = getattr(args, "kv_mixed", False)
    f4i = getattr(args, "index_fp4", False)
    t0 = time.time()
    lays = {layer: build_decode_state(w, layer, L, T, gen, args.copies, fp8=True,
                                      kmix=kmix,
                                      index_fp4=f4i and layer == "csa")
            for layer in ("csa", "hca")}
    log(f"[bench] {w.name}: state built in {time.time() - t0:.1f}s")
    Oc, Oh = torch.empty_like(lays["csa"][1]["Q"]), torch.empty_like(lays["hca"][1]["Q"])
    ws_c = ws_h = None
    steps = []
    for i in range(args.copies):
        sc = StepCall(T, lays["csa"][0][i], lays["csa"][1], L, Oc, ws_c)
        sh = StepCall(T, lays["hca"][0][i], lays["hca"][1], L, Oh, ws_h)
        ws_c, ws_h = sc.ws, sh.ws            # the copies share one workspace per layer
        steps.append(Seq(sc, sh))
    ms = time_steps(steps, K, W)
    scan_ms, cnt = kernel_avg_ms(T, T.K_INDEXER_SCAN, lambda i: steps[i % len(steps)](), max(16, K))
    kernels = kernel_table(T, lambda i: steps[i % len(steps)](), 8)
    T.check_device_error()
    nv, nvh = nvis(L, w.m_csa, w.n_win), nvis(L, w.m_hca, w.n_win)
    B = w.B
    # indexer key bytes per visible block: 128 (bf16), or 32 bytes of fp4
    # codes + 2 scale bytes
    key_b = 34 if f4i else 128
    scan_bytes = int(B * nv * key_b)
    kv_b = 320 if kmix else 256          # K + V bytes per compressed entry (fp8; mixed K 192)
    step_bytes = B * (nv * key_b + w.k_csa * kv_b + nvh * kv_b + 2 * w.n_win * 512 +
                      4 * w.H * 256)
    extra = {}
    if f4i:
        st = lays["csa"][1]
        q = T.Queries.list(st["pos"], L)
        i8, _ = T.indexer_topk(q, st["qI"], st["w"], lays["csa"][0][0].kic, w.m_csa, w.n_win,
                               w.k_csa, ws_key="recall")
        i16, _ = T.indexer_topk(q, st["qI"], st["w"], st["kic_bf16"], w.m_csa, w.n_win,
                                w.k_csa, ws_key="recall")
        rec = [len(set(i8[b].tolist()) & set(i16[b].tolist())) / w.k_csa for b in range(B)]
        extra["index_recall_vs_bf16_keys"] = round(float(np.mean(rec)), 4)
    roof = roofline_hbm("idx_scan_kernel", w.name, scan_bytes, scan_ms, cnt)
    if f4i:
        roof["traffic"] = None
    del lays, steps
    return {"value": B / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms, "steps": K,
            "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_algorithmic_bytes": int(step_bytes), **extra,
            "config": {"workload": w.name, "batch": B, "context": L, "heads": w.H, "kv_heads": 1,
                       "d": 128, "topk": w.k_csa, "window": w.n_win, "indexer": "4x64",
                       "indexer_keys": "fp4_e2m1+e8m0_per_32" if f4i else "bf16",
                       "layers": "csa+hca (one hsa_decode_step each)",
                       "kv_dtype": ("k: fp8_e4m3 x64 + bf16 rope x64, v: fp8_e4m3+page_scale"
                                    if kmix else "fp8_e4m3+page_scale"),
                       "cache_copies": args.copies},
            "roofline": roof, "kernels": kernels}


def bench_csa_decode(args, w, K, W):
    """CSA decode step at 128K, batch 32 (one hsa_decode_step per step)."""
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    L = w.L
    nd = getattr(args, "draft", 1)
    t0 = time.time()
    layers, step = build_decode_state(w, "csa", L, T, gen, args.copies, draft=nd)
    log(f"[bench] {w.name}: state built in {time.time() - t0:.1f}s")
    O = torch.empty_like(step["Q"])
    if nd > 1:
        calls = [DraftCall(T, lay, step, L + nd - 1, O, nd) for lay in layers]
    else:
        ws = None
        calls = []
        for lay in layers:
            c = StepCall(T, lay, step, L, O, ws)
            ws = c.ws
            calls.append(c)
    ms = time_steps(calls, K, W)
    scan_ms, cnt = kernel_avg_ms(T, T.K_INDEXER_SCAN, lambda i: calls[i % len(calls)](),
                                 max(16, K))
    kernels = kernel_table(T, lambda i: calls[i % len(calls)](), 8)
    T.check_device_error()
    nv = nvis(L, w.m_csa, w.n_win)
    scan_bytes = w.B * nv * 128
    step_bytes = w.B * (nv * 128 + nd * (w.k_csa * 512 + w.n_win * 512 + 2 * w.H * 128 * 2))
    del layers, calls
    roof = roofline_hbm("idx_scan_kernel", w.name, scan_bytes, scan_ms, cnt)
    if nd > 1:
        roof["traffic"] = None
    return {"value": w.B * nd / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms, "steps": K,
            "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_algorithmic_bytes": int(step_bytes),
            "config": {"workload": w.name, "batch": w.B, "context": L, "heads": w.H, "kv_heads": 1,
                       "d": 128, "topk": w.k_csa, "window": w.n_win, "indexer": "4x64",
                       "kv_dtype": "bf16", "cache_copies": args.copies,
                       **({"draft_tokens": nd} if nd > 1 else {})},
            "roofline": roof, "kernels": kernels}


def bench_prefill(args, w):
    """128K hybrid prefill: one pass = compression of both layers (CSA K, V and
    indexer keys; HCA K, V), the CSA indexer + top-k and attention, and the HCA
    attention.  Median of 5 passes of each layer."""
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    Tn = w.T
    st = {}
    t0 = time.time()
    for layer in ("csa", "hca"):
        inp = gen.prefill_layer(w, layer)
        m = w.m(layer)
        d = {"Q": bf(inp["q"]), "m": m, "tok": {}, "alpha": {}, "cache": {}}
        for name, x, zn in [("kc", "k", "zk"), ("vc", "v", "zv")] + \
                ([("kic", "ki", "zi")] if layer == "csa" else []):
            d["tok"][x] = T.Tokens(bf(inp[x])[None].contiguous())
            d["alpha"][name] = T.pooling_weights(torch.from_numpy(inp[zn]).cuda())
            d["cache"][name] = (T.PagedCache.allocate(1, Tn // m, inp[x].shape[1]), x)
        if layer == "csa":
            d["qI"], d["w"] = bf(inp["qi"]), torch.from_numpy(inp["w"]).cuda()
        st[layer] = d
        if not args.no_cpu_baseline:
            _PREFILL_INPUTS[layer] = inp
        del inp
    log(f"[bench] {w.name}: inputs built in {time.time() - t0:.1f}s")
    q = T.Queries.span(Tn)
    s16 = getattr(args, "index_bf16_scores", False)

    def compress(layer):
        d = st[layer]
        for name, (c, x) in d["cache"].items():
            T.kv_compress(d["tok"][x], c, 0, 0, Tn // d["m"], d["m"], d["alpha"][name])

    def select(bf16_scores):
        d = st["csa"]
        return T.indexer_topk(q, d["qI"], d["w"], d["cache"]["kic"][0], w.m_csa, w.n_win, w.k_csa,
                              bf16_scores=bf16_scores)[0]

    def csa_serial():
        compress("csa")
        d = st["csa"]
        idx = select(s16)
        T.csa_attn(q, d["Q"], d["tok"]["k"], d["tok"]["v"], w.n_win, d["cache"]["kc"][0],
                   d["cache"]["vc"][0], w.m_csa, idx, w.k_csa)

    def csa():
        # the layer's selection and attention in one call, pipelined over
        # stages of queries (the bf16-score option keeps the separate calls)
        if s16 or getattr(args, "csa_separate_calls", False):
            return csa_serial()
        compress("csa")
        d = st["csa"]
        T.csa_prefill(q, d["qI"], d["w"], d["cache"]["kic"][0], d["Q"], d["tok"]["k"],
                      d["tok"]["v"], w.n_win, d["cache"]["kc"][0], d["cache"]["vc"][0], w.m_csa,
                      w.k_csa)

    def hca():
        compress("hca")
        d = st["hca"]
        T.hca_attn(q, d["Q"], d["tok"]["k"], d["tok"]["v"], w.n_win, d["cache"]["kc"][0],
                   d["cache"]["vc"][0], w.m_hca)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    n = 5
    ms_csa, ms_hca = timed(csa, n), timed(hca, n)
    tot = ms_csa + ms_hca
    ms_csa_serial = timed(csa_serial, n)
    # per-kernel averages over 2 more passes of each layer, the CSA layer as
    # separate calls on one stream (no kernel shares the GPU with another)
    att_csa_ms, _ = kernel_avg_ms(T, T.K_ATTN, lambda i: csa_serial(), 2)
    att_hca_ms, _ = kernel_avg_ms(T, T.K_ATTN, lambda i: hca(), 2)
    gemm_ms, gemm_n = kernel_avg_ms(T, T.K_INDEXER_GEMM, lambda i: csa_serial(), 2)
    sel_ms, sel_n = kernel_avg_ms(T, T.K_INDEXER_SEL, lambda i: csa_serial(), 2)
    comp_c_ms, comp_c_n = kernel_avg_ms(T, T.K_COMPRESS, lambda i: compress("csa"), 2)
    comp_h_ms, comp_h_n = kernel_avg_ms(T, T.K_COMPRESS, lambda i: compress("hca"), 2)
    T.check_device_error()
    # algorithmic work: attention 4*H*d flops per (query, entry); indexer 2*4*64
    # per (query, visible block); compression reads m*dim*2 bytes and writes
    # dim*2 bytes per entry
    t = np.arange(Tn)
    s = np.maximum(0, t - w.n_win + 1)
    nw_ = t - s + 1
    nv_c = np.minimum(-(-s // w.m_csa), (t + 1) // w.m_csa)
    nv_h = np.minimum(-(-s // w.m_hca), (t + 1) // w.m_hca)
    fl_csa_att = float(np.sum(nw_ + np.minimum(nv_c, w.k_csa))) * 4 * w.H * 128
    fl_idx = float(np.sum(nv_c)) * 2 * 4 * 64
    fl_hca = float(np.sum(nw_ + nv_h)) * 4 * w.H * 128
    comp_bytes = {"csa": Tn * (128 + 128 + 64) * 2 + (Tn // w.m_csa) * (128 + 128 + 64) * 2,
                  "hca": Tn * (128 + 128) * 2 + (Tn // w.m_hca) * (128 + 128) * 2}
    comp_ms = {"csa": comp_c_ms * comp_c_n / 2, "hca": comp_h_ms * comp_h_n / 2}
    frac = lambda fl, ms_: round(fl / (ms_ * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    hfrac = lambda b, ms_: round(b / (ms_ * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    kernels = {"attn_kernel (CSA)": {"ms": round(att_csa_ms, 4), "mfma_frac": frac(fl_csa_att, att_csa_ms)},
               "attn_pair_kernel (HCA)": {"ms": round(att_hca_ms, 4), "mfma_frac": frac(fl_hca, att_hca_ms)},
               "idx_gemm_kernel": {"ms_total": round(gemm_ms * gemm_n / 2, 4),
                                   "launches": gemm_n // 2,
                                   "mfma_frac": frac(fl_idx, gemm_ms * gemm_n / 2)},
               "selection (histogram + top-k)": {"ms_total": round(sel_ms * sel_n / 2, 4)},
               "compress (CSA K, V, KI)": {"ms_total": round(comp_ms["csa"], 4),
                                           "bytes": comp_bytes["csa"],
                                           "hbm_frac": hfrac(comp_bytes["csa"], comp_ms["csa"])},
               "compress (HCA K, V)": {"ms_total": round(comp_ms["hca"], 4),
                                       "bytes": comp_bytes["hca"],
                                       "hbm_frac": hfrac(comp_bytes["hca"], comp_ms["hca"])}}
    # dominant kernel: the attention launch with the larger share of the pair
    if att_hca_ms >= att_csa_ms:
        roof = roofline_mfma("attn_pair_kernel", w.name, fl_hca, att_hca_ms, 2)
    else:
        roof = roofline_mfma("attn_kernel", w.name, fl_csa_att, att_csa_ms, 2)
    extra = {}
    if s16:
        ms32, ms16 = timed(lambda: select(False), n), timed(lambda: select(True), n)
        i32, i16 = select(False).clone(), select(True).clone()
        big = torch.iinfo(torch.int32).max
        i16s = torch.where(i16 < 0, torch.full_like(i16, big), i16)
        pos = torch.searchsorted(i16s, torch.where(i32 < 0, torch.full_like(i32, big), i32))
        hit = (i16s.gather(1, pos.clamp(max=w.k_csa - 1)) == i32) & (i32 >= 0)
        extra = {"selector_ms_fp32_scores": round(ms32, 4), "selector_ms_bf16_scores": round(ms16, 4),
                 "index_recall_vs_fp32_scores": round(hit.sum().item() / (i32 >= 0).sum().item(), 5)}
        del i32, i16, i16s, pos, hit
    del st
    return {"value": Tn / (tot * 1e-3) / 1e3, "unit": "Ktok/s", "ms_per_step": tot, "steps": 2 * n,
            "ms_csa_layer": round(ms_csa, 4), "ms_hca_layer": round(ms_hca, 4),
            "ms_csa_layer_unpipelined": round(ms_csa_serial, 4),
            "pair_mfma_frac": frac(fl_csa_att + fl_idx + fl_hca, tot),
            "algorithmic_tflop": round((fl_csa_att + fl_idx + fl_hca) / 1e12, 3), **extra,
            "config": {"workload": w.name, "T": Tn, "heads": w.H, "kv_heads": 1, "d": 128,
                       "topk": w.k_csa, "window": w.n_win, "layers": "csa+hca", "planted": True,
                       "timed_pass": "compress + indexer + top-k + attention, both layers",
                       "csa_layer": ("separate indexer_topk + csa_attn calls"
                                     if s16 or getattr(args, "csa_separate_calls", False) else
                                     "hsa_csa_prefill: the selections of the next stages beside "
                                     "the attention of each stage (16384-query stages)"),
                       **({"index_scores": "bf16"} if s16 else {})},
            "roofline": roof, "kernels": kernels}


def _ragged_cache(T, torch, need, dim, name, w, gen):
    """A bf16 paged cache whose pool holds exactly the pages the requests need,
    handed out in a seeded shuffled order (table rows past a request's need
    repeat its first page and are never read)."""
    pages = [-(-max(1, n) // 64) for n in need]
    ppr = max(pages)
    perm = gen.page_permutation(w, name, sum(pages))
    table = np.zeros((len(need), ppr), dtype=np.int32)
    o = 0
    for r, p in enumerate(pages):
        table[r, :p] = perm[o:o + p]
        table[r, p:] = perm[o]
        o += p
    data = torch.zeros((sum(pages), 64, dim), dtype=torch.bfloat16, device="cuda")
    return T.PagedCache(data, torch.from_numpy(table).cuda(),
                        torch.zeros(len(need), dtype=torch.int32, device="cuda"))


def bench_ragged(args, w):
    """Ragged serving: 16 requests, 256 decode steps of a CSA and an HCA layer
    (one hsa_decode_step each; blocks appended every 4 / 128 tokens).
    RAGGED_COPIES independent copies of the batch take the steps in turn, so a
    step does not find its copy's indexer keys in the Infinity Cache; every
    copy runs all 256 steps.  The whole run is one HIP graph, replayed once
    untimed and once timed, the caches' entry counts restored before each."""
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    Ls = [int(x) for x in gen.ragged_lengths(w)]
    B, S = len(Ls), w.steps
    t0 = time.time()
    state = {}
    for layer in ("csa", "hca"):
        m = w.m(layer)
        z = gen.pool_logits(w, layer)
        alpha = {k: T.pooling_weights(torch.from_numpy(z["z" + k]).cuda())
                 for k in (["k", "v", "i"] if layer == "csa" else ["k", "v"])}
        need = [(x + S) // m + 1 for x in Ls]
        names = ["kc", "vc"] + (["kic"] if layer == "csa" else [])
        caches = {n: _ragged_cache(T, torch, need, 64 if n == "kic" else 128, f"ragged.{layer}", w,
                                   gen) for n in names}
        ring_k = torch.zeros((B, w.n_win, 128), dtype=torch.bfloat16, device="cuda")
        ring_v = torch.zeros_like(ring_k)
        tail = torch.zeros((B, m, 64), dtype=torch.bfloat16, device="cuda") if layer == "csa" else None
        ins = {k: [] for k in ("Q", "k_new", "v_new", "qI", "kI_new", "w")}
        for r, L in enumerate(Ls):
            d = gen.decode_request(w, layer, r, L=L, extra_tokens=S, n_queries=S)
            nb = L // m
            for name, x, a in [("kc", "k", "k"), ("vc", "v", "v")] + \
                    ([("kic", "ki", "i")] if layer == "csa" else []):
                T.kv_compress(T.Tokens(bf(d[x][:L])[None].contiguous()), caches[name], r, 0, nb, m,
                              alpha[a])
            lo = max(0, L - w.n_win)
            ring_k[r, torch.arange(lo, L) % w.n_win] = bf(d["k"][lo:L])
            ring_v[r, torch.arange(lo, L) % w.n_win] = bf(d["v"][lo:L])
            if layer == "csa":
                tail[r, torch.arange(nb * m, L) % m] = bf(d["ki"][nb * m:L])
                ins["qI"].append(d["qi"])
                ins["kI_new"].append(d["ki"][L:L + S])
                ins["w"].append(d["w"])
            ins["Q"].append(d["q"])
            ins["k_new"].append(d["k"][L:L + S])
            ins["v_new"].append(d["v"][L:L + S])
            del d
            torch.cuda.synchronize()
        # per-step inputs [S][B][...]
        steps_in = {k: bf(np.stack(v, axis=1)) for k, v in ins.items() if v and k != "w"}
        if layer == "csa":
            steps_in["w"] = torch.from_numpy(np.stack(ins["w"], axis=1)).cuda()
        pos = torch.tensor([[L + s for L in Ls] for s in range(S)], dtype=torch.int64, device="cuda")
        copies = []
        for c in range(RAGGED_COPIES):
            cl = lambda pc: T.PagedCache(pc.data.clone(), pc.page_table, pc.n_entries.clone())
            cc = caches if c == 0 else {k: cl(v) for k, v in caches.items()}
            kw = dict(kind=T.LAYER_CSA if layer == "csa" else T.LAYER_HCA, H=w.H, n_win=w.n_win,
                      m=m, alpha_k=alpha["k"], alpha_v=alpha["v"],
                      ring_k=T.Tokens(ring_k if c == 0 else ring_k.clone()),
                      ring_v=T.Tokens(ring_v if c == 0 else ring_v.clone()),
                      kc=cc["kc"], vc=cc["vc"])
            if layer == "csa":
                kw.update(topk=w.k_csa, alpha_i=alpha["i"],
                          tail_i=T.Tokens(tail if c == 0 else tail.clone()), kic=cc["kic"])
            copies.append(T.Layer(**kw))
        state[layer] = {"copies": copies, "in": steps_in, "pos": pos, "names": names}
    log(f"[bench] {w.name}: state built in {time.time() - t0:.1f}s")
    max_pos = max(Ls) + S
    O = {l: torch.empty((B, w.H, 128), dtype=torch.bfloat16, device="cuda") for l in ("csa", "hca")}
    ws = {}
    calls = []        # call i: copy i % RAGGED_COPIES at its step i // RAGGED_COPIES
    for i in range(S * RAGGED_COPIES):
        c, s = i % RAGGED_COPIES, i // RAGGED_COPIES
        pair = []
        for layer in ("csa", "hca"):
            sl = state[layer]
            step = {k: v[s] for k, v in sl["in"].items()}
            step["pos"] = sl["pos"][s]
            sc = StepCall(T, sl["copies"][c], step, max_pos, O[layer], ws.get(layer))
            ws[layer] = sc.ws
            pair.append(sc)
        calls.append(Seq(*pair))
    entries0 = [(getattr(lay, n).n_entries, getattr(lay, n).n_entries.clone())
                for l in ("csa", "hca") for lay in state[l]["copies"] for n in state[l]["names"]]

    def restore():
        for dst, src in entries0:
            dst.copy_(src)
        torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        with torch.cuda.graph(g, stream=s_):
            for cl_ in calls:
                cl_()
    torch.cuda.synchronize()
    restore()
    g.replay()
    torch.cuda.synchronize()
    restore()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    del g
    T.check_device_error()
    ms = total_ms / len(calls)
    # the dominant kernel's live duration: the scan over all 256 steps of copy 0
    restore()
    # (no warm-up calls: the steps advance every request's position in order)
    scan_ms, cnt = kernel_avg_ms(T, T.K_INDEXER_SCAN, lambda i: calls[i * RAGGED_COPIES](), S,
                                 warm=0)
    restore()
    T.check_device_error()
    # algorithmic bytes per step (averaged over the 256 steps), from the seeded lengths
    scan_b = step_b = 0.0
    for s in range(S):
        for L in Ls:
            t = L + s
            nc, nh = nvis(t, w.m_csa, w.n_win), nvis(t, w.m_hca, w.n_win)
            scan_b += nc * 128
            step_b += (nc * 128 + min(nc, w.k_csa) * 512 + nh * 512 + 2 * w.n_win * 512 +
                       2 * w.H * 128 * 2 * 2)
    scan_b /= S
    step_b /= S
    del calls, state
    return {"value": B / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms,
            "steps": S * RAGGED_COPIES, "total_ms_256_steps": round(ms * S, 3),
            "step_hbm_frac": round(step_b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_algorithmic_bytes": int(step_b),
            "config": {"workload": w.name, "requests": B, "contexts": Ls, "decode_steps": S,
                       "heads": w.H, "kv_heads": 1, "d": 128, "topk": w.k_csa, "window": w.n_win,
                       "layers": "csa+hca (one hsa_decode_step each)", "kv_dtype": "bf16",
                       "pages": "64 entries, shuffled pool", "batch_copies": RAGGED_COPIES},
            "roofline": roofline_hbm("idx_scan_kernel", w.name, scan_b, scan_ms, cnt)}


# ----------------------------------------------------------------------------- calibration

def calibrate_read(nbytes=134_217_728, reps=48):
    """Per-launch time of a library reduction (row maxima of a [n, 4096] fp32
    tensor) that reads nbytes once and writes almost nothing, over 8 buffers
    so the Infinity Cache cannot hold them: the reference point for a single
    streaming pass over as many bytes as the decode scan reads."""
    import torch
    bufs = [torch.randn(nbytes // 4 // 4096, 4096, device="cuda") for _ in range(8)]
    out = torch.empty(bufs[0].shape[0], device="cuda")
    ms = []
    for i in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.amax(bufs[i % 8], dim=1, out=out)
        e1.record()
        e1.synchronize()
        if i >= 8:
            ms.append(e0.elapsed_time(e1))
    mean = sum(ms) / len(ms)
    return {"calibration": "read", "bytes": nbytes, "mean_us": round(mean * 1e3, 2),
            "best_us": round(min(ms) * 1e3, 2), "mean_TBps": round(nbytes / (mean * 1e-3) / 1e12, 3)}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed steps of the headline decode")
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--copies", type=int, default=COPIES)
    ap.add_argument("--workload", default="all",
                    choices=["all", "pro_decode_1m", "csa_decode_128k", "hybrid_prefill_128k",
                             "ragged_serving"],
                    help="all (default): the Pro decode as the headline, the other three in "
                         "`workloads`; a name: only that workload (for profiling)")
    ap.add_argument("--draft", type=int, default=1,
                    help="csa_decode_128k: verify a draft of N tokens per request (1-3 at the "
                         "128K position: no block completes inside it, so replays append "
                         "nothing); tok/s counts draft tokens")
    ap.add_argument("--index-fp4", action="store_true",
                    help="pro_decode_1m: fp4 indexer keys (e2m1, an e8m0 scale per 32 channels; "
                         "the indexer computes in FP4); also reports the selection recall "
                         "against bf16 keys")
    ap.add_argument("--kv-mixed", action="store_true",
                    help="pro_decode_1m: K caches hold mixed entries (the 64 RoPE channels bf16, "
                         "the other 64 fp8 with a page scale); V stays fp8")
    ap.add_argument("--index-bf16-scores", action="store_true",
                    help="hybrid_prefill_128k: the CSA selector ranks index scores rounded to bf16 "
                         "(hsa_indexer_topk_bf16_scores); also times the selector alone both ways "
                         "and reports the recall of the fp32-score selection")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--csa-separate-calls", action="store_true",
                    help="prefill: time the CSA layer as hsa_indexer_topk + hsa_csa_attn "
                         "instead of hsa_csa_prefill (the library's pipeline streams are then "
                         "never created; used for counter runs)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work per workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--calibrate-read", action="store_true",
                    help="only time single launches of a plain 134 MB read (row maxima), "
                         "rotating over 8 buffers: what one pass over the scan's bytes costs")
    ap.add_argument("--traffic-summary", nargs=6,
                    metavar=("KERNEL", "WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                             "COPY_WRITE_CSV"),
                    help="(no GPU) turn rocprofv3 --pmc counter files into HBM bytes per launch")
    ap.add_argument("--grid", type=int, default=None,
                    help="--traffic-summary: only launches of this grid size (threads)")
    ap.add_argument("--label", default="",
                    help="--traffic-summary: suffix of the summary's name (e.g. csa, hca)")
    ap.add_argument("--mfma-summary", nargs=4,
                    metavar=("KERNEL", "WORKLOAD", "PMC_CSV", "ALGORITHMIC_FLOPS"),
                    help="(no GPU) turn a rocprofv3 --pmc run of the MFMA counters into MFMA "
                         "utilisation per launch")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.mfma_summary:
        mfma_summary(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; how the path would shard "
                                   "over several GPUs is a design note only",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.draft != 1 and (args.workload != "csa_decode_128k" or not 1 <= args.draft <= 3):
        ap.error("--draft takes 1..3 with --workload csa_decode_128k")
    if (args.index_fp4 or args.kv_mixed) and args.workload != "pro_decode_1m":
        ap.error("--index-fp4 / --kv-mixed apply to --workload pro_decode_1m")
    if args.index_bf16_scores and args.workload != "hybrid_prefill_128k":
        ap.error("--index-bf16-scores applies to --workload hybrid_prefill_128k")
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be >= 1 and --warmup >= 0")
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes": 1 << 30}))
        return
    if args.calibrate_read:
        print(json.dumps(calibrate_read()))
        return
    from synth import configs
    K, W = args.steps, args.warmup
    runners = {
        "pro_decode_1m": (lambda: bench_pro_decode(args, configs.PRO_DECODE_1M, K, W),
                          lambda: cpu_baseline_pro_decode(configs.PRO_DECODE_1M, args.cpu_budget)),
        "csa_decode_128k": (lambda: bench_csa_decode(args, configs.CSA_DECODE_128K, K, W),
                            lambda: cpu_baseline_csa_decode(configs.CSA_DECODE_128K, args.cpu_budget)),
        "hybrid_prefill_128k": (lambda: bench_prefill(args, configs.HYBRID_PREFILL_128K),
                                lambda: cpu_baseline_prefill(configs.HYBRID_PREFILL_128K,
                                                             args.cpu_budget)),
        "ragged_serving": (lambda: bench_ragged(args, configs.RAGGED_SERVING),
                           lambda: cpu_baseline_ragged(configs.RAGGED_SERVING, args.cpu_budget)),
    }
    head = "pro_decode_1m" if args.workload == "all" else args.workload
    order = [head] + ([n for n in runners if n != head] if args.workload == "all" else [])
    results = {}
    for name in order:
        t0 = time.time()
        try:
            results[name] = runners[name][0]()
        except Exception as e:   # report it and keep the line
            if name == head:
                raise
            results[name] = {"error": repr(e)[:300]}
        torch.cuda.empty_cache()
        log(f"[bench] {name}: {time.time() - t0:.1f}s on the GPU")
    if not args.no_cpu_baseline:
        for name in order:
            if "error" in results[name]:
                continue
            t0 = time.time()
            results[name]["cpu_baseline"] = runners[name][1]()
            log(f"[bench] {name}: oracle baseline in {time.time() - t0:.1f}s")
    res = results[head]
    line = {"metric": METRIC, "value": round(res["value"], 1), "unit": res["unit"], "n_gpus": 1,
            "steps": res["steps"], "warmup": W, "ms_per_step": round(res["ms_per_step"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) tokens; caches compressed on the GPU)",
            "config": res["config"], "roofline": res["roofline"]}
    for key, v in res.items():
        if key not in line and key not in ("value", "unit", "steps", "ms_per_step"):
            line[key] = v
    if len(order) > 1:
        line["workloads"] = {n: results[n] for n in order[1:]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
