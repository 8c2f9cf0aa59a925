#!/usr/bin/env python3
"""Throughput of the hybrid-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra]

Default workload: the CSA decode step at 128K context (batch 32, 64 query
heads, one KV head, d = 128, top-k 512, window 128, indexer 4 x 64, bf16).
A step is one hsa_decode_step of a CSA layer: ring/tail upkeep, lightning
indexer + top-k over the 32,737 visible compressed blocks of every request,
and the gather attention over window + selected entries.  Inputs are seeded
synthetic tokens; the compressed caches are built by hsa_kv_compress before
timing and stay resident in HBM.  Timed steps rotate over 8 independent cache
copies (>= 1 GiB in total) so that the 256 MB Infinity Cache cannot hold the
working set; the 8 steps are captured in one HIP graph and replayed.

Prints ONE JSON line with the metric, a roofline object for the dominant
kernel (the indexer score scan: its algorithmic bytes are the compressed
indexer keys it must read, divided by its average duration measured with HIP
events on its stream) and a cpu_baseline object (the oracle, on a bounded
sample of the same workload, on this host's cores).  --extra adds the 1M-token
Pro decode (fp8 caches, CSA + HCA) and the 128K hybrid prefill to the line.
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- decode state

def build_decode_state(w, layer, L, T, gen, copies, fp8=False, shuffle=False, index_fp8=False,
                       draft=1, kmix=False, index_fp4=False):
    """Caches of B requests holding tokens 0..L-1, rings up to L-1, and the new
    token's inputs (position L).  Returns (layers[copies], step inputs).
    index_fp8: the indexer keys are stored fp8 (e4m3fn, one scale per page), and
    step["kic_bf16"] holds the same keys in bf16 (for the selection recall).
    draft > 1: the step's inputs are [B][draft][...] (tokens L .. L+draft-1) and
    the rings hold n_win + draft - 1 tokens.
    kmix: the K caches hold mixed entries (RoPE channels bf16, the rest fp8; V fp8).
    index_fp4: the indexer keys are stored fp4 (e2m1, an e8m0 scale per 32
    channels); step["kic_bf16"] holds the same keys in bf16."""
    import torch
    B, m, n_win = w.B, w.m(layer), w.n_win
    z = gen.pool_logits(w, layer)
    alpha = {k: T.pooling_weights(torch.from_numpy(z["z" + k]).cuda())
             for k in (["k", "v", "i"] if layer == "csa" else ["k", "v"])}
    n_ent = L // m + 2
    ppr = -(-n_ent // 64)
    perm = torch.from_numpy(gen.page_permutation(w, layer, B * ppr)) if shuffle else None
    kc = T.PagedCache.allocate(B, n_ent, 128, fp8=fp8, page_order=perm, mixed=kmix)
    vc = T.PagedCache.allocate(B, n_ent, 128, fp8=fp8, page_order=perm)
    kic = (T.PagedCache.allocate(B, n_ent, 64, fp8=index_fp8, fp4=index_fp4, page_order=perm)
           if layer == "csa" else None)
    kic16 = (T.PagedCache.allocate(B, n_ent, 64, page_order=perm)
             if layer == "csa" and (index_fp8 or index_fp4) else None)
    cap = n_win + draft - 1
    ring_k = torch.zeros((B, cap, 128), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    tail = (torch.zeros((B, m + draft - 1, 64), dtype=torch.bfloat16, device="cuda")
            if layer == "csa" else None)
    inp = {"Q": [], "k_new": [], "v_new": [], "qI": [], "kI_new": [], "w": []}

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

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
                            None if c.scale is None else c.scale.clone(), c.mixed, c.fp4)

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
    """Pre-marshalled hsa_decode_step arguments (no per-call Python work beyond
    the foreign call)."""

    def __init__(self, T, layer, step, L_max, O, ws_key):
        import torch
        self.T = T
        self.lc = layer.c()
        B = step["pos"].shape[0]
        nb = T.lib().hsa_decode_step_workspace_bytes(C.byref(self.lc), B, L_max)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
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


def time_graph(calls, steps, warmup):
    """Capture one graph of len(calls) steps; replay it; return ms per step."""
    import torch
    for _ in range(max(1, warmup // len(calls))):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
    torch.cuda.synchronize()
    reps = max(1, steps // len(calls))
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(calls)), reps * len(calls)


def kernel_avg_ms(T, kid, fn, n):
    """Average duration of one kernel over n eager calls of fn (HIP events on
    the kernel's stream, recorded by the library around each launch)."""
    import torch
    torch.cuda.synchronize()
    T.kernel_timing_read(kid)
    T.kernel_timing(kid, True)
    for i in range(n):
        fn(i)
    torch.cuda.synchronize()
    T.kernel_timing(kid, False)
    ms, cnt = T.kernel_timing_read(kid)
    return ms / max(cnt, 1), cnt


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_hybrid_kv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("source_hash") != src_hash:
        return None
    return t.get("bytes_per_launch")


def _pmc_per_dispatch(path, counter, kernel_regex):
    """Mean value of one rocprofv3 counter per dispatch of the kernels whose
    name matches kernel_regex (a --pmc run written with --output-format csv)."""
    import csv
    import re
    rx = re.compile(kernel_regex)
    per = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter or not rx.search(row.get("Kernel_Name", "")):
                continue
            key = row.get("Dispatch_Id") or row.get("Correlation_Id")
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {kernel_regex!r}")
    return sum(per.values()) / len(per), len(per)


def traffic_summary(args):
    """HBM-side bytes per launch of a kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the
    same counter reads for an elementwise copy of a known 1 GiB
    (bench.py --calibrate-copy).  Writes profiles/traffic_<kernel>_<workload>.json;
    the benchmark reports it while the kernel's source is unchanged."""
    kernel, workload, fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.traffic_summary
    fk, nf = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE", kernel)
    wk, nw = _pmc_per_dispatch(write_csv, "WRITE_SIZE", kernel)
    cf, _ = _pmc_per_dispatch(cfetch_csv, "FETCH_SIZE", "elementwise")
    cw, _ = _pmc_per_dispatch(cwrite_csv, "WRITE_SIZE", "elementwise")
    kib = float(1 << 20)   # the copy reads and writes 1 GiB
    f_scale, w_scale = kib / cf, kib / cw
    out = {"kernel": kernel, "workload": workload,
           "source_hash": source_hash("indexer.hip", "common.h", "update.h") if kernel.startswith("idx_")
           else source_hash("attention.hip", "common.h"),
           "fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wk, 1),
           "dispatches": [nf, nw],
           "copy_calibration": {"fetch_kib": round(cf, 1), "write_kib": round(cw, 1),
                                "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "bytes_per_launch": int(round((fk * f_scale + wk * w_scale) * 1024))}
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


# ----------------------------------------------------------------------------- workloads

def bench_csa_decode(args, w):
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
        calls = [StepCall(T, lay, step, L, O, f"d{i}") for i, lay in enumerate(layers)]
    ms, n = time_graph(calls, args.steps, args.warmup)
    # dominant kernel: the indexer score scan, timed eagerly
    scan_ms, cnt = kernel_avg_ms(T, T.K_INDEXER_SCAN, lambda i: calls[i % len(calls)](),
                                 max(16, args.steps // 2))
    nv = (L - w.n_win + 1 + w.m_csa - 1) // w.m_csa
    scan_bytes = w.B * nv * 128
    gbs = scan_bytes / (scan_ms * 1e-3) / 1e9
    src = source_hash("indexer.hip", "common.h", "update.h")
    res = {
        "value": w.B * nd / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms, "steps": n,
        "config": {"workload": w.name, "batch": w.B, "context": L, "heads": w.H, "kv_heads": 1,
                   "d": 128, "topk": w.k_csa, "window": w.n_win, "indexer": "4x64",
                   "kv_dtype": "bf16", "cache_copies": args.copies,
                   **({"draft_tokens": nd} if nd > 1 else {})},
        "roofline": {"bound": "hbm", "kernel": "idx_scan_kernel", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if nd > 1 else committed_traffic("idx_scan_kernel", w.name, src),
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "avg_launch_ms": round(scan_ms, 5), "launches_timed": cnt},
    }
    step_bytes = w.B * (nv * 128 + nd * (w.k_csa * 512 + w.n_win * 512 + 2 * w.H * 128 * 2))
    res["step_hbm_frac"] = round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    return res, layers, step


def cpu_baseline_csa_decode(w, budget_s):
    """The oracle's decode step (indexer, top-k, attention) on a sample of the
    same requests; caches are precomputed outside the timed region."""
    from oracle import hybrid as orc
    from synth import gen
    cores = _cores()
    sample = []
    for r in range(2):
        d = gen.decode_request(w, "csa", r)
        z = gen.pool_logits(w, "csa")
        L = w.L
        caches = dict(kc=orc.compress(d["k"][:L], z["zk"], w.m_csa),
                      vc=orc.compress(d["v"][:L], z["zv"], w.m_csa),
                      kic=orc.compress(d["ki"][:L], z["zi"], w.m_csa))
        sample.append((d, caches))
    done, t0 = 0, time.time()
    while time.time() - t0 < budget_s:
        d, c = sample[done % len(sample)]
        orc.csa_query(w.L, d["q"][0], d["qi"][0], d["w"][0], d["k"], d["v"], c["kc"], c["vc"],
                      c["kic"], w.m_csa, w.n_win, w.k_csa)
        done += 1
    dt = time.time() - t0
    return {"value": done / dt, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} decode queries of 2 requests at context {w.L} "
                      f"(indexer over {orc.n_visible(w.L, w.m_csa, w.n_win)} blocks, top-{w.k_csa}, "
                      f"attention over {w.n_win + w.k_csa} entries, float64), {dt:.1f}s"}


class RawCall:
    """A library call with pre-marshalled arguments; the stream is the caller's
    current stream at call time (so the call can be captured in a graph)."""

    def __init__(self, T, fn, args, name):
        self.T, self.fn, self.args, self.name = T, fn, args, name

    def __call__(self):
        import torch
        st = self.fn(*self.args, C.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            self.T._check(st, self.name)


class StepGroup:
    def __init__(self, calls):
        self.calls = calls

    def __call__(self):
        for c in self.calls:
            c()


def pro_decode_calls(T, w, lay_c, st_c, lay_h, st_h, L, keep):
    """indexer_topk + csa_attn (CSA layer) and hca_attn (HCA layer) for one cache copy."""
    import torch
    B = w.B
    p = lambda t: None if t is None else C.c_void_p(t.data_ptr())
    q = T.Queries.list(st_c["pos"], L)
    qc = q.c()
    kic, kc, vc = lay_c.kic.c(), lay_c.kc.c(), lay_c.vc.c()
    wk, wv = lay_c.ring_k.c(), lay_c.ring_v.c()
    kch, vch = lay_h.kc.c(), lay_h.vc.c()
    wkh, wvh = lay_h.ring_k.c(), lay_h.ring_v.c()
    lib = T.lib()
    idx = torch.empty((B, w.k_csa), dtype=torch.int32, device="cuda")
    O_c = torch.empty_like(st_c["Q"])
    O_h = torch.empty_like(st_h["Q"])
    ws_i = torch.empty(max(1, lib.hsa_indexer_topk_workspace_bytes(C.byref(qc), w.m_csa, w.n_win, w.k_csa)),
                       dtype=torch.uint8, device="cuda")
    ws_c = torch.empty(max(1, lib.hsa_csa_attn_workspace_bytes(C.byref(qc), w.H, w.n_win, w.k_csa)),
                       dtype=torch.uint8, device="cuda")
    ws_h = torch.empty(max(1, lib.hsa_hca_attn_workspace_bytes(C.byref(qc), w.H, w.n_win, w.m_hca)),
                       dtype=torch.uint8, device="cuda")
    keep.extend([qc, kic, kc, vc, wk, wv, kch, vch, wkh, wvh, idx, O_c, O_h, ws_i, ws_c, ws_h, q])
    scale = 1.0 / math.sqrt(128)
    ci = RawCall(T, lib.hsa_indexer_topk,
                 (C.byref(qc), p(st_c["qI"]), p(st_c["w"]), 4, 64, C.byref(kic), w.m_csa, w.n_win,
                  w.k_csa, p(idx), None, p(ws_i), ws_i.numel()), "indexer_topk")
    ca = RawCall(T, lib.hsa_csa_attn,
                 (C.byref(qc), p(st_c["Q"]), w.H, 128, C.byref(wk), C.byref(wv), w.n_win, C.byref(kc),
                  C.byref(vc), w.m_csa, p(idx), w.k_csa, C.c_float(scale), p(O_c), T.BF16, None,
                  p(ws_c), ws_c.numel()), "csa_attn")
    ha = RawCall(T, lib.hsa_hca_attn,
                 (C.byref(qc), p(st_h["Q"]), w.H, 128, C.byref(wkh), C.byref(wvh), w.n_win,
                  C.byref(kch), C.byref(vch), w.m_hca, C.c_float(scale), p(O_h), T.BF16, None,
                  p(ws_h), ws_h.numel()), "hca_attn")
    return StepGroup([ci, ca, ha])


def _cores():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return 1


def cpu_baseline_pro_decode(w, budget_s):
    """The oracle's step (indexer, top-k, CSA attention, HCA attention) for one
    request at 1M context; caches (fp8) are precomputed outside the timing."""
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
    done, t0 = 0, time.time()
    while time.time() - t0 < budget_s or done == 0:
        orc.csa_query(L, dc["q"][0], dc["qi"][0], dc["w"][0], dc["k"], dc["v"], cc["kc"], cc["vc"],
                      cc["kic"], w.m_csa, w.n_win, w.k_csa)
        orc.hca_query(L, dh["q"][0], dh["k"], dh["v"], ch["kc"], ch["vc"], w.m_hca, w.n_win)
        done += 1
    dt = time.time() - t0
    return {"value": done / dt, "unit": "tok/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{done} decode steps (CSA top-{w.k_csa} over "
                      f"{orc.n_visible(L, w.m_csa, w.n_win)} blocks + HCA over "
                      f"{orc.n_visible(L, w.m_hca, w.n_win)} entries) of one request at context {L}, "
                      f"float64, {dt:.1f}s"}


def cpu_baseline_prefill(w, budget_s):
    """The oracle's CSA and HCA outputs for sampled query rows of the 128K
    prefill (every 997th row from the end), scaled to Ktok/s of a layer pair."""
    from oracle import hybrid as orc
    from synth import gen
    T = 16384 + 1
    inc = gen.prefill_layer(w, "csa", T=T)
    inh = gen.prefill_layer(w, "hca", T=T)
    cc, ch = orc.layer_caches(inc, "csa", w.m_csa), orc.layer_caches(inh, "hca", w.m_hca)
    rows = list(range(T - 1, 0, -997))
    done, t0 = 0, time.time()
    while (time.time() - t0 < budget_s and done < len(rows)) or done == 0:
        t = rows[done % len(rows)]
        orc.prefill_rows(inc, "csa", [t], w.m_csa, w.n_win, topk=w.k_csa, caches=cc)
        orc.prefill_rows(inh, "hca", [t], w.m_hca, w.n_win, caches=ch)
        done += 1
    dt = time.time() - t0
    return {"value": done / dt / 1e3, "unit": "Ktok/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{done} query rows (CSA + HCA) at positions up to {T - 1} of the planted "
                      f"prefill (a row's cost grows with its position; the full 128K layer has "
                      f"rows up to 131071, so this overstates the oracle's rate), float64, {dt:.1f}s"}


def bench_pro_decode(args, w):
    """1M-token Pro decode: CSA (fp8 K/V, top-1024) + HCA (fp8), batch 4.  A step
    is the indexer + top-k + CSA attention and the HCA attention (no block
    completes at t = 2^20, so there is no cache upkeep to do)."""
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    L = w.L
    f8i = getattr(args, "index_fp8", False)
    kmix = getattr(args, "kv_mixed", False)
    f4i = getattr(args, "index_fp4", False)
    lays = {layer: build_decode_state(w, layer, L, T, gen, args.copies, fp8=True,
                                      index_fp8=f8i and layer == "csa", kmix=kmix,
                                      index_fp4=f4i and layer == "csa")
            for layer in ("csa", "hca")}
    log(f"[bench] {w.name}: state built")
    keep = []
    steps = [pro_decode_calls(T, w, lays["csa"][0][i], lays["csa"][1], lays["hca"][0][i],
                              lays["hca"][1], L, keep) for i in range(args.copies)]
    ms, n = time_graph(steps, args.steps, args.warmup)
    scan_ms, cnt = kernel_avg_ms(T, T.K_INDEXER_SCAN, lambda i: steps[i % len(steps)](), 16)
    nv = (L - w.n_win + 1 + w.m_csa - 1) // w.m_csa
    nvh = (L - w.n_win + 1 + w.m_hca - 1) // w.m_hca
    B = w.B
    # indexer key bytes per visible block: 128 (bf16), 64 fp8 codes + the page
    # scale, or 32 bytes of fp4 codes + 2 scale bytes
    key_b = 64 + 4 / 64 if f8i else (34 if f4i else 128)
    scan_bytes = int(B * nv * key_b)
    # K + V bytes per compressed entry: fp8 128 + 128, or a mixed K row of 192
    kv_b = 320 if kmix else 256
    step_bytes = B * (nv * key_b + w.k_csa * kv_b + nvh * kv_b + 2 * w.n_win * 512 + 4 * w.H * 256)
    gbs = scan_bytes / (scan_ms * 1e-3) / 1e9
    src = source_hash("indexer.hip", "common.h", "update.h")
    extra = {}
    if f8i or f4i:
        # selection recall: how much of each query's top-k over the bf16 keys the
        # low-precision keys select (the same tokens, compressed both ways)
        st = lays["csa"][1]
        q = T.Queries.list(st["pos"], L)
        i8, _ = T.indexer_topk(q, st["qI"], st["w"], lays["csa"][0][0].kic, w.m_csa, w.n_win,
                               w.k_csa, ws_key="recall")
        i16, _ = T.indexer_topk(q, st["qI"], st["w"], st["kic_bf16"], w.m_csa, w.n_win,
                                w.k_csa, ws_key="recall")
        rec = [len(set(i8[b].tolist()) & set(i16[b].tolist())) / w.k_csa for b in range(B)]
        extra["index_recall_vs_bf16_keys"] = round(float(np.mean(rec)), 4)
    return {"value": B / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms, "steps": n,
            "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), **extra,
            "config": {"workload": w.name, "batch": B, "context": L, "heads": w.H, "kv_heads": 1,
                       "d": 128, "topk": w.k_csa, "window": w.n_win, "indexer": "4x64",
                       "indexer_keys": ("fp8_e4m3+page_scale" if f8i else
                                        "fp4_e2m1+e8m0_per_32" if f4i else "bf16"),
                       "layers": "csa+hca",
                       "kv_dtype": ("k: fp8_e4m3 x64 + bf16 rope x64, v: fp8_e4m3+page_scale"
                                    if kmix else "fp8_e4m3+page_scale"),
                       "cache_copies": args.copies},
            "roofline": {"bound": "hbm", "kernel": "idx_scan_kernel", "achieved": round(gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": (None if f8i or f4i
                                     else committed_traffic("idx_scan_kernel", w.name, src)),
                         "algorithmic_bytes_per_launch": scan_bytes,
                         "avg_launch_ms": round(scan_ms, 5), "launches_timed": cnt}}


def bench_prefill(args, w):
    """128K hybrid prefill: one CSA layer and one HCA layer (independent inputs)."""
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    Tn = w.T

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    st = {}
    for layer in ("csa", "hca"):
        inp = gen.prefill_layer(w, layer)
        m = w.m(layer)
        d = {"Q": bf(inp["q"]), "k": T.Tokens(bf(inp["k"])[None].contiguous()),
             "v": T.Tokens(bf(inp["v"])[None].contiguous())}
        for name, x, zn in [("kc", "k", "zk"), ("vc", "v", "zv")] + \
                ([("kic", "ki", "zi")] if layer == "csa" else []):
            a = T.pooling_weights(torch.from_numpy(inp[zn]).cuda())
            c = T.PagedCache.allocate(1, Tn // m, inp[x].shape[1])
            src = d[x] if x in d else T.Tokens(bf(inp[x])[None].contiguous())
            T.kv_compress(src, c, 0, 0, Tn // m, m, a)
            d[name] = c
        if layer == "csa":
            d["qI"], d["w"] = bf(inp["qi"]), torch.from_numpy(inp["w"]).cuda()
        st[layer] = d
        del inp
    log(f"[bench] {w.name}: inputs built")
    q = T.Queries.span(Tn)
    s16 = getattr(args, "index_bf16_scores", False)

    def select(bf16_scores):
        d = st["csa"]
        return T.indexer_topk(q, d["qI"], d["w"], d["kic"], w.m_csa, w.n_win, w.k_csa,
                              bf16_scores=bf16_scores)[0]

    def csa():
        d = st["csa"]
        idx = select(s16)
        T.csa_attn(q, d["Q"], d["k"], d["v"], w.n_win, d["kc"], d["vc"], w.m_csa, idx, w.k_csa)

    def hca():
        d = st["hca"]
        T.hca_attn(q, d["Q"], d["k"], d["v"], w.n_win, d["kc"], d["vc"], w.m_hca)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(2, min(5, args.steps // 10))
    ms_csa, ms_hca = timed(csa, n), timed(hca, n)
    att_csa_ms, _ = kernel_avg_ms(T, T.K_ATTN, lambda i: csa(), 2)
    att_hca_ms, _ = kernel_avg_ms(T, T.K_ATTN, lambda i: hca(), 2)
    # algorithmic MFMA work (flops): attention 4*H*d per (query, entry); indexer 2*4*64 per pair
    nv = lambda t, m: min(-(-max(0, t - w.n_win + 1) // m), (t + 1) // m)
    t = np.arange(Tn)
    s = np.maximum(0, t - w.n_win + 1)
    nw = t - s + 1
    nv_c = np.minimum(-(-s // w.m_csa), (t + 1) // w.m_csa)
    nv_h = np.minimum(-(-s // w.m_hca), (t + 1) // w.m_hca)
    fl_csa_att = float(np.sum(nw + np.minimum(nv_c, w.k_csa))) * 4 * w.H * 128
    fl_idx = float(np.sum(nv_c)) * 2 * 4 * 64
    fl_hca = float(np.sum(nw + nv_h)) * 4 * w.H * 128
    tot = ms_csa + ms_hca
    # dominant kernel: the attention launch with the larger share of the pair
    if att_hca_ms >= att_csa_ms:
        kname, kms, kfl = "attn_pair_kernel (HCA)", att_hca_ms, fl_hca
    else:
        kname, kms, kfl = "attn_kernel (CSA)", att_csa_ms, fl_csa_att
    tf = kfl / (kms * 1e-3) / 1e12
    extra = {}
    if s16:
        # the selector alone with fp32 and with bf16 scores, and how many of the
        # fp32 selection's blocks the bf16 selection keeps (rows ascending,
        # -1 padded: padding sorts last as INT_MAX)
        ms32, ms16 = timed(lambda: select(False), n), timed(lambda: select(True), n)
        i32, i16 = select(False).clone(), select(True).clone()
        big = torch.iinfo(torch.int32).max
        i16s = torch.where(i16 < 0, torch.full_like(i16, big), i16)
        pos = torch.searchsorted(i16s, torch.where(i32 < 0, torch.full_like(i32, big), i32))
        hit = (i16s.gather(1, pos.clamp(max=w.k_csa - 1)) == i32) & (i32 >= 0)
        extra = {"selector_ms_fp32_scores": round(ms32, 4), "selector_ms_bf16_scores": round(ms16, 4),
                 "index_recall_vs_fp32_scores": round(hit.sum().item() / (i32 >= 0).sum().item(), 5)}
        del i32, i16, i16s, pos, hit
    return {"value": Tn / (tot * 1e-3) / 1e3, "unit": "Ktok/s", "ms_per_step": tot, "steps": 2 * n,
            "ms_csa_layer": ms_csa, "ms_hca_layer": ms_hca,
            "ms_attn_csa": att_csa_ms, "ms_attn_hca": att_hca_ms,
            "pair_mfma_frac": round((fl_csa_att + fl_idx + fl_hca) / (tot * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "algorithmic_tflop": round((fl_csa_att + fl_idx + fl_hca) / 1e12, 3),
            **extra,
            "config": {"workload": w.name, "T": Tn, "heads": w.H, "kv_heads": 1, "d": 128,
                       "topk": w.k_csa, "window": w.n_win, "layers": "csa+hca", "planted": True,
                       **({"index_scores": "bf16"} if s16 else {})},
            "roofline": {"bound": "mfma", "kernel": kname, "achieved": round(tf, 2),
                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "algorithmic_flops_per_launch": kfl, "avg_launch_ms": round(kms, 4)}}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--copies", type=int, default=COPIES)
    ap.add_argument("--workload", default="csa_decode_128k",
                    choices=["csa_decode_128k", "pro_decode_1m", "hybrid_prefill_128k"])
    ap.add_argument("--extra", action="store_true", help="also the other two workloads")
    ap.add_argument("--draft", type=int, default=1,
                    help="csa_decode_128k: verify a draft of N tokens per request (1-3 at the "
                         "128K position: no block completes inside it, so replays append "
                         "nothing); tok/s counts draft tokens")
    ap.add_argument("--index-fp8", action="store_true",
                    help="pro_decode_1m with fp8 indexer keys (a next row of the scope: the "
                         "scan reads half the bytes); reports the selection recall against "
                         "bf16 keys")
    ap.add_argument("--index-fp4", action="store_true",
                    help="pro_decode_1m: fp4 indexer keys (e2m1, an e8m0 scale per 32 channels); "
                         "also reports the selection recall against bf16 keys")
    ap.add_argument("--kv-mixed", action="store_true",
                    help="pro_decode_1m: K caches hold mixed entries (the 64 RoPE channels bf16, "
                         "the other 64 fp8 with a page scale); V stays fp8")
    ap.add_argument("--index-bf16-scores", action="store_true",
                    help="hybrid_prefill_128k: the CSA selector ranks index scores rounded to bf16 "
                         "(hsa_indexer_topk_bf16_scores); also times the selector alone both ways "
                         "and reports the recall of the fp32-score selection")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    ap.add_argument("--calibrate-read", action="store_true",
                    help="only time single launches of a plain 134 MB read (row maxima), "
                         "rotating over 8 buffers: what one pass over the scan's bytes costs")
    ap.add_argument("--traffic-summary", nargs=6,
                    metavar=("KERNEL", "WORKLOAD", "FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                             "COPY_WRITE_CSV"),
                    help="(no GPU) turn rocprofv3 --pmc counter files into HBM bytes per launch")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.draft != 1 and (args.workload != "csa_decode_128k" or not 1 <= args.draft <= 3):
        ap.error("--draft takes 1..3 with --workload csa_decode_128k")
    if args.index_fp8 and args.workload != "pro_decode_1m":
        ap.error("--index-fp8 applies to --workload pro_decode_1m")
    if args.index_fp4 and (args.workload != "pro_decode_1m" or args.index_fp8):
        ap.error("--index-fp4 applies to --workload pro_decode_1m (without --index-fp8)")
    if args.kv_mixed and args.workload != "pro_decode_1m":
        ap.error("--kv-mixed applies to --workload pro_decode_1m")
    if args.index_bf16_scores and args.workload != "hybrid_prefill_128k":
        ap.error("--index-bf16-scores applies to --workload hybrid_prefill_128k")
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU sharding is a "
                                   "design note only", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB
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
    runners = {"csa_decode_128k": (lambda a, w: bench_csa_decode(a, w)[0], configs.CSA_DECODE_128K,
                                   cpu_baseline_csa_decode),
               "pro_decode_1m": (bench_pro_decode, configs.PRO_DECODE_1M, cpu_baseline_pro_decode),
               "hybrid_prefill_128k": (bench_prefill, configs.HYBRID_PREFILL_128K,
                                       cpu_baseline_prefill)}
    fn, w, cpu_fn = runners[args.workload]
    res = fn(args, w)
    torch.cuda.empty_cache()
    line = {"metric": METRIC, "value": round(res["value"], 1), "unit": res["unit"], "n_gpus": 1,
            "steps": res["steps"], "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) tokens; caches compressed on the GPU)",
            "config": res["config"], "roofline": res["roofline"]}
    for key in ("step_hbm_frac", "pair_mfma_frac", "ms_csa_layer", "ms_hca_layer",
                "index_recall_vs_bf16_keys", "selector_ms_fp32_scores", "selector_ms_bf16_scores",
                "index_recall_vs_fp32_scores"):
        if key in res:
            line[key] = res[key]
    if args.extra:
        extra = {}
        for name, (efn, ew, _) in runners.items():
            if name == args.workload:
                continue
            try:
                extra[name] = efn(args, ew)
            except Exception as e:   # report, keep the main line
                extra[name] = {"error": repr(e)[:300]}
            torch.cuda.empty_cache()
        line["extra"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_fn(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
