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

def build_decode_state(w, layer, L, T, gen, copies, fp8=False, shuffle=False):
    """Caches of B requests holding tokens 0..L-1, rings up to L-1, and the new
    token's inputs (position L).  Returns (layers[copies], step inputs)."""
    import torch
    B, m, n_win = w.B, w.m(layer), w.n_win
    z = gen.pool_logits(w, layer)
    alpha = {k: T.pooling_weights(torch.from_numpy(z["z" + k]).cuda())
             for k in (["k", "v", "i"] if layer == "csa" else ["k", "v"])}
    n_ent = L // m + 2
    ppr = -(-n_ent // 64)
    perm = torch.from_numpy(gen.page_permutation(w, layer, B * ppr)) if shuffle else None
    kc = T.PagedCache.allocate(B, n_ent, 128, fp8=fp8, page_order=perm)
    vc = T.PagedCache.allocate(B, n_ent, 128, fp8=fp8, page_order=perm)
    kic = T.PagedCache.allocate(B, n_ent, 64, page_order=perm) if layer == "csa" else None
    ring_k = torch.zeros((B, n_win, 128), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    tail = torch.zeros((B, m, 64), dtype=torch.bfloat16, device="cuda") if layer == "csa" else None
    inp = {"Q": [], "k_new": [], "v_new": [], "qI": [], "kI_new": [], "w": []}

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    for r in range(B):
        d = gen.decode_request(w, layer, r, L=L)
        nb = L // m
        T.kv_compress(T.Tokens(bf(d["k"][:L])[None].contiguous()), kc, r, 0, nb, m, alpha["k"])
        T.kv_compress(T.Tokens(bf(d["v"][:L])[None].contiguous()), vc, r, 0, nb, m, alpha["v"])
        if layer == "csa":
            T.kv_compress(T.Tokens(bf(d["ki"][:L])[None].contiguous()), kic, r, 0, nb, m, alpha["i"])
            t0 = nb * m
            if t0 < L:
                tail[r, torch.arange(t0, L) % m] = bf(d["ki"][t0:L])
            inp["qI"].append(d["qi"][0])
            inp["kI_new"].append(d["ki"][L])
            inp["w"].append(d["w"][0])
        lo = max(0, L - n_win)
        ring_k[r, torch.arange(lo, L) % n_win] = bf(d["k"][lo:L])
        ring_v[r, torch.arange(lo, L) % n_win] = bf(d["v"][lo:L])
        inp["Q"].append(d["q"][0])
        inp["k_new"].append(d["k"][L])
        inp["v_new"].append(d["v"][L])
        torch.cuda.synchronize()
    step = {"Q": bf(np.stack(inp["Q"])), "k_new": bf(np.stack(inp["k_new"])),
            "v_new": bf(np.stack(inp["v_new"]))}
    if layer == "csa":
        step.update(qI=bf(np.stack(inp["qI"])), kI_new=bf(np.stack(inp["kI_new"])),
                    w=torch.from_numpy(np.stack(inp["w"])).cuda())
    step["pos"] = torch.full((B,), L, dtype=torch.int64, device="cuda")

    def clone_cache(c):
        if c is None:
            return None
        return T.PagedCache(c.data.clone(), c.page_table, c.n_entries.clone(),
                            None if c.scale is None else c.scale.clone())

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


# ----------------------------------------------------------------------------- workloads

def bench_csa_decode(args, w):
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    L = w.L
    t0 = time.time()
    layers, step = build_decode_state(w, "csa", L, T, gen, args.copies)
    log(f"[bench] {w.name}: state built in {time.time() - t0:.1f}s")
    O = torch.empty_like(step["Q"])
    calls = [StepCall(T, lay, step, L, O, f"d{i}") for i, lay in enumerate(layers)]
    ms, n = time_graph(calls, args.steps, args.warmup)
    # dominant kernel: the indexer score scan, timed eagerly
    scan_ms, cnt = kernel_avg_ms(T, T.K_INDEXER_SCAN, lambda i: calls[i % len(calls)](),
                                 max(16, args.steps // 2))
    nv = (L - w.n_win + 1 + w.m_csa - 1) // w.m_csa
    scan_bytes = w.B * nv * 128
    gbs = scan_bytes / (scan_ms * 1e-3) / 1e9
    src = source_hash("indexer.hip", "common.h")
    res = {
        "value": w.B / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms, "steps": n,
        "config": {"workload": w.name, "batch": w.B, "context": L, "heads": w.H, "kv_heads": 1,
                   "d": 128, "topk": w.k_csa, "window": w.n_win, "indexer": "4x64",
                   "kv_dtype": "bf16", "cache_copies": args.copies},
        "roofline": {"bound": "hbm", "kernel": "idx_scan_kernel", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": committed_traffic("idx_scan_kernel", w.name, src),
                     "algorithmic_bytes_per_launch": scan_bytes,
                     "avg_launch_ms": round(scan_ms, 5), "launches_timed": cnt},
    }
    step_bytes = w.B * (nv * 128 + w.k_csa * 512 + w.n_win * 512 + 2 * w.H * 128 * 2)
    res["step_hbm_frac"] = round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    return res, layers, step


def cpu_baseline_csa_decode(w, budget_s):
    """The oracle's decode step (indexer, top-k, attention) on a sample of the
    same requests; caches are precomputed outside the timed region."""
    from oracle import hybrid as orc
    from synth import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
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


def bench_pro_decode(args, w):
    """1M-token Pro decode: CSA (fp8 K/V, top-1024) + HCA (fp8), B = 4.  The
    step runs the three ops (no block completes at t = 2^20)."""
    import torch
    from long_context_hybrid_kv_amd import _lib as T
    from synth import gen
    L = w.L
    lays = {}
    for layer in ("csa", "hca"):
        lays[layer] = build_decode_state(w, layer, L, T, gen, args.copies, fp8=True)
    log(f"[bench] {w.name}: state built")
    B = w.B
    q = T.Queries.list(lays["csa"][1]["pos"], L)
    outs = []

    def one(i):
        lc, sc = lays["csa"][0][i % args.copies], lays["csa"][1]
        lh, sh = lays["hca"][0][i % args.copies], lays["hca"][1]
        idx, _ = T.indexer_topk(q, sc["qI"], sc["w"], lc.kic, w.m_csa, w.n_win, w.k_csa)
        T.csa_attn(q, sc["Q"], lc.ring_k, lc.ring_v, w.n_win, lc.kc, lc.vc, w.m_csa, idx, w.k_csa)
        T.hca_attn(q, sh["Q"], lh.ring_k, lh.ring_v, w.n_win, lh.kc, lh.vc, w.m_hca)

    for i in range(args.warmup):
        one(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = args.steps
    e0.record()
    for i in range(n):
        one(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    scan_ms, _ = kernel_avg_ms(T, T.K_INDEXER_SCAN, one, 16)
    nv = (L - w.n_win + 1 + w.m_csa - 1) // w.m_csa
    nvh = (L - w.n_win + 1 + w.m_hca - 1) // w.m_hca
    scan_bytes = B * nv * 128
    step_bytes = B * (nv * 128 + w.k_csa * 256 + nvh * 256 + 2 * w.n_win * 512 + 4 * w.H * 256)
    return {"value": B / (ms * 1e-3), "unit": "tok/s", "ms_per_step": ms,
            "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "scan_hbm_frac": round(scan_bytes / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "scan_avg_ms": round(scan_ms, 5), "timing": "eager (python launches)",
            "config": {"workload": w.name, "batch": B, "context": L, "heads": w.H,
                       "topk": w.k_csa, "kv_dtype": "fp8_e4m3+page_scale"}}


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

    def csa():
        d = st["csa"]
        idx, _ = T.indexer_topk(q, d["qI"], d["w"], d["kic"], w.m_csa, w.n_win, w.k_csa)
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
    return {"value": Tn / (tot * 1e-3) / 1e3, "unit": "Ktok/s", "ms_per_layer_pair": tot,
            "ms_csa_layer": ms_csa, "ms_hca_layer": ms_hca,
            "mfma_frac": round((fl_csa_att + fl_idx + fl_hca) / (tot * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "algorithmic_tflop": round((fl_csa_att + fl_idx + fl_hca) / 1e12, 3),
            "config": {"workload": w.name, "T": Tn, "heads": w.H, "topk": w.k_csa,
                       "layers": "csa+hca", "planted": True}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--copies", type=int, default=COPIES)
    ap.add_argument("--extra", action="store_true", help="also the 1M Pro decode and 128K prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; multi-GPU sharding is a "
                                   "design note only", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes": 1 << 30}))
        return
    from synth import configs
    w = configs.CSA_DECODE_128K
    res, layers, step = bench_csa_decode(args, w)
    line = {"metric": METRIC, "value": round(res["value"], 1), "unit": res["unit"], "n_gpus": 1,
            "steps": res["steps"], "warmup": args.warmup, "ms_per_step": round(res["ms_per_step"], 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) tokens; caches compressed on the GPU)",
            "config": res["config"], "roofline": res["roofline"],
            "step_hbm_frac": res["step_hbm_frac"]}
    del layers, step
    torch.cuda.empty_cache()
    if args.extra:
        extra = {}
        for fn, wl in ((bench_pro_decode, configs.PRO_DECODE_1M),
                       (bench_prefill, configs.HYBRID_PREFILL_128K)):
            try:
                extra[wl.name] = fn(args, wl)
            except Exception as e:   # report, keep the main line
                extra[wl.name] = {"error": repr(e)[:300]}
            torch.cuda.empty_cache()
        line["extra"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_csa_decode(w, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
