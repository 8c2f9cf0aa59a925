"""Graph replays of the decode paths the benchmark times.  The benchmark
captures its steps in a HIP graph and replays it; here a captured step is
replayed several times, with eager calls of the same step and host
synchronisation in between, and every replay must give the eager result bit
for bit.  Positions are chosen so that no block completes during the step,
which makes the step idempotent (the cache upkeep rewrites the same ring rows).
"""
import numpy as np
import pytest
import torch

from synth import configs

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _replays_match(fn, n=3):
    ref = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            outs = fn()
    torch.cuda.synchronize()
    for i in range(n):
        for t in outs:
            t.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(_bits(a), _bits(b)), f"replay {i}"
        again = fn()                       # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(again, ref):
            assert torch.equal(_bits(a), _bits(b)), f"eager call after replay {i}"
    L.check_device_error()


def _step_inputs(st, Ls, n_tok):
    reqs = st["reqs"]
    pick = (lambda f: np.stack([f(r, d, 0) for r, d in enumerate(reqs)])) if n_tok == 1 else \
        (lambda f: np.stack([np.stack([f(r, d, i) for i in range(n_tok)])
                             for r, d in enumerate(reqs)]))
    x = dict(Q=T.dev_bf16(pick(lambda r, d, i: d["q"][i])),
             k_new=T.dev_bf16(pick(lambda r, d, i: d["k"][Ls[r] + i])),
             v_new=T.dev_bf16(pick(lambda r, d, i: d["v"][Ls[r] + i])))
    if "kic" in st:
        x.update(qI=T.dev_bf16(pick(lambda r, d, i: d["qi"][i])),
                 kI_new=T.dev_bf16(pick(lambda r, d, i: d["ki"][Ls[r] + i])),
                 w=torch.from_numpy(pick(lambda r, d, i: d["w"][i])).cuda())
    return x


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_decode_step_graph_replays(layer):
    w = configs.shrink(configs.CSA_DECODE_128K, B=4)
    Ls = [1001, 5001, 20001, 70001]        # (L + 1) % m != 0: no block completes
    st = T.build_state(w, layer, Ls)
    lay = T.layer_of(w, layer, st)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    x = _step_inputs(st, Ls, 1)

    def step():
        O, lse, idx = L.decode_step(lay, pos, max(Ls), with_lse=True, with_idx=True, **x)
        return [O, lse] + ([idx] if idx is not None else [])

    _replays_match(step)


def test_decode_draft_graph_replays():
    w = configs.shrink(configs.CSA_DECODE_128K, B=4)
    n_tok = 3
    Ls = [1000, 5000, 20000, 70000]        # L % 4 == 0: no block completes in L .. L+2
    st = T.build_state(w, "csa", Ls, steps=n_tok, ring_cap=w.n_win + n_tok - 1,
                       tail_cap=w.m_csa + n_tok - 1)
    lay = T.layer_of(w, "csa", st)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    x = _step_inputs(st, Ls, n_tok)

    def step():
        O, lse, idx = L.decode_draft(lay, pos, max(Ls) + n_tok - 1, with_lse=True, with_idx=True,
                                     **x)
        return [O, lse, idx]

    _replays_match(step)


def test_pro_ops_graph_replays():
    """The 1M Pro step's ops (indexer, top-k, CSA and HCA attention over fp8
    caches) at shorter rows; the new tokens are written into the rings before
    the capture (the ops read them, the step itself writes nothing)."""
    Ls = [3000, 70001]
    w = configs.shrink(configs.PRO_DECODE_1M, B=len(Ls))
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    q = L.Queries.list(pos, max(Ls))
    prep = {}
    for layer in ("csa", "hca"):
        s = T.build_state(w, layer, Ls, fp8=True)
        for r, d in enumerate(s["reqs"]):
            s["ring_k"].data[r, Ls[r] % w.n_win] = T.dev_bf16(d["k"][Ls[r]])
            s["ring_v"].data[r, Ls[r] % w.n_win] = T.dev_bf16(d["v"][Ls[r]])
        s["Q"] = T.dev_bf16(np.stack([d["q"][0] for d in s["reqs"]]))
        if layer == "csa":
            s["qI"] = T.dev_bf16(np.stack([d["qi"][0] for d in s["reqs"]]))
            s["wt"] = torch.from_numpy(np.stack([d["w"][0] for d in s["reqs"]])).cuda()
        prep[layer] = s

    def step():
        c, h = prep["csa"], prep["hca"]
        idx, _ = L.indexer_topk(q, c["qI"], c["wt"], c["kic"], w.m_csa, w.n_win, w.k_csa)
        O, lse = L.csa_attn(q, c["Q"], c["ring_k"], c["ring_v"], w.n_win, c["kc"], c["vc"],
                            w.m_csa, idx, w.k_csa, with_lse=True, out_fp32=True)
        O2, lse2 = L.hca_attn(q, h["Q"], h["ring_k"], h["ring_v"], w.n_win, h["kc"], h["vc"],
                              w.m_hca, with_lse=True, out_fp32=True)
        return [idx, O, lse, O2, lse2]

    _replays_match(step)
