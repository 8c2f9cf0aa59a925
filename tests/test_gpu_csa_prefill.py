"""hsa_csa_prefill (a CSA layer's indexer, top-k and attention over a span,
pipelined over stages on two streams) against the two separate calls on the
same span -- bit for bit -- and, on sampled rows, against the oracle."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def _separate(gc, q, qi, wt, Q, tk, tv, w, out_fp32):
    m, n_win, k = w.m_csa, w.n_win, w.k_csa
    idx, _ = L.indexer_topk(q, qi, wt, gc["kic"], m, n_win, k)
    O, lse = L.csa_attn(q, Q, tk, tv, n_win, gc["kc"], gc["vc"], m, idx, k, with_lse=True,
                        out_fp32=out_fp32)
    return idx, O, lse


@pytest.mark.parametrize("stage_q,out_fp32,page_order", [(1000, True, None), (0, False, "shuffle"),
                                                         (2048, False, None), (4096, True, "shuffle")])
def test_csa_prefill_equals_separate_calls(stage_q, out_fp32, page_order):
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    T_ = inp["k"].shape[0]
    print(f"csa_prefill 4K stage_q={stage_q} fp32={out_fp32} pages={page_order}", flush=True)
    po = (torch.from_numpy(gen.page_permutation(w, "csa_prefill", T_ // w.m_csa // 64))
          if page_order else None)
    gc = T.compress_layer(inp, "csa", w.m_csa, page_order=po)
    q = L.Queries.span(T_)
    qi, wt = T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda()
    Q, tk, tv = T.dev_bf16(inp["q"]), T.tokens(inp["k"]), T.tokens(inp["v"])
    idx0, O0, lse0 = _separate(gc, q, qi, wt, Q, tk, tv, w, out_fp32)
    idx1, O1, lse1 = L.csa_prefill(q, qi, wt, gc["kic"], Q, tk, tv, w.n_win, gc["kc"], gc["vc"],
                                   w.m_csa, w.k_csa, with_lse=True, out_fp32=out_fp32,
                                   stage_q=stage_q)
    # work on the caller's stream after the call sees every stage's output
    s1 = O1.float().sum()
    L.check_device_error()
    assert torch.equal(idx0, idx1)
    assert torch.equal(O0, O1)
    assert torch.equal(lse0, lse1)
    assert float(s1) == float(O0.float().sum())
    # sampled rows against the oracle (stage boundaries and the ragged tail)
    rows = [0, 999, 1000, 2047, 2048, 3000, T_ - 1]
    oc = orc.layer_caches(inp, "csa", w.m_csa, "bf16")
    Ob, idh = T.to_f64(O1), idx1.cpu().numpy()
    for t in rows:
        r = orc.csa_query(t, inp["q"][t], inp["qi"][t], inp["w"][t], inp["k"], inp["v"],
                          oc["kc"], oc["vc"], oc["kic"], w.m_csa, w.n_win, w.k_csa)
        T.check_topk(idh[t], r["scores"], w.k_csa, where=f"row {t}")
        if np.array_equal(idh[t], r["idx"]):
            assert np.max(np.abs(Ob[t] - r["o"])) <= T.OUT_TOL, f"row {t}"


def test_csa_prefill_offset_span():
    """A span that starts past position 0 (a later chunk of a prompt) with a
    ragged last stage."""
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    T_ = inp["k"].shape[0]
    gc = T.compress_layer(inp, "csa", w.m_csa)
    p0, n = 1100, 2901
    print(f"csa_prefill offset span p0={p0} n={n}", flush=True)
    q = L.Queries.span(n, pos0=p0)
    qi = T.dev_bf16(inp["qi"][p0:p0 + n])
    wt = torch.from_numpy(np.ascontiguousarray(inp["w"][p0:p0 + n])).cuda()
    Q = T.dev_bf16(inp["q"][p0:p0 + n])
    tk, tv = T.tokens(inp["k"]), T.tokens(inp["v"])
    idx0, O0, lse0 = _separate(gc, q, qi, wt, Q, tk, tv, w, True)
    idx1, O1, lse1 = L.csa_prefill(q, qi, wt, gc["kic"], Q, tk, tv, w.n_win, gc["kc"], gc["vc"],
                                   w.m_csa, w.k_csa, with_lse=True, out_fp32=True, stage_q=700)
    L.check_device_error()
    assert torch.equal(idx0, idx1) and torch.equal(O0, O1) and torch.equal(lse0, lse1)
    assert T_ >= p0 + n


def test_csa_prefill_graph_replays():
    """hsa_csa_prefill captured in a HIP graph (its own streams join the capture
    through its fork and join events): every replay, with eager calls and host
    synchronisation between them, equals the eager result bit for bit."""
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    T_ = inp["k"].shape[0]
    gc = T.compress_layer(inp, "csa", w.m_csa)
    q = L.Queries.span(T_)
    qi, wt = T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda()
    Q, tk, tv = T.dev_bf16(inp["q"]), T.tokens(inp["k"]), T.tokens(inp["v"])
    args = (q, qi, wt, gc["kic"], Q, tk, tv, w.n_win, gc["kc"], gc["vc"], w.m_csa, w.k_csa)
    idx0, O0, _ = L.csa_prefill(*args, stage_q=1000, ws_key="graph_eager")
    idx0, O0 = idx0.clone(), O0.clone()
    torch.cuda.synchronize()
    print("csa_prefill graph capture", flush=True)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            idx_g, O_g, _ = L.csa_prefill(*args, stage_q=1000, ws_key="graph")
    torch.cuda.synchronize()
    for rep in range(3):
        idx_g.fill_(-7)
        O_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx0), f"replay {rep}: idx"
        assert torch.equal(O_g, O0), f"replay {rep}: O"
        # eager work between the replays
        idx_e, O_e, _ = L.csa_prefill(*args, stage_q=1000, ws_key="graph_eager")
        torch.cuda.synchronize()
        assert torch.equal(O_e, O0)
    L.check_device_error()
    del g
