"""Device-side faults that an input can raise without harming the GPU: a
listed request id outside the caches (HSA_FAULT_REQ: the query reads request
0 instead, so every access stays in bounds), and a V value outside fp16's
range (HSA_FAULT_RANGE: V is staged in fp16 for the P V product, so the
affected outputs are not finite and the fault word says so instead of
returning a silent inf)."""
import ctypes as C

import numpy as np
import pytest
import torch

from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu

FAULT_REQ, FAULT_RANGE = 16, 32


def fault_bits():
    """Synchronise, read and clear the fault word (no exception)."""
    bits = C.c_int32(0)
    L.lib().hsa_check_device_error(C.c_void_p(torch.cuda.current_stream().cuda_stream),
                                   C.byref(bits))
    return bits.value


def test_request_id_out_of_range_raises_req_fault():
    w = configs.shrink(configs.CSA_DECODE_128K, B=2, H=64, k_csa=64)
    Ls = [3000, 5000]
    for layer in ("csa", "hca"):
        st = T.build_state(w, layer, Ls)
        assert fault_bits() == 0
        pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
        req = torch.tensor([0, 7], dtype=torch.int32, device="cuda")     # the caches hold 2
        q = L.Queries.list(pos, max(Ls), req=req)
        Q = T.dev_bf16(np.stack([d["q"][0] for d in st["reqs"]]))
        print(f"request id 7 of 2, {layer}", flush=True)
        if layer == "csa":
            qi = T.dev_bf16(np.stack([d["qi"][0] for d in st["reqs"]]))
            wt = torch.from_numpy(np.stack([d["w"][0] for d in st["reqs"]])).cuda()
            idx, _ = L.indexer_topk(q, qi, wt, st["kic"], w.m_csa, w.n_win, w.k_csa)
            assert fault_bits() & FAULT_REQ
            L.csa_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_csa, idx,
                       w.k_csa)
        else:
            L.hca_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_hca)
        assert fault_bits() & FAULT_REQ
        # valid ids raise nothing (the requests swapped, each at its own position)
        pos2 = torch.tensor(Ls[::-1], dtype=torch.int64, device="cuda")
        q = L.Queries.list(pos2, max(Ls), req=torch.tensor([1, 0], dtype=torch.int32, device="cuda"))
        L.hca_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m(layer))
        assert fault_bits() == 0
        del st


def _prefill(inp, layer, w, big_rows, scale_v):
    """A prefill layer whose V rows `big_rows` are multiplied by scale_v."""
    v = nx.bf16_value(inp["v"]).copy()
    v[big_rows] *= scale_v
    inp = dict(inp, v=nx.bf16_bits_from_f64(v))
    m = w.m(layer)
    c = T.compress_layer(inp, layer, m)
    q = L.Queries.span(inp["k"].shape[0])
    tk, tv = T.tokens(inp["k"]), T.tokens(inp["v"])
    if layer == "csa":
        idx, _ = L.indexer_topk(q, T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda(),
                                c["kic"], m, w.n_win, w.k_csa)
        O, _ = L.csa_attn(q, T.dev_bf16(inp["q"]), tk, tv, w.n_win, c["kc"], c["vc"], m, idx,
                          w.k_csa, out_fp32=True)
    else:
        O, _ = L.hca_attn(q, T.dev_bf16(inp["q"]), tk, tv, w.n_win, c["kc"], c["vc"], m,
                          out_fp32=True)
    return O


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_v_beyond_fp16_range_raises_range_fault(layer):
    """bf16 V values near 1e5 (beyond fp16's 65504) in a 600-token prefill:
    the outputs that attend to them are not finite and the range bit is set;
    values of 6e4 stay finite and raise nothing."""
    w = configs.shrink(configs.PREFILL_4K, T=600, k_csa=16)
    inp = gen.prefill_layer(w, layer)
    rows = np.arange(200, 208)
    assert fault_bits() == 0
    print(f"V x 1e5 on rows 200..207, {layer} prefill", flush=True)
    O = _prefill(inp, layer, w, rows, 1e5)
    bits = fault_bits()
    assert bits & FAULT_RANGE, bits
    assert not torch.isfinite(O[200:328]).all()
    O = _prefill(inp, layer, w, rows, 6e4 / 4.5)     # |v| <= ~6e4 for |N(0,1)| <= 4.5
    assert fault_bits() == 0
    assert torch.isfinite(O).all()


def test_v_beyond_fp16_range_raises_range_fault_in_decode_splits():
    """A decode query whose window row carries |v| ~ 1e5: its entries are
    split over workgroups and merged; the merged output is not finite and the
    range bit is set."""
    w = configs.shrink(configs.CSA_DECODE_128K, B=2, H=64, k_csa=512)
    Ls = [40000, 20000]
    st = T.build_state(w, "csa", Ls)
    assert fault_bits() == 0
    big = torch.full((128,), 1e5, dtype=torch.bfloat16, device="cuda")
    st["ring_v"].data[0, (Ls[0] - 3) % w.n_win] = big
    print("decode with a window V row of 1e5", flush=True)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    for r, d in enumerate(st["reqs"]):
        st["ring_k"].data[r, Ls[r] % w.n_win] = T.dev_bf16(d["k"][Ls[r]])
        st["ring_v"].data[r, Ls[r] % w.n_win] = T.dev_bf16(d["v"][Ls[r]])
    q = L.Queries.list(pos, max(Ls))
    qi = T.dev_bf16(np.stack([d["qi"][0] for d in st["reqs"]]))
    wt = torch.from_numpy(np.stack([d["w"][0] for d in st["reqs"]])).cuda()
    idx, _ = L.indexer_topk(q, qi, wt, st["kic"], w.m_csa, w.n_win, w.k_csa)
    O, _ = L.csa_attn(q, T.dev_bf16(np.stack([d["q"][0] for d in st["reqs"]])), st["ring_k"],
                      st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_csa, idx, w.k_csa,
                      out_fp32=True)
    assert fault_bits() & FAULT_RANGE
    assert not torch.isfinite(O[0]).all()
    assert torch.isfinite(O[1]).all()


@pytest.mark.parametrize("H", [64, 16])
def test_page_table_entry_out_of_range_raises_page_fault(H):
    """A K page-table entry outside the pool, on a page that holds selected
    blocks: the CSA decode attention reads zeros for those rows and raises
    HSA_FAULT_PAGE (H = 64 reads the request's page table into LDS, H = 16
    looks each page up in memory); the restored table raises nothing and gives
    the first output back."""
    FAULT_PAGE = 1
    w = configs.shrink(configs.CSA_DECODE_128K, B=2, H=H, k_csa=64)
    Ls = [9000, 6000]
    st = T.build_state(w, "csa", Ls)
    assert fault_bits() == 0
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    q = L.Queries.list(pos, max(Ls))
    Q = T.dev_bf16(np.stack([d["q"][0] for d in st["reqs"]]))
    qi = T.dev_bf16(np.stack([d["qi"][0] for d in st["reqs"]]))
    wt = torch.from_numpy(np.stack([d["w"][0] for d in st["reqs"]])).cuda()
    idx, _ = L.indexer_topk(q, qi, wt, st["kic"], w.m_csa, w.n_win, w.k_csa)
    O0, _ = L.csa_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_csa,
                       idx, w.k_csa, out_fp32=True)
    assert fault_bits() == 0
    r, lp = 1, int(idx[1, 0].item()) // 64          # a page request 1 attends to
    table = st["kc"].page_table
    good = int(table[r, lp].item())
    print(f"H={H}: page table entry ({r}, {lp}) set past the pool", flush=True)
    table[r, lp] = st["kc"].data.shape[0] + 5
    O1, _ = L.csa_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_csa,
                       idx, w.k_csa, out_fp32=True)
    assert fault_bits() & FAULT_PAGE
    assert torch.equal(O1[0], O0[0])                 # request 0 does not use the entry
    assert torch.isfinite(O1).all()
    table[r, lp] = good
    O2, _ = L.csa_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_csa,
                       idx, w.k_csa, out_fp32=True)
    assert fault_bits() == 0
    assert torch.equal(O2, O0)
