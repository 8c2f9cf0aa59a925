"""GPU parity of the prefill path (span queries) against the oracle:
compression, indexer top-k, CSA and HCA attention."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def _oracle_caches(inp, layer, m, fp8=False):
    return orc.layer_caches(inp, layer, m, "fp8" if fp8 else "bf16")


def test_pooling_weights_bitexact():
    for m, dim in [(4, 128), (128, 128), (4, 64), (1, 64)]:
        z = (0.1 * np.random.default_rng(m + dim).standard_normal((m, dim))).astype(np.float32)
        got = L.pooling_weights(torch.from_numpy(z).cuda()).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), orc.pooling_weights(z).view(np.uint32)), (m, dim)


@pytest.mark.parametrize("layer,m", [("csa", 4), ("hca", 128)])
def test_compress_bf16_bitexact(layer, m):
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, layer)
    perm = torch.from_numpy(gen.page_permutation(w, "t", -(-4096 // m // 64) or 1))
    gc = T.compress_layer(inp, layer, m, page_order=perm)
    oc = _oracle_caches(inp, layer, m)
    nb = 4096 // m
    for name in gc:
        if name.startswith("alpha"):
            continue
        assert int(gc[name].n_entries[0]) == nb
        assert np.array_equal(T.cache_bits(gc[name], 0, nb), oc[name].bits), name


def test_compress_fp8_bitexact():
    w = configs.shrink(configs.PRO_DECODE_1M, L=16384)
    d = gen.decode_request(w, "hca", 0, L=16384, extra_tokens=0)
    zk = gen.pool_logits(w, "csa")["zk"]
    for m in (4, 128):
        z = zk if m == 4 else gen.pool_logits(w, "hca")["zk"]
        alpha = L.pooling_weights(torch.from_numpy(z).cuda())
        nb = 16384 // m
        c = L.PagedCache.allocate(1, nb, 128, fp8=True)
        L.kv_compress(T.tokens(d["k"]), c, 0, 0, nb, m, alpha)
        codes, scales = orc.store_fp8_pages(orc.compress_exact(d["k"], orc.pooling_weights(z), m))
        assert np.array_equal(T.cache_bits(c, 0, nb), codes), m
        assert np.array_equal(c.logical_scales(0, nb).cpu().numpy().view(np.uint32),
                              scales.view(np.uint32)), m
    L.check_device_error()


def _run_prefill_csa(w, inp, rows=None, page_order=None, out_fp32=True, kmix=False):
    m, n_win, k, T_ = w.m_csa, w.n_win, w.k_csa, inp["k"].shape[0]
    gc = T.compress_layer(inp, "csa", m, page_order=page_order, kmix=kmix)
    q = L.Queries.span(T_)
    qi = T.dev_bf16(inp["qi"])
    wt = torch.from_numpy(inp["w"]).cuda()
    idx, score = L.indexer_topk(q, qi, wt, gc["kic"], m, n_win, k, with_score=True)
    Q = T.dev_bf16(inp["q"])
    tk, tv = T.tokens(inp["k"]), T.tokens(inp["v"])
    O, lse = L.csa_attn(q, Q, tk, tv, n_win, gc["kc"], gc["vc"], m, idx, k, with_lse=True,
                        out_fp32=out_fp32)
    L.check_device_error()
    return idx.cpu().numpy(), score.cpu().numpy(), O, lse.cpu().numpy()


def _check_csa_rows(w, inp, idx, score, O, lse, rows, dtype="bf16"):
    m, n_win, k = w.m_csa, w.n_win, w.k_csa
    oc = orc.layer_caches(inp, "csa", m, dtype)
    Ob = T.to_f64(O)
    n_diff = 0
    for t in rows:
        r = orc.csa_query(t, inp["q"][t], inp["qi"][t], inp["w"][t], inp["k"], inp["v"],
                          oc["kc"], oc["vc"], oc["kic"], m, n_win, k)
        n_diff += T.check_topk(idx[t], r["scores"], k, where=f"row {t}")
        sel = idx[t][idx[t] >= 0]
        # scores reported with the selection are the kernel's fp32 scores
        assert np.allclose(score[t][: len(sel)], r["scores"][sel], rtol=1e-4, atol=1e-3)
        if not np.array_equal(sel, r["idx"][r["idx"] >= 0]):
            # a tie-band swap: compare with the oracle attention over the GPU's selection
            s = orc.window_start(t, n_win)
            K = np.concatenate([nx.bf16_value(inp["k"][s:t + 1]), oc["kc"].values[sel]])
            V = np.concatenate([nx.bf16_value(inp["v"][s:t + 1]), oc["vc"].values[sel]])
            o, l = orc.attend(nx.bf16_value(inp["q"][t]), K, V, T.scale_of())
            r = {"o": o, "lse": l}
        err = np.max(np.abs(Ob[t] - r["o"]))
        assert err <= T.OUT_TOL, f"row {t}: {err}"
        assert np.max(np.abs(lse[t] - r["lse"])) <= T.LSE_TOL, f"row {t} lse"
    return n_diff


def test_prefill_4k_csa_all_rows():
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    idx, score, O, lse = _run_prefill_csa(w, inp)
    _check_csa_rows(w, inp, idx, score, O, lse, range(4096))


def test_prefill_4k_hca_all_rows():
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "hca")
    m, n_win = w.m_hca, w.n_win
    gc = T.compress_layer(inp, "hca", m)
    q = L.Queries.span(4096)
    O, lse = L.hca_attn(q, T.dev_bf16(inp["q"]), T.tokens(inp["k"]), T.tokens(inp["v"]), n_win,
                        gc["kc"], gc["vc"], m, with_lse=True, out_fp32=True)
    L.check_device_error()
    oc = _oracle_caches(inp, "hca", m)
    Ob, lse = T.to_f64(O), lse.cpu().numpy()
    for t in range(4096):
        r = orc.hca_query(t, inp["q"][t], inp["k"], inp["v"], oc["kc"], oc["vc"], m, n_win)
        assert np.max(np.abs(Ob[t] - r["o"])) <= T.OUT_TOL, t
        assert np.max(np.abs(lse[t] - r["lse"])) <= T.LSE_TOL, t


@pytest.mark.parametrize("H,n_win,k,T_", [(32, 100, 40, 1037), (48, 128, 7, 777), (16, 4, 3, 300)])
def test_prefill_ragged_shapes(H, n_win, k, T_):
    """Odd lengths, a window that is not a tile multiple, H served by 2- and
    1-wave workgroups, shuffled pages."""
    w = configs.shrink(configs.PREFILL_4K, H=H, n_win=n_win, k_csa=k, T=T_,
                       m_hca=min(128, n_win))
    inp = gen.prefill_layer(w, "csa")
    perm = torch.from_numpy(gen.page_permutation(w, "r", max(1, -(-(T_ // 4) // 64))))
    idx, score, O, lse = _run_prefill_csa(w, inp, page_order=perm)
    _check_csa_rows(w, inp, idx, score, O, lse, range(T_))
    inp = gen.prefill_layer(w, "hca")
    m = min(w.m_hca, n_win)
    gc = T.compress_layer(inp, "hca", m)
    O, lse = L.hca_attn(L.Queries.span(T_), T.dev_bf16(inp["q"]), T.tokens(inp["k"]),
                        T.tokens(inp["v"]), n_win, gc["kc"], gc["vc"], m, with_lse=True,
                        out_fp32=True)
    L.check_device_error()
    oc = _oracle_caches(inp, "hca", m)
    Ob = T.to_f64(O)
    for t in range(T_):
        r = orc.hca_query(t, inp["q"][t], inp["k"], inp["v"], oc["kc"], oc["vc"], m, n_win)
        assert np.max(np.abs(Ob[t] - r["o"])) <= T.OUT_TOL, t


def test_m1_full_window_is_dense_causal():
    """m = 1 and a window covering the sequence: dense causal MQA (torch SDPA
    in float32 on the CPU as the reference)."""
    w = configs.shrink(configs.PREFILL_4K, T=700, n_win=1024, m_csa=1, m_hca=1, k_csa=8)
    inp = gen.prefill_layer(w, "hca")
    gc = T.compress_layer(inp, "hca", 1)
    O, _ = L.hca_attn(L.Queries.span(700), T.dev_bf16(inp["q"]), T.tokens(inp["k"]),
                      T.tokens(inp["v"]), 1024, gc["kc"], gc["vc"], 1, out_fp32=True)
    q = torch.from_numpy(nx.bf16_value(inp["q"])).float().permute(1, 0, 2)
    kk = torch.from_numpy(nx.bf16_value(inp["k"])).float()[None].expand(16, -1, -1)
    vv = torch.from_numpy(nx.bf16_value(inp["v"])).float()[None].expand(16, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, is_causal=True)
    T.check_out(O, ref.permute(1, 0, 2).double().numpy(), "m=1 dense")


def test_unit_values_and_head_permutation():
    w = configs.shrink(configs.PREFILL_4K, T=1500, k_csa=16)
    inp = gen.prefill_layer(w, "csa")
    one = dict(inp)
    one["v"] = gen.bf16_bits(np.ones((1500, 128), np.float32))
    one["zv"] = inp["zv"]
    idx, _, O, _ = _run_prefill_csa(w, one, out_fp32=False)
    assert np.max(np.abs(T.to_f64(O) - 1.0)) < 1e-6
    perm = np.random.default_rng(0).permutation(16)
    pinp = dict(inp)
    pinp["q"] = np.ascontiguousarray(inp["q"][:, perm])
    _, _, O1, _ = _run_prefill_csa(w, inp)
    _, _, O2, _ = _run_prefill_csa(w, pinp)
    assert torch.equal(O1[:, perm], O2)


def test_bf16_output_is_rounded_fp32_output():
    """The bf16 output store is exactly the round-to-nearest-even of the fp32
    output (same accumulation), for CSA prefill, HCA prefill and decode splits."""
    w = configs.shrink(configs.PREFILL_4K, T=2000, k_csa=32)
    inp = gen.prefill_layer(w, "csa")
    _, _, O32, l32 = _run_prefill_csa(w, inp, out_fp32=True)
    _, _, O16, l16 = _run_prefill_csa(w, inp, out_fp32=False)
    assert torch.equal(O32.to(torch.bfloat16), O16)
    assert np.array_equal(l32, l16)
    wd = configs.shrink(configs.PRO_DECODE_1M, H=128)
    Ls = [3000, 70000]
    st = T.build_state(wd, "hca", Ls, fp8=True)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    q = L.Queries.list(pos, max(Ls))
    Q = T.dev_bf16(np.stack([d["q"][0] for d in st["reqs"]]))
    a, _ = L.hca_attn(q, Q, st["ring_k"], st["ring_v"], wd.n_win, st["kc"], st["vc"], wd.m_hca,
                      out_fp32=True)
    b, _ = L.hca_attn(q, Q, st["ring_k"], st["ring_v"], wd.n_win, st["kc"], st["vc"], wd.m_hca)
    L.check_device_error()
    assert torch.equal(a.to(torch.bfloat16), b)


@pytest.mark.parametrize("H,n_win,m,T_,pos0", [(64, 128, 128, 2049, 0), (128, 64, 16, 1501, 0),
                                               (64, 128, 4, 1200, 37), (64, 32, 8, 1026, 0)])
def test_hca_prefill_query_pairs(H, n_win, m, T_, pos0):
    """The paired-query HCA prefill path (H a multiple of 64, bf16): odd and
    even query counts (a last query without a partner), spans that start at an
    odd position, m from 4 to 128, windows shorter than a tile, shuffled pages;
    every row against the oracle."""
    w = configs.shrink(configs.PREFILL_4K, H=H, n_win=n_win, T=T_, m_hca=m)
    inp = gen.prefill_layer(w, "hca")
    perm = torch.from_numpy(gen.page_permutation(w, "p", max(1, -(-(T_ // m) // 64))))
    gc = T.compress_layer(inp, "hca", m, page_order=perm)
    n = T_ - pos0
    O, lse = L.hca_attn(L.Queries.span(n, pos0), T.dev_bf16(inp["q"][pos0:]), T.tokens(inp["k"]),
                        T.tokens(inp["v"]), n_win, gc["kc"], gc["vc"], m, with_lse=True,
                        out_fp32=True)
    L.check_device_error()
    oc = _oracle_caches(inp, "hca", m)
    Ob, lse = T.to_f64(O), lse.cpu().numpy()
    for i in range(n):
        t = pos0 + i
        r = orc.hca_query(t, inp["q"][t], inp["k"], inp["v"], oc["kc"], oc["vc"], m, n_win)
        assert np.max(np.abs(Ob[i] - r["o"])) <= T.OUT_TOL, t
        assert np.max(np.abs(lse[i] - r["lse"])) <= T.LSE_TOL, t
