"""GPU parity of the decode path (listed queries, rings, paged caches) against
the oracle: indexer top-k over long contexts, CSA / HCA attention over bf16 and
fp8 caches, and hsa_decode_step's cache upkeep over several steps."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def build_state(w, layer, Ls, steps=1, fp8=False, shuffle=True):
    """Caches holding tokens 0..L_r-1 of every request, rings/tails up to L_r-1,
    and the per-request token/query streams for `steps` decode steps."""
    B = len(Ls)
    m = w.m(layer)
    n_win = w.n_win
    reqs = [gen.decode_request(w, layer, r, L=int(Ls[r]), extra_tokens=steps, n_queries=steps)
            for r in range(B)]
    z = gen.pool_logits(w, layer)
    max_entries = int(max(Ls)) // m + steps // m + 2
    ppr = -(-max_entries // 64)
    perm = (torch.from_numpy(gen.page_permutation(w, layer, B * ppr)) if shuffle else None)
    def cache(dim, f8):
        return L.PagedCache.allocate(B, max_entries, dim, fp8=f8, page_order=perm)
    st = {"reqs": reqs, "z": z, "m": m}
    st["alpha_k"] = L.pooling_weights(torch.from_numpy(z["zk"]).cuda())
    st["alpha_v"] = L.pooling_weights(torch.from_numpy(z["zv"]).cuda())
    st["kc"], st["vc"] = cache(128, fp8), cache(128, fp8)
    ring_k = torch.zeros((B, n_win, 128), dtype=torch.bfloat16, device="cuda")
    ring_v = torch.zeros_like(ring_k)
    if layer == "csa":
        st["alpha_i"] = L.pooling_weights(torch.from_numpy(z["zi"]).cuda())
        st["kic"] = cache(64, False)
        tail = torch.zeros((B, m, 64), dtype=torch.bfloat16, device="cuda")
    for r, d in enumerate(reqs):
        Lr = int(Ls[r])
        nb = Lr // m
        for name, x, a in [("kc", "k", "alpha_k"), ("vc", "v", "alpha_v")] + \
                ([("kic", "ki", "alpha_i")] if layer == "csa" else []):
            if nb > 0:
                L.kv_compress(T.tokens(d[x][:Lr]), st[name], r, 0, nb, m, st[a])
        lo = max(0, Lr - n_win)
        slots = torch.arange(lo, Lr) % n_win
        ring_k[r, slots] = T.dev_bf16(d["k"][lo:Lr])
        ring_v[r, slots] = T.dev_bf16(d["v"][lo:Lr])
        if layer == "csa":
            t0 = nb * m
            tail[r, torch.arange(t0, Lr) % m] = T.dev_bf16(d["ki"][t0:Lr])
    st["ring_k"], st["ring_v"] = L.Tokens(ring_k), L.Tokens(ring_v)
    if layer == "csa":
        st["tail_i"] = L.Tokens(tail)
    return st


def oracle_row(w, layer, d, t, s, fp8=False):
    """Oracle at position t for request stream d (query row s)."""
    m = w.m(layer)
    z = gen.pool_logits(w, layer)
    kc = orc.compress(d["k"][:t], z["zk"], m, "fp8" if fp8 else "bf16")
    vc = orc.compress(d["v"][:t], z["zv"], m, "fp8" if fp8 else "bf16")
    if layer == "csa":
        kic = orc.compress(d["ki"][:t], z["zi"], m)
        return orc.csa_query(t, d["q"][s], d["qi"][s], d["w"][s], d["k"][: t + 1], d["v"][: t + 1],
                             kc, vc, kic, m, w.n_win, w.k_csa), (kc, vc)
    return orc.hca_query(t, d["q"][s], d["k"][: t + 1], d["v"][: t + 1], kc, vc, m, w.n_win), (kc, vc)


def run_ops(w, layer, st, Ls, s=0):
    """One decode query per request through the separate ops (window already
    holds the new token)."""
    B = len(Ls)
    pos = torch.tensor([int(x) + s for x in Ls], dtype=torch.int64, device="cuda")
    for r, d in enumerate(st["reqs"]):
        p = int(Ls[r]) + s
        st["ring_k"].data[r, p % w.n_win] = T.dev_bf16(d["k"][p])
        st["ring_v"].data[r, p % w.n_win] = T.dev_bf16(d["v"][p])
    q = L.Queries.list(pos, int(pos.max().item()))
    Q = T.dev_bf16(np.stack([d["q"][s] for d in st["reqs"]]))
    out = {}
    if layer == "csa":
        qi = T.dev_bf16(np.stack([d["qi"][s] for d in st["reqs"]]))
        wt = torch.from_numpy(np.stack([d["w"][s] for d in st["reqs"]])).cuda()
        idx, score = L.indexer_topk(q, qi, wt, st["kic"], w.m_csa, w.n_win, w.k_csa, with_score=True)
        O, lse = L.csa_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_csa,
                            idx, w.k_csa, with_lse=True)
        out["idx"] = idx.cpu().numpy()
    else:
        O, lse = L.hca_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"], w.m_hca,
                            with_lse=True)
    L.check_device_error()
    out["O"], out["lse"] = T.to_f64(O), lse.cpu().numpy()
    return out


def compare(w, layer, st, Ls, out, s=0, fp8=False):
    for r, d in enumerate(st["reqs"]):
        t = int(Ls[r]) + s
        ref, (kc, vc) = oracle_row(w, layer, d, t, s, fp8)
        if layer == "csa":
            T.check_topk(out["idx"][r], ref["scores"], w.k_csa, where=f"req {r} t {t}")
            sel = out["idx"][r][out["idx"][r] >= 0]
            if not np.array_equal(sel, ref["idx"][ref["idx"] >= 0]):
                s0 = orc.window_start(t, w.n_win)
                K = np.concatenate([nx.bf16_value(d["k"][s0:t + 1]), kc.values[sel]])
                V = np.concatenate([nx.bf16_value(d["v"][s0:t + 1]), vc.values[sel]])
                o, l = orc.attend(nx.bf16_value(d["q"][s]), K, V, T.scale_of())
                ref = {"o": o, "lse": l}
        err = np.max(np.abs(out["O"][r] - ref["o"]))
        assert err <= T.OUT_TOL, f"req {r} t {t}: {err}"
        assert np.max(np.abs(out["lse"][r] - ref["lse"])) <= T.LSE_TOL, f"req {r} lse"


LS_SMALL = [1, 127, 128, 131, 700, 4099, 9001, 40000]


@pytest.mark.parametrize("H", [64, 128])
def test_csa_decode_ops(H):
    w = configs.shrink(configs.CSA_DECODE_128K, H=H, k_csa=512)
    st = build_state(w, "csa", LS_SMALL)
    out = run_ops(w, "csa", st, LS_SMALL)
    compare(w, "csa", st, LS_SMALL, out)


@pytest.mark.parametrize("fp8", [False, True])
def test_hca_decode_ops(fp8):
    w = configs.shrink(configs.PRO_DECODE_1M, H=128)
    Ls = [1, 200, 1000, 70000, 200000]
    st = build_state(w, "hca", Ls, fp8=fp8)
    out = run_ops(w, "hca", st, Ls)
    compare(w, "hca", st, Ls, out, fp8=fp8)


def test_csa_decode_fp8_ops():
    w = configs.shrink(configs.PRO_DECODE_1M, H=128, k_csa=1024)
    Ls = [3000, 70000]
    st = build_state(w, "csa", Ls, fp8=True)
    out = run_ops(w, "csa", st, Ls)
    compare(w, "csa", st, Ls, out, fp8=True)


def _layer(w, layer, st):
    kw = dict(kind=L.LAYER_CSA if layer == "csa" else L.LAYER_HCA, H=w.H, n_win=w.n_win,
              m=w.m(layer), alpha_k=st["alpha_k"], alpha_v=st["alpha_v"], ring_k=st["ring_k"],
              ring_v=st["ring_v"], kc=st["kc"], vc=st["vc"])
    if layer == "csa":
        kw.update(topk=w.k_csa, alpha_i=st["alpha_i"], tail_i=st["tail_i"], kic=st["kic"])
    return L.Layer(**kw)


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_decode_step_upkeep_and_outputs(layer):
    """Several decode steps through hsa_decode_step: every step's output and
    selection match the oracle recomputed from the full history, and the
    appended cache entries equal a from-scratch compression, bit for bit."""
    w = configs.shrink(configs.RAGGED_SERVING, H=64, k_csa=64)
    Ls = [5, 126, 1000, 1021, 3000, 8190]
    S = 12 if layer == "csa" else 10
    st = build_state(w, layer, Ls, steps=S)
    lay = _layer(w, layer, st)
    max_pos = max(Ls) + S
    m = w.m(layer)
    for s in range(S):
        pos = torch.tensor([x + s for x in Ls], dtype=torch.int64, device="cuda")
        reqs = st["reqs"]
        Q = T.dev_bf16(np.stack([d["q"][s] for d in reqs]))
        kn = T.dev_bf16(np.stack([d["k"][Ls[r] + s] for r, d in enumerate(reqs)]))
        vn = T.dev_bf16(np.stack([d["v"][Ls[r] + s] for r, d in enumerate(reqs)]))
        extra = {}
        if layer == "csa":
            extra = dict(qI=T.dev_bf16(np.stack([d["qi"][s] for d in reqs])),
                         kI_new=T.dev_bf16(np.stack([d["ki"][Ls[r] + s] for r, d in enumerate(reqs)])),
                         w=torch.from_numpy(np.stack([d["w"][s] for d in reqs])).cuda())
        O, lse, idx = L.decode_step(lay, pos, max_pos, Q, kn, vn, with_lse=True,
                                    with_idx=(layer == "csa"), **extra)
        L.check_device_error()
        out = {"O": T.to_f64(O), "lse": lse.cpu().numpy()}
        if idx is not None:
            out["idx"] = idx.cpu().numpy()
        compare(w, layer, st, Ls, out, s=s)
    # caches after the steps equal a from-scratch compression of the history
    for r, d in enumerate(st["reqs"]):
        n = (Ls[r] + S) // m
        for name, x, z in [("kc", "k", "zk"), ("vc", "v", "zv")] + \
                ([("kic", "ki", "zi")] if layer == "csa" else []):
            assert int(st[name].n_entries[r]) == n
            ref = orc.compress(d[x][: Ls[r] + S], st["z"][z], m)
            assert np.array_equal(T.cache_bits(st[name], r, n), ref.bits), (r, name)
