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
    st = T.build_state(w, "csa", LS_SMALL)
    out = T.run_ops(w, "csa", st, LS_SMALL)
    compare(w, "csa", st, LS_SMALL, out)


@pytest.mark.parametrize("fp8", [False, True])
def test_hca_decode_ops(fp8):
    w = configs.shrink(configs.PRO_DECODE_1M, H=128)
    Ls = [1, 200, 1000, 70000, 200000]
    st = T.build_state(w, "hca", Ls, fp8=fp8)
    out = T.run_ops(w, "hca", st, Ls)
    compare(w, "hca", st, Ls, out, fp8=fp8)


def test_csa_decode_fp8_ops():
    w = configs.shrink(configs.PRO_DECODE_1M, H=128, k_csa=1024)
    Ls = [3000, 70000]
    st = T.build_state(w, "csa", Ls, fp8=True)
    out = T.run_ops(w, "csa", st, Ls)
    compare(w, "csa", st, Ls, out, fp8=True)


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_decode_step_upkeep_and_outputs(layer):
    """Several decode steps through hsa_decode_step: every step's output and
    selection match the oracle recomputed from the full history, and the
    appended cache entries equal a from-scratch compression, bit for bit."""
    w = configs.shrink(configs.RAGGED_SERVING, H=64, k_csa=64)
    Ls = [5, 126, 1000, 1021, 3000, 8190]
    S = 12 if layer == "csa" else 10
    st = T.build_state(w, layer, Ls, steps=S)
    lay = T.layer_of(w, layer, st)
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


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_listed_queries_name_their_request(layer):
    """Queries that name their request: several queries of one request at
    consecutive positions (as when a request verifies several new tokens at
    once), interleaved across requests, with the full token arrays as the
    window source.  Indexer + top-k and attention against the oracle."""
    w = configs.shrink(configs.CSA_DECODE_128K, H=64, k_csa=64)
    Ls = [3000, 9001]
    S = 3
    st = T.build_state(w, layer, Ls, steps=S)
    m = w.m(layer)
    reqs = st["reqs"]
    cap = max(Ls) + S
    full_k = np.zeros((2, cap, 128), dtype=np.uint16)
    full_v = np.zeros_like(full_k)
    for r, d in enumerate(reqs):
        full_k[r, : Ls[r] + S] = d["k"]
        full_v[r, : Ls[r] + S] = d["v"]
    tk = L.Tokens(T.dev_bf16(full_k))
    tv = L.Tokens(T.dev_bf16(full_v))
    order = [(1, 0), (0, 0), (1, 1), (0, 1), (1, 2), (0, 2)]     # (request, step)
    req = torch.tensor([r for r, _ in order], dtype=torch.int32, device="cuda")
    pos = torch.tensor([Ls[r] + s for r, s in order], dtype=torch.int64, device="cuda")
    q = L.Queries.list(pos, cap - 1, req=req)
    Q = T.dev_bf16(np.stack([reqs[r]["q"][s] for r, s in order]))
    if layer == "csa":
        qi = T.dev_bf16(np.stack([reqs[r]["qi"][s] for r, s in order]))
        wt = torch.from_numpy(np.stack([reqs[r]["w"][s] for r, s in order])).cuda()
        idx, _ = L.indexer_topk(q, qi, wt, st["kic"], m, w.n_win, w.k_csa)
        O, lse = L.csa_attn(q, Q, tk, tv, w.n_win, st["kc"], st["vc"], m, idx, w.k_csa,
                            with_lse=True, out_fp32=True)
        idx = idx.cpu().numpy()
    else:
        O, lse = L.hca_attn(q, Q, tk, tv, w.n_win, st["kc"], st["vc"], m, with_lse=True,
                            out_fp32=True)
    L.check_device_error()
    Ob, lse = T.to_f64(O), lse.cpu().numpy()
    for i, (r, s) in enumerate(order):
        d, t = reqs[r], Ls[r] + s
        ref, (kc, vc) = oracle_row(w, layer, d, t, s)
        if layer == "csa":
            T.check_topk(idx[i], ref["scores"], w.k_csa, where=f"query {i}")
            sel = idx[i][idx[i] >= 0]
            if not np.array_equal(sel, ref["idx"][ref["idx"] >= 0]):
                s0 = orc.window_start(t, w.n_win)
                K = np.concatenate([nx.bf16_value(d["k"][s0:t + 1]), kc.values[sel]])
                V = np.concatenate([nx.bf16_value(d["v"][s0:t + 1]), vc.values[sel]])
                o, l = orc.attend(nx.bf16_value(d["q"][s]), K, V, T.scale_of())
                ref = {"o": o, "lse": l}
        assert np.max(np.abs(Ob[i] - ref["o"])) <= T.OUT_TOL, f"query {i}"
        assert np.max(np.abs(lse[i] - ref["lse"])) <= T.LSE_TOL, f"query {i} lse"
