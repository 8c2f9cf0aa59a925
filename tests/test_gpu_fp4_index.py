"""GPU parity of the indexer over fp4 compressed indexer keys (the wiki's §8
FP4 indexer, read as OCP MX FP4: e2m1 codes in 32-channel blocks with a
power-of-two e8m0 scale) against the oracle fed the same fp4 cache.

The compressor's codes and scale bytes equal the oracle's bit for bit.  Over
fp4 keys the indexer computes in FP4: the kernels quantize each query head to
MX FP4 by the keys' rule and score on the MX-scaled MFMA, so every product is
exact and the scores are fp32 sums of them; the oracle's indexer_scores_fp4
quantizes the same way and sums in float64.  The selection is compared with
the same tie band as the bf16 path."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def _fp4_kic(rows_by_req, alpha, m, max_entries, page_order=None):
    c = L.PagedCache.allocate(len(rows_by_req), max_entries, 64, fp4=True, page_order=page_order)
    for r, rows in enumerate(rows_by_req):
        nb = rows.shape[0] // m
        if nb > 0:
            L.kv_compress(T.tokens(rows), c, r, 0, nb, m, alpha)
    return c


def test_compress_fp4_indexer_keys_bitexact():
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    m, z = w.m_csa, inp["zi"]
    alpha = L.pooling_weights(torch.from_numpy(z).cuda())
    nb = inp["ki"].shape[0] // m
    perm = torch.from_numpy(gen.page_permutation(w, "fp4", -(-nb // 64)))
    c = _fp4_kic([inp["ki"]], alpha, m, nb, page_order=perm)
    L.check_device_error()
    codes, sb = orc.store_fp4_mx(orc.compress_exact(inp["ki"], orc.pooling_weights(z), m))
    assert np.array_equal(T.cache_bits(c, 0, nb), codes)
    assert np.array_equal(c.logical_scales(0, nb).cpu().numpy(), sb)


@pytest.mark.parametrize("k", [64, 200])
def test_prefill_indexer_fp4_keys(k):
    """Every query row of the 4K prefill (span queries: the score GEMM path)."""
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    m, n_win, T_ = w.m_csa, w.n_win, inp["ki"].shape[0]
    alpha = L.pooling_weights(torch.from_numpy(inp["zi"]).cuda())
    kic = _fp4_kic([inp["ki"]], alpha, m, T_ // m)
    q = L.Queries.span(T_)
    idx, score = L.indexer_topk(q, T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda(), kic,
                                m, n_win, k, with_score=True)
    L.check_device_error()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    ok = orc.compress(inp["ki"], inp["zi"], m, "fp4")
    for t in range(T_):
        nv = orc.n_visible(t, m, n_win)
        s = orc.indexer_scores_fp4(inp["qi"][t], inp["w"][t], ok.values[:nv])
        T.check_topk(idx[t], s, k, where=f"row {t}")
        sel = idx[t][idx[t] >= 0]
        assert np.allclose(score[t][: len(sel)], s[sel], rtol=1e-4, atol=1e-3), t


@pytest.mark.parametrize("Ls", [[1, 131, 700, 4099, 9001], [40000, 70001], [600001]])
def test_decode_indexer_fp4_keys(Ls):
    """One query per request (the scan path): rows under and over the fused
    selection's 16384 blocks, and one of 150,000 blocks (the scan's four-chunk
    workgroups), on a shuffled page pool."""
    w = configs.shrink(configs.CSA_DECODE_128K, B=len(Ls))
    m, n_win, k = w.m_csa, w.n_win, w.k_csa
    reqs = [gen.decode_request(w, "csa", r, L=int(Ls[r])) for r in range(len(Ls))]
    z = gen.pool_logits(w, "csa")["zi"]
    alpha = L.pooling_weights(torch.from_numpy(z).cuda())
    max_entries = max(Ls) // m + 2
    ppr = -(-max_entries // 64)
    perm = torch.from_numpy(gen.page_permutation(w, "fp4idx", len(Ls) * ppr))
    kic = _fp4_kic([d["ki"][: int(Ls[r])] for r, d in enumerate(reqs)], alpha, m, max_entries,
                   page_order=perm)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    q = L.Queries.list(pos, int(max(Ls)))
    qi = T.dev_bf16(np.stack([d["qi"][0] for d in reqs]))
    wt = torch.from_numpy(np.stack([d["w"][0] for d in reqs])).cuda()
    idx, score = L.indexer_topk(q, qi, wt, kic, m, n_win, k, with_score=True)
    L.check_device_error()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    for r, d in enumerate(reqs):
        t = int(Ls[r])
        ok = orc.compress(d["ki"][:t], z, m, "fp4")
        nv = orc.n_visible(t, m, n_win)
        s = orc.indexer_scores_fp4(d["qi"][0], d["w"][0], ok.values[:nv])
        T.check_topk(idx[r], s, k, where=f"req {r} t {t}")
        sel = idx[r][idx[r] >= 0]
        assert np.allclose(score[r][: len(sel)], s[sel], rtol=1e-4, atol=1e-3), r


def test_decode_steps_into_fp4_indexer_keys():
    """hsa_decode_step over an fp4 indexer-key cache: every step's selection
    (scored in FP4) and output against the oracle recomputed from the full
    history, and the MX entries the steps append (codes and scale bytes) bit
    for bit after the steps.  Rows under and over 16,384 blocks (the two
    selection paths); blocks complete during the steps."""
    w = configs.shrink(configs.RAGGED_SERVING, H=64, k_csa=64)
    Ls = [5, 126, 1000, 1021, 3000, 70001]
    S = 9
    m = w.m_csa
    st = T.build_state(w, "csa", Ls, steps=S, index_fp4=True)
    lay = T.layer_of(w, "csa", st)
    max_pos = max(Ls) + S
    z = st["z"]
    for s in range(S):
        pos = torch.tensor([x + s for x in Ls], dtype=torch.int64, device="cuda")
        reqs = st["reqs"]
        Q = T.dev_bf16(np.stack([d["q"][s] for d in reqs]))
        kn = T.dev_bf16(np.stack([d["k"][Ls[r] + s] for r, d in enumerate(reqs)]))
        vn = T.dev_bf16(np.stack([d["v"][Ls[r] + s] for r, d in enumerate(reqs)]))
        O, lse, idx = L.decode_step(
            lay, pos, max_pos, Q, kn, vn, with_lse=True, with_idx=True,
            qI=T.dev_bf16(np.stack([d["qi"][s] for d in reqs])),
            kI_new=T.dev_bf16(np.stack([d["ki"][Ls[r] + s] for r, d in enumerate(reqs)])),
            w=torch.from_numpy(np.stack([d["w"][s] for d in reqs])).cuda())
        L.check_device_error()
        O, lse, idx = T.to_f64(O), lse.cpu().numpy(), idx.cpu().numpy()
        for r, d in enumerate(reqs):
            t = Ls[r] + s
            kc = orc.compress(d["k"][:t], z["zk"], m)
            vc = orc.compress(d["v"][:t], z["zv"], m)
            kic = orc.compress(d["ki"][:t], z["zi"], m, "fp4")
            ref = orc.csa_query(t, d["q"][s], d["qi"][s], d["w"][s], d["k"][: t + 1],
                                d["v"][: t + 1], kc, vc, kic, m, w.n_win, w.k_csa)
            T.check_topk(idx[r], ref["scores"], w.k_csa, where=f"req {r} t {t}")
            sel = idx[r][idx[r] >= 0]
            if not np.array_equal(sel, ref["idx"][ref["idx"] >= 0]):
                s0 = orc.window_start(t, w.n_win)
                K = np.concatenate([nx.bf16_value(d["k"][s0:t + 1]), kc.values[sel]])
                V = np.concatenate([nx.bf16_value(d["v"][s0:t + 1]), vc.values[sel]])
                o, l = orc.attend(nx.bf16_value(d["q"][s]), K, V, T.scale_of())
                ref = {"o": o, "lse": l}
            assert np.max(np.abs(O[r] - ref["o"])) <= T.OUT_TOL, (r, t)
            assert np.max(np.abs(lse[r] - ref["lse"])) <= T.LSE_TOL, (r, t)
    for r, d in enumerate(st["reqs"]):
        n = (Ls[r] + S) // m
        assert int(st["kic"].n_entries[r]) == n
        ref = orc.compress(d["ki"][: Ls[r] + S], z["zi"], m, "fp4")
        assert np.array_equal(T.cache_bits(st["kic"], r, n), ref.bits), r
        assert np.array_equal(st["kic"].logical_scales(r, n).cpu().numpy(), ref.scales), r
