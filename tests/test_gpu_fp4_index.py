"""GPU parity of the indexer over fp4 compressed indexer keys (the wiki's §8
FP4 indexer, read as OCP MX FP4: e2m1 codes in 32-channel blocks with a
power-of-two e8m0 scale) against the oracle fed the same fp4 cache.

The compressor's codes and scale bytes equal the oracle's bit for bit.  The
kernels widen each code times its block scale to bf16 exactly (a power-of-two
scale keeps an e2m1 value a bf16 value), so the scores are the fp32 sums of
exact products and the selection is compared with the same tie band as the
bf16 path."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
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
        s = orc.indexer_scores(inp["qi"][t], inp["w"][t], ok.values[:nv])
        T.check_topk(idx[t], s, k, where=f"row {t}")
        sel = idx[t][idx[t] >= 0]
        assert np.allclose(score[t][: len(sel)], s[sel], rtol=1e-4, atol=1e-3), t


@pytest.mark.parametrize("Ls", [[1, 131, 700, 4099, 9001], [40000, 70001]])
def test_decode_indexer_fp4_keys(Ls):
    """One query per request (the scan path): rows under and over the fused
    selection's 16384 blocks, on a shuffled page pool."""
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
        s = orc.indexer_scores(d["qi"][0], d["w"][0], ok.values[:nv])
        T.check_topk(idx[r], s, k, where=f"req {r} t {t}")
        sel = idx[r][idx[r] >= 0]
        assert np.allclose(score[r][: len(sel)], s[sel], rtol=1e-4, atol=1e-3), r
