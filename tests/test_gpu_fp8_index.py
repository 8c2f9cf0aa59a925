"""GPU parity of the indexer over fp8 compressed indexer keys (e4m3fn codes,
one fp32 scale per 64-entry page) against the oracle fed the same fp8 cache.

The selection rule does not change with the key format: the top-k of
sum_h w_h * ReLU(qI_h . k) over the decoded keys, compared by the same tie
band as the bf16 path.  The oracle decodes each key as code value times its
page scale (float64); the kernels widen the codes to bf16 exactly and apply
the page scale to the head sum, which equals the oracle's sum in exact
arithmetic because ReLU commutes with a positive scale."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def _fp8_kic(rows_by_req, alpha, m, max_entries, page_order=None):
    """GPU fp8 indexer-key cache of several requests, compressed on the GPU."""
    c = L.PagedCache.allocate(len(rows_by_req), max_entries, 64, fp8=True, page_order=page_order)
    for r, rows in enumerate(rows_by_req):
        nb = rows.shape[0] // m
        if nb > 0:
            L.kv_compress(T.tokens(rows), c, r, 0, nb, m, alpha)
    return c


def test_compress_fp8_indexer_keys_bitexact():
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    m = w.m_csa
    z = inp["zi"]
    alpha = L.pooling_weights(torch.from_numpy(z).cuda())
    nb = inp["ki"].shape[0] // m
    c = _fp8_kic([inp["ki"]], alpha, m, nb)
    codes, scales = orc.store_fp8_pages(orc.compress_exact(inp["ki"], orc.pooling_weights(z), m))
    assert np.array_equal(T.cache_bits(c, 0, nb), codes)
    assert np.array_equal(c.logical_scales(0, nb).cpu().numpy().view(np.uint32),
                          scales.view(np.uint32))
    L.check_device_error()


@pytest.mark.parametrize("k", [64, 200])
def test_prefill_indexer_fp8_keys(k):
    """Every query row of the 4K prefill (span queries: the score GEMM path)."""
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    m, n_win, T_ = w.m_csa, w.n_win, inp["ki"].shape[0]
    alpha = L.pooling_weights(torch.from_numpy(inp["zi"]).cuda())
    kic = _fp8_kic([inp["ki"]], alpha, m, T_ // m)
    q = L.Queries.span(T_)
    idx, score = L.indexer_topk(q, T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda(), kic,
                                m, n_win, k, with_score=True)
    L.check_device_error()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    ok = orc.compress(inp["ki"], inp["zi"], m, "fp8")
    for t in range(T_):
        nv = orc.n_visible(t, m, n_win)
        s = orc.indexer_scores(inp["qi"][t], inp["w"][t], ok.values[:nv])
        T.check_topk(idx[t], s, k, where=f"row {t}")
        sel = idx[t][idx[t] >= 0]
        assert np.allclose(score[t][: len(sel)], s[sel], rtol=1e-4, atol=1e-3), t


@pytest.mark.parametrize("Ls", [[1, 131, 700, 4099, 9001], [40000, 70001]])
def test_decode_indexer_fp8_keys(Ls):
    """One query per request (the scan path): rows under and over the fused
    selection's 16384 blocks, on a shuffled page pool."""
    w = configs.shrink(configs.CSA_DECODE_128K, B=len(Ls))
    m, n_win, k = w.m_csa, w.n_win, w.k_csa
    reqs = [gen.decode_request(w, "csa", r, L=int(Ls[r])) for r in range(len(Ls))]
    z = gen.pool_logits(w, "csa")["zi"]
    alpha = L.pooling_weights(torch.from_numpy(z).cuda())
    max_entries = max(Ls) // m + 2
    ppr = -(-max_entries // 64)
    perm = torch.from_numpy(gen.page_permutation(w, "fp8idx", len(Ls) * ppr))
    kic = _fp8_kic([d["ki"][: int(Ls[r])] for r, d in enumerate(reqs)], alpha, m, max_entries,
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
        ok = orc.compress(d["ki"][:t], z, m, "fp8")
        nv = orc.n_visible(t, m, n_win)
        s = orc.indexer_scores(d["qi"][0], d["w"][0], ok.values[:nv])
        T.check_topk(idx[r], s, k, where=f"req {r} t {t}")
        sel = idx[r][idx[r] >= 0]
        assert np.allclose(score[r][: len(sel)], s[sel], rtol=1e-4, atol=1e-3), r
