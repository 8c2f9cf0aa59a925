"""GPU parity of hsa_indexer_topk_bf16_scores: the top-k over index scores
rounded to bf16 (ties: lower block), against the oracle's selection over the
exact scores rounded once to bf16.

The GPU rounds its fp32 score, the oracle the exact one; the two bf16 values
can differ only where a rounding boundary lies within the fp32 error bound of
the exact score.  hsa_testlib.check_topk_bf16 states the exact rule: the
selection must be the top-k for some choice of values inside each block's
bracket, and a row with no such block must equal the oracle's selection."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("k", [64, 200])
def test_prefill_bf16_scores(k):
    """Every query row of the 4K prefill (span queries: score GEMM, histogram
    and fused selection)."""
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    m, n_win, T_ = w.m_csa, w.n_win, inp["ki"].shape[0]
    alpha = L.pooling_weights(torch.from_numpy(inp["zi"]).cuda())
    kic = L.PagedCache.allocate(1, T_ // m, 64)
    L.kv_compress(T.tokens(inp["ki"]), kic, 0, 0, T_ // m, m, alpha)
    q = L.Queries.span(T_)
    idx, score = L.indexer_topk(q, T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda(), kic,
                                m, n_win, k, with_score=True, bf16_scores=True)
    L.check_device_error()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    kc = orc.compress(inp["ki"], inp["zi"], m)
    same = 0
    for t in range(T_):
        nv = orc.n_visible(t, m, n_win)
        exact = orc.indexer_scores(inp["qi"][t], inp["w"][t], kc.values[:nv])
        A = T.score_abs_bound(inp["qi"][t], inp["w"][t], kc.values[:nv])
        same += T.check_topk_bf16(idx[t], score[t], exact, A, k, f"row {t}")
    print(f"prefill k={k}: {same} of {T_} rows equal the oracle's bf16-score selection")


@pytest.mark.parametrize("Ls", [[1, 131, 700, 4099, 9001], [40000, 70001]])
def test_decode_bf16_scores(Ls):
    """One query per request (the scan path): rows under and over the fused
    selection's 16384 blocks, on a shuffled page pool."""
    w = configs.shrink(configs.CSA_DECODE_128K, B=len(Ls))
    m, n_win, k = w.m_csa, w.n_win, w.k_csa
    reqs = [gen.decode_request(w, "csa", r, L=int(Ls[r])) for r in range(len(Ls))]
    z = gen.pool_logits(w, "csa")["zi"]
    alpha = L.pooling_weights(torch.from_numpy(z).cuda())
    max_entries = max(Ls) // m + 2
    ppr = -(-max_entries // 64)
    perm = torch.from_numpy(gen.page_permutation(w, "bf16s", len(Ls) * ppr))
    kic = L.PagedCache.allocate(len(Ls), max_entries, 64, page_order=perm)
    for r, d in enumerate(reqs):
        nb = int(Ls[r]) // m
        if nb > 0:
            L.kv_compress(T.tokens(d["ki"][: int(Ls[r])]), kic, r, 0, nb, m, alpha)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    q = L.Queries.list(pos, int(max(Ls)))
    qi = T.dev_bf16(np.stack([d["qi"][0] for d in reqs]))
    wt = torch.from_numpy(np.stack([d["w"][0] for d in reqs])).cuda()
    idx, score = L.indexer_topk(q, qi, wt, kic, m, n_win, k, with_score=True, bf16_scores=True)
    L.check_device_error()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    for r, d in enumerate(reqs):
        t = int(Ls[r])
        kc = orc.compress(d["ki"][:t], z, m)
        vals = kc.values[:orc.n_visible(t, m, n_win)]
        exact = orc.indexer_scores(d["qi"][0], d["w"][0], vals)
        A = T.score_abs_bound(d["qi"][0], d["w"][0], vals)
        T.check_topk_bf16(idx[r], score[r], exact, A, k, f"req {r} t {t}")
