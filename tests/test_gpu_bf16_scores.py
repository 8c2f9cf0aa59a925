"""GPU parity of hsa_indexer_topk_bf16_scores: the top-k over index scores
rounded to bf16 (ties: lower block), against the oracle's selection over the
exact scores rounded once to bf16.

The GPU rounds its fp32 score, the oracle the exact one; the two bf16 values
differ by one bf16 step when the exact score lies within fp32 rounding of a
midpoint between bf16 neighbours.  So the check is: every block whose bf16
score is more than a small margin away from the k-th largest is classified as
the oracle classifies it, the count and order are right, and nearly every row
(ties at the threshold are common at these sizes, so the tie rule decides most
rows) equals the oracle's selection exactly."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def _check(gpu_idx, gpu_score, exact, k, where):
    """Returns whether the row equals the oracle's selection exactly."""
    ref16 = nx.bf16_round_value(exact)
    n = exact.shape[0]
    n_sel = min(k, n)
    g = gpu_idx[:n_sel]
    assert np.all(gpu_idx[n_sel:] == -1), f"{where}: padding"
    assert n_sel == 0 or (g.min() >= 0 and g.max() < n and np.all(np.diff(g) > 0)), \
        f"{where}: ids not ascending and in range"
    if n > k:
        t = np.sort(ref16)[::-1][k - 1]                  # the k-th largest bf16 score
        margin = 2.0 ** -5 * abs(t) + 1e-30
        sel = np.zeros(n, dtype=bool)
        sel[g] = True
        assert np.all(sel[ref16 > t + margin]), f"{where}: a clearly higher block left out"
        assert not np.any(sel[ref16 < t - margin]), f"{where}: a clearly lower block selected"
    # reported scores: bf16 values within one bf16 step of the oracle's
    s = gpu_score[:n_sel].astype(np.float64)
    assert np.array_equal(nx.bf16_round_value(s), s), f"{where}: scores are not bf16 values"
    assert np.all(np.abs(s - ref16[g]) <= 2.0 ** -7 * np.abs(ref16[g]) + 1e-30), f"{where}: scores"
    return np.array_equal(g, orc.topk_blocks(ref16, k)[:n_sel])


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
        same += _check(idx[t], score[t], exact, k, f"row {t}")
    assert same >= 0.97 * T_, f"{same} of {T_} rows equal the oracle's selection"
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
    mismatched = 0
    for r, d in enumerate(reqs):
        t = int(Ls[r])
        kc = orc.compress(d["ki"][:t], z, m)
        exact = orc.indexer_scores(d["qi"][0], d["w"][0], kc.values[:orc.n_visible(t, m, n_win)])
        mismatched += not _check(idx[r], score[r], exact, k, f"req {r} t {t}")
    assert mismatched <= 1, f"{mismatched} rows differ from the oracle's selection"
