"""GPU parity of the selection paths that only extreme rows reach:

* a tie storm: more than 2,048 blocks share the k-th score exactly, so the
  candidates of the threshold bin do not fit in LDS and the refine passes run
  on the workspace copies (fused rows up to 16,384 blocks, and the
  multi-workgroup path beyond);
* rows longer than 524,288 blocks, whose selection bitmap does not fit in LDS
  (up to the longest row the decode indexer takes, 2^21 blocks).

The compressed indexer keys are written straight into the paged cache
(seeded N(0, 0.5^2) bf16 values), so the rows can be millions of blocks long
without compressing tens of millions of raw tokens; the oracle scores the
same bf16 keys.  Selections are compared with the oracle's exactly (ties to
the lower block) where the construction makes the k-th score an exact tie,
and by the 1e-4 band otherwise; the bf16-score selector by the exact rule of
hsa_testlib.check_topk_bf16."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu

W = configs.CSA_DECODE_128K
M, N_WIN = W.m_csa, W.n_win


def pos_for(nv):
    """A query position whose visible blocks number exactly nv (nv >= 1)."""
    t = M * nv + N_WIN - 2
    assert orc.n_visible(t, M, N_WIN) == nv
    return t


def fill_cache(rows_per_req, name):
    """A shuffled paged cache holding the given bf16 key rows per request."""
    B = len(rows_per_req)
    max_e = max(r.shape[0] for r in rows_per_req)
    ppr = -(-max_e // 64)
    perm = torch.from_numpy(gen.page_permutation(W, name, B * ppr))
    c = L.PagedCache.allocate(B, max_e, 64, page_order=perm)
    table = c.page_table.long().cpu()
    for r, rows in enumerate(rows_per_req):
        n = rows.shape[0]
        npg = -(-n // 64)
        pad = np.zeros((npg * 64, 64), np.uint16)
        pad[:n] = rows
        c.data[table[r, :npg].cuda()] = T.dev_bf16(pad).reshape(npg, 64, 64)
        c.n_entries[r] = n
    torch.cuda.synchronize()
    return c


def storm_keys(r, nv, n_tie, n_above, q):
    """Random keys, with n_tie blocks holding the query's head-0 vector u (an
    exact tie well above every random score) and n_above blocks holding 2u."""
    g = gen.rng(W.seed, f"storm.{r}.{nv}")
    keys = nx.bf16_bits_from_f64(0.5 * g.standard_normal((nv, 64)))
    which = g.permutation(nv)
    keys[which[:n_tie]] = q[0]
    keys[which[n_tie:n_tie + n_above]] = nx.bf16_bits_from_f64(2.0 * nx.bf16_value(q[0]))
    return keys


@pytest.mark.parametrize("bf16_scores", [False, True])
@pytest.mark.parametrize("nvs,k", [([12000, 9000], 1024), ([40000, 300000], 1024),
                                   ([40000, 12000], 512)])
def test_tie_storm(nvs, k, bf16_scores):
    """3,000 blocks tie at the k-th score (100 score above them): the lowest
    k - 100 tied blocks must be chosen.  Rows of 12,000 and 9,000 blocks take
    the fused selection, 40,000 and 300,000 the threshold / select / refine
    kernels; all of them hold more candidates than LDS does."""
    B = len(nvs)
    g = gen.rng(W.seed, f"storm.q.{nvs}")
    qs = [nx.bf16_bits_from_f64(g.standard_normal((4, 64))) for _ in range(B)]
    wt = np.ones((B, 4), dtype=np.float32)
    keys = [storm_keys(r, nv, 3000, 100, qs[r]) for r, nv in enumerate(nvs)]
    kic = fill_cache(keys, f"storm.{nvs}")
    pos = torch.tensor([pos_for(nv) for nv in nvs], dtype=torch.int64, device="cuda")
    print(f"tie storm: rows {nvs}, k {k}, bf16 scores {bf16_scores}", flush=True)
    q = L.Queries.list(pos, int(pos.max()))
    idx, score = L.indexer_topk(q, T.dev_bf16(np.stack(qs)), torch.from_numpy(wt).cuda(), kic, M,
                                N_WIN, k, with_score=True, bf16_scores=bf16_scores)
    L.check_device_error()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    for r in range(B):
        vals = nx.bf16_value(keys[r])
        exact = orc.indexer_scores(qs[r], wt[r], vals)
        # the construction: 100 blocks above an exact 3,000-way tie at the k-th score
        tie = exact[np.all(keys[r] == qs[r][0], axis=1)]
        assert np.all(tie == tie[0]) and np.sum(exact > tie[0]) == 100
        assert np.sum(exact == tie[0]) == 3000
        ref = orc.topk_blocks(nx.bf16_round_value(exact) if bf16_scores else exact, k)
        assert np.array_equal(idx[r], ref), f"req {r}: selection differs from the oracle's"
        if bf16_scores:
            T.check_topk_bf16(idx[r], score[r], exact, T.score_abs_bound(qs[r], wt[r], vals), k,
                              f"req {r}")


@pytest.mark.parametrize("bf16_scores", [False, True])
def test_longest_rows(bf16_scores):
    """Rows of 2^21 blocks (the longest the decode indexer takes: an 8M-token
    context at m = 4) and 530,001 blocks: the selection bitmap of 16,384+
    words lives in the workspace; a 1,000-block row rides in the same call."""
    nvs = [1 << 21, 530_001, 1000]
    k = 1024
    B = len(nvs)
    g = gen.rng(W.seed, "longest.q")
    qs = [nx.bf16_bits_from_f64(g.standard_normal((4, 64))) for _ in range(B)]
    wt = gen.rng(W.seed, "longest.w").random((B, 4), dtype=np.float32)
    keys = [nx.bf16_bits_from_f64(0.5 * gen.rng(W.seed, f"longest.k.{r}").standard_normal((nv, 64)))
            for r, nv in enumerate(nvs)]
    kic = fill_cache(keys, "longest")
    pos = torch.tensor([pos_for(nv) for nv in nvs], dtype=torch.int64, device="cuda")
    print(f"longest rows: {nvs}, bf16 scores {bf16_scores}", flush=True)
    q = L.Queries.list(pos, int(pos.max()))
    idx, score = L.indexer_topk(q, T.dev_bf16(np.stack(qs)), torch.from_numpy(wt).cuda(), kic, M,
                                N_WIN, k, with_score=True, bf16_scores=bf16_scores)
    L.check_device_error()
    idx, score = idx.cpu().numpy(), score.cpu().numpy()
    for r in range(B):
        vals = nx.bf16_value(keys[r])
        exact = orc.indexer_scores(qs[r], wt[r], vals)
        if bf16_scores:
            T.check_topk_bf16(idx[r], score[r], exact, T.score_abs_bound(qs[r], wt[r], vals), k,
                              f"req {r}")
        else:
            T.check_topk(idx[r], exact, k, where=f"req {r}")
            sel = idx[r][idx[r] >= 0]
            assert np.allclose(score[r][: sel.shape[0]], exact[sel], rtol=1e-4, atol=1e-6)
