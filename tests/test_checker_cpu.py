"""The bf16-score selection rule of the GPU tests (hsa_testlib.check_topk_bf16),
exercised on the CPU: a selection computed the way the GPU computes it (fp32
sums in another order, then one rounding to bf16) passes, and selections with
a planted mistake (a block swapped for a lower one, a wrong tie, a score off by
one bf16 step) fail."""
import numpy as np
import pytest

from oracle import hybrid as orc
from oracle import numerics as nx

import hsa_testlib as T


def _case(seed, n, ties=False):
    g = np.random.default_rng(seed)
    q = nx.bf16_bits_from_f64(g.standard_normal((4, 64)))
    w = g.random(4).astype(np.float32)
    keys = nx.bf16_value(nx.bf16_bits_from_f64(0.5 * g.standard_normal((n, 64))))
    if ties:
        keys[g.choice(n, n // 3, replace=False)] = keys[0]
    return q, w, keys


def _fp32_pipeline(q, w, keys, k):
    """fp32 dot products summed from the last channel down, the head sum in
    fp32, one rounding to bf16, the top-k with ties to the lower block."""
    qf = nx.bf16_value(q).astype(np.float32)
    kf = keys.astype(np.float32)
    acc = np.zeros((keys.shape[0], 4), dtype=np.float32)
    for c in range(63, -1, -1):
        acc = (acc + kf[:, c:c + 1] * qf[None, :, c]).astype(np.float32)
    s = np.zeros(keys.shape[0], dtype=np.float32)
    for h in range(4):
        s = (s + np.float32(w[h]) * np.maximum(acc[:, h], np.float32(0))).astype(np.float32)
    s16 = nx.bf16_round_value(s.astype(np.float64))
    idx = orc.topk_blocks(s16, k)
    sel = idx[idx >= 0]
    score = np.zeros(k, dtype=np.float32)
    score[: sel.shape[0]] = s16[sel]
    return idx, score


@pytest.mark.parametrize("seed,n,k,ties", [(1, 3000, 64, False), (2, 5000, 512, False),
                                           (3, 4000, 200, True), (4, 50, 64, False)])
def test_fp32_selection_passes(seed, n, k, ties):
    q, w, keys = _case(seed, n, ties)
    exact = orc.indexer_scores(q, w, keys)
    A = T.score_abs_bound(q, w, keys)
    idx, score = _fp32_pipeline(q, w, keys, k)
    T.check_topk_bf16(idx, score, exact, A, k, "fp32 pipeline")


def test_planted_mistakes_fail():
    q, w, keys = _case(5, 4000, ties=True)
    k = 300
    exact = orc.indexer_scores(q, w, keys)
    A = T.score_abs_bound(q, w, keys)
    idx, score = _fp32_pipeline(q, w, keys, k)
    ref16 = nx.bf16_round_value(exact)
    # a selected block swapped for the best block left out whose score is lower
    order = np.lexsort((np.arange(exact.shape[0]), -ref16))
    inside, outside = order[k - 1], next(b for b in order[k:] if ref16[b] < ref16[order[k - 1]])
    bad = np.sort(np.append(idx[idx != inside], outside)).astype(np.int32)
    bad_score = nx.bf16_round_value(exact[bad]).astype(np.float32)
    with pytest.raises(AssertionError):
        T.check_topk_bf16(bad, bad_score, exact, A, k, "swapped")
    # the wrong member of a tie at the k-th score (a higher block id instead)
    t = ref16[order[k - 1]]
    tied_out = [b for b in order[k:] if ref16[b] == t]
    if tied_out:
        bad = np.sort(np.append(idx[idx != order[k - 1]], tied_out[-1])).astype(np.int32)
        with pytest.raises(AssertionError):
            T.check_topk_bf16(bad, nx.bf16_round_value(exact[bad]).astype(np.float32), exact, A,
                              k, "tie")
    # a reported score one bf16 step away from its block's bracket
    s2 = score.copy()
    v = np.float64(s2[0])
    s2[0] = np.float32(nx.bf16_round_value(v * (1 + 2.0 ** -6)))
    with pytest.raises(AssertionError):
        T.check_topk_bf16(idx, s2, exact, A, k, "score")
