"""Pins of the oracle's visibility rule, indexer, top-k and attention: brute
force on tiny inputs, torch's scaled_dot_product_attention where the method
reduces to dense causal MQA, and the invariants the method must keep."""
import math

import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen


def small(layer_m=4, T=300, H=4, n_win=128, k=16, planted=False):
    return configs.shrink(configs.PREFILL_4K, T=T, H=H, n_win=n_win, m_csa=layer_m,
                          m_hca=layer_m, k_csa=k, planted=planted)


def dense_causal_sdpa(inp):
    q = torch.from_numpy(nx.bf16_value(inp["q"])).permute(1, 0, 2)          # [H, T, d]
    H = q.shape[0]
    k = torch.from_numpy(nx.bf16_value(inp["k"]))[None].expand(H, -1, -1)
    v = torch.from_numpy(nx.bf16_value(inp["v"]))[None].expand(H, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    return o.permute(1, 0, 2).numpy()                                      # [T, H, d]


# ----------------------------------------------------------------------------- visibility

@pytest.mark.parametrize("m", [1, 2, 4, 8, 128])
@pytest.mark.parametrize("n_win", [1, 4, 128, 200])
def test_visibility_matches_enumeration(m, n_win):
    for t in range(0, 700):
        s = orc.window_start(t, n_win)
        assert s == max(0, t - n_win + 1)
        assert t - s + 1 == min(n_win, t + 1)
        brute = [b for b in range(t + 2) if (b + 1) * m <= t + 1 and b * m < s]
        nv = orc.n_visible(t, m, n_win)
        assert brute == list(range(nv)), (t, m, n_win)
        if m > n_win:
            continue                    # the rule needs m <= n_win (the library rejects it)
        # together, window and visible blocks cover every past token
        covered = set(range(s, t + 1)) | {j for b in range(nv) for j in range(b * m, b * m + m)}
        assert covered == set(range(t + 1))
        # overlap with the window is at most m - 1 tokens
        assert max(0, nv * m - s) <= m - 1


def test_visible_counts_at_workload_sizes():
    assert orc.n_visible(131072, 4, 128) == 32737
    assert orc.n_visible(1048576, 4, 128) == 262113
    assert orc.n_visible(1048576, 128, 128) == 8192


# ----------------------------------------------------------------------------- indexer, top-k

def test_indexer_scores_bruteforce():
    r = np.random.default_rng(4)
    qi = gen.bf16_bits(r.standard_normal((4, 8)).astype(np.float32))
    w = r.random(4, dtype=np.float32)
    kic = nx.bf16_value(gen.bf16_bits(r.standard_normal((50, 8)).astype(np.float32)))
    got = orc.indexer_scores(qi, w, kic)
    qv = nx.bf16_value(qi)
    for b in range(50):
        tot = 0.0
        for h in range(4):
            dot = 0.0
            for c in range(8):
                dot += qv[h, c] * kic[b, c]
            tot += float(w[h]) * (dot if dot > 0 else 0.0)
        assert abs(got[b] - tot) <= 1e-12 * (1 + abs(tot))
    # a negative-definite query scores zero everywhere
    assert np.all(orc.indexer_scores(qi, w, np.zeros((3, 8))) == 0)


def test_topk_bruteforce_and_ties():
    r = np.random.default_rng(5)
    for n, k in [(10, 3), (10, 10), (5, 8), (200, 64), (1, 1)]:
        s = np.round(r.standard_normal(n), 1)           # many ties
        got = orc.topk_blocks(s, k)
        ref = sorted(sorted(range(n), key=lambda b: (-s[b], b))[: min(n, k)])
        assert got[: len(ref)].tolist() == ref
        assert np.all(got[len(ref):] == -1)
    # equal scores: the lower block wins
    assert orc.topk_blocks(np.array([1.0, 2.0, 2.0, 2.0, 0.5]), 2).tolist() == [1, 2]


# ----------------------------------------------------------------------------- attention

def test_m1_full_window_equals_dense_causal():
    w = small(layer_m=1, T=96, n_win=128, k=200)
    for layer in ("csa", "hca"):
        inp = gen.prefill_layer(w, layer)
        ref = dense_causal_sdpa(inp)
        rows = orc.prefill_rows(inp, layer, range(96), 1, 128, topk=200)
        got = np.stack([r["o"] for r in rows])
        assert np.max(np.abs(got - ref)) < 1e-10


@pytest.mark.parametrize("n_win", [1, 7, 32])
def test_m1_any_window_with_full_topk_equals_dense_causal(n_win):
    T = 80
    w = small(layer_m=1, T=T, n_win=n_win, k=T)
    for layer in ("csa", "hca"):
        inp = gen.prefill_layer(w, layer)
        ref = dense_causal_sdpa(inp)
        rows = orc.prefill_rows(inp, layer, range(T), 1, n_win, topk=T)
        got = np.stack([r["o"] for r in rows])
        assert np.max(np.abs(got - ref)) < 1e-10


def test_csa_with_topk_covering_all_blocks_equals_hca():
    w = small(layer_m=4, T=400, n_win=32, k=100)
    inp = gen.prefill_layer(w, "csa")
    caches = orc.layer_caches(inp, "csa", 4)
    for t in [0, 31, 32, 35, 36, 200, 399]:
        a = orc.csa_query(t, inp["q"][t], inp["qi"][t], inp["w"][t], inp["k"], inp["v"],
                          caches["kc"], caches["vc"], caches["kic"], 4, 32, 100)
        b = orc.hca_query(t, inp["q"][t], inp["k"], inp["v"], caches["kc"], caches["vc"], 4, 32)
        assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def test_csa_selects_by_indexer_and_is_a_sparse_subset():
    w = small(layer_m=4, T=400, n_win=32, k=8)
    inp = gen.prefill_layer(w, "csa")
    caches = orc.layer_caches(inp, "csa", 4)
    t = 399
    a = orc.csa_query(t, inp["q"][t], inp["qi"][t], inp["w"][t], inp["k"], inp["v"],
                      caches["kc"], caches["vc"], caches["kic"], 4, 32, 8)
    nv = orc.n_visible(t, 4, 32)
    assert np.all(np.diff(a["idx"]) > 0) and a["idx"].shape == (8,)
    best = np.sort(np.argsort(-a["scores"], kind="stable")[:8])
    assert np.array_equal(a["idx"], best)
    # attention over exactly window + selected
    Kw = nx.bf16_value(inp["k"][t - 31: t + 1])
    Vw = nx.bf16_value(inp["v"][t - 31: t + 1])
    K = np.concatenate([Kw, caches["kc"].values[a["idx"]]])
    V = np.concatenate([Vw, caches["vc"].values[a["idx"]]])
    q = nx.bf16_value(inp["q"][t])
    lg = q @ K.T / math.sqrt(128)
    p = np.exp(lg - lg.max(1, keepdims=True))
    ref = (p / p.sum(1, keepdims=True)) @ V
    assert np.max(np.abs(ref - a["o"])) < 1e-12
    assert nv > 8


def test_short_sequence_is_plain_causal():
    w = small(layer_m=4, T=100, n_win=128, k=4)
    inp = gen.prefill_layer(w, "csa")
    ref = dense_causal_sdpa(inp)
    rows = orc.prefill_rows(inp, "csa", range(100), 4, 128, topk=4)
    assert np.max(np.abs(np.stack([r["o"] for r in rows]) - ref)) < 1e-10


def test_unit_values_give_unit_output_and_heads_permute():
    w = small(layer_m=4, T=300, n_win=16, k=8)
    inp = gen.prefill_layer(w, "csa")
    one = dict(inp)
    one["v"] = gen.bf16_bits(np.ones_like(nx.bf16_value(inp["v"]), dtype=np.float32))
    rows = orc.prefill_rows(one, "csa", [5, 150, 299], 4, 16, topk=8)
    for r in rows:
        assert np.max(np.abs(r["o"] - 1.0)) < 1e-12
    perm = np.array([2, 0, 3, 1])
    permd = dict(inp)
    permd["q"] = inp["q"][:, perm]
    for t in [17, 299]:
        a = orc.prefill_rows(inp, "hca", [t], 4, 16)[0]
        b = orc.prefill_rows(permd, "hca", [t], 4, 16)[0]
        assert np.array_equal(a["o"][perm], b["o"])
        a = orc.prefill_rows(inp, "csa", [t], 4, 16, topk=8)[0]
        b = orc.prefill_rows(permd, "csa", [t], 4, 16, topk=8)[0]
        assert np.array_equal(a["o"][perm], b["o"]) and np.array_equal(a["idx"], b["idx"])


def test_lse_is_log_partition():
    w = small(layer_m=4, T=200, n_win=16, k=8)
    inp = gen.prefill_layer(w, "hca")
    caches = orc.layer_caches(inp, "hca", 4)
    t = 150
    r = orc.hca_query(t, inp["q"][t], inp["k"], inp["v"], caches["kc"], caches["vc"], 4, 16)
    q = nx.bf16_value(inp["q"][t])
    K = np.concatenate([nx.bf16_value(inp["k"][135:151]), caches["kc"].values[:orc.n_visible(t, 4, 16)]])
    lg = q @ K.T / math.sqrt(128)
    assert np.allclose(r["lse"], np.log(np.exp(lg).sum(1)), rtol=0, atol=1e-12)


def test_decode_equals_prefill_row():
    """A decode query at position L over a cache of L tokens equals prefill row L."""
    w = small(layer_m=4, T=260, n_win=32, k=8)
    inp = gen.prefill_layer(w, "csa")
    L = 259
    full = orc.prefill_rows(inp, "csa", [L], 4, 32, topk=8)[0]
    # decode: caches built from the L cached tokens only (+ the new token's raw K/V)
    hist = {k: (v[:L] if k in ("k", "v", "ki") else v) for k, v in inp.items()}
    caches = orc.layer_caches(hist, "csa", 4)
    dec = orc.csa_query(L, inp["q"][L], inp["qi"][L], inp["w"][L], inp["k"][: L + 1], inp["v"][: L + 1],
                        caches["kc"], caches["vc"], caches["kic"], 4, 32, 8)
    assert np.array_equal(dec["o"], full["o"]) and np.array_equal(dec["idx"], full["idx"])


def test_bf16_score_selection_closed_form():
    """Scores known in closed form (one head, two channels): the bf16 selector
    rounds after the head sum, to nearest with ties to even, and breaks equal
    rounded scores toward the lower block."""
    qi = np.zeros((4, 8), dtype=np.float32)
    qi[0, :2] = 1.0                                  # head 0 = channels 0 + 1
    w = np.array([1.0, 0.0, 0.0, 0.0], dtype=np.float32)
    kic = np.zeros((5, 8))
    kic[:, 0] = [1.0, 1.0, 1.0, 0.5, 1.0]
    kic[:, 1] = [0.0, 2.0 ** -9, 2.0 ** -8 + 2.0 ** -9, 0.0, 2.0 ** -8]
    exact = orc.indexer_scores(gen.bf16_bits(qi), w, kic)
    assert exact.tolist() == [1.0, 1 + 2.0 ** -9, 1 + 2.0 ** -8 + 2.0 ** -9, 0.5, 1 + 2.0 ** -8]
    s16 = orc.indexer_scores_bf16(gen.bf16_bits(qi), w, kic)
    # the bf16 grid near 1 has spacing 2^-7: 1 + 2^-9 rounds down, 1 + 3 * 2^-9
    # rounds up, and the midpoint 1 + 2^-8 goes to the even neighbour 1
    assert s16.tolist() == [1.0, 1.0, 1 + 2.0 ** -7, 0.5, 1.0]
    assert orc.topk_blocks(exact, 2).tolist() == [2, 4]
    assert orc.topk_blocks(s16, 2).tolist() == [0, 2]          # ties at 1.0: blocks 0, 1, 4
    assert orc.topk_blocks(s16, 3).tolist() == [0, 1, 2]
    assert orc.topk_blocks(s16, 4).tolist() == [0, 1, 2, 4]


def test_bf16_scores_are_rounded_bruteforce_scores():
    r = np.random.default_rng(6)
    qi = gen.bf16_bits(r.standard_normal((4, 8)).astype(np.float32))
    w = (r.random(4) - 0.3).astype(np.float32)        # a negative weight too
    kic = nx.bf16_value(gen.bf16_bits(r.standard_normal((300, 8)).astype(np.float32)))
    got = orc.indexer_scores_bf16(qi, w, kic)
    qv = nx.bf16_value(qi)
    for b in range(300):
        tot = sum(float(w[h]) * max(0.0, sum(qv[h, c] * kic[b, c] for c in range(8)))
                  for h in range(4))
        # a bf16 value (its bits round-trip) within half a bf16 ulp of the sum
        assert nx.bf16_value(nx.bf16_bits_from_f64(np.array([got[b]])))[0] == got[b]
        if tot != 0.0:
            ulp = 2.0 ** (math.floor(math.log2(abs(tot))) - 7)
            assert abs(got[b] - tot) <= ulp / 2 + 1e-12 * abs(tot)
        else:
            assert got[b] == 0.0
