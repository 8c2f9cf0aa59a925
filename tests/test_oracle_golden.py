"""The oracle against hand-derived values (tests/golden/tiny_hand.json)."""
import json
import os
from fractions import Fraction

import numpy as np

from oracle import hybrid as orc
from synth.gen import bf16_bits

HERE = os.path.dirname(os.path.abspath(__file__))


def test_tiny_hand_fixture():
    g = json.load(open(os.path.join(HERE, "golden", "tiny_hand.json")))
    T, m, n_win = 8, 2, 2
    k = bf16_bits(np.zeros((T, 2), np.float32))
    v = bf16_bits(np.array([[j, -j] for j in range(T)], np.float32))
    q = bf16_bits(np.ones((T, 1, 2), np.float32))
    ki = bf16_bits(np.array([[j, 0] for j in range(T)], np.float32))
    qi = bf16_bits(np.array([[[1, 0]]] * T, np.float32))
    w = np.ones((T, 1), np.float32)
    z = np.zeros((m, 2), np.float32)
    inp = dict(q=q, k=k, v=v, qi=qi, ki=ki, w=w, zk=z, zv=z, zi=z)
    hca = orc.prefill_rows(inp, "hca", range(T), m, n_win)
    for t, r in enumerate(hca):
        exp = float(Fraction(g["hca"]["o_first"][t]))
        assert abs(r["o"][0, 0] - exp) < 1e-12 and abs(r["o"][0, 1] + exp) < 1e-12
        assert abs(r["lse"][0] - np.log(g["hca"]["n_entries"][t])) < 1e-12
    csa = orc.prefill_rows(inp, "csa", range(T), m, n_win, topk=1)
    for t, r in enumerate(csa):
        assert r["idx"][0] == g["csa_top1"]["idx0"][t]
        assert abs(r["o"][0, 0] - float(Fraction(g["csa_top1"]["o_first"][t]))) < 1e-12
    r = orc.prefill_rows(inp, "csa", [7], m, n_win, topk=2)[0]
    assert r["idx"].tolist() == g["csa_top2"]["idx"]
    assert abs(r["o"][0, 0] - float(Fraction(g["csa_top2"]["o_first"][0]))) < 1e-12
