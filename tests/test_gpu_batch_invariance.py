"""Batch-invariant decode: a request's selection, output and LSE are the same,
bit for bit, whether its query runs alone or inside a batch of other requests
(in any order).  The selection is exact per query; the attention cuts a
query's entries into splits of a layer-constant size and merges them in a
fixed order, so the batch changes nothing but the number of empty splits."""
import numpy as np
import pytest
import torch

from synth import configs

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu

LS = [300, 5000, 20000, 70001]


def _queries(st, Ls, order):
    """Listed queries for the requests in `order` (query i -> request order[i])."""
    pos = torch.tensor([int(Ls[r]) for r in order], dtype=torch.int64, device="cuda")
    req = torch.tensor(order, dtype=torch.int32, device="cuda")
    return L.Queries.list(pos, int(pos.max().item()), req=req)


def _run(w, layer, st, Ls, order):
    q = _queries(st, Ls, order)
    Q = T.dev_bf16(np.stack([st["reqs"][r]["q"][0] for r in order]))
    out = {}
    if layer == "csa":
        qi = T.dev_bf16(np.stack([st["reqs"][r]["qi"][0] for r in order]))
        wt = torch.from_numpy(np.stack([st["reqs"][r]["w"][0] for r in order])).cuda()
        idx, _ = L.indexer_topk(q, qi, wt, st["kic"], w.m_csa, w.n_win, w.k_csa, ws_key="inv_i")
        O, lse = L.csa_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"],
                            w.m_csa, idx, w.k_csa, with_lse=True, out_fp32=True, ws_key="inv_a")
        out["idx"] = idx.cpu().numpy()
    else:
        O, lse = L.hca_attn(q, Q, st["ring_k"], st["ring_v"], w.n_win, st["kc"], st["vc"],
                            w.m_hca, with_lse=True, out_fp32=True, ws_key="inv_a")
    L.check_device_error()
    out["O"] = O.cpu().numpy().view(np.uint32)
    out["lse"] = lse.cpu().numpy().view(np.uint32)
    return out


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_decode_is_batch_invariant(layer):
    w = configs.shrink(configs.CSA_DECODE_128K, B=len(LS), H=64)
    st = T.build_state(w, layer, LS, steps=1, shuffle=True)
    # the new token of every request sits in its window ring
    for r, d in enumerate(st["reqs"]):
        p = int(LS[r])
        st["ring_k"].data[r, p % w.n_win] = T.dev_bf16(d["k"][p])
        st["ring_v"].data[r, p % w.n_win] = T.dev_bf16(d["v"][p])
    B = len(LS)
    batch = _run(w, layer, st, LS, list(range(B)))
    rev = _run(w, layer, st, LS, list(reversed(range(B))))
    for r in range(B):
        alone = _run(w, layer, st, LS, [r])
        for key in batch:
            assert np.array_equal(batch[key][r], alone[key][0]), (layer, r, key, "alone")
            assert np.array_equal(batch[key][r], rev[key][B - 1 - r]), (layer, r, key, "reversed")
