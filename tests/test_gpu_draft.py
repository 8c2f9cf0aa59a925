"""GPU parity of hsa_decode_draft (several tokens per request, as speculative
decoding verifies them): every draft query's selection and output equal the
oracle's at its own position, recomputed from the full token history, and the
caches after the draft equal a from-scratch compression of that history, bit
for bit."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L
from test_gpu_decode import oracle_row

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layer,n_tok", [("csa", 6), ("csa", 4), ("hca", 5), ("csa", 1)])
def test_draft_matches_oracle_and_caches(layer, n_tok):
    """CSA drafts of 6 and 4 tokens score their queries in groups of 3 and 4
    per pass over the keys; a 1-token draft takes the single-query scan."""
    w = configs.shrink(configs.RAGGED_SERVING, H=64, k_csa=64)
    # requests whose drafts complete blocks at different offsets (CSA m = 4;
    # HCA m = 128: 126 -> block at 127; 1021 -> block at 1023); 70,001 tokens:
    # 35 scan chunks and the long-row selection (over 16,384 blocks)
    Ls = [5, 126, 1000, 1021, 3000, 70001]
    st = T.build_state(w, layer, Ls, steps=n_tok, ring_cap=w.n_win + n_tok - 1,
                       tail_cap=w.m(layer) + n_tok - 1)
    lay = T.layer_of(w, layer, st)
    reqs = st["reqs"]
    B = len(Ls)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    max_pos = max(Ls) + n_tok - 1
    stack = lambda f: np.stack([np.stack([f(r, d, i) for i in range(n_tok)])
                                for r, d in enumerate(reqs)])
    Q = T.dev_bf16(stack(lambda r, d, i: d["q"][i]))
    kn = T.dev_bf16(stack(lambda r, d, i: d["k"][Ls[r] + i]))
    vn = T.dev_bf16(stack(lambda r, d, i: d["v"][Ls[r] + i]))
    extra = {}
    if layer == "csa":
        extra = dict(qI=T.dev_bf16(stack(lambda r, d, i: d["qi"][i])),
                     kI_new=T.dev_bf16(stack(lambda r, d, i: d["ki"][Ls[r] + i])),
                     w=torch.from_numpy(stack(lambda r, d, i: d["w"][i])).cuda())
    O, lse, idx = L.decode_draft(lay, pos, max_pos, Q, kn, vn, with_lse=True,
                                 with_idx=(layer == "csa"), **extra)
    L.check_device_error()
    Ob, lse = T.to_f64(O), lse.cpu().numpy()
    idx = idx.cpu().numpy() if idx is not None else None
    m = w.m(layer)
    for r, d in enumerate(reqs):
        for i in range(n_tok):
            t = Ls[r] + i
            ref, (kc, vc) = oracle_row(w, layer, d, t, i)
            if layer == "csa":
                T.check_topk(idx[r, i], ref["scores"], w.k_csa, where=f"req {r} t {t}")
                sel = idx[r, i][idx[r, i] >= 0]
                if not np.array_equal(sel, ref["idx"][ref["idx"] >= 0]):
                    s0 = orc.window_start(t, w.n_win)
                    K = np.concatenate([nx.bf16_value(d["k"][s0:t + 1]), kc.values[sel]])
                    V = np.concatenate([nx.bf16_value(d["v"][s0:t + 1]), vc.values[sel]])
                    o, l = orc.attend(nx.bf16_value(d["q"][i]), K, V, T.scale_of())
                    ref = {"o": o, "lse": l}
            err = np.max(np.abs(Ob[r, i] - ref["o"]))
            assert err <= T.OUT_TOL, f"req {r} t {t}: {err}"
            assert np.max(np.abs(lse[r, i] - ref["lse"])) <= T.LSE_TOL, f"req {r} t {t} lse"
    for r, d in enumerate(reqs):
        n = (Ls[r] + n_tok) // m
        for name, x, z in [("kc", "k", "zk"), ("vc", "v", "zv")] + \
                ([("kic", "ki", "zi")] if layer == "csa" else []):
            assert int(st[name].n_entries[r]) == n, (r, name)
            ref = orc.compress(d[x][: Ls[r] + n_tok], st["z"][z], m)
            assert np.array_equal(T.cache_bits(st[name], r, n), ref.bits), (r, name)
