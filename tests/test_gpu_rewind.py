"""GPU parity of a draft that speculative decoding partly rejects: draft four
tokens per request, keep the first j (a different j per request, 0 to 4),
rewind the caches to them with hsa_decode_rewind, then decode four more
tokens one step at a time.  Every decode step's selection, output and LSE
equal the oracle's recomputed from the accepted history (the rejected tokens
never happened), and the caches at the end equal a from-scratch compression
of that history, bit for bit.  (zjai.club episode 163 page, "Deep dive" §16:
the caches stay in step across prefill, decode and speculative decode.)"""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L
from test_gpu_decode import oracle_row

pytestmark = pytest.mark.gpu

N_TOK, N_AFTER = 4, 4


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_rewind_then_decode_matches_oracle(layer):
    w = configs.shrink(configs.RAGGED_SERVING, H=64, k_csa=64)
    m = w.m(layer)
    # drafts that complete blocks at different offsets (CSA m = 4; HCA m = 128:
    # 1021 + 3 completes block 7 at 1023, 126 + 1 completes block 0 at 127)
    Ls = [5, 126, 1000, 1021, 3000, 70001]
    keep = [2, 0, 3, 1, 4, 2]          # accepted draft tokens per request
    B = len(Ls)
    st = T.build_state(w, layer, Ls, steps=N_TOK + N_AFTER, ring_cap=w.n_win + N_TOK - 1,
                       tail_cap=m + N_TOK - 1)
    lay = T.layer_of(w, layer, st)
    reqs = st["reqs"]
    rej = [gen.rejected_tokens(w, layer, r, N_TOK) for r in range(B)]
    max_pos = max(Ls) + N_TOK + N_AFTER
    print(f"rewind {layer}: Ls {Ls}, keep {keep}", flush=True)

    # ---- the draft: accepted tokens are the history's, rejected ones are not
    def tok(name, r, i):
        return reqs[r][name][Ls[r] + i] if i < keep[r] else rej[r][name][i]

    stack = lambda f: np.stack([np.stack([f(r, i) for i in range(N_TOK)]) for r in range(B)])
    Q = T.dev_bf16(stack(lambda r, i: reqs[r]["q"][i]))
    kn, vn = T.dev_bf16(stack(lambda r, i: tok("k", r, i))), T.dev_bf16(stack(lambda r, i: tok("v", r, i)))
    extra = {}
    if layer == "csa":
        extra = dict(qI=T.dev_bf16(stack(lambda r, i: reqs[r]["qi"][i])),
                     kI_new=T.dev_bf16(stack(lambda r, i: tok("ki", r, i))),
                     w=torch.from_numpy(stack(lambda r, i: reqs[r]["w"][i])).cuda())
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
    L.decode_draft(lay, pos, max_pos, Q, kn, vn, **extra)
    L.check_device_error()

    # ---- rewind to the accepted tokens
    kept = torch.tensor([Ls[r] + keep[r] for r in range(B)], dtype=torch.int64, device="cuda")
    L.decode_rewind(lay, kept)
    L.check_device_error()
    for name in ["kc", "vc"] + (["kic"] if layer == "csa" else []):
        got = st[name].n_entries.cpu().numpy()
        assert np.array_equal(got, [(Ls[r] + keep[r]) // m for r in range(B)]), name

    # ---- four single-token steps on the accepted history
    worst = 0.0
    for s in range(N_AFTER):
        p = [Ls[r] + keep[r] + s for r in range(B)]
        qrow = N_TOK + s
        one = lambda name, f: T.dev_bf16(np.stack([f(r) for r in range(B)]))
        args = dict(Q=one("q", lambda r: reqs[r]["q"][qrow]),
                    k_new=one("k", lambda r: reqs[r]["k"][p[r]]),
                    v_new=one("v", lambda r: reqs[r]["v"][p[r]]))
        if layer == "csa":
            args.update(qI=one("qi", lambda r: reqs[r]["qi"][qrow]),
                        kI_new=one("ki", lambda r: reqs[r]["ki"][p[r]]),
                        w=torch.from_numpy(np.stack([reqs[r]["w"][qrow] for r in range(B)])).cuda())
        pt = torch.tensor(p, dtype=torch.int64, device="cuda")
        O, lse, idx = L.decode_step(lay, pt, max_pos, with_lse=True, with_idx=(layer == "csa"), **args)
        L.check_device_error()
        O, lse = T.to_f64(O), lse.cpu().numpy()
        idx = idx.cpu().numpy() if idx is not None else None
        for r, d in enumerate(reqs):
            ref, (kc, vc) = oracle_row(w, layer, d, p[r], qrow)
            if layer == "csa":
                T.check_topk(idx[r], ref["scores"], w.k_csa, where=f"step {s} req {r}")
                sel = idx[r][idx[r] >= 0]
                assert np.array_equal(sel, ref["idx"][ref["idx"] >= 0]), f"step {s} req {r}: selection"
            err = np.max(np.abs(O[r] - ref["o"]))
            assert err <= T.OUT_TOL, f"step {s} req {r}: max abs error {err}"
            assert np.max(np.abs(lse[r] - ref["lse"])) <= T.LSE_TOL, f"step {s} req {r}: lse"
            worst = max(worst, err)

    # ---- the caches equal a from-scratch compression of the accepted history
    for r, d in enumerate(reqs):
        n_hist = Ls[r] + keep[r] + N_AFTER
        n = n_hist // m
        for name, x, z in [("kc", "k", "zk"), ("vc", "v", "zv")] + \
                ([("kic", "ki", "zi")] if layer == "csa" else []):
            assert int(st[name].n_entries[r]) == n, (r, name)
            ref = orc.compress(d[x][:n_hist], st["z"][z], m)
            assert np.array_equal(T.cache_bits(st[name], r, n), ref.bits), (r, name)
    print(f"rewind {layer}: max abs error {worst:.3e}")
