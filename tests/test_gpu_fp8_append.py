"""GPU parity of decoding into fp8 K / V caches (the all-fp8 entry and the
mixed entry with bf16 RoPE channels): hsa_decode_step appends a block every m
tokens, keeping its exact value in the cache's stash and re-encoding the page
still filling, so after every step each cache equals a from-scratch
compression of the history (codes and page scales, bit for bit; a partial
page takes the scale of the entries it holds), and the step's outputs match
the oracle attending over those caches.  A draft whose rejected tokens are
large (so they inflate a page's scale) is rewound: the kept page is
re-encoded with the scale of the entries it keeps."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def oracle_after_append(w, layer, d, t, s, kdt):
    """Oracle for the query at t (query row s) over caches holding every block
    complete at t -- the state hsa_decode_step attends to after its append
    (the block completed at t is not visible, but shares its page's scale)."""
    m = w.m(layer)
    z = gen.pool_logits(w, layer)
    kc = orc.compress(d["k"][:t + 1], z["zk"], m, kdt)
    vc = orc.compress(d["v"][:t + 1], z["zv"], m, "fp8")
    if layer == "csa":
        kic = orc.compress(d["ki"][:t + 1], z["zi"], m)
        return orc.csa_query(t, d["q"][s], d["qi"][s], d["w"][s], d["k"][: t + 1], d["v"][: t + 1],
                             kc, vc, kic, m, w.n_win, w.k_csa), (kc, vc)
    return orc.hca_query(t, d["q"][s], d["k"][: t + 1], d["v"][: t + 1], kc, vc, m, w.n_win), (kc, vc)


def check_step(w, layer, reqs, pos, s, O, lse, idx, kdt, where):
    for r, d in enumerate(reqs):
        t = pos[r]
        ref, (kc, vc) = oracle_after_append(w, layer, d, t, s, kdt)
        if layer == "csa":
            T.check_topk(idx[r], ref["scores"], w.k_csa, where=f"{where} req {r}")
            sel = idx[r][idx[r] >= 0]
            if not np.array_equal(sel, ref["idx"][ref["idx"] >= 0]):
                s0 = orc.window_start(t, w.n_win)
                K = np.concatenate([nx.bf16_value(d["k"][s0:t + 1]), kc.values[sel]])
                V = np.concatenate([nx.bf16_value(d["v"][s0:t + 1]), vc.values[sel]])
                o, l = orc.attend(nx.bf16_value(d["q"][s]), K, V, T.scale_of())
                ref = {"o": o, "lse": l}
        err = np.max(np.abs(O[r] - ref["o"]))
        assert err <= T.OUT_TOL, f"{where} req {r} t {t}: {err}"
        assert np.max(np.abs(lse[r] - ref["lse"])) <= T.LSE_TOL, f"{where} req {r} lse"


def check_caches(w, layer, st, hist, kdt, where):
    """Caches of every request equal a from-scratch compression of hist[r]
    (token arrays of the history), codes and page scales."""
    m = w.m(layer)
    for r, h in enumerate(hist):
        n = h["k"].shape[0] // m
        for name, x, z, dt in [("kc", "k", "zk", kdt), ("vc", "v", "zv", "fp8")] + \
                ([("kic", "ki", "zi", "bf16")] if layer == "csa" else []):
            assert int(st[name].n_entries[r]) == n, (where, r, name)
            ref = orc.compress(h[x], st["z"][z], m, dt)
            assert np.array_equal(T.cache_bits(st[name], r, n), ref.bits), (where, r, name)
            if dt != "bf16" and n > 0:
                got = st[name].logical_scales(r, n).cpu().numpy()
                assert np.array_equal(got.view(np.uint32), ref.scales.view(np.uint32)), (where, r, name, "scale")


def step_inputs(layer, reqs, pos, s):
    one = lambda f: T.dev_bf16(np.stack([f(r, d) for r, d in enumerate(reqs)]))
    a = dict(Q=one(lambda r, d: d["q"][s]), k_new=one(lambda r, d: d["k"][pos[r]]),
             v_new=one(lambda r, d: d["v"][pos[r]]))
    if layer == "csa":
        a.update(qI=one(lambda r, d: d["qi"][s]), kI_new=one(lambda r, d: d["ki"][pos[r]]),
                 w=torch.from_numpy(np.stack([d["w"][s] for d in reqs])).cuda())
    return a


@pytest.mark.parametrize("layer,kmix", [("csa", False), ("csa", True), ("hca", False),
                                        ("hca", True)])
def test_decode_step_into_fp8_caches(layer, kmix):
    """Steps that complete blocks mid-page, fill a page and open the next
    (CSA: entries 63 / 64 and 255 / 256; HCA: entries 0, 23, 63, 64)."""
    w = configs.shrink(configs.PRO_DECODE_1M, H=128, k_csa=256)
    Ls = [5, 253, 1021, 3000] if layer == "csa" else [122, 3065, 8186, 8315]
    S = 12 if layer == "csa" else 10
    kdt = "mixed" if kmix else "fp8"
    st = T.build_state(w, layer, Ls, steps=S, fp8=True, kmix=kmix, stash=True)
    lay = T.layer_of(w, layer, st)
    reqs = st["reqs"]
    max_pos = max(Ls) + S
    print(f"fp8 append {layer} {kdt}: Ls {Ls}, {S} steps", flush=True)
    for s in range(S):
        p = [x + s for x in Ls]
        O, lse, idx = L.decode_step(lay, torch.tensor(p, dtype=torch.int64, device="cuda"), max_pos,
                                    with_lse=True, with_idx=(layer == "csa"),
                                    **step_inputs(layer, reqs, p, s))
        L.check_device_error()
        check_step(w, layer, reqs, p, s, T.to_f64(O), lse.cpu().numpy(),
                   None if idx is None else idx.cpu().numpy(), kdt, f"step {s}")
        check_caches(w, layer, st, [{x: d[x][: p[r] + 1] for x in d if x in ("k", "v", "ki")}
                                    for r, d in enumerate(reqs)], kdt, f"step {s}")


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_fp8_draft_rewind(layer):
    """A draft of 8 (CSA) or 4 (HCA) tokens whose rejected tokens are 16x the
    history's scale: the blocks they complete raise their page's scale (CSA
    also opens the next page), then the rewind drops those blocks and
    re-encodes the kept page; four decode steps follow."""
    w = configs.shrink(configs.PRO_DECODE_1M, H=128, k_csa=256)
    m = w.m(layer)
    n_tok = 8 if layer == "csa" else 4
    Ls = [1021, 250, 3000] if layer == "csa" else [8190, 3070, 122]
    keep = [1, 3, 0] if layer == "csa" else [0, 1, 2]
    B = len(Ls)
    st = T.build_state(w, layer, Ls, steps=n_tok + 4, fp8=True, stash=True,
                       ring_cap=w.n_win + n_tok - 1, tail_cap=m + n_tok - 1)
    lay = T.layer_of(w, layer, st)
    reqs = st["reqs"]
    big = lambda a: nx.bf16_bits_from_f64(16.0 * nx.bf16_value(a))
    rej = [{x: big(a) for x, a in gen.rejected_tokens(w, layer, r, n_tok).items()} for r in range(B)]
    max_pos = max(Ls) + n_tok + 4
    print(f"fp8 rewind {layer}: Ls {Ls}, keep {keep}", flush=True)

    def tok(name, r, i):
        return reqs[r][name][Ls[r] + i] if i < keep[r] else rej[r][name][i]

    stack = lambda f: np.stack([np.stack([f(r, i) for i in range(n_tok)]) for r in range(B)])
    args = dict(Q=T.dev_bf16(stack(lambda r, i: reqs[r]["q"][i])),
                k_new=T.dev_bf16(stack(lambda r, i: tok("k", r, i))),
                v_new=T.dev_bf16(stack(lambda r, i: tok("v", r, i))))
    if layer == "csa":
        args.update(qI=T.dev_bf16(stack(lambda r, i: reqs[r]["qi"][i])),
                    kI_new=T.dev_bf16(stack(lambda r, i: tok("ki", r, i))),
                    w=torch.from_numpy(stack(lambda r, i: reqs[r]["w"][i])).cuda())
    L.decode_draft(lay, torch.tensor(Ls, dtype=torch.int64, device="cuda"), max_pos, **args)
    L.check_device_error()
    L.decode_rewind(lay, torch.tensor([Ls[r] + keep[r] for r in range(B)], dtype=torch.int64,
                                      device="cuda"))
    L.check_device_error()
    hist = lambda extra: [{x: d[x][: Ls[r] + keep[r] + extra] for x in ("k", "v", "ki") if x in d}
                          for r, d in enumerate(reqs)]
    check_caches(w, layer, st, hist(0), "fp8", "after rewind")
    for s in range(4):
        p = [Ls[r] + keep[r] + s for r in range(B)]
        O, lse, idx = L.decode_step(lay, torch.tensor(p, dtype=torch.int64, device="cuda"), max_pos,
                                    with_lse=True, with_idx=(layer == "csa"),
                                    **step_inputs(layer, reqs, p, n_tok + s))
        L.check_device_error()
        check_step(w, layer, reqs, p, n_tok + s, T.to_f64(O), lse.cpu().numpy(),
                   None if idx is None else idx.cpu().numpy(), "fp8", f"step {s}")
    check_caches(w, layer, st, hist(4), "fp8", "end")
