"""GPU parity of the partial RoPE against the oracle.

* hsa_rope turns the last 64 channels of bf16 rows bit for bit as the oracle
  does (key rows and 64- / 128-head query rows; spans and listed positions up
  to 2^21; in place and out of place, where the other channels are copied).
* hsa_decode_step with rope_theta turns its new key before the key enters the
  ring, and its queries before attending: after every step the ring and the
  caches (bf16, fp8, mixed K) equal the oracle's over turned keys, bit for
  bit, and the outputs match the oracle attending with turned queries.  Both
  routes of the CSA upkeep are taken: its own launch (short rows) and the
  candidate selection launch (a row over 16,384 blocks).
* The same at full size: the 1M-token Pro decode (4 requests, fp8 caches,
  128 heads, top-1024) over a turned history, one step that completes a
  block in both layers, every request checked.
* hsa_decode_draft turns every draft token at its own position.
* A 4K prefill that turns its K rows and queries with hsa_rope, then
  compresses, selects and attends, matches the oracle's prefill over turned
  inputs; so does the 128K prefill, on sampled rows."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from oracle import numerics as nx
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu

THETA = 10000.0


def _bits(t):
    return T.host_bits(t)


@pytest.mark.parametrize("theta", [THETA, 1e6])
def test_rope_rows_bitexact(theta):
    r = np.random.default_rng(7)
    # key rows (one head): a span starting near 2^20, and listed positions
    k = nx.bf16_bits_from_f64(r.standard_normal((3001, 128)) * 3)
    x = T.dev_bf16(k)
    p0 = (1 << 20) - 77
    y = L.rope(x, theta, pos0=p0)
    assert np.array_equal(_bits(y), orc.rope(k, p0 + np.arange(3001), theta))
    pos = np.concatenate([[0, 1, 2, (1 << 21) - 1, 1 << 21], r.integers(0, 1 << 21, 2996)])
    y = L.rope(x, theta, pos=torch.from_numpy(pos).cuda())
    assert np.array_equal(_bits(y), orc.rope(k, pos, theta))
    # in place: only the RoPE channels change
    xi = x.clone()
    L.rope(xi, theta, pos=torch.from_numpy(pos).cuda(), out=xi)
    assert np.array_equal(_bits(xi), orc.rope(k, pos, theta))
    # query rows: 64 and 128 heads, 13 rows (a ragged last workgroup)
    for H in (64, 128):
        q = nx.bf16_bits_from_f64(r.standard_normal((13, H, 128)))
        qp = r.integers(0, 1 << 21, 13)
        y = L.rope(T.dev_bf16(q), theta, pos=torch.from_numpy(qp).cuda())
        assert np.array_equal(_bits(y), orc.rope(q, qp[:, None], theta)), H
    L.check_device_error()


def _turned(reqs, Ls):
    """The requests' token streams as a RoPE layer holds them: K row p turned
    at p, query s (position Ls[r] + s) at its position."""
    out = []
    for r, d in enumerate(reqs):
        e = dict(d)
        e["k"] = orc.rope(d["k"], np.arange(d["k"].shape[0]), THETA)
        e["q"] = orc.rope(d["q"], (Ls[r] + np.arange(d["q"].shape[0]))[:, None], THETA)
        out.append(e)
    return out


def _oracle(w, layer, d, t, s, kdt, vdt):
    """The query at t (query row s) over caches holding every block complete
    at t (the state the step attends to after its append)."""
    m = w.m(layer)
    z = gen.pool_logits(w, layer)
    kc = orc.compress(d["k"][:t + 1], z["zk"], m, kdt)
    vc = orc.compress(d["v"][:t + 1], z["zv"], m, vdt)
    if layer == "csa":
        kic = orc.compress(d["ki"][:t + 1], z["zi"], m)
        return orc.csa_query(t, d["q"][s], d["qi"][s], d["w"][s], d["k"][: t + 1],
                             d["v"][: t + 1], kc, vc, kic, m, w.n_win, w.k_csa), (kc, vc)
    return orc.hca_query(t, d["q"][s], d["k"][: t + 1], d["v"][: t + 1], kc, vc, m,
                         w.n_win), (kc, vc)


def _check_query(w, layer, d, t, s, O, lse, idx, kdt, vdt, where):
    ref, (kc, vc) = _oracle(w, layer, d, t, s, kdt, vdt)
    _compare(w, layer, d, t, s, ref, kc, vc, O, lse, idx, where)


def _check_output(w, layer, d, t, s, c, O, lse, idx, where):
    """As _check_query, over caches c the caller has compressed."""
    if layer == "csa":
        ref = orc.csa_query(t, d["q"][s], d["qi"][s], d["w"][s], d["k"][: t + 1],
                            d["v"][: t + 1], c["kc"], c["vc"], c["kic"], w.m(layer), w.n_win,
                            w.k_csa)
    else:
        ref = orc.hca_query(t, d["q"][s], d["k"][: t + 1], d["v"][: t + 1], c["kc"], c["vc"],
                            w.m(layer), w.n_win)
    _compare(w, layer, d, t, s, ref, c["kc"], c["vc"], O, lse, idx, where)


def _compare(w, layer, d, t, s, ref, kc, vc, O, lse, idx, where):
    if layer == "csa":
        T.check_topk(idx, ref["scores"], w.k_csa, where=where)
        sel = idx[idx >= 0]
        if not np.array_equal(sel, ref["idx"][ref["idx"] >= 0]):
            s0 = orc.window_start(t, w.n_win)
            K = np.concatenate([nx.bf16_value(d["k"][s0:t + 1]), kc.values[sel]])
            V = np.concatenate([nx.bf16_value(d["v"][s0:t + 1]), vc.values[sel]])
            o, l = orc.attend(nx.bf16_value(d["q"][s]), K, V, T.scale_of())
            ref = {"o": o, "lse": l}
    err = np.max(np.abs(O - ref["o"]))
    assert err <= T.OUT_TOL, f"{where}: {err}"
    assert np.max(np.abs(lse - ref["lse"])) <= T.LSE_TOL, f"{where} lse"


def _check_state(w, layer, st, rot, upto, kdt, vdt, where):
    """Ring rows of every kept window token and every cache, bit for bit."""
    m = w.m(layer)
    cap = st["ring_k"].data.shape[1]
    ring = _bits(st["ring_k"].data)
    for r, d in enumerate(rot):
        p_hi = upto[r]
        for p in range(max(0, p_hi - cap + 1), p_hi + 1):
            assert np.array_equal(ring[r, p % cap], d["k"][p]), (where, r, p, "ring")
        n = (p_hi + 1) // m
        for name, x, z, dt in [("kc", "k", "zk", kdt), ("vc", "v", "zv", vdt)] + \
                ([("kic", "ki", "zi", "bf16")] if layer == "csa" else []):
            assert int(st[name].n_entries[r]) == n, (where, r, name)
            ref = orc.compress(d[x][:p_hi + 1], st["z"][z], m, dt)
            assert np.array_equal(T.cache_bits(st[name], r, n), ref.bits), (where, r, name)
            if dt != "bf16" and n > 0:
                got = st[name].logical_scales(r, n).cpu().numpy()
                assert np.array_equal(got.view(np.uint32), ref.scales.view(np.uint32)), \
                    (where, r, name, "scale")


def _inputs(layer, reqs, pos, s):
    one = lambda f: T.dev_bf16(np.stack([f(r, d) for r, d in enumerate(reqs)]))
    a = dict(Q=one(lambda r, d: d["q"][s]), k_new=one(lambda r, d: d["k"][pos[r]]),
             v_new=one(lambda r, d: d["v"][pos[r]]))
    if layer == "csa":
        a.update(qI=one(lambda r, d: d["qi"][s]), kI_new=one(lambda r, d: d["ki"][pos[r]]),
                 w=torch.from_numpy(np.stack([d["w"][s] for d in reqs])).cuda())
    return a


@pytest.mark.parametrize("layer,fmt,Ls", [
    ("csa", "bf16", [5, 253, 1021, 3000]),      # upkeep in its own launch
    ("csa", "fp8", [5, 1021, 70001]),           # upkeep in the candidate selection launch
    ("csa", "bf16", [126, 70001]),
    ("hca", "bf16", [122, 3065, 8186, 8315]),
    ("hca", "mixed", [122, 3065, 8186, 8315]),
])
def test_decode_steps_with_rope(layer, fmt, Ls):
    """Steps that complete blocks (CSA every 4 tokens; HCA at 127, 3071, 8191
    and 8319): raw keys and queries in, turned ones in the ring, the caches
    and the attention."""
    w = configs.shrink(configs.PRO_DECODE_1M, H=128, k_csa=256)
    S = 9 if layer == "csa" else 6
    fp8 = fmt != "bf16"
    kdt = {"bf16": "bf16", "fp8": "fp8", "mixed": "mixed"}[fmt]
    vdt = "bf16" if fmt == "bf16" else "fp8"
    st = T.build_state(w, layer, Ls, steps=S, fp8=fp8, kmix=fmt == "mixed", stash=fp8,
                       rope=THETA)
    lay = T.layer_of(w, layer, st, rope=THETA)
    reqs = st["reqs"]
    rot = _turned(reqs, Ls)
    max_pos = max(Ls) + S
    print(f"rope decode {layer} {fmt}: Ls {Ls}, {S} steps", flush=True)
    for s in range(S):
        p = [x + s for x in Ls]
        O, lse, idx = L.decode_step(lay, torch.tensor(p, dtype=torch.int64, device="cuda"),
                                    max_pos, with_lse=True, with_idx=(layer == "csa"),
                                    **_inputs(layer, reqs, p, s))
        L.check_device_error()
        Ob, lb = T.to_f64(O), lse.cpu().numpy()
        ib = None if idx is None else idx.cpu().numpy()
        for r, d in enumerate(rot):
            _check_query(w, layer, d, p[r], s, Ob[r], lb[r], None if ib is None else ib[r],
                         kdt, vdt, f"step {s} req {r}")
        _check_state(w, layer, st, rot, p, kdt, vdt, f"step {s}")


@pytest.fixture(scope="module", params=["csa", "hca"])
def pro_1m_rope(request):
    """The benchmark's Pro decode at full size (4 requests x 1M tokens, fp8
    caches with their stashes, 128 heads, CSA top-1024) with partial RoPE: one
    step at position 2^20 - 1, which completes a block in both layers (the
    upkeep pools turned keys and re-encodes the open fp8 page)."""
    layer = request.param
    w = configs.PRO_DECODE_1M
    p = [w.L - 1] * w.B
    st = T.build_state(w, layer, p, steps=1, fp8=True, stash=True, shuffle=False, rope=THETA)
    lay = T.layer_of(w, layer, st, rope=THETA)
    print(f"rope pro decode {layer}: {w.B} x {w.L - 1}", flush=True)
    O, lse, idx = L.decode_step(lay, torch.tensor(p, dtype=torch.int64, device="cuda"), max(p),
                                with_lse=True, with_idx=(layer == "csa"),
                                **_inputs(layer, st["reqs"], p, 0))
    L.check_device_error()
    yield dict(w=w, layer=layer, st=st, p=p, O=T.to_f64(O), lse=lse.cpu().numpy(),
               idx=None if idx is None else idx.cpu().numpy())


@pytest.mark.parametrize("r", range(4))
def test_pro_decode_1m_with_rope_full(pro_1m_rope, r):
    """One request of the full-size step: its output against the oracle over
    its turned history, and its ring rows and caches bit for bit (the oracle
    compresses each cache once, for both checks)."""
    f = pro_1m_rope
    w, layer, st, t = f["w"], f["layer"], f["st"], f["p"][r]
    d = _turned([st["reqs"][r]], [t])[0]
    m = w.m(layer)
    c = {"kc": orc.compress(d["k"][:t + 1], st["z"]["zk"], m, "fp8"),
         "vc": orc.compress(d["v"][:t + 1], st["z"]["zv"], m, "fp8")}
    if layer == "csa":
        c["kic"] = orc.compress(d["ki"][:t + 1], st["z"]["zi"], m)
    _check_output(w, layer, d, t, 0, c, f["O"][r], f["lse"][r],
                  None if f["idx"] is None else f["idx"][r], f"req {r}")
    cap = st["ring_k"].data.shape[1]
    ring = _bits(st["ring_k"].data)
    for q in range(t - cap + 1, t + 1):
        assert np.array_equal(ring[r, q % cap], d["k"][q]), (r, q, "ring")
    for name, ref in c.items():
        assert int(st[name].n_entries[r]) == (t + 1) // m, (r, name)
        assert np.array_equal(T.cache_bits(st[name], r, len(ref)), ref.bits), (r, name)
        if ref.scales is not None:
            got = st[name].logical_scales(r, len(ref)).cpu().numpy()
            assert np.array_equal(got.view(np.uint32), ref.scales.view(np.uint32)), \
                (r, name, "scale")


@pytest.mark.parametrize("layer,n_tok", [("csa", 4), ("hca", 3)])
def test_draft_with_rope(layer, n_tok):
    w = configs.shrink(configs.RAGGED_SERVING, H=64, k_csa=64)
    Ls = [5, 126, 1021, 70001] if layer == "csa" else [126, 1021, 3000]
    st = T.build_state(w, layer, Ls, steps=n_tok, ring_cap=w.n_win + n_tok - 1,
                       tail_cap=w.m(layer) + n_tok - 1, rope=THETA)
    lay = T.layer_of(w, layer, st, rope=THETA)
    reqs = st["reqs"]
    rot = _turned(reqs, Ls)
    pos = torch.tensor(Ls, dtype=torch.int64, device="cuda")
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
    O, lse, idx = L.decode_draft(lay, pos, max(Ls) + n_tok - 1, Q, kn, vn, with_lse=True,
                                 with_idx=(layer == "csa"), **extra)
    L.check_device_error()
    Ob, lb = T.to_f64(O), lse.cpu().numpy()
    ib = idx.cpu().numpy() if idx is not None else None
    for r, d in enumerate(rot):
        for i in range(n_tok):
            _check_query(w, layer, d, Ls[r] + i, i, Ob[r, i], lb[r, i],
                         None if ib is None else ib[r, i], "bf16", "bf16", f"req {r} tok {i}")
    _check_state(w, layer, st, rot, [x + n_tok - 1 for x in Ls], "bf16", "bf16", "draft")


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_prefill_with_rope(layer):
    """hsa_rope over the 4K prefill's K rows and queries, then the prefill
    path on the turned rows; every 5th row against the oracle."""
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, layer)
    T_ = inp["k"].shape[0]
    kr = _bits(L.rope(T.dev_bf16(inp["k"]), THETA))
    qr = _bits(L.rope(T.dev_bf16(inp["q"]), THETA))
    want = orc.rotate_tokens(inp, THETA)
    assert np.array_equal(kr, want["k"]) and np.array_equal(qr, want["q"])
    gin = dict(inp, k=kr, q=qr)
    m = w.m(layer)
    rows = list(range(0, T_, 5)) + [T_ - 1]
    gc = T.compress_layer(gin, layer, m)
    oc = orc.layer_caches(want, layer, m)
    nb = T_ // m
    for name in ("kc", "vc"):
        assert np.array_equal(T.cache_bits(gc[name], 0, nb), oc[name].bits), name
    q = L.Queries.span(T_)
    tk, tv = T.tokens(kr), T.tokens(inp["v"])
    if layer == "csa":
        idx, _ = L.indexer_topk(q, T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda(),
                                gc["kic"], m, w.n_win, w.k_csa)
        O, lse = L.csa_attn(q, T.dev_bf16(qr), tk, tv, w.n_win, gc["kc"], gc["vc"], m, idx,
                            w.k_csa, with_lse=True, out_fp32=True)
        idx = idx.cpu().numpy()
    else:
        O, lse = L.hca_attn(q, T.dev_bf16(qr), tk, tv, w.n_win, gc["kc"], gc["vc"], m,
                            with_lse=True, out_fp32=True)
    L.check_device_error()
    Ob, lb = T.to_f64(O), lse.cpu().numpy()
    for t in rows:
        if layer == "csa":
            ref = orc.csa_query(t, want["q"][t], want["qi"][t], want["w"][t], want["k"][:t + 1],
                                want["v"][:t + 1], oc["kc"], oc["vc"], oc["kic"], m, w.n_win,
                                w.k_csa)
            T.check_topk(idx[t], ref["scores"], w.k_csa, where=f"row {t}")
            sel = idx[t][idx[t] >= 0]
            if not np.array_equal(sel, ref["idx"][ref["idx"] >= 0]):
                s0 = orc.window_start(t, w.n_win)
                K = np.concatenate([nx.bf16_value(want["k"][s0:t + 1]), oc["kc"].values[sel]])
                V = np.concatenate([nx.bf16_value(want["v"][s0:t + 1]), oc["vc"].values[sel]])
                o, l = orc.attend(nx.bf16_value(want["q"][t]), K, V, T.scale_of())
                ref = {"o": o, "lse": l}
        else:
            ref = orc.hca_query(t, want["q"][t], want["k"][:t + 1], want["v"][:t + 1], oc["kc"],
                                oc["vc"], m, w.n_win)
        assert np.max(np.abs(Ob[t] - ref["o"])) <= T.OUT_TOL, f"row {t}"
        assert np.max(np.abs(lb[t] - ref["lse"])) <= T.LSE_TOL, f"row {t} lse"


PREFILL_ROWS = [0, 1, 127, 128, 129, 4095, 4096, 65535, 65536, 100000, 131070, 131071]


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_prefill_128k_with_rope_sampled(layer):
    """The 128K prefill with RoPE at full size: hsa_rope over all K rows (bit
    for bit against the oracle) and all queries (bit for bit on the sampled
    rows), the caches compressed from the turned keys (bit for bit), then the
    selection and attention; sampled rows against the oracle one by one."""
    w = configs.HYBRID_PREFILL_128K
    inp = gen.prefill_layer(w, layer)
    Tn, m = w.T, w.m(layer)
    print(f"rope prefill 128k {layer}", flush=True)
    kr = L.rope(T.dev_bf16(inp["k"]), THETA)
    Qr = L.rope(T.dev_bf16(inp["q"]), THETA)
    kt = orc.rope(inp["k"], np.arange(Tn), THETA)
    assert np.array_equal(_bits(kr), kt)
    rows = sorted(set(PREFILL_ROWS) | set(np.random.default_rng(5).integers(0, Tn, 21).tolist()))
    qt = orc.rope(inp["q"][rows], np.array(rows)[:, None], THETA)
    assert np.array_equal(_bits(Qr[rows]), qt)
    gc = T.compress_layer(dict(inp, k=_bits(kr)), layer, m)
    oc = orc.layer_caches(dict(inp, k=kt), layer, m)
    for name in oc:
        assert np.array_equal(T.cache_bits(gc[name], 0, len(oc[name])), oc[name].bits), name
    q = L.Queries.span(Tn)
    tk, tv = T.tokens(_bits(kr)), T.tokens(inp["v"])
    if layer == "csa":
        idx, _ = L.indexer_topk(q, T.dev_bf16(inp["qi"]), torch.from_numpy(inp["w"]).cuda(),
                                gc["kic"], m, w.n_win, w.k_csa)
        O, lse = L.csa_attn(q, Qr, tk, tv, w.n_win, gc["kc"], gc["vc"], m, idx, w.k_csa,
                            with_lse=True, out_fp32=True)
        idx = idx.cpu().numpy()
    else:
        O, lse = L.hca_attn(q, Qr, tk, tv, w.n_win, gc["kc"], gc["vc"], m, with_lse=True,
                            out_fp32=True)
    L.check_device_error()
    Ob, lb = T.to_f64(O[rows]), lse[rows].cpu().numpy()
    d = {"q": qt, "k": kt, "v": inp["v"]}
    if layer == "csa":
        d.update(qi=inp["qi"][rows], w=inp["w"][rows])
    for j, t in enumerate(rows):
        _check_output(w, layer, d, t, j, oc, Ob[j], lb[j], idx[t] if layer == "csa" else None,
                      f"{layer} row {t}")
