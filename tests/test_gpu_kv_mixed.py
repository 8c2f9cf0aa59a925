"""GPU parity of the mixed KV entry (the wiki's §8: RoPE channels in BF16, the
others in FP8): compressed K caches stored as HSA_FP8_BF16_ROPE -- the first
64 channels e4m3 codes with a page scale over those channels, the 64 RoPE
channels bf16 -- with an fp8 V cache, against the oracle over the same
storage: the caches bit for bit, and CSA and HCA outputs, decode and prefill,
within the tolerances of the other formats."""
import numpy as np
import pytest
import torch

from oracle import hybrid as orc
from synth import configs, gen

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L
from test_gpu_fullsize import check_decode
from test_gpu_prefill import _check_csa_rows, _run_prefill_csa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_compress_mixed_bitexact(layer):
    w = configs.PREFILL_4K
    d = gen.prefill_layer(w, layer)
    m = w.m(layer)
    nb = d["k"].shape[0] // m
    perm = torch.from_numpy(gen.page_permutation(w, "mix" + layer, -(-nb // 64)))
    c = L.PagedCache.allocate(1, nb, 128, mixed=True, page_order=perm)
    L.kv_compress(T.tokens(d["k"]), c, 0, 0, nb, m, L.pooling_weights(torch.from_numpy(d["zk"]).cuda()))
    L.check_device_error()
    rows, scales = orc.store_mixed_pages(orc.compress_exact(d["k"], orc.pooling_weights(d["zk"]), m))
    assert int(c.n_entries[0]) == nb
    assert np.array_equal(T.cache_bits(c, 0, nb), rows)
    assert np.array_equal(c.logical_scales(0, nb).cpu().numpy().view(np.uint32), scales.view(np.uint32))


def _oracle_caches(w, layer, d, n):
    m = w.m(layer)
    z = gen.pool_logits(w, layer)
    out = {"kc": orc.compress(d["k"][:n], z["zk"], m, "mixed"),
           "vc": orc.compress(d["v"][:n], z["zv"], m, "fp8")}
    if layer == "csa":
        out["kic"] = orc.compress(d["ki"][:n], z["zi"], m)
    return out


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_decode_mixed(layer):
    """The Pro decode shape (128 heads, CSA top-1024 and HCA) on rows of 131 to
    70,000 tokens, shuffled pages."""
    Ls = [131, 3000, 20001, 70000]
    w = configs.shrink(configs.PRO_DECODE_1M, B=len(Ls))
    st = T.build_state(w, layer, Ls, kmix=True)
    out = T.run_ops(w, layer, st, Ls)
    worst = 0.0
    for r, d in enumerate(st["reqs"]):
        oc = _oracle_caches(w, layer, d, Ls[r])
        for name in ("kc", "vc"):
            n = len(oc[name])
            assert np.array_equal(T.cache_bits(st[name], r, n), oc[name].bits), (r, name)
            assert np.array_equal(st[name].logical_scales(r, n).cpu().numpy().view(np.uint32),
                                  oc[name].scales.view(np.uint32)), (r, name)
        worst = max(worst, check_decode(w, layer, d, Ls[r], 0, oc,
                                        out["idx"][r] if layer == "csa" else None,
                                        out["O"][r], out["lse"][r], f"{layer} req {r}"))
    print(f"mixed K decode {layer}: max abs error {worst:.3e}")


def test_prefill_mixed_csa():
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "csa")
    idx, score, O, lse = _run_prefill_csa(w, inp, kmix=True)
    _check_csa_rows(w, inp, idx, score, O, lse, range(0, 4096, 3), dtype="mixed")


def test_prefill_mixed_hca():
    w = configs.PREFILL_4K
    inp = gen.prefill_layer(w, "hca")
    m, n_win = w.m_hca, w.n_win
    gc = T.compress_layer(inp, "hca", m, kmix=True)
    q = L.Queries.span(4096)
    O, lse = L.hca_attn(q, T.dev_bf16(inp["q"]), T.tokens(inp["k"]), T.tokens(inp["v"]), n_win,
                        gc["kc"], gc["vc"], m, with_lse=True, out_fp32=True)
    L.check_device_error()
    oc = orc.layer_caches(inp, "hca", m, "mixed")
    Ob, lse = T.to_f64(O), lse.cpu().numpy()
    for t in range(0, 4096, 3):
        r = orc.hca_query(t, inp["q"][t], inp["k"], inp["v"], oc["kc"], oc["vc"], m, n_win)
        assert np.max(np.abs(Ob[t] - r["o"])) <= T.OUT_TOL, t
        assert np.max(np.abs(lse[t] - r["lse"])) <= T.LSE_TOL, t
