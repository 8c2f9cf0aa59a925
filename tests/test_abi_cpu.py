"""The C ABI library loads, exports every entry point its header declares, and
rejects invalid arguments on the host before touching the GPU."""
import ctypes as C
import os
import re

import pytest

from long_context_hybrid_kv_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hsa_attn.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hsa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    names = declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(L._SIGS), "binding misses a declared entry point"
    assert lib.hsa_abi_version() == 1


def test_status_strings():
    lib = L.lib()
    assert lib.hsa_status_string(0) == b"ok"
    assert lib.hsa_status_string(-3) == b"workspace too small"


def _paged(dim=128, dtype=0, ppr=4, fake=0x1000):
    return L._Paged(fake, fake if dtype in (1, 3, 4) else None, fake, fake, 1, ppr, ppr, 64, dim, dtype)


def _tokens(cap=4096, dim=128, fake=0x1000):
    return L._Tokens(fake, cap, 1, dim)


def test_validation_rejects_before_any_launch():
    lib = L.lib()
    q = L._Queries(4, None, None, 0, 0, 3)
    pc = _paged()
    tk = _tokens()
    # null pooling pointer
    assert lib.hsa_pooling_weights(None, 4, 128, None, None) == -1
    # compress: fp8 range not on a page boundary
    p8 = _paged(dtype=1)
    assert lib.hsa_kv_compress(C.byref(tk), 0, C.byref(p8), 0, 3, 10, 4, C.c_void_p(0x1000), None) == -1
    assert b"page boundary" in lib.hsa_last_error()
    # compress: range beyond the page table
    assert lib.hsa_kv_compress(C.byref(tk), 0, C.byref(pc), 0, 0, 4 * 64 + 1, 4, C.c_void_p(0x1000), None) == -1
    # compress: unsupported dim
    p96 = _paged(dim=96)
    assert lib.hsa_kv_compress(C.byref(_tokens(dim=96)), 0, C.byref(p96), 0, 0, 1, 4, C.c_void_p(0x1000), None) == -2
    # indexer: bad head count, m > n_win, workspace too small
    ki = _paged(dim=64)
    f = C.c_void_p(0x1000)
    assert lib.hsa_indexer_topk(C.byref(q), f, f, 8, 64, C.byref(ki), 4, 128, 16, f, None, f, 1 << 30, None) == -2
    assert lib.hsa_indexer_topk(C.byref(q), f, f, 4, 64, C.byref(ki), 256, 128, 16, f, None, f, 1 << 30, None) == -2
    assert lib.hsa_indexer_topk(C.byref(q), f, f, 4, 64, C.byref(ki), 4, 128, 16, f, None, f, 16, None) == -3
    # empty query set
    q0 = L._Queries(0, None, None, 0, 0, 0)
    assert lib.hsa_indexer_topk(C.byref(q0), f, f, 4, 64, C.byref(ki), 4, 128, 16, f, None, f, 1 << 30, None) == -1
    # the bf16-score selector checks its arguments the same way
    bs = lib.hsa_indexer_topk_bf16_scores
    assert bs(C.byref(q), f, f, 8, 64, C.byref(ki), 4, 128, 16, f, None, f, 1 << 30, None) == -2
    assert bs(C.byref(q), f, f, 4, 64, C.byref(ki), 4, 128, 16, f, None, f, 16, None) == -3
    assert bs(C.byref(q0), f, f, 4, 64, C.byref(ki), 4, 128, 16, f, None, f, 1 << 30, None) == -1
    assert bs(C.byref(q), f, f, 4, 64, C.byref(ki), 4, 128, 0, f, None, f, 1 << 30, None) == -1
    # attention: H not a multiple of 16, d != 128, window capacity too small
    assert lib.hsa_hca_attn(C.byref(q), f, 24, 128, C.byref(tk), C.byref(tk), 128, C.byref(pc), C.byref(pc), 128, 0.1, f, 0, None, f, 1 << 30, None) == -2
    assert lib.hsa_hca_attn(C.byref(q), f, 16, 64, C.byref(tk), C.byref(tk), 128, C.byref(pc), C.byref(pc), 128, 0.1, f, 0, None, f, 1 << 30, None) == -2
    small = _tokens(cap=2)
    assert lib.hsa_hca_attn(C.byref(q), f, 16, 128, C.byref(small), C.byref(small), 128, C.byref(pc), C.byref(pc), 128, 0.1, f, 0, None, f, 1 << 30, None) == -1
    # span beyond max_pos
    qb = L._Queries(4, None, None, 0, 10, 3)
    assert lib.hsa_hca_attn(C.byref(qb), f, 16, 128, C.byref(tk), C.byref(tk), 128, C.byref(pc), C.byref(pc), 128, 0.1, f, 0, None, f, 1 << 30, None) == -1
    # unknown output dtype
    assert lib.hsa_hca_attn(C.byref(q), f, 16, 128, C.byref(tk), C.byref(tk), 128, C.byref(pc), C.byref(pc), 128, 0.1, f, 1, None, f, 1 << 30, None) == -1
    # non-positive or non-finite logit scale
    for bad in (0.0, -0.1, float("inf"), float("nan")):
        assert lib.hsa_hca_attn(C.byref(q), f, 16, 128, C.byref(tk), C.byref(tk), 128, C.byref(pc), C.byref(pc), 128, bad, f, 0, None, f, 1 << 30, None) == -1
    assert b"scale" in lib.hsa_last_error()
    # the mixed bf16-RoPE / fp8 entry: K caches of dim 128 with an fp8 V cache only
    km, k8 = _paged(dtype=L.FP8_BF16_ROPE), _paged(dtype=L.FP8)
    hca = lambda kc, vc: lib.hsa_hca_attn(C.byref(q), f, 16, 128, C.byref(tk), C.byref(tk), 128, C.byref(kc), C.byref(vc), 128, 0.1, f, 0, None, f, 1 << 30, None)
    assert hca(km, pc) == -2                      # with a bf16 V
    assert hca(km, km) == -2                      # as the V cache
    assert hca(pc, k8) == -2                      # bf16 K with fp8 V
    assert lib.hsa_indexer_topk(C.byref(q), f, f, 4, 64, C.byref(_paged(dim=64, dtype=L.FP8_BF16_ROPE)), 4, 128, 16, f, None, f, 1 << 30, None) == -2
    assert lib.hsa_kv_compress(C.byref(_tokens(dim=64)), 0, C.byref(_paged(dim=64, dtype=L.FP8_BF16_ROPE)), 0, 0, 1, 4, f, None) == -2
    assert lib.hsa_kv_compress(C.byref(tk), 0, C.byref(km), 0, 3, 10, 4, f, None) == -1   # not page-aligned
    assert lib.hsa_kv_compress(C.byref(tk), 0, C.byref(L._Paged(0x1000, None, 0x1000, 0x1000, 1, 4, 4, 64, 128, L.FP8_BF16_ROPE)), 0, 0, 1, 4, f, None) == -1   # no scales
    # fp4: compressed indexer keys of dim 64 only
    k4 = _paged(dim=64, dtype=L.FP4)
    assert hca(_paged(dtype=L.FP4), _paged(dtype=L.FP4)) == -2          # as K / V caches
    assert lib.hsa_kv_compress(C.byref(tk), 0, C.byref(_paged(dtype=L.FP4)), 0, 0, 1, 4, f, None) == -2
    assert lib.hsa_kv_compress(C.byref(_tokens(dim=64)), 0, C.byref(k4), 0, 3, 10, 4, f, None) == -1
    # CSA without idx
    assert lib.hsa_csa_attn(C.byref(q), f, 16, 128, C.byref(tk), C.byref(tk), 128, C.byref(pc), C.byref(pc), 4, None, 64, 0.1, f, 0, None, f, 1 << 30, None) == -1


def test_decode_step_rejects_fp8_append_and_bad_layers():
    lib = L.lib()
    f = C.c_void_p(0x1000)
    Lr = L._Layer()
    Lr.kind, Lr.H, Lr.d, Lr.n_win, Lr.m, Lr.topk, Lr.H_I, Lr.d_I = 1, 64, 128, 128, 128, 0, 4, 64
    Lr.scale = 0.088
    Lr.alpha_k = Lr.alpha_v = 0x1000
    Lr.ring_k = Lr.ring_v = L._Tokens(0x1000, 128, 1, 128)
    Lr.kc = Lr.vc = _paged(dtype=1)
    assert lib.hsa_decode_step(C.byref(Lr), 1, f, 1000, f, f, f, None, None, None, f, None, None, f, 1 << 30, None) == -2
    Lr.kc = Lr.vc = _paged()
    Lr.kind = 7
    assert lib.hsa_decode_step(C.byref(Lr), 1, f, 1000, f, f, f, None, None, None, f, None, None, f, 1 << 30, None) == -1
    Lr.kind = 0   # CSA without indexer inputs
    assert lib.hsa_decode_step(C.byref(Lr), 1, f, 1000, f, f, f, None, None, None, f, None, None, f, 1 << 30, None) == -1
    assert lib.hsa_decode_step_workspace_bytes(C.byref(Lr), 0, 1000) == 0


def test_decode_draft_validation():
    """Drafts need 1 <= n_tok <= 256 and rings that keep the first draft
    query's window while the later tokens are written (n_win + n_tok - 1)."""
    lib = L.lib()
    f = C.c_void_p(0x1000)
    Lr = L._Layer()
    Lr.kind, Lr.H, Lr.d, Lr.n_win, Lr.m, Lr.topk, Lr.H_I, Lr.d_I = 1, 64, 128, 128, 128, 0, 4, 64
    Lr.scale = 0.088
    Lr.alpha_k = Lr.alpha_v = 0x1000
    Lr.ring_k = Lr.ring_v = L._Tokens(0x1000, 128, 1, 128)     # capacity n_win only
    Lr.kc = Lr.vc = _paged()
    call = lambda n_tok: lib.hsa_decode_draft(C.byref(Lr), 1, n_tok, f, 1000, f, f, f, None, None,
                                              None, f, None, None, f, 1 << 30, None)
    assert call(0) == -1
    assert call(257) == -1
    assert call(4) == -1                       # ring too small for a 4-token draft
    assert lib.hsa_decode_draft_workspace_bytes(C.byref(Lr), 1, 0, 1000) == 0
    assert lib.hsa_decode_draft_workspace_bytes(C.byref(Lr), 2, 4, 1000) > 0


def test_workspace_sizes_are_consistent():
    lib = L.lib()
    q = L._Queries(4, None, C.c_void_p(0x1000), 0, 0, 1048576)
    a = lib.hsa_indexer_topk_workspace_bytes(C.byref(q), 4, 128, 1024)
    assert a > 4 * 262113 * 4          # at least the fp32 scores
    qs = L._Queries(131072, None, None, 0, 0, 131071)
    b = lib.hsa_indexer_topk_workspace_bytes(C.byref(qs), 4, 128, 512)
    assert 0 < b < 8 << 30             # prefill is processed in query chunks
    assert lib.hsa_csa_attn_workspace_bytes(C.byref(qs), 64, 128, 512) == 0   # no split in prefill
