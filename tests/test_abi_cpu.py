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
    assert lib.hsa_abi_version() == 3


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


def test_decode_step_fp8_append_rules_and_bad_layers():
    """Appending to fp8 caches needs a stash per cache (the exact values of the
    page still filling); K and V must be both bf16 or both fp8 (K may be mixed)."""
    lib = L.lib()
    f = C.c_void_p(0x1000)
    Lr = L._Layer()
    Lr.kind, Lr.H, Lr.d, Lr.n_win, Lr.m, Lr.topk, Lr.H_I, Lr.d_I = 1, 64, 128, 128, 128, 0, 4, 64
    Lr.scale = 0.088
    Lr.alpha_k = Lr.alpha_v = 0x1000
    Lr.ring_k = Lr.ring_v = L._Tokens(0x1000, 128, 1, 128)
    # 10^6 tokens of context: 7,812 HCA entries need a split workspace, so a
    # valid call stops at the (16-byte) workspace check before any launch
    step = lambda ws=1 << 30: lib.hsa_decode_step(C.byref(Lr), 1, f, 10 ** 6, f, f, f, None,
                                                   None, None, f, None, None, f, ws, None)
    Lr.kc = Lr.vc = _paged(dtype=1, ppr=256)
    assert step() == -1 and b"stash" in lib.hsa_last_error()
    stashed = _paged(dtype=1, ppr=256)
    stashed.stash = 0x1000
    Lr.kc, Lr.vc = stashed, _paged(ppr=256)
    assert step() == -2                       # fp8 K with a bf16 V
    Lr.kc = Lr.vc = stashed
    assert lib.hsa_decode_step_workspace_bytes(C.byref(Lr), 1, 10 ** 6) > 16
    assert step(16) == -3                     # valid: stops at the workspace check
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


def _csa_layer(m=4, tail_cap=4, topk=1024, ring_cap=131):
    Lr = L._Layer()
    Lr.kind, Lr.H, Lr.d, Lr.n_win, Lr.m, Lr.topk, Lr.H_I, Lr.d_I = 0, 64, 128, 128, m, topk, 4, 64
    Lr.scale = 0.088
    Lr.alpha_k = Lr.alpha_v = Lr.alpha_i = 0x1000
    Lr.ring_k = Lr.ring_v = L._Tokens(0x1000, ring_cap, 1, 128)
    Lr.tail_i = L._Tokens(0x1000, tail_cap, 1, 64)
    Lr.kc = Lr.vc = _paged(ppr=1 << 14)
    Lr.kic = _paged(dim=64, ppr=1 << 14)
    return Lr


def test_decode_rewind_validation():
    lib = L.lib()
    f = C.c_void_p(0x1000)
    Lr = _csa_layer()
    assert lib.hsa_decode_rewind(None, 1, f, None) == -1
    assert lib.hsa_decode_rewind(C.byref(Lr), 0, f, None) == -1
    assert lib.hsa_decode_rewind(C.byref(Lr), 1, None, None) == -1
    assert lib.hsa_decode_rewind(C.byref(Lr), 2, f, None) == -1      # caches hold 1 request
    Lr.kc = Lr.vc = _paged(dtype=L.FP8)
    assert lib.hsa_decode_rewind(C.byref(Lr), 1, f, None) == -1     # fp8 without stashes
    Lr.kc = _paged()
    assert lib.hsa_decode_rewind(C.byref(Lr), 1, f, None) == -2     # bf16 K, fp8 V


def test_draft_needs_a_tail_for_rewinds():
    """A CSA draft of n tokens needs an indexer tail of m + n - 1 rows: a
    rejected token must not overwrite a kept token of the block still open."""
    lib = L.lib()
    f = C.c_void_p(0x1000)
    # a 16-byte workspace: a call that passes validation stops at the
    # workspace check (-3) before anything is enqueued
    call = lambda Lr, n_tok: lib.hsa_decode_draft(C.byref(Lr), 1, n_tok, f, 1000, f, f, f, f, f,
                                                  f, f, None, None, f, 16, None)
    assert call(_csa_layer(tail_cap=4), 4) == -1
    assert b"tail_i" in lib.hsa_last_error()
    assert call(_csa_layer(tail_cap=4 + 3), 4) == -3
    # fp4 indexer keys: single-token steps only (the grouped draft scan has no fp4 path)
    Lr = _csa_layer(tail_cap=4 + 3)
    Lr.kic = _paged(dim=64, dtype=L.FP4, ppr=1 << 14)
    assert call(Lr, 4) == -2
    assert b"fp4" in lib.hsa_last_error()
    # fp8 indexer keys stay outside the decode step
    Lr.kic = _paged(dim=64, dtype=L.FP8, ppr=1 << 14)
    assert call(Lr, 4) == -2


def _rnd(b):
    return (b + 255) // 256 * 256


def _grouped_indexer_bytes(nq, nvis):
    """The draft scan's workspace layout: one histogram list of up to 512 bins
    per 512-block chunk, fp32 scores, a bitmap, two candidate arrays and the
    per-2048-block candidate counts, for nq queries over rows of R blocks."""
    R = max(2048, -(-nvis // 2048) * 2048)
    n_lists = R // 512
    return (_rnd(4 * 8 * nq) + _rnd(4 * n_lists * nq) + _rnd(4 * 512 * n_lists * nq) +
            _rnd(4 * R * nq) + _rnd(R // 8 * nq) + 2 * _rnd(8 * R * nq) + _rnd(4 * (R // 2048) * nq))


@pytest.mark.parametrize("max_pos", [600_000, 1_048_579])
def test_draft_workspace_covers_the_grouped_scan(max_pos):
    """At rows of more than 131,072 blocks the single-query scan groups four
    chunks per histogram list, the draft scan does not; a draft's workspace
    must hold the draft scan's (larger) list layout."""
    lib = L.lib()
    B, n_tok, topk = 4, 4, 1024
    Lr = _csa_layer(tail_cap=4 + n_tok - 1, topk=topk, ring_cap=128 + n_tok - 1)
    n = B * n_tok
    nvis = min(-(-max(0, max_pos - 127) // 4), (max_pos + 1) // 4)
    q = L._Queries(n, C.c_void_p(0x1000), C.c_void_p(0x1000), 0, 0, max_pos)
    attn = _rnd(lib.hsa_csa_attn_workspace_bytes(C.byref(q), 64, 128, topk))
    need = _rnd(8 * n) + _rnd(4 * n) + _rnd(_grouped_indexer_bytes(n, nvis)) + _rnd(4 * n * topk) + attn
    assert lib.hsa_decode_draft_workspace_bytes(C.byref(Lr), B, n_tok, max_pos) >= need


def test_noalloc_step_refuses_steps_beyond_its_scratch():
    """A step whose workspace exceeds the library's 128 MiB scratch returns
    HSA_ERR_WORKSPACE before anything is enqueued."""
    lib = L.lib()
    f = C.c_void_p(0x1000)
    Lr = _csa_layer(topk=1024)
    Lr.kc = Lr.vc = _paged(ppr=1 << 16)
    Lr.kic = _paged(dim=64, ppr=1 << 16)
    B = 1
    Lr.kc.n_req = Lr.vc.n_req = Lr.kic.n_req = 64
    Lr.ring_k.n_req = Lr.ring_v.n_req = Lr.tail_i.n_req = 64
    need = lib.hsa_decode_step_workspace_bytes(C.byref(Lr), 64, 4 << 20)
    assert need > 128 << 20
    assert lib.hsa_decode_step_noalloc(C.byref(Lr), 64, f, 4 << 20, f, f, f, f, f, f, f, None,
                                       None, None) == -3
    assert b"scratch" in lib.hsa_last_error()


def test_rope_validation():
    """hsa_rope: heads >= 1, dim a multiple of 8 in [64, 4096], theta > 0 and
    finite, 16-byte aligned rows, y equal to x or apart from it, positions
    that cannot overflow; an empty call is a no-op."""
    lib = L.lib()
    f, g = C.c_void_p(0x1000), C.c_void_p(0x1000 + 64 * 128 * 2)
    r = lambda x=f, y=f, n=64, h=1, d=128, pos=None, p0=0, th=10000.0: lib.hsa_rope(
        x, y, n, h, d, pos, p0, th, None)
    assert r(n=0, x=None, y=None) == 0
    assert r(x=None) == -1
    assert r(n=-1) == -1
    assert r(h=0) == -1
    assert r(d=32) == -1 and r(d=100) == -1
    assert r(th=0.0) == -1 and r(th=-1.0) == -1 and r(th=float("inf")) == -1
    assert r(x=C.c_void_p(0x1008)) == -1                     # not 16-byte aligned
    assert r(y=C.c_void_p(0x1000 + 128)) == -1                # overlaps x, not equal
    assert r(p0=-1) == -1
    assert r(p0=(1 << 63) - 10) == -1                         # pos0 + n overflows
    assert b"rope" in lib.hsa_last_error()


def test_decode_rope_theta_rules_and_workspace():
    """A layer's rope_theta must be finite and >= 0; with RoPE the step's
    workspace also holds the turned queries (B x H x 128 bf16)."""
    lib = L.lib()
    f = C.c_void_p(0x1000)
    Lr = _csa_layer(tail_cap=4)
    base = lib.hsa_decode_step_workspace_bytes(C.byref(Lr), 2, 1000)
    Lr.rope_theta = 10000.0
    with_rope = lib.hsa_decode_step_workspace_bytes(C.byref(Lr), 2, 1000)
    assert with_rope >= base + 2 * 64 * 128 * 2
    d0 = lib.hsa_decode_draft_workspace_bytes(C.byref(Lr), 2, 3, 1000)
    Lr.rope_theta = 0.0
    assert d0 >= lib.hsa_decode_draft_workspace_bytes(C.byref(Lr), 2, 3, 1000) + 6 * 64 * 128 * 2
    for bad in (-1.0, float("nan"), float("inf")):
        Lr.rope_theta = bad
        assert lib.hsa_decode_step(C.byref(Lr), 1, f, 1000, f, f, f, f, f, f, f, None, None, f,
                                   1 << 30, None) == -1
        assert b"rope_theta" in lib.hsa_last_error()


def test_csa_prefill_validation():
    """hsa_csa_prefill takes spans only and checks the indexer's and the
    attention's arguments, its stage size and its workspace, on the host."""
    lib = L.lib()
    f = C.c_void_p(0x1000)
    q = L._Queries(4, None, None, 0, 0, 3)
    pc, ki, tk = _paged(), _paged(dim=64), _tokens()
    nb = lib.hsa_csa_prefill_workspace_bytes(C.byref(q), 16, 4, 128, 16)
    assert nb >= lib.hsa_indexer_topk_workspace_bytes(C.byref(q), 4, 128, 16) > 0
    big = 1 << 30

    def call(qq=q, hi=4, kic=ki, idx=f, ws_bytes=big, stage=0, H=16, o_dtype=0):
        return lib.hsa_csa_prefill(C.byref(qq), f, f, hi, 64, C.byref(kic), f, H, 128,
                                   C.byref(tk), C.byref(tk), 128, C.byref(pc), C.byref(pc), 4,
                                   16, 0.1, idx, f, o_dtype, None, stage, f, ws_bytes, None)

    pos = C.c_void_p(0x2000)
    listed = L._Queries(4, None, pos, 0, 0, 3)
    assert call(qq=listed) == -1 and b"span" in lib.hsa_last_error()
    assert call(idx=None) == -1
    assert call(hi=8) == -2
    assert call(stage=-1) == -1
    assert call(H=24) == -2
    assert call(o_dtype=7) == -1
    assert call(ws_bytes=16) == -3
    assert call(kic=_paged(dim=128)) == -2
