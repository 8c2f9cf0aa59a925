"""ctypes binding of libhsa_attn.so: argument marshalling only.

Every entry point here forwards to the C ABI declared in include/hsa_attn.h
with the same name (minus the `hsa_` prefix).  Tensors are torch tensors on
the current HIP device; pointers and the current stream are passed through,
workspaces are allocated with torch (the library itself never allocates).
No computation happens in Python: if the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes as C
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch  # load torch's HIP runtime first: the library binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
# HSA_ATTN_LIB names another build of the same library (the host-sanitizer
# build); by default the in-tree libhsa_attn.so
LIB_PATH = os.environ.get("HSA_ATTN_LIB") or os.path.join(_HERE, "libhsa_attn.so")

BF16, FP8, FP32, FP8_BF16_ROPE, FP4 = 0, 1, 2, 3, 4
LAYER_CSA, LAYER_HCA = 0, 1
FAULT_BITS = {1: "page", 2: "pos", 4: "entries", 8: "index", 16: "req", 32: "range"}


class HsaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class _Tokens(C.Structure):
    _fields_ = [("data", C.c_void_p), ("capacity", C.c_int64), ("n_req", C.c_int32),
                ("dim", C.c_int32)]


class _Paged(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scale", C.c_void_p), ("page_table", C.c_void_p),
                ("n_entries", C.c_void_p), ("n_req", C.c_int32), ("pages_per_req", C.c_int32),
                ("n_pages", C.c_int32), ("page_size", C.c_int32), ("dim", C.c_int32),
                ("dtype", C.c_int32), ("stash", C.c_void_p)]


class _Queries(C.Structure):
    _fields_ = [("n", C.c_int32), ("req", C.c_void_p), ("pos", C.c_void_p),
                ("span_req", C.c_int32), ("span_pos0", C.c_int64), ("max_pos", C.c_int64)]


class _Layer(C.Structure):
    _fields_ = [("kind", C.c_int32), ("H", C.c_int32), ("d", C.c_int32), ("n_win", C.c_int32),
                ("m", C.c_int32), ("topk", C.c_int32), ("H_I", C.c_int32), ("d_I", C.c_int32),
                ("scale", C.c_float), ("o_dtype", C.c_int32), ("alpha_k", C.c_void_p), ("alpha_v", C.c_void_p),
                ("alpha_i", C.c_void_p), ("ring_k", _Tokens), ("ring_v", _Tokens),
                ("tail_i", _Tokens), ("kc", _Paged), ("vc", _Paged), ("kic", _Paged),
                ("rope_theta", C.c_double)]


_SIGS = {
    "hsa_abi_version": (C.c_int32, []),
    "hsa_rope": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p,
                           C.c_int64, C.c_double, C.c_void_p]),
    "hsa_last_error": (C.c_char_p, []),
    "hsa_status_string": (C.c_char_p, [C.c_int]),
    "hsa_check_device_error": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32)]),
    "hsa_pooling_weights": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "hsa_kv_compress": (C.c_int, [C.POINTER(_Tokens), C.c_int32, C.POINTER(_Paged), C.c_int32,
                                  C.c_int64, C.c_int64, C.c_int32, C.c_void_p, C.c_void_p]),
    "hsa_indexer_topk_workspace_bytes": (C.c_size_t, [C.POINTER(_Queries), C.c_int32, C.c_int32,
                                                      C.c_int32]),
    "hsa_indexer_topk": (C.c_int, [C.POINTER(_Queries), C.c_void_p, C.c_void_p, C.c_int32,
                                   C.c_int32, C.POINTER(_Paged), C.c_int32, C.c_int32, C.c_int32,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "hsa_indexer_topk_bf16_scores": (C.c_int, [C.POINTER(_Queries), C.c_void_p, C.c_void_p,
                                               C.c_int32, C.c_int32, C.POINTER(_Paged), C.c_int32,
                                               C.c_int32, C.c_int32, C.c_void_p, C.c_void_p,
                                               C.c_void_p, C.c_size_t, C.c_void_p]),
    "hsa_csa_attn_workspace_bytes": (C.c_size_t, [C.POINTER(_Queries), C.c_int32, C.c_int32,
                                                  C.c_int32]),
    "hsa_csa_attn": (C.c_int, [C.POINTER(_Queries), C.c_void_p, C.c_int32, C.c_int32,
                               C.POINTER(_Tokens), C.POINTER(_Tokens), C.c_int32,
                               C.POINTER(_Paged), C.POINTER(_Paged), C.c_int32, C.c_void_p,
                               C.c_int32, C.c_float, C.c_void_p, C.c_int32, C.c_void_p,
                               C.c_void_p, C.c_size_t, C.c_void_p]),
    "hsa_csa_prefill_workspace_bytes": (C.c_size_t, [C.POINTER(_Queries), C.c_int32, C.c_int32,
                                                     C.c_int32, C.c_int32]),
    "hsa_csa_prefill": (C.c_int, [C.POINTER(_Queries), C.c_void_p, C.c_void_p, C.c_int32,
                                  C.c_int32, C.POINTER(_Paged), C.c_void_p, C.c_int32, C.c_int32,
                                  C.POINTER(_Tokens), C.POINTER(_Tokens), C.c_int32,
                                  C.POINTER(_Paged), C.POINTER(_Paged), C.c_int32, C.c_int32,
                                  C.c_float, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                  C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]),
    "hsa_hca_attn_workspace_bytes": (C.c_size_t, [C.POINTER(_Queries), C.c_int32, C.c_int32,
                                                  C.c_int32]),
    "hsa_hca_attn": (C.c_int, [C.POINTER(_Queries), C.c_void_p, C.c_int32, C.c_int32,
                               C.POINTER(_Tokens), C.POINTER(_Tokens), C.c_int32,
                               C.POINTER(_Paged), C.POINTER(_Paged), C.c_int32, C.c_float,
                               C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t,
                               C.c_void_p]),
    "hsa_kernel_timing": (C.c_int, [C.c_int32, C.c_int32]),
    "hsa_kernel_timing_read": (C.c_int, [C.c_int32, C.POINTER(C.c_double),
                                         C.POINTER(C.c_int64)]),
    "hsa_decode_step_workspace_bytes": (C.c_size_t, [C.POINTER(_Layer), C.c_int32, C.c_int64]),
    "hsa_decode_step": (C.c_int, [C.POINTER(_Layer), C.c_int32, C.c_void_p, C.c_int64,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_size_t, C.c_void_p]),
    "hsa_decode_step_noalloc": (C.c_int, [C.POINTER(_Layer), C.c_int32, C.c_void_p, C.c_int64,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                          C.c_void_p, C.c_void_p]),
    "hsa_decode_rewind": (C.c_int, [C.POINTER(_Layer), C.c_int32, C.c_void_p, C.c_void_p]),
    "hsa_decode_draft_workspace_bytes": (C.c_size_t, [C.POINTER(_Layer), C.c_int32, C.c_int32,
                                                      C.c_int64]),
    "hsa_decode_draft": (C.c_int, [C.POINTER(_Layer), C.c_int32, C.c_int32, C.c_void_p, C.c_int64,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_size_t, C.c_void_p]),
}

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m long_context_hybrid_kv_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def _check(status: int, where: str):
    if status != 0:
        L = lib()
        raise HsaError(status, where,
                       f"{L.hsa_status_string(status).decode()}: {L.hsa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


# ----------------------------------------------------------------------------- descriptors

@dataclass
class Tokens:
    """Raw bf16 rows [n_req, capacity, dim]; token p of request r is row p % capacity."""
    data: torch.Tensor

    def c(self) -> _Tokens:
        n_req, cap, dim = self.data.shape
        assert self.data.dtype == torch.bfloat16 and self.data.is_contiguous()
        return _Tokens(self.data.data_ptr(), cap, n_req, dim)


@dataclass
class PagedCache:
    """Compressed cache: pages [n_pages, 64, dim] (bf16, or uint8 fp8 codes with
    `scale` [n_pages]; mixed: uint8 rows of dim/2 fp8 codes then dim/2 bf16
    RoPE channels, [n_pages, 64, 3*dim/2] bytes, with `scale`), page_table
    [n_req, pages_per_req], n_entries [n_req]."""
    data: torch.Tensor
    page_table: torch.Tensor
    n_entries: torch.Tensor
    scale: Optional[torch.Tensor] = None
    mixed: bool = False
    fp4: bool = False
    stash: Optional[torch.Tensor] = None    # fp8 caches appended to: float64 [n_req, 128, dim]

    @property
    def dtype(self) -> int:
        if self.mixed:
            return FP8_BF16_ROPE
        if self.fp4:
            return FP4
        return FP8 if self.data.dtype == torch.uint8 else BF16

    @property
    def dim(self) -> int:
        if self.mixed:
            return self.data.shape[-1] * 2 // 3
        return self.data.shape[-1] * 2 if self.fp4 else self.data.shape[-1]

    @staticmethod
    def allocate(n_req: int, max_entries: int, dim: int, fp8: bool = False,
                 page_order: Optional[torch.Tensor] = None, device="cuda",
                 mixed: bool = False, fp4: bool = False, stash: bool = False) -> "PagedCache":
        """mixed: HSA_FP8_BF16_ROPE rows (compressed K caches); fp4:
        HSA_FP4_E2M1_MX rows (indexer keys) with `scale` the e8m0 block-scale
        bytes [n_pages, 64, dim / 32]; stash (fp8 and mixed): the float64
        values of each request's last 128 entries, which decoding needs to
        append to an fp8 cache."""
        ppr = max(1, -(-max_entries // 64))
        n_pages = n_req * ppr
        if mixed:
            data = torch.zeros((n_pages, 64, dim // 2 * 3), dtype=torch.uint8, device=device)
        elif fp4:
            data = torch.zeros((n_pages, 64, dim // 2), dtype=torch.uint8, device=device)
        else:
            dt = torch.uint8 if fp8 else torch.bfloat16
            data = torch.zeros((n_pages, 64, dim), dtype=dt, device=device)
        if page_order is None:
            page_order = torch.arange(n_pages, dtype=torch.int32)
        table = page_order.to(torch.int32).reshape(n_req, ppr).to(device)
        if fp4:
            scale = torch.full((n_pages, 64, dim // 32), 127, dtype=torch.uint8, device=device)
        else:
            scale = (torch.ones(n_pages, dtype=torch.float32, device=device) if fp8 or mixed
                     else None)
        st = (torch.zeros((n_req, 128, dim), dtype=torch.float64, device=device)
              if stash and (fp8 or mixed) else None)
        return PagedCache(data, table.contiguous(),
                          torch.zeros(n_req, dtype=torch.int32, device=device), scale, mixed, fp4,
                          st)

    def c(self) -> _Paged:
        n_pages, ps, _ = self.data.shape
        n_req, ppr = self.page_table.shape
        return _Paged(self.data.data_ptr(), None if self.scale is None else self.scale.data_ptr(),
                      self.page_table.data_ptr(), self.n_entries.data_ptr(), n_req, ppr, n_pages,
                      ps, self.dim, self.dtype,
                      None if self.stash is None else self.stash.data_ptr())

    def logical(self, r: int, n: Optional[int] = None) -> torch.Tensor:
        """Entries 0..n-1 of request r in logical order (a gather, for inspection)."""
        n = int(self.n_entries[r].item()) if n is None else n
        pages = self.page_table[r, : -(-n // 64)].long()
        return self.data[pages].reshape(-1, self.data.shape[-1])[:n]

    def logical_scales(self, r: int, n: int) -> torch.Tensor:
        """Page scales of the pages holding entries 0..n-1 (fp4: the block-scale
        bytes of entries 0..n-1, [n, dim / 32])."""
        pages = self.page_table[r, : -(-n // 64)].long()
        if self.fp4:
            return self.scale[pages].reshape(-1, self.scale.shape[-1])[:n]
        return self.scale[pages]


@dataclass
class Queries:
    """A span of consecutive positions of one request, or a list of (req, pos)."""
    n: int
    max_pos: int
    span_req: int = 0
    span_pos0: int = 0
    pos: Optional[torch.Tensor] = None      # int64 [n]
    req: Optional[torch.Tensor] = None      # int32 [n]

    @staticmethod
    def span(n: int, pos0: int = 0, req: int = 0) -> "Queries":
        return Queries(n=n, max_pos=pos0 + n - 1, span_req=req, span_pos0=pos0)

    @staticmethod
    def list(pos: torch.Tensor, max_pos: int, req: Optional[torch.Tensor] = None) -> "Queries":
        return Queries(n=pos.shape[0], max_pos=max_pos, pos=pos, req=req)

    def c(self) -> _Queries:
        return _Queries(self.n, None if self.req is None else self.req.data_ptr(),
                        None if self.pos is None else self.pos.data_ptr(), self.span_req,
                        self.span_pos0, self.max_pos)


class Workspaces:
    """Device workspaces, one per call site, grown on demand and reused across
    calls (the library clears what it needs at the start of every call)."""

    def __init__(self):
        self._ws = {}

    def get(self, key, nbytes: int, device) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes or t.device != torch.device(device):
            t = torch.empty(nbytes, dtype=torch.uint8, device=device)
            self._ws[key] = t
        return t


_WS = Workspaces()


def _ws_args(ws: Optional[torch.Tensor]):
    return (None, 0) if ws is None else (C.c_void_p(ws.data_ptr()), ws.numel())


# ----------------------------------------------------------------------------- entry points

def abi_version() -> int:
    return lib().hsa_abi_version()


def check_device_error() -> int:
    """Synchronise the current stream; raise if a kernel set a fault bit."""
    bits = C.c_int32(0)
    st = lib().hsa_check_device_error(_stream(), C.byref(bits))
    if st != 0:
        names = [v for k, v in FAULT_BITS.items() if bits.value & k]
        _check(st, f"device fault {names}")
    return bits.value


K_INDEXER_SCAN, K_INDEXER_GEMM, K_INDEXER_SEL, K_ATTN, K_COMPRESS = range(5)


def kernel_timing(kernel_id: int, enable: bool) -> None:
    _check(lib().hsa_kernel_timing(kernel_id, int(enable)), "kernel_timing")


def kernel_timing_read(kernel_id: int):
    """(total milliseconds, launches) of a timed kernel since the last read."""
    ms, n = C.c_double(0), C.c_int64(0)
    _check(lib().hsa_kernel_timing_read(kernel_id, C.byref(ms), C.byref(n)), "kernel_timing_read")
    return ms.value, n.value


def pooling_weights(z: torch.Tensor) -> torch.Tensor:
    z = z.contiguous().float()
    alpha = torch.empty_like(z)
    _check(lib().hsa_pooling_weights(_ptr(z), z.shape[0], z.shape[1], _ptr(alpha), _stream()),
           "pooling_weights")
    return alpha


def rope(x: torch.Tensor, theta: float, pos: Optional[torch.Tensor] = None, pos0: int = 0,
         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hsa_rope over bf16 rows x [n_rows, dim] or [n_rows, heads, dim]: row i at
    position pos[i] (int64, device) or pos0 + i.  out=x turns in place; by
    default a new tensor receives the result."""
    x = x.contiguous()
    heads, dim = (1, x.shape[1]) if x.dim() == 2 else (x.shape[1], x.shape[2])
    y = torch.empty_like(x) if out is None else out
    _check(lib().hsa_rope(_ptr(x), _ptr(y), x.shape[0], heads, dim, _ptr(pos), pos0, float(theta),
                          _stream()), "rope")
    return y


def kv_compress(x: Tokens, out: PagedCache, req: int, first_block: int, n_blocks: int, m: int,
                alpha: torch.Tensor, x_req: int = 0) -> None:
    """Pool blocks [first_block, first_block + n_blocks) of request x_req of x into
    request req of out."""
    xt, pc = x.c(), out.c()
    _check(lib().hsa_kv_compress(C.byref(xt), x_req, C.byref(pc), req, first_block, n_blocks, m,
                                 _ptr(alpha), _stream()), "kv_compress")


def indexer_topk(q: Queries, qI: torch.Tensor, w: torch.Tensor, kIc: PagedCache, m: int,
                 n_win: int, k: int, with_score: bool = False, ws_key="indexer",
                 bf16_scores: bool = False):
    """hsa_indexer_topk, or hsa_indexer_topk_bf16_scores (bf16_scores=True)."""
    qc, kc = q.c(), kIc.c()
    idx = torch.empty((q.n, k), dtype=torch.int32, device=qI.device)
    score = torch.empty((q.n, k), dtype=torch.float32, device=qI.device) if with_score else None
    nb = lib().hsa_indexer_topk_workspace_bytes(C.byref(qc), m, n_win, k)
    ws, wsb = _ws_args(_WS.get(ws_key, nb, qI.device))
    fn = lib().hsa_indexer_topk_bf16_scores if bf16_scores else lib().hsa_indexer_topk
    _check(fn(C.byref(qc), _ptr(qI), _ptr(w), qI.shape[-2], qI.shape[-1], C.byref(kc), m, n_win,
              k, _ptr(idx), _ptr(score), ws, wsb, _stream()), "indexer_topk")
    return idx, score


def csa_attn(q: Queries, Q: torch.Tensor, win_k: Tokens, win_v: Tokens, n_win: int,
             kc: PagedCache, vc: PagedCache, m: int, idx: torch.Tensor, k: int,
             scale: Optional[float] = None, with_lse: bool = False, out_fp32: bool = False,
             ws_key="csa"):
    H, d = Q.shape[-2], Q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qc, wk, wv, kcc, vcc = q.c(), win_k.c(), win_v.c(), kc.c(), vc.c()
    O = torch.empty(Q.shape, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=Q.device)
    lse = torch.empty((q.n, H), dtype=torch.float32, device=Q.device) if with_lse else None
    nb = lib().hsa_csa_attn_workspace_bytes(C.byref(qc), H, n_win, k)
    ws, wsb = _ws_args(_WS.get(ws_key, nb, Q.device))
    _check(lib().hsa_csa_attn(C.byref(qc), _ptr(Q), H, d, C.byref(wk), C.byref(wv), n_win,
                              C.byref(kcc), C.byref(vcc), m, _ptr(idx), k, scale, _ptr(O),
                              FP32 if out_fp32 else BF16, _ptr(lse), ws, wsb, _stream()), "csa_attn")
    return O, lse


def csa_prefill(q: Queries, qI: torch.Tensor, w: torch.Tensor, kIc: PagedCache, Q: torch.Tensor,
                win_k: Tokens, win_v: Tokens, n_win: int, kc: PagedCache, vc: PagedCache, m: int,
                k: int, scale: Optional[float] = None, with_lse: bool = False,
                out_fp32: bool = False, stage_q: int = 0, ws_key="csa_prefill"):
    """hsa_csa_prefill: a CSA layer's indexer, top-k and attention over a span.
    Returns (idx, O, lse)."""
    H, d = Q.shape[-2], Q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qc, kic, wk, wv, kcc, vcc = q.c(), kIc.c(), win_k.c(), win_v.c(), kc.c(), vc.c()
    idx = torch.empty((q.n, k), dtype=torch.int32, device=Q.device)
    O = torch.empty(Q.shape, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=Q.device)
    lse = torch.empty((q.n, H), dtype=torch.float32, device=Q.device) if with_lse else None
    nb = lib().hsa_csa_prefill_workspace_bytes(C.byref(qc), H, m, n_win, k)
    ws, wsb = _ws_args(_WS.get(ws_key, nb, Q.device))
    _check(lib().hsa_csa_prefill(C.byref(qc), _ptr(qI), _ptr(w), qI.shape[-2], qI.shape[-1],
                                 C.byref(kic), _ptr(Q), H, d, C.byref(wk), C.byref(wv), n_win,
                                 C.byref(kcc), C.byref(vcc), m, k, scale, _ptr(idx), _ptr(O),
                                 FP32 if out_fp32 else BF16, _ptr(lse), stage_q, ws, wsb,
                                 _stream()), "csa_prefill")
    return idx, O, lse


def hca_attn(q: Queries, Q: torch.Tensor, win_k: Tokens, win_v: Tokens, n_win: int,
             kc: PagedCache, vc: PagedCache, m: int, scale: Optional[float] = None,
             with_lse: bool = False, out_fp32: bool = False, ws_key="hca"):
    H, d = Q.shape[-2], Q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    qc, wk, wv, kcc, vcc = q.c(), win_k.c(), win_v.c(), kc.c(), vc.c()
    O = torch.empty(Q.shape, dtype=torch.float32 if out_fp32 else torch.bfloat16, device=Q.device)
    lse = torch.empty((q.n, H), dtype=torch.float32, device=Q.device) if with_lse else None
    nb = lib().hsa_hca_attn_workspace_bytes(C.byref(qc), H, n_win, m)
    ws, wsb = _ws_args(_WS.get(ws_key, nb, Q.device))
    _check(lib().hsa_hca_attn(C.byref(qc), _ptr(Q), H, d, C.byref(wk), C.byref(wv), n_win,
                              C.byref(kcc), C.byref(vcc), m, scale, _ptr(O),
                              FP32 if out_fp32 else BF16, _ptr(lse), ws, wsb, _stream()), "hca_attn")
    return O, lse


@dataclass
class Layer:
    """One layer's decode state: pooling weights, window rings, caches."""
    kind: int
    H: int
    n_win: int
    m: int
    alpha_k: torch.Tensor
    alpha_v: torch.Tensor
    ring_k: Tokens
    ring_v: Tokens
    kc: PagedCache
    vc: PagedCache
    topk: int = 0
    alpha_i: Optional[torch.Tensor] = None
    tail_i: Optional[Tokens] = None
    kic: Optional[PagedCache] = None
    d: int = 128
    H_I: int = 4
    d_I: int = 64
    scale: Optional[float] = None
    out_fp32: bool = False
    rope_theta: float = 0.0           # > 0: the step turns its keys and queries (partial RoPE)

    def c(self) -> _Layer:
        L = _Layer()
        L.kind, L.H, L.d, L.n_win, L.m, L.topk = self.kind, self.H, self.d, self.n_win, self.m, self.topk
        L.H_I, L.d_I = self.H_I, self.d_I
        L.scale = 1.0 / math.sqrt(self.d) if self.scale is None else self.scale
        L.o_dtype = FP32 if self.out_fp32 else BF16
        L.alpha_k, L.alpha_v = self.alpha_k.data_ptr(), self.alpha_v.data_ptr()
        L.alpha_i = self.alpha_i.data_ptr() if self.alpha_i is not None else None
        L.ring_k, L.ring_v = self.ring_k.c(), self.ring_v.c()
        L.kc, L.vc = self.kc.c(), self.vc.c()
        if self.kind == LAYER_CSA:
            L.tail_i, L.kic = self.tail_i.c(), self.kic.c()
        L.rope_theta = self.rope_theta
        return L


def decode_draft(layer: Layer, pos: torch.Tensor, max_pos: int, Q: torch.Tensor,
                 k_new: torch.Tensor, v_new: torch.Tensor, qI=None, kI_new=None, w=None,
                 with_lse: bool = False, with_idx: bool = False, ws_key="draft"):
    """n_tok tokens per request (arrays [B, n_tok, ...]); returns O [B, n_tok, H, d],
    lse [B, n_tok, H] or None, idx [B, n_tok, topk] or None."""
    B, n_tok = Q.shape[0], Q.shape[1]
    Lc = layer.c()
    O = torch.empty(Q.shape, dtype=torch.float32 if layer.out_fp32 else torch.bfloat16,
                    device=Q.device)
    lse = torch.empty((B, n_tok, layer.H), dtype=torch.float32, device=Q.device) if with_lse else None
    idx = (torch.empty((B, n_tok, layer.topk), dtype=torch.int32, device=Q.device)
           if with_idx and layer.kind == LAYER_CSA else None)
    nb = lib().hsa_decode_draft_workspace_bytes(C.byref(Lc), B, n_tok, max_pos)
    ws, wsb = _ws_args(_WS.get((ws_key, layer.kind), nb, Q.device))
    _check(lib().hsa_decode_draft(C.byref(Lc), B, n_tok, _ptr(pos), max_pos, _ptr(Q), _ptr(k_new),
                                  _ptr(v_new), _ptr(qI), _ptr(kI_new), _ptr(w), _ptr(O),
                                  _ptr(lse), _ptr(idx), ws, wsb, _stream()), "decode_draft")
    return O, lse, idx


def decode_step(layer: Layer, pos: torch.Tensor, max_pos: int, Q: torch.Tensor,
                k_new: torch.Tensor, v_new: torch.Tensor, qI=None, kI_new=None, w=None,
                with_lse: bool = False, with_idx: bool = False, O: Optional[torch.Tensor] = None,
                ws_key="decode"):
    B = pos.shape[0]
    Lc = layer.c()
    if O is None:
        O = torch.empty(Q.shape, dtype=torch.float32 if layer.out_fp32 else torch.bfloat16,
                        device=Q.device)
    lse = torch.empty((B, layer.H), dtype=torch.float32, device=Q.device) if with_lse else None
    idx = (torch.empty((B, layer.topk), dtype=torch.int32, device=Q.device)
           if with_idx and layer.kind == LAYER_CSA else None)
    nb = lib().hsa_decode_step_workspace_bytes(C.byref(Lc), B, max_pos)
    ws, wsb = _ws_args(_WS.get((ws_key, layer.kind), nb, Q.device))
    _check(lib().hsa_decode_step(C.byref(Lc), B, _ptr(pos), max_pos, _ptr(Q), _ptr(k_new),
                                 _ptr(v_new), _ptr(qI), _ptr(kI_new), _ptr(w), _ptr(O),
                                 _ptr(lse), _ptr(idx), ws, wsb, _stream()), "decode_step")
    return O, lse, idx


def decode_rewind(layer: Layer, keep: torch.Tensor) -> None:
    """hsa_decode_rewind: request b keeps tokens 0 .. keep[b]-1 (int64 [B], device)."""
    Lc = layer.c()
    _check(lib().hsa_decode_rewind(C.byref(Lc), keep.shape[0], _ptr(keep), _stream()),
           "decode_rewind")


def decode_step_noalloc(layer: Layer, pos: torch.Tensor, max_pos: int, Q: torch.Tensor,
                        k_new: torch.Tensor, v_new: torch.Tensor, qI=None, kI_new=None, w=None,
                        O: torch.Tensor = None, lse: Optional[torch.Tensor] = None,
                        idx: Optional[torch.Tensor] = None):
    """hsa_decode_step_noalloc: the caller passes every output buffer (O
    [B, H, d], lse [B, H] or None, idx [B, topk] or None); the library's own
    device scratch serves as the workspace."""
    B = pos.shape[0]
    Lc = layer.c()
    _check(lib().hsa_decode_step_noalloc(C.byref(Lc), B, _ptr(pos), max_pos, _ptr(Q), _ptr(k_new),
                                         _ptr(v_new), _ptr(qI), _ptr(kI_new), _ptr(w), _ptr(O),
                                         _ptr(lse), _ptr(idx), _stream()), "decode_step_noalloc")
