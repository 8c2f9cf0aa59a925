"""The hybrid long-context attention, written out plainly in float64.

Test infrastructure (see the package docstring): nothing in the product path
imports this module.

Sources (page titles; the pages print no formulas, so each step below states
the plain reading taken where a page leaves it open):

* group-reading wiki, "DeepSeek-V4 深度研究剖析":
  §5.2 SWA keeps the most recent n_win = 128 uncompressed KV;
  §5.3 CSA compresses every m = 4 tokens' KV into one entry, a lightning
       indexer scores the compressed blocks and a per-query top-k of them
       (512 Flash, 1024 Pro) enters the main attention;
  §5.4 HCA compresses every m' = 128 tokens into one entry and attends to all
       of them densely;
  §11.4 the caches: compressed KV, compressed indexer keys, raw SWA KV and the
       tail of a block not yet complete.
* zjai.club episode 163 "Deep dive" §14 and the aifrontier EP95 walkthrough of
  the sparse attention: one shared KV head (MQA); window and compressed entries
  are concatenated and attended together.

Readings taken where the pages are silent:
* compression is a softmax-weighted pooling: entry = sum_j alpha[j, c] * x[j, c]
  over the m tokens of a block, alpha = softmax over the slot axis of seeded
  per-slot, per-channel logits;
* indexer score I[t, b] = sum_h w[t, h] * ReLU(qI[t, h] . KI_c[b]) (no scale);
* top-k per query token, shared by all heads; ties go to the lower block;
* block b is visible to the query at t iff it is complete and starts before the
  window: b < min(ceil(s(t)/m), floor((t+1)/m)), s(t) = max(0, t - n_win + 1);
* the window W(t) = {s(t), ..., t} includes the query token;
* one softmax over window + compressed entries, logits scaled by 1/sqrt(d).
* positional rotation (optional, rope_theta > 0): the last 64 channels of every
  key and query head turn as adjacent pairs (rope_exact); a key is rotated at
  its own position before it enters the window or a block, so a compressed
  entry pools rotated keys and a query's scores depend only on offsets.
"""
from __future__ import annotations

import math

import numpy as np

from . import numerics as nx


# ----------------------------------------------------------------------------- visibility

def window_start(t: int, n_win: int) -> int:
    """First raw token of the SWA window of the query at position t."""
    return max(0, t - n_win + 1)


def n_visible(t: int, m: int, n_win: int) -> int:
    """Number of compressed blocks visible at t: complete, and starting before
    the window (so they cover exactly the tokens the window does not, up to the
    m-1 tokens of the block that straddles the window's start)."""
    s = window_start(t, n_win)
    return min(-(-s // m), (t + 1) // m)


# ----------------------------------------------------------------------------- positional rotation

ROPE_DIM = 64   # rotated channels: the last 64 of a key row or of a query head


def rope_inv_freq(theta: float) -> np.ndarray:
    """Rotation frequency of channel pair i < 32: theta^(-2i/64), held in
    float32 (the usual inverse-frequency table), returned as float64 values.

    The group-reading wiki "DeepSeek-V4 深度研究剖析" §8 keeps the KV cache's
    RoPE channels apart from the others and names no rotation; this is the
    rotary embedding's textbook form (RoFormer) over the last 64 channels."""
    i = np.arange(ROPE_DIM // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / ROPE_DIM).astype(np.float32).astype(np.float64)


def rope_exact(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate the last 64 channels of every row of x (float64 values, last axis
    the channels) in float64, without rounding to a storage format.

    pos holds the position of each row (x's shape without the channel axis,
    or anything broadcasting to it).  Pair i is channels (d-64+2i, d-63+2i);
    at position p it turns by the angle p * f_i (f_i from rope_inv_freq):
        x' = x cos - y sin,   y' = x sin + y cos,
    each product rounded to float64, then the sum (no fused multiply-add).
    The other channels are returned unchanged."""
    x = np.array(x, dtype=np.float64, copy=True)
    d = x.shape[-1]
    assert d >= ROPE_DIM and d % 2 == 0
    r0 = d - ROPE_DIM
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(theta)
    c, s = np.cos(ang), np.sin(ang)
    ev = x[..., r0::2].copy()
    od = x[..., r0 + 1::2].copy()
    x[..., r0::2] = ev * c - od * s
    x[..., r0 + 1::2] = ev * s + od * c
    return x


def rope(x_bits: np.ndarray, pos, theta: float) -> np.ndarray:
    """bf16 rows (bit patterns) rotated at their positions: rope_exact of
    their values, rounded once to bf16.  This is what enters the window ring
    and the compression (a key is rotated at its own position before it is
    cached; a compressed entry pools rotated keys) and what a query attends
    with."""
    return nx.bf16_bits_from_f64(rope_exact(nx.bf16_value(x_bits), pos, theta))


def rotate_tokens(inp: dict, theta: float) -> dict:
    """A layer's raw inputs with K and Q rotated: K row t at position t, the
    query of position t (q[t], all heads) at t.  Other inputs unchanged."""
    out = dict(inp)
    T = inp["k"].shape[0]
    out["k"] = rope(inp["k"], np.arange(T), theta)
    nq = inp["q"].shape[0]
    out["q"] = rope(inp["q"], np.arange(nq)[:, None], theta)
    return out


# ----------------------------------------------------------------------------- compression

def pooling_weights(z: np.ndarray) -> np.ndarray:
    """alpha = softmax over slots (axis 0) of the logits z [m, D], in float64,
    summed in slot order, rounded once to float32."""
    z = np.asarray(z, dtype=np.float32).astype(np.float64)
    e = np.exp(z - z.max(axis=0, keepdims=True))
    s = e[0].copy()
    for j in range(1, e.shape[0]):
        s = s + e[j]
    return (e / s).astype(np.float32)


def compress_exact(x_bits: np.ndarray, alpha: np.ndarray, m: int) -> np.ndarray:
    """Pooled value of every complete block: sum_j alpha[j] * x[b*m + j], float64.

    x_bits: bf16 bits [T, D]; alpha: float32 [m, D].  Returns float64 [T//m, D].
    Each product of a float32 weight and a bf16 value is exact in float64; the
    m products are added in slot order."""
    x = nx.bf16_value(x_bits)
    nb = x.shape[0] // m
    a = np.asarray(alpha, dtype=np.float32).astype(np.float64)
    acc = np.zeros((nb, x.shape[1]), dtype=np.float64)
    for j in range(m):
        acc = acc + a[j][None, :] * x[j: nb * m: m]
    return acc


def store_bf16(c: np.ndarray) -> np.ndarray:
    """Compressed entries as stored in a bf16 cache (bit patterns)."""
    return nx.bf16_bits_from_f64(c)


def store_fp8_pages(c: np.ndarray, page: int = 64):
    """Compressed entries as stored in an fp8 cache: one float32 scale per
    `page` consecutive entries (all channels), scale = amax / 448 rounded to
    float32 (1 if the page is all zero), code = e4m3fn(entry / scale).
    A final partial page takes its scale over the entries present.
    Returns (codes uint8 [n, D], scales float32 [ceil(n/page)])."""
    n = c.shape[0]
    n_pages = -(-n // page)
    codes = np.zeros(c.shape, dtype=np.uint8)
    scales = np.zeros(n_pages, dtype=np.float32)
    for p in range(n_pages):
        blk = c[p * page:(p + 1) * page]
        amax = np.abs(blk).max() if blk.size else 0.0
        sc = np.float32(amax / nx.E4M3_MAX) if amax > 0 else np.float32(1.0)
        scales[p] = sc
        codes[p * page:(p + 1) * page] = nx.e4m3_encode(blk / np.float64(sc))
    return codes, scales


def fp8_values(codes: np.ndarray, scales: np.ndarray, page: int = 64) -> np.ndarray:
    """float64 values of an fp8 cache: code value times its page's scale."""
    v = nx.e4m3_decode(codes)
    s = np.repeat(scales.astype(np.float64), page)[: codes.shape[0]]
    return v * s[:, None]


def store_mixed_pages(c: np.ndarray, page: int = 64):
    """Compressed K entries stored as the wiki's §8 KV entry: RoPE channels in
    bf16, the others in fp8.  Reading (the pages give no widths): the last D/2
    channels are the RoPE channels.  The first D/2 channels are stored as
    store_fp8_pages stores a cache (one float32 scale per page, amax over those
    channels only), the last D/2 as bf16.  Returns (rows uint8 [n, D/2 + D]:
    the codes, then each bf16 channel as its two little-endian bytes; scales
    float32 [ceil(n/page)])."""
    n, d = c.shape
    h = d // 2
    codes, scales = store_fp8_pages(c[:, :h], page)
    rope = np.ascontiguousarray(store_bf16(c[:, h:]))
    return np.concatenate([codes, rope.view(np.uint8).reshape(n, 2 * (d - h))], axis=1), scales


def mixed_values(rows: np.ndarray, scales: np.ndarray, page: int = 64) -> np.ndarray:
    """float64 values of a mixed cache: code value times the page scale for the
    first D/2 channels, the bf16 value for the RoPE channels."""
    h = rows.shape[1] // 3
    lo = fp8_values(rows[:, :h], scales, page)
    hi = nx.bf16_value(np.ascontiguousarray(rows[:, h:]).view(np.uint16))
    return np.concatenate([lo, hi], axis=1)


def store_fp4_mx(c: np.ndarray, block: int = 32):
    """Compressed indexer keys in fp4 (the wiki's §8 names an FP4 indexer and no
    format).  Reading: OCP MX (Microscaling) FP4 -- e2m1 elements in blocks of
    `block` consecutive channels of one key, each block sharing a power-of-two
    scale 2^x stored as the e8m0 byte x + 127, with x = floor(log2(amax of the
    block)) - 2 (2: the largest e2m1 exponent) and element = e2m1(value / 2^x),
    clamped to +-6; a block of zeros stores x = 0.  Returns (codes uint8
    [n, D/2], channel 2j in the low nibble of byte j; scale bytes uint8
    [n, D/block])."""
    n, d = c.shape
    blk = c.reshape(n, d // block, block)
    amax = np.abs(blk).max(axis=2)
    _, E = np.frexp(amax)                   # amax = f * 2^E, f in [0.5, 1)
    x = np.clip(np.where(amax > 0, E - 1 - 2, 0), -127, 127)
    codes = nx.e2m1_encode(blk / np.ldexp(1.0, x)[:, :, None]).reshape(n, d)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, (x + 127).astype(np.uint8)


def fp4_values(packed: np.ndarray, scale_bytes: np.ndarray, block: int = 32) -> np.ndarray:
    """float64 values of fp4 keys: element value times 2^(scale byte - 127)."""
    n = packed.shape[0]
    codes = np.empty((n, 2 * packed.shape[1]), dtype=np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    x = scale_bytes.astype(np.int64) - 127
    d = codes.shape[1]
    return (nx.e2m1_decode(codes).reshape(n, d // block, block) *
            np.ldexp(1.0, x)[:, :, None]).reshape(n, d)


class Cache:
    """One compressed cache as stored: `bits` (bf16 uint16, fp8 uint8, or the
    rows of a mixed cache as uint8), `scales` (fp8 and mixed) and the float64
    `values` the attention reads."""

    def __init__(self, exact: np.ndarray, dtype: str = "bf16", page: int = 64):
        self.dtype = dtype
        if dtype == "bf16":
            self.bits = store_bf16(exact)
            self.scales = None
            self.values = nx.bf16_value(self.bits)
        elif dtype == "fp8":
            self.bits, self.scales = store_fp8_pages(exact, page)
            self.values = fp8_values(self.bits, self.scales, page)
        elif dtype == "fp4":
            self.bits, self.scales = store_fp4_mx(exact)
            self.values = fp4_values(self.bits, self.scales)
        elif dtype == "mixed":
            self.bits, self.scales = store_mixed_pages(exact, page)
            self.values = mixed_values(self.bits, self.scales, page)
        else:
            raise ValueError(dtype)

    def __len__(self):
        return self.values.shape[0]


def compress(x_bits, z, m, dtype="bf16", page=64) -> Cache:
    """Pool the complete blocks of x with weights softmax(z) and store them."""
    return Cache(compress_exact(x_bits, pooling_weights(z), m), dtype, page)


# ----------------------------------------------------------------------------- indexer and top-k

def indexer_scores(qi_bits: np.ndarray, w: np.ndarray, kic_values: np.ndarray) -> np.ndarray:
    """I[b] = sum_h w[h] * max(0, qI[h] . KI_c[b]) for every row b of kic_values.
    qi_bits: bf16 [H_I, d_I]; w: float32 [H_I]; kic_values: float64 [n, d_I]."""
    qi = nx.bf16_value(qi_bits)
    dots = kic_values @ qi.T                        # [n, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float32).astype(np.float64)


def indexer_scores_fp4(qi_bits: np.ndarray, w: np.ndarray, kic_values: np.ndarray) -> np.ndarray:
    """The index scores computed in FP4 (the wiki's §8: the lightning
    indexer's attention computation runs in FP4), over fp4 keys.  Reading:
    both operands in the format the keys are stored in (store_fp4_mx) -- each
    query head's d_I channels quantized in 32-channel blocks, each block with
    its own power-of-two scale by the same rule -- so that every product of a
    query value and a key value is exact; then I[b] = sum_h w[h] *
    max(0, q4[h] . KI_c[b]) in float64 as indexer_scores.
    qi_bits: bf16 [H_I, d_I]; w: float32 [H_I]; kic_values: the fp4 keys'
    float64 values [n, d_I]."""
    qi = nx.bf16_value(qi_bits)
    packed, sb = store_fp4_mx(qi.reshape(-1, qi.shape[-1]))
    q4 = fp4_values(packed, sb).reshape(qi.shape)
    dots = kic_values @ q4.T                        # [n, H_I]
    return np.maximum(dots, 0.0) @ np.asarray(w, dtype=np.float32).astype(np.float64)


def indexer_scores_bf16(qi_bits: np.ndarray, w: np.ndarray, kic_values: np.ndarray) -> np.ndarray:
    """The index scores as a bf16 selector ranks them (wiki §8: the scores are
    cast from fp32 to bf16 before the top-k): every score rounded once, after
    the weighted head sum, to the nearest bf16 value (ties to even), as
    float64.  The selection over them is topk_blocks (ties: lower block)."""
    return nx.bf16_round_value(indexer_scores(qi_bits, w, kic_values))


def topk_blocks(scores: np.ndarray, k: int) -> np.ndarray:
    """The min(k, n) blocks with the largest score (ties: lower block first),
    listed in ascending block order and padded with -1 to length k."""
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))     # by score desc, then index asc
    sel = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


# ----------------------------------------------------------------------------- attention

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """One softmax over all entries, per head.  q [H, d]; K, V [E, d] (float64).
    Returns (O [H, d], lse [H]) with lse the natural log of the softmax
    denominator of the scaled logits."""
    logits = (q @ K.T) * scale                      # [H, E]
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    s = p.sum(axis=1, keepdims=True)
    P = p / s
    assert np.all(np.abs(P.sum(axis=1) - 1.0) < 1e-12), "softmax rows must sum to 1"
    return P @ V, (mx + np.log(s))[:, 0]


def _window_rows(t, n_win, k_bits, v_bits):
    s = window_start(t, n_win)
    return nx.bf16_value(k_bits[s: t + 1]), nx.bf16_value(v_bits[s: t + 1])


def csa_query(t, q_bits, qi_bits, w, k_bits, v_bits, kc: Cache, vc: Cache, kic: Cache,
              m, n_win, topk, scale=None):
    """CSA + SWA for the query at position t.

    k_bits/v_bits: raw bf16 tokens of the request (at least 0..t);
    kc/vc/kic: compressed caches (at least the visible blocks).
    Returns dict(o, lse, idx, scores) where idx are the selected blocks
    (ascending, -1 padded) and scores the indexer scores of all visible blocks
    (float64).  Over fp4 indexer keys the scores are computed in FP4
    (indexer_scores_fp4)."""
    d = q_bits.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nv = n_visible(t, m, n_win)
    score = indexer_scores_fp4 if kic.dtype == "fp4" else indexer_scores
    sc = score(qi_bits, w, kic.values[:nv])
    idx = topk_blocks(sc, topk)
    sel = idx[idx >= 0]
    Kw, Vw = _window_rows(t, n_win, k_bits, v_bits)
    K = np.concatenate([Kw, kc.values[sel]])
    V = np.concatenate([Vw, vc.values[sel]])
    o, lse = attend(nx.bf16_value(q_bits), K, V, scale)
    return {"o": o, "lse": lse, "idx": idx, "scores": sc}


def hca_query(t, q_bits, k_bits, v_bits, kc: Cache, vc: Cache, m, n_win, scale=None):
    """HCA + SWA for the query at position t: window plus every visible block."""
    d = q_bits.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    nv = n_visible(t, m, n_win)
    Kw, Vw = _window_rows(t, n_win, k_bits, v_bits)
    K = np.concatenate([Kw, kc.values[:nv]])
    V = np.concatenate([Vw, vc.values[:nv]])
    o, lse = attend(nx.bf16_value(q_bits), K, V, scale)
    return {"o": o, "lse": lse}


# ----------------------------------------------------------------------------- layers

def layer_caches(inp: dict, layer: str, m: int, dtype: str = "bf16", page: int = 64) -> dict:
    """Compressed caches of one layer from its raw tokens (every complete block).
    dtype "mixed": the K cache holds mixed entries, the V cache fp8."""
    vdtype = "fp8" if dtype == "mixed" else dtype
    out = {"kc": compress(inp["k"], inp["zk"], m, dtype, page),
           "vc": compress(inp["v"], inp["zv"], m, vdtype, page)}
    if layer == "csa":
        out["kic"] = compress(inp["ki"], inp["zi"], m, "bf16", page)
    return out


def prefill_rows(inp: dict, layer: str, rows, m: int, n_win: int, topk: int = 0,
                 caches: dict | None = None, dtype: str = "bf16"):
    """Outputs of a prefill layer at the query positions `rows`."""
    caches = layer_caches(inp, layer, m, dtype) if caches is None else caches
    res = []
    for t in rows:
        if layer == "csa":
            res.append(csa_query(t, inp["q"][t], inp["qi"][t], inp["w"][t], inp["k"], inp["v"],
                                 caches["kc"], caches["vc"], caches["kic"], m, n_win, topk))
        else:
            res.append(hca_query(t, inp["q"][t], inp["k"], inp["v"],
                                 caches["kc"], caches["vc"], m, n_win))
    return res
