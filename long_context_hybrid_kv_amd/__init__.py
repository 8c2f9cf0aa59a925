"""Hybrid long-context attention (SWA + CSA + HCA over one shared KV head) for
AMD MI355X: hand-written gfx950 HIP kernels behind the C ABI in
include/hsa_attn.h, with a thin ctypes binding of the same names."""
from ._lib import (BF16, FP8, LAYER_CSA, LAYER_HCA, HsaError, Layer, PagedCache, Queries,  # noqa: F401
                   Tokens, abi_version, check_device_error, csa_attn, decode_step, hca_attn,
                   indexer_topk, kv_compress, lib, pooling_weights)
