"""Oracle: a plain, slow, float64 CPU statement of the hybrid attention.

THIS IS TEST INFRASTRUCTURE.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import or run it.  The GPU library and its
Python binding never import it, and it shares no code with them: the only
common module is `synth`, which draws the seeded inputs and holds none of the
method's arithmetic.

Contents
  numerics  bf16 and fp8 e4m3fn storage, each one rounding from float64
  hybrid    visibility (SWA window, visible compressed blocks), compression
            (softmax-weighted pooling of m-token blocks, bf16 or fp8 + per-page
            scale), lightning-indexer scores, top-k selection, and the single
            softmax over window + compressed entries for CSA and HCA

Sources: the group-reading wiki page "DeepSeek-V4 深度研究剖析" §5.2-§5.4, §8,
§11.4; the zjai.club episode page "163: DeepSeek V4 Explained ..." ("Deep dive"
§14); the aifrontier page "EP 95 解读 DeepSeek-V4 论文" (sections on the three
sparse-attention components and on the Lightning Indexer and top-k).  Every
function docstring states the step it follows and the reading taken.

Pins (each function is checked against something other than itself, in
tests/test_oracle_*.py): bf16/e4m3 against torch's converters and hand-built
halfway cases; pooling weights against closed forms; compression against exact
rational arithmetic; visibility against brute-force enumeration; indexer and
top-k against pure-Python loops and a full sort; attention against
torch.nn.functional.scaled_dot_product_attention (m = 1, window >= T, or any
window with top-k >= visible blocks), CSA == HCA when top-k covers every
visible block, V = 1 => O = 1, head permutation; a hand-derived fixture in
tests/golden/.  No function is left unpinned.
"""
