"""hsa_decode_step_noalloc (the decode step for callers that cannot allocate:
its workspace is the library's own device scratch) against hsa_decode_step
with a caller workspace: two identical copies of the caches, two calls in a
row on each -- the second with fewer requests and a shorter context -- and the
outputs, LSEs, selections and caches of both paths equal bit for bit."""
import numpy as np
import pytest
import torch

from synth import configs

import hsa_testlib as T
from long_context_hybrid_kv_amd import _lib as L

pytestmark = pytest.mark.gpu


def _step_args(st, layer, Ls, rows, s):
    reqs = st["reqs"]
    pick = lambda f: np.stack([f(reqs[r], int(Ls[r]) + s) for r in rows])
    a = dict(Q=T.dev_bf16(pick(lambda d, p: d["q"][s])),
             k_new=T.dev_bf16(pick(lambda d, p: d["k"][p])),
             v_new=T.dev_bf16(pick(lambda d, p: d["v"][p])))
    if layer == "csa":
        a.update(qI=T.dev_bf16(pick(lambda d, p: d["qi"][s])),
                 kI_new=T.dev_bf16(pick(lambda d, p: d["ki"][p])),
                 w=torch.from_numpy(pick(lambda d, p: d["w"][s])).cuda())
    return a


@pytest.mark.parametrize("layer", ["csa", "hca"])
def test_noalloc_step_equals_decode_step(layer):
    w = configs.shrink(configs.CSA_DECODE_128K if layer == "csa" else configs.RAGGED_SERVING,
                       H=64, k_csa=512)
    # the second call takes requests 0-2 only: the three shortest contexts
    Ls = [9001, 127, 700, 40000, 131071, 70001]
    st_a = T.build_state(w, layer, Ls, steps=2)
    st_b = T.build_state(w, layer, Ls, steps=2)
    lay_a, lay_b = T.layer_of(w, layer, st_a), T.layer_of(w, layer, st_b)
    for call, rows in enumerate([list(range(len(Ls))), [0, 1, 2]]):
        # the second call: three requests, one step further, a shorter context
        B = len(rows)
        pos = torch.tensor([Ls[r] + call for r in rows], dtype=torch.int64, device="cuda")
        max_pos = int(pos.max())
        print(f"noalloc {layer}: call {call}, B {B}, max_pos {max_pos}", flush=True)
        args = _step_args(st_a, layer, Ls, rows, call)
        Oa, la, ia = L.decode_step(lay_a, pos, max_pos, with_lse=True,
                                   with_idx=(layer == "csa"), **args)
        Ob = torch.empty_like(Oa)
        lb = torch.empty_like(la)
        ib = torch.empty_like(ia) if ia is not None else None
        L.decode_step_noalloc(lay_b, pos, max_pos, O=Ob, lse=lb, idx=ib, **args)
        L.check_device_error()
        assert torch.equal(Oa.view(torch.int32), Ob.view(torch.int32)), f"call {call}: O"
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), f"call {call}: lse"
        if ia is not None:
            assert torch.equal(ia, ib), f"call {call}: idx"
        for name in ["kc", "vc"] + (["kic"] if layer == "csa" else []):
            assert torch.equal(st_a[name].n_entries, st_b[name].n_entries), (call, name)
            assert torch.equal(st_a[name].data.view(torch.uint8), st_b[name].data.view(torch.uint8)), (call, name)
        for name in ["ring_k", "ring_v"] + (["tail_i"] if layer == "csa" else []):
            assert torch.equal(st_a[name].data.view(torch.int16), st_b[name].data.view(torch.int16)), (call, name)
