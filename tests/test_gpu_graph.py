"""The decode step's calls captured in a HIP graph and replayed (MI355X only).

The full-size layer pair (batch 4 at a 1M context, the benchmark's inputs)
runs once eagerly; its outputs and the caches it writes are kept.  The same
calls are then captured in one graph and replayed three times, with the
call outputs overwritten by eager work before each replay (the caches keep
their prefix: each step rewrites only its new entries, with the same values)
and a synchronisation after it.  Every call is deterministic (fixed split order, exact top-k), so
every replay must reproduce the eager results bit for bit.
"""
import os
import sys

import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from long_context_attention_23_amd import api  # noqa: E402

pytestmark = pytest.mark.gpu

OUTS = ["top", "o_csa", "y_csa", "o_hca", "y_hca"]
CACHES = ["win_csa", "csa_c", "keys", "win_hca", "hca_c"]


def _tensors(s, name):
    v = s[name]
    if isinstance(v, api.KVCache):
        return [v.rec]
    if isinstance(v, api.IdxCache):
        return [v.codes] + ([v.scales] if v.scales is not None else [])
    return [v]


def test_decode_step_graph_replays_match_eager():
    print("graph capture of the decode step (batch 4, 1M context)", flush=True)
    sets, sh = bench.build_state(torch, api, 1)
    s = sets[0]
    fns = bench.call_fns(api)
    for f in fns:
        f(s, sh)
    torch.cuda.synchronize()
    ref = {n: [t.clone() for t in _tensors(s, n)] for n in OUTS + CACHES}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in fns:
            f(s, sh)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f(s, sh)
    for rep in range(3):
        for n in OUTS:                                 # eager work between replays
            for t in _tensors(s, n):
                t.fill_(0x55 if t.dtype == torch.uint8 else 7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n in OUTS + CACHES:
            for a, b in zip(_tensors(s, n), ref[n]):
                assert torch.equal(a, b), f"replay {rep}: {n} differs from the eager result"
