"""A decode step recorded as a HIP graph (runner.Workload.capture) replays
the same launches: every replay must reproduce the eager step's outputs and
index cache byte for byte, with other eager work (another layer pattern
through the same workspace, fills of the outputs) and synchronisations
between the replays."""
import dataclasses

import pytest
import torch

from helpers import log
from long_context_sparse_idx_amd import inputs
from long_context_sparse_idx_amd.runner import Workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,B", [("decode131k", 32), ("decode1m", 8)])
def test_graph_replays_equal_eager_step(name, B):
    wl = dataclasses.replace(inputs.WORKLOADS[name], B=B, q_pos0=40000, T_kv=40001)
    log(f"[graph] {name} B={B} T_kv={wl.T_kv}: capture, 3 replays against the eager step")
    L = wl.n_layers
    path = Workload(wl, f_layers=range(L))
    allf = path.plan(tuple(1 for _ in range(L)))
    plan = path.plan(wl.pattern)
    path.step(plan)
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in path.outs]
    ref_cache = path.cache.clone()
    g = path.capture(plan)
    for r in range(3):
        path.step(allf)  # other eager work through the same workspace and outputs
        torch.cuda.synchronize()
        for o in path.outs:
            o.fill_(float("nan"))
        path.cache.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(path.outs[l].view(torch.int16), ref_out[l].view(torch.int16)), (r, l)
        assert torch.equal(path.cache, ref_cache), r
    log("  3 replays byte-identical to the eager step")
