"""GPU: the sampling-loop driver and HIP-graph capture of the forward, through the C ABI.

- A forward captured into a graph is replayed several times.  New inputs are written into
  its buffers before each replay, with eager forwards and synchronisations in between.
  Every replay must equal the eager forward on the same inputs, bit for bit (the kernels
  are deterministic).
- The dense fallback (keep 100%, no gate) must match the fp64 oracle's dense attention.
"""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import parity as PAR
from workloads.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _driver(w, **kw):
    from block_sparse_video_geometry_amd.driver import LayerDriver, Schedule
    return LayerDriver(w.segments(), w.batch, *w.grid, w.heads, w.keep, sink=w.sink, select=w.select,
                       coarse=w.coarse, tau=w.tau, schedule=Schedule(**kw))


def test_graph_replay_matches_eager():
    import block_sparse_video_geometry_amd as V
    w = WORKLOADS["mid"]
    print(f"[gpu] graph replay on {w.name}", flush=True)
    drv = _driver(w)
    x0 = make_inputs(w)
    q, k, v, g = (_dev(x0[n]) for n in "qkvg")
    o = torch.empty_like(q)
    drv.capture(True, q, k, v, g, o)
    o_eager = torch.empty_like(q)
    for r in range(3):
        x = make_inputs(dataclasses.replace(w, seed=w.seed + 100 + r))
        for dst, n in zip((q, k, v, g), "qkvg"):
            dst.copy_(_dev(x[n]))
        drv.replay(True)
        torch.cuda.synchronize()
        o_graph = o.clone()
        V.vsa_forward(drv.sparse_plan, q, k, v, g, o_eager, drv.workspace)
        torch.cuda.synchronize()
        assert torch.equal(o_graph.view(torch.int16), o_eager.view(torch.int16)), f"replay {r} differs"


def test_driver_dense_fallback_matches_oracle():
    w = WORKLOADS["tiny"]  # 1,152 tokens: under min_tokens, so every call runs dense
    print(f"[gpu] dense fallback on {w.name}", flush=True)
    drv = _driver(w)
    x = make_inputs(w)
    q, k, v, g = (_dev(x[n]) for n in "qkvg")
    o = torch.empty_like(q)
    assert drv.forward(1, 4, 3, q, k, v, g, o) is False
    torch.cuda.synchronize()
    gpu = PAR.gpu_results_to_numpy(drv.dense_plan, drv.workspace, o)
    PAR.check_parity(dataclasses.replace(w, keep=100.0), dict(x, g=None), gpu)


def test_driver_sparse_call_matches_forward():
    import block_sparse_video_geometry_amd as V
    w = WORKLOADS["mid"]  # 17,792 tokens: sparse outside the first layer
    print(f"[gpu] driver sparse call on {w.name}", flush=True)
    drv = _driver(w)
    x = make_inputs(w)
    q, k, v, g = (_dev(x[n]) for n in "qkvg")
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    assert drv.forward(0, 4, 1, q, k, v, g, o1) is True
    ws = V.alloc_workspace(drv.sparse_plan)
    V.vsa_forward(drv.sparse_plan, q, k, v, g, o2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert drv.forward(0, 4, 0, q, k, v, g, o1) is False  # first layer: dense
