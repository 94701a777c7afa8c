"""GPU: the no-allocation forward (vsa_forward_noalloc, the library's static device
scratch as workspace) against vsa_forward with a caller workspace, through the C ABI.

Two calls in a row, the second on a smaller input, so the second runs over scratch the
first left behind; each output must equal vsa_forward's bit for bit (same kernels, same
order of arithmetic) and match the fp64 oracle.  A plan whose workspace exceeds the
scratch is rejected before anything runs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import parity as PAR
from workloads.synth import WORKLOADS, Workload, make_inputs, scaled_down

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run_both(V, w):
    print(f"[gpu] noalloc vs workspace forward on {w.name}", flush=True)
    x = make_inputs(w)
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128, w.keep if w.keep > 0 else 100.0,
                               sink=w.sink, select=w.select, coarse=w.coarse, tau=w.tau, extra_tokens=w.extra)
    assert plan.workspace_bytes <= V.VSA_NOALLOC_SCRATCH_BYTES
    q, k, v, g = (_dev(x[n]) for n in "qkvg")
    o_static = torch.empty_like(q)
    V.vsa_forward_noalloc(plan, q, k, v, g, o_static)
    torch.cuda.synchronize()
    o_ws = torch.empty_like(q)
    ws = V.alloc_workspace(plan)
    V.vsa_forward(plan, q, k, v, g, o_ws, ws)
    torch.cuda.synchronize()
    assert torch.equal(o_static.view(torch.int16), o_ws.view(torch.int16)), f"{w.name}: outputs differ"
    return plan, ws, x, o_static


def test_noalloc_matches_workspace_forward():
    import block_sparse_video_geometry_amd as V
    # first a larger input (tau mode, log-mass, three heads), then a smaller one
    big = scaled_down(WORKLOADS["full_tau_1.5"], heads=3, grid=(8, 24, 44), name="noalloc_big")
    small = WORKLOADS["tiny"]
    for w in (big, small):
        plan, ws, x, o = _run_both(V, w)
        # the caller-workspace run's intermediates and the static run's output against the oracle
        gpu = PAR.gpu_results_to_numpy(plan, ws, o)
        rep = PAR.check_parity(w, x, gpu)
        print(f"[noalloc] {w.name}: rows={rep['rows']} max_abs={rep['max_abs']:.3e} rel_l2={rep['rel_l2']:.3e}",
              flush=True)


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    import block_sparse_video_geometry_amd as V
    w = WORKLOADS["full_extra64"]
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128, w.keep,
                               sink=w.sink, extra_tokens=w.extra)
    assert plan.workspace_bytes > V.VSA_NOALLOC_SCRATCH_BYTES
    t = torch.empty((w.batch, w.n_tokens, w.heads, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(t)
    with pytest.raises(V.VsaError) as e:
        V.vsa_forward_noalloc(plan, t, t, t, None, o)
    assert e.value.status == V.VSA_ERR_WORKSPACE
    assert "static scratch" in str(e.value)
