"""GPU: the sampling-loop driver and HIP-graph capture of the forward, through the C ABI.

- A forward captured into a graph is replayed several times.  New inputs are written into
  its buffers before each replay, with eager forwards and synchronisations in between.
  Every replay must equal the eager forward on the same inputs, bit for bit (the kernels
  are deterministic).
- The dense fallback (the plan's dense mode) must match the fp64 oracle's dense
  attention (keep 100%, no gate), and so must a direct dense-mode forward, also at full size
  on sampled query tiles.
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
    d = drv.dense_plan.desc
    assert d.n_dense_rows == d.n_tiles and d.n_sparse_rows == 0
    _check_dense(w, x, o)


def _check_dense(w, x, o):
    """GPU output against the oracle's keep-100% forward with no gate (dense attention)."""
    from oracle import vsa_oracle as O
    ref, _ = O.forward(dict(x, g=None), w.segments(), w.grid, 100.0, w.sink)
    got = PAR.bits_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
    diff = got - ref
    max_abs = float(np.abs(diff).max())
    rel = float(np.sqrt((diff ** 2).sum() / (ref ** 2).sum()))
    print(f"[dense] {w.name}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= PAR.TOL_ABS and rel <= PAR.TOL_REL


@pytest.mark.parametrize("name", ["tiny", "ragged"])
def test_dense_mode_matches_oracle(name):
    """A dense-mode plan runs every query tile over every key tile with no coarse term,
    whatever the gate: ragged prefix tiles, two batch items, video span first."""
    import block_sparse_video_geometry_amd as V
    from workloads.synth import Workload, SEG_TEXT, SEG_REF_IMAGE, SINK_EXACT_KV_AND_ROWS
    w = WORKLOADS["tiny"] if name == "tiny" else Workload(
        "dense_ragged", 3, ((SEG_TEXT, 100), (SEG_REF_IMAGE, 30)), (8, 12, 16), 10.0,
        SINK_EXACT_KV_AND_ROWS, seed=101, recipe="scaled", batch=2, video_first=True)
    print(f"[gpu] dense mode on {w.name}", flush=True)
    x = make_inputs(w)
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128, 100.0,
                               select=V.VSA_SELECT_DENSE)
    q, k, v, g = (_dev(x[n]) for n in "qkvg")
    o = torch.empty_like(q)
    ws = V.alloc_workspace(plan)
    V.vsa_forward(plan, q, k, v, g, o, ws)
    st = V.vsa_read_stats(plan, ws)
    d = plan.desc
    assert st["executed_pairs"] == st["dense_pairs"] == w.batch * w.heads * d.n_tiles ** 2
    assert st["sparse_rows"] == 0
    _check_dense(w, x, o)


def test_dense_mode_full_size_sampled():
    """The dense call at full size, in the launch configuration bench.py times (four query
    tiles of a head per workgroup sharing each K/V tile): sampled query tiles of two heads,
    prefix and video, against the oracle's dense attention over all 36,096 tokens."""
    import zlib
    import block_sparse_video_geometry_amd as V
    from oracle import vsa_oracle as O
    w = WORKLOADS["full"]
    print(f"[gpu] dense mode on {w.name} (sampled rows)", flush=True)
    x = make_inputs(w)
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128, 100.0,
                               select=V.VSA_SELECT_DENSE)
    q, k, v, g = (_dev(x[n]) for n in "qkvg")
    o = torch.empty_like(q)
    ws = V.alloc_workspace(plan)
    V.vsa_forward(plan, q, k, v, g, o, ws)
    torch.cuda.synchronize()
    got_all = o.view(torch.int16).cpu().numpy().view(np.uint16)
    del q, k, v, g, o, ws
    geom = O.map_geometry(w.segments(), *w.grid)
    rng = np.random.default_rng(zlib.crc32(b"dense_full_sampled"))
    heads = [0, int(rng.integers(1, w.heads))]
    rows = sorted(set([0, geom.n_prefix - 1, geom.n_prefix, geom.n_tiles - 1] +
                      [int(r) for r in rng.integers(0, geom.n_tiles, size=4)]))
    max_abs, err2, ref2 = 0.0, 0.0, 0.0
    for h in heads:
        Q, K, Vh = (PAR.bits_to_f64(x[n][0, :, h]) for n in "qkv")
        # keep 100% without a gate: every row attends to every valid token, no coarse term
        ref, _ = O.forward_head(Q, K, Vh, None, geom, 100.0, w.sink, O.SELECT_TOPK, O.COARSE_MEAN, 0.0,
                                rows=rows)
        got = PAR.bits_to_f64(got_all[0, :, h])
        for r in rows:
            toks = np.asarray(geom.tiles[r])
            d = got[toks] - ref[toks]
            max_abs = max(max_abs, float(np.abs(d).max()))
            err2 += float((d ** 2).sum())
            ref2 += float((ref[toks] ** 2).sum())
    rel = float(np.sqrt(err2 / ref2))
    print(f"[dense-full] heads={heads} rows={rows}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= PAR.TOL_ABS and rel <= PAR.TOL_REL


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
