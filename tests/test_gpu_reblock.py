"""GPU: Spark-Reblock adaptive video tiles (options.reblock = 1) against the fp64 oracle,
through the C ABI.

The mapper's tiles are checked node by node from the root of the oracle's tree: exact
wherever the oracle's split has a projection gap above 1e-4 at its cut, elsewhere a valid
split within 1e-4 that the oracle adopts.  The forward's intermediates and outputs are
then compared with the oracle run on those tiles, under the usual tolerances.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import parity as PAR
from oracle import vsa_oracle as O
from workloads.synth import (WORKLOADS, Workload, make_inputs, scaled_down, SEG_TEXT, SEG_REF_IMAGE,
                             SEG_REF_AUDIO, SINK_OFF, SINK_EXACT_KV, SINK_EXACT_KV_AND_ROWS, SELECT_TAU,
                             COARSE_MEAN_LOGMASS, COARSE_WEIGHTED_LOGMASS)

pytestmark = pytest.mark.gpu


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run(w, x):
    import block_sparse_video_geometry_amd as V
    print(f"[gpu] {w.name} heads={w.heads} grid={w.grid} keep={w.keep} sink={w.sink} select={w.select} "
          f"coarse={w.coarse} batch={w.batch} reblock={w.reblock}", flush=True)
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128, w.keep if w.keep > 0 else 100.0,
                               sink=w.sink, select=w.select, coarse=w.coarse, tau=w.tau, reblock=w.reblock)
    q, k, v = _dev(x["q"]), _dev(x["k"]), _dev(x["v"])
    g = _dev(x["g"]) if x.get("g") is not None else None
    o = torch.empty_like(q)
    ws = V.alloc_workspace(plan)
    V.vsa_forward(plan, q, k, v, g, o, ws)
    torch.cuda.synchronize()
    tiles = V.debug_tensor(plan, ws, "tiles").cpu().numpy()
    return plan, ws, o, tiles


RB_CASES = [
    # smooth queries (clustered by cube), 32 video tiles
    Workload("rb_smooth", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 40)), (8, 16, 16), 25.0, SINK_EXACT_KV,
             seed=111, recipe="smooth", reblock=1),
    # the full recipe on 132 video tiles (groups of odd size), dense prefix rows
    scaled_down(WORKLOADS["full_reblock"], heads=3, grid=(8, 24, 44), name="rb_full_small"),
    Workload("rb_tau_logmass", 2, ((SEG_TEXT, 64),), (8, 16, 20), 0.0, SINK_EXACT_KV, SELECT_TAU,
             COARSE_MEAN_LOGMASS, 1.0, seed=112, recipe="offset", reblock=1),
    Workload("rb_sink_off_video_first", 2, ((SEG_TEXT, 100), (SEG_REF_IMAGE, 30)), (8, 12, 16), 20.0, SINK_OFF,
             seed=113, recipe="scaled", video_first=True, reblock=1),
    Workload("rb_weighted_batch2", 2, ((SEG_TEXT, 64),), (4, 8, 16), 25.0, SINK_EXACT_KV_AND_ROWS,
             coarse=COARSE_WEIGHTED_LOGMASS, seed=114, recipe="offset", batch=2, reblock=1),
    Workload("rb_one_tile", 1, ((SEG_TEXT, 10),), (4, 4, 4), 100.0, SINK_EXACT_KV, seed=115, reblock=1),
    Workload("rb_three_tiles", 2, ((SEG_TEXT, 64),), (4, 4, 12), 50.0, SINK_EXACT_KV, seed=116,
             recipe="scaled", reblock=1),
]


@pytest.mark.parametrize("w", RB_CASES, ids=[w.name for w in RB_CASES])
def test_reblock_small(w):
    x = make_inputs(w)
    plan, ws, o, tiles = _run(w, x)
    heads = [(b, h) for b in range(w.batch) for h in range(w.heads)]
    geoms, trep = PAR.check_reblock_tiles(w, x, tiles, heads)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    rep = PAR.check_parity(w, x, gpu, geoms=geoms)
    print(f"[reblock] {w.name}: nodes={trep['nodes']} exact={trep['exact_nodes']} adopted={trep['adopted_nodes']} "
          f"min_gap={trep['min_gap']:.2e} rows={rep['rows']} max_abs={rep['max_abs']:.3e} "
          f"rel_l2={rep['rel_l2']:.3e}", flush=True)


def test_reblock_ties():
    """Every video query of head 0 the same: all projections of every node tie, so each
    split keeps the lower token ids on the left and tile j is the video tokens
    64 j .. 64 j + 63 in packed order, exactly (no adoption)."""
    w = Workload("rb_ties", 2, ((SEG_TEXT, 64),), (8, 8, 12), 25.0, SINK_EXACT_KV, seed=117, recipe="scaled",
                 reblock=1)
    x = make_inputs(w)
    geom = O.map_geometry(w.segments(), *w.grid)
    vstart = geom.video_start
    q = x["q"].copy()
    q[0, vstart:vstart + w.n_video, 0] = q[0, vstart, 0]
    x = dict(x, q=q)
    plan, ws, o, tiles = _run(w, x)
    vids = vstart + np.arange(w.n_video)
    assert np.array_equal(tiles[0, 0], vids.reshape(-1, 64)), "tied projections must keep token order"
    geoms, _ = PAR.check_reblock_tiles(w, x, tiles, [(0, 0), (0, 1)])
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    PAR.check_parity(w, x, gpu, geoms=geoms)


@pytest.mark.parametrize("name", ["full_reblock", "full_smooth_reblock_20"])
def test_reblock_full_size_sampled(name):
    """Full size in the benchmark's launch configuration: every head's tiles partition the
    video tokens; two heads' trees node by node; sampled rows' outputs."""
    import zlib
    w = WORKLOADS[name]
    x = make_inputs(w)
    plan, ws, o, tiles = _run(w, x)
    geom = O.map_geometry(w.segments(), *w.grid)
    vids = geom.video_start + np.arange(w.n_video)
    for h in range(w.heads):
        assert np.array_equal(np.sort(tiles[0, h].ravel()), vids), f"h{h}: tiles do not partition the video"
        assert np.all(np.diff(tiles[0, h], axis=1) > 0), f"h{h}: tokens not ascending inside a tile"
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    heads = [(0, 0), (0, int(rng.integers(1, w.heads)))]
    geoms, trep = PAR.check_reblock_tiles(w, x, tiles, heads)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o, fields=("scores", "lists", "counts", "qbar", "kbar", "vbar",
                                                        "bias", "ocoarse", "thr"))
    P, Tq = geom.n_prefix, geom.n_tiles
    rows = sorted(set([0, P - 1, P, Tq - 1] + [int(r) for r in rng.integers(0, Tq, size=4)]))
    rep = PAR.check_parity(w, x, gpu, heads=heads, rows=rows, geoms=geoms)
    print(f"[reblock-full] {name}: nodes={trep['nodes']} exact={trep['exact_nodes']} "
          f"adopted={trep['adopted_nodes']} rows={rep['rows']} max_abs={rep['max_abs']:.3e}", flush=True)
