"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every output element; the full-size workloads run in the
launch configuration the benchmark times and are compared on sampled
(batch, head, query tile) rows plus properties that hold at any size.
"""
import functools
import zlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import parity as PAR
from oracle import vsa_oracle as O
from workloads.synth import (WORKLOADS, Workload, make_inputs, scaled_down, SEG_TEXT,
                             SEG_REF_IMAGE, SEG_REF_AUDIO, SINK_OFF, SINK_EXACT_KV, SINK_EXACT_KV_AND_ROWS,
                             SELECT_TOPK, SELECT_TAU, COARSE_MEAN, COARSE_MEAN_LOGMASS,
                             COARSE_WEIGHTED_LOGMASS)

pytestmark = pytest.mark.gpu


def _lib():
    import block_sparse_video_geometry_amd as V
    return V


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def run_gpu(w, x, use_gate=True):
    V = _lib()
    print(f"[gpu] {w.name} heads={w.heads} grid={w.grid} keep={w.keep} sink={w.sink} "
          f"select={w.select} coarse={w.coarse} tau={w.tau} extra={w.extra}", flush=True)
    plan = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128, w.keep if w.keep > 0 else 100.0,
                               sink=w.sink, select=w.select, coarse=w.coarse, tau=w.tau,
                               extra_tokens=w.extra)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    g = to_dev(x["g"]) if (use_gate and x.get("g") is not None) else None
    o = torch.empty_like(q)
    ws = V.alloc_workspace(plan)
    V.vsa_forward(plan, q, k, v, g, o, ws)
    torch.cuda.synchronize()
    return plan, ws, o, (q, k, v, g)


FULL_SMALL_GRID = (8, 24, 44)
SMALL_CASES = [
    WORKLOADS["tiny"],
    WORKLOADS["mid"],
    scaled_down(WORKLOADS["full"], heads=3, grid=FULL_SMALL_GRID, name="full_small"),
    scaled_down(WORKLOADS["full_smooth_20"], heads=2, grid=FULL_SMALL_GRID, name="smooth20_small"),
    scaled_down(WORKLOADS["full_smooth_100"], heads=2, grid=FULL_SMALL_GRID, name="smooth100_small"),
    scaled_down(WORKLOADS["full_tau_1.0"], heads=2, grid=FULL_SMALL_GRID, name="tau1_small"),
    scaled_down(WORKLOADS["full_tau_1.5"], heads=2, grid=FULL_SMALL_GRID, name="tau15_small"),
    scaled_down(WORKLOADS["full_tau_2.0"], heads=2, grid=FULL_SMALL_GRID, name="tau2_small"),
    scaled_down(WORKLOADS["full_logmass"], heads=2, grid=FULL_SMALL_GRID, name="logmass_small"),
    scaled_down(WORKLOADS["full_weighted"], heads=2, grid=FULL_SMALL_GRID, name="weighted_small"),
    Workload("weighted_tau", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 40)), (8, 16, 16), 0.0,
             SINK_EXACT_KV, SELECT_TAU, COARSE_WEIGHTED_LOGMASS, 1.0, seed=84, recipe="offset"),
    # ragged prefix tiles, video span first, exact_kv rows, odd head count
    Workload("ragged_video_first", 3, ((SEG_TEXT, 100), (SEG_REF_IMAGE, 64), (SEG_REF_AUDIO, 30)),
             (8, 12, 16), 20.0, SINK_EXACT_KV, seed=71, recipe="scaled", video_first=True),
    Workload("ragged_rows", 2, ((SEG_TEXT, 77), (SEG_REF_AUDIO, 129)), (4, 16, 20), 15.0,
             SINK_EXACT_KV_AND_ROWS, seed=72, recipe="iid"),
    Workload("no_prefix", 2, (), (8, 8, 16), 25.0, SINK_EXACT_KV, seed=73, recipe="scaled"),
    Workload("no_prefix_rows", 1, (), (4, 8, 8), 50.0, SINK_EXACT_KV_AND_ROWS, seed=74),
    Workload("keep_one_tile", 2, ((SEG_TEXT, 64),), (8, 8, 8), 0.5, SINK_EXACT_KV, seed=75,
             recipe="scaled"),
    Workload("keep_all", 2, ((SEG_TEXT, 40),), (4, 8, 12), 100.0, SINK_EXACT_KV, seed=76),
    Workload("batch2", 2, ((SEG_TEXT, 64), (SEG_REF_IMAGE, 128)), (4, 8, 16), 25.0,
             SINK_EXACT_KV_AND_ROWS, seed=77, recipe="scaled", batch=2),
    Workload("one_video_tile", 1, ((SEG_TEXT, 10),), (4, 4, 4), 100.0, SINK_EXACT_KV, seed=78),
    Workload("tau_logmass", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 64)), (8, 16, 16), 0.0,
             SINK_EXACT_KV, SELECT_TAU, COARSE_MEAN_LOGMASS, 1.5, seed=79, recipe="offset"),
    Workload("smooth_gate_rows", 4, ((SEG_TEXT, 128), (SEG_REF_IMAGE, 256)), (8, 16, 24), 10.0,
             SINK_EXACT_KV_AND_ROWS, seed=80, recipe="smooth"),
    # an odd number of video tiles (3 x 5 x 7 = 105) spanning two 64-tile chunks of the
    # coarse kernel, and a sparse row count that is not a multiple of its 64-row blocks
    Workload("odd_video_grid", 2, ((SEG_TEXT, 70),), (12, 20, 28), 20.0, SINK_EXACT_KV_AND_ROWS,
             seed=82, recipe="scaled"),
    Workload("odd_video_grid_tau", 2, ((SEG_TEXT, 70),), (12, 20, 28), 0.0, SINK_EXACT_KV,
             SELECT_TAU, COARSE_MEAN_LOGMASS, 1.0, seed=83, recipe="offset"),
    # sink_conditioning off: prefix tiles compete (168 candidates: three selector slots per
    # lane, three 64-tile chunks of the coarse kernel)
    scaled_down(WORKLOADS["full_sink_off"], heads=3, grid=FULL_SMALL_GRID, name="sink_off_small"),
    Workload("sink_off_ragged", 3, ((SEG_TEXT, 100), (SEG_REF_IMAGE, 64), (SEG_REF_AUDIO, 30)),
             (8, 12, 16), 20.0, SINK_OFF, seed=85, recipe="scaled", video_first=True),
    # partial prefix tiles of 1 and 30 tokens in the log-mass and weighted summaries
    Workload("sink_off_logmass", 2, ((SEG_TEXT, 65), (SEG_REF_AUDIO, 30)), (8, 16, 16), 15.0,
             SINK_OFF, SELECT_TOPK, COARSE_MEAN_LOGMASS, seed=86, recipe="offset"),
    Workload("sink_off_weighted_tau", 2, ((SEG_TEXT, 65), (SEG_REF_AUDIO, 30)), (8, 16, 16), 0.0,
             SINK_OFF, SELECT_TAU, COARSE_WEIGHTED_LOGMASS, 1.0, seed=87, recipe="offset"),
    Workload("sink_off_keep_all", 2, ((SEG_TEXT, 40),), (4, 8, 12), 100.0, SINK_OFF, seed=88),
    # extra tokens: 64 per row on the full recipe (dense prefix rows take none), ragged
    # prefix tiles with a video span first, sink off with tau, and keep 100% (no token
    # left outside the lists: every count is 0)
    scaled_down(WORKLOADS["full_extra64"], heads=2, grid=FULL_SMALL_GRID, name="extra64_small"),
    Workload("extra_ragged", 3, ((SEG_TEXT, 100), (SEG_REF_IMAGE, 64), (SEG_REF_AUDIO, 30)),
             (8, 12, 16), 20.0, SINK_EXACT_KV, seed=89, recipe="scaled", video_first=True, extra=17),
    Workload("extra_off_tau", 2, ((SEG_TEXT, 65), (SEG_REF_AUDIO, 30)), (8, 16, 16), 0.0,
             SINK_OFF, SELECT_TAU, COARSE_MEAN_LOGMASS, 1.5, seed=90, recipe="offset", extra=40),
    Workload("extra_keep_all", 2, ((SEG_TEXT, 40),), (4, 8, 12), 100.0, SINK_EXACT_KV, seed=91,
             extra=64),
    Workload("extra_one", 2, ((SEG_TEXT, 64),), (8, 8, 8), 5.0, SINK_EXACT_KV, seed=92,
             recipe="smooth", extra=1),
    # batch 2 with the options: the batch offsets of the extra-token staging and of the
    # sink-off candidate range and weighted summaries
    Workload("extra_batch2", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 50)), (4, 8, 16), 25.0,
             SINK_EXACT_KV_AND_ROWS, seed=93, recipe="scaled", batch=2, extra=33),
    Workload("sink_off_batch2", 2, ((SEG_TEXT, 70), (SEG_REF_IMAGE, 64)), (4, 8, 16), 20.0,
             SINK_OFF, SELECT_TOPK, COARSE_WEIGHTED_LOGMASS, seed=94, recipe="offset", batch=2),
    # 210 candidate tiles (four 64-tile chunks): the coarse kernel cuts them into two slices
    # per row block and merges the partial softmaxes; tau sums over both slices
    Workload("coarse_slices_tau", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 40)), (8, 32, 52), 0.0,
             SINK_OFF, SELECT_TAU, COARSE_WEIGHTED_LOGMASS, 1.5, seed=96, recipe="offset"),
]


@pytest.mark.parametrize("w", SMALL_CASES, ids=[w.name for w in SMALL_CASES])
def test_parity_small(w):
    x = make_inputs(w)
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    rep = PAR.check_parity(w, x, gpu)
    print(f"[parity] {w.name}: rows={rep['rows']} exact={rep['exact_rows']} adopted={rep['adopted_rows']} "
          f"extra exact={rep['extra_exact']} adopted={rep['extra_adopted']} "
          f"max_abs={rep['max_abs']:.3e} rel_l2={rep['rel_l2']:.3e} s_err={rep['max_s_err']:.2e}",
          flush=True)


# Exact ties in the top-k selection: every video key tile a copy of video tile 0 (K only,
# mean pooling, no bias), so every logit of a row ties exactly, in fp32 on the GPU as in
# fp64 in the oracle.  The lowest video tile indices must win, compared with no adoption.
# 32 candidates (one selector slot per lane) and 80 (two slots per lane, dense prefix rows).
TIE_CASES = [
    Workload("ties_one_slot", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 40)), (8, 16, 16), 25.0,
             SINK_EXACT_KV, seed=97, recipe="scaled"),
    Workload("ties_two_slots", 2, ((SEG_TEXT, 64),), (16, 16, 20), 20.0, SINK_EXACT_KV_AND_ROWS,
             seed=98, recipe="scaled"),
]


@pytest.mark.parametrize("w", TIE_CASES, ids=[w.name for w in TIE_CASES])
def test_topk_exact_ties(w):
    x = make_inputs(w)
    geom = O.map_geometry(w.segments(), *w.grid)
    k = x["k"].copy()
    first = geom.tiles[geom.n_prefix]
    for toks in geom.tiles[geom.n_prefix + 1:]:
        k[:, toks] = x["k"][:, first]
    x = dict(x, k=k)
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    d = plan.desc
    P, kk = d.n_prefix_tiles, d.k
    assert d.n_candidates == geom.n_video and 0 < kk < geom.n_video
    sc = gpu["scores"]
    assert np.array_equal(sc, np.broadcast_to(sc[..., :1], sc.shape)), "GPU logits of a row do not tie"
    want = np.array(list(range(P)) + [P + j for j in range(kk)])
    assert np.all(gpu["counts"] == P + kk)
    assert np.array_equal(gpu["lists"][..., :P + kk], np.broadcast_to(want, gpu["lists"][..., :P + kk].shape)), \
        "ties must go to the lowest video tile indices"
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, want_intermediates=True, fine=False)
    for it in inter.values():
        for i in it["sparse_rows"]:
            assert np.array_equal(it["lists"][i], want), f"oracle row {i}"
    rep = PAR.check_parity(w, x, gpu)
    print(f"[ties] {w.name}: k={kk} rows={rep['rows']} max_abs={rep['max_abs']:.3e}", flush=True)


def test_extra_tokens_exact_ties():
    """One token of every video tile holds the same key, aligned with head 0's mean
    query so it out-scores every other token: for every sparse row of head 0 its copies
    outside the listed tiles tie exactly, and the three lowest token indices must win,
    compared with the oracle's choice with no adoption."""
    from workloads.synth import f32_to_bf16_bits
    w = Workload("extra_ties", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 40)), (8, 16, 16), 25.0,
                 SINK_EXACT_KV, seed=99, recipe="offset", extra=3)
    x = make_inputs(w)
    geom = O.map_geometry(w.segments(), *w.grid)
    mu = PAR.bits_to_f64(x["q"][0, :, 0]).mean(axis=0)
    key = f32_to_bf16_bits((3.0 * np.sqrt(128.0) * mu / np.linalg.norm(mu)).astype(np.float32))
    k = x["k"].copy()
    for t in range(geom.n_prefix, geom.n_tiles):
        k[0, geom.tiles[t][5], 0] = key
    x = dict(x, k=k)
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, heads=[(0, 0)], want_intermediates=True,
                         extra_tokens=w.extra)
    it = inter[(0, 0)]
    copies = {int(geom.tiles[t][5]) for t in range(geom.n_prefix, geom.n_tiles)}
    for i in it["sparse_rows"]:
        s = i   # exact_kv: no dense rows
        cnt = int(gpu["counts"][0, 0, s])
        assert np.array_equal(gpu["lists"][0, 0, s, :cnt], it["lists"][i]), f"row {i} list"
        xc = int(gpu["xcnt"][0, 0, s])
        gx = gpu["xtok"][0, 0, s, :xc].astype(np.int64)
        ox = it["extras"][i]
        assert set(ox.tolist()) <= copies and len(ox) == 3, f"row {i}: oracle extras {ox} are not tied copies"
        assert np.array_equal(gx, ox), f"row {i}: GPU extras {gx} != oracle {ox} (lowest token ids)"
    rep = PAR.check_parity(w, x, gpu)
    print(f"[ties] extra tokens: rows={rep['rows']} max_abs={rep['max_abs']:.3e}", flush=True)


def test_extra_tokens_overflow_fallback():
    """Every video key is one and the same vector, so every row's scores all tie: the
    two-pass select's candidate list then holds every eligible key (more than it keeps
    per row), so each row takes the streaming fallback.  The extra tokens must be the E
    lowest eligible token ids, as the oracle picks them, with no adoption."""
    w = Workload("extra_overflow", 2, ((SEG_TEXT, 64),), (8, 16, 16), 25.0, SINK_EXACT_KV, seed=100,
                 recipe="scaled", extra=64)
    x = make_inputs(w)
    geom = O.map_geometry(w.segments(), *w.grid)
    vid = np.concatenate([geom.tiles[t] for t in range(geom.n_prefix, geom.n_tiles)])
    k = x["k"].copy()
    k[:, vid] = x["k"][:, vid[:1]]
    x = dict(x, k=k)
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    d = plan.desc
    eligible = (geom.n_tiles - geom.n_prefix - d.k) * 64
    assert eligible > 1024, "the case must overflow the per-row candidate list"
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, want_intermediates=True,
                         extra_tokens=w.extra)
    for (b, h), it in inter.items():
        for i in it["sparse_rows"]:
            xc = int(gpu["xcnt"][b, h, i])
            gx = gpu["xtok"][b, h, i, :xc].astype(np.int64)
            assert np.array_equal(gx, it["extras"][i]), f"(b{b},h{h}) row {i}: {gx[:8]} != {it['extras'][i][:8]}"
    rep = PAR.check_parity(w, x, gpu)
    print(f"[overflow] extra tokens: rows={rep['rows']} max_abs={rep['max_abs']:.3e}", flush=True)


def test_extra_tokens_screen_bound():
    """The first pass screens (row, tile) pairs with hi(qbar), the first bf16 term of the
    pooled query, and widens its maxima by a bound on the difference to the exact score.
    Built so that the screen ranks the wrong key first: every query alternates 2 and
    2 + 2^-6 in dim 0 (qbar = 2 + 2^-7, exactly halfway, so hi = 2 and the residual is 2^-7)
    and is 1 in dim 1.  Key A = (1, 255/256) screens at 2.99609375 but scores 3.00390625
    exactly; key B = (0, 3) scores 3 either way; every other video tile holds keys
    (0.5, 0.5), which win the coarse selection (so A's and B's tiles stay unlisted) and
    score 1.50390625.  With one extra token every sparse row must take A, as the oracle
    does: a missing or too small bound would leave A's tile out of the candidates."""
    from workloads.synth import f32_to_bf16_bits
    w = Workload("extra_screen", 1, ((SEG_TEXT, 64),), (8, 8, 16), 25.0, SINK_EXACT_KV, seed=103,
                 recipe="scaled", extra=1)
    x = make_inputs(w)
    geom = O.map_geometry(w.segments(), *w.grid)
    P = geom.n_prefix
    q = np.zeros((1, w.n_tokens, 1, 128), np.float32)
    q[0, 0::2, 0, 0] = 2.0
    q[0, 1::2, 0, 0] = 2.0 + 2.0 ** -6
    q[0, :, 0, 1] = 1.0
    k = np.zeros_like(q)
    ta, tb = P + 1, P + 6  # two of the 16 video tiles
    for t in range(P, geom.n_tiles):
        if t not in (ta, tb):
            k[0, geom.tiles[t], 0, 0] = 0.5
            k[0, geom.tiles[t], 0, 1] = 0.5
    tok_a, tok_b = int(geom.tiles[ta][5]), int(geom.tiles[tb][7])
    k[0, tok_a, 0, :2] = (1.0, 255.0 / 256.0)
    k[0, tok_b, 0, :2] = (0.0, 3.0)
    x = dict(x, q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k))
    # the case is what it claims: hi(qbar) ranks B above A, the exact score A above B
    qbar = np.float32(2.0 + 2.0 ** -7)
    hi = np.float32(2.0)
    assert hi * 1.0 + 255.0 / 256.0 < 3.0 < float(qbar) * 1.0 + 255.0 / 256.0
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, want_intermediates=True, extra_tokens=w.extra)
    it = inter[(0, 0)]
    rows = it["sparse_rows"]
    assert len(rows) > 0
    for i in rows:
        assert ta not in it["lists"][i] and tb not in it["lists"][i], f"row {i} lists A's or B's tile"
        xc = int(gpu["xcnt"][0, 0, i])
        gx = gpu["xtok"][0, 0, i, :xc].astype(np.int64)
        assert it["extras"][i].tolist() == [tok_a], f"row {i}: oracle extras {it['extras'][i]}"
        assert gx.tolist() == [tok_a], f"row {i}: GPU extras {gx.tolist()} (A = {tok_a}, B = {tok_b})"
    rep = PAR.check_parity(w, x, gpu)
    print(f"[screen] extra tokens: rows={rep['rows']} max_abs={rep['max_abs']:.3e}", flush=True)


def test_parity_no_gate():
    w = scaled_down(WORKLOADS["full"], heads=2, grid=(8, 16, 16), name="nogate")
    x = make_inputs(w)
    plan, ws, o, _ = run_gpu(w, x, use_gate=False)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    PAR.check_parity(w, dict(x, g=None), gpu)


def test_deterministic_and_stats():
    V = _lib()
    w = scaled_down(WORKLOADS["full"], heads=2, grid=FULL_SMALL_GRID, name="det")
    x = make_inputs(w)
    plan, ws, o, (q, k, v, g) = run_gpu(w, x)
    o2 = torch.empty_like(o)
    V.vsa_forward(plan, q, k, v, g, o2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    st = V.vsa_read_stats(plan, ws)
    d = plan.desc
    P, Vt, Tq, kk = d.n_prefix_tiles, d.n_video_tiles, d.n_tiles, d.k
    exp_pairs = w.heads * (Vt * (P + kk) + P * Tq)
    assert st["executed_pairs"] == exp_pairs
    assert st["dense_pairs"] == w.heads * Tq * Tq
    assert st["kept_video_tiles"] == w.heads * Vt * kk
    assert 0 < st["executed_pairs"] < st["dense_pairs"]
    assert st["extra_tokens"] == 0


def test_stats_extra():
    """Every sparse row with tokens left outside its list attends to exactly E of them,
    as one more (staged) tile."""
    V = _lib()
    w = scaled_down(WORKLOADS["full_extra64"], heads=2, grid=FULL_SMALL_GRID, name="det_extra")
    x = make_inputs(w)
    plan, ws, o, _ = run_gpu(w, x)
    st = V.vsa_read_stats(plan, ws)
    d = plan.desc
    P, Vt, Tq, kk = d.n_prefix_tiles, d.n_video_tiles, d.n_tiles, d.k
    assert st["extra_tokens"] == w.heads * Vt * w.extra
    assert st["executed_pairs"] == w.heads * (Vt * (P + kk + 1) + P * Tq)


def test_stats_sink_off():
    """sink off: every query tile keeps k = ceil(keep Tq / 100) tiles and nothing else."""
    V = _lib()
    w = scaled_down(WORKLOADS["full_sink_off"], heads=2, grid=FULL_SMALL_GRID, name="det_off")
    x = make_inputs(w)
    plan, ws, o, _ = run_gpu(w, x)
    st = V.vsa_read_stats(plan, ws)
    d = plan.desc
    assert (d.first_candidate, d.n_candidates, d.n_dense_rows) == (0, d.n_tiles, 0)
    assert d.k == int(np.ceil(w.keep * d.n_tiles / 100 - 1e-9))
    assert st["executed_pairs"] == w.heads * d.n_tiles * d.k
    assert st["kept_video_tiles"] == w.heads * d.n_tiles * d.k


def test_abi_errors_on_device():
    V = _lib()
    w = WORKLOADS["tiny"]
    x = make_inputs(w)
    plan = V.vsa_plan_geometry(w.segments(), 1, *w.grid, w.heads, 128, w.keep)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    o = torch.empty_like(q)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(V.VsaError) as e:
        V.vsa_forward(plan, q, k, v, None, o, small)
    assert e.value.status == V.VSA_ERR_WORKSPACE
    ws = V.alloc_workspace(plan)
    with pytest.raises(V.VsaError) as e:
        V.vsa_forward(plan, q, k, v, None, q, ws)   # output aliases an input
    assert e.value.status == V.VSA_ERR_INVALID_ARGUMENT
    V.vsa_forward(plan, q, k, v, None, o, ws)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- full size
@functools.lru_cache(maxsize=1)
def _inputs_for_seed(name):
    return make_inputs(WORKLOADS[name])


FULL_CASES = ["full", "full_smooth_20", "full_smooth_100", "full_tau_1.0", "full_tau_1.5",
              "full_tau_2.0", "full_logmass", "full_weighted", "full_sink_off", "full_extra64"]


@pytest.mark.parametrize("name", FULL_CASES)
def test_parity_full_size_sampled(name):
    w = WORKLOADS[name]
    # workloads that share a seed share their inputs
    src = {"full_smooth_100": "full_smooth_20", "full_tau_1.5": "full_tau_1.0",
           "full_tau_2.0": "full_tau_1.0", "full_logmass": "full_tau_1.0",
           "full_weighted": "full_tau_1.0", "full_sink_off": "full", "full_extra64": "full"}.get(name, name)
    x = _inputs_for_seed(src)
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o, fields=("scores", "lists", "counts", "qbar", "kbar",
                                                          "vbar", "bias", "ocoarse", "thr", "xtok", "xcnt"))
    d = plan.desc
    P, Tq = d.n_prefix_tiles, d.n_tiles
    pinned = 0 if w.sink == SINK_OFF else P
    # properties over every row
    cnt = gpu["counts"]
    if w.select == SELECT_TOPK:
        assert np.all(cnt == pinned + d.k)
    else:
        assert np.all((cnt >= pinned) & (cnt <= pinned + d.n_candidates))
    lists = gpu["lists"]
    assert np.all(lists[..., :pinned] == np.arange(pinned))
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    heads = [(0, 0), (0, int(rng.integers(1, w.heads)))]
    rows = sorted(set([0, P - 1, P, Tq - 1] + [int(r) for r in rng.integers(0, Tq, size=4)]))
    rep = PAR.check_parity(w, x, gpu, heads=heads, rows=rows)
    print(f"[parity-full] {name}: rows={rep['rows']} exact={rep['exact_rows']} adopted={rep['adopted_rows']} "
          f"max_abs={rep['max_abs']:.3e} rel_l2={rep['rel_l2']:.3e}", flush=True)
    # every sparse row's selection and logits on four heads (head 0 and three others)
    others = rng.choice(np.arange(1, w.heads), size=3, replace=False)
    lheads = [(0, 0)] + [(0, int(hh)) for hh in sorted(others)]
    lrep = PAR.check_lists(w, x, gpu, heads=lheads)
    print(f"[lists-full] {name}: heads={[hh for _, hh in lheads]} rows={lrep['rows']} "
          f"exact={lrep['exact_rows']} adopted={lrep['adopted_rows']} s_err={lrep['max_s_err']:.2e}", flush=True)


# The plan's limits: 16 prefix segments (most of them partial tiles), a sparse row list at
# its 2048-entry capacity (keep 100%: 8 prefix + 2040 video tiles), and 4096 video tiles
# (the selector's 64-slots-per-lane path, 64 chunks of the coarse kernel), also with 64
# extra tokens.  Sampled rows.
LIMIT_CASES = [
    Workload("max_prefix_segs", 2,
             tuple((k % 4, n) for k, n in enumerate([1, 7, 64, 65, 100, 3, 128, 30, 64, 9, 200, 17, 63, 2, 77, 40])),
             (4, 8, 8), 25.0, SINK_EXACT_KV, seed=93, recipe="scaled"),
    Workload("max_list", 1, ((SEG_TEXT, 300), (SEG_REF_AUDIO, 148)), (32, 60, 68), 100.0, SINK_EXACT_KV,
             seed=94, recipe="scaled"),
    Workload("max_video_tiles", 1, ((SEG_TEXT, 64),), (64, 64, 64), 1.0, SINK_EXACT_KV_AND_ROWS, seed=95,
             recipe="scaled"),
    # the same shape with 64 extra tokens: each row's scoring streams all 4,097 key tiles
    Workload("max_video_tiles_extra", 1, ((SEG_TEXT, 64),), (64, 64, 64), 1.0, SINK_EXACT_KV_AND_ROWS,
             seed=95, recipe="scaled", extra=64),
    # 1,025 and 2,049 tiles with 64 extra tokens: the extra-token threshold kernel's shapes for
    # up to 2,048 and up to 4,096 tiles per row (8 and 4 rows per workgroup)
    Workload("long_video_extra_1k", 1, ((SEG_TEXT, 64),), (32, 32, 64), 2.0, SINK_EXACT_KV, seed=101,
             recipe="scaled", extra=64),
    Workload("long_video_extra_2k", 1, ((SEG_TEXT, 64),), (32, 64, 64), 1.0, SINK_EXACT_KV, seed=102,
             recipe="scaled", extra=64),
]


@pytest.mark.parametrize("w", LIMIT_CASES, ids=[w.name for w in LIMIT_CASES])
def test_parity_limits(w):
    x = make_inputs(w)
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    d = plan.desc
    P, Tq = d.n_prefix_tiles, d.n_tiles
    cnt = gpu["counts"]
    assert np.all(cnt == P + d.k)
    assert d.list_capacity <= 2048
    rng = np.random.default_rng(zlib.crc32(w.name.encode()))
    rows = sorted(set([0, P - 1, P, Tq - 1] + [int(r) for r in rng.integers(0, Tq, size=3)]))
    rep = PAR.check_parity(w, x, gpu, heads=[(0, h) for h in range(w.heads)], rows=rows)
    print(f"[parity-limit] {w.name}: P={P} Vt={d.n_video_tiles} cap={d.list_capacity} rows={rep['rows']} "
          f"exact={rep['exact_rows']} adopted={rep['adopted_rows']} max_abs={rep['max_abs']:.3e}", flush=True)


def test_parity_growing_logits():
    """Keys scaled up tile by tile (x1 for the prefix tile, up to x17 for the last video
    tile), so along every row's list the running max grows by far more than the lazy
    threshold (2^16): the rare rescale of O and l runs on every wave, several times on most."""
    from workloads.synth import bf16_bits_to_f32, f32_to_bf16_bits
    w = Workload("growing_logits", 2, ((SEG_TEXT, 64),), (8, 8, 16), 100.0, SINK_EXACT_KV_AND_ROWS,
                 seed=81, recipe="iid")
    x = make_inputs(w)
    geom = O.map_geometry(w.segments(), *w.grid)
    kf = bf16_bits_to_f32(x["k"])
    for t, toks in enumerate(geom.tiles):
        kf[:, toks] *= np.float32(1.0 + 1.0 * t)
    x = dict(x, k=f32_to_bf16_bits(kf))
    plan, ws, o, _ = run_gpu(w, x)
    gpu = PAR.gpu_results_to_numpy(plan, ws, o)
    rep = PAR.check_parity(w, x, gpu)
    print(f"[parity] growing_logits: rows={rep['rows']} max_abs={rep['max_abs']:.3e} rel_l2={rep['rel_l2']:.3e}",
          flush=True)
