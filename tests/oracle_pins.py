"""Pins of the fp64 oracle against things other than itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with an
independent statement of what it must compute: a library routine (torch's
scaled_dot_product_attention in float64, Python's exact ``statistics``
module), an independent formulation (the video grid sliced into 4x4x4 cubes
with numpy reshapes), brute force on tiny inputs, closed forms (log cosh),
invariants and metamorphic relations.  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutations.py`` plants plausible mistakes in
the oracle and checks that some pin fails.

Pages are cited by the short tags defined in the oracle's header.
"""
from __future__ import annotations

import itertools
import json
import math
import statistics
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

from oracle import vsa_oracle as O
from workloads.synth import (Workload, make_inputs, f32_to_bf16_bits, SEG_TEXT,
                             SEG_REF_IMAGE, SEG_REF_AUDIO, SEG_VIDEO, SINK_OFF, SINK_EXACT_KV,
                             SINK_EXACT_KV_AND_ROWS, SELECT_TOPK, SELECT_TAU,
                             COARSE_MEAN, COARSE_MEAN_LOGMASS, COARSE_WEIGHTED_LOGMASS)

GOLDEN = json.loads((Path(__file__).parent / "golden" / "page_numbers.json").read_text())
D = 128

# small shapes: several tiles, partial prefix tiles, both segment orders
SMALL = Workload("small", 2, ((SEG_TEXT, 100), (SEG_REF_IMAGE, 64), (SEG_REF_AUDIO, 30)),
                 (4, 8, 12), 25.0, SINK_EXACT_KV, seed=7, recipe="iid")
SMALL_VIDEO_FIRST = Workload("small_vf", 1, ((SEG_TEXT, 70), (SEG_REF_AUDIO, 64)), (8, 4, 8),
                             30.0, SINK_EXACT_KV, seed=8, recipe="scaled", video_first=True)
# every video axis holds more than one tile
GEOM_3D = Workload("geom3d", 1, ((SEG_REF_IMAGE, 200),), (8, 12, 16), 25.0, SINK_EXACT_KV, seed=6)


def as_f64(bits):
    return O.bf16_bits_to_f64(bits)


def torch_sdpa(q, k, v, mask=None):
    """Textbook softmax(q k^T / sqrt(d) + mask) v in float64 via torch."""
    tq = torch.from_numpy(np.ascontiguousarray(q))[None, None]
    tk = torch.from_numpy(np.ascontiguousarray(k))[None, None]
    tv = torch.from_numpy(np.ascontiguousarray(v))[None, None]
    tm = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask))[None, None]
    with torch.no_grad():
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm)
    return out[0, 0].numpy()


def video_cube_tokens(w: Workload):
    """Token ids of every 4x4x4 video cube, from a reshape of the packed grid.

    Independent of the oracle's index arithmetic: the video span is viewed as
    a (T, H, W) array of token ids (raster, w fastest) and sliced."""
    T, H, W = w.grid
    vstart = [s for s, n, kd in w.segments() if kd == SEG_VIDEO][0]
    ids = vstart + np.arange(T * H * W).reshape(T, H, W)
    cubes = ids.reshape(T // 4, 4, H // 4, 4, W // 4, 4).transpose(0, 2, 4, 1, 3, 5)
    return cubes.reshape(-1, 64)


def prefix_chunks(w: Workload):
    """Token ids of each 64-token run of every prefix segment, packed order."""
    out = []
    for s, n, kd in sorted(w.segments()):
        if kd == SEG_VIDEO:
            continue
        for off in range(0, n, 64):
            out.append(np.arange(s + off, s + min(off + 64, n)))
    return out


def independent_pool(X, w: Workload):
    """Per-tile means: prefix chunks by slicing, video cubes by reshape+mean."""
    T, H, W = w.grid
    vstart = [s for s, n, kd in w.segments() if kd == SEG_VIDEO][0]
    pre = np.stack([X[c].mean(axis=0) for c in prefix_chunks(w)])
    vid = X[vstart:vstart + T * H * W].reshape(T // 4, 4, H // 4, 4, W // 4, 4, X.shape[1])
    vid = vid.mean(axis=(1, 3, 5)).reshape(-1, X.shape[1])
    return pre, vid


def geom_of(w: Workload):
    return O.map_geometry(w.segments(), *w.grid)


# ---------------------------------------------------------------- P-4 geometry
def check_geometry(w: Workload):
    geom = geom_of(w)
    cubes = video_cube_tokens(w)
    chunks = prefix_chunks(w)
    assert geom.n_prefix == len(chunks)
    assert geom.n_video == len(cubes)
    for i, c in enumerate(chunks):
        assert np.array_equal(geom.tiles[i], c), f"prefix tile {i}"
    for j, c in enumerate(cubes):
        assert np.array_equal(geom.tiles[geom.n_prefix + j], c), f"video tile {j}"
    # partition of the valid tokens
    allt = np.concatenate(geom.tiles)
    assert np.array_equal(np.sort(allt), np.arange(w.n_tokens))
    # segment purity and cube shape
    kind_of = np.empty(w.n_tokens, dtype=np.int64)
    for s, n, kd in w.segments():
        kind_of[s:s + n] = kd
    for t, toks in enumerate(geom.tiles):
        assert len(set(kind_of[toks].tolist())) == 1, f"tile {t} mixes segments"
        assert 1 <= len(toks) <= GOLDEN["tile_tokens"]["value"]
    T, H, W = w.grid
    vstart = geom.video_start
    e = GOLDEN["tile_edge"]["value"]
    for toks in geom.tiles[geom.n_prefix:]:
        r = toks - vstart
        t, h, ww = r // (H * W), (r // W) % H, r % W
        for ax in (t, h, ww):
            assert ax.max() - ax.min() == e - 1 and ax.min() % e == 0
            assert len(set(ax.tolist())) == e
    # gather then scatter is the identity, bitwise
    X = np.random.default_rng(3).standard_normal((w.n_tokens, 5))
    gathered = [X[toks] for toks in geom.tiles]
    Y = np.full_like(X, np.nan)
    for toks, g in zip(geom.tiles, gathered):
        Y[toks] = g
    assert np.array_equal(X, Y)


def check_keep_counts():
    """k from a keep percent at the pages' operating points and the workloads' grids."""
    assert O.keep_count(10.0, 528) == 53
    assert O.keep_count(20.0, 528) == 106
    assert O.keep_count(25.0, 264) == 66
    assert O.keep_count(25.0, 16) == 4
    assert O.keep_count(100.0, 528) == 528
    assert O.keep_count(0.01, 528) == 1
    for p in GOLDEN["keep_operating_points_percent"]["value"]:
        k = O.keep_count(float(p), 528)
        assert k - 1 < p * 528 / 100 <= k


# ---------------------------------------------------------------- P-1 fine branch
def check_dense_equivalence(w: Workload):
    """keep 100%, no gate: every list holds every tile, so the output is plain
    dense softmax attention over all tokens ([BSA-es]/[SPK-es]: sparse results
    are compared with the dense run)."""
    x = make_inputs(w, with_gate=False)
    out, _ = O.forward(x, w.segments(), w.grid, 100.0, w.sink)
    for b in range(w.batch):
        for h in range(w.heads):
            ref = torch_sdpa(as_f64(x["q"][b, :, h]), as_f64(x["k"][b, :, h]), as_f64(x["v"][b, :, h]))
            err = np.abs(out[b, :, h] - ref).max()
            assert err < 1e-12, f"dense equivalence b{b} h{h}: {err}"


def check_dense_rows_and_gate(w: Workload):
    """exact_kv_and_rows at keep 100% with a gate: prefix rows are dense with no
    coarse term; video rows are dense plus G * O_coarse of their tile."""
    x = make_inputs(w, with_gate=True)
    out, _ = O.forward(x, w.segments(), w.grid, 100.0, SINK_EXACT_KV_AND_ROWS)
    cubes = video_cube_tokens(w)
    for b in range(w.batch):
        for h in range(w.heads):
            Q, K, V, G = (as_f64(x[n][b, :, h]) for n in "qkvg")
            dense = torch_sdpa(Q, K, V)
            _, qv = independent_pool(Q, w)
            _, kv = independent_pool(K, w)
            _, vv = independent_pool(V, w)
            oc = torch_sdpa(qv, kv, vv)                    # [Vt, D]
            ref = dense.copy()
            for j, toks in enumerate(cubes):
                ref[toks] += G[toks] * oc[j][None, :]
            err = np.abs(out[b, :, h] - ref).max()
            assert err < 1e-12, f"dense rows + gate b{b} h{h}: {err}"


# ---------------------------------------------------------------- P-2 coarse
def check_pooling(w: Workload):
    x = make_inputs(w)
    geom = geom_of(w)
    for h in range(w.heads):
        X = as_f64(x["q"][0, :, h])
        pre, vid = independent_pool(X, w)
        got = O.pool_tiles(X, geom.tiles)
        assert np.abs(got[:geom.n_prefix] - pre).max() < 1e-13
        assert np.abs(got[geom.n_prefix:] - vid).max() < 1e-13


def check_coarse(w: Workload, coarse=COARSE_MEAN):
    """O_coarse is dense attention on the pooled summaries (plus the bias as an
    additive mask in log-mass mode); prefix key tiles are not in it."""
    x = make_inputs(w)
    geom = geom_of(w)
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, SINK_EXACT_KV, coarse=coarse,
                         want_intermediates=True)
    for h in range(w.heads):
        Q, K, V = (as_f64(x[n][0, :, h]) for n in "qkv")
        qp, qv = independent_pool(Q, w)
        _, kv = independent_pool(K, w)
        _, vv = independent_pool(V, w)
        it = inter[(0, h)]
        assert it["sparse_rows"] == list(range(geom.n_tiles))
        qall = np.concatenate([qp, qv])
        mask = np.broadcast_to(it["bias"][None, :], (qall.shape[0], kv.shape[0]))
        ref = torch_sdpa(qall, kv, vv, mask=mask)
        assert np.abs(it["Oc"] - ref).max() < 1e-12
        S_ref = qall @ kv.T / math.sqrt(D) + mask
        assert np.abs(it["S"] - S_ref).max() < 1e-12
        if coarse == COARSE_MEAN:
            assert np.all(it["bias"] == 0.0)


# ---------------------------------------------------------------- P-3 prefix exemption
def check_prefix_exempt(w: Workload):
    x = make_inputs(w)
    geom = geom_of(w)
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, want_intermediates=True)
    k = O.keep_count(w.keep, geom.n_video)
    sparse, dense = O.row_classes(geom, w.sink)
    for it in inter.values():
        for i, lst in it["lists"].items():
            lst = list(lst)
            assert lst == sorted(lst)
            assert set(range(geom.n_prefix)) <= set(lst), f"row {i} lost a prefix tile"
            if i in dense:
                assert lst == list(range(geom.n_tiles))
            else:
                assert len(lst) == geom.n_prefix + k
                assert all(t >= geom.n_prefix for t in lst[geom.n_prefix:])


# ---------------------------------------------------------------- P-5 top-k
def brute_topk(s, k):
    """All k-subsets; keep those with the largest sorted value profile, then the
    lexicographically smallest index set (ties -> lowest indices)."""
    best = None
    for comb in itertools.combinations(range(len(s)), k):
        key = (sorted((s[j] for j in comb), reverse=True), [-j for j in comb])
        # compare value profile first (larger better), then prefer smaller indices
        if best is None or key[0] > best[0][0] or (key[0] == best[0][0] and list(comb) < best[1]):
            best = (key, list(comb))
    return best[1]


def check_topk_bruteforce():
    rng = np.random.default_rng(11)
    for trial in range(60):
        n = int(rng.integers(3, 9))
        k = int(rng.integers(1, n + 1))
        vals = rng.integers(0, 4, size=n).astype(np.float64) if trial % 2 else rng.standard_normal(n)
        got = list(O.select_topk(vals, k))
        assert got == brute_topk(list(vals), k), (vals, k, got)


def check_topk_ties_in_forward():
    """Every video key tile a copy of video tile 0: all coarse logits of a row
    tie, so each sparse row must keep video tiles 0..k-1."""
    w = Workload("ties", 1, ((SEG_TEXT, 64),), (4, 8, 8), 25.0, SINK_EXACT_KV, seed=5)
    x = make_inputs(w)
    geom = geom_of(w)
    k = x["k"].copy()
    first = geom.tiles[geom.n_prefix]
    for toks in geom.tiles[geom.n_prefix:]:
        k[0, toks] = x["k"][0, first]
    x["k"] = k
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, want_intermediates=True)
    kk = O.keep_count(w.keep, geom.n_video)
    for lst in inter[(0, 0)]["lists"].values():
        assert list(lst) == list(range(geom.n_prefix)) + [geom.n_prefix + j for j in range(kk)]


# ---------------------------------------------------------------- P-6 tau
def check_tau_threshold():
    rng = np.random.default_rng(21)
    S = rng.standard_normal((7, 11)) * 0.3 + 0.1
    vals = [Fraction(float(v)) for v in S.ravel()]
    mu = statistics.fmean(S.ravel())
    sd = statistics.pstdev(S.ravel().tolist())
    for tau in (1.0, 1.5, 2.0, -0.5):
        thr = O.tau_threshold(S, tau)
        assert abs(thr - (mu + tau * sd)) < 1e-12
    assert len(vals) == 77


def check_tau_limits(w: Workload):
    x = make_inputs(w)
    geom = geom_of(w)
    for tau, expect_video in ((1e6, 0), (-1e6, geom.n_video)):
        _, inter = O.forward(x, w.segments(), w.grid, 0.0, SINK_EXACT_KV, select=SELECT_TAU,
                             tau=tau, want_intermediates=True)
        for lst in inter[(0, 0)]["lists"].values():
            assert len(lst) == geom.n_prefix + expect_video


def check_tau_dense_rows(tau: float = 0.7):
    """Tau mode under exact_kv_and_rows ([BSA-es] Sol-Attn item; [FH3] "The inputs that
    matter"): the conditioning query tiles run dense, so the moments run over the video
    rows x video tiles logits only (Python's exact statistics module on independently
    pooled tiles).  Each video row lists every prefix tile, then the video tiles above
    the threshold; each prefix row lists every tile and its output is dense attention
    over all tokens with no coarse term, although a gate is given."""
    w = Workload("tau_rows", 2, SMALL.prefix, (8, 8, 12), 0.0, SINK_EXACT_KV_AND_ROWS,
                 SELECT_TAU, seed=13, recipe="offset")
    x = make_inputs(w, with_gate=True)
    P = len(prefix_chunks(w))
    assert P >= 2
    cubes = video_cube_tokens(w)
    Vt = len(cubes)
    out, inter = O.forward(x, w.segments(), w.grid, 0.0, SINK_EXACT_KV_AND_ROWS, select=SELECT_TAU,
                           tau=tau, want_intermediates=True)
    kept = 0
    for h in range(w.heads):
        Q, K, V = (as_f64(x[n][0, :, h]) for n in "qkv")
        _, qv = independent_pool(Q, w)
        _, kv = independent_pool(K, w)
        S = qv @ kv.T / math.sqrt(D)                      # video rows x video tiles
        thr = statistics.fmean(S.ravel()) + tau * statistics.pstdev(S.ravel().tolist())
        it = inter[(0, h)]
        assert abs(it["thr"] - thr) < 1e-12, f"h{h}: thr {it['thr']} != {thr}"
        for j in range(Vt):
            want = list(range(P)) + [P + c for c in range(Vt) if S[j, c] > thr]
            assert list(it["lists"][P + j]) == want, f"h{h} video row {j}"
            kept += len(want) - P
        dense = torch_sdpa(Q, K, V)
        for i, toks in enumerate(prefix_chunks(w)):
            assert list(it["lists"][i]) == list(range(P + Vt)), f"h{h} prefix row {i} not dense"
            assert np.abs(out[0, toks, h] - dense[toks]).max() < 1e-12, f"h{h} prefix row {i} output"
    assert 0 < kept < w.heads * Vt * Vt, "the threshold must keep some tiles and drop others"


def check_tau_fractions():
    """On near-Gaussian pooled logits the kept share of video tiles follows the
    pages' tau -> share table (statistical sanity, loose bound)."""
    w = Workload("taufrac", 2, ((SEG_TEXT, 128),), (16, 16, 16), 0.0, SINK_EXACT_KV, seed=31)
    x = make_inputs(w, with_gate=False)
    geom = geom_of(w)
    for tau_s, page in GOLDEN["tau_kept_fraction"]["value"].items():
        tau = float(tau_s)
        _, inter = O.forward(x, w.segments(), w.grid, 0.0, SINK_EXACT_KV, select=SELECT_TAU,
                             tau=tau, rows=[], want_intermediates=True)
        kept = 0
        total = 0
        for it in inter.values():
            kept += int((it["S"] > it["thr"]).sum())
            total += it["S"].size
        frac = kept / total
        assert abs(frac - page) <= max(0.01, 0.2 * page), (tau, frac, page)


# ---------------------------------------------------------------- P-7 log-mass
def check_logmass():
    """Jensen (b >= 0), constant tiles (b = 0) and a closed form: when the
    anchored token logits of a tile are +d and -d in equal numbers,
    b = log cosh d ([SPK-es] Spark-Reweight and its figure: the biased pooled
    logit's exponential equals the mean exponential)."""
    w = Workload("lm", 1, ((SEG_TEXT, 64),), (4, 8, 8), 25.0, SINK_EXACT_KV, seed=41)
    x = make_inputs(w)
    geom = geom_of(w)
    q = np.zeros((1, w.n_tokens, 1, D), np.float32)
    k = np.zeros_like(q)
    u = np.zeros(D, np.float32)
    u[3] = 1.5
    vs = geom.video_start
    q[0, :, 0] = np.asarray(O.bf16_bits_to_f64(x["q"][0, :, 0]), np.float32)
    q[0, vs:, 0] = u                                  # every video query equals u
    rng = np.random.default_rng(42)
    tiles = geom.tiles[geom.n_prefix:]
    amp = {}
    for j, toks in enumerate(tiles):
        base = rng.integers(-8, 8, size=D).astype(np.float32) / 4
        if j % 3 == 0:                                # constant tile -> b = 0
            k[0, toks, 0] = base
            amp[j] = 0.0
        elif j % 3 == 1:                              # +/- a along e3 -> log cosh
            a = float(j % 5 + 1) / 2
            sgn = np.where(np.arange(len(toks)) % 2 == 0, 1.0, -1.0).astype(np.float32)
            k[0, toks, 0] = base
            k[0, toks, 0, 3] += sgn * a
            amp[j] = 1.5 * a / math.sqrt(D)
        else:                                         # random tile: Jensen only
            k[0, toks, 0] = rng.standard_normal((len(toks), D)).astype(np.float32)
    Qh = O.bf16_bits_to_f64(f32_to_bf16_bits(q)[0, :, 0])
    Kh = O.bf16_bits_to_f64(f32_to_bf16_bits(k)[0, :, 0])
    b, q_a = O.logmass_bias(Qh, Kh, geom, 1.0 / math.sqrt(D))
    assert np.allclose(q_a, u, atol=0, rtol=0)
    assert np.all(b >= -1e-15)
    for j, d in amp.items():
        assert abs(b[j] - math.log(math.cosh(d))) < 1e-12, (j, b[j], d)
    # the biased pooled logit's exponential equals the mean token exponential
    for j, toks in enumerate(tiles):
        s = 1.0 / math.sqrt(D)
        lhs = math.exp(s * float(u.astype(np.float64) @ Kh[toks].mean(axis=0)) + b[j])
        rhs = float(np.mean([math.exp(s * float(u.astype(np.float64) @ Kh[t])) for t in toks]))
        assert abs(lhs - rhs) <= 1e-12 * rhs


def check_weighted_summaries():
    """Weighted key / value summaries ([SPK-es] Spark-Reweight; weights read as the
    anchor's attention over the tile) against an independent routine and reductions:
      * vtil_j and ktil_j are torch's float64 scaled_dot_product_attention of the
        anchor (the mean of the video queries, taken over the 4x4x4 cubes of an
        independent reshape) over tile j's keys and values / keys;
      * exp(s q_a . ktil_j + b_j) is the mean token exponential, summed directly;
      * a tile whose keys are all equal gives ktil = that key, vtil = the mean value
        and b = 0;
      * a zero anchor (video queries in +q / -q pairs) weighs every token equally,
        so the whole forward equals the plain-mean mode's."""
    w = Workload("ws", 1, ((SEG_TEXT, 64),), (4, 8, 8), 25.0, SINK_EXACT_KV, seed=43, recipe="offset")
    x = make_inputs(w)
    geom = geom_of(w)
    cubes = video_cube_tokens(w)
    # tile 0: every key equal to its first one
    kb = x["k"].copy()
    kb[0, cubes[0], 0] = kb[0, cubes[0][0], 0]
    Qh, Kh, Vh = as_f64(x["q"][0, :, 0]), as_f64(kb[0, :, 0]), as_f64(x["v"][0, :, 0])
    s = 1.0 / math.sqrt(D)
    ktil, vtil, b, q_a = O.weighted_summaries(Qh, Kh, Vh, geom, s)
    q_ref = Qh[np.concatenate(cubes)].mean(axis=0)
    assert np.abs(q_a - q_ref).max() < 1e-14
    for j, toks in enumerate(cubes):
        v_ref = torch_sdpa(q_ref[None, :], Kh[toks], Vh[toks])[0]
        k_ref = torch_sdpa(q_ref[None, :], Kh[toks], Kh[toks])[0]
        assert np.abs(vtil[j] - v_ref).max() < 1e-12 * (1 + np.abs(v_ref).max()), j
        assert np.abs(ktil[j] - k_ref).max() < 1e-12 * (1 + np.abs(k_ref).max()), j
        lhs = math.exp(s * float(q_ref @ k_ref) + b[j])
        rhs = math.fsum(math.exp(s * float(q_ref @ Kh[t])) for t in toks) / len(toks)
        assert abs(lhs - rhs) <= 1e-12 * rhs, (j, lhs, rhs)
    assert np.abs(ktil[0] - Kh[cubes[0][0]]).max() < 1e-14
    assert np.abs(vtil[0] - Vh[cubes[0]].mean(axis=0)).max() < 1e-14
    assert abs(b[0]) < 1e-14
    # zero anchor: pair every video query with its negation
    xz = dict(x)
    qz = x["q"].copy()
    vid = np.concatenate(cubes)
    qz[0, vid[1::2], 0] = qz[0, vid[0::2], 0] ^ np.uint16(0x8000)
    xz["q"] = qz
    ow, iw = O.forward(xz, w.segments(), w.grid, w.keep, w.sink, coarse=COARSE_WEIGHTED_LOGMASS,
                       want_intermediates=True)
    om, im = O.forward(xz, w.segments(), w.grid, w.keep, w.sink, coarse=COARSE_MEAN,
                       want_intermediates=True)
    assert np.abs(iw[(0, 0)]["anchor"]).max() == 0.0
    assert np.abs(iw[(0, 0)]["S"] - im[(0, 0)]["S"]).max() < 1e-12
    assert np.abs(ow - om).max() < 1e-12


# ---------------------------------------------------------------- P-8 combine
def check_combine(w: Workload):
    x = make_inputs(w, with_gate=True)
    segs = w.segments()
    o1, _ = O.forward(x, segs, w.grid, w.keep, w.sink)
    x0 = dict(x, g=None)
    o0, _ = O.forward(x0, segs, w.grid, w.keep, w.sink)
    xz = dict(x, g=np.zeros_like(x["g"]))
    oz, _ = O.forward(xz, segs, w.grid, w.keep, w.sink)
    assert np.array_equal(o0, oz)
    # linear in G: doubling G (exact in bf16) doubles O - O(G=0)
    g2 = f32_to_bf16_bits(2 * O.bf16_bits_to_f64(x["g"]).astype(np.float32))
    o2, _ = O.forward(dict(x, g=g2), segs, w.grid, w.keep, w.sink)
    assert np.abs((o2 - o0) - 2 * (o1 - o0)).max() < 1e-12
    assert np.abs(o1 - o0).max() > 1e-3


# ---------------------------------------------------------------- P-9 metamorphic
def check_metamorphic(w: Workload):
    x = make_inputs(w, with_gate=True)
    geom = geom_of(w)
    rng = np.random.default_rng(51)
    for h in range(w.heads):
        Q, K, V, G = (as_f64(x[n][0, :, h]) for n in "qkvg")
        for coarse in (COARSE_MEAN, COARSE_MEAN_LOGMASS):
            args = (geom, w.keep, w.sink, SELECT_TOPK, coarse, 0.0)
            o, it = O.forward_head(Q, K, V, G, *args, want_intermediates=True)
            c = rng.standard_normal(D)
            o2, it2 = O.forward_head(Q, K + c[None, :], V, G, *args, want_intermediates=True)
            for i in it["lists"]:
                assert np.array_equal(it["lists"][i], it2["lists"][i])
            assert np.abs(o - o2).max() < 1e-9
            assert np.abs(it["bias"] - it2["bias"]).max() < 1e-9
            o3, _ = O.forward_head(Q, K, 3.0 * V, G, *args)
            assert np.abs(o3 - 3.0 * o).max() < 1e-9


def check_prefix_permutation():
    """Reordering the conditioning segments permutes the outputs of their
    tokens and leaves every video token's output unchanged."""
    pre = ((SEG_TEXT, 64), (SEG_REF_IMAGE, 128), (SEG_REF_AUDIO, 64))
    w = Workload("perm", 1, pre, (4, 8, 8), 25.0, SINK_EXACT_KV, seed=61)
    x = make_inputs(w)
    perm_pre = (pre[2], pre[0], pre[1])
    w2 = Workload("perm2", 1, perm_pre, (4, 8, 8), 25.0, SINK_EXACT_KV, seed=61)
    # token map: new position -> old position
    old_start = {kd: s for s, n, kd in w.segments()}
    idx = []
    for s, n, kd in sorted(w2.segments()):
        idx.extend(range(old_start[kd], old_start[kd] + n))
    idx = np.asarray(idx)
    x2 = {n: x[n][:, idx] for n in "qkvg"}
    o, _ = O.forward(x, w.segments(), w.grid, w.keep, w.sink)
    o2, _ = O.forward(x2, w2.segments(), w2.grid, w2.keep, w2.sink)
    assert np.abs(o2 - o[:, idx]).max() < 1e-12


# ---------------------------------------------------------------- P-10 sink off
# [FH3] "The inputs that matter", sink_conditioning: off protects no conditioning
# tile, so the prefix tiles compete with the video tiles in the coarse branch and
# the selection.  The pins rebuild every step from independent pieces: the tiles
# from slicing and a reshape of the grid, the pooled logits from a matmul, the
# selection by brute force over all k-subsets, the attention from torch's sdpa.
SINK_OFF_W = Workload("off", 2, SMALL.prefix, SMALL.grid, 30.0, SINK_OFF, seed=71, recipe="scaled")
# partial prefix tiles of 64 + 1 and 30 tokens
SINK_OFF_PARTIAL = Workload("off_part", 1, ((SEG_TEXT, 65), (SEG_REF_AUDIO, 30)), (4, 8, 8), 20.0,
                            SINK_OFF, seed=72, recipe="offset")


def _all_tiles(w: Workload):
    """Token ids of every tile in tile-id order: prefix chunks, then video cubes."""
    return prefix_chunks(w) + [c for c in video_cube_tokens(w)]


def _pool_all(X, w: Workload):
    pre, vid = independent_pool(X, w)
    return np.concatenate([pre, vid])


def check_sink_off_dense(w: Workload):
    """keep 100% with sink off keeps all Tq tiles (not Vt of them): with no gate the
    output is dense attention over every token."""
    x = make_inputs(w, with_gate=False)
    out, _ = O.forward(x, w.segments(), w.grid, 100.0, SINK_OFF)
    for h in range(w.heads):
        ref = torch_sdpa(as_f64(x["q"][0, :, h]), as_f64(x["k"][0, :, h]), as_f64(x["v"][0, :, h]))
        err = np.abs(out[0, :, h] - ref).max()
        assert err < 1e-12, f"sink off dense h{h}: {err}"


def check_sink_off_selection(w: Workload, k: int):
    """Selection and output with sink off, rebuilt from independent pieces; k is the
    expected keep count over all Tq tiles, given as a literal."""
    x = make_inputs(w, with_gate=True)
    tiles = _all_tiles(w)
    Tq, P = len(tiles), len(prefix_chunks(w))
    out, inter = O.forward(x, w.segments(), w.grid, w.keep, SINK_OFF, want_intermediates=True)
    kept_pre = dropped_pre = 0
    for h in range(w.heads):
        Q, K, V, G = (as_f64(x[n][0, :, h]) for n in "qkvg")
        qall, kall, vall = _pool_all(Q, w), _pool_all(K, w), _pool_all(V, w)
        S = qall @ kall.T / math.sqrt(D)
        oc = torch_sdpa(qall, kall, vall)
        it = inter[(0, h)]
        assert it["sparse_rows"] == list(range(Tq)), "sink off: every query tile is a sparse row"
        assert it["S"].shape == S.shape, f"coarse logits shape {it['S'].shape} != {S.shape}"
        assert np.abs(it["S"] - S).max() < 1e-12
        assert np.abs(it["Oc"] - oc).max() < 1e-12
        for i in range(Tq):
            pick = brute_topk(list(S[i]), k)
            assert list(it["lists"][i]) == pick, f"h{h} row {i}: {list(it['lists'][i])} != {pick}"
            keys = np.concatenate([tiles[t] for t in pick])
            ref = torch_sdpa(Q[tiles[i]], K[keys], V[keys]) + G[tiles[i]] * oc[i][None, :]
            assert np.abs(out[0, tiles[i], h] - ref).max() < 1e-12, f"h{h} row {i} output"
            n_pre = sum(1 for t in pick if t < P)
            kept_pre += n_pre
            dropped_pre += P - n_pre
    assert kept_pre > 0 and dropped_pre > 0, "prefix tiles must both win and lose somewhere"


def check_sink_off_tau(w: Workload, tau: float):
    """Tau mode with sink off: the threshold's moments run over every (query tile, tile)
    logit, prefix tiles included, and a row keeps the tiles above it (Python's exact
    statistics module for the moments)."""
    x = make_inputs(w, with_gate=False)
    tiles = _all_tiles(w)
    _, inter = O.forward(x, w.segments(), w.grid, 0.0, SINK_OFF, select=SELECT_TAU, tau=tau,
                         want_intermediates=True)
    for h in range(w.heads):
        Q, K = as_f64(x["q"][0, :, h]), as_f64(x["k"][0, :, h])
        S = _pool_all(Q, w) @ _pool_all(K, w).T / math.sqrt(D)
        thr = statistics.fmean(S.ravel()) + tau * statistics.pstdev(S.ravel().tolist())
        it = inter[(0, h)]
        assert abs(it["thr"] - thr) < 1e-12
        for i in range(len(tiles)):
            want = [j for j in range(len(tiles)) if S[i, j] > thr]
            assert list(it["lists"][i]) == want, f"h{h} row {i}"


def check_sink_off_logmass():
    """Log-mass bias and weighted summaries over partial prefix tiles (sink off): the
    means run over a tile's valid tokens only, so a one-token tile has b = 0 and its
    weighted summary is that token; every tile's biased pooled exponential equals
    the mean token exponential summed directly; the anchor is the mean of the video
    queries alone."""
    w = SINK_OFF_PARTIAL
    x = make_inputs(w)
    geom = geom_of(w)
    tiles = _all_tiles(w)
    assert [len(t) for t in tiles[:3]] == [64, 1, 30]
    s = 1.0 / math.sqrt(D)
    Q, K, V = (as_f64(x[n][0, :, 0]) for n in "qkv")
    q_a = Q[np.concatenate(video_cube_tokens(w))].mean(axis=0)
    kmean = _pool_all(K, w)
    cand = list(range(len(tiles)))
    b, qa = O.logmass_bias(Q, K, geom, s, cand)
    assert np.abs(qa - q_a).max() < 1e-14
    assert len(b) == len(tiles)
    assert abs(b[1]) < 1e-15, f"one-token tile bias {b[1]}"
    for j, toks in enumerate(tiles):
        lhs = math.exp(s * float(q_a @ kmean[j]) + b[j])
        rhs = math.fsum(math.exp(s * float(q_a @ K[t])) for t in toks) / len(toks)
        assert abs(lhs - rhs) <= 1e-12 * rhs, (j, lhs, rhs)
    kt, vt, bw, _ = O.weighted_summaries(Q, K, V, geom, s, cand)
    assert np.abs(kt[1] - K[tiles[1][0]]).max() < 1e-15 and np.abs(vt[1] - V[tiles[1][0]]).max() < 1e-15
    assert abs(bw[1]) < 1e-15
    for j, toks in enumerate(tiles):
        v_ref = torch_sdpa(q_a[None, :], K[toks], V[toks])[0]
        assert np.abs(vt[j] - v_ref).max() < 1e-12 * (1 + np.abs(v_ref).max()), j
    # the forward uses these over all Tq tiles
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, SINK_OFF, coarse=COARSE_MEAN_LOGMASS,
                         want_intermediates=True)
    S_ref = _pool_all(Q, w) @ kmean.T * s + b[None, :]
    assert np.abs(inter[(0, 0)]["S"] - S_ref).max() < 1e-12


def check_sink_off_no_prefix():
    """With no conditioning segment there is nothing to protect: sink off and
    exact_kv give the same output."""
    w = Workload("nopre", 2, (), (4, 8, 12), 25.0, SINK_OFF, seed=73, recipe="scaled")
    x = make_inputs(w)
    o_off, _ = O.forward(x, w.segments(), w.grid, w.keep, SINK_OFF)
    o_kv, _ = O.forward(x, w.segments(), w.grid, w.keep, SINK_EXACT_KV)
    assert np.array_equal(o_off, o_kv)
    o_off, _ = O.forward(x, w.segments(), w.grid, 0.0, SINK_OFF, select=SELECT_TAU, tau=0.5)
    o_kv, _ = O.forward(x, w.segments(), w.grid, 0.0, SINK_EXACT_KV, select=SELECT_TAU, tau=0.5)
    assert np.array_equal(o_off, o_kv)


# ---------------------------------------------------------------- P-11 extra tokens
# [BSA-es], schedule paragraph: extra_tokens adds the best-scoring single tokens
# beyond the selected blocks.  Reading: scored with the row's pooled query, like the
# coarse branch, over the valid tokens outside the listed tiles; ties to the lower
# token index.
EXTRA_W = Workload("extra", 2, ((SEG_TEXT, 100), (SEG_REF_AUDIO, 30)), (4, 8, 12), 25.0,
                   SINK_EXACT_KV, seed=91, recipe="scaled")


def check_extra_dense():
    """With more extra tokens than there are tokens, every sparse row sees every token:
    no gate gives plain dense attention, for top-k and for tau."""
    w = EXTRA_W
    x = make_inputs(w, with_gate=False)
    for sel, tau in ((SELECT_TOPK, 0.0), (SELECT_TAU, 1.5)):
        out, _ = O.forward(x, w.segments(), w.grid, w.keep, w.sink, select=sel, tau=tau,
                           extra_tokens=10 ** 6)
        for h in range(w.heads):
            ref = torch_sdpa(as_f64(x["q"][0, :, h]), as_f64(x["k"][0, :, h]), as_f64(x["v"][0, :, h]))
            assert np.abs(out[0, :, h] - ref).max() < 1e-12, (sel, h)


def _check_extra_choice(w: Workload, x, n_extra: int, sink: int):
    tiles = _all_tiles(w)
    out, inter = O.forward(x, w.segments(), w.grid, w.keep, sink, want_intermediates=True,
                           extra_tokens=n_extra)
    sparse, dense = O.row_classes(geom_of(w), sink)
    ties = 0
    for h in range(w.heads):
        Q, K, V, G = (as_f64(x[n][0, :, h]) for n in "qkvg")
        qall = _pool_all(Q, w)
        it = inter[(0, h)]
        assert set(it["extras"]) == set(sparse)
        for i in sparse:
            listed = np.concatenate([tiles[t] for t in it["lists"][i]]) if len(it["lists"][i]) else \
                np.zeros(0, np.int64)
            elig = np.setdiff1d(np.arange(w.n_tokens), listed)
            X = np.asarray(it["extras"][i])
            assert len(X) == min(n_extra, len(elig)), (h, i, len(X))
            assert np.all(np.diff(X) > 0) and np.isin(X, elig).all(), (h, i)
            z = K[elig] @ qall[i] / math.sqrt(D)
            chosen = np.isin(elig, X)
            if chosen.any() and (~chosen).any():
                zmin, zmax = z[chosen].min(), z[~chosen].max()
                assert zmin >= zmax, (h, i, zmin, zmax)
                if zmin == zmax:  # a tie at the boundary goes to the lower token
                    assert elig[chosen][z[chosen] == zmin].max() < elig[~chosen][z[~chosen] == zmax].min()
                    ties += 1
            keys = np.concatenate([listed, X]).astype(np.int64)
            ref = torch_sdpa(Q[tiles[i]], K[keys], V[keys])
            got = out[0, tiles[i], h] - G[tiles[i]] * it["Oc"][it["sparse_rows"].index(i)][None, :]
            assert np.abs(got - ref).max() < 1e-12, (h, i)
        for i in dense:
            assert i not in it["extras"]
    return ties


def check_extra_choice():
    """The chosen extra tokens are the best-scoring eligible ones (independent pooling,
    a matmul and comparisons, not a sort), none in a listed tile, and the output is
    torch's sdpa over the listed tokens plus them; dense rows take none."""
    w = EXTRA_W
    x = make_inputs(w, with_gate=True)
    _check_extra_choice(w, x, 20, SINK_EXACT_KV)
    _check_extra_choice(w, x, 7, SINK_OFF)
    _check_extra_choice(w, x, 64, SINK_EXACT_KV_AND_ROWS)


def check_extra_ties():
    """One token of every video tile holds the same key, aligned with the mean query so it
    out-scores every other token: its copies outside the listed tiles tie for every row,
    and the lower token indices must win."""
    w = Workload("extra_tie", 1, EXTRA_W.prefix, EXTRA_W.grid, EXTRA_W.keep, SINK_EXACT_KV,
                 seed=92, recipe="offset")
    x = make_inputs(w)
    geom = geom_of(w)
    mu = as_f64(x["q"][0, :, 0]).mean(axis=0)
    key = f32_to_bf16_bits((3.0 * math.sqrt(D) * mu / np.linalg.norm(mu)).astype(np.float32))
    k = x["k"].copy()
    for t in range(geom.n_prefix, geom.n_tiles):
        k[0, geom.tiles[t][5], 0] = key
    x = dict(x, k=k)
    ties = _check_extra_choice(w, x, 3, SINK_EXACT_KV)
    assert ties == len(geom.tiles), f"expected a boundary tie on every row, got {ties}"


def check_extra_zero():
    """extra_tokens = 0 is the plain method."""
    w = EXTRA_W
    x = make_inputs(w)
    a, _ = O.forward(x, w.segments(), w.grid, w.keep, w.sink, extra_tokens=0)
    b, _ = O.forward(x, w.segments(), w.grid, w.keep, w.sink)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- Spark-Reblock
# [SPK-es] "Que cambia Spark-Attn", Spark-Reblock item.  The pins below use float64
# arrays handed straight to reblock_geometry (no bf16 rounding needed).
RB_W = Workload("rb", 2, ((SEG_TEXT, 100), (SEG_REF_AUDIO, 30)), (8, 8, 12), 25.0, SINK_EXACT_KV,
                seed=41, recipe="offset")       # 12 video tiles: groups of 3 occur


def _rb_geom(w: Workload):
    return O.map_geometry(w.segments(), *w.grid)


def _video_ids(w: Workload):
    vstart = [s0 for s0, n, kd in w.segments() if kd == SEG_VIDEO][0]
    return vstart + np.arange(w.n_video)


def _leaf_sets(g):
    return [frozenset(t.tolist()) for t in g.tiles[g.n_prefix:]]


def check_reblock_partition():
    """The leaves partition the video tokens into tiles of exactly 64, ascending inside a
    leaf; the prefix tiles are the fixed geometry's (segment-pure); a forward with reblock
    reports each head's own partition."""
    w = RB_W
    x = make_inputs(w)
    base = _rb_geom(w)
    _, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, reblock=True, want_intermediates=True,
                         fine=False)
    vids = _video_ids(w)
    seen = []
    for (b, h), it in inter.items():
        g = it["geom"]
        assert g.n_video == base.n_video and g.n_prefix == base.n_prefix
        for i in range(base.n_prefix):
            assert np.array_equal(g.tiles[i], base.tiles[i]), f"h{h} prefix tile {i} changed"
        leaves = g.tiles[g.n_prefix:]
        assert all(len(t) == 64 and np.all(np.diff(t) > 0) for t in leaves)
        assert np.array_equal(np.sort(np.concatenate(leaves)), vids), f"h{h}: leaves do not partition the video"
        seen.append(_leaf_sets(g))
    assert seen[0] != seen[1], "the partition must follow the head's own inputs"
    assert seen[0] != _leaf_sets(base), "reblock left the fixed cubes in place"


def _planted(rng, n_tok, centers, noise):
    """Queries around planted centres: token i of a random order belongs to cluster i // 64."""
    perm = rng.permutation(n_tok)
    q = np.empty((n_tok, D))
    for c, cen in enumerate(centers):
        ids = perm[64 * c:64 * (c + 1)]
        q[ids] = cen[None, :] + noise * rng.standard_normal((64, D))
    return q, [frozenset(perm[64 * c:64 * (c + 1)].tolist()) for c in range(len(centers))]


def _keys_with_moment(rng, n_tok, scales):
    """Keys whose second moment is exactly diag(scales^2): orthonormal columns, rescaled."""
    Qm, _ = np.linalg.qr(rng.standard_normal((n_tok, D)))
    return Qm * math.sqrt(n_tok) * np.asarray(scales)[None, :]


def _embed(w: Workload, qv, kv):
    """Full-length Q, K with the video rows given and random prefix rows."""
    rng = np.random.default_rng(5)
    Q = rng.standard_normal((w.n_tokens, D))
    K = rng.standard_normal((w.n_tokens, D))
    vids = _video_ids(w)
    Q[vids], K[vids] = qv, kv
    return Q, K


def check_reblock_planted_tree():
    """Queries planted on a binary tree of 16 clusters (offsets 27, 9, 3, 1 along four
    axes, small noise) with an isotropic key moment: the leaves are the 16 clusters."""
    w = Workload("rb16", 1, ((SEG_TEXT, 64),), (4, 16, 16), 25.0, SINK_EXACT_KV, seed=1)
    rng = np.random.default_rng(42)
    cents = []
    for c in range(16):
        v = np.zeros(D)
        v[0] = 100.0
        for lvl, amp in enumerate((27.0, 9.0, 3.0, 1.0)):
            v[1 + lvl] = amp * (1 if (c >> (3 - lvl)) & 1 else -1)
        cents.append(v)
    qv, groups = _planted(rng, w.n_video, cents, 0.05)
    kv = _keys_with_moment(rng, w.n_video, np.ones(D))
    Q, K = _embed(w, qv, kv)
    g = O.reblock_geometry(Q, K, _rb_geom(w))
    vids = _video_ids(w)
    want = {frozenset((vids[list(gr)]).tolist()) for gr in groups}
    assert set(_leaf_sets(g)) == want, "planted clusters not recovered"


def check_reblock_metric():
    """The metric is the keys' second moment: clusters split by 5 along e1 and by 1 along
    e2, with key scales 0.1 (e1) and 10 (e2).  In the metric, e2 separates them by 10 and
    e1 by 0.5, so the root split follows e2; in plain (or query-moment) geometry it would
    follow e1."""
    w = Workload("rb4", 1, ((SEG_TEXT, 64),), (4, 4, 16), 25.0, SINK_EXACT_KV, seed=1)
    rng = np.random.default_rng(43)
    cents = []
    for s1 in (-1, 1):
        for s2 in (-1, 1):
            v = np.zeros(D)
            v[0], v[1], v[2] = 10.0, 5.0 * s1, 1.0 * s2
            cents.append(v)
    qv, groups = _planted(rng, w.n_video, cents, 0.01)
    scales = np.ones(D)
    scales[1], scales[2] = 0.1, 10.0
    kv = _keys_with_moment(rng, w.n_video, scales)
    Q, K = _embed(w, qv, kv)
    g = O.reblock_geometry(Q, K, _rb_geom(w))
    vids = _video_ids(w)
    leaves = _leaf_sets(g)
    root_left = leaves[0] | leaves[1]
    e2_neg = frozenset(vids[list(groups[0] | groups[2])].tolist())   # centres with s2 = -1
    e2_pos = frozenset(vids[list(groups[1] | groups[3])].tolist())
    assert root_left in (e2_neg, e2_pos), "the root split must follow the key metric (e2)"
    assert set(leaves) == {frozenset(vids[list(gr)].tolist()) for gr in groups}


def check_reblock_vs_eigh():
    """One split with a dominant axis, against an independent formulation: explicit
    whitening with the Cholesky factor of M, the top eigenvector of the centred
    covariance (numpy eigh), and a sort by (projection, token)."""
    w = Workload("rb2", 1, ((SEG_TEXT, 64),), (4, 4, 8), 25.0, SINK_EXACT_KV, seed=1)
    rng = np.random.default_rng(44)
    n = w.n_video
    u = rng.standard_normal(D)
    u[0] = 0.0
    u /= np.linalg.norm(u)
    qv = 10.0 * np.eye(D)[0][None, :] + 3.0 * rng.standard_normal((n, 1)) * u[None, :] \
        + 0.15 * rng.standard_normal((n, D))
    kv = _keys_with_moment(rng, n, rng.uniform(0.5, 2.0, size=D))   # anisotropic, well conditioned
    Q, K = _embed(w, qv, kv)
    g = O.reblock_geometry(Q, K, _rb_geom(w))
    vids = _video_ids(w)
    M = kv.T @ kv / n
    L = np.linalg.cholesky(M)
    phi = qv @ L
    phi /= np.linalg.norm(phi, axis=1, keepdims=True)
    C = np.cov(phi.T, bias=True)
    evals, evecs = np.linalg.eigh(C)
    top = evecs[:, -1]
    assert evals[-1] > 20 * evals[-2]
    proj = phi @ top
    srt = np.sort(proj)
    assert srt[64] - srt[63] > 1e-6, "pick a seed without a near tie at the median"
    lower = frozenset(vids[np.argsort(proj)[:64]].tolist())
    upper = frozenset(vids[np.argsort(proj)[64:]].tolist())
    leaves = _leaf_sets(g)
    assert set(leaves) == {lower, upper}, "split differs from the principal axis"


def check_reblock_invariance():
    """Cosine similarity in the key metric: scaling each query by its own positive factor,
    or all keys by one factor, leaves the leaves unchanged; relabelling the video tokens
    (Q and K rows permuted together) relabels the leaves and keeps their order."""
    w = RB_W
    x = make_inputs(w)
    Q, K = as_f64(x["q"][0, :, 0]), as_f64(x["k"][0, :, 0])
    base = _rb_geom(w)
    ref = _leaf_sets(O.reblock_geometry(Q, K, base))
    rng = np.random.default_rng(45)
    Q2 = Q * rng.uniform(0.5, 2.0, size=(Q.shape[0], 1))
    assert _leaf_sets(O.reblock_geometry(Q2, 3.0 * K, base)) == ref
    vids = _video_ids(w)
    perm = rng.permutation(len(vids))
    Q3, K3 = Q.copy(), K.copy()
    Q3[vids[perm]], K3[vids[perm]] = Q[vids], K[vids]     # token vids[i] moves to vids[perm[i]]
    new_of = dict(zip(vids.tolist(), vids[perm].tolist()))
    got = _leaf_sets(O.reblock_geometry(Q3, K3, base))
    assert got == [frozenset(new_of[t] for t in leaf) for leaf in ref]


def check_reblock_ties():
    """Every video query equal: every projection ties, so each split keeps the lower token
    ids on the left and the leaves are the video tokens in ascending runs of 64."""
    w = RB_W
    x = make_inputs(w)
    Q, K = as_f64(x["q"][0, :, 0]), as_f64(x["k"][0, :, 0])
    vids = _video_ids(w)
    Q[vids] = Q[vids[0]]
    g = O.reblock_geometry(Q, K, _rb_geom(w))
    for j, leaf in enumerate(g.tiles[g.n_prefix:]):
        assert np.array_equal(leaf, vids[64 * j:64 * (j + 1)]), f"leaf {j}"


def check_reblock_split_sizes():
    """Three planted clusters (three tiles) A = -4 e1, B = e1 + 2 e3, C = 3 e1 - 2 e3 (plus a
    shared 20 e0): the root axis is mostly e1 with A lowest, so the left child is A alone
    (floor(3/2) = 1 tile) and the right child {B, C} splits along its own axis, C first;
    the leaves in tree order are A, C, B.  (A left child of ceil(3/2) tiles would be {A, B},
    giving A, B, C; the upper half on the left would put C first.)"""
    w = Workload("rb3", 1, ((SEG_TEXT, 64),), (4, 4, 12), 25.0, SINK_EXACT_KV, seed=1)
    rng = np.random.default_rng(46)
    cents = []
    for c1, c3 in ((-4.0, 0.0), (1.0, 2.0), (3.0, -2.0)):
        v = np.zeros(D)
        v[0], v[1], v[3] = 20.0, c1, c3
        cents.append(v)
    qv, groups = _planted(rng, w.n_video, cents, 0.01)
    kv = _keys_with_moment(rng, w.n_video, np.ones(D))
    Q, K = _embed(w, qv, kv)
    g = O.reblock_geometry(Q, K, _rb_geom(w))
    vids = _video_ids(w)
    want = [frozenset(vids[list(groups[i])].tolist()) for i in (0, 2, 1)]
    assert _leaf_sets(g) == want, "leaves must be A, C, B"


def check_reblock_forward():
    """A forward on the reblocked tiles, rebuilt from independent pieces: pooled means of
    each leaf, the coarse branch as torch sdpa on them, brute-force top-k, and every row's
    output as sdpa over its listed tiles plus the gated coarse term."""
    w = Workload("rbf", 2, ((SEG_TEXT, 64), (SEG_REF_AUDIO, 40)), (8, 8, 8), 25.0, SINK_EXACT_KV,
                 seed=47, recipe="smooth")
    x = make_inputs(w, with_gate=True)
    out, inter = O.forward(x, w.segments(), w.grid, w.keep, w.sink, reblock=True, want_intermediates=True)
    for h in range(w.heads):
        Q, K, V, G = (as_f64(x[n][0, :, h]) for n in "qkvg")
        g = inter[(0, h)]["geom"]
        P, tiles = g.n_prefix, g.tiles
        pool = lambda X, ts: np.stack([X[t].sum(axis=0) / len(t) for t in ts])
        qall = pool(Q, tiles)
        kv, vv = pool(K, tiles[P:]), pool(V, tiles[P:])
        S = qall @ kv.T / math.sqrt(D)
        oc = torch_sdpa(qall, kv, vv)
        k = O.keep_count(w.keep, g.n_video)
        for i in range(len(tiles)):
            pick = list(range(P)) + [P + j for j in brute_topk(list(S[i]), k)] if k < 8 else None
            if pick is None:
                order = sorted(range(g.n_video), key=lambda j: (-S[i, j], j))[:k]
                pick = list(range(P)) + sorted(P + j for j in order)
            assert list(inter[(0, h)]["lists"][i]) == pick, f"h{h} row {i}"
            keys = np.concatenate([tiles[t] for t in pick])
            ref = torch_sdpa(Q[tiles[i]], K[keys], V[keys]) + G[tiles[i]] * oc[i][None, :]
            assert np.abs(out[0, tiles[i], h] - ref).max() < 1e-12, f"h{h} row {i} output"


ALL_CHECKS = [
    ("geometry", lambda: (check_geometry(SMALL), check_geometry(SMALL_VIDEO_FIRST),
                          check_geometry(GEOM_3D))),
    ("keep_counts", check_keep_counts),
    ("dense_equivalence", lambda: (check_dense_equivalence(SMALL), check_dense_equivalence(SMALL_VIDEO_FIRST))),
    ("dense_rows_and_gate", lambda: check_dense_rows_and_gate(SMALL)),
    ("pooling", lambda: check_pooling(SMALL)),
    ("coarse_mean", lambda: check_coarse(SMALL, COARSE_MEAN)),
    ("coarse_logmass", lambda: check_coarse(SMALL_VIDEO_FIRST, COARSE_MEAN_LOGMASS)),
    ("prefix_exempt", lambda: (check_prefix_exempt(SMALL), check_prefix_exempt(
        Workload("pe", 1, SMALL.prefix, SMALL.grid, 10.0, SINK_EXACT_KV_AND_ROWS, seed=9)))),
    ("topk_bruteforce", check_topk_bruteforce),
    ("topk_ties", check_topk_ties_in_forward),
    ("tau_threshold", check_tau_threshold),
    ("tau_limits", lambda: check_tau_limits(SMALL)),
    ("tau_dense_rows", check_tau_dense_rows),
    ("tau_fractions", check_tau_fractions),
    ("logmass", check_logmass),
    ("weighted_summaries", check_weighted_summaries),
    ("combine", lambda: check_combine(SMALL)),
    ("metamorphic", lambda: check_metamorphic(SMALL_VIDEO_FIRST)),
    ("prefix_permutation", check_prefix_permutation),
    ("sink_off_dense", lambda: (check_sink_off_dense(SINK_OFF_W), check_sink_off_dense(SINK_OFF_PARTIAL))),
    ("sink_off_selection", lambda: check_sink_off_selection(SINK_OFF_W, 3)),
    ("sink_off_tau", lambda: (check_sink_off_tau(SINK_OFF_W, 1.0), check_sink_off_tau(SINK_OFF_PARTIAL, 0.5))),
    ("sink_off_logmass", check_sink_off_logmass),
    ("sink_off_no_prefix", check_sink_off_no_prefix),
    ("extra_dense", check_extra_dense),
    ("extra_choice", check_extra_choice),
    ("extra_ties", check_extra_ties),
    ("extra_zero", check_extra_zero),
    ("reblock_partition", check_reblock_partition),
    ("reblock_planted_tree", check_reblock_planted_tree),
    ("reblock_metric", check_reblock_metric),
    ("reblock_vs_eigh", check_reblock_vs_eigh),
    ("reblock_invariance", check_reblock_invariance),
    ("reblock_ties", check_reblock_ties),
    ("reblock_split_sizes", check_reblock_split_sizes),
    ("reblock_forward", check_reblock_forward),
]
