"""Compare the HIP path's results with the fp64 oracle.

Selections: per (batch, head, sparse query tile) let S(k) and S(k+1) be the
oracle's k-th and (k+1)-th largest coarse logits.  Where S(k) - S(k+1) > GAP
the GPU list must equal the oracle's.  Elsewhere the GPU list must be a
valid top-k within GAP (size P + k, every protected prefix tile, every kept
logit >= S(k) - GAP, every dropped logit <= S(k+1) + GAP; with sink off no
tile is protected and P is 0 here); the oracle then adopts
the GPU's list for that row before the outputs are compared.  Tau mode: the
GPU must agree wherever |S - thr| > GAP and its choice is adopted elsewhere.
Extra tokens: the same rule on the token scores z of the row's eligible tokens
(given the row's list): exact where z(E) - z(E+1) > GAP, else a valid top-E
within GAP, adopted.

Outputs, over every valid element produced, against the unrounded fp64 oracle:
|O_gpu - O_ref| <= 2e-2 (the contract's flat bound) and
||O_gpu - O_ref||_2 / ||O_ref||_2 <= 1e-2.  Also reported and bounded by the same
2e-2: the error beyond h, exactly half a bf16 ulp at the larger of |O_gpu| and
|O_ref| (2^(e-8) for a magnitude in [2^e, 2^(e+1))).  The output is bf16, so its
own rounding moves an element by up to h whatever the arithmetic (0.0156 for |O|
in [4, 8), 0.031 from 8 on); the excess beyond h is what the arithmetic (bf16
inputs, bf16 probabilities in the PV product, fp32 accumulation in any order)
contributes.  ``max_abs`` is the raw largest error.
"""
from __future__ import annotations

import numpy as np

from oracle import vsa_oracle as O

GAP = 1e-4
TOL_ABS = 2e-2
TOL_REL = 1e-2


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x| (8 significant bits): 2^(e-8) for |x| in [2^e, 2^(e+1)); 0 at 0."""
    _, e = np.frexp(np.abs(x))          # |x| = m 2^e with m in [0.5, 1)
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def bits_to_f64(b):
    return O.bf16_bits_to_f64(b)


def gpu_results_to_numpy(plan, ws, o, fields=("scores", "lists", "counts", "qbar", "kbar", "vbar",
                                              "bias", "ocoarse", "thr", "anchor", "xtok", "xcnt")):
    """Copy the output and the workspace intermediates to host numpy arrays."""
    import torch
    from block_sparse_video_geometry_amd import debug_tensor
    res = {"o": o.view(torch.int16).cpu().numpy().view(np.uint16)}
    for f in fields:
        if f in ("xtok", "xcnt") and plan.desc.options.extra_tokens == 0:
            continue
        res[f] = debug_tensor(plan, ws, f).cpu().numpy()
    return res


def check_parity(w, x, gpu, heads=None, rows=None, gap=GAP, tol_abs=TOL_ABS, tol_rel=TOL_REL,
                 check_intermediates=True, geoms=None):
    """Raise AssertionError on a mismatch; return a report dict.

    w: workload, x: input bit arrays, gpu: dict from gpu_results_to_numpy.
    heads: (b, h) pairs to check (None = all); rows: query tile ids (None = all).
    geoms: {(b, h): Geometry} per-head tiles (adaptive partitions), else the fixed tiles."""
    geom = O.map_geometry(w.segments(), *w.grid)
    fixed_geom = geom
    sparse, dense = O.row_classes(geom, w.sink)
    n_dense = len(dense)
    P = 0 if w.sink == O.SINK_OFF else geom.n_prefix   # protected (always listed) tiles
    cand = O.key_candidates(geom, w.sink)
    c0, nc = cand[0], len(cand)                        # candidates are tile ids c0 .. c0 + nc - 1
    B, N, H, D = x["q"].shape
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    E = getattr(w, "extra", 0)
    rep = dict(rows=0, exact_rows=0, adopted_rows=0, extra_exact=0, extra_adopted=0, max_abs=0.0,
               max_excess=0.0, err2=0.0, ref2=0.0,
               max_s_err=0.0, max_pool_err=0.0, max_oc_err=0.0, max_bias_err=0.0, s_mag=1.0,
               bias_mag=1.0)
    g_all = x.get("g")
    for b, h in heads:
        geom = geoms[(b, h)] if geoms is not None else fixed_geom
        Q, K, V = (bits_to_f64(x[n][b, :, h]) for n in "qkv")
        G = bits_to_f64(g_all[b, :, h]) if g_all is not None else None
        _, it = O.forward_head(Q, K, V, G, geom, w.keep, w.sink, w.select, w.coarse, w.tau,
                               rows=rows, want_intermediates=True, extra_tokens=E)
        need = it["sparse_rows"]
        S_ref = it["S"]
        if S_ref.size:
            rep["s_mag"] = max(rep["s_mag"], float(np.abs(S_ref).max()))
        rep["bias_mag"] = max(rep["bias_mag"], float(np.abs(it["bias"]).max()))
        if check_intermediates:
            kb = gpu["kbar"][b, h].astype(np.float64)
            vb = gpu["vbar"][b, h].astype(np.float64)
            rep["max_pool_err"] = max(rep["max_pool_err"], np.abs(kb - it["Kbar"]).max(),
                                      np.abs(vb - it["Vbar"]).max())
            if need:
                qb = gpu["qbar"][b, h][np.asarray(need)].astype(np.float64)
                rep["max_pool_err"] = max(rep["max_pool_err"], np.abs(qb - it["Qbar"]).max())
                oc = gpu["ocoarse"][b, h][np.asarray(need) - n_dense].astype(np.float64)
                rep["max_oc_err"] = max(rep["max_oc_err"], np.abs(oc - it["Oc"]).max())
            rep["max_bias_err"] = max(rep["max_bias_err"],
                                      np.abs(gpu["bias"][b, h].astype(np.float64) - it["bias"]).max())
        override = {}
        for n_i, i in enumerate(need):
            if rows is not None and i not in set(rows):
                continue
            s = i - n_dense
            srow_ref = S_ref[n_i]
            srow_gpu = gpu["scores"][b, h, s].astype(np.float64)
            rep["max_s_err"] = max(rep["max_s_err"], np.abs(srow_gpu - srow_ref).max())
            cnt = int(gpu["counts"][b, h, s])
            glist = gpu["lists"][b, h, s, :cnt].astype(np.int64)
            olist = it["lists"][i]
            assert list(glist[:P]) == list(range(P)), f"(b{b},h{h},tile {i}) prefix tiles missing"
            gvid = glist[P:] - c0
            assert np.all(np.diff(gvid) > 0), f"(b{b},h{h},tile {i}) list not ascending"
            assert gvid.size == 0 or (gvid.min() >= 0 and gvid.max() < nc)
            if w.select == O.SELECT_TOPK:
                k = it["k"]
                assert cnt == P + k, f"(b{b},h{h},tile {i}) count {cnt} != {P + k}"
                srt = np.sort(srow_ref)[::-1]
                sk = srt[k - 1]
                sk1 = srt[k] if k < len(srt) else -np.inf
                if sk - sk1 > gap:
                    assert np.array_equal(glist, olist), \
                        f"(b{b},h{h},tile {i}) selection differs at gap {sk - sk1:.3g}"
                    rep["exact_rows"] += 1
                else:
                    sel = np.zeros(nc, bool)
                    sel[gvid] = True
                    assert np.all(srow_ref[sel] >= sk - gap), f"(b{b},h{h},tile {i}) weak pick"
                    assert np.all(srow_ref[~sel] <= sk1 + gap), f"(b{b},h{h},tile {i}) weak drop"
                    override[i] = glist
                    rep["adopted_rows"] += 1
            else:
                thr = it["thr"]
                sel = np.zeros(nc, bool)
                sel[gvid] = True
                clear = np.abs(srow_ref - thr) > gap
                assert np.array_equal(sel[clear], (srow_ref > thr)[clear]), \
                    f"(b{b},h{h},tile {i}) tau selection differs away from the threshold"
                if np.array_equal(glist, olist):
                    rep["exact_rows"] += 1
                else:
                    override[i] = glist
                    rep["adopted_rows"] += 1
        xover = {}
        if E > 0:
            # the oracle's extra tokens given the GPU's lists
            _, it2 = O.forward_head(Q, K, V, G, geom, w.keep, w.sink, w.select, w.coarse, w.tau,
                                    rows=rows, list_override=override or None, want_intermediates=True,
                                    extra_tokens=E)
            scale = O.softmax_scale(D)
            for n_i, i in enumerate(it2["sparse_rows"]):
                if rows is not None and i not in set(rows):
                    continue
                s = i - n_dense
                xc = int(gpu["xcnt"][b, h, s])
                gx = gpu["xtok"][b, h, s, :xc].astype(np.int64)
                ox = it2["extras"][i]
                listed = [geom.tiles[t] for t in it2["lists"][i]]
                listed = np.concatenate(listed) if listed else np.zeros(0, np.int64)
                elig = np.setdiff1d(np.concatenate(geom.tiles), listed)
                assert xc == min(E, len(elig)), f"(b{b},h{h},tile {i}) {xc} extra tokens, expected {min(E, len(elig))}"
                assert np.all(np.diff(gx) > 0) and np.isin(gx, elig).all(), \
                    f"(b{b},h{h},tile {i}) extra tokens not ascending or not eligible"
                z = scale * (K[elig] @ it2["Qbar"][n_i])
                zs = np.sort(z)[::-1]
                ze = zs[xc - 1] if xc > 0 else np.inf
                ze1 = zs[xc] if xc < len(zs) else -np.inf
                if ze - ze1 > gap:
                    assert np.array_equal(gx, ox), f"(b{b},h{h},tile {i}) extra tokens differ at gap {ze - ze1:.3g}"
                    rep["extra_exact"] += 1
                else:
                    chosen = np.isin(elig, gx)
                    assert np.all(z[chosen] >= ze - gap), f"(b{b},h{h},tile {i}) weak extra pick"
                    assert np.all(z[~chosen] <= ze1 + gap), f"(b{b},h{h},tile {i}) weak extra drop"
                    xover[i] = gx
                    rep["extra_adopted"] += 1
        Oref, _ = O.forward_head(Q, K, V, G, geom, w.keep, w.sink, w.select, w.coarse, w.tau,
                                 rows=rows, list_override=override or None, extra_tokens=E,
                                 extra_override=xover or None)
        row_ids = range(geom.n_tiles) if rows is None else rows
        toks = np.concatenate([geom.tiles[i] for i in row_ids])
        og = bits_to_f64(gpu["o"][b, toks, h])
        orf = Oref[toks]
        assert np.all(np.isfinite(og)), f"(b{b},h{h}) non-finite GPU output"
        diff = og - orf
        rep["max_abs"] = max(rep["max_abs"], float(np.abs(diff).max()))
        h_ulp = bf16_half_ulp(np.maximum(np.abs(og), np.abs(orf)))
        rep["max_excess"] = max(rep["max_excess"], float((np.abs(diff) - h_ulp).max()))
        rep["err2"] += float((diff ** 2).sum())
        rep["ref2"] += float((orf ** 2).sum())
        rep["rows"] += len(list(row_ids))
    rep["rel_l2"] = (rep["err2"] / rep["ref2"]) ** 0.5 if rep["ref2"] > 0 else 0.0
    assert rep["max_abs"] <= tol_abs, f"max abs error {rep['max_abs']:.3g} > {tol_abs}"
    assert rep["max_excess"] <= tol_abs, \
        f"error beyond half a bf16 ulp {rep['max_excess']:.3g} > {tol_abs} (max abs {rep['max_abs']:.3g})"
    assert rep["rel_l2"] <= tol_rel, f"relative L2 error {rep['rel_l2']:.3g} > {tol_rel}"
    if check_intermediates:
        # fp32 dot products of length 128 on pooled values: ~1e-6 relative to the logit size
        assert rep["max_s_err"] < 1e-5 * rep["s_mag"], f"coarse logits differ by {rep['max_s_err']:.3g}"
        assert rep["max_pool_err"] < 1e-5, f"pooled means differ by {rep['max_pool_err']:.3g}"
        assert rep["max_oc_err"] < 1e-4, f"O_coarse differs by {rep['max_oc_err']:.3g}"
        assert rep["max_bias_err"] < 1e-5 * rep["bias_mag"], \
            f"log-mass bias differs by {rep['max_bias_err']:.3g}"
    return rep


def check_lists(w, x, gpu, heads, gap=GAP):
    """Selections of every sparse row of the given (batch, head) pairs against the
    oracle (its selection only: no fine branch), with the gap rule above, plus the
    coarse logits.  Returns a report dict; raises AssertionError on a mismatch."""
    geom = O.map_geometry(w.segments(), *w.grid)
    sparse, dense = O.row_classes(geom, w.sink)
    n_dense = len(dense)
    P = 0 if w.sink == O.SINK_OFF else geom.n_prefix
    cand = O.key_candidates(geom, w.sink)
    c0, nc = cand[0], len(cand)
    rep = dict(rows=0, exact_rows=0, adopted_rows=0, max_s_err=0.0, s_mag=1.0)
    for b, h in heads:
        Q, K, V = (bits_to_f64(x[n][b, :, h]) for n in "qkv")
        _, it = O.forward_head(Q, K, V, None, geom, w.keep, w.sink, w.select, w.coarse, w.tau,
                               rows=sparse, want_intermediates=True, fine=False)
        S_ref = it["S"]
        rep["s_mag"] = max(rep["s_mag"], float(np.abs(S_ref).max()))
        for n_i, i in enumerate(it["sparse_rows"]):
            s = i - n_dense
            srow_ref = S_ref[n_i]
            rep["max_s_err"] = max(rep["max_s_err"],
                                   float(np.abs(gpu["scores"][b, h, s].astype(np.float64) - srow_ref).max()))
            cnt = int(gpu["counts"][b, h, s])
            glist = gpu["lists"][b, h, s, :cnt].astype(np.int64)
            olist = it["lists"][i]
            assert list(glist[:P]) == list(range(P)), f"(b{b},h{h},tile {i}) prefix tiles missing"
            gvid = glist[P:] - c0
            assert np.all(np.diff(gvid) > 0), f"(b{b},h{h},tile {i}) list not ascending"
            assert gvid.size == 0 or (gvid.min() >= 0 and gvid.max() < nc)
            sel = np.zeros(nc, bool)
            sel[gvid] = True
            if w.select == O.SELECT_TOPK:
                k = it["k"]
                assert cnt == P + k, f"(b{b},h{h},tile {i}) count {cnt} != {P + k}"
                srt = np.sort(srow_ref)[::-1]
                sk = srt[k - 1]
                sk1 = srt[k] if k < len(srt) else -np.inf
                if sk - sk1 > gap:
                    assert np.array_equal(glist, olist), \
                        f"(b{b},h{h},tile {i}) selection differs at gap {sk - sk1:.3g}"
                    rep["exact_rows"] += 1
                else:
                    assert np.all(srow_ref[sel] >= sk - gap), f"(b{b},h{h},tile {i}) weak pick"
                    assert np.all(srow_ref[~sel] <= sk1 + gap), f"(b{b},h{h},tile {i}) weak drop"
                    rep["adopted_rows"] += 1
            else:
                thr = it["thr"]
                clear = np.abs(srow_ref - thr) > gap
                assert np.array_equal(sel[clear], (srow_ref > thr)[clear]), \
                    f"(b{b},h{h},tile {i}) tau selection differs away from the threshold"
                if np.array_equal(glist, olist):
                    rep["exact_rows"] += 1
                else:
                    rep["adopted_rows"] += 1
            rep["rows"] += 1
    assert rep["max_s_err"] < 1e-5 * rep["s_mag"], f"coarse logits differ by {rep['max_s_err']:.3g}"
    return rep


def check_reblock_tiles(w, x, gpu_tiles, heads, gap=GAP):
    """The GPU's adaptive tiles against the oracle's tree, node by node from the root.

    At a node the oracle sorts its tokens by projection; with p(k), p(k+1) the k-th and
    (k+1)-th smallest (k = 64 floor(m/2)), where p(k+1) - p(k) > gap the GPU's left child
    (the union of its leaves in the left tile range) must equal the oracle's exactly.
    Elsewhere the GPU's split must be valid within gap (left projections <= p(k+1) + gap,
    right ones >= p(k) - gap) and the oracle adopts it.  Returns ({(b, h): the oracle's
    geometry with the adoptions}, report)."""
    base = O.map_geometry(w.segments(), *w.grid)
    rep = dict(nodes=0, exact_nodes=0, adopted_nodes=0, min_gap=np.inf)
    geoms = {}
    for b, h in heads:
        Q, K = bits_to_f64(x["q"][b, :, h]), bits_to_f64(x["k"][b, :, h])
        tiles = np.asarray(gpu_tiles[b, h], dtype=np.int64)

        def hook(t0, m, toks, p, left, right, tiles=tiles, b=b, h=h):
            ml = m // 2
            gl = np.sort(tiles[t0:t0 + ml].ravel())
            gr = np.sort(tiles[t0 + ml:t0 + m].ravel())
            assert np.array_equal(np.sort(np.concatenate([gl, gr])), toks), \
                f"(b{b},h{h}) node tiles [{t0},{t0 + m}): GPU tokens differ from the node's"
            srt = np.sort(p)
            kl = 64 * ml
            pk, pk1 = srt[kl - 1], srt[kl]
            rep["nodes"] += 1
            rep["min_gap"] = min(rep["min_gap"], float(pk1 - pk))
            if pk1 - pk > gap:
                assert np.array_equal(gl, left), \
                    f"(b{b},h{h}) node [{t0},{t0 + m}) split differs at gap {pk1 - pk:.3g}"
                rep["exact_nodes"] += 1
                return left, right
            pos = {int(t): i for i, t in enumerate(toks)}
            pl = p[[pos[int(t)] for t in gl]]
            pr = p[[pos[int(t)] for t in gr]]
            assert np.all(pl <= pk1 + gap) and np.all(pr >= pk - gap), \
                f"(b{b},h{h}) node [{t0},{t0 + m}) GPU split invalid within {gap}"
            rep["adopted_nodes"] += 1
            return gl, gr

        gh = O.reblock_geometry(Q, K, base, hook)
        for j in range(base.n_video):
            assert np.array_equal(gh.tiles[base.n_prefix + j], tiles[j]), f"(b{b},h{h}) leaf {j}"
        geoms[(b, h)] = gh
    return geoms, rep
