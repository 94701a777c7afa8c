"""Plant plausible mistakes in the oracle (on the CPU) and check a pin fails.

Each mutation replaces one oracle function with a wrong variant; the named
pin must then raise.  This shows the pins can tell a right oracle from a
plausibly wrong one, so agreement with them means something.
"""
import math

import numpy as np
import pytest

import oracle_pins as P
from oracle import vsa_oracle as O

_orig = {n: getattr(O, n) for n in ("softmax_scale", "map_geometry", "select_topk", "row_list",
                                      "logmass_bias", "coarse_branch", "tau_threshold",
                                      "keep_count", "pool_tiles", "fine_row", "weighted_summaries",
                                      "key_candidates", "extra_tokens_for_row", "tau_rows",
                                      "reblock_metric", "reblock_features", "principal_projection",
                                      "reblock_order", "reblock_left_tiles")}


def _geom_swapped_axes(segments, T, H, W):
    g = _orig["map_geometry"](segments, T, H, W)
    # video tiles enumerated (th, tt, tw) instead of (tt, th, tw)
    nt, nh, nw = T // 4, H // 4, W // 4
    vid = g.tiles[g.n_prefix:]
    order = [tt * nh * nw + th * nw + tw for th in range(nh) for tt in range(nt) for tw in range(nw)]
    g.tiles = g.tiles[:g.n_prefix] + [vid[o] for o in order]
    return g


def _geom_token_order(segments, T, H, W):
    g = _orig["map_geometry"](segments, T, H, W)
    # tokens inside a video tile in (dw, dh, dt) order
    perm = np.arange(64).reshape(4, 4, 4).transpose(2, 1, 0).ravel()
    g.tiles = g.tiles[:g.n_prefix] + [t[perm] for t in g.tiles[g.n_prefix:]]
    return g


def _topk_high_ties(S_row, k):
    order = sorted(range(len(S_row)), key=lambda j: (-S_row[j], -j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def _topk_smallest(S_row, k):
    order = sorted(range(len(S_row)), key=lambda j: (S_row[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def _bias_flipped(Q, K, geom, scale, cand=None):
    b, qa = _orig["logmass_bias"](Q, K, geom, scale, cand)
    return -b, qa


def _bias_no_anchor(Q, K, geom, scale, cand=None):
    return np.zeros(geom.n_video if cand is None else len(cand)), np.zeros(Q.shape[1])


def _bias_mean_over_64(Q, K, geom, scale, cand=None):
    """The mean inside the log divided by 64 instead of the tile's valid token count."""
    b, qa = _orig["logmass_bias"](Q, K, geom, scale, cand)
    ids = range(geom.n_prefix, geom.n_tiles) if cand is None else cand
    return np.array([bj + math.log(len(geom.tiles[t]) / 64.0) for bj, t in zip(b, ids)]), qa


def _off_video_only(geom, sink):
    return list(range(geom.n_prefix, geom.n_tiles))


def _row_list_always_pinned(geom, sel, sink=1):
    sel = np.asarray(sel, dtype=np.int64)
    if sink == O.SINK_OFF:
        return np.unique(np.concatenate([np.arange(geom.n_prefix, dtype=np.int64), sel]))
    return _orig["row_list"](geom, sel, sink)


def _coarse_no_bias(Qbar, Kbar, Vbar, bias, scale):
    return _orig["coarse_branch"](Qbar, Kbar, Vbar, np.zeros_like(bias), scale)


def _tau_variance(S, tau):
    vals = S.ravel()
    mu = float(np.mean(vals))
    return mu + tau * float(np.mean((vals - mu) ** 2))


def _weighted_plain_means(Q, K, V, geom, scale, cand=None):
    kt, vt, b, qa = _orig["weighted_summaries"](Q, K, V, geom, scale, cand)
    tiles = geom.tiles[geom.n_prefix:] if cand is None else [geom.tiles[t] for t in cand]
    return (np.stack([K[t].mean(axis=0) for t in tiles]), np.stack([V[t].mean(axis=0) for t in tiles]),
            b, qa)


def _weighted_unnormalized(Q, K, V, geom, scale, cand=None):
    kt, vt, b, qa = _orig["weighted_summaries"](Q, K, V, geom, scale, cand)
    tiles = geom.tiles[geom.n_prefix:] if cand is None else [geom.tiles[t] for t in cand]
    ell = [scale * (K[t] @ qa) for t in tiles]
    e = [np.exp(l - l.max()) for l in ell]
    return np.stack([ei @ K[t] for ei, t in zip(e, tiles)]), np.stack([ei @ V[t] for ei, t in zip(e, tiles)]), b, qa


def _weighted_bias_vs_mean(Q, K, V, geom, scale, cand=None):
    kt, vt, b, qa = _orig["weighted_summaries"](Q, K, V, geom, scale, cand)
    tiles = geom.tiles[geom.n_prefix:] if cand is None else [geom.tiles[t] for t in cand]
    b2 = np.array([b[j] + scale * (qa @ kt[j]) - scale * (qa @ K[t].mean(axis=0)) for j, t in enumerate(tiles)])
    return kt, vt, b2, qa


def _tau_rows_all_tiles(geom, sink):
    """The prefix query tiles counted in the tau moments although they run dense."""
    return list(range(geom.n_tiles))


def _fine_k_for_v(Q, K, V, geom, qtile, key_tiles, scale, extra=None):
    return _orig["fine_row"](Q, K, K, geom, qtile, key_tiles, scale, extra)


def _extra_ignores_list(qbar_i, K, geom, key_tiles, n_extra, scale):
    return _orig["extra_tokens_for_row"](qbar_i, K, geom, [], n_extra, scale)


def _extra_lowest(qbar_i, K, geom, key_tiles, n_extra, scale):
    return _orig["extra_tokens_for_row"](-qbar_i, K, geom, key_tiles, n_extra, scale)


def _extra_ties_high(qbar_i, K, geom, key_tiles, n_extra, scale):
    listed = set(int(t) for t in key_tiles)
    toks = np.concatenate([geom.tiles[t] for t in range(geom.n_tiles) if t not in listed])
    z = scale * (K[toks] @ qbar_i)
    order = sorted(range(len(toks)), key=lambda a: (-z[a], -toks[a]))
    return np.sort(toks[order[:n_extra]])


def _rb_identity_metric(Q, K, geom):
    return np.eye(K.shape[1])


def _rb_query_metric(Q, K, geom):
    """The queries' own second moment instead of the keys' (the wrong side)."""
    vt = np.concatenate(geom.tiles[geom.n_prefix:])
    return Q[vt].T @ Q[vt] / len(vt)


def _rb_inverse_metric(Q, K, geom):
    return np.linalg.inv(_orig["reblock_metric"](Q, K, geom))


def _uncentred_projection(X, M):
    """Power steps on the group's uncentred second moment instead of its covariance."""
    n = X.shape[0]
    z = np.ones(X.shape[1])
    for _ in range(_orig_steps()):
        a = M @ z
        a = a / math.sqrt(float(z @ a))
        z = X.T @ (X @ a) / n
    a = M @ z
    return X @ (a / math.sqrt(float(z @ a)))


def _orig_steps():
    return O.REBLOCK_POWER_STEPS


MUTATIONS = [
    ("scale_1_over_d", "softmax_scale", lambda d=128: 1.0 / d, "dense_equivalence"),
    ("tile_axes_swapped", "map_geometry", _geom_swapped_axes, "geometry"),
    ("tile_token_order", "map_geometry", _geom_token_order, "geometry"),
    ("ties_to_highest", "select_topk", _topk_high_ties, "topk_ties"),
    ("topk_smallest", "select_topk", _topk_smallest, "topk_bruteforce"),
    ("prefix_dropped", "row_list",
     lambda geom, sel, sink=1: geom.n_prefix + np.asarray(sel, dtype=np.int64), "prefix_exempt"),
    ("bias_sign", "logmass_bias", _bias_flipped, "logmass"),
    ("bias_no_anchor", "logmass_bias", _bias_no_anchor, "logmass"),
    ("coarse_ignores_bias", "coarse_branch", _coarse_no_bias, "coarse_logmass"),
    ("tau_uses_variance", "tau_threshold", _tau_variance, "tau_threshold"),
    ("tau_moments_with_dense_rows", "tau_rows", _tau_rows_all_tiles, "tau_dense_rows"),
    ("keep_floor", "keep_count", lambda p, n: max(1, min(n, math.floor(p * n / 100.0))), "keep_counts"),
    ("pool_sum", "pool_tiles", lambda X, tiles: np.stack([X[t].sum(axis=0) for t in tiles]), "pooling"),
    ("fine_k_as_v", "fine_row", _fine_k_for_v, "dense_equivalence"),
    ("weighted_plain_means", "weighted_summaries", _weighted_plain_means, "weighted_summaries"),
    ("weighted_unnormalized", "weighted_summaries", _weighted_unnormalized, "weighted_summaries"),
    ("weighted_bias_vs_mean", "weighted_summaries", _weighted_bias_vs_mean, "weighted_summaries"),
    ("off_video_only", "key_candidates", _off_video_only, "sink_off_selection"),
    ("off_video_only_tau", "key_candidates", _off_video_only, "sink_off_tau"),
    ("off_prefix_pinned", "row_list", _row_list_always_pinned, "sink_off_selection"),
    ("bias_mean_over_64", "logmass_bias", _bias_mean_over_64, "sink_off_logmass"),
    ("extra_ignores_list", "extra_tokens_for_row", _extra_ignores_list, "extra_dense"),
    ("extra_ignores_list_choice", "extra_tokens_for_row", _extra_ignores_list, "extra_choice"),
    ("extra_lowest", "extra_tokens_for_row", _extra_lowest, "extra_choice"),
    ("extra_ties_high", "extra_tokens_for_row", _extra_ties_high, "extra_ties"),
    ("reblock_no_normalisation", "reblock_features", lambda qv, M: qv.copy(), "reblock_invariance"),
    ("reblock_identity_metric", "reblock_metric", _rb_identity_metric, "reblock_metric"),
    ("reblock_query_metric", "reblock_metric", _rb_query_metric, "reblock_metric"),
    ("reblock_inverse_metric", "reblock_metric", _rb_inverse_metric, "reblock_metric"),
    ("reblock_uncentred", "principal_projection", _uncentred_projection, "reblock_planted_tree"),
    ("reblock_upper_half_left", "principal_projection",
     lambda X, M: -_orig["principal_projection"](X, M), "reblock_split_sizes"),
    ("reblock_left_ceil", "reblock_left_tiles", lambda m: m - m // 2, "reblock_split_sizes"),
    ("reblock_ties_high", "reblock_order", lambda p, toks: np.lexsort((-toks, p)), "reblock_ties"),
]


@pytest.mark.parametrize("name,attr,bad,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, attr, bad, pin):
    monkeypatch.setattr(O, attr, bad)
    check = dict(P.ALL_CHECKS)[pin]
    with pytest.raises(AssertionError):
        check()


def test_combine_sign_is_caught(monkeypatch):
    """O_fine - G*O_coarse instead of +: the dense-rows-with-gate pin fails."""
    orig = O.forward_head

    def bad(Q, K, V, G, *a, **kw):
        return orig(Q, K, V, None if G is None else -G, *a, **kw)
    monkeypatch.setattr(O, "forward_head", bad)
    with pytest.raises(AssertionError):
        P.check_dense_rows_and_gate(P.SMALL)
