"""Plain fp64 CPU oracle of the two-branch video sparse attention forward.

TEST INFRASTRUCTURE.  Only tests/, ``__graft_entry__.smoke()`` and the
cpu_baseline leg of ``bench.py`` may import this module.  It shares no code
with the HIP path (no kernel, header, table or helper); the two read the same
seeded arrays from ``workloads.synth`` and nothing else.

Every step is written straight from its definition, in float64, with numpy
matmul as the only library primitive.  No blocking, fusion or reordering
beyond what a step's definition states.

Pages cited (title; site):
  [R2V-fr]  "Ref2VA VSA : noeud d'attention sparse pour le Ref2VA H3"
            (comfyui-wiki.com, French news item)
  [R2V-en]  "ComfyUI-Ref2VA-VSA: Ultra-Fast Character Video Generation
            (72s on RTX 4090)" (upstar.dev README)
  [FH3]     "BSAI FastH3 Native VSA (recipe)" (comfy.icu node page)
  [BSA-es]  "ComfyUI Agrega Nodo Central de Atencion Dispersa y Compilador
            Comfy" (comfyui-wiki.com, Spanish news item)
  [SPK-es]  "Spark-H3: atencion dispersa por bloques acelera MiniMax-H3 en
            ComfyUI" (comfyui-wiki.com, Spanish news item)

Method, in the pages' order:
  1. geometry mapper: video span -> 4x4x4 tiles of 64 tokens; text,
     reference-image and reference-audio segments -> segment-pure tiles
     ([R2V-fr] "Le correctif d'attention a deux niveaux" item 1; [R2V-en]
     "Technical Architecture" and "The Solution"; [FH3] "The mechanism").
  2. coarse branch: mean-pooled Q/K/V per tile, scores of query tiles
     against video key tiles, softmax, attend ([BSA-es] "tres backends",
     VSA item; [SPK-es] "Que cambia Spark-Attn").
  3. optional log-mass bias on the pooled logits, anchored at the mean video
     query ([SPK-es] "Que cambia Spark-Attn", Spark-Reweight item, and the
     figure caption on exp(E[x]) vs E[exp(x)]); optionally with weighted key /
     value summaries in place of the means (same Spark-Reweight item).
  4. selection: top-k video key tiles per query tile at a keep fraction
     ([FH3] "The mechanism"; [BSA-es] top-k item), or a per-head threshold
     mean + tau * std ([BSA-es] Sol-Attn item); prefix tiles never pruned
     ([R2V-fr] items 1-2; [R2V-en] "The Solution"), unless sink_conditioning
     is off, where they compete like video tiles ([FH3] "The inputs that
     matter").
  5. fine branch: exact attention over the listed tiles ([BSA-es] first
     paragraph; [SPK-es] "Que cambia Spark-Attn"); conditioning query rows
     run dense under exact_kv_and_rows ([FH3] "The inputs that matter",
     sink_conditioning); optionally plus the extra_tokens best-scoring
     single key tokens outside the listed tiles ([BSA-es], schedule
     paragraph: extra_tokens).
  6. gated combine O = O_fine + G * O_coarse with G the to_gate_compress
     output ([R2V-fr] item 3; [R2V-en] "Technical Architecture"; [BSA-es]
     VSA item).

Readings taken where the pages are silent or loose (each one also listed in
the design notes):
  * video tokens are packed raster (t, h, w) with w fastest; video tiles are
    numbered raster (tt, th, tw); tokens inside a tile raster (dt, dh, dw);
  * tile numbering: all prefix tiles first, in packed order, then video tiles;
    the video key index used for ties is the raster rank j in [0, Vt);
  * a prefix segment becomes ceil(len/64) tiles of consecutive tokens; the
    last one may be partial and its missing rows are padding, which takes
    no part in pooling, softmax or output;
  * softmax scale 1/sqrt(128) in both branches;
  * k = ceil(keep * Vt / 100 - 1e-9) clamped to [1, Vt];
  * the coarse branch scores and attends over every video key tile; prefix
    key tiles are always exact and are not in the coarse branch;
  * exact_kv: prefix query tiles are ordinary sparse rows;
    exact_kv_and_rows: prefix query tiles are dense rows with no coarse term;
  * G has the output's shape; no gate means no coarse term in the output
    (the coarse scores still drive the selection); O_coarse of a query tile
    is broadcast to each of its tokens;
  * ranking uses the logit S (scale and bias included), ties go to the
    lowest video tile index;
  * tau statistics: per (batch, head), population mean and std (two-pass)
    over every (sparse query tile, video key tile) logit; keep S > thr; a
    row whose list ends up empty has a zero fine output;
  * log-mass bias b_j = log(mean_t exp(l_t - p_j)) with l_t = s q_a . k_t,
    p_j = s q_a . kbar_j and q_a the mean of all video queries;
  * sink_conditioning off ([FH3] only says it is the cheapest setting and that
    conditioning is then not protected): the prefix tiles lose their
    exemption and join the candidate key tiles.  The coarse branch, the
    log-mass bias and the selection then run over all Tq tiles in tile-id
    order (a partial prefix tile is summarised over its valid tokens), every
    query tile is a sparse row, k = ceil(keep * Tq / 100 - 1e-9) clamped to
    [1, Tq], ties go to the lowest tile id, and the anchor stays the mean of
    the video queries;
  * extra_tokens E ([BSA-es] only says the best-scoring tokens beyond the
    selected blocks are added, to stay closer to dense): per sparse query
    tile i, every valid key token t outside the tiles of i's list is scored
    with the same pooled query as the coarse branch, z_t = s qbar_i . k_t (no
    bias: the bias is a tile's, not a token's); the E largest, ties to the
    lowest packed token index, join the key set of every query of tile i
    (all of them if fewer than E remain).  Dense rows take none (they already
    see every token).  The coarse branch and its output are unchanged;
  * weighted summaries (the page does not give the weights): the anchor's own
    attention over the tile, w_t = softmax_t(l_t); ktil_j = sum_t w_t k_t,
    vtil_j = sum_t w_t v_t; the bias keeps the same anchor identity,
    b_j = log(mean_t exp(l_t)) - s q_a . ktil_j;
  * Spark-Reblock ([SPK-es] "Que cambia Spark-Attn", Spark-Reblock item, and
    reblock_layout=q_reuse_k in its "Flujos de trabajo"; the page gives the
    similarity and the hierarchical splitting down to the block size in
    O(N log N), not the split rule): per (batch, head) the video tokens are
    partitioned by a fixed-shape binary tree.  M = mean over the video keys of
    k k^T (the opposite side's second moment); a query's M-normalised form is
    psi = q / sqrt(q^T M q), so the M-cosine of two queries is the cosine of
    their score patterns over the video keys.  A group of m tiles (64 m
    tokens, m >= 2) is split along its principal axis: the group's centred
    psi covariance C, REBLOCK_POWER_STEPS power steps z <- C M z from z = 1
    (z scaled to M-norm 1 at every step), projections p = psi^T M z; tokens
    sorted by (p, token id), the first 64 floor(m/2) form the left child
    (tiles [t0, t0 + floor(m/2))), the rest the right.  Leaves are the video
    tiles in tree order (the tie-break index), tokens ascending inside a
    leaf; key tiles reuse the query partition; prefix tiles are unchanged.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

TILE_EDGE = 4
TILE_TOKENS = TILE_EDGE ** 3       # 64
HEAD_DIM = 128

SEG_TEXT, SEG_REF_IMAGE, SEG_REF_AUDIO, SEG_OTHER_PREFIX, SEG_VIDEO = 0, 1, 2, 3, 4
SINK_OFF, SINK_EXACT_KV, SINK_EXACT_KV_AND_ROWS = 0, 1, 2
SELECT_TOPK, SELECT_TAU = 0, 1
COARSE_MEAN, COARSE_MEAN_LOGMASS, COARSE_WEIGHTED_LOGMASS = 0, 1, 2


def softmax_scale(head_dim: int = HEAD_DIM) -> float:
    """1/sqrt(d): the plain attention scale (pages silent; reading above)."""
    return 1.0 / math.sqrt(head_dim)


# --------------------------------------------------------------------------
# 1. geometry mapper
# --------------------------------------------------------------------------
@dataclass
class Geometry:
    n_tokens: int
    tiles: list            # tile id -> int64 array of packed token indices (valid tokens only)
    tile_kind: list        # tile id -> segment kind
    n_prefix: int          # P
    n_video: int           # Vt
    grid: tuple            # (T, H, W)
    video_start: int

    @property
    def n_tiles(self) -> int:
        return self.n_prefix + self.n_video


def map_geometry(segments, T: int, H: int, W: int) -> Geometry:
    """Cut the packed sequence into segment-pure tiles.

    [R2V-fr] "Le correctif..." item 1 and [R2V-en] "The Solution": the mapper
    isolates text / reference-image / reference-audio tokens in tiles of
    their own.  [R2V-en] "Technical Architecture" and [FH3] "The mechanism":
    video tokens are grouped in 4x4x4 spatio-temporal tiles of 64 tokens.
    """
    segs = sorted((int(s), int(n), int(kd)) for s, n, kd in segments)
    pos = 0
    for s, n, _ in segs:
        if s != pos or n <= 0:
            raise ValueError("segments must partition [0, N) with positive lengths")
        pos += n
    n_tokens = pos
    videos = [sg for sg in segs if sg[2] == SEG_VIDEO]
    if len(videos) != 1:
        raise ValueError("exactly one video segment is required")
    vstart, vlen, _ = videos[0]
    if vlen != T * H * W or T % TILE_EDGE or H % TILE_EDGE or W % TILE_EDGE:
        raise ValueError("video span must be T*H*W tokens with T, H, W multiples of 4")

    tiles, kinds = [], []
    for s, n, kd in segs:                      # prefix tiles, packed order
        if kd == SEG_VIDEO:
            continue
        for off in range(0, n, TILE_TOKENS):
            tiles.append(np.arange(s + off, s + min(off + TILE_TOKENS, n), dtype=np.int64))
            kinds.append(kd)
    n_prefix = len(tiles)
    for tt in range(T // TILE_EDGE):           # video tiles, raster (tt, th, tw)
        for th in range(H // TILE_EDGE):
            for tw in range(W // TILE_EDGE):
                toks = []
                for dt in range(TILE_EDGE):    # tokens raster (dt, dh, dw)
                    for dh in range(TILE_EDGE):
                        for dw in range(TILE_EDGE):
                            t = TILE_EDGE * tt + dt
                            h = TILE_EDGE * th + dh
                            w = TILE_EDGE * tw + dw
                            toks.append(vstart + (t * H + h) * W + w)
                tiles.append(np.asarray(toks, dtype=np.int64))
                kinds.append(SEG_VIDEO)
    n_video = len(tiles) - n_prefix
    return Geometry(n_tokens, tiles, kinds, n_prefix, n_video, (T, H, W), vstart)


def keep_count(keep_percent: float, n_video: int) -> int:
    """Number k of candidate key tiles kept per query tile at a keep percent.

    [FH3] "The inputs that matter": video_keep_percent; the plain reading of
    a percent of the candidates (Vt, or Tq with sink off) that is not an
    integer is to round up.
    """
    k = math.ceil(keep_percent * n_video / 100.0 - 1e-9)
    return max(1, min(n_video, k))


def key_candidates(geom: Geometry, sink: int) -> list:
    """Tile ids that compete in the coarse branch and the selection.

    [FH3] "The inputs that matter", sink_conditioning: exact_kv and
    exact_kv_and_rows protect the conditioning keys, so only video tiles
    compete; off protects nothing, so every tile competes.
    """
    if sink == SINK_OFF:
        return list(range(geom.n_tiles))
    if sink in (SINK_EXACT_KV, SINK_EXACT_KV_AND_ROWS):
        return list(range(geom.n_prefix, geom.n_tiles))
    raise ValueError("unsupported sink mode")


def row_classes(geom: Geometry, sink: int):
    """(sparse query tiles, dense query tiles).

    [FH3] "The inputs that matter", sink_conditioning: exact_kv keeps the
    conditioning keys exact for every query; exact_kv_and_rows also runs the
    conditioning queries dense.
    """
    prefix = list(range(geom.n_prefix))
    video = list(range(geom.n_prefix, geom.n_tiles))
    if sink in (SINK_OFF, SINK_EXACT_KV):
        return prefix + video, []
    if sink == SINK_EXACT_KV_AND_ROWS:
        return video, prefix
    raise ValueError("unsupported sink mode")


# --------------------------------------------------------------------------
# 1b. Spark-Reblock: an adaptive partition of the video tokens
# --------------------------------------------------------------------------
REBLOCK_POWER_STEPS = 3


def reblock_metric(Q: np.ndarray, K: np.ndarray, geom: Geometry) -> np.ndarray:
    """M = (1/Nv) sum over the video keys of k k^T ([SPK-es] Spark-Reblock: the
    metric is induced by the second moment of the opposite side; for the query
    partition that is the keys).  Q is not used; it is an argument so that the
    choice of side is explicit."""
    vt = np.concatenate(geom.tiles[geom.n_prefix:])
    Kv = K[vt]
    return Kv.T @ Kv / len(vt)


def reblock_features(qv: np.ndarray, M: np.ndarray) -> np.ndarray:
    """psi = q / sqrt(q^T M q) per row of qv: the M-cosine of two queries is the
    M inner product of their psi.  A query with q^T M q = 0 takes psi = 0."""
    nrm = np.sqrt(np.maximum(np.einsum("id,de,ie->i", qv, M, qv), 0.0))
    return np.where(nrm[:, None] > 0, qv / np.where(nrm > 0, nrm, 1.0)[:, None], 0.0)


def principal_projection(X: np.ndarray, M: np.ndarray) -> np.ndarray:
    """Projections of a group's psi rows X on the group's principal axis in the
    metric M: REBLOCK_POWER_STEPS power steps z <- C M z from z = 1 with C the
    centred covariance of X, z scaled to M-norm 1 before each step; then
    p_i = X_i^T M z / |z|_M (in [-1, 1]).  A zero axis gives p = 0 everywhere."""
    n = X.shape[0]
    Xc = X - X.mean(axis=0)
    z = np.ones(X.shape[1])
    for _ in range(REBLOCK_POWER_STEPS):
        a = M @ z
        za = float(z @ a)
        a = a / math.sqrt(za) if za > 0 else np.zeros_like(a)
        z = Xc.T @ (Xc @ a) / n
    a = M @ z
    za = float(z @ a)
    a = a / math.sqrt(za) if za > 0 else np.zeros_like(a)
    return X @ a


def reblock_order(p: np.ndarray, toks: np.ndarray) -> np.ndarray:
    """Positions of a group's tokens sorted by projection, equal projections by
    the lower token id."""
    return np.lexsort((toks, p))


def reblock_left_tiles(m: int) -> int:
    """Tiles of the left (lower-projection) child of a group of m tiles."""
    return m // 2


def reblock_geometry(Q: np.ndarray, K: np.ndarray, geom: Geometry, split_hook=None) -> Geometry:
    """The fixed-tile geometry with its video tiles replaced by the Spark-Reblock
    leaves of one (batch, head) ([SPK-es] "Que cambia Spark-Attn", Spark-Reblock item).

    Two queries are similar when their score patterns over the keys are: the
    cosine of K q and K q' is the M-cosine q^T M q' / (|q|_M |q'|_M) with M the
    keys' second moment.  A hierarchical splitter halves each group of m tiles
    along its principal axis in that metric (the lower-projection 64 floor(m/2)
    tokens form the left child) until every leaf holds one tile of 64 tokens: a
    fixed tree shape of ceil(log2 Vt) levels, O(N log N) work.  Leaves are
    numbered left to right; tokens ascending inside a leaf; key tiles reuse the
    query partition.

    split_hook(t0, m, toks, p, left, right) -> (left, right), if given, may replace
    the split of a node (tests adopt another valid split where projections nearly
    tie); toks are the group's tokens ascending, p their projections.
    """
    M = reblock_metric(Q, K, geom)
    vt = np.sort(np.concatenate(geom.tiles[geom.n_prefix:]))
    psi = reblock_features(Q[vt], M)
    row_of = {int(t): i for i, t in enumerate(vt)}
    leaves = [None] * geom.n_video

    def split(toks, t0, m):
        if m == 1:
            leaves[t0] = toks
            return
        X = psi[[row_of[int(t)] for t in toks]]
        p = principal_projection(X, M)
        order = reblock_order(p, toks)
        ml = reblock_left_tiles(m)
        kl = TILE_TOKENS * ml
        left, right = np.sort(toks[order[:kl]]), np.sort(toks[order[kl:]])
        if split_hook is not None:
            left, right = split_hook(t0, m, toks, p, left, right)
        split(left, t0, ml)
        split(right, t0 + ml, m - ml)

    split(vt, 0, geom.n_video)
    return Geometry(geom.n_tokens, list(geom.tiles[:geom.n_prefix]) + leaves, list(geom.tile_kind),
                    geom.n_prefix, geom.n_video, geom.grid, geom.video_start)


# --------------------------------------------------------------------------
# 2. coarse branch summaries
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bfloat16 -> float64 (a bf16 is the top 16 bits of a float32)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def pool_tiles(X: np.ndarray, tiles) -> np.ndarray:
    """Mean of the valid tokens of each tile ([SPK-es]: the compressed branch's
    summary is a mean pool).  X is [N, D] for one (batch, head)."""
    return np.stack([X[t].mean(axis=0) for t in tiles])


def logmass_bias(Q: np.ndarray, K: np.ndarray, geom: Geometry, scale: float, cand=None):
    """Per candidate key tile log-mass bias, anchored at the mean video query.

    [SPK-es] "Que cambia Spark-Attn", Spark-Reweight: mean pooling puts
    exp(E[x]) in place of E[exp(x)]; a bias restores the missing mass, and the
    score uses the mean of the video queries as a per-head anchor.
      q_a = mean of Q over all valid video tokens
      l_t = s q_a . k_t,  p_j = s q_a . kbar_j
      b_j = log( mean_{t in j} exp(l_t - p_j) )   (mean over the valid tokens)
    cand: candidate tile ids (default: the video tiles).
    Returns (b [len(cand)], q_a [D]).
    """
    video_tokens = np.concatenate(geom.tiles[geom.n_prefix:])
    q_a = Q[video_tokens].mean(axis=0)
    ct = geom.tiles[geom.n_prefix:] if cand is None else [geom.tiles[t] for t in cand]
    b = np.empty(len(ct))
    for j, toks in enumerate(ct):
        kbar = K[toks].mean(axis=0)
        p = scale * (q_a @ kbar)
        ell = scale * (K[toks] @ q_a)
        b[j] = math.log(np.mean(np.exp(ell - p)))
    return b, q_a


def weighted_summaries(Q: np.ndarray, K: np.ndarray, V: np.ndarray, geom: Geometry, scale: float,
                       cand=None):
    """Weighted key / value summaries of the candidate tiles plus the log-mass bias.

    [SPK-es] "Que cambia Spark-Attn", Spark-Reweight: weighted summaries replace
    the mean-pooled key / value summary, with the log-mass bias on top and the
    mean video query as the per-head anchor.  The weights are the anchor's
    attention over the tile's keys (the page does not give them):
      q_a = mean of Q over all valid video tokens
      l_t = s q_a . k_t,  w_t = exp(l_t) / sum_{t' in j} exp(l_t')
      ktil_j = sum_t w_t k_t,  vtil_j = sum_t w_t v_t
      b_j = log( mean_{t in j} exp(l_t) ) - s q_a . ktil_j
    so that exp(s q_a . ktil_j + b_j) is mean_t exp(l_t), as for the plain bias
    (sums and means over the tile's valid tokens).
    cand: candidate tile ids (default: the video tiles).
    Returns (ktil [n, D], vtil [n, D], b [n], q_a [D]) with n = len(cand).
    """
    q_a = Q[np.concatenate(geom.tiles[geom.n_prefix:])].mean(axis=0)
    ct = geom.tiles[geom.n_prefix:] if cand is None else [geom.tiles[t] for t in cand]
    D = K.shape[1]
    ktil, vtil, b = np.empty((len(ct), D)), np.empty((len(ct), D)), np.empty(len(ct))
    for j, toks in enumerate(ct):
        ell = scale * (K[toks] @ q_a)
        m = ell.max()
        e = np.exp(ell - m)
        w = e / e.sum()
        ktil[j] = w @ K[toks]
        vtil[j] = w @ V[toks]
        b[j] = m + math.log(np.mean(e)) - scale * (q_a @ ktil[j])
    return ktil, vtil, b, q_a


def coarse_branch(Qbar: np.ndarray, Kbar: np.ndarray, Vbar: np.ndarray,
                  bias: np.ndarray, scale: float):
    """Coarse scores, softmax and output for a set of query tiles.

    S_ij = s qbar_i . kbar_j + b_j over the candidate key tiles j; P = row softmax;
    O_c,i = sum_j P_ij vbar_j.  Returns (S, O_c).
    """
    S = scale * (Qbar @ Kbar.T) + bias[None, :]
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    P = E / E.sum(axis=1, keepdims=True)
    return S, P @ Vbar


# --------------------------------------------------------------------------
# 4. selection
# --------------------------------------------------------------------------
def select_topk(S_row: np.ndarray, k: int) -> np.ndarray:
    """The k largest logits; equal logits go to the lowest candidate index.
    Returns the kept candidate indices in ascending order."""
    order = sorted(range(len(S_row)), key=lambda j: (-S_row[j], j))
    return np.array(sorted(order[:k]), dtype=np.int64)


def tau_rows(geom: Geometry, sink: int) -> list:
    """Query tiles whose coarse logits enter the tau moments: the sparse rows.

    [BSA-es] Sol-Attn: the threshold is in sigmas of the score distribution,
    and only rows that select have coarse scores.  Under exact_kv_and_rows the
    conditioning query tiles run dense ([FH3] "The inputs that matter"), so
    they score nothing and stay out of the moments."""
    return row_classes(geom, sink)[0]


def tau_threshold(S: np.ndarray, tau: float) -> float:
    """mu + tau * sigma over every logit of one (batch, head), population
    moments in two passes ([BSA-es] Sol-Attn: a per-head threshold in sigmas
    of the score distribution)."""
    vals = S.ravel()
    n = vals.size
    mu = float(np.sum(vals)) / n
    var = float(np.sum((vals - mu) ** 2)) / n
    return mu + tau * math.sqrt(var)


def select_tau(S_row: np.ndarray, thr: float) -> np.ndarray:
    return np.nonzero(S_row > thr)[0].astype(np.int64)


def row_list(geom: Geometry, video_sel, sink: int = SINK_EXACT_KV) -> np.ndarray:
    """Key tiles of one sparse row, as ascending tile ids.  With the prefix
    protected: every prefix tile (never pruned) then the kept video tiles;
    with sink off: the kept candidates, which are tile ids themselves."""
    sel = np.asarray(video_sel, dtype=np.int64)
    if sink == SINK_OFF:
        return sel
    return np.concatenate([np.arange(geom.n_prefix, dtype=np.int64), geom.n_prefix + sel])


# --------------------------------------------------------------------------
# 5. fine branch
# --------------------------------------------------------------------------
def extra_tokens_for_row(qbar_i: np.ndarray, K: np.ndarray, geom: Geometry, key_tiles,
                         n_extra: int, scale: float) -> np.ndarray:
    """The n_extra best-scoring key tokens outside the listed tiles of one sparse row.

    [BSA-es], schedule paragraph: extra_tokens adds the top-scoring tokens
    beyond the selected blocks.  z_t = s qbar_i . k_t over every valid token t
    not in a listed tile; the largest z first, equal z to the lower token index.
    Returns the chosen packed token indices in ascending order.
    """
    if n_extra <= 0:
        return np.zeros(0, dtype=np.int64)
    listed = set(int(t) for t in key_tiles)
    elig = [geom.tiles[t] for t in range(geom.n_tiles) if t not in listed]
    if not elig:
        return np.zeros(0, dtype=np.int64)
    toks = np.concatenate(elig)
    z = scale * (K[toks] @ qbar_i)
    order = np.lexsort((toks, -z))   # by -z, then by token
    return np.sort(toks[order[:n_extra]])


def fine_row(Q: np.ndarray, K: np.ndarray, V: np.ndarray, geom: Geometry,
             qtile: int, key_tiles, scale: float, extra=None) -> np.ndarray:
    """Exact softmax attention of the valid queries of one query tile over the
    valid tokens of the listed key tiles, plus the extra tokens if given.
    Returns [n_valid, D].  An empty key set (possible only with no prefix
    and nothing above the tau threshold) attends to nothing and gives zeros."""
    rows = geom.tiles[qtile]
    parts = [geom.tiles[t] for t in key_tiles]
    if extra is not None and len(extra):
        parts.append(np.asarray(extra, dtype=np.int64))
    if not parts:
        return np.zeros((len(rows), Q.shape[1]))
    keys = np.concatenate(parts)
    z = scale * (Q[rows] @ K[keys].T)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e @ V[keys]) / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# whole forward for one (batch, head)
# --------------------------------------------------------------------------
def forward_head(Q, K, V, G, geom: Geometry, keep_percent: float, sink: int,
                 select: int, coarse: int, tau: float, rows=None,
                 list_override=None, want_intermediates=False, extra_tokens: int = 0,
                 extra_override=None, fine: bool = True):
    """Run the method for one (batch, head).

    Q, K, V, G: float64 [N, D] (G may be None).  rows: query tile ids to
    produce (None = all).  list_override: {query tile id: tile id array} to
    replace the selection of some sparse rows (used when several selections
    are correct); extra_override does the same for the extra tokens.
    fine=False stops after the selection (lists only: no extra tokens, no
    fine branch, O left NaN).
    Returns (O [N, D] with NaN outside the produced rows, intermediates dict
    or None).
    """
    scale = softmax_scale(Q.shape[1])
    sparse, dense = row_classes(geom, sink)
    if rows is None:
        rows = list(range(geom.n_tiles))
    rows_set = set(int(r) for r in rows)
    cand = key_candidates(geom, sink)
    ct = [geom.tiles[t] for t in cand]
    Kbar = pool_tiles(K, ct)
    Vbar = pool_tiles(V, ct)
    if coarse == COARSE_MEAN_LOGMASS:
        bias, q_a = logmass_bias(Q, K, geom, scale, cand)
    elif coarse == COARSE_WEIGHTED_LOGMASS:
        Kbar, Vbar, bias, q_a = weighted_summaries(Q, K, V, geom, scale, cand)
    elif coarse == COARSE_MEAN:
        bias, q_a = np.zeros(len(ct)), None
    else:
        raise ValueError("unsupported coarse mode")

    # tau mode reports every sparse row's logits (tests read them); top-k only the rows asked for
    need = sparse if select == SELECT_TAU else [i for i in sparse if i in rows_set]
    need_idx = {i: n for n, i in enumerate(need)}
    Qbar = pool_tiles(Q, [geom.tiles[i] for i in need]) if need else np.zeros((0, Q.shape[1]))
    S, Oc = coarse_branch(Qbar, Kbar, Vbar, bias, scale) if need else (np.zeros((0, len(ct))), None)
    thr = None
    if select == SELECT_TAU:
        # the moments run over the logits of every row of the tau population, asked for or not
        pop = tau_rows(geom, sink)
        Qpop = pool_tiles(Q, [geom.tiles[i] for i in pop]) if pop else np.zeros((0, Q.shape[1]))
        Spop = coarse_branch(Qpop, Kbar, Vbar, bias, scale)[0] if pop else np.zeros((0, len(ct)))
        thr = tau_threshold(Spop, tau)
    k = keep_count(keep_percent, len(cand)) if select == SELECT_TOPK else None

    O = np.full_like(Q, np.nan)
    lists, extras = {}, {}
    dense_set = set(dense)
    all_tiles = np.arange(geom.n_tiles, dtype=np.int64)
    for i in sorted(rows_set):
        toks = geom.tiles[i]
        if i in dense_set:
            lst = all_tiles
        else:
            srow = S[need_idx[i]]
            if select == SELECT_TOPK:
                sel = select_topk(srow, k)
            else:
                sel = select_tau(srow, thr)
            lst = row_list(geom, sel, sink)
            if list_override is not None and i in list_override:
                lst = np.asarray(list_override[i], dtype=np.int64)
        lists[i] = lst
        if not fine:
            continue
        ex = None
        if i not in dense_set and extra_tokens > 0:
            ex = extra_tokens_for_row(Qbar[need_idx[i]], K, geom, lst, extra_tokens, scale)
            if extra_override is not None and i in extra_override:
                ex = np.asarray(extra_override[i], dtype=np.int64)
            extras[i] = ex
        of = fine_row(Q, K, V, geom, i, lst, scale, ex)
        if i not in dense_set and G is not None:
            of = of + G[toks] * Oc[need_idx[i]][None, :]
        O[toks] = of
    inter = None
    if want_intermediates:
        inter = dict(Kbar=Kbar, Vbar=Vbar, bias=bias, anchor=q_a, sparse_rows=need, cand=cand,
                     Qbar=Qbar, S=S, Oc=Oc, thr=thr, k=k, lists=lists, extras=extras)
    return O, inter


def forward(inputs: dict, segments, grid, keep_percent: float, sink: int,
            select: int = SELECT_TOPK, coarse: int = COARSE_MEAN, tau: float = 0.0,
            heads=None, rows=None, list_override=None, want_intermediates=False,
            extra_tokens: int = 0, fine: bool = True, reblock: bool = False, split_hooks=None):
    """Oracle forward on bf16 bit arrays q, k, v, g ([B, N, H, D] uint16; g
    may be None).  Returns (O float64 [B, N, H, D] (NaN where not produced),
    {(b, h): intermediates}).  heads: iterable of (b, h) to run (None = all).
    list_override: {(b, h): {query tile: tile ids}}.  fine=False: selection only.
    reblock: Spark-Reblock video tiles per (b, h) (the intermediates then hold the
    head's geometry under "geom"); split_hooks: {(b, h): split_hook}."""
    q, k, v, g = inputs["q"], inputs["k"], inputs["v"], inputs.get("g")
    B, N, H, D = q.shape
    T, Hh, W = grid
    geom = map_geometry(segments, T, Hh, W)
    if geom.n_tokens != N:
        raise ValueError("segments do not cover the token axis")
    O = np.full((B, N, H, D), np.nan)
    inter = {}
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        Qh = bf16_bits_to_f64(q[b, :, h, :])
        Kh = bf16_bits_to_f64(k[b, :, h, :])
        Vh = bf16_bits_to_f64(v[b, :, h, :])
        Gh = bf16_bits_to_f64(g[b, :, h, :]) if g is not None else None
        for arr in (Qh, Kh, Vh) + ((Gh,) if Gh is not None else ()):
            if not np.all(np.isfinite(arr)):
                raise ValueError("inputs must be finite")
        lo = None if list_override is None else list_override.get((b, h))
        gh = geom
        if reblock:
            hook = None if split_hooks is None else split_hooks.get((b, h))
            gh = reblock_geometry(Qh, Kh, geom, hook)
        O[b, :, h, :], it = forward_head(Qh, Kh, Vh, Gh, gh, keep_percent, sink, select,
                                         coarse, tau, rows=rows, list_override=lo,
                                         want_intermediates=want_intermediates,
                                         extra_tokens=extra_tokens, fine=fine)
        if it is not None and reblock:
            it["geom"] = gh
        inter[(b, h)] = it
    return O, inter
