"""Seeded synthetic inputs for the two-branch video sparse attention forward.

This module only draws numbers and describes workload shapes.  It holds none
of the method's arithmetic: no tiling table, pooling, scoring, selection or
attention.  Both the fp64 oracle (test infrastructure) and the HIP path read
the arrays it returns, so neither depends on the other for its inputs.

The shapes stand in for the 1344x768 clips measured on the pages (the clips,
their prompts and reference images are not available): a conditioning prefix
of text, reference-image and reference-audio tokens followed by a video latent
grid of T x H x W tokens, heads interleaved, head dimension 128.

Draw recipe (numpy ``Generator(PCG64(seed))``, float32 ``standard_normal``,
rounded to bfloat16 round-to-nearest-even; draw order Q, K, V, G, then the
recipe's extra draws):

* ``iid``     Q, K, V, G ~ N(0, 1).
* ``scaled``  Q, K ~ sqrt(3) N(0, 1) so token logits have std about 3;
              V, G ~ N(0, 1).
* ``smooth``  Q and K: a per (64-token block, head, dim) mean ~ N(0, 1) plus
              0.3 N(0, 1) per token.  Blocks are 4x4x4 cubes of the video grid
              and runs of 64 consecutive tokens of each prefix segment.
              V ~ N(0, 1).  G = sigmoid(Q_h . w_h) with w_h ~ N(0, 1/128)^128
              per head, broadcast over the head dimension.
* ``offset``  ``scaled`` plus a per-head query offset mu_h ~ sqrt(3) N(0,1)^128
              added to every Q token, so the mean video query is far from 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

HEAD_DIM = 128

# segment kinds, same numbering as the C ABI
SEG_TEXT, SEG_REF_IMAGE, SEG_REF_AUDIO, SEG_OTHER_PREFIX, SEG_VIDEO = 0, 1, 2, 3, 4
SINK_OFF, SINK_EXACT_KV, SINK_EXACT_KV_AND_ROWS = 0, 1, 2
SELECT_TOPK, SELECT_TAU = 0, 1
COARSE_MEAN, COARSE_MEAN_LOGMASS, COARSE_WEIGHTED_LOGMASS = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    prefix: tuple            # ((kind, length), ...) in packed order, before the video
    grid: tuple              # (T, H, W) of the video latent grid
    keep: float              # keep percent of video key tiles (top-k mode)
    sink: int
    select: int = SELECT_TOPK
    coarse: int = COARSE_MEAN
    tau: float = 0.0
    seed: int = 0
    recipe: str = "iid"
    batch: int = 1
    video_first: bool = False   # put the video span before the prefix (edge case)
    extra: int = 0              # extra_tokens per sparse query tile (0: off)
    reblock: int = 0            # 1: adaptive (Spark-Reblock) video tiles per (batch, head)

    @property
    def n_video(self) -> int:
        T, H, W = self.grid
        return T * H * W

    @property
    def n_tokens(self) -> int:
        return sum(n for _, n in self.prefix) + self.n_video

    def segments(self):
        """Segment spans [(start, length, kind)] in packed order."""
        segs = []
        pos = 0
        if self.video_first:
            segs.append((0, self.n_video, SEG_VIDEO))
            pos = self.n_video
        for kind, n in self.prefix:
            segs.append((pos, n, kind))
            pos += n
        if not self.video_first:
            segs.append((pos, self.n_video, SEG_VIDEO))
        return segs


_FULL_PREFIX = ((SEG_TEXT, 512), (SEG_REF_IMAGE, 1536), (SEG_REF_AUDIO, 256))
_FULL_GRID = (32, 24, 44)

WORKLOADS = {
    "tiny": Workload("tiny", 2, ((SEG_TEXT, 64), (SEG_REF_IMAGE, 64)), (4, 16, 16), 25.0,
                     SINK_EXACT_KV, seed=1001, recipe="iid"),
    "mid": Workload("mid", 8, ((SEG_TEXT, 256), (SEG_REF_IMAGE, 512), (SEG_REF_AUDIO, 128)),
                    (16, 24, 44), 25.0, SINK_EXACT_KV, seed=1002, recipe="iid"),
    "full": Workload("full", 32, _FULL_PREFIX, _FULL_GRID, 10.0, SINK_EXACT_KV_AND_ROWS,
                     seed=1003, recipe="scaled"),
    "full_smooth_20": Workload("full_smooth_20", 32, _FULL_PREFIX, _FULL_GRID, 20.0,
                               SINK_EXACT_KV_AND_ROWS, seed=1004, recipe="smooth"),
    "full_smooth_100": Workload("full_smooth_100", 32, _FULL_PREFIX, _FULL_GRID, 100.0,
                                SINK_EXACT_KV_AND_ROWS, seed=1004, recipe="smooth"),
    "full_tau_1.0": Workload("full_tau_1.0", 32, _FULL_PREFIX, _FULL_GRID, 0.0,
                             SINK_EXACT_KV_AND_ROWS, SELECT_TAU, COARSE_MEAN, 1.0,
                             seed=1005, recipe="offset"),
    "full_tau_1.5": Workload("full_tau_1.5", 32, _FULL_PREFIX, _FULL_GRID, 0.0,
                             SINK_EXACT_KV_AND_ROWS, SELECT_TAU, COARSE_MEAN, 1.5,
                             seed=1005, recipe="offset"),
    "full_tau_2.0": Workload("full_tau_2.0", 32, _FULL_PREFIX, _FULL_GRID, 0.0,
                             SINK_EXACT_KV_AND_ROWS, SELECT_TAU, COARSE_MEAN, 2.0,
                             seed=1005, recipe="offset"),
    "full_logmass": Workload("full_logmass", 32, _FULL_PREFIX, _FULL_GRID, 10.0,
                             SINK_EXACT_KV_AND_ROWS, SELECT_TOPK, COARSE_MEAN_LOGMASS,
                             seed=1005, recipe="offset"),
    # the log-mass workload with weighted key / value summaries in place of the means
    "full_weighted": Workload("full_weighted", 32, _FULL_PREFIX, _FULL_GRID, 10.0,
                              SINK_EXACT_KV_AND_ROWS, SELECT_TOPK, COARSE_WEIGHTED_LOGMASS,
                              seed=1005, recipe="offset"),
    # the full workload's inputs with sink_conditioning off: prefix tiles compete
    "full_sink_off": Workload("full_sink_off", 32, _FULL_PREFIX, _FULL_GRID, 10.0, SINK_OFF,
                              seed=1003, recipe="scaled"),
    # the full workload's inputs plus 64 extra tokens per sparse query tile
    "full_extra64": Workload("full_extra64", 32, _FULL_PREFIX, _FULL_GRID, 10.0,
                             SINK_EXACT_KV_AND_ROWS, seed=1003, recipe="scaled", extra=64),
    # adaptive video tiles: on the full workload's inputs, and on the smooth inputs (whose
    # queries cluster by 4x4x4 cube) at 20% keep
    "full_reblock": Workload("full_reblock", 32, _FULL_PREFIX, _FULL_GRID, 10.0,
                             SINK_EXACT_KV_AND_ROWS, seed=1003, recipe="scaled", reblock=1),
    "full_smooth_reblock_20": Workload("full_smooth_reblock_20", 32, _FULL_PREFIX, _FULL_GRID, 20.0,
                                       SINK_EXACT_KV_AND_ROWS, seed=1004, recipe="smooth", reblock=1),
}


def scaled_down(w: Workload, heads: int | None = None, grid: tuple | None = None,
                prefix: tuple | None = None, **kw) -> Workload:
    """Same recipe and options on a smaller shape (parity cases the oracle finishes fast)."""
    d = dict(w.__dict__)
    if heads is not None:
        d["heads"] = heads
    if grid is not None:
        d["grid"] = grid
    if prefix is not None:
        d["prefix"] = prefix
    d.update(kw)
    return Workload(**d)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_means(rng, w: Workload, shape_tail):
    """One N(0,1) draw per 64-token block of every segment, broadcast to tokens.

    Video blocks are 4x4x4 cubes of the (T, H, W) grid (np.repeat along each
    axis); prefix blocks are runs of 64 consecutive tokens of one segment.
    """
    B = w.batch
    out = np.empty((B, w.n_tokens) + shape_tail, dtype=np.float32)
    for start, n, kind in w.segments():
        if kind == SEG_VIDEO:
            T, H, W = w.grid
            m = rng.standard_normal((B, T // 4, H // 4, W // 4) + shape_tail, dtype=np.float32)
            m = np.repeat(np.repeat(np.repeat(m, 4, axis=1), 4, axis=2), 4, axis=3)
            out[:, start:start + n] = m.reshape((B, n) + shape_tail)
        else:
            nb = -(-n // 64)
            m = rng.standard_normal((B, nb) + shape_tail, dtype=np.float32)
            out[:, start:start + n] = np.repeat(m, 64, axis=1)[:, :n]
    return out


def make_inputs(w: Workload, with_gate: bool = True) -> dict:
    """Seeded bf16 inputs as uint16 bit arrays of shape [B, N, heads, 128]."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    shape = (w.batch, w.n_tokens, w.heads, HEAD_DIM)
    out = {}
    if w.recipe in ("iid", "scaled", "offset"):
        qs = np.float32(np.sqrt(3.0)) if w.recipe in ("scaled", "offset") else np.float32(1.0)
        q = rng.standard_normal(shape, dtype=np.float32) * qs
        k = rng.standard_normal(shape, dtype=np.float32) * qs
        v = rng.standard_normal(shape, dtype=np.float32)
        g = rng.standard_normal(shape, dtype=np.float32) if with_gate else None
        if w.recipe == "offset":
            mu = rng.standard_normal((w.heads, HEAD_DIM), dtype=np.float32) * np.float32(np.sqrt(3.0))
            q += mu[None, None]
        out["q"] = f32_to_bf16_bits(q)
        del q
        out["k"] = f32_to_bf16_bits(k)
        del k
        out["v"] = f32_to_bf16_bits(v)
        del v
        out["g"] = f32_to_bf16_bits(g) if g is not None else None
    elif w.recipe == "smooth":
        tail = (w.heads, HEAD_DIM)
        q = _block_means(rng, w, tail)
        q += np.float32(0.3) * rng.standard_normal(shape, dtype=np.float32)
        k = _block_means(rng, w, tail)
        k += np.float32(0.3) * rng.standard_normal(shape, dtype=np.float32)
        v = rng.standard_normal(shape, dtype=np.float32)
        out["q"] = f32_to_bf16_bits(q)
        del q
        out["k"] = f32_to_bf16_bits(k)
        del k
        out["v"] = f32_to_bf16_bits(v)
        del v
        if with_gate:
            wv = rng.standard_normal((w.heads, HEAD_DIM)).astype(np.float64) / np.sqrt(HEAD_DIM)
            qf = bf16_bits_to_f32(out["q"]).astype(np.float64)
            logit = np.einsum("bnhd,hd->bnh", qf, wv)
            del qf
            gate = (1.0 / (1.0 + np.exp(-logit))).astype(np.float32)
            out["g"] = f32_to_bf16_bits(np.broadcast_to(gate[..., None], shape))
        else:
            out["g"] = None
    else:
        raise ValueError(f"unknown recipe {w.recipe}")
    return out
