"""Host-side checks of the C ABI (no GPU needed): exports, plan validation
status codes, plan shapes against the oracle's geometry, workspace layout."""
import ctypes
import re
from pathlib import Path

import pytest

import block_sparse_video_geometry_amd as V
from block_sparse_video_geometry_amd import vsa as VB
from oracle import vsa_oracle as O
from workloads.synth import WORKLOADS

HEADER = Path(__file__).resolve().parents[1] / "include" / "vsa.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(VB._LIB_PATH))
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in vsa.h but not exported"
    assert set(names) == set(VB.EXPORTS)


def test_status_strings():
    for code, name in [(0, "VSA_OK"), (-1, "VSA_ERR_INVALID_ARGUMENT"), (-2, "VSA_ERR_UNSUPPORTED"),
                       (-3, "VSA_ERR_WORKSPACE"), (-4, "VSA_ERR_HIP"), (-5, "VSA_ERR_NO_MEMORY")]:
        assert V.vsa_status_string(code) == name
    assert V.vsa_status_string(7) == "VSA_ERR_UNKNOWN"


GOOD = [(0, 64, 0), (64, 64, 1), (128, 1024, 4)]


def plan_status(segs, batch=1, T=4, H=16, W=16, heads=2, hd=128, keep=25.0, **kw):
    try:
        V.vsa_plan_geometry(segs, batch, T, H, W, heads, hd, keep, **kw)
        return 0
    except V.VsaError as e:
        return e.status


@pytest.mark.parametrize("case,expect", [
    (dict(segs=GOOD), 0),
    (dict(segs=list(reversed(GOOD))), 0),                            # any order
    (dict(segs=[(0, 64, 0), (70, 58, 1), (128, 1024, 4)]), -1),       # gap
    (dict(segs=[(0, 70, 0), (64, 64, 1), (128, 1024, 4)]), -1),       # overlap
    (dict(segs=[(0, 0, 0), (0, 128, 1), (128, 1024, 4)]), -1),        # empty span
    (dict(segs=[(-1, 65, 0), (64, 64, 1), (128, 1024, 4)]), -1),      # negative start
    (dict(segs=[(0, 64, 0), (64, 64, 9), (128, 1024, 4)]), -1),       # unknown kind
    (dict(segs=[(0, 64, 0), (64, 1000, 4)]), -1),                     # video length != T*H*W
    (dict(segs=[(0, 128, 0)]), -2),                                   # no video span
    (dict(segs=[(0, 1024, 4), (1024, 1024, 4)]), -2),                 # two video spans
    (dict(segs=GOOD, hd=64), -2),                                     # head_dim
    (dict(segs=[(0, 128, 0), (128, 5 * 16 * 16, 4)], T=5), -2),       # grid not multiple of 4
    (dict(segs=GOOD, keep=0.0), -2),
    (dict(segs=GOOD, keep=100.5), -2),
    (dict(segs=GOOD, keep=float("nan")), -2),
    (dict(segs=GOOD, keep=0.0, select=1, tau=1.0), 0),                # keep unused in tau mode
    (dict(segs=GOOD, select=1, tau=float("inf")), -2),
    (dict(segs=GOOD, sink=3), -2),
    (dict(segs=GOOD, sink=-1), -2),
    (dict(segs=GOOD, sink=0), 0),                                     # sink_conditioning off
    (dict(segs=[(0, 64, 0), (64, 4 * 256 * 256, 4)], T=4, H=256, W=256), 0),          # 4096 video tiles
    (dict(segs=[(0, 64, 0), (64, 4 * 256 * 256, 4)], T=4, H=256, W=256, sink=0), -2),  # 4097 candidates
    (dict(segs=GOOD, select=2), 0),                                   # dense mode
    (dict(segs=GOOD, select=2, keep=0.0, sink=0, coarse=2), 0),       # ... ignores keep, sink, coarse
    (dict(segs=GOOD, select=2, extra_tokens=4), -2),                  # ... takes no extra tokens
    (dict(segs=GOOD, select=3), -2),
    (dict(segs=GOOD, reblock=1), 0),                                  # adaptive video tiles
    (dict(segs=GOOD, reblock=1, sink=0, select=1, tau=1.0, coarse=2), 0),
    (dict(segs=GOOD, reblock=2), -2),
    (dict(segs=GOOD, reblock=1, extra_tokens=8), -2),                 # not with extra tokens
    (dict(segs=GOOD, reblock=1, select=2), -2),                       # nor the dense mode
    (dict(segs=GOOD, coarse=5), -2),
    (dict(segs=GOOD, coarse=2), 0),                                   # weighted summaries
    (dict(segs=GOOD, extra_tokens=64), 0),                            # extra tokens: 0 .. 64
    (dict(segs=GOOD, extra_tokens=65), -2),
    (dict(segs=GOOD, extra_tokens=-1), -1),
    (dict(segs=GOOD, heads=0), -1),
    (dict(segs=GOOD, batch=0), -1),
    (dict(segs=[(i * 4, 4, 0) for i in range(17)] + [(68, 1024, 4)]), -2),   # > 16 prefix spans
    (dict(segs=[(0, 64, 0), (64, 4 * 4 * 4 * 64 * 65, 4)], T=4, H=256, W=260), -2),  # > 4096 video tiles
    (dict(segs=[(0, 64 * 65536, 0), (64 * 65536, 1024, 4)], heads=1), -2),  # > 65535 tiles
    (dict(segs=GOOD, heads=7000), 0),                                 # N*H*128 just under 2^30
    (dict(segs=GOOD, heads=7300), -2),                                # N*H*128 >= 2^30 (32-bit offsets)
])
def test_plan_validation(case, expect):
    assert plan_status(**case) == expect


def test_dense_plan_shape():
    """The dense mode: every query tile is a dense row; nothing is pooled or selected, so
    the workspace holds only empty sections."""
    w = WORKLOADS["full"]
    p = V.vsa_plan_geometry(w.segments(), 1, *w.grid, w.heads, 128, 100.0, sink=w.sink,
                            select=V.VSA_SELECT_DENSE)
    d = p.desc
    assert d.n_dense_rows == d.n_tiles == 564 and d.n_sparse_rows == 0
    assert d.k == 0 and d.list_capacity == 0 and d.n_candidates == 0
    assert p.workspace_bytes <= 64 * 256


def test_null_options_defaults():
    p = V.vsa_plan_geometry(GOOD, 1, 4, 16, 16, 2, 128, 25.0, use_options=False)
    o = p.desc.options
    assert (o.sink, o.select, o.coarse) == (V.VSA_SINK_EXACT_KV, V.VSA_SELECT_TOPK, V.VSA_COARSE_MEAN)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_plan_shapes_match_oracle_geometry(name):
    w = WORKLOADS[name]
    p = V.vsa_plan_geometry(w.segments(), w.batch, *w.grid, w.heads, 128,
                            w.keep if w.keep > 0 else 100.0, sink=w.sink, select=w.select,
                            coarse=w.coarse, tau=w.tau)
    geom = O.map_geometry(w.segments(), *w.grid)
    sparse, dense = O.row_classes(geom, w.sink)
    cand = O.key_candidates(geom, w.sink)
    pinned = 0 if w.sink == O.SINK_OFF else geom.n_prefix
    d = p.desc
    assert d.n_prefix_tiles == geom.n_prefix
    assert d.n_video_tiles == geom.n_video
    assert d.n_tiles == geom.n_tiles
    assert d.n_dense_rows == len(dense) and d.n_sparse_rows == len(sparse)
    assert d.n_tokens == w.n_tokens
    assert (d.first_candidate, d.n_candidates) == (cand[0], len(cand))
    if w.select == V.VSA_SELECT_TOPK:
        assert d.k == O.keep_count(w.keep, len(cand))
        assert d.list_capacity == pinned + d.k
    else:
        assert d.list_capacity == pinned + len(cand)


@pytest.mark.parametrize("extra", [0, 64])
def test_workspace_layout(extra):
    w = WORKLOADS["full_tau_1.0"]
    p = V.vsa_plan_geometry(w.segments(), 1, *w.grid, w.heads, 128, 100.0, sink=w.sink,
                            select=w.select, tau=w.tau, extra_tokens=extra)
    dbg = p.debug
    d = p.desc
    B, H, Tq, Vt, Qs, cap = 1, d.heads, d.n_tiles, d.n_candidates, d.n_sparse_rows, d.list_capacity
    sizes = {"qbar": B * H * Tq * 512, "kbar": B * H * Vt * 512, "vbar": B * H * Vt * 512,
             "bias": B * H * Vt * 4, "anchor": B * H * 512, "scores": B * H * Qs * Vt * 4,
             "ocoarse": B * H * Qs * 512, "thr": B * H * 4, "lists": B * H * Qs * cap * 4,
             "counts": B * H * Qs * 4}
    if extra:
        sizes.update(xtok=B * H * Qs * 64 * 4, xcnt=B * H * Qs * 4)
    spans = sorted((getattr(dbg, n), getattr(dbg, n) + s) for n, s in sizes.items())
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    for n in sizes:
        assert getattr(dbg, n) % 256 == 0
    assert spans[-1][1] <= dbg.total_bytes == p.workspace_bytes


def test_forward_rejects_before_touching_the_gpu():
    """Null pointers and a missing workspace are caught on the host."""
    lib = VB._lib
    p = V.vsa_plan_geometry(GOOD, 1, 4, 16, 16, 2, 128, 25.0)
    rc = lib.vsa_forward(p.handle, None, None, None, None, None, None, 0, None)
    assert rc == V.VSA_ERR_INVALID_ARGUMENT
    fake = ctypes.c_void_p(1 << 40)
    rc = lib.vsa_forward(p.handle, fake, fake, fake, None, fake, None, 0, None)
    assert rc == V.VSA_ERR_WORKSPACE
    rc = lib.vsa_forward(None, fake, fake, fake, None, fake, fake, 1 << 30, None)
    assert rc == V.VSA_ERR_INVALID_ARGUMENT
    st = VB.vsa_stats()
    assert lib.vsa_read_stats(None, None, None, ctypes.byref(st)) == V.VSA_ERR_INVALID_ARGUMENT


def _random_layout(rng):
    """Random packed layouts: 0-5 prefix segments of 1-300 tokens and one video span, in a
    random order; sometimes a gap, an overlap, a second video span or a bad grid."""
    T, H, W = (int(rng.choice([4, 8, 12, 16])) for _ in range(3))
    parts = [(int(rng.integers(0, 4)), int(rng.integers(1, 301))) for _ in range(int(rng.integers(0, 6)))]
    parts.append((4, T * H * W))
    rng.shuffle(parts)
    segs, pos = [], 0
    for kind, n in parts:
        segs.append([pos, n, kind])
        pos += n
    flaw = int(rng.integers(0, 8))
    if flaw == 0 and len(segs) > 1:
        segs[1][0] += 1                      # gap
    elif flaw == 1 and len(segs) > 1:
        segs[1][0] -= 1                      # overlap
    elif flaw == 2:
        segs.append([pos, 64, 4])            # a second video span
    elif flaw == 3:
        T += 2                               # video grid not a multiple of 4 ...
    elif flaw == 4:
        H += 4                               # ... or not matching the span's length
    order = rng.permutation(len(segs))
    return [tuple(segs[i]) for i in order], (T, H, W)


def test_plan_agrees_with_oracle_geometry_on_random_layouts():
    """The C plan accepts exactly the layouts the oracle's geometry mapper accepts, and then
    has the same prefix, video and total tile counts, k and list capacity."""
    import numpy as np
    rng = np.random.default_rng(2024)
    accepted = rejected = 0
    for trial in range(400):
        segs, grid = _random_layout(rng)
        sink = int(rng.integers(0, 3))
        keep = float(rng.choice([0.5, 10.0, 33.3, 100.0]))
        try:
            geom = O.map_geometry(segs, *grid)
            ok = True
        except ValueError:
            ok = False
        try:
            p = V.vsa_plan_geometry(segs, 1, *grid, 2, 128, keep, sink=sink)
        except V.VsaError as e:
            assert not ok, f"plan rejected {segs} {grid}: {e}"
            rejected += 1
            continue
        assert ok, f"plan accepted {segs} {grid}, the oracle does not"
        accepted += 1
        d = p.desc
        cand = O.key_candidates(geom, sink)
        k = O.keep_count(keep, len(cand))
        pinned = 0 if sink == O.SINK_OFF else geom.n_prefix
        assert (d.n_prefix_tiles, d.n_video_tiles, d.n_tiles) == (geom.n_prefix, geom.n_video, geom.n_tiles)
        assert (d.first_candidate, d.n_candidates) == (cand[0], len(cand))
        assert d.k == k and d.list_capacity == pinned + k
        assert d.n_dense_rows == len(O.row_classes(geom, sink)[1])
    assert accepted > 100 and rejected > 50


def test_reblock_workspace_and_tiles_view():
    """With reblock the workspace also holds the mapper's buffers and the permuted
    inputs and output (five tensors); the tiles view is [B, H, Vt, 64] and needs the option."""
    torch = pytest.importorskip("torch")
    w = WORKLOADS["full_reblock"]
    p0 = V.vsa_plan_geometry(w.segments(), 1, *w.grid, w.heads, 128, w.keep, sink=w.sink)
    p1 = V.vsa_plan_geometry(w.segments(), 1, *w.grid, w.heads, 128, w.keep, sink=w.sink, reblock=1)
    tb = w.n_tokens * w.heads * 128 * 2
    assert p1.workspace_bytes >= p0.workspace_bytes + 5 * tb
    assert p1.desc.options.reblock == 1 and p0.desc.options.reblock == 0
    small = V.vsa_plan_geometry(GOOD, 1, 4, 16, 16, 2, 128, 25.0, reblock=1)
    ws = torch.empty(small.workspace_bytes, dtype=torch.uint8)
    assert tuple(V.debug_tensor(small, ws, "tiles").shape) == (1, 2, 16, 64)
    plain = V.vsa_plan_geometry(GOOD, 1, 4, 16, 16, 2, 128, 25.0)
    with pytest.raises(ValueError):
        V.debug_tensor(plain, torch.empty(plain.workspace_bytes, dtype=torch.uint8), "tiles")


def test_extra_token_views_need_the_option():
    torch = pytest.importorskip("torch")
    p = V.vsa_plan_geometry(GOOD, 1, 4, 16, 16, 2, 128, 25.0)
    ws = torch.empty(p.workspace_bytes, dtype=torch.uint8)
    with pytest.raises(ValueError):
        V.debug_tensor(p, ws, "xtok")
    p2 = V.vsa_plan_geometry(GOOD, 1, 4, 16, 16, 2, 128, 25.0, extra_tokens=8)
    ws2 = torch.empty(p2.workspace_bytes, dtype=torch.uint8)
    assert tuple(V.debug_tensor(p2, ws2, "xtok").shape) == (1, 2, p2.desc.n_sparse_rows, 64)
