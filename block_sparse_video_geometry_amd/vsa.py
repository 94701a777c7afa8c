"""ctypes binding of libvsa.so (include/vsa.h), same names as the C ABI.

Argument marshalling only: every step of the forward runs in the HIP kernels
of libvsa.so.  torch supplies device memory and the current stream.  If the
library is not built this module raises on import: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from pathlib import Path

_LIB_PATH = Path(__file__).resolve().parent / "_lib" / "libvsa.so"

VSA_OK = 0
VSA_ERR_INVALID_ARGUMENT = -1
VSA_ERR_UNSUPPORTED = -2
VSA_ERR_WORKSPACE = -3
VSA_ERR_HIP = -4
VSA_ERR_NO_MEMORY = -5

VSA_SEG_TEXT, VSA_SEG_REF_IMAGE, VSA_SEG_REF_AUDIO, VSA_SEG_OTHER_PREFIX, VSA_SEG_VIDEO = range(5)
VSA_SINK_OFF, VSA_SINK_EXACT_KV, VSA_SINK_EXACT_KV_AND_ROWS = 0, 1, 2
VSA_SELECT_TOPK, VSA_SELECT_TAU, VSA_SELECT_DENSE = 0, 1, 2
VSA_COARSE_MEAN, VSA_COARSE_MEAN_LOGMASS, VSA_COARSE_WEIGHTED_LOGMASS = 0, 1, 2

HEAD_DIM = 128


class vsa_segment(C.Structure):
    _fields_ = [("start", C.c_int64), ("length", C.c_int64), ("kind", C.c_int32),
                ("reserved", C.c_int32)]


class vsa_options(C.Structure):
    _fields_ = [("sink", C.c_int32), ("select", C.c_int32), ("coarse", C.c_int32),
                ("tau", C.c_float), ("extra_tokens", C.c_int32), ("reblock", C.c_int32)]


class vsa_plan_desc(C.Structure):
    _fields_ = [("batch", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("n_tokens", C.c_int64), ("n_prefix_tiles", C.c_int32),
                ("n_video_tiles", C.c_int32), ("n_tiles", C.c_int32), ("k", C.c_int32),
                ("n_dense_rows", C.c_int32), ("n_sparse_rows", C.c_int32),
                ("list_capacity", C.c_int32), ("options", vsa_options),
                ("keep_percent", C.c_float), ("first_candidate", C.c_int32),
                ("n_candidates", C.c_int32)]


class vsa_stats(C.Structure):
    _fields_ = [("executed_pairs", C.c_int64), ("dense_pairs", C.c_int64),
                ("sparse_rows", C.c_int64), ("dense_rows", C.c_int64),
                ("kept_video_tiles", C.c_int64), ("k", C.c_int32), ("reserved", C.c_int32),
                ("extra_tokens", C.c_int64)]


class vsa_debug(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in ("qbar", "kbar", "vbar", "bias", "anchor", "scores",
                                           "ocoarse", "thr", "lists", "counts", "xtok", "xcnt",
                                           "tiles", "total_bytes")]


class vsa_kernel_time(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("launches", C.c_int32), ("total_ms", C.c_double)]


VSA_NOALLOC_SCRATCH_BYTES = 160 << 20

EXPORTS = ["vsa_plan_geometry", "vsa_plan_workspace_bytes", "vsa_plan_describe", "vsa_forward",
           "vsa_forward_noalloc",
           "vsa_read_stats", "vsa_debug_views", "vsa_plan_destroy", "vsa_status_string",
           "vsa_last_error",
           "vsa_timer_create", "vsa_timer_destroy", "vsa_timer_reset", "vsa_forward_timed",
           "vsa_timer_read"]


def _load():
    # torch ships its own HIP runtime; it must be initialised in the process before
    # libvsa.so pulls in the system one, or the second runtime finds no device.  Loading
    # torch first makes both share one set of GPU queues and allocations.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not _LIB_PATH.exists():
        raise ImportError(f"{_LIB_PATH} is not built: run `python "
                          f"block_sparse_video_geometry_amd/build.py` (no fallback path exists)")
    lib = C.CDLL(str(_LIB_PATH))
    P, I, S = C.c_void_p, C.c_int, C.c_size_t
    sig = {
        "vsa_plan_geometry": (I, [C.POINTER(vsa_segment), I, I, I, I, I, I, I, C.c_float,
                                  C.POINTER(vsa_options), C.POINTER(P)]),
        "vsa_plan_workspace_bytes": (I, [P, C.POINTER(S)]),
        "vsa_plan_describe": (I, [P, C.POINTER(vsa_plan_desc)]),
        "vsa_forward": (I, [P, P, P, P, P, P, P, S, P]),
        "vsa_forward_noalloc": (I, [P, P, P, P, P, P, P]),
        "vsa_read_stats": (I, [P, P, P, C.POINTER(vsa_stats)]),
        "vsa_debug_views": (I, [P, C.POINTER(vsa_debug)]),
        "vsa_plan_destroy": (I, [P]),
        "vsa_status_string": (C.c_char_p, [I]),
        "vsa_last_error": (C.c_char_p, []),
        "vsa_timer_create": (I, [C.POINTER(P)]),
        "vsa_timer_destroy": (I, [P]),
        "vsa_timer_reset": (I, [P]),
        "vsa_forward_timed": (I, [P, P, P, P, P, P, P, S, P, P]),
        "vsa_timer_read": (I, [P, C.POINTER(vsa_kernel_time), I, C.POINTER(I)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


class VsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = _lib.vsa_last_error().decode() if status in (VSA_ERR_HIP, VSA_ERR_WORKSPACE) else ""
        super().__init__(f"{what}: {vsa_status_string(status)} ({status}) {detail}".rstrip())


def vsa_status_string(status: int) -> str:
    return _lib.vsa_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != VSA_OK:
        raise VsaError(status, what)


class Plan:
    """Owner of a vsa_plan* (freed with vsa_plan_destroy)."""

    def __init__(self, handle: int):
        self.handle = C.c_void_p(handle)
        self.desc = vsa_plan_describe(self)
        self.workspace_bytes = vsa_plan_workspace_bytes(self)
        self.debug = vsa_debug_views(self)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            _lib.vsa_plan_destroy(h)
            self.handle = None


def vsa_plan_geometry(segments, batch: int, video_T: int, video_H: int, video_W: int,
                      heads: int, head_dim: int = HEAD_DIM, keep_percent: float = 10.0,
                      sink: int = VSA_SINK_EXACT_KV, select: int = VSA_SELECT_TOPK,
                      coarse: int = VSA_COARSE_MEAN, tau: float = 0.0, use_options: bool = True,
                      extra_tokens: int = 0, reblock: int = 0) -> Plan:
    """segments: iterable of (start, length, kind).  Raises VsaError on a bad layout."""
    segs = list(segments)
    arr = (vsa_segment * max(1, len(segs)))()
    for i, (s, n, kd) in enumerate(segs):
        arr[i] = vsa_segment(int(s), int(n), int(kd), 0)
    opts = vsa_options(int(sink), int(select), int(coarse), float(tau), int(extra_tokens), int(reblock))
    out = C.c_void_p()
    rc = _lib.vsa_plan_geometry(arr, len(segs), int(batch), int(video_T), int(video_H), int(video_W),
                                int(heads), int(head_dim), float(keep_percent),
                                C.byref(opts) if use_options else None, C.byref(out))
    _check(rc, "vsa_plan_geometry")
    return Plan(out.value)


def vsa_plan_workspace_bytes(plan: Plan) -> int:
    n = C.c_size_t()
    _check(_lib.vsa_plan_workspace_bytes(plan.handle, C.byref(n)), "vsa_plan_workspace_bytes")
    return n.value


def vsa_plan_describe(plan: Plan) -> vsa_plan_desc:
    d = vsa_plan_desc()
    _check(_lib.vsa_plan_describe(plan.handle, C.byref(d)), "vsa_plan_describe")
    return d


def vsa_debug_views(plan: Plan) -> vsa_debug:
    d = vsa_debug()
    _check(_lib.vsa_debug_views(plan.handle, C.byref(d)), "vsa_debug_views")
    return d


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _check_tensor(name, t, shape):
    import torch
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
        raise ValueError(f"{name}: expected a contiguous bf16 CUDA tensor of shape {shape}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def _forward_args(plan, q, k, v, g, o, workspace):
    d = plan.desc
    shape = (d.batch, d.n_tokens, d.heads, HEAD_DIM)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)) + ((("g", g),) if g is not None else ()):
        _check_tensor(name, t, shape)
    import torch
    if workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise ValueError("workspace: expected a uint8 CUDA tensor")
    return (plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), _ptr(workspace),
            C.c_size_t(workspace.numel()))


def vsa_forward(plan: Plan, q, k, v, g, o, workspace, stream=None) -> None:
    """Enqueue the forward on `stream` (default: torch's current stream)."""
    args = _forward_args(plan, q, k, v, g, o, workspace)
    _check(_lib.vsa_forward(*args, _stream_handle(stream)), "vsa_forward")


def vsa_forward_noalloc(plan: Plan, q, k, v, g, o, stream=None) -> None:
    """Enqueue the forward with the library's static device scratch as its workspace
    (no allocation; calls that overlap on one GPU race)."""
    d = plan.desc
    shape = (d.batch, d.n_tokens, d.heads, HEAD_DIM)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)) + ((("g", g),) if g is not None else ()):
        _check_tensor(name, t, shape)
    _check(_lib.vsa_forward_noalloc(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o),
                                    _stream_handle(stream)), "vsa_forward_noalloc")


def vsa_read_stats(plan: Plan, workspace, stream=None) -> dict:
    st = vsa_stats()
    _check(_lib.vsa_read_stats(plan.handle, _ptr(workspace), _stream_handle(stream), C.byref(st)),
           "vsa_read_stats")
    return {n: getattr(st, n) for n, _ in vsa_stats._fields_ if n != "reserved"}


class Timer:
    """Per-kernel HIP event timer (vsa_timer)."""

    def __init__(self):
        h = C.c_void_p()
        _check(_lib.vsa_timer_create(C.byref(h)), "vsa_timer_create")
        self.handle = h

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            _lib.vsa_timer_destroy(h)
            self.handle = None

    def reset(self):
        _check(_lib.vsa_timer_reset(self.handle), "vsa_timer_reset")

    def read(self) -> dict:
        arr = (vsa_kernel_time * 32)()
        n = C.c_int()
        _check(_lib.vsa_timer_read(self.handle, arr, 32, C.byref(n)), "vsa_timer_read")
        return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


def vsa_forward_timed(plan: Plan, q, k, v, g, o, workspace, timer: Timer, stream=None) -> None:
    args = _forward_args(plan, q, k, v, g, o, workspace)
    _check(_lib.vsa_forward_timed(*args, _stream_handle(stream), timer.handle), "vsa_forward_timed")


def alloc_workspace(plan: Plan, device="cuda"):
    """A uint8 device tensor of the plan's workspace size (256-byte aligned)."""
    import torch
    ws = torch.empty(max(256, plan.workspace_bytes), dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("workspace allocation is not 256-byte aligned")
    return ws


def debug_tensor(plan: Plan, workspace, field: str):
    """View of one intermediate in the workspace (see vsa_debug in include/vsa.h)."""
    import torch
    d = plan.desc
    B, H, Tq, Kc, Qs, cap = (d.batch, d.heads, d.n_tiles, d.n_candidates, d.n_sparse_rows,
                             d.list_capacity)
    spec = {
        "qbar": (torch.float32, (B, H, Tq, HEAD_DIM)),
        "kbar": (torch.float32, (B, H, Kc, HEAD_DIM)),
        "vbar": (torch.float32, (B, H, Kc, HEAD_DIM)),
        "bias": (torch.float32, (B, H, Kc)),
        "anchor": (torch.float32, (B, H, HEAD_DIM)),
        "scores": (torch.float32, (B, H, Qs, Kc)),
        "ocoarse": (torch.float32, (B, H, Qs, HEAD_DIM)),
        "thr": (torch.float32, (B, H)),
        "lists": (torch.int32, (B, H, Qs, cap)),
        "counts": (torch.int32, (B, H, Qs)),
        "xtok": (torch.int32, (B, H, Qs, 64)),
        "xcnt": (torch.int32, (B, H, Qs)),
        "tiles": (torch.int32, (B, H, d.n_video_tiles, 64)),
    }[field]
    if field in ("xtok", "xcnt") and d.options.extra_tokens == 0:
        raise ValueError(f"{field}: the plan has no extra tokens (extra_tokens = 0)")
    if field == "tiles" and d.options.reblock == 0:
        raise ValueError("tiles: the plan has the fixed video tiles (reblock = 0)")
    dtype, shape = spec
    off = getattr(plan.debug, field)
    n = 1
    for s in shape:
        n *= s
    nbytes = n * 4
    return workspace[off:off + nbytes].view(dtype).view(shape)
