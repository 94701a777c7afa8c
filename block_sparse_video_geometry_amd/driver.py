"""Sampling-loop driver: a plan pair reused across layers and steps, the dense/sparse
schedule window, and HIP-graph capture of the forward.

Policy follows the pages; none of it lives in the library, which only runs a forward:
- "BSAI FastH3 Native VSA (recipe)", "The inputs that matter": min_tokens keeps short
  sequences dense; start_percent / end_percent run dense outside a window of the
  sampling steps.
- "ComfyUI Agrega Nodo Central de Atencion Dispersa y Compilador Comfy", the schedule
  paragraph: a 0.2 - 1.0 window keeps the first denoise steps dense; its benchmark
  paragraph keeps the first transformer layer dense at every step.
- Same page: outside the window or under min_tokens the ordinary dense attention runs.
  Here that is the library's dense plan (select mode DENSE): every query tile attends
  to every key tile exactly, and no pooling, coarse branch or selection runs.

Every forward runs in libvsa.so's kernels; this module only picks the plan and the
buffers.  A captured graph replays the same kernel launches on fixed buffers.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import vsa as _v


@dataclass(frozen=True)
class Schedule:
    """When a (step, layer) call runs sparse.

    A step's progress is step / n_steps, in [0, 1).  It runs sparse iff
    start_percent <= progress < end_percent (end_percent = 1 keeps the last step sparse),
    the sequence has at least min_tokens tokens, and the layer is not in dense_layers.
    """
    start_percent: float = 0.0
    end_percent: float = 1.0
    min_tokens: int = 8192
    dense_layers: tuple = (0,)

    def __post_init__(self):
        if not (0.0 <= self.start_percent <= self.end_percent <= 1.0):
            raise ValueError("need 0 <= start_percent <= end_percent <= 1")
        if self.min_tokens < 0:
            raise ValueError("min_tokens must be >= 0")

    def sparse(self, step: int, n_steps: int, layer: int, n_tokens: int) -> bool:
        if n_steps <= 0 or not (0 <= step < n_steps):
            raise ValueError("need 0 <= step < n_steps")
        if n_tokens < self.min_tokens or layer in self.dense_layers:
            return False
        progress = step / n_steps
        return self.start_percent <= progress and (progress < self.end_percent or self.end_percent >= 1.0)


class LayerDriver:
    """One sparse plan and one dense plan for a fixed shape, sharing one workspace.

    forward(step, n_steps, layer, q, k, v, g, o) enqueues the forward the schedule picks
    (sparse, or dense with no gate) on the stream and returns True when it ran sparse.
    Calls on one driver must be ordered on one stream (they share the workspace).
    """

    def __init__(self, segments, batch: int, video_T: int, video_H: int, video_W: int, heads: int,
                 keep_percent: float, sink: int = _v.VSA_SINK_EXACT_KV, select: int = _v.VSA_SELECT_TOPK,
                 coarse: int = _v.VSA_COARSE_MEAN, tau: float = 0.0, schedule: Schedule = Schedule(),
                 device: str = "cuda", extra_tokens: int = 0):
        self.schedule = schedule
        self.sparse_plan = _v.vsa_plan_geometry(segments, batch, video_T, video_H, video_W, heads, _v.HEAD_DIM,
                                                keep_percent, sink=sink, select=select, coarse=coarse, tau=tau,
                                                extra_tokens=extra_tokens)
        self.dense_plan = _v.vsa_plan_geometry(segments, batch, video_T, video_H, video_W, heads, _v.HEAD_DIM,
                                               100.0, sink=sink, select=_v.VSA_SELECT_DENSE)
        self.n_tokens = int(self.sparse_plan.desc.n_tokens)
        big = max(self.sparse_plan.workspace_bytes, self.dense_plan.workspace_bytes)
        import torch
        self.workspace = torch.empty(max(256, big), dtype=torch.uint8, device=device)
        if self.workspace.data_ptr() % 256:
            raise RuntimeError("workspace allocation is not 256-byte aligned")
        self._graphs = {}

    def plan_for(self, step: int, n_steps: int, layer: int):
        sparse = self.schedule.sparse(step, n_steps, layer, self.n_tokens)
        return (self.sparse_plan if sparse else self.dense_plan), sparse

    def forward(self, step: int, n_steps: int, layer: int, q, k, v, g, o, stream=None) -> bool:
        plan, sparse = self.plan_for(step, n_steps, layer)
        _v.vsa_forward(plan, q, k, v, g if sparse else None, o, self.workspace, stream)
        return sparse

    def capture(self, sparse: bool, q, k, v, g, o):
        """Capture one forward (sparse or dense) on these fixed tensors into a HIP graph.

        The caller writes each call's inputs into q, k, v, g and reads o after replay().
        The forward is run once eagerly first, so the capture records only kernel launches.
        """
        import torch
        plan = self.sparse_plan if sparse else self.dense_plan
        gg = g if sparse else None
        _v.vsa_forward(plan, q, k, v, gg, o, self.workspace)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            _v.vsa_forward(plan, q, k, v, gg, o, self.workspace)
        self._graphs[sparse] = graph
        return graph

    def replay(self, sparse: bool) -> None:
        self._graphs[sparse].replay()
