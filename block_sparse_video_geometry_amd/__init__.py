"""MI355X (gfx950) two-branch video sparse attention forward.

The compute lives in libvsa.so (hand-written HIP kernels behind the C ABI in
include/vsa.h); this package is its ctypes binding.  Importing it raises when
the library has not been built.
"""
from .vsa import *  # noqa: F401,F403
from .vsa import (Plan, Timer, VsaError, alloc_workspace, debug_tensor, vsa_plan_geometry,
                  vsa_forward, vsa_forward_noalloc, vsa_forward_timed, vsa_read_stats, vsa_debug_views,
                  vsa_plan_describe, vsa_plan_workspace_bytes, vsa_status_string, EXPORTS)
