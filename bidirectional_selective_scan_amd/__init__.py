"""Bidirectional selective scan (Vision-Mamba style S6, forward plus index-reversed) on AMD
MI355X (gfx950).

``bidir_fwd`` runs the whole path in the hand-written HIP kernels of ``libvimscan.so`` through
its C ABI (declared in ``include/vimscan.h``); PyTorch only supplies device memory and the
stream. Importing this package loads nothing: the library is opened on first use, and a missing
library raises instead of falling back to anything else.
"""
from .configs import WORKLOADS, HEADLINE, Workload, D_STATE  # noqa: F401


def __getattr__(name):
    if name in ("bidir_fwd", "workspace_bytes", "status_string", "VimscanError", "lib_path",
                "load_library", "launch_info"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
