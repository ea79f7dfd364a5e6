"""MI355X (gfx950) sigmoid group-limited MoE gate and expert-major dispatch.

The work runs in hand-written HIP kernels behind the C ABI of
``libsiggate.so`` (``include/siggate.h``); this package is its thin Python
binding (``binding``), the in-tree build (``build``) and the seeded synthetic
inputs (``workloads``).  Importing the package does not load the library;
the first call does, and raises if it is not built.
"""
from .binding import (Cfg, DispatchOut, SiggateError, load_library, siggate_combine,
                      siggate_dispatch, siggate_ep_dedup, siggate_ep_regroup,
                      siggate_ep_send_splits, siggate_ep_workspace_bytes, siggate_forward,
                      siggate_forward_noalloc, siggate_logits, siggate_status_str,
                      siggate_workspace_bytes, workspace)

__all__ = ["Cfg", "DispatchOut", "SiggateError", "load_library", "siggate_combine",
           "siggate_dispatch", "siggate_ep_dedup", "siggate_ep_regroup",
           "siggate_ep_send_splits", "siggate_ep_workspace_bytes", "siggate_forward",
           "siggate_forward_noalloc", "siggate_logits", "siggate_status_str",
           "siggate_workspace_bytes", "workspace"]
