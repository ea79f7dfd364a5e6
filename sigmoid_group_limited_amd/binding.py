"""Thin ctypes binding of libsiggate.so (include/siggate.h).

Argument marshalling only: every step of the gate and the dispatch runs in the
HIP kernels of the library.  PyTorch supplies device memory (tensors) and the
current stream.  Workspaces and outputs the wrappers allocate themselves are
allocated on the stream the call runs on (``stream=``, else the current
one).  The library is loaded on first use; when it is missing or cannot be
loaded the call raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libsiggate.so")

SIGGATE_OK = 0
SIGGATE_EINVAL = -1
SIGGATE_EUNSUPPORTED = -2
SIGGATE_EWORKSPACE = -3
SIGGATE_EHIP = -4
SIGGATE_ESCRATCH = -5
SIGGATE_SCRATCH_BYTES = 128 << 20

# Symbols declared in include/siggate.h
EXPORTS = ("siggate_workspace_bytes", "siggate_forward", "siggate_forward_noalloc",
           "siggate_dispatch",
           "siggate_combine", "siggate_ep_send_splits", "siggate_ep_regroup",
           "siggate_ep_workspace_bytes", "siggate_ep_dedup", "siggate_logits",
           "siggate_status_str")


class SiggateError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {siggate_status_str(status)} ({status})")


class siggate_cfg_t(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("route_scale", ctypes.c_float),
                ("order", ctypes.c_int32), ("score_func", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("mask_zero", ctypes.c_int32),
                ("denom_eps", ctypes.c_float), ("logits_path", ctypes.c_int32)]


@dataclass(frozen=True)
class Cfg:
    """Python mirror of siggate_cfg_t (see include/siggate.h)."""
    T: int
    d: int
    E: int
    n_group: int
    topk_group: int
    top_k: int
    route_scale: float
    order: int = 0
    score_func: int = 0      # 0 sigmoid, 1 softmax
    renorm: int = 0          # 0 iff sigmoid, 1 always, 2 never
    mask_zero: int = 0       # dropped groups: 0 -> -inf, 1 -> 0.0
    denom_eps: float = 0.0   # added to the renormalisation denominator
    logits_path: int = 0     # 0 float32 MFMA, 1 exact bfloat16 three-way split

    def c(self) -> siggate_cfg_t:
        return siggate_cfg_t(self.T, self.d, self.E, self.n_group, self.topk_group,
                             self.top_k, self.route_scale, self.order, self.score_func,
                             self.renorm, self.mask_zero, self.denom_eps, self.logits_path)

    def with_T(self, T: int) -> "Cfg":
        return dataclasses.replace(self, T=T)


_lib = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libsiggate.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                           "or python -m sigmoid_group_limited_amd.build")
    # The tensors and streams this binding passes come from PyTorch's HIP
    # runtime.  Loading torch first makes the library bind to that same
    # runtime; loaded first, it would bind to the system's copy, and a
    # second runtime in the process cannot launch on torch's streams.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i32p, fp = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)
    cfgp = ctypes.POINTER(siggate_cfg_t)
    lib.siggate_workspace_bytes.restype = ctypes.c_size_t
    lib.siggate_workspace_bytes.argtypes = [cfgp]
    lib.siggate_forward.restype = ctypes.c_int
    lib.siggate_forward.argtypes = [vp, vp, vp, cfgp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.siggate_forward_noalloc.restype = ctypes.c_int
    lib.siggate_forward_noalloc.argtypes = [vp, vp, vp, cfgp, vp, vp, vp]
    lib.siggate_dispatch.restype = ctypes.c_int
    lib.siggate_dispatch.argtypes = [vp, vp, cfgp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.siggate_combine.restype = ctypes.c_int
    lib.siggate_combine.argtypes = [vp, vp, vp, cfgp, vp, vp]
    i32 = ctypes.c_int32
    lib.siggate_ep_send_splits.restype = ctypes.c_int
    lib.siggate_ep_send_splits.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.siggate_ep_regroup.restype = ctypes.c_int
    lib.siggate_ep_regroup.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.siggate_ep_workspace_bytes.restype = ctypes.c_size_t
    lib.siggate_ep_workspace_bytes.argtypes = [cfgp, i32]
    lib.siggate_ep_dedup.restype = ctypes.c_int
    lib.siggate_ep_dedup.argtypes = [vp, cfgp, i32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.siggate_logits.restype = ctypes.c_int
    lib.siggate_logits.argtypes = [vp, vp, cfgp, vp, vp, ctypes.c_size_t, vp]
    lib.siggate_status_str.restype = ctypes.c_char_p
    lib.siggate_status_str.argtypes = [ctypes.c_int]
    del i32p, fp
    _lib = lib
    return lib


def siggate_status_str(status: int) -> str:
    return load_library().siggate_status_str(int(status)).decode()


def siggate_workspace_bytes(cfg: Cfg) -> int:
    c = cfg.c()
    return int(load_library().siggate_workspace_bytes(ctypes.byref(c)))


# ---------------------------------------------------------------------------
# torch-facing wrappers (torch is imported lazily: plumbing only)

def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream(stream) -> int | None:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _on_stream(stream):
    """Context in which the wrappers allocate their workspace and outputs:
    the stream the kernels will run on.  The caching allocator ties a block
    to the stream current at its allocation, so a workspace released on
    return is not handed to other work before this call's kernels are done
    with it.  stream may be None (the current stream), a torch stream, or a
    raw hipStream_t handle."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream))
    return torch.cuda.stream(stream)


def _check_dev(name, t, dtype_bytes=None, numel=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype_bytes is not None and t.element_size() != dtype_bytes:
        raise ValueError(f"{name} has element size {t.element_size()}, expected {dtype_bytes}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def workspace(cfg: Cfg, device=None):
    """A device byte tensor large enough for ``cfg`` (at least 256 bytes)."""
    import torch
    n = max(256, siggate_workspace_bytes(cfg))
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def siggate_forward(x, W, bias, cfg: Cfg, weights=None, indices=None, ws=None, stream=None):
    """Gate: returns (weights float32 [T, top_k], indices int32 [T, top_k]).
    x is bfloat16 (or int16 bit patterns) [T, d]; W float32 [E, d]; bias
    float32 [E] or None (the no-bias variant)."""
    import torch
    T, K = cfg.T, cfg.top_k
    dev = x.device
    with _on_stream(stream):
        if weights is None:
            weights = torch.empty((T, K), dtype=torch.float32, device=dev)
        if indices is None:
            indices = torch.empty((T, K), dtype=torch.int32, device=dev)
        if ws is None:
            ws = workspace(cfg, dev)
    _check_dev("x", x, 2, cfg.T * cfg.d)
    _check_dev("W", W, 4, cfg.E * cfg.d)
    if bias is not None:
        _check_dev("bias", bias, 4, cfg.E)
    _check_dev("weights", weights, 4, T * K)
    _check_dev("indices", indices, 4, T * K)
    c = cfg.c()
    rc = load_library().siggate_forward(_ptr(x), _ptr(W), _ptr(bias), ctypes.byref(c),
                                        _ptr(weights), _ptr(indices), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_forward")
    return weights, indices


def siggate_forward_noalloc(x, W, bias, cfg: Cfg, weights=None, indices=None, stream=None):
    """Gate on the library's static device scratch (no workspace argument;
    the library allocates nothing).  Outputs not given are allocated here,
    on the call's stream."""
    import torch
    T, K = cfg.T, cfg.top_k
    dev = x.device
    with _on_stream(stream):
        if weights is None:
            weights = torch.empty((T, K), dtype=torch.float32, device=dev)
        if indices is None:
            indices = torch.empty((T, K), dtype=torch.int32, device=dev)
    _check_dev("x", x, 2, cfg.T * cfg.d)
    _check_dev("W", W, 4, cfg.E * cfg.d)
    if bias is not None:
        _check_dev("bias", bias, 4, cfg.E)
    _check_dev("weights", weights, 4, T * K)
    _check_dev("indices", indices, 4, T * K)
    c = cfg.c()
    rc = load_library().siggate_forward_noalloc(_ptr(x), _ptr(W), _ptr(bias), ctypes.byref(c),
                                                _ptr(weights), _ptr(indices), _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_forward_noalloc")
    return weights, indices


def siggate_logits(x, W, cfg: Cfg, logits=None, ws=None, stream=None):
    """float32 logits [T, E] as siggate_forward computes them."""
    import torch
    with _on_stream(stream):
        if logits is None:
            logits = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = workspace(cfg, x.device)
    _check_dev("x", x, 2, cfg.T * cfg.d)
    _check_dev("W", W, 4, cfg.E * cfg.d)
    _check_dev("logits", logits, 4, cfg.T * cfg.E)
    c = cfg.c()
    rc = load_library().siggate_logits(_ptr(x), _ptr(W), ctypes.byref(c), _ptr(logits),
                                       _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_logits")
    return logits


@dataclass
class DispatchOut:
    tokens_per_expert: object   # int32 [E]
    offsets: object             # int32 [E+1] or None
    perm: object                # int32 [T*K]
    dest: object                # int32 [T*K] or None
    permuted_x: object          # bfloat16 [T*K, d]


def siggate_dispatch(x, indices, cfg: Cfg, out: DispatchOut | None = None, ws=None,
                     stream=None, with_offsets: bool = True,
                     with_dest: bool = True) -> DispatchOut:
    """Dispatch: per-expert counts, offsets, stable expert-major permutation,
    its inverse and the permuted rows."""
    import torch
    T, K, E, d = cfg.T, cfg.top_k, cfg.E, cfg.d
    dev = x.device
    with _on_stream(stream):
        if out is None:
            out = DispatchOut(
                torch.empty(E, dtype=torch.int32, device=dev),
                torch.empty(E + 1, dtype=torch.int32, device=dev) if with_offsets else None,
                torch.empty(T * K, dtype=torch.int32, device=dev),
                torch.empty(T * K, dtype=torch.int32, device=dev) if with_dest else None,
                torch.empty((T * K, d), dtype=x.dtype, device=dev))
        if ws is None:
            ws = workspace(cfg, dev)
    _check_dev("x", x, 2, T * d)
    _check_dev("indices", indices, 4, T * K)
    _check_dev("tokens_per_expert", out.tokens_per_expert, 4, E)
    _check_dev("offsets", out.offsets, 4, E + 1)
    _check_dev("perm", out.perm, 4, T * K)
    _check_dev("dest", out.dest, 4, T * K)
    _check_dev("permuted_x", out.permuted_x, 2, T * K * d)
    c = cfg.c()
    rc = load_library().siggate_dispatch(
        _ptr(x), _ptr(indices), ctypes.byref(c), _ptr(out.tokens_per_expert),
        _ptr(out.offsets), _ptr(out.perm), _ptr(out.dest), _ptr(out.permuted_x),
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_dispatch")
    return out


def siggate_combine(expert_out, weights, dest, cfg: Cfg, y=None, stream=None):
    """y[t] = bf16(sum_k weights[t,k] * expert_out[dest[t*K+k]]) : bfloat16
    [T, d] from expert outputs in dispatch order [T*K, d]."""
    import torch
    T, K, d = cfg.T, cfg.top_k, cfg.d
    if y is None:
        with _on_stream(stream):
            y = torch.empty((T, d), dtype=expert_out.dtype, device=expert_out.device)
    _check_dev("expert_out", expert_out, 2, T * K * d)
    _check_dev("weights", weights, 4, T * K)
    _check_dev("dest", dest, 4, T * K)
    _check_dev("y", y, 2, T * d)
    c = cfg.c()
    rc = load_library().siggate_combine(_ptr(expert_out), _ptr(weights), _ptr(dest),
                                        ctypes.byref(c), _ptr(y), _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_combine")
    return y


# -- expert-parallel metadata ------------------------------------------------

def siggate_ep_send_splits(tokens_per_expert, ep_size: int, stream=None):
    """(send_counts [ep_size], send_offsets [ep_size + 1]) int32."""
    import torch
    E = tokens_per_expert.numel()
    _check_dev("tokens_per_expert", tokens_per_expert, 4, E)
    dev = tokens_per_expert.device
    with _on_stream(stream):
        counts = torch.empty(ep_size, dtype=torch.int32, device=dev)
        offsets = torch.empty(ep_size + 1, dtype=torch.int32, device=dev)
    rc = load_library().siggate_ep_send_splits(_ptr(tokens_per_expert), E, ep_size,
                                               _ptr(counts), _ptr(offsets), _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_ep_send_splits")
    return counts, offsets


def siggate_ep_regroup(counts, capacity: int, stream=None):
    """counts [ep_size, per] int32 -> (local_counts [per], regroup [capacity])."""
    import torch
    R, per = counts.shape
    _check_dev("counts", counts, 4, R * per)
    dev = counts.device
    with _on_stream(stream):
        local = torch.empty(per, dtype=torch.int32, device=dev)
        regroup = torch.empty(max(capacity, 1), dtype=torch.int32, device=dev)
    rc = load_library().siggate_ep_regroup(_ptr(counts), R, per, capacity, _ptr(local),
                                           _ptr(regroup), _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_ep_regroup")
    return local, regroup[:capacity]


def siggate_ep_workspace_bytes(cfg: Cfg, ep_size: int) -> int:
    c = cfg.c()
    return int(load_library().siggate_ep_workspace_bytes(ctypes.byref(c), ep_size))


def siggate_ep_dedup(indices, cfg: Cfg, ep_size: int, ws=None, stream=None):
    """(rank_counts, rank_offsets, send_tokens [T*K], pair_slot [T*K]); the
    first rank_offsets[-1] entries of send_tokens are valid."""
    import torch
    T, K = cfg.T, cfg.top_k
    _check_dev("indices", indices, 4, T * K)
    dev = indices.device
    with _on_stream(stream):
        if ws is None:
            ws = torch.empty(max(256, siggate_ep_workspace_bytes(cfg, ep_size)),
                             dtype=torch.uint8, device=dev)
        rcnt = torch.empty(ep_size, dtype=torch.int32, device=dev)
        roff = torch.empty(ep_size + 1, dtype=torch.int32, device=dev)
        send = torch.empty(max(T * K, 1), dtype=torch.int32, device=dev)
        slot = torch.empty(max(T * K, 1), dtype=torch.int32, device=dev)
    c = cfg.c()
    rc = load_library().siggate_ep_dedup(_ptr(indices), ctypes.byref(c), ep_size, _ptr(rcnt),
                                         _ptr(roff), _ptr(send), _ptr(slot), _ptr(ws),
                                         ws.numel() * ws.element_size(), _stream(stream))
    if rc != SIGGATE_OK:
        raise SiggateError(rc, "siggate_ep_dedup")
    return rcnt, roff, send, slot[:T * K]
