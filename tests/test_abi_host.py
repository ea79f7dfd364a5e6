"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every function include/siggate.h declares, sizes workspaces, and rejects bad
arguments before anything is enqueued."""
import ctypes
import dataclasses
import os
import re

import numpy as np
import pytest

import sigmoid_group_limited_amd as sg
from sigmoid_group_limited_amd import binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "siggate.h")

DSV3 = sg.Cfg(T=64, d=7168, E=256, n_group=8, topk_group=4, top_k=8, route_scale=2.5)
KIMI = sg.Cfg(T=256, d=7168, E=384, n_group=1, topk_group=1, top_k=8, route_scale=2.827)
# 16-byte aligned and never dereferenced: every call below fails a host-side
# check before anything is enqueued
FAKE = 0x10000


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(siggate_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sg.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), f"libsiggate.so does not export {n}"
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_exports_nothing_else(lib):
    """The library's dynamic symbol table defines exactly the functions
    siggate.h declares: internal C++ symbols stay hidden."""
    import subprocess
    res = subprocess.run(["nm", "-D", "--defined-only", binding.LIBRARY],
                         capture_output=True, text=True, check=True)
    defined = sorted(ln.split()[-1] for ln in res.stdout.splitlines() if ln.strip())
    assert defined == declared_functions()


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert sg.siggate_status_str(code).startswith("SIGGATE_")
    assert "unknown" in sg.siggate_status_str(7)


def test_workspace_bytes():
    # fused path at large T needs only the dispatch workspace
    big = DSV3.with_T(16384)
    nb = 16384 // 256
    dispatch = 2 * nb * 256 * 4 + 16384 * 8 * 4
    assert sg.siggate_workspace_bytes(big) == dispatch
    # split-k at small T needs partial logits
    assert sg.siggate_workspace_bytes(KIMI) >= 256 * 384 * 4 * 2
    assert sg.siggate_workspace_bytes(sg.Cfg(0, 7168, 256, 8, 4, 8, 2.5)) == 0
    # the bfloat16 three-way route always writes partial logits (at least one
    # slice), for the reduction that runs the selection
    x3 = dataclasses.replace(big, logits_path=1)
    assert sg.siggate_workspace_bytes(x3) >= 16384 * 256 * 4
    # large batches: one slice of partial logits, then the three bf16 planes
    kimi_big = dataclasses.replace(KIMI.with_T(16384), logits_path=1)
    assert sg.siggate_workspace_bytes(kimi_big) == 16384 * 384 * 4 + 3 * 384 * 7168 * 2
    assert sg.siggate_workspace_bytes(dataclasses.replace(KIMI, logits_path=1)) >= 256 * 384 * 4
    # E an odd multiple of 64: float32 partial rows span whole 128-expert
    # tiles, bfloat16x3 ones exactly E
    e192 = sg.Cfg(256, 7168, 192, 8, 4, 8, 2.5)
    fp = sg.siggate_workspace_bytes(e192)
    x3 = sg.siggate_workspace_bytes(dataclasses.replace(e192, logits_path=1))
    assert fp % (256 * 256 * 4) == 0 and fp >= 256 * 256 * 4
    assert x3 % (256 * 192 * 4) == 0 and x3 >= 256 * 192 * 4


def call_forward(cfg, x=FAKE, W=FAKE, bias=FAKE, w=FAKE, i=FAKE, ws=FAKE, ws_bytes=1 << 40):
    c = cfg.c()
    return sg.load_library().siggate_forward(x, W, bias, ctypes.byref(c), w, i, ws, ws_bytes, None)


def call_dispatch(cfg, x=FAKE, idx=FAKE, tpe=FAKE, off=FAKE, perm=FAKE, dest=FAKE, px=FAKE,
                  ws=FAKE, ws_bytes=1 << 40):
    c = cfg.c()
    return sg.load_library().siggate_dispatch(x, idx, ctypes.byref(c), tpe, off, perm, dest, px,
                                              ws, ws_bytes, None)


@pytest.mark.parametrize("bad", [
    dict(n_group=3), dict(topk_group=0), dict(topk_group=9), dict(top_k=0),
    dict(top_k=33, topk_group=1), dict(order=2), dict(T=-1), dict(d=0),
    dict(route_scale=float("nan")), dict(E=256, n_group=256, topk_group=1, top_k=1),
    dict(score_func=2), dict(renorm=3), dict(renorm=-1), dict(mask_zero=2),
    dict(denom_eps=-1e-20), dict(denom_eps=float("nan")), dict(logits_path=2), dict(logits_path=-1),
])
def test_forward_rejects_invalid(bad):
    fields = DSV3.__dict__ | bad
    assert call_forward(sg.Cfg(**fields)) == binding.SIGGATE_EINVAL


@pytest.mark.parametrize("unsup", [
    dict(E=96, n_group=8), dict(E=640, n_group=8), dict(E=576, n_group=8), dict(E=160, n_group=8),
    dict(n_group=128, topk_group=4, top_k=4), dict(top_k=9, topk_group=8, n_group=8),
    dict(d=7164),
])
def test_forward_rejects_unsupported(unsup):
    fields = DSV3.__dict__ | unsup
    assert call_forward(sg.Cfg(**fields)) == binding.SIGGATE_EUNSUPPORTED


def test_forward_pointer_and_workspace_checks():
    assert call_forward(DSV3, x=0) == binding.SIGGATE_EINVAL
    assert call_forward(DSV3, W=0) == binding.SIGGATE_EINVAL
    assert call_forward(DSV3, W=FAKE + 4) == binding.SIGGATE_EINVAL
    assert call_forward(DSV3, w=FAKE + 8) == binding.SIGGATE_EINVAL
    need = sg.siggate_workspace_bytes(DSV3)
    assert need > 0
    assert call_forward(DSV3, ws_bytes=need - 256) == binding.SIGGATE_EWORKSPACE
    assert call_forward(DSV3, ws=0) == binding.SIGGATE_EWORKSPACE
    # T = 0 enqueues nothing and needs no data pointers
    assert call_forward(DSV3.with_T(0), x=0, w=0, i=0, ws=0, ws_bytes=0) == binding.SIGGATE_OK


def call_noalloc(cfg, x=FAKE, W=FAKE, bias=FAKE, w=FAKE, i=FAKE):
    c = cfg.c()
    return sg.load_library().siggate_forward_noalloc(x, W, bias, ctypes.byref(c), w, i, None)


@pytest.mark.parametrize("bad", [dict(n_group=3), dict(top_k=0), dict(order=2), dict(T=-1),
                                 dict(logits_path=2)])
def test_noalloc_rejects_invalid(bad):
    assert call_noalloc(sg.Cfg(**(DSV3.__dict__ | bad))) == binding.SIGGATE_EINVAL


def test_noalloc_rejects_beyond_scratch():
    """Checked on the host before the scratch is looked up or anything is
    enqueued: an unsupported shape, then a workspace need above the scratch."""
    assert call_noalloc(sg.Cfg(**(DSV3.__dict__ | dict(E=640, n_group=8)))) == \
        binding.SIGGATE_EUNSUPPORTED
    big = dataclasses.replace(KIMI.with_T(131072), logits_path=1)
    assert sg.siggate_workspace_bytes(big) > binding.SIGGATE_SCRATCH_BYTES
    assert call_noalloc(big) == binding.SIGGATE_ESCRATCH
    # every batch of the float32 route fits
    for T in (1, 256, 4096, 6144, 8191, 65536):
        assert sg.siggate_workspace_bytes(KIMI.with_T(T)) <= binding.SIGGATE_SCRATCH_BYTES


def test_float32_plans_fit_the_scratch():
    """The float32 planner skips plans whose partial logits exceed 120 MiB,
    so every batch of that route fits the no-allocation scratch, at every
    supported expert count and row length."""
    rng = np.random.default_rng(7)
    Ts = sorted(set([1, 2, 255, 256, 257] + [int(t) for t in np.geomspace(300, 300000, 60)] +
                    [int(t) for t in rng.integers(1, 70000, 60)]))
    for E in range(64, 513, 64):
        for d in (96, 1024, 7168):
            for T in Ts:
                c = sg.Cfg(T, d, E, 1, 1, 8, 1.0)
                assert sg.siggate_workspace_bytes(c) <= binding.SIGGATE_SCRATCH_BYTES, (E, d, T)


def test_scratch_size_matches_header():
    with open(HEADER) as f:
        text = f.read()
    m = re.search(r"#define SIGGATE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.SIGGATE_SCRATCH_BYTES


def test_dispatch_checks():
    cfg = DSV3.with_T(1000)
    assert call_dispatch(cfg.__class__(**(cfg.__dict__ | dict(E=513)))) == \
        binding.SIGGATE_EUNSUPPORTED
    assert call_dispatch(cfg.__class__(**(cfg.__dict__ | dict(top_k=9, E=300)))) == \
        binding.SIGGATE_EUNSUPPORTED
    assert call_dispatch(cfg.__class__(**(cfg.__dict__ | dict(top_k=0)))) == binding.SIGGATE_EINVAL
    assert call_dispatch(cfg, tpe=0) == binding.SIGGATE_EINVAL
    assert call_dispatch(cfg, perm=FAKE + 4) == binding.SIGGATE_EINVAL
    need_with_dest = sg.siggate_workspace_bytes(cfg)
    nb = (1000 + 255) // 256
    cnt = ((nb * 256 * 4 + 255) // 256) * 256
    # without a caller-provided dest the workspace must also hold it
    assert call_dispatch(cfg, dest=0, ws_bytes=2 * cnt) == binding.SIGGATE_EWORKSPACE
    assert need_with_dest >= 2 * cnt + 1000 * 8 * 4


def test_python_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((64, 7168), dtype=torch.bfloat16)
    W = torch.zeros((256, 7168))
    b = torch.zeros(256)
    with pytest.raises(ValueError):
        sg.siggate_forward(x, W, b, DSV3, weights=torch.zeros((64, 8)),
                           indices=torch.zeros((64, 8), dtype=torch.int32),
                           ws=torch.zeros(1 << 20, dtype=torch.uint8))


def call_combine(cfg, out=FAKE, w=FAKE, dest=FAKE, y=FAKE):
    c = cfg.c()
    return sg.load_library().siggate_combine(out, w, dest, ctypes.byref(c), y, None)


def test_combine_checks():
    cfg = DSV3.with_T(100)
    assert call_combine(cfg.__class__(**(cfg.__dict__ | dict(top_k=9)))) == \
        binding.SIGGATE_EUNSUPPORTED
    assert call_combine(cfg.__class__(**(cfg.__dict__ | dict(d=12)))) == \
        binding.SIGGATE_EUNSUPPORTED
    assert call_combine(cfg.__class__(**(cfg.__dict__ | dict(top_k=0)))) == binding.SIGGATE_EINVAL
    assert call_combine(cfg, out=0) == binding.SIGGATE_EINVAL
    assert call_combine(cfg, dest=FAKE + 4) == binding.SIGGATE_EINVAL
    assert call_combine(cfg.with_T(0), out=0, w=0, dest=0, y=0) == binding.SIGGATE_OK


def test_cfg_struct_layout():
    """The ctypes mirror matches the C struct: 13 four-byte fields."""
    assert ctypes.sizeof(binding.siggate_cfg_t) == 52
    names = [f[0] for f in binding.siggate_cfg_t._fields_]
    with open(HEADER) as f:
        text = f.read()
    body = text[text.index("typedef struct siggate_cfg {"):text.index("} siggate_cfg_t;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    declared = re.findall(r"(?:int32_t|float)\s+(\w+);", body)
    assert declared == names


def test_ep_checks():
    lib = sg.load_library()
    c = DSV3.with_T(100).c()
    assert lib.siggate_ep_send_splits(FAKE, 256, 3, FAKE, FAKE, None) == binding.SIGGATE_EINVAL
    assert lib.siggate_ep_send_splits(FAKE, 256, 0, FAKE, FAKE, None) == binding.SIGGATE_EINVAL
    assert lib.siggate_ep_send_splits(0, 256, 8, FAKE, FAKE, None) == binding.SIGGATE_EINVAL
    assert lib.siggate_ep_regroup(FAKE, 8, 0, 10, FAKE, FAKE, None) == binding.SIGGATE_EINVAL
    assert lib.siggate_ep_regroup(FAKE, 64, 128, 10, FAKE, FAKE, None) == \
        binding.SIGGATE_EUNSUPPORTED
    assert lib.siggate_ep_workspace_bytes(ctypes.byref(c), 3) == 0
    need = lib.siggate_ep_workspace_bytes(ctypes.byref(c), 8)
    assert need >= 3 * 100 * 8 * 4
    assert lib.siggate_ep_dedup(FAKE, ctypes.byref(c), 3, FAKE, FAKE, FAKE, FAKE, FAKE,
                                1 << 30, None) == binding.SIGGATE_EINVAL
    assert lib.siggate_ep_dedup(FAKE, ctypes.byref(c), 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                need - 256, None) == binding.SIGGATE_EWORKSPACE
    assert lib.siggate_ep_dedup(FAKE, ctypes.byref(c), 8, FAKE, FAKE, FAKE + 4, FAKE, FAKE,
                                need, None) == binding.SIGGATE_EINVAL
