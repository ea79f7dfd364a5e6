"""siggate_forward_noalloc: the gate on the library's static device scratch
(no workspace, no allocation), called through the C ABI, against
siggate_forward with a caller workspace on the same inputs.  Needs an MI355X.

Both run the same kernels in the same order, so the outputs must be equal
bit for bit.  Two calls in a row on one device share the scratch: the second,
on a smaller batch, must not see anything of the first."""
import ctypes

import numpy as np
import pytest

import sigmoid_group_limited_amd as sg
from sigmoid_group_limited_amd import binding
from sigmoid_group_limited_amd import workloads as wl
from parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()
    yield
    torch.cuda.synchronize()


def _noalloc_c_abi(x, W, b, cfg):
    """One call through the C ABI (ctypes), outputs allocated here."""
    lib = sg.load_library()
    w = torch.empty((cfg.T, cfg.top_k), dtype=torch.float32, device="cuda")
    i = torch.empty((cfg.T, cfg.top_k), dtype=torch.int32, device="cuda")
    c = cfg.c()
    rc = lib.siggate_forward_noalloc(x.data_ptr(), W.data_ptr(),
                                     None if b is None else b.data_ptr(), ctypes.byref(c),
                                     w.data_ptr(), i.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == binding.SIGGATE_OK, sg.siggate_status_str(rc)
    return w, i


# (model, first T, second smaller T, logits route)
CASES = [(wl.KIMI_K2, 256, 64, 0), (wl.DSV3, 4096, 100, 0), (wl.KIMI_K2, 16384, 256, 0),
         (wl.DSV3, 2048, 33, 1), (wl.KIMI_K2, 256, 7, 1),
         # 192 experts: float32 partial rows padded to whole 128-expert tiles
         (wl.GateConfig(192, 8, 4, 8, 2.5), 300, 40, 0)]


@pytest.mark.parametrize("gc,T1,T2,lp", CASES,
                         ids=[f"E{c[0].n_experts}_T{c[1]}_then_T{c[2]}_lp{c[3]}" for c in CASES])
def test_noalloc_matches_forward(gc, T1, T2, lp):
    say(f"[noalloc] E={gc.n_experts} T={T1} then T={T2} logits_path={lp}")
    d = 7168
    gi = wl.make_gate_inputs(T1, d, gc, seed=T1 + lp)
    x = torch.from_numpy(gi.x.view(np.int16)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(gi.W).cuda()
    b = torch.from_numpy(gi.bias).cuda()
    for T in (T1, T2):
        cfg = sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                     logits_path=lp)
        # the smaller batch takes rows from the end of the first, so that its
        # inputs differ from the rows the first call left in the scratch
        xs = x[T1 - T:].contiguous()
        w0, i0 = sg.siggate_forward(xs, W, b, cfg)
        w1, i1 = _noalloc_c_abi(xs, W, b, cfg)
        torch.cuda.synchronize()
        assert torch.equal(i1, i0), f"T={T}: indices differ from siggate_forward"
        assert torch.equal(w1, w0), f"T={T}: weights differ from siggate_forward"


def test_noalloc_binding_and_variants():
    """The Python wrapper, with no bias and order 1."""
    gc = wl.DSV3
    T, d = 200, 7168
    gi = wl.make_gate_inputs(T, d, gc, seed=5)
    x = torch.from_numpy(gi.x.view(np.int16)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(gi.W).cuda()
    cfg = sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                 order=1)
    w0, i0 = sg.siggate_forward(x, W, None, cfg)
    w1, i1 = sg.siggate_forward_noalloc(x, W, None, cfg)
    torch.cuda.synchronize()
    assert torch.equal(i1, i0) and torch.equal(w1, w0)


def test_noalloc_rejects_beyond_scratch():
    """A configuration whose workspace exceeds the scratch is rejected before
    anything is enqueued, with its own status."""
    gc = wl.KIMI_K2
    cfg = sg.Cfg(131072, 7168, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k,
                 gc.route_scale, logits_path=1)
    assert sg.siggate_workspace_bytes(cfg) > binding.SIGGATE_SCRATCH_BYTES
    x = torch.empty((8, 7168), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((gc.n_experts, 7168), device="cuda")
    lib = sg.load_library()
    c = cfg.c()
    out = torch.empty(16, device="cuda")
    rc = lib.siggate_forward_noalloc(x.data_ptr(), W.data_ptr(), None, ctypes.byref(c),
                                     out.data_ptr(), out.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream)
    assert rc == binding.SIGGATE_ESCRATCH
    assert "SIGGATE_ESCRATCH" in sg.siggate_status_str(rc)
