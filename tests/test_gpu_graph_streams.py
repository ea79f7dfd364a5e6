"""The library's calls under HIP graph capture and on concurrent streams.
Needs an MI355X.

The library launches kernels only (no memsets, no allocation), so a whole
route -- gate, dispatch, combine -- can be captured in one graph.  Each
replay here follows eager work that rewrites the input, and every replay is
checked against eager calls on the same input."""
import numpy as np
import pytest

import sigmoid_group_limited_amd as sg
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


def _route(x, W, b, cfg, bufs):
    w, i, ws, out, y = bufs
    sg.siggate_forward(x, W, b, cfg, w, i, ws)
    sg.siggate_dispatch(x, i, cfg, out, ws)
    sg.siggate_combine(out.permuted_x, w, out.dest, cfg, y)


def _bufs(cfg):
    T, K, E, d = cfg.T, cfg.top_k, cfg.E, cfg.d
    dev = "cuda"
    out = sg.DispatchOut(torch.empty(E, dtype=torch.int32, device=dev),
                         torch.empty(E + 1, dtype=torch.int32, device=dev),
                         torch.empty(T * K, dtype=torch.int32, device=dev),
                         torch.empty(T * K, dtype=torch.int32, device=dev),
                         torch.empty((T * K, d), dtype=torch.bfloat16, device=dev))
    return (torch.empty((T, K), dtype=torch.float32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev),
            sg.workspace(cfg, dev), out, torch.empty((T, d), dtype=torch.bfloat16, device=dev))


def _snapshot(bufs):
    w, i, _, out, y = bufs
    return [t.clone() for t in (w, i, out.tokens_per_expert, out.offsets, out.perm, out.dest,
                                out.permuted_x, y)]


@pytest.mark.parametrize("gc,T,d", [(wl.KIMI_K2, 256, 7168), (wl.DSV3, 64, 7168),
                                    (wl.DSV3, 2048, 1024), (wl.KIMI_K2, 4096, 7168),
                                    (wl.KIMI_K2, 16384, 512)],
                         ids=["kimi_T256", "dsv3_T64", "dsv3_T2048", "kimi_T4096", "kimi_T16384"])
@pytest.mark.parametrize("lp", [0, 1], ids=["fp32", "bf16x3"])
def test_graph_replay_matches_eager(gc, T, d, lp):
    say(f"[graph] E={gc.n_experts} T={T} d={d} logits_path={lp}")
    cfg = sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                 logits_path=lp)
    inputs = [wl.make_gate_inputs(T, d, gc, seed=s) for s in (21, 22, 23)]
    x = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    W = torch.from_numpy(inputs[0].W).cuda()
    b = torch.from_numpy(inputs[0].bias).cuda()
    graph_bufs, eager_bufs = _bufs(cfg), _bufs(cfg)
    x.copy_(torch.from_numpy(inputs[0].x.view(np.int16)).cuda().view(torch.bfloat16))
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        _route(x, W, b, cfg, graph_bufs)          # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            _route(x, W, b, cfg, graph_bufs)
    torch.cuda.synchronize()
    for rep, gi in enumerate(inputs * 2):
        # eager work between replays: a new input, then the reference route
        x.copy_(torch.from_numpy(gi.x.view(np.int16)).cuda().view(torch.bfloat16))
        _route(x, W, b, cfg, eager_bufs)
        torch.cuda.synchronize()
        want = _snapshot(eager_bufs)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(graph_bufs)
        for k, (a, c) in enumerate(zip(got, want)):
            assert torch.equal(a, c), f"replay {rep}: output {k} differs from the eager call"


@pytest.mark.parametrize("lp", [0, 1], ids=["fp32", "bf16x3"])
def test_concurrent_streams_match_sequential(lp):
    """Independent batches on two streams at once, each with its own
    workspace and outputs, give exactly the sequential results."""
    gc = wl.DSV3
    cfgs = [sg.Cfg(T, 7168, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                   logits_path=lp) for T in (16384, 256)]
    gis = [wl.make_gate_inputs(c.T, 7168, gc, seed=31 + k) for k, c in enumerate(cfgs)]
    xs = [torch.from_numpy(g.x.view(np.int16)).cuda().view(torch.bfloat16) for g in gis]
    W = torch.from_numpy(gis[0].W).cuda()
    b = torch.from_numpy(gis[0].bias).cuda()
    seq = []
    for x, c in zip(xs, cfgs):
        bufs = _bufs(c)
        _route(x, W, b, c, bufs)
        torch.cuda.synchronize()
        seq.append(_snapshot(bufs))
    par_bufs = [_bufs(c) for c in cfgs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for _ in range(3):
        for s, x, c, bufs in zip(streams, xs, cfgs, par_bufs):
            with torch.cuda.stream(s):
                _route(x, W, b, c, bufs)
    torch.cuda.synchronize()
    for want, bufs in zip(seq, par_bufs):
        for k, (a, c) in enumerate(zip(_snapshot(bufs), want)):
            assert torch.equal(a, c), f"output {k} differs from the sequential run"


@pytest.mark.parametrize("lp", [0, 1], ids=["fp32", "bf16x3"])
@pytest.mark.parametrize("raw", [False, True], ids=["torch_stream", "raw_handle"])
def test_explicit_stream_without_workspace(lp, raw):
    """A call given stream= but no workspace allocates it (and its outputs)
    on that stream: work queued right after on the current stream, which
    allocates and overwrites memory of the same sizes, cannot take the
    workspace while the call's kernels still use it."""
    gc = wl.KIMI_K2
    T, d = 4096, 7168                     # split GEMM: partial logits in the workspace
    cfg = sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                 logits_path=lp)
    gi = wl.make_gate_inputs(T, d, gc, seed=41)
    x = torch.from_numpy(gi.x.view(np.int16)).cuda().view(torch.bfloat16)
    W = torch.from_numpy(gi.W).cuda()
    b = torch.from_numpy(gi.bias).cuda()
    w0, i0 = sg.siggate_forward(x, W, b, cfg)
    out0 = sg.siggate_dispatch(x, i0, cfg)
    torch.cuda.synchronize()
    nbytes = max(256, sg.siggate_workspace_bytes(cfg))
    side = torch.cuda.Stream()
    handle = int(side.cuda_stream) if raw else side
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        w, i = sg.siggate_forward(x, W, b, cfg, stream=handle)
        junk = [torch.full((nbytes // 4,), -1.0, device="cuda") for _ in range(4)]
        side.synchronize()
        out = sg.siggate_dispatch(x, i, cfg, stream=handle)
        junk += [torch.full((nbytes // 4,), 7.0, device="cuda") for _ in range(4)]
        torch.cuda.synchronize()
        del junk
        assert torch.equal(w, w0) and torch.equal(i, i0), f"rep {rep}: gate differs"
        assert torch.equal(out.perm, out0.perm), f"rep {rep}: perm differs"
        assert torch.equal(out.permuted_x, out0.permuted_x), f"rep {rep}: rows differ"
