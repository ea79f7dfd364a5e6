"""Parity of the expert-parallel metadata calls with the CPU oracle, through
the C ABI.  Needs an MI355X."""
import numpy as np
import pytest

import oracle
import sigmoid_group_limited_amd as sg
from sigmoid_group_limited_amd import workloads as wl
from parity import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sg.load_library()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("E,R", [(256, 8), (384, 8), (384, 3), (384, 384), (128, 1)])
def test_ep_send_splits(o, E, R):
    rng = np.random.default_rng(E + R)
    tpe = rng.integers(0, 5000, size=E).astype(np.int32)
    c, off = sg.siggate_ep_send_splits(torch.from_numpy(tpe).cuda(), R)
    wc, woff = o.ep_send_splits(tpe, R)
    assert np.array_equal(c.cpu().numpy(), wc) and np.array_equal(off.cpu().numpy(), woff)


@pytest.mark.parametrize("R,per,hi", [(8, 32, 600), (8, 48, 40), (3, 5, 3), (1, 384, 9), (64, 4, 0)])
def test_ep_regroup(o, R, per, hi):
    rng = np.random.default_rng(R * per)
    counts = rng.integers(0, hi + 1, size=(R, per)).astype(np.int32)
    n = int(counts.sum())
    lc, rg = sg.siggate_ep_regroup(torch.from_numpy(counts).cuda(), n)
    wlc, wrg = o.ep_regroup(counts)
    assert np.array_equal(lc.cpu().numpy(), wlc)
    assert np.array_equal(rg.cpu().numpy(), wrg)


@pytest.mark.parametrize("T,K,E,R", [(16384, 8, 256, 8), (16384, 8, 384, 8), (1000, 8, 384, 48),
                                     (257, 4, 128, 4), (0, 8, 256, 8), (300, 8, 256, 1)])
def test_ep_dedup(o, T, K, E, R):
    say(f"[ep dedup] T={T} K={K} E={E} R={R}")
    if T:
        idx = wl.random_indices(T, K, E, seed=T + R)
    else:
        idx = np.zeros((0, K), np.int32)
    cfg = sg.Cfg(T, 8, E, 1, 1, K, 1.0)
    rcnt, roff, send, slot = sg.siggate_ep_dedup(torch.from_numpy(idx).cuda(), cfg, R)
    torch.cuda.synchronize()
    wc, woff, wsend, wslot = o.ep_dedup(idx, E, R)
    assert np.array_equal(rcnt.cpu().numpy(), wc)
    assert np.array_equal(roff.cpu().numpy(), woff)
    total = int(woff[-1])
    assert np.array_equal(send.cpu().numpy()[:total], wsend)
    assert np.array_equal(slot.cpu().numpy(), wslot)
    if T:
        say(f"    pairs {T * K} -> sends {total} ({total / (T * K):.2f})")


def test_ep_dedup_on_gate_indices(o):
    """De-duplication on real group-limited selections (DeepSeek-V3, 8
    ranks = 8 groups): every token reaches at most topk_group = 4 ranks."""
    gc = wl.DSV3
    T, d = 4096, 512
    gi = wl.make_gate_inputs(T, d, gc, seed=77)
    cfg = sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale)
    x = torch.from_numpy(gi.x.view(np.int16)).cuda().view(torch.bfloat16)
    _, idx = sg.siggate_forward(x, torch.from_numpy(gi.W).cuda(), torch.from_numpy(gi.bias).cuda(), cfg)
    rcnt, roff, send, slot = sg.siggate_ep_dedup(idx, cfg, 8)
    idx_np = idx.cpu().numpy()
    wc, woff, wsend, wslot = o.ep_dedup(idx_np, gc.n_experts, 8)
    assert np.array_equal(rcnt.cpu().numpy(), wc) and np.array_equal(slot.cpu().numpy(), wslot)
    assert int(woff[-1]) <= T * gc.topk_group
