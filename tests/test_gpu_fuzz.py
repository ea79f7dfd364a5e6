"""Seeded random configurations against the CPU oracle, on both logits
routes.  Needs an MI355X.

Each case draws a supported configuration -- E, a power-of-two group count
with at least two experts per group, topk_group, top_k, T, d (a multiple of
8), the output order, the scoring function, the renormalisation switch, the
fill of dropped groups, the denominator epsilon, with or without a bias --
and compares the gate with the oracle under the same rules as the other
parity tests (indices bit-exact outside the 1e-6 margin exemption, weights
1e-5 relative), then the dispatch of the GPU's indices in full."""
import dataclasses

import numpy as np
import pytest

import oracle
import sigmoid_group_limited_amd as sg
from sigmoid_group_limited_amd import workloads as wl
from parity import compare_dispatch, compare_gate, dev_inputs, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_CASES = 40


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


def draw_case(seed: int):
    """A supported configuration and its sizes, from one seed."""
    r = np.random.default_rng(1000 + seed)
    E = int(r.choice([64, 128, 192, 256, 320, 384, 448, 512]))
    groups = [g for g in (1, 2, 4, 8, 16, 32, 64) if E % g == 0 and E // g >= 2]
    G = int(r.choice(groups))
    KG = int(r.integers(1, G + 1))
    K = int(r.integers(1, min(8, KG * (E // G)) + 1))
    T = int(r.choice([1, 2, 7, 63, 64, 65, 300, 511, 1000, 1023, 1024, 1500, 3000, 4100, 6000]))
    d = int(8 * r.integers(1, 257))
    opts = dict(order=int(r.integers(0, 2)), score_func=int(r.random() < 0.25),
                renorm=int(r.choice([0, 0, 1, 2])), mask_zero=int(r.random() < 0.25),
                denom_eps=float(r.choice([0.0, 1e-20])))
    no_bias = bool(r.random() < 0.2)
    scale = float(r.choice([1.0, 2.5, 2.827]))
    return wl.GateConfig(E, G, KG, K, scale), T, d, opts, no_bias


@pytest.mark.parametrize("seed", range(N_CASES))
@pytest.mark.parametrize("lp", [0, 1], ids=["fp32", "bf16x3"])
def test_random_configuration(o, seed, lp):
    gc, T, d, opts, no_bias = draw_case(seed)
    say(f"[fuzz {seed}] E={gc.n_experts} G={gc.n_group} KG={gc.topk_group} K={gc.top_k} "
        f"T={T} d={d} {opts} no_bias={no_bias} logits_path={lp}")
    gi = wl.make_gate_inputs(T, d, gc, seed=seed)
    cfg = dataclasses.replace(sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k,
                                     gc.route_scale, logits_path=lp), **opts)
    x, W, b = dev_inputs(gi)
    bias = None if no_bias else b
    w, i = sg.siggate_forward(x, W, bias, cfg)
    torch.cuda.synchronize()
    w_np, i_np = w.cpu().numpy(), i.cpu().numpy()
    ref = o.gate(gi.x, gi.W, None if no_bias else gi.bias, gc.n_group, gc.topk_group, gc.top_k,
                 gc.route_scale, cfg.order, score_func=cfg.score_func, renorm=cfg.renorm,
                 mask_zero=cfg.mask_zero, denom_eps=cfg.denom_eps, with_scores=True)
    renorm = cfg.renorm == 1 or (cfg.renorm == 0 and cfg.score_func == 0)
    tie = dict(topk_group=gc.topk_group, renorm=renorm, mask_zero=cfg.mask_zero,
               denom_eps=cfg.denom_eps)
    if cfg.order == 0:
        stats = compare_gate(w_np, i_np, ref, gc.route_scale, check_sum=renorm, **tie)
    else:
        # compare as sets (sorted by id); the order itself is pinned elsewhere
        si = np.argsort(i_np, axis=1, kind="stable")
        sr = np.argsort(ref.indices, axis=1, kind="stable")
        ref_sorted = oracle.GateResult(np.take_along_axis(ref.weights, sr, 1),
                                       np.take_along_axis(ref.indices, sr, 1), ref.margins,
                                       ref.scores)
        stats = compare_gate(np.take_along_axis(w_np, si, 1), np.take_along_axis(i_np, si, 1),
                             ref_sorted, gc.route_scale, check_sum=renorm, **tie)
    assert i_np.min() >= 0 and i_np.max() < gc.n_experts
    say(f"    {stats}")
    out = sg.siggate_dispatch(x, i, cfg)
    torch.cuda.synchronize()
    dref = o.dispatch(i_np, gc.n_experts)
    compare_dispatch(out, dref, i_np, gi.x, gc.top_k, np.arange(len(dref.perm)), o)
