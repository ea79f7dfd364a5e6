"""Parity of the bfloat16 three-way logits route (cfg.logits_path = 1) with
the CPU oracle, through the C ABI.  Needs an MI355X.

The route must give the same float32 logits as a float32 GEMM up to
summation order, so it is held to the same bar as the float32 route: indices
and dispatch bit-exact outside the 1e-6 margin exemption, weights 1e-5
relative, logits 1e-4 relative.  Two pins are specific to it: one-hot x rows
make every logit a single exact product, so the split of W into three
bfloat16 parts must reproduce W bit for bit over a wide exponent range; and
the two routes' logits are compared with each other."""
import dataclasses

import numpy as np
import pytest

import oracle
import sigmoid_group_limited_amd as sg
from sigmoid_group_limited_amd import workloads as wl
from parity import (LOGIT_RTOL, check_rows_valid, compare_dispatch, compare_gate, dev_inputs, say,
                    score_error)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

X3 = 1


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


def cfg_of(gc: wl.GateConfig, T: int, d: int, order: int = 0) -> sg.Cfg:
    return sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                  order, logits_path=X3)


def oracle_gate(o, gi, cfg, rows=None):
    x = gi.x if rows is None else gi.x[rows]
    return o.gate(x, gi.W, gi.bias, cfg.n_group, cfg.topk_group, cfg.top_k,
                  cfg.route_scale, cfg.order, with_scores=True)


def to_dev_x(x_bits: np.ndarray):
    return torch.from_numpy(x_bits.view(np.int16)).cuda().view(torch.bfloat16)


SMALL = [
    ("dsv3_T64", wl.DSV3, 64, 7168),
    ("kimi_T256", wl.KIMI_K2, 256, 7168),
    ("e128_g4_T333_d1000", wl.GateConfig(128, 4, 2, 6, 1.0), 333, 1000),
    ("e256_g64_T97_d512", wl.GateConfig(256, 64, 16, 8, 2.5), 97, 512),
    ("e384_g8_T1", wl.GateConfig(384, 8, 3, 8, 2.827), 1, 7168),
    ("e384_g2_T129_d264", wl.GateConfig(384, 2, 1, 8, 2.827), 129, 264),
    ("e256_g8_k3_T4100_d256", wl.GateConfig(256, 8, 4, 3, 2.5), 4100, 256),
    ("kimi_T16389_d256", wl.KIMI_K2, 16389, 256),
    ("dsv3_T16447_d200", wl.DSV3, 16447, 200),
    ("e128_g4_T16400_d96", wl.GateConfig(128, 4, 2, 6, 1.0), 16400, 96),
    ("e128_g64_kg4_k8_all_kept_T300_d512", wl.GateConfig(128, 64, 4, 8, 1.0), 300, 512),
    ("e512_g8_T200_d7168", wl.GateConfig(512, 8, 4, 8, 2.5), 200, 7168),
    ("e512_g1_T2100_d1000", wl.GateConfig(512, 1, 1, 8, 2.827), 2100, 1000),
    # odd multiples of 64 experts: 64-expert tiles (and 192-expert ones at 192)
    ("e192_g8_T100_d7168", wl.GateConfig(192, 8, 4, 8, 2.5), 100, 7168),
    ("e320_g1_T1500_d1000", wl.GateConfig(320, 1, 1, 8, 2.827), 1500, 1000),
    ("e448_g8_T64_d4096", wl.GateConfig(448, 8, 4, 8, 1.0), 64, 4096),
    ("e64_g4_T2000_d512", wl.GateConfig(64, 4, 2, 6, 1.0), 2000, 512),
    ("e192_g4_T3000_d256", wl.GateConfig(192, 4, 2, 8, 1.0), 3000, 256),
]


@pytest.mark.parametrize("name,gc,T,d", SMALL, ids=[s[0] for s in SMALL])
def test_x3_gate_parity_small(o, name, gc, T, d):
    say(f"[x3 gate] {name}")
    gi = wl.make_gate_inputs(T, d, gc, seed=T + d)
    cfg = cfg_of(gc, T, d)
    x, W, b = dev_inputs(gi)
    w, i = sg.siggate_forward(x, W, b, cfg)
    torch.cuda.synchronize()
    w, i = w.cpu().numpy(), i.cpu().numpy()
    stats = compare_gate(w, i, oracle_gate(o, gi, cfg), gc.route_scale, topk_group=gc.topk_group)
    check_rows_valid(i, gc.n_experts, gc.n_group, gc.topk_group)
    say(f"    {stats}")


# largest |v32 - v64| of the choice scores allowed: below the 1e-6 margin
# under which a token is exempt, as on the float32 route
SCORE_ERR_MAX = 1e-6

# batch sizes across the route's plan at d=7168 (tile shape and k-slices)
PLAN_SWEEP = [(2, 256), (33, 384), (65, 256), (129, 384), (300, 256), (511, 384),
              (1000, 256), (2047, 384), (4000, 256), (8191, 256), (12000, 384), (16384, 128),
              (256, 512), (5000, 512)]


@pytest.mark.parametrize("T,E", PLAN_SWEEP, ids=[f"T{t}_E{e}" for t, e in PLAN_SWEEP])
def test_x3_plan_sweep(o, T, E):
    gc = {128: wl.GateConfig(128, 4, 2, 6, 1.0), 256: wl.DSV3, 384: wl.KIMI_K2,
          512: wl.GateConfig(512, 8, 4, 8, 2.5)}[E]
    d = 7168
    say(f"[x3 plan] T={T} E={E}")
    gi = wl.make_gate_inputs(T, d, gc, seed=T * 7 + E)
    cfg = cfg_of(gc, T, d)
    x, W, b = dev_inputs(gi)
    w, i = sg.siggate_forward(x, W, b, cfg)
    torch.cuda.synchronize()
    w, i = w.cpu().numpy(), i.cpu().numpy()
    check_rows_valid(i, gc.n_experts, gc.n_group, gc.topk_group)
    rng = np.random.default_rng(T)
    rows = np.arange(T) if T <= 300 else np.unique(np.r_[0, 63, 64, 127, 128, T - 1,
                                                         rng.integers(0, T, 200)])
    ref = oracle_gate(o, gi, cfg, rows)
    stats = compare_gate(w, i, ref, gc.route_scale, rows, topk_group=gc.topk_group)
    lg = sg.siggate_logits(x, W, cfg).cpu().numpy()[rows]
    stats.update(score_error(lg, o.logits(gi.x[rows], gi.W), gi.bias, ref.margins,
                             np.all(i[rows] == ref.indices, axis=1)))
    say(f"    {stats}")
    assert stats["score_max_abs_err"] < SCORE_ERR_MAX, stats


@pytest.mark.parametrize("T,E,d", [(100, 256, 7168), (16384, 384, 96), (9000, 128, 40),
                                   (300, 384, 264), (16384, 384, 7168), (2048, 256, 7168)])
def test_x3_logits_exact_on_integer_inputs(o, T, E, d):
    """x small integers, W integers times 2^-8: every partial sum is exact,
    so the logits equal the oracle's bit for bit."""
    say(f"[x3 logits-exact] T={T} E={E} d={d}")
    rng = np.random.default_rng(T)
    x = wl.bf16_bits(rng.integers(-8, 9, size=(T, d)).astype(np.float32))
    W = (rng.integers(-8, 9, size=(E, d)) / 256.0).astype(np.float32)
    cfg = sg.Cfg(T, d, E, 1, 1, 8, 1.0, logits_path=X3)
    got = sg.siggate_logits(to_dev_x(x), torch.from_numpy(W).cuda(), cfg).cpu().numpy()
    rows = np.arange(T) if T <= 1000 else np.unique(np.r_[0, T - 1, rng.integers(0, T, 500)])
    assert np.array_equal(got[rows].astype(np.float64), o.logits(x[rows], W))


@pytest.mark.parametrize("E,d", [(384, 7168), (256, 1000), (128, 64)])
def test_x3_split_is_exact(E, d):
    """One-hot x rows (a single nonzero c in {+-1, +-2, +-0.5} at column k):
    the logit is the single product c * W[e, k], exact in float32, so the
    three bfloat16 parts must add back to W bit for bit.  W spans 2^-40 ..
    2^40 in magnitude with full 24-bit significands, both signs."""
    rng = np.random.default_rng(E + d)
    T = 256
    W = (rng.standard_normal((E, d)) * np.exp2(rng.integers(-40, 41, (E, d)))).astype(np.float32)
    cols = rng.integers(0, d, T)
    cols[:4] = [0, d - 1, d // 2, 31 % d]
    coef = rng.choice(np.array([1.0, -1.0, 2.0, -2.0, 0.5, -0.5], np.float32), T)
    xf = np.zeros((T, d), np.float32)
    xf[np.arange(T), cols] = coef
    say(f"[x3 split] E={E} d={d}")
    cfg = sg.Cfg(T, d, E, 1, 1, 8, 1.0, logits_path=X3)
    got = sg.siggate_logits(to_dev_x(wl.bf16_bits(xf)), torch.from_numpy(W).cuda(), cfg).cpu().numpy()
    want = coef[:, None] * W[:, cols].T
    bad = got != want
    assert not bad.any(), f"{int(bad.sum())} logits differ, e.g. {got[bad][:3]} vs {want[bad][:3]}"


@pytest.mark.parametrize("name", ["dsv3-tiny", "kimi-k2-decode", "kimi-k2-prefill"])
def test_x3_logits_tolerance(o, name):
    """Against the float64 oracle (1e-4 relative, floor 1) and against the
    float32 route (the same sum in another order)."""
    w = wl.WORKLOADS[name]
    say(f"[x3 logits] {name}")
    gi = wl.workload_inputs(w)
    cfg = cfg_of(w.cfg, w.T, w.d)
    x, W, _ = dev_inputs(gi)
    got = sg.siggate_logits(x, W, cfg).cpu().numpy()
    f32 = sg.siggate_logits(x, W, dataclasses.replace(cfg, logits_path=0)).cpu().numpy()
    rng = np.random.default_rng(5)
    rows = np.arange(w.T) if w.T <= 256 else np.unique(rng.integers(0, w.T, 256))
    want = o.logits(gi.x[rows], gi.W)
    err = np.abs(got[rows] - want) / np.maximum(np.abs(want), 1.0)
    err32 = np.abs(f32[rows] - want) / np.maximum(np.abs(want), 1.0)
    between = np.abs(got - f32).max()
    say(f"    x3 max rel err {err.max():.3e}; float32 route {err32.max():.3e}; "
        f"max |x3 - float32| {between:.3e}")
    assert err.max() <= LOGIT_RTOL
    assert between <= 1e-5 * max(1.0, float(np.abs(f32).max()))


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_x3_workload_full_size(o, name):
    """Full-size workload on the bfloat16 three-way route: every token
    against the oracle, row properties everywhere, exact twin ties, and the
    dispatch of the route's indices."""
    w = wl.WORKLOADS[name]
    say(f"[x3 workload] {name}: T={w.T} E={w.cfg.n_experts}")
    gi = wl.workload_inputs(w)
    cfg = cfg_of(w.cfg, w.T, w.d)
    x, W, b = dev_inputs(gi)
    wg, ig = sg.siggate_forward(x, W, b, cfg)
    torch.cuda.synchronize()
    w_np, i_np = wg.cpu().numpy(), ig.cpu().numpy()
    check_rows_valid(i_np, w.cfg.n_experts, w.cfg.n_group, w.cfg.topk_group)
    # the oracle on every token (its float64 logits once, then its selection)
    rows = np.arange(w.T)
    lg64 = o.logits(gi.x, gi.W)
    ref = o.select(lg64, gi.bias, cfg.n_group, cfg.topk_group, cfg.top_k,
                   cfg.route_scale, cfg.order, with_scores=True)
    stats = compare_gate(w_np, i_np, ref, w.cfg.route_scale, rows, topk_group=w.cfg.topk_group)
    lg_all = sg.siggate_logits(x, W, cfg).cpu().numpy()
    lg = lg_all[rows]
    stats.update(score_error(lg, lg64, gi.bias, ref.margins,
                             np.all(i_np[rows] == ref.indices, axis=1)))
    # every token: the oracle's selection on the GPU's own logits (the
    # selection epilogue apart from the GEMM's rounding), same rules
    sel = o.select(lg_all.astype(np.float64), gi.bias, w.cfg.n_group, w.cfg.topk_group,
                   w.cfg.top_k, w.cfg.route_scale, with_scores=True)
    s_all = compare_gate(w_np, i_np, sel, w.cfg.route_scale, topk_group=w.cfg.topk_group)
    stats["select_on_gpu_logits"] = {k: s_all[k] for k in ("tokens", "exempt", "index_mismatch_nonexempt",
                                                           "exempt_differ_valid", "weight_max_rel")}
    # the exemption margin must stay above the float32 score error (one
    # chain per k-half of d measured 1.1-1.3e-6 here; blocked summation less)
    assert stats["score_max_abs_err"] < SCORE_ERR_MAX, stats
    if gi.twins:
        dec = np.zeros(len(rows), bool)
        for a, bb in gi.twins:
            dec |= (ref.indices == a).any(1) ^ (ref.indices == bb).any(1)
        matched = int(np.all(i_np[rows][dec] == ref.indices[dec], 1).sum())
        stats["twin_decisive"], stats["twin_decisive_matched"] = int(dec.sum()), matched
        assert matched == int(dec.sum()), "exact twin ties must resolve to the lower expert id"
    say(f"    gate {stats}")
    if not w.dispatch:
        return
    out = sg.siggate_dispatch(x, ig, cfg)
    torch.cuda.synchronize()
    dref = o.dispatch(i_np, w.cfg.n_experts)
    # every permuted row, in host-sized chunks
    compare_dispatch(out, dref, i_np, gi.x, w.cfg.top_k, None, o)


def test_x3_twin_columns_tie_exactly(o):
    gc = wl.KIMI_K2
    T, d = 512, 7168
    gi = wl.make_gate_inputs(T, d, gc, seed=9)
    # disjoint pairs, across the 16-, 64- and 192-expert blocks of the tiles
    pairs = [(3, 200), (17, 18), (100, 383), (0, 191), (192, 255), (63, 64)]
    for a, b in pairs:
        gi.W[b] = gi.W[a]
        gi.bias[b] = gi.bias[a]
    cfg = cfg_of(gc, T, d)
    x, W, b = dev_inputs(gi)
    lg = sg.siggate_logits(x, W, cfg).cpu().numpy()
    for a, bb in pairs:
        assert np.array_equal(lg[:, a], lg[:, bb])
    w, i = sg.siggate_forward(x, W, b, cfg)
    torch.cuda.synchronize()
    w, i = w.cpu().numpy(), i.cpu().numpy()
    compare_gate(w, i, oracle_gate(o, gi, cfg), gc.route_scale, topk_group=gc.topk_group)
    for a, bb in pairs:
        assert not ((i == bb).any(1) & ~(i == a).any(1)).any(), "higher twin chosen over lower"


def test_x3_deterministic_repeat():
    gc = wl.DSV3
    gi = wl.make_gate_inputs(4096, 7168, gc, seed=2)
    x, W, b = dev_inputs(gi)
    for T in (4096, 64):
        cfg = cfg_of(gc, T, 7168)
        xs = x[:T].contiguous()
        r1 = [t.clone() for t in sg.siggate_forward(xs, W, b, cfg)]
        r2 = sg.siggate_forward(xs, W, b, cfg)
        assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])
