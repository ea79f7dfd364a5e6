"""Parity of the gate variants (softmax scoring, no bias, renormalisation
switch, 0.0 fill, denominator epsilon) and of the combine step with the CPU
oracle, through the C ABI.  Needs an MI355X."""
import dataclasses

import numpy as np
import pytest

import oracle
import sigmoid_group_limited_amd as sg
from sigmoid_group_limited_amd import workloads as wl
from parity import check_rows_valid, combine_tolerance, compare_gate, dev_inputs, say

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


VARIANTS = [
    # (name, GateConfig, T, d, options, bias: "yes" | "none" | "negative")
    ("dsv3_softmax", wl.DSV3, 300, 1024, dict(score_func=1), "yes"),
    ("kimi_softmax_fused", wl.KIMI_K2, 8229, 256, dict(score_func=1), "yes"),
    ("dsv3_nobias", wl.DSV3, 300, 1024, dict(), "none"),
    ("dsv3_nobias_fused64", wl.DSV3, 16400, 128, dict(), "none"),
    ("dsv3_softmax_nobias", wl.DSV3, 257, 2048, dict(score_func=1), "none"),
    ("dsv3_softmax_renorm", wl.DSV3, 200, 512, dict(score_func=1, renorm=1), "yes"),
    ("kimi_renorm_off", wl.KIMI_K2, 200, 512, dict(renorm=2), "yes"),
    ("dsv3_kimi_compat", wl.DSV3, 300, 1024, dict(mask_zero=1, denom_eps=1e-20), "yes"),
    ("dsv3_zero_fill_negative", wl.DSV3, 300, 1024, dict(mask_zero=1, denom_eps=1e-20), "negative"),
    ("dsv3_zero_fill_fused", wl.DSV3, 16400, 128, dict(mask_zero=1), "negative"),
]


@pytest.mark.parametrize("name,gc,T,d,opts,bias_kind", VARIANTS, ids=[v[0] for v in VARIANTS])
@pytest.mark.parametrize("lp", [0, 1], ids=["fp32", "bf16x3"])
def test_gate_variant(o, name, gc, T, d, opts, bias_kind, lp):
    """Each variant on both logits routes (the selection is shared)."""
    say(f"[variant] {name} logits_path={lp}")
    gi = wl.make_gate_inputs(T, d, gc, seed=T + 7)
    bias = None if bias_kind == "none" else gi.bias
    if bias_kind == "negative":
        # most choice scores below zero: a 0.0 fill then beats kept experts
        bias = (gi.bias - np.float32(0.9)).astype(np.float32)
    cfg = dataclasses.replace(sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k,
                                     gc.route_scale, logits_path=lp), **opts)
    x, W, _ = dev_inputs(gi)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    w, i = sg.siggate_forward(x, W, b, cfg)
    torch.cuda.synchronize()
    w, i = w.cpu().numpy(), i.cpu().numpy()
    ref = o.gate(gi.x, gi.W, bias, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                 score_func=cfg.score_func, renorm=cfg.renorm, mask_zero=cfg.mask_zero,
                 denom_eps=cfg.denom_eps, with_scores=True)
    renorm = cfg.renorm == 1 or (cfg.renorm == 0 and cfg.score_func == 0)
    stats = compare_gate(w, i, ref, gc.route_scale, check_sum=renorm, topk_group=gc.topk_group,
                         renorm=renorm, mask_zero=cfg.mask_zero, denom_eps=cfg.denom_eps)
    assert i.min() >= 0 and i.max() < gc.n_experts
    if not cfg.mask_zero:
        check_rows_valid(i, gc.n_experts, gc.n_group, gc.topk_group)
    else:
        S = gc.n_experts // gc.n_group
        outside = 0
        for t in range(T):
            # winners outside the kept groups may only appear with the 0.0 fill
            outside += len(set(i[t] // S)) > gc.topk_group
        stats["tokens_using_zero_filled_groups"] = outside
        if bias_kind == "negative":
            assert outside > 0, "the negative-bias case does not exercise the 0.0 fill"
    say(f"    {stats}")


def test_combine_parity(o):
    """Combine on real gate weights and dispatch positions: bfloat16 output
    equal to the oracle's float64 sum within one bfloat16 unit plus the
    float32 accumulation bound; almost all elements equal bit for bit."""
    gc = wl.DSV3
    T, d = 1000, 512
    say(f"[combine] T={T} d={d}")
    gi = wl.make_gate_inputs(T, d, gc, seed=41)
    cfg = sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale)
    x, W, b = dev_inputs(gi)
    w, i = sg.siggate_forward(x, W, b, cfg)
    disp = sg.siggate_dispatch(x, i, cfg)
    rng = np.random.default_rng(3)
    outs = wl.bf16_bits(rng.standard_normal((T * gc.top_k, d), dtype=np.float32))
    outs_d = torch.from_numpy(outs.view(np.int16)).cuda().view(torch.bfloat16)
    y = sg.siggate_combine(outs_d, w, disp.dest, cfg)
    torch.cuda.synchronize()
    y16 = y.view(torch.int16).cpu().numpy().view(np.uint16)
    w64, dest = w.cpu().numpy().astype(np.float64), disp.dest.cpu().numpy()
    y64, want16 = o.combine(outs, w64, dest)
    diff = y16 != want16
    got = wl.bf16_to_f32(y16).astype(np.float64)
    tol = combine_tolerance(o, outs, w64, dest, y64, gc.top_k)
    assert np.all(np.abs(got - y64) <= tol), "combine outside the rounding bound"
    say(f"    elements {diff.size}, not bit-equal {int(diff.sum())}")
    assert diff.mean() < 1e-2
    # identity experts: the dispatched rows come back scaled by route_scale
    y = sg.siggate_combine(disp.permuted_x, w, disp.dest, cfg)
    yi = wl.bf16_to_f32(y.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    xs = wl.bf16_to_f32(gi.x).astype(np.float64)
    assert np.allclose(yi, gc.route_scale * xs, rtol=2.0 ** -7, atol=0)


def test_combine_full_size(o):
    """Kimi-K2 prefill shape: 16384 tokens x 8 slots x 7168 columns; sampled
    tokens against the oracle."""
    gc = wl.KIMI_K2
    T, d, K = 16384, 7168, gc.top_k
    say(f"[combine] full size T={T} d={d}")
    rng = np.random.default_rng(5)
    idx = wl.random_indices(T, K, gc.n_experts, seed=11)
    perm = np.argsort(idx.ravel(), kind="stable")
    dest = np.empty(T * K, np.int32)
    dest[perm] = np.arange(T * K, dtype=np.int32)
    wts = rng.uniform(0.0, 0.7, size=(T, K)).astype(np.float32)
    gen = torch.Generator(device="cuda").manual_seed(5)
    outs_d = torch.randn((T * K, d), device="cuda", generator=gen).to(torch.bfloat16)
    cfg = sg.Cfg(T, d, gc.n_experts, 1, 1, K, gc.route_scale)
    y = sg.siggate_combine(outs_d, torch.from_numpy(wts).cuda(), torch.from_numpy(dest).cuda(), cfg)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, T - 1, rng.integers(0, T, 64)])
    sub_dest = dest.reshape(T, K)[rows]
    need = torch.from_numpy(sub_dest.ravel().astype(np.int64)).cuda()
    sub_out = outs_d[need].view(torch.int16).cpu().numpy().view(np.uint16)
    local = np.arange(len(rows) * K, dtype=np.int32)
    w64 = wts[rows].astype(np.float64)
    y64, want16 = o.combine(sub_out, w64, local)
    got16 = y[torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    got = wl.bf16_to_f32(got16).astype(np.float64)
    tol = combine_tolerance(o, sub_out, w64, local, y64, K)
    assert np.all(np.abs(got - y64) <= tol)
    assert (got16 != want16).mean() < 1e-2


@pytest.mark.parametrize("K,d", [(3, 40), (5, 7168), (1, 264), (8, 1032)])
def test_combine_slots_and_skips(o, K, d):
    """Every top_k from one template, row widths that leave a ragged last
    pass, and dest entries out of range (-1 or >= n_pos), which contribute
    nothing; the oracle sees those slots as weight 0 on a valid row."""
    T = 300
    say(f"[combine] K={K} d={d}")
    rng = np.random.default_rng(K * 1000 + d)
    n_pos = T * K
    dest = rng.permutation(n_pos).astype(np.int32)
    skip = rng.random(n_pos) < 0.1
    dest_gpu = dest.copy()
    dest_gpu[skip] = np.where(rng.random(int(skip.sum())) < 0.5, -1, n_pos + 7)
    wts = rng.uniform(0.0, 0.7, size=(T, K)).astype(np.float32)
    outs = wl.bf16_bits(rng.standard_normal((n_pos, d), dtype=np.float32))
    cfg = sg.Cfg(T, d, 8, 1, 1, K, 1.0)
    y = sg.siggate_combine(torch.from_numpy(outs.view(np.int16)).cuda().view(torch.bfloat16),
                           torch.from_numpy(wts).cuda(), torch.from_numpy(dest_gpu).cuda(), cfg)
    torch.cuda.synchronize()
    got16 = y.view(torch.int16).cpu().numpy().view(np.uint16)
    w64 = wts.astype(np.float64)
    w64[skip.reshape(T, K)] = 0.0
    y64, want16 = o.combine(outs, w64, dest)
    got = wl.bf16_to_f32(got16).astype(np.float64)
    assert np.all(np.abs(got - y64) <= combine_tolerance(o, outs, w64, dest, y64, K))
    assert (got16 != want16).mean() < 1e-2
