"""Throughput of the MoE gate + dispatch on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the whole path on one batch that is already resident in HBM:
siggate_forward (logits GEMM + selection) followed by siggate_dispatch
(histogram, stable permutation, row gather).  The JSON line's ``value`` is
routed tokens/s = T / step time.  The default workload is the Kimi-K2
prefill batch (T=16384, E=384 in one group, d=7168); the DeepSeek-V3
prefill batch (T=16384, E=256, 8 groups keep 4) is reported beside it under
``secondary``.

``roofline`` is for the dominant kernel, the fused gate GEMM: algorithmic
flops 2*T*d*E per launch over its average duration, measured with HIP events
on the launch stream over the timed steps, against the fp32 MFMA peak.
``traffic`` is read from profiles/gate_traffic.json (rocprofv3 FETCH_SIZE and
WRITE_SIZE, scaled by a plain-copy calibration) when that file was taken
from the current gate kernel source, else null.

Every timed section first runs its own work back to back for ``settle_ms``
(default 200 ms) before its warm-up: after idle, the GPU's clocks take tens
of milliseconds of load to settle (the Kimi-K2 prefill gate runs about 15%
slower over its first 15 ms), so the timed steps see the sustained clocks
that a continuously loaded serving or training loop runs at.  The JSON line
gives ``settle_ms`` and the main section's ``settle_steps``.

``stages`` also carries the medians of the per-step event times, and
``cold`` the medians of steps that each follow a 1 GiB scrub write (x and W
then come from HBM, not the 256 MB Infinity Cache).

``decode`` reports the decode-size batches (Kimi-K2 T=256, DeepSeek-V3
T=64): 20 calls captured in one HIP graph and replayed, so the figure is GPU
time per call without host launch cost; the replayed outputs are checked
against an eager call.  Their gate roofline is the larger of the fp32 MFMA
and the HBM time (MFMA binds at both sizes).

``secondary.variants`` times the gate alone on the DeepSeek-V3 batch with
each option of the configuration: softmax scoring, no bias (group maximum),
and the 0.0 fill with the 1e-20 denominator epsilon, beside the default.

``skewed`` is the DeepSeek-V3 batch of T=65536 tokens whose 16 hot experts
(two per group) draw half of the 524288 pairs: whole steps as for the main
workload, with the share of pairs that went to the hot experts.

``overlap`` runs independent batches of the workload with the gates on one
HIP stream and the dispatches on another (two batches in flight), so that
one batch's HBM-bound dispatch overlaps the next batch's MFMA-bound gate; it
reports tokens/s over the batches and is not part of ``value``.

``bf16x3`` repeats the step, the secondary batch and the decode lines with
the logits on the bfloat16 three-way route (cfg.logits_path = 1): W split
exactly into hi + mid + lo bfloat16 parts, every product exact, float32
accumulation on the bf16 matrix cores.  Same outputs up to float32 summation
order (``rows_equal_float32_route``); its roofline counts the 3 * 2*T*d*E
bf16 flops it executes against the bf16 peak.  ``value`` stays the float32
route's.

``cpu_baseline`` times the CPU oracle (float64, all host threads) on a
bounded sample of the same workload, and reports how the GPU's result on
those tokens compares with it (``gpu_parity``: tokens exempt for a score
margin below 1e-6, non-exempt index mismatches, largest weight error, the
largest error of the GPU's float32 choice scores, and the tokens whose
margin lies between 1e-6 and twice that error).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
GATE_SOURCE = os.path.join(ROOT, "sigmoid_group_limited_amd", "csrc", "gate.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_traffic.json")
# wall time each timed section runs its work before its warm-up (--settle-ms)
SETTLE_MS = 200.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def settle(fn, ms: float | None = None) -> int:
    """Runs ``fn`` (which enqueues GPU work) back to back, four calls between
    device synchronisations, until ``ms`` (default SETTLE_MS) milliseconds of
    wall time have passed, so that the GPU's clocks have settled under load.
    Returns the number of calls."""
    import torch
    ms = SETTLE_MS if ms is None else ms
    n = 0
    t_end = time.perf_counter() + ms * 1e-3
    torch.cuda.synchronize()
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n


def source_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def gate_traffic(workload: str, n_launch_bytes: float):
    """HBM bytes per gate launch from a committed counter profile of the
    current kernel source, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("gate_source_sha") != source_sha(GATE_SOURCE):
        return None
    return entry.get("hbm_bytes_per_launch")


class Case:
    """Device-resident inputs, outputs and workspace of one workload."""

    def __init__(self, name: str, logits_path: int = 0):
        import torch

        import sigmoid_group_limited_amd as sg
        from sigmoid_group_limited_amd import workloads as wl
        self.w = wl.WORKLOADS[name]
        c = self.w.cfg
        t0 = time.time()
        self.gi = wl.workload_inputs(self.w)
        log(f"[bench] {name}: inputs drawn in {time.time() - t0:.1f}s")
        self.cfg = sg.Cfg(self.w.T, self.w.d, c.n_experts, c.n_group, c.topk_group,
                          c.top_k, c.route_scale, logits_path=logits_path)
        dev = "cuda"
        self.x = torch.from_numpy(self.gi.x.view(np.int16)).to(dev).view(torch.bfloat16)
        self.W = torch.from_numpy(self.gi.W).to(dev)
        self.b = torch.from_numpy(self.gi.bias).to(dev)
        T, K, E, d = self.w.T, c.top_k, c.n_experts, self.w.d
        self.weights = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.indices = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.ws = sg.workspace(self.cfg, dev)
        self.out = sg.DispatchOut(
            torch.empty(E, dtype=torch.int32, device=dev),
            torch.empty(E + 1, dtype=torch.int32, device=dev),
            torch.empty(T * K, dtype=torch.int32, device=dev),
            torch.empty(T * K, dtype=torch.int32, device=dev),
            torch.empty((T * K, d), dtype=torch.bfloat16, device=dev))
        self.sg = sg

    def forward(self):
        self.sg.siggate_forward(self.x, self.W, self.b, self.cfg, self.weights,
                                self.indices, self.ws)

    def dispatch(self):
        self.sg.siggate_dispatch(self.x, self.indices, self.cfg, self.out, self.ws)

    def run(self, steps: int, warmup: int):
        """Times ``steps`` whole steps (wall clock between two device
        synchronisations) and, inside the same region, each stage with HIP
        events recorded on the launch stream; before the ``warmup`` steps,
        whole steps run for the settle time."""
        import torch
        self.settle_steps = settle(lambda: (self.forward(), self.dispatch()))
        for _ in range(warmup):
            self.forward()
            self.dispatch()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i][0].record()
            self.forward()
            ev[i][1].record()
            self.dispatch()
            ev[i][2].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        g = [e[0].elapsed_time(e[1]) for e in ev]
        dd = [e[1].elapsed_time(e[2]) for e in ev]
        self.medians = (float(np.median(g)), float(np.median(dd)))
        return wall / steps * 1e3, float(np.mean(g)), float(np.mean(dd))

    def run_cold(self, steps: int):
        """Each step after writing a 1 GiB scrub buffer (larger than the
        256 MB Infinity Cache), so x and W come from HBM; gate and dispatch
        timed with HIP events.  Returns medians in ms."""
        import torch
        scrub = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(steps):
            scrub.fill_(i & 0xff)
            ev[i][0].record()
            self.forward()
            ev[i][1].record()
            self.dispatch()
            ev[i][2].record()
        torch.cuda.synchronize()
        del scrub
        return (float(np.median([e[0].elapsed_time(e[1]) for e in ev])),
                float(np.median([e[1].elapsed_time(e[2]) for e in ev])))

    def run_next_rows(self, steps: int, warmup: int):
        """Times the steps after the path, on this workload's own outputs:
        the combine (identity experts: the dispatched rows come back) and the
        expert-parallel metadata for 8 ranks.  Returns a dict."""
        import torch
        sg = self.sg
        y = torch.empty_like(self.x)
        for _ in range(warmup):
            sg.siggate_combine(self.out.permuted_x, self.weights, self.out.dest, self.cfg, y)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(steps):
            sg.siggate_combine(self.out.permuted_x, self.weights, self.out.dest, self.cfg, y)
        ev[1].record()
        for _ in range(steps):
            sg.siggate_ep_send_splits(self.out.tokens_per_expert, 8)
            sg.siggate_ep_dedup(self.indices, self.cfg, 8)
        ev[2].record()
        torch.cuda.synchronize()
        T, K, d = self.w.T, self.cfg.top_k, self.w.d
        comb_ms = ev[0].elapsed_time(ev[1]) / steps
        comb_bytes = T * K * d * 2 + T * d * 2 + T * K * 8
        return {"combine_ms": comb_ms,
                "combine_algorithmic_GBps": comb_bytes / (comb_ms * 1e-3) / 1e9,
                "combine_hbm_frac": comb_bytes / (comb_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "ep8_metadata_ms": ev[1].elapsed_time(ev[2]) / steps}

    def run_variants(self, steps: int, warmup: int):
        """Gate-only time of the gate's variants on this workload's inputs:
        softmax scoring, no bias (group maximum), and the 0.0 fill with the
        1e-20 denominator epsilon.  Median of ``steps`` HIP-event timings."""
        import dataclasses

        import torch
        sg = self.sg
        out = {}
        for name, opts, bias in (("sigmoid_default", {}, self.b),
                                 ("softmax", {"score_func": 1}, self.b),
                                 ("no_bias", {}, None),
                                 ("zero_fill_eps", {"mask_zero": 1, "denom_eps": 1e-20}, self.b)):
            cfg = dataclasses.replace(self.cfg, **opts)
            call = (lambda cfg=cfg, bias=bias:
                    sg.siggate_forward(self.x, self.W, bias, cfg, self.weights, self.indices, self.ws))
            for _ in range(warmup):
                call()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
            torch.cuda.synchronize()
            for e in ev:
                e[0].record()
                call()
                e[1].record()
            torch.cuda.synchronize()
            out[name + "_gate_ms"] = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
        return out

    def algorithmic(self):
        T, d, E, K = self.w.T, self.w.d, self.cfg.E, self.cfg.top_k
        gate_flops = 2.0 * T * d * E
        gate_bytes = T * d * 2 + E * d * 4 + E * 4 + T * K * 8
        row = d * 2
        disp_bytes = T * K * 4 + T * K * 4 * 2 + T * row + T * K * row
        return gate_flops, gate_bytes, disp_bytes


def overlap_line(name: str, steps: int, warmup: int):
    """Two independent batches of the workload in flight on two HIP streams
    (default priority): one stream runs every batch's gate in turn, the other
    each batch's dispatch once its gate is done, so one batch's HBM-bound
    dispatch runs beside the next batch's MFMA-bound gate (a batch's buffers
    are reused two batches later, after its dispatch).  Reports the wall time
    per batch over ``steps`` batches, and checks that both batches' outputs
    equal a sequential run's."""
    import torch
    cases = [Case(name), Case(name)]
    for c in cases:
        c.forward()
        c.dispatch()
    torch.cuda.synchronize()
    ref = [(c.indices.clone(), c.out.perm.clone()) for c in cases]
    gate_s, disp_s = torch.cuda.Stream(), torch.cuda.Stream()

    def run(n):
        gate_done = [torch.cuda.Event() for _ in range(n)]
        disp_done = [torch.cuda.Event() for _ in range(n)]
        for i in range(n):
            c = cases[i % 2]
            with torch.cuda.stream(gate_s):
                if i >= 2:
                    gate_s.wait_event(disp_done[i - 2])
                c.forward()
                gate_done[i].record(gate_s)
            with torch.cuda.stream(disp_s):
                disp_s.wait_event(gate_done[i])
                c.dispatch()
                disp_done[i].record(disp_s)

    # a run's batches are ordered among themselves only: synchronise after each
    settle(lambda: (run(8), torch.cuda.synchronize()))
    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    same = all(torch.equal(c.indices, r[0]) and torch.equal(c.out.perm, r[1])
               for c, r in zip(cases, ref))
    T = cases[0].w.T
    del cases
    return {"workload": name, "streams": 2, "batches": steps,
            "ms_per_batch": wall / steps * 1e3, "tokens_per_s": T * steps / wall,
            "outputs_match_sequential": bool(same),
            "note": "gates on one stream, dispatches on another, two batches in flight; "
                    "not the step of value"}


def bf16x3_line(name: str, steps: int, warmup: int, ref_indices=None):
    """The same step with the logits on the bfloat16 three-way route
    (cfg.logits_path = 1: W split exactly into three bfloat16 parts, three
    exact products per term accumulated in float32).  Its roofline counts the
    3 * 2*T*d*E bf16 MFMA flops the route executes against the bf16 peak.
    ``rows_equal_float32_route`` is the share of tokens whose indices equal
    those of the float32 route."""
    case = Case(name, logits_path=1)
    ms, g, dd = case.run(steps, warmup)
    T, d, E = case.w.T, case.w.d, case.cfg.E
    x3_flops = 3 * 2.0 * T * d * E
    out = {"workload": name, "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
           "gate_ms": g, "dispatch_ms": dd,
           "gate_ms_median": case.medians[0], "dispatch_ms_median": case.medians[1],
           "gate_equivalent_fp32_tflops": 2.0 * T * d * E / (g * 1e-3) / 1e12,
           "roofline": {"bound": "mfma", "achieved": x3_flops / (g * 1e-3) / 1e12,
                        "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                        "frac": x3_flops / (g * 1e-3) / 1e12 / PEAK_BF16_MFMA_TFLOPS,
                        "note": "whole gate (W split, GEMM, selection) against 3*2*T*d*E bf16 flops"}}
    if ref_indices is not None:
        out["rows_equal_float32_route"] = float((case.indices == ref_indices).all(1).float().mean())
    del case
    return out


def decode_line(name: str, calls: int = 20, replays: int = 5, logits_path: int = 0):
    """Gate and gate+dispatch of one decode-size batch, timed by replaying
    ``calls`` back-to-back calls captured in a HIP graph."""
    import torch
    case = Case(name, logits_path)
    case.forward()
    case.dispatch()
    torch.cuda.synchronize()
    ref_i = case.indices.clone()
    ref_p = case.out.perm.clone()
    ref_x = case.out.permuted_x.clone()

    def per_call(fn):
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(calls):
                    fn()
        torch.cuda.synchronize()
        settle(g.replay)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (replays * calls)

    gate_us = per_call(case.forward)
    path_us = per_call(lambda: (case.forward(), case.dispatch()))
    same = (torch.equal(case.indices, ref_i) and torch.equal(case.out.perm, ref_p)
            and torch.equal(case.out.permuted_x, ref_x))
    T = case.w.T
    flops, gate_bytes, disp_bytes = case.algorithmic()
    # the bfloat16 three-way route executes 3x the flops on the bf16 peak
    t_mfma = (flops / (PEAK_FP32_MFMA_TFLOPS * 1e12) if logits_path == 0
              else 3 * flops / (PEAK_BF16_MFMA_TFLOPS * 1e12)) * 1e6
    t_hbm = gate_bytes / (PEAK_HBM_GBS * 1e9) * 1e6
    t_roof = max(t_mfma, t_hbm)
    return {"workload": name, "T": T, "E": case.cfg.E, "logits_path": logits_path,
            "gate_us": gate_us, "dispatch_us": path_us - gate_us, "path_us": path_us,
            "gate_tokens_per_s": T / (gate_us * 1e-6), "path_tokens_per_s": T / (path_us * 1e-6),
            "gate_bound": "mfma" if t_mfma >= t_hbm else "hbm",
            "gate_roofline_us": t_roof, "gate_roofline_frac": t_roof / gate_us,
            "gate_tflops": flops / (gate_us * 1e-6) / 1e12,
            "gate_algorithmic_GBps": gate_bytes / (gate_us * 1e-6) / 1e9,
            "graph_replay_matches_eager": bool(same)}


def gate_sweep():
    """Gate time per call across batch sizes, both logits routes, for the
    DeepSeek-V3 (E=256) and Kimi-K2 (E=384) gates at d=7168: graph-replayed
    back-to-back calls on seeded synthetic inputs; one JSON line each."""
    import torch

    import sigmoid_group_limited_amd as sg
    from sigmoid_group_limited_amd import workloads as wl
    d = 7168
    for gc in (wl.DSV3, wl.KIMI_K2):
        for T in (1, 16, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384):
            gi = wl.make_gate_inputs(T, d, gc, seed=T)
            x = torch.from_numpy(gi.x.view(np.int16)).cuda().view(torch.bfloat16)
            W = torch.from_numpy(gi.W).cuda()
            b = torch.from_numpy(gi.bias).cuda()
            w = torch.empty((T, gc.top_k), dtype=torch.float32, device="cuda")
            i = torch.empty((T, gc.top_k), dtype=torch.int32, device="cuda")
            calls = 20 if T <= 1024 else 4
            for lp in (0, 1):
                cfg = sg.Cfg(T, d, gc.n_experts, gc.n_group, gc.topk_group, gc.top_k,
                             gc.route_scale, logits_path=lp)
                ws = sg.workspace(cfg)

                def fn():
                    sg.siggate_forward(x, W, b, cfg, w, i, ws)
                fn()
                s = torch.cuda.Stream()
                with torch.cuda.stream(s):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        for _ in range(calls):
                            fn()
                torch.cuda.synchronize()
                settle(g.replay)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(5):
                    g.replay()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / (5 * calls)
                flops = 2.0 * T * d * gc.n_experts
                print(json.dumps({"gate_sweep": True, "E": gc.n_experts, "T": T, "logits_path": lp,
                                  "gate_us": round(us, 2), "tokens_per_s": T / (us * 1e-6),
                                  "fp32_tflops_equivalent": flops / (us * 1e-6) / 1e12,
                                  "fp32_mfma_frac": flops / (us * 1e-6) / 1e12 / PEAK_FP32_MFMA_TFLOPS}),
                      flush=True)


def clock_ramp(name: str = "kimi-k2-prefill", calls: int = 400, block: int = 20):
    """The gate's time per call after 2 s of idle: ``calls`` back-to-back
    calls, each bracketed by HIP events on the launch stream, reported as the
    median of each block of ``block`` calls with the elapsed time at the
    block's end.  Shows how long the clocks take to settle under load."""
    import torch
    case = Case(name)
    case.forward()
    torch.cuda.synchronize()
    time.sleep(2.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(calls + 1)]
    ev[0].record()
    for k in range(calls):
        case.forward()
        ev[k + 1].record()
    torch.cuda.synchronize()
    us = np.array([ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(calls)])
    print(json.dumps({"clock_ramp": True, "workload": name, "block_calls": block,
                      "median_us": [round(float(np.median(us[j:j + block])), 1)
                                    for j in range(0, calls, block)],
                      "elapsed_ms_at_block_end": [round(float(us[:j + block].sum()) / 1e3, 1)
                                                  for j in range(0, calls, block)]}), flush=True)


def skewed_line(logits_path: int, steps: int, warmup: int) -> dict:
    """The skewed DeepSeek-V3 batch: T=65536 with 16 hot experts (two per
    group) that draw half of the 524288 pairs.  Whole steps as for the main
    workload, against the path roofline t_gate + t_dispatch."""
    case = Case("dsv3-skewed", logits_path)
    ms, gate_ms, disp_ms = case.run(steps, warmup)
    flops, _, disp_bytes = case.algorithmic()
    T = case.w.T
    mfma_flops = flops if logits_path == 0 else 3 * flops
    peak = PEAK_FP32_MFMA_TFLOPS if logits_path == 0 else PEAK_BF16_MFMA_TFLOPS
    t_roof = mfma_flops / (peak * 1e12) + disp_bytes / (PEAK_HBM_GBS * 1e9)
    hot = float(np.isin(case.indices.cpu().numpy(), case.gi.hot).mean())
    out = {"workload": case.w.name, "T": T, "E": case.cfg.E, "logits_path": logits_path,
           "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
           "gate_ms": gate_ms, "dispatch_ms": disp_ms,
           "gate_mfma_frac": mfma_flops / (gate_ms * 1e-3) / 1e12 / peak,
           "dispatch_algorithmic_GBps": disp_bytes / (disp_ms * 1e-3) / 1e9,
           "roofline_tokens_per_s": T / t_roof, "path_roofline_frac": t_roof / (ms * 1e-3),
           "hot_share": hot}
    del case
    return out


def score_error(case: Case, o, n: int, margins: np.ndarray, same: np.ndarray) -> dict:
    """How far the GPU's float32 choice scores v = sigmoid(L) + b can be
    from the oracle's float64 ones on the first n tokens: the largest
    |v32 - v64| over every token and expert, with v32 formed in float32 from
    the GPU's own logits.  Tokens whose decision margin lies between the
    1e-6 exemption threshold and twice that error are not exempt, yet the
    score error alone could flip them: they are counted, with how many of
    them differ from the oracle."""
    c = case.cfg
    lg = case.sg.siggate_logits(case.x[:n], case.W, c.with_T(n)).cpu().numpy()
    lr = o.logits(case.gi.x[:n], case.gi.W)
    one = np.float32(1.0)
    s32 = one / (one + np.exp(-lg))          # float32 arithmetic
    v32 = s32 + case.gi.bias.astype(np.float32)[None, :]
    v64 = 1.0 / (1.0 + np.exp(-lr)) + case.gi.bias.astype(np.float64)[None, :]
    err = float(np.abs(v32.astype(np.float64) - v64).max())
    margin = np.minimum(margins[:, 0], margins[:, 1])
    band = (margin >= 1e-6) & (margin < 2.0 * err)
    return {"score_max_abs_err": err, "near_band": [1e-6, 2.0 * err],
            "near_band_tokens": int(band.sum()),
            "near_band_mismatch": int((band & ~same).sum())}


def cpu_baseline(case: Case, budget_s: float = 12.0, min_total_s: float = 10.0):
    """The oracle, as it stands, on the first n tokens of the workload: gate,
    then dispatch and row gather of those tokens' pairs.  n grows from 256
    until the run takes about budget_s / 4, then one timed run at the size
    that fits the budget; when that is the whole batch and shorter than
    min_total_s, the run is repeated until the timed runs add up to it."""
    import oracle
    o = oracle.load()
    c = case.cfg
    gi = case.gi

    split = {}

    def one(n):
        t0 = time.perf_counter()
        r = o.gate(gi.x[:n], gi.W, gi.bias, c.n_group, c.topk_group, c.top_k, c.route_scale)
        t1 = time.perf_counter()
        dr = o.dispatch(r.indices, c.E)
        o.gather_rows(gi.x[:n], dr.perm, c.top_k)
        t2 = time.perf_counter()
        split["gate"], split["dispatch"], split["result"] = t1 - t0, t2 - t1, r
        return t2 - t0

    n = 256
    dt = one(n)
    while dt < budget_s / 4 and n * 2 <= case.w.T:
        n *= 2
        dt = one(n)
    if dt < budget_s / 2:
        n_final = min(case.w.T, int(n * (budget_s / 2) / max(dt, 1e-3)))
        n_final = max(n, n_final // 256 * 256)
        if n_final != n:
            n = n_final
            dt = one(n)
    runs, total = 1, dt
    gate_total, disp_total = split["gate"], split["dispatch"]
    while total < min_total_s:
        total += one(n)
        gate_total += split["gate"]
        disp_total += split["dispatch"]
        runs += 1
    # the same tokens on the GPU (the last timed step's outputs) against the
    # oracle run just timed, with the exemption rule of the parity tests
    r = split["result"]
    idx = case.indices[:n].cpu().numpy()
    wts = case.weights[:n].cpu().numpy().astype(np.float64)
    exempt = np.minimum(r.margins[:, 0], r.margins[:, 1]) < 1e-6
    same = np.all(idx == r.indices, axis=1)
    rel = np.abs(wts[same] - r.weights[same]) / np.maximum(np.abs(r.weights[same]), 1e-30)
    parity = {"tokens": n, "exempt": int(exempt.sum()),
              "exempt_matched": int((exempt & same).sum()),
              "index_mismatch_nonexempt": int((~same & ~exempt).sum()),
              "weight_max_rel": float(rel.max()) if rel.size else 0.0}
    parity.update(score_error(case, o, n, r.margins, same))
    return dict(value=n * runs / total, unit="tokens/s", cores=o.num_threads(), kind="oracle",
                gate_tokens_per_s=n * runs / gate_total,
                dispatch_tokens_per_s=n * runs / disp_total,
                gpu_parity=parity,
                sample=f"first {n} of {case.w.T} tokens of {case.w.name}: float64 gate, "
                       f"dispatch and row gather of their {n * c.top_k} pairs; "
                       f"{runs} timed run{'s' if runs > 1 else ''}, {total:.2f} s")


def main():
    global SETTLE_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="kimi-k2-prefill")
    ap.add_argument("--secondary", default="dsv3-prefill-ties")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the graph-replayed decode-size lines")
    ap.add_argument("--no-cold", action="store_true", help="skip the scrubbed (cold) steps")
    ap.add_argument("--no-skewed", action="store_true",
                    help="skip the skewed DeepSeek-V3 batch (T=65536, hot experts)")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the two-stream run of two independent batches")
    ap.add_argument("--no-bf16x3", action="store_true",
                    help="skip the lines of the bfloat16 three-way logits route")
    ap.add_argument("--logits-path", type=int, choices=(0, 1), default=0,
                    help="logits route of the main step: 0 float32 MFMA (default), "
                         "1 the bfloat16 three-way route (then its roofline is bf16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="wall time each timed section runs its work before its warm-up")
    ap.add_argument("--clock-ramp", action="store_true",
                    help="only time 400 back-to-back gate calls after 2 s idle (clock settling)")
    ap.add_argument("--gate-sweep", action="store_true",
                    help="only time the gate per call across batch sizes (both routes)")
    args = ap.parse_args()
    SETTLE_MS = args.settle_ms

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X "
              "(sharding is by tokens and needs no exchange for the gate); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    if args.gate_sweep:
        gate_sweep()
        return

    if args.clock_ramp:
        clock_ramp(args.workload)
        return

    lp = args.logits_path
    case = Case(args.workload, lp)
    ms, gate_ms, disp_ms = case.run(args.steps, args.warmup)
    T = case.w.T
    flops, gate_bytes, disp_bytes = case.algorithmic()
    # the bfloat16 three-way route executes 3 bf16 products per term
    mfma_flops = flops if lp == 0 else 3 * flops
    peak = PEAK_FP32_MFMA_TFLOPS if lp == 0 else PEAK_BF16_MFMA_TFLOPS
    achieved = mfma_flops / (gate_ms * 1e-3) / 1e12
    traffic = gate_traffic(case.w.name, gate_bytes) if lp == 0 else None
    result = {
        "metric": "routed tokens/s (gate+dispatch)",
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": SETTLE_MS,
        "settle_steps": case.settle_steps,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if lp == 0 else "bf16x3 products, f32 accumulation",
        "data": "synthetic (seeded; x ~ N(0,1) in bfloat16, W ~ N(0,1/d), bias ~ U(-0.05,0.05))",
        "config": {"workload": case.w.name, "T": T, "d": case.w.d, "E": case.cfg.E,
                   "n_group": case.cfg.n_group, "topk_group": case.cfg.topk_group,
                   "top_k": case.cfg.top_k, "route_scale": case.cfg.route_scale,
                   "parallelism": "single GPU", "logits_path": lp},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": traffic},
        "stages": {
            "gate_ms": gate_ms, "dispatch_ms": disp_ms,
            "gate_tflops": flops / (gate_ms * 1e-3) / 1e12,
            "dispatch_algorithmic_GBps": disp_bytes / (disp_ms * 1e-3) / 1e9,
            "dispatch_hbm_frac": disp_bytes / (disp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "pairs_per_s": T * case.cfg.top_k / (ms * 1e-3),
            "roofline_tokens_per_s": T / (mfma_flops / (peak * 1e12)
                                          + disp_bytes / (PEAK_HBM_GBS * 1e9)),
        },
    }
    result["stages"]["path_roofline_frac"] = result["value"] / result["stages"]["roofline_tokens_per_s"]
    result["stages"]["gate_ms_median"], result["stages"]["dispatch_ms_median"] = case.medians
    if not args.no_cold:
        cg, cd = case.run_cold(max(5, args.steps // 2))
        result["cold"] = {"gate_ms_median": cg, "dispatch_ms_median": cd,
                          "tokens_per_s": T / ((cg + cd) * 1e-3),
                          "note": "1 GiB scrub written before each step"}
    result["after_path"] = case.run_next_rows(max(3, args.steps // 2), 2)
    if args.secondary:
        sec = Case(args.secondary, lp)
        ms2, g2, d2 = sec.run(args.steps, args.warmup)
        f2, _, db2 = sec.algorithmic()
        result["secondary"] = {
            "workload": sec.w.name, "E": sec.cfg.E, "value": sec.w.T / (ms2 * 1e-3),
            "ms_per_step": ms2, "gate_ms": g2, "dispatch_ms": d2,
            "gate_tflops": f2 / (g2 * 1e-3) / 1e12,
            "gate_mfma_frac": (f2 if lp == 0 else 3 * f2) / (g2 * 1e-3) / 1e12 / peak,
            "dispatch_algorithmic_GBps": db2 / (d2 * 1e-3) / 1e9,
            "variants": sec.run_variants(max(5, args.steps // 2), 2),
        }
        del sec
    if not args.no_skewed:
        result["skewed"] = skewed_line(lp, max(5, args.steps // 2), 2)
    if not args.no_overlap:
        result["overlap"] = overlap_line(args.workload, max(8, args.steps), 2)
    if not args.no_decode:
        result["decode"] = [decode_line("kimi-k2-decode", logits_path=lp),
                            decode_line("dsv3-tiny", logits_path=lp)]
    if not args.no_bf16x3 and lp == 0:
        ref = case.indices.clone()
        x3 = {"default": bf16x3_line(args.workload, args.steps, args.warmup, ref)}
        if args.secondary:
            x3["secondary"] = bf16x3_line(args.secondary, max(5, args.steps // 2), 2)
        if not args.no_decode:
            x3["decode"] = [decode_line("kimi-k2-decode", logits_path=1),
                            decode_line("dsv3-tiny", logits_path=1)]
        result["bf16x3"] = x3
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
