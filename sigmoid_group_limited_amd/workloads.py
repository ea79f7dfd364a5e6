"""Seeded synthetic inputs for the MoE gate and dispatch.

This module only draws random numbers and shapes them.  It holds none of the
gate's arithmetic; the HIP library and the CPU oracle both consume what it
produces, and it imports neither of them.

Shapes and model constants come from the pages:
  * DeepSeek-V3 (671B): 256 routed experts, 8 activated, 8 expert groups of
    which 4 are kept, sigmoid scoring, route_scale 2.5 (AI Engineer
    Exhaustive · DeepSeek-V3 MoE Router, "Official code"; DeepSeek-V3.2-Exp ·
    Normalize weights, equation for G_i);
  * Kimi K2: 384 routed experts in one group, 8 activated, route_scale 2.827
    (Kimi K2 · Normalize weights: equation for G_i, in/out shapes, and the
    "Direct evidence" note that there is one group);
  * hidden size d = 7168 (Kimi K2 · Add shared output, in/out shapes).

Distributions (the pages publish none; these stand in for real activations and
trained router weights): x ~ N(0, 1) rounded to bfloat16 (round to nearest
even), W ~ N(0, 1/d) in float32 so logits are about N(0, 1), bias ~ U(-0.05,
0.05) in float32.  Two structured variants:
  * twins: P pairs of experts inside one group get identical W rows and
    biases, so their choice scores tie exactly for every token;
  * hot experts: 2 experts per group get ``hot_shift`` added to their bias so
    that about half of all (token, slot) pairs land on them.
The constants TIE_PAIRS and HOT_SHIFT were fitted with the CPU oracle by
``tests/golden/calibrate_workloads.py`` (results in
``tests/golden/workload_calibration.json``).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

D_MODEL = 7168

# Fitted by tests/golden/calibrate_workloads.py at seed 0 (see module doc).
TIE_PAIRS = 3
HOT_SHIFT = 0.2763


@dataclass(frozen=True)
class GateConfig:
    """Router hyper-parameters: E experts in n_group groups, keep topk_group
    groups, select top_k experts, scale the renormalised weights."""
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    route_scale: float


DSV3 = GateConfig(n_experts=256, n_group=8, topk_group=4, top_k=8, route_scale=2.5)
KIMI_K2 = GateConfig(n_experts=384, n_group=1, topk_group=1, top_k=8, route_scale=2.827)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    cfg: GateConfig
    seed: int = 0
    tie_pairs: int = 0
    hot_per_group: int = 0
    hot_shift: float = 0.0
    dispatch: bool = False
    description: str = ""


WORKLOADS = {
    w.name: w for w in [
        Workload("dsv3-tiny", 64, D_MODEL, DSV3,
                 description="DeepSeek-V3 gate, 64 tokens"),
        Workload("kimi-k2-decode", 256, D_MODEL, KIMI_K2,
                 description="Kimi-K2 gate, decode batch of 256 tokens"),
        Workload("dsv3-prefill-ties", 16384, D_MODEL, DSV3,
                 tie_pairs=TIE_PAIRS, dispatch=True,
                 description="DeepSeek-V3 gate + dispatch, 16384 tokens, twin "
                             "expert rows forcing exact score ties"),
        Workload("kimi-k2-prefill", 16384, D_MODEL, KIMI_K2, dispatch=True,
                 description="Kimi-K2 gate + dispatch, 16384 tokens"),
        Workload("dsv3-skewed", 65536, D_MODEL, DSV3, hot_per_group=2,
                 hot_shift=HOT_SHIFT, dispatch=True,
                 description="DeepSeek-V3 gate + dispatch, 65536 tokens, 16 hot "
                             "experts taking about half of the assignments"),
    ]
}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs here are finite, so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


@dataclass
class GateInputs:
    x: np.ndarray          # uint16 bfloat16 bits [T, d]
    W: np.ndarray          # float32 [E, d]
    bias: np.ndarray       # float32 [E]
    twins: list = field(default_factory=list)   # [(source, copy)] expert pairs
    hot: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.default_rng(s) for s in ss.spawn(5)]


def make_x(T: int, d: int, rng: np.random.Generator, chunk: int = 4096) -> np.ndarray:
    """x ~ N(0,1) as bfloat16 bits, drawn in row chunks of ``chunk`` tokens."""
    x = np.empty((T, d), dtype=np.uint16)
    for r0 in range(0, T, chunk):
        r1 = min(T, r0 + chunk)
        x[r0:r1] = bf16_bits(rng.standard_normal((r1 - r0, d), dtype=np.float32))
    return x


def make_gate_inputs(T: int, d: int, cfg: GateConfig, seed: int = 0,
                     tie_pairs: int = 0, hot_per_group: int = 0,
                     hot_shift: float = 0.0, x: bool = True) -> GateInputs:
    """Seeded x, W and bias; ``x=False`` skips drawing x (empty array)."""
    rx, rw, rb, rt, rh = _streams(seed)
    E = cfg.n_experts
    W = (rw.standard_normal((E, d), dtype=np.float32)
         * np.float32(1.0 / np.sqrt(d))).astype(np.float32)
    bias = rb.uniform(-0.05, 0.05, size=E).astype(np.float32)
    S = E // cfg.n_group
    twins = []
    if tie_pairs:
        groups = rt.choice(cfg.n_group, size=tie_pairs,
                           replace=tie_pairs > cfg.n_group)
        used = set()
        for g in groups:
            while True:
                a, b = rt.choice(S, size=2, replace=False) + g * S
                if a not in used and b not in used:
                    break
            used.update((int(a), int(b)))
            W[b] = W[a]
            bias[b] = bias[a]
            twins.append((int(a), int(b)))
    hot = np.zeros(0, dtype=np.int64)
    if hot_per_group:
        hot = np.concatenate([rh.choice(S, size=hot_per_group, replace=False) + g * S
                              for g in range(cfg.n_group)]).astype(np.int64)
        hot.sort()
        bias[hot] = (bias[hot] + np.float32(hot_shift)).astype(np.float32)
    xa = make_x(T, d, rx) if x else np.zeros((0, d), dtype=np.uint16)
    return GateInputs(xa, W, bias, twins, hot)


def workload_inputs(w: Workload | str, T: int | None = None, x: bool = True) -> GateInputs:
    """Inputs of a named workload; ``T`` overrides the token count (the
    weights and bias do not depend on T)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_gate_inputs(w.T if T is None else T, w.d, w.cfg, w.seed,
                            w.tie_pairs, w.hot_per_group, w.hot_shift, x=x)


def random_indices(T: int, K: int, E: int, seed: int = 0,
                   hot: np.ndarray | None = None, hot_prob: float = 0.0) -> np.ndarray:
    """int32 [T, K] rows of K distinct expert ids, for dispatch-only tests.
    With ``hot`` given, each slot prefers a hot expert with ``hot_prob``."""
    rng = np.random.default_rng(seed)
    out = np.empty((T, K), dtype=np.int32)
    keys = rng.random((T, E))
    if hot is not None and len(hot) and hot_prob > 0:
        keys[:, hot] += hot_prob * 4.0
    out[:] = np.argsort(-keys, axis=1, kind="stable")[:, :K]
    # shuffle slots so rows are not sorted by key
    perm = rng.permuted(np.tile(np.arange(K), (T, 1)), axis=1)
    return np.take_along_axis(out, perm, axis=1).astype(np.int32)
