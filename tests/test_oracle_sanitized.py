"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only) and run through its entry points on small inputs in a
child process: any out-of-bounds access, use after free or undefined
behaviour aborts the child and fails the test.  CPU only."""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    from sigmoid_group_limited_amd import workloads as wl
    o = oracle.Oracle(LIB)
    for gc, T, d in [(wl.DSV3, 37, 64), (wl.KIMI_K2, 20, 40), (wl.GateConfig(128, 64, 4, 8, 1.0), 9, 24),
                     (wl.DSV3, 1, 8), (wl.GateConfig(512, 8, 4, 8, 2.5), 5, 16),
                     (wl.GateConfig(192, 8, 4, 8, 2.5), 11, 24), (wl.GateConfig(64, 4, 2, 6, 1.0), 7, 8)]:
        gi = wl.make_gate_inputs(T, d, gc, seed=T)
        for opts in ({}, {"score_func": 1}, {"mask_zero": 1, "denom_eps": 1e-20}, {"renorm": 2}):
            for bias in (gi.bias, None):
                r = o.gate(gi.x, gi.W, bias, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                           order=1, **opts)
        r = o.gate(gi.x, gi.W, gi.bias, gc.n_group, gc.topk_group, gc.top_k, gc.route_scale,
                   with_scores=True)
        o.scores(o.logits(gi.x, gi.W), None, gc.n_group, score_func=1)
        dr = o.dispatch(r.indices, gc.n_experts)
        o.gather_rows(gi.x, dr.perm, gc.top_k)
        outs = wl.bf16_bits(np.random.default_rng(1).standard_normal((T * gc.top_k, d), dtype=np.float32))
        o.combine(outs, r.weights, np.argsort(dr.perm).astype(np.int32))
        o.logits(gi.x, gi.W)
        for ranks in (1, 2, 4):
            if gc.n_experts % ranks == 0:
                o.ep_send_splits(dr.counts, ranks)
                o.ep_dedup(r.indices, gc.n_experts, ranks)
                o.ep_regroup(np.asarray(dr.counts).reshape(ranks, -1))
    o.dispatch(np.zeros((0, 8), np.int32), 256)
    print("sanitized oracle ok")
""")


def test_oracle_under_asan_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    if not (os.path.isabs(asan) and os.path.exists(asan) and os.path.exists(ubsan)):
        pytest.skip("gcc sanitizer runtimes not available")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall",
                    oracle.SOURCE, "-o", lib, "-lm"], check=True)
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0 and "sanitized oracle ok" in r.stdout, r.stderr[-4000:]
