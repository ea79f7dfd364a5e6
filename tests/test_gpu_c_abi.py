"""The C ABI used from a plain C++ program (no Python, no PyTorch): the
example binary built with the library allocates with hipMalloc, runs the
gate, the dispatch and the combine, and checks what the results must
satisfy (ids, groups, weight sums, counts, offsets, a stable expert-major
permutation and its inverse, rows copied bit for bit, identity-expert
combine).  Needs an MI355X."""
import json
import os
import subprocess

import pytest

from parity import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "sigmoid_group_limited_amd", "route_c")


@pytest.mark.parametrize("model,T,d,route", [("kimi", 256, 7168, "fp32"), ("dsv3", 64, 7168, "fp32"),
                                             ("dsv3", 1000, 520, "fp32"), ("kimi", 16390, 256, "fp32"),
                                             ("dsv3", 0, 7168, "fp32"), ("kimi", 256, 7168, "x3"),
                                             ("kimi", 16390, 256, "x3"), ("dsv3", 5000, 1000, "x3")])
def test_c_example(model, T, d, route):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built (the package build makes it)")
    say(f"[c-abi] {model} T={T} d={d} {route}")
    r = subprocess.run([EXE, model, str(T), str(d), route], capture_output=True, text=True,
                       timeout=100)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-2000:]
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["checks_failed"] == 0
