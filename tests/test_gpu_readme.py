"""The Python example in README.md runs as written.  Needs an MI355X."""
import os
import re

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with open(os.path.join(ROOT, "README.md")) as f:
        text = f.read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README.md has no python example"
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)   # noqa: S102 (the repository's own text)
    torch.cuda.synchronize()
    T, K = env["cfg"].T, env["cfg"].top_k
    assert tuple(env["weights"].shape) == (T, K) and tuple(env["indices"].shape) == (T, K)
    assert int(env["out"].tokens_per_expert.sum()) == T * K
    # identity experts: the combine gives back route_scale * x (bf16 rounding)
    want = env["x"].float() * env["cfg"].route_scale
    assert torch.allclose(env["y"].float(), want, rtol=1 / 64, atol=1e-30)
