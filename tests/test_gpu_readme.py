"""The Python example in README.md runs as written on the GPU, and its
results hold what the README says of them: the exchanges round-trip bit for
bit, the Ring partials merge to the single pass, the backward's gradients are
finite."""
import os
import re

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README.md has no python example"
    env = {}
    exec(compile(blocks[0], "README.md", "exec"), env)
    torch.cuda.synchronize()
    assert torch.equal(env["back"], env["shards"])
    o, o2, lse, lse2 = env["o"], env["o2"], env["lse"], env["lse2"]
    assert (o.float() - o2.float()).abs().max().item() <= 2e-2
    assert (lse - lse2).abs().max().item() <= 1e-3
    for g in ("dq", "dk", "dv", "delta"):
        assert torch.isfinite(env[g]).all(), g
