"""The Python example in README.md runs as written."""

import os
import re

import pytest
import torch

from helpers import ensure_built

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_readme_example_runs():
    ensure_built()
    assert torch.cuda.is_available()
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, flags=re.S)
    assert blocks, "README.md has a python example"
    scope = {}
    exec(compile(blocks[0], "README.md", "exec"), scope)
    torch.cuda.synchronize()
    o, state = scope["o"], scope["state"]
    assert o.shape == (8, 4, 16, 128) and torch.isfinite(o).all()
    assert torch.isfinite(state).all()
