"""The Python example in README.md runs as written: one prefill into a
4-row cache and eight decode steps, leaving every row at its new length."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def readme_example():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "README holds one Python example"
    return blocks[0]


def test_readme_example_compiles():
    compile(readme_example(), "README.md", "exec")


@pytest.mark.gpu
def test_readme_example_runs():
    ns = {}
    exec(compile(readme_example(), "README.md", "exec"), ns)
    cache, out, L, B = ns["cache"], ns["out"], ns["L"], ns["B"]
    assert cache.n_tokens.tolist() == [L + 8] * B
    assert bool(out.float().isfinite().all())
