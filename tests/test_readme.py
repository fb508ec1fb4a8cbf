"""The usage example of README.md: on the CPU, that it parses and names only
functions the binding has; on the GPU, that it runs and its own checks hold."""

import ast
import os
import re

import pytest

import cg_streaming_vector_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def readme_example():
    text = open(os.path.join(ROOT, "README.md")).read()
    blocks = re.findall(r"```python\n(.*?)```", text, re.S)
    assert len(blocks) == 1, "README.md should hold one python example"
    return blocks[0]


def test_readme_example_names_exist():
    tree = ast.parse(readme_example())
    used = {node.attr for node in ast.walk(tree)
            if isinstance(node, ast.Attribute) and isinstance(node.value, ast.Name) and node.value.id == "bs"}
    assert used, "the example calls nothing from the binding"
    missing = sorted(name for name in used if not hasattr(bs, name))
    assert not missing, f"README names functions the binding lacks: {missing}"


@pytest.mark.gpu
def test_readme_example_runs():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    print("README example on cuda:0", flush=True)
    exec(compile(readme_example(), "README.md", "exec"), {"__name__": "readme_example"})
