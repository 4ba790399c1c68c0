"""CPU tests of the Python binding's contract (no GPU needed):

* the product path has no CPU fallback: a missing library, a plan on a CPU
  device and CPU tensors handed to a run all raise;
* the product package never imports the CPU oracle, and the oracle never
  imports the product package.
"""
import ast
import os
import subprocess
import sys

import pytest
import torch

import paged_kv_cache_plan_amd as pka

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_raises(tmp_path):
    code = ("import paged_kv_cache_plan_amd as pka\n"
            "try:\n"
            f"    pka.load_library({str(tmp_path / 'libpka.so')!r})\n"
            "except RuntimeError as e:\n"
            "    print('raised', e)\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert "raised" in out.stdout and "not built" in out.stdout


def test_plan_on_cpu_device_raises():
    with pytest.raises(ValueError, match="GPU"):
        pka.Plan([0, 3], [0, 1], [0], [3], 4, 2, 64, 4, causal=True, num_pages=1, device="cpu")


def test_cpu_tensors_are_rejected():
    with pytest.raises(ValueError, match="GPU tensor"):
        pka._dev_ptr(torch.zeros(4), "q")
    v = torch.zeros((2, 2, 1, 64), dtype=torch.float32)
    s = torch.zeros((2, 2, 1), dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        pka.merge_states(v, s)


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "paged_kv_cache_plan_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            assert "oracle" not in _imports(os.path.join(pkg, f)), f
    csrc = os.path.join(pkg, "csrc")
    for f in os.listdir(csrc):
        assert "oracle" not in open(os.path.join(csrc, f)).read(), f
    code = "import sys, paged_kv_cache_plan_amd\nprint('oracle' in sys.modules)"
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert out.stdout.strip() == "False", out.stdout + out.stderr


def test_oracle_never_imports_the_product():
    odir = os.path.join(ROOT, "oracle")
    for f in os.listdir(odir):
        if f.endswith(".py"):
            assert "paged_kv_cache_plan_amd" not in _imports(os.path.join(odir, f)), f
