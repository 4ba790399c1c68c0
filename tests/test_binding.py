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


def test_product_never_imports_the_input_generator():
    pkg = os.path.join(ROOT, "paged_kv_cache_plan_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            assert "inputs" not in _imports(os.path.join(pkg, f)), f


def test_oracle_never_imports_the_input_generator():
    """The oracle takes its inputs as arguments: it shares nothing with the
    generator that draws them."""
    odir = os.path.join(ROOT, "oracle")
    for f in os.listdir(odir):
        if f.endswith(".py"):
            assert "inputs" not in _imports(os.path.join(odir, f)), f


# ---------------------------------------------------------------------------
# Run arguments are checked against the plan before any pointer is passed
# ---------------------------------------------------------------------------

def _io(out_fp32=False):
    return pka.IoShape(total_q=10, num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=4, num_pages=7,
                       total_kv=30, out_fp32=out_fp32)


def _t(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="meta")


GOOD = dict(q=((10, 4, 64), torch.bfloat16), o=((10, 4, 64), torch.bfloat16), lse=((10, 4), torch.float32),
            paged_kv=((7, 2, 4, 2, 64), torch.bfloat16))

BAD = {
    "q_heads": dict(q=((10, 3, 64), torch.bfloat16)),
    "q_rows": dict(q=((9, 4, 64), torch.bfloat16)),
    "q_dtype": dict(q=((10, 4, 64), torch.float16)),
    "q_head_dim": dict(q=((10, 4, 128), torch.bfloat16)),
    "o_dtype": dict(o=((10, 4, 64), torch.float32)),
    "o_rows": dict(o=((9, 4, 64), torch.bfloat16)),
    "lse_shape": dict(lse=((10, 3), torch.float32)),
    "lse_dtype": dict(lse=((10, 4), torch.bfloat16)),
    "pool_pages": dict(paged_kv=((6, 2, 4, 2, 64), torch.bfloat16)),
    "pool_page_size": dict(paged_kv=((7, 2, 8, 2, 64), torch.bfloat16)),
    "pool_kv_heads": dict(paged_kv=((7, 2, 4, 1, 64), torch.bfloat16)),
    "pool_dims": dict(paged_kv=((7, 4, 2, 64), torch.bfloat16)),
    "pool_dtype": dict(paged_kv=((7, 2, 4, 2, 64), torch.float32)),
}


def _call(spec, out_fp32=False, **extra):
    t = {k: _t(*v) for k, v in {**GOOD, **spec}.items()}
    pka.check_io(_io(out_fp32), t["q"], t["o"], t["lse"], paged_kv=t["paged_kv"], **extra)


def test_run_arguments_accepted():
    _call({})
    # larger buffers (a graph-stable plan's) are fine
    _call(dict(q=((12, 4, 64), torch.bfloat16), o=((12, 4, 64), torch.bfloat16), lse=((12, 4), torch.float32),
               paged_kv=((9, 2, 4, 2, 64), torch.bfloat16)))
    _call(dict(o=((10, 4, 64), torch.float32)), out_fp32=True)
    _call({}, k=_t((30, 2, 64)), v=_t((31, 2, 64)))


@pytest.mark.parametrize("name", sorted(BAD))
def test_run_arguments_rejected(name):
    with pytest.raises(ValueError):
        _call(BAD[name])


def test_out_fp32_plan_rejects_bf16_output():
    with pytest.raises(ValueError, match="output dtype"):
        _call({}, out_fp32=True)


@pytest.mark.parametrize("kw", [dict(k=((29, 2, 64),)), dict(v=((30, 2, 32),)), dict(k_cache=((6, 4, 2, 64),))])
def test_kv_tensors_rejected(kw):
    with pytest.raises(ValueError):
        _call({}, **{k: _t(*v) for k, v in kw.items()})
