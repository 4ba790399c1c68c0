"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU, no GPU).

The planner does all of the plan's index and offset arithmetic (tiling,
split-KV, queue ordering, image layout), and the HIP-free entry points wrap
it; both are built on their own, with g++ -fsanitize=address,undefined, into
libpka_planner_host.so.  This test reruns the planner tests (restatement,
coverage, named workloads, queues, edge lengths, error codes, mixed batches)
in a child process that loads that library instead of libpka.so, with the
ASan runtime preloaded, and fails on any sanitizer report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_LIB = os.path.join(ROOT, "paged_kv_cache_plan_amd", "libpka_planner_host.so")


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True, timeout=60)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_planner_tests_pass_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime for the host compiler")
    if not os.path.exists(HOST_LIB):
        from paged_kv_cache_plan_amd import build as B
        B.build_host_sanitized()
    env = dict(os.environ)
    env.update({
        "PKA_LIBRARY": HOST_LIB,
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1:exitcode=87",
    })
    # every planner test but the two that need the full library (its exports,
    # and the run / create entry points)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_planner.py"),
           "-k", "not exports_every_declared_symbol and not run_errors_without_a_gpu"]
    out = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    text = out.stdout + out.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-6000:]
    assert out.returncode == 0, text[-6000:]
    assert " passed" in out.stdout and " failed" not in out.stdout, out.stdout[-3000:]
