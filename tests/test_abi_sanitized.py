"""The C-ABI host checks under AddressSanitizer and UndefinedBehaviorSanitizer:
api.cpp is rebuilt by the host compiler with both sanitizers (the device code
is the regular build's), and the CPU tests of tests/test_abi.py run against
that build in a child process with the sanitizer runtimes preloaded.  Any
sanitizer report fails the child (-fno-sanitize-recover, halt_on_error)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_abi_checks_under_asan_and_ubsan():
    if shutil.which("g++") is None:
        pytest.skip("no host compiler")
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("the ABI tests run on CPU-only hosts (fake device addresses)")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("sanitizer runtimes not installed")
    from causal_self_attention_mha_amd import build
    if not all(os.path.exists(os.path.join(build.BUILD, s + ".o")) for s in build.SOURCES):
        pytest.skip("regular build objects missing")
    lib = build.build_sanitized()
    env = dict(os.environ)
    env.update(NA_ATTN_LIBRARY=lib, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in out
