"""The C-ABI layer under host sanitizers: capi.cpp built by g++ with
AddressSanitizer and UndefinedBehaviorSanitizer (any report is fatal), linked
with the kernel objects, and the ABI tests (argument checks, status codes,
error text, the no-device path) run against it in a child process with the
sanitizer runtimes preloaded.  No GPU needed."""
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_under_host_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("sanitizer runtimes not installed")
    from mxfp4_mixture_experts_amd import build_lib
    lib = build_lib.build_host_sanitized()
    env = dict(os.environ)
    env.update({
        "MXFP4_MOE_LIB": lib,
        "LD_PRELOAD": f"{asan} {ubsan}",
        # the interpreter and the HIP runtime keep allocations until exit: leaks are not this layer's
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    text = res.stdout + res.stderr
    assert res.returncode == 0, text[-4000:]
    assert "AddressSanitizer" not in text and "runtime error" not in text, text[-4000:]
    assert " passed" in text
