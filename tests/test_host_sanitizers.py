"""The C ABI's host code under the address and undefined-behaviour
sanitizers: argument rejection and workspace planning over many shapes, run
on the CPU by a small driver (tests/host/abi_driver.cpp) linked with a
sanitizer build of the host code and the uninstrumented kernels.  No case
reaches a HIP call."""
import os
import subprocess

import pytest

from chunked_kl_loss_logit_amd import build as B


@pytest.fixture(scope="module")
def driver():
    try:
        return B.build_host_sanitizer_driver()
    except RuntimeError as e:  # pragma: no cover - toolchain problems are reported, not hidden
        pytest.fail(str(e))


def test_abi_host_code_is_clean_under_sanitizers(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ok: 0 failure(s)" in r.stdout
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out
