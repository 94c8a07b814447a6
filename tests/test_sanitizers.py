"""AddressSanitizer and UndefinedBehaviorSanitizer builds (CPU only): the C
oracle running every routine on small inputs and rejected arguments, and the
library's host-side argument checking on the workload shapes, null and forged
handles and thousands of seeded configurations (tests/sanitize/*.c).  A
sanitizer report makes the driver exit non-zero."""
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "sanitize"))
import build as san  # noqa: E402

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert r.returncode == 0, f"{os.path.basename(exe)} exited {r.returncode}:\n{r.stdout[-2000:]}\n{r.stderr[-6000:]}"
    return r.stdout


def test_oracle_under_sanitizers():
    assert "oracle checks ok" in _run(san.oracle_checks())


@pytest.mark.timeout(900)
def test_host_checks_under_sanitizers():
    out = _run(san.host_checks())
    assert "host checks ok" in out, out
