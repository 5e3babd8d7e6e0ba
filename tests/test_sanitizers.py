"""Memory safety of the host code, on the CPU: the oracle and the C ABI's
argument validation run under AddressSanitizer and UndefinedBehaviorSanitizer
(tests/sanitizers/: the drivers and their build).  The oracle driver calls
every oracle function on small and edge-case shapes; the ABI driver calls every
entry point with arguments validation must reject (no call reaches a GPU)."""
import os
import shutil
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "sanitizers"))

import build_and_run  # noqa: E402


def test_oracle_under_asan_ubsan():
    rc, out = build_and_run.oracle()
    assert rc == 0 and out.endswith("oracle driver ok"), out[-3000:]


@pytest.mark.skipif(not os.path.exists(build_and_run.HIPCC) or shutil.which("gcc") is None,
                    reason="needs hipcc")
def test_c_abi_validation_under_asan_ubsan():
    rc, out = build_and_run.abi()
    assert rc == 0 and out.endswith("abi driver ok"), out[-3000:]
