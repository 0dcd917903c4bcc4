"""The C ABI from plain C: tests/c_abi_check.c (no PyTorch, no Python in the process) runs the
producer and the three GEMVs on small seeded inputs and checks them against the CPU oracle.
It is started as a child process."""
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import c_abi_build  # noqa: E402


@pytest.mark.gpu
def test_plain_c_consumer_matches_the_oracle():
    if not os.path.exists(c_abi_build.BIN):
        pytest.fail(f"{c_abi_build.BIN} is not built: run __graft_entry__.build() first")
    print("running", c_abi_build.BIN, flush=True)
    r = subprocess.run([c_abi_build.BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout[-4000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "c_abi_check PASS" in r.stdout
