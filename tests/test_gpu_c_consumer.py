"""The library driven from plain C (tests/c_consumer/abi_consumer.c): device
memory from hipMalloc, prefill, step and commit through the C header alone,
each checked against the C oracle, plus a rejected call.  The program is
built by the package build step; this test only runs it."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_consumer", "abi_consumer")


def test_c_consumer():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build() first")
    print("running the C consumer", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=100)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, f"C consumer exited {r.returncode}:\n{r.stdout}\n{r.stderr}"
    assert "all checks passed" in r.stdout
