"""The C ABI from plain C: tests/c_abi/example (built by
__graft_entry__.build() with gcc from example.c, which includes only
include/lioncub.h, the HIP runtime's C API and the oracle's header) runs
three steps of every aggregation mode through lioncub_step and compares
theta and the momenta bit for bit with the CPU oracle, and two cases
through the allocation-free lioncub_step_static; it also checks that
argument errors are returned as status codes.  Run as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "example")


def test_plain_c_consumer_matches_the_oracle():
    assert os.path.exists(EXE), f"{EXE} is not built; run __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("OK")
    for case in ("vote", "l1-sum n=4", "average", "max-norm n=3", "allocation-free l1-sum n=8",
                 "allocation-free vote"):
        assert f"{case}: 0 values differ from the oracle" in r.stdout
