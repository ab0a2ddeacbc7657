"""The C ABI used from C: a plain C program (tests/c_abi/abi_check.c, built
by __graft_entry__.build() with gcc against the HIP runtime only) runs the
plan (with a workspace and allocation-free), the EPLB remap/prune with its
send map in both balance modes, the pack, the grouping and the combine
through include/mep.h and checks them bit for bit against the C oracle. It
runs as a child process."""
import os
import subprocess

import pytest

from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_check")


def test_c_consumer_matches_oracle():
    require_gpu()
    if not os.path.exists(BIN):
        pytest.skip("tests/c_abi/abi_check is not built (run __graft_entry__.build())")
    note("c abi consumer")
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi ok" in r.stdout
