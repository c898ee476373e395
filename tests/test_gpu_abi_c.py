"""The library called from plain C (tests/abi_c_demo.c, compiled by __graft_entry__.build()):
device buffers from the HIP runtime, greedy and chain verification of hand-worked cases,
and the chain workspace back at zero.  No Python or torch in the caller."""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_c_demo")


def test_c_caller():
    assert os.path.exists(EXE), "tests/abi_c_demo is missing: run __graft_entry__.build()"
    say("C caller of the library")
    out = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.strip() == "ok"
