"""The chain and greedy kernels' block-index -> work-item orders, checked on the host: the
kernels' own order functions (compiled from csrc/chain.hip and csrc/greedy.hip for the host)
must map the grid one-to-one onto the work items, and every item must follow the items whose
words it awaits (a lazy row group follows the request's earlier groups; terminal items and
deciders follow every group).  The kernels' progress argument rests on the second property."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.parametrize("kernel", ["chain", "greedy"])
def test_block_orders_are_bijective_and_respect_dependencies(tmp_path, kernel):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "block_order_check")
    cmd = [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops"] + (["-DCHECK_GREEDY"] if kernel == "greedy" else []) + ["-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "exact_rejection_sampling_amd", "csrc"),
           os.path.join(HERE, "block_order_check.hip"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "ok" in out.stdout
