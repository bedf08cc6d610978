"""The C ABI used from plain C with no Python in the process: a child process
runs tests/c_abi/moe_c_cycle (built by __graft_entry__.build()), which
drives two dispatch + combine cycles with identity experts and weights
summing to one, and checks out == x itself."""
import os
import subprocess

import pytest

from tests.gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c_abi", "moe_c_cycle")


def test_cycle_from_plain_c():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(BIN), f"{BIN} not built; run __graft_entry__.build()"
    say("[gpu] c-abi cycle from a plain C process")
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    say(res.stdout.strip())
    assert res.returncode == 0, res.stdout + res.stderr
    assert "mismatches=0 expert_offsets=ok" in res.stdout
