"""The work plans for fewer compute units than the device has (a partitioned
MI355X, or a GPU shared with other work: ATTN_GQA_CUS caps the count the
library plans for) give the oracle's results on the GPU. Each count runs in a
child process (the cap is read once per process): tests/cus_limit_check.py."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
@pytest.mark.parametrize("cus", [32, 100])
def test_calls_planned_for_fewer_compute_units_match_the_oracle(cus):
    print(f"child process with ATTN_GQA_CUS={cus}", flush=True)
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "cus_limit_check.py")],
                          env=dict(os.environ, ATTN_GQA_CUS=str(cus)), capture_output=True,
                          text=True, timeout=300)
    print(proc.stdout[-3000:], flush=True)
    assert proc.returncode == 0, proc.stdout[-3000:] + proc.stderr[-3000:]
    assert "all ok" in proc.stdout
