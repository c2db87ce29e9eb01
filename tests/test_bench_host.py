"""bench.py's accounting, without a GPU: the algorithmic bytes behind the roofline
figures, and the single-GPU contract."""
import os
import subprocess
import sys

import bench
from workloads import PAIR_DEC_128K_BF16

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_scoring_bytes_per_launch():
    """Per query at 128K: 32735 visible keys x 128 dims in bf16, the 64 x 128 bf16
    indexer query and 64 fp32 head weights; a launch scores 32 queries."""
    ab = bench.algorithmic_bytes(PAIR_DEC_128K_BF16)
    assert ab["score"] == 32735 * 128 * 2 + 64 * 128 * 2 + 64 * 4
    assert ab["score"] * PAIR_DEC_128K_BF16.B == 268_697_600


def test_step_bytes_per_query():
    """Both layers' reads and writes of one decode query: keys and indexer inputs,
    the kept indices, CSA rows 1024 + window 128 and HCA rows 1022 + window 128 of
    1 KB each, the bf16 queries and the fp32 outputs of 64 heads x 512."""
    ab = bench.algorithmic_bytes(PAIR_DEC_128K_BF16)
    rows = (1024 + 128 + 1022 + 128) * 512 * 2
    qo = 2 * (64 * 512 * 2 + 64 * 512 * 4)
    assert ab["step"] == ab["score"] + 1024 * 4 + 1024 * 4 + rows + qo
    assert ab["step"] * PAIR_DEC_128K_BF16.B == 356_974_592


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
