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


def test_committed_counter_summaries_parse():
    """Every committed per-kernel counter summary names its kernels with calibrated
    bytes, algorithmic bytes and a source digest."""
    for name in (bench.STEP_COUNTERS, bench.STEP_1M_COUNTERS, bench.COMPRESS_COUNTERS, bench.PREFILL_COUNTERS,
                 bench.FP4_COUNTERS):
        c = bench.kernel_counters(name)
        assert c, name
        for label, v in c.items():
            assert v["alg_B"] > 0 and v["profiled_us"] > 0, (name, label)
            if not v["stale"]:
                assert v["traffic_B"] == v["fetch_B"] + v["write_B"]
    assert "index_score_decode" in bench.kernel_counters(bench.STEP_COUNTERS)


def test_counter_summary_on_other_sources_reports_no_traffic(tmp_path, monkeypatch):
    src = os.path.join(bench.PROFILES, bench.STEP_COUNTERS)
    with open(src) as f:
        text = f.read()
    lines = [ln if not ln.startswith("counter: topk_kernel ") else ln.rsplit("sha256=", 1)[0] + "sha256=" + "0" * 64
             for ln in text.splitlines()]
    (tmp_path / "s.txt").write_text("\n".join(lines) + "\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    c = bench.kernel_counters("s.txt")
    assert c["topk_kernel"]["stale"] and c["topk_kernel"]["traffic_B"] is None
    assert bench.kernel_counters("missing.txt") == {}


def test_read_reference_library_rejects_bad_arguments():
    """The benchmark's read references (libsckv_bench.so) export the streaming read
    and the row gather, and refuse null pointers and empty shapes before any HIP
    call (hipErrorInvalidValue = 1), so this runs without a GPU."""
    import ctypes as C
    lib_path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "sequence_compressed_kv_amd", "libsckv_bench.so")
    if not os.path.exists(lib_path):
        import pytest
        pytest.skip("libsckv_bench.so not built")
    lib = C.CDLL(lib_path)
    lib.sckv_bench_stream_read.argtypes = [C.c_void_p, C.c_size_t, C.c_void_p, C.c_int, C.c_void_p]
    lib.sckv_bench_gather_rows.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p,
                                           C.c_void_p]
    fake = C.c_void_p(16)                      # never dereferenced: the checks fail first
    assert lib.sckv_bench_stream_read(None, 1024, fake, 1, None) == 1
    assert lib.sckv_bench_stream_read(fake, 1000, fake, 1, None) == 1    # not a multiple of 16
    assert lib.sckv_bench_gather_rows(None, fake, 1, 1, 1, fake, None) == 1
    assert lib.sckv_bench_gather_rows(fake, None, 1, 1, 0, fake, None) == 1
    assert lib.sckv_bench_gather_rows(fake, fake, 0, 1, 1, fake, None) == 1
    assert lib.sckv_bench_gather_rows(fake, fake, 1, 0, 0, fake, None) == 1
