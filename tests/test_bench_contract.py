"""Host-side checks of bench.py's contract (no GPU needed): more than one GPU
is refused with a message, and the algorithmic byte counts it reports follow
from the cache formats."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_attention_decode_e2m1_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kv_bytes_per_query_of_the_decode_group():
    """Four layers at 256K context: the Full and Reindex layers scan every
    72-byte index row; every layer gathers 2048 FP4 rows of 324 bytes and
    128 FP8 window rows of 576 bytes."""
    w = I.WORKLOADS["C3_group_b4_256k"]
    kv = bench.kv_bytes_per_query(w)
    attn = 2048 * 324 + 128 * 576
    scan = 262144 * 72
    assert kv["per_layer"] == [attn + scan, attn + scan, attn, attn]
    assert kv["index_scan_per_step"] == 2 * scan * 4
    assert kv["total"] == 4 * attn + 2 * scan
