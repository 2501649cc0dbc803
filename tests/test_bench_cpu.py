"""Host logic of bench.py (no GPU): algorithmic bytes, the input copies of the step clock
and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_headline_algorithmic_bytes():
    """64 rows x (32768 x 128 B keys + 2048 x 400 B entries + 128 x 64 x 512 B window) plus
    queries, Top-K output and fp32 outputs: 606,177,280 bytes per step."""
    w = synth.workload(2)
    a = bench.algorithmic_bytes(w)
    assert a["idx_score"] == 64 * (32768 * 128 + 8 * (64 * 2 + 4))
    assert a["topk"] == 64 * 2048 * 4
    assert a["sparse_attn"] == 64 * 2048 * 400 + 64 * 64 * (576 * 2 + 512 * 4 + 4)
    assert a["swa"] == 64 * 128 * 64 * 512 + 64 * 64 * (128 * 2 + 128 * 4 + 4)
    assert sum(a.values()) == 606_177_280


@pytest.mark.parametrize("idx,copies", [(2, 2), (3, 2), (4, 5), (5, 2)])
def test_input_copies(idx, copies):
    """Enough copies that two steps on one copy are at least 512 MiB of streamed bytes
    apart (the 4 x 1M decode moves 155 MB per step)."""
    w = synth.workload(idx)
    n = bench.input_copies(w)
    assert n == copies
    per = sum(bench.algorithmic_bytes(w).values()) if 3 not in w.modes else None
    if per is not None:
        assert (n - 1) * per >= 2 * bench.LLC_BYTES


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
