"""Host-side checks of bench.py's bookkeeping (no GPU): the closed-form prefill FLOP count
against the oracle's own count, and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
from paged_split_kv_pa_amd import workloads as wl  # noqa: E402


def test_prefill_flops_matches_oracle_count():
    for i in range(len(wl.PREFILL_CONFIG_NAMES)):
        w = wl.prefill_config(i)
        assert bench.prefill_flops(w) == oracle.prefill_flops(
            w.context_lens, w.query_start, w.num_q_heads, w.head_dim), w.name


def test_prefill_flops_small_case_by_hand():
    # one sequence, prefix 3, two new tokens, 1 head, D = 2: token 0 sees 4 keys, token 1
    # sees 5; 4 D FLOP per (row, key) pair
    class W:
        num_seqs, num_q_heads, head_dim = 1, 1, 2
        context_lens = np.array([3])
        query_start = np.array([0, 2])
    assert bench.prefill_flops(W) == 4 * 2 * (4 + 5)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
