"""Host logic of bench.py on the CPU: the allowed-pair count that every TFLOP/s figure is
built on, pinned against the oracle's mask definition (brute force over small shapes)
and closed forms; and the refusal of more than one GPU."""
import subprocess
import sys

import numpy as np
import pytest

import bench
from exact_io_aware_46_amd import inputs as inp
from oracle import attention as orc


def brute(N, causal, bm, kv, window):
    return int(orc.allowed(np.arange(N), N, causal, bm, kv, window).sum())


@pytest.mark.parametrize("seed", range(12))
def test_allowed_pairs_equals_the_oracle_mask_count(seed):
    rng = np.random.Generator(np.random.PCG64(900 + seed))
    N = int(rng.integers(1, 420))
    causal = bool(rng.integers(2))
    kv = None if rng.integers(2) else int(rng.integers(0, N + 1))
    window = None if rng.integers(2) else (int(rng.integers(-1, N + 2)),
                                           int(rng.integers(-1, N + 2)))
    bm = None if rng.integers(2) else inp.draw_block_mask(rng, N, 0.5)
    assert bench.allowed_pairs(N, causal, bm, kv, window) == brute(N, causal, bm, kv, window)


def test_allowed_pairs_closed_forms():
    N = 16384
    assert bench.allowed_pairs(N, False, None, None) == N * N
    assert bench.allowed_pairs(N, True, None, None) == N * (N + 1) // 2
    # 16 heads of 16K causal queries: the figure the long causal workload's FLOPs use
    assert 16 * bench.allowed_pairs(N, True, None, None) == 2_147_614_720
    assert bench.allowed_pairs(N, False, None, 300) == N * 300
    w = 4095  # causal window of 4096 keys
    assert bench.allowed_pairs(N, True, None, None, (w, 0)) == \
        sum(min(i + 1, w + 1) for i in range(N))
    assert bench.allowed_pairs(N, False, None, None, (0, 0)) == N
    nb = inp.n_blocks(N)
    assert bench.allowed_pairs(N, False, np.eye(nb, dtype=np.uint8), None) == nb * 128 * 128


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
