"""Host checks of bench.py's byte and flop models (no GPU): the C3 launch's
algorithmic bytes from the tile sizes the pages fix (a 6-bit 128 x 128 tile is
12,800 bytes: 6 bits per code plus one 16-bit scale per row and per column),
the window model's per-position terms, the prefill flop count of the chunk form,
and --gpus N > 1 refused with a message."""
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import Workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_tile_bytes_from_the_pages():
    assert bench.tile_bytes(6, 128, 128) == 128 * 128 * 6 // 8 + 2 * 256 == 12800
    assert bench.tile_bytes(16, 128, 128) == 2 * 128 * 128      # binary16 pivot head, no scales
    rows = np.array([4] * 64 + [8] * 64)
    assert bench.tile_bytes(rows, 128, 128) == 64 * 64 + 64 * 128 + 2 * 256


def test_c3_launch_bytes():
    wl = Workload("C3")
    tiles = sum(bench.tile_bytes(b, 128, 128) for b in wl.bits)
    io = 4 * (2 * 128 + 128) + 4 + 4 + 4 * 128
    assert bench.algorithmic_bytes(wl) == 512 * (2 * tiles + 32 * io) == 460980224


def test_window_bytes_per_position():
    wl = Workload("C5")
    t = bench.tile_bytes(4, 128, 128)
    ent = 4 * (128 + 128 + 1)
    io = bench.io_bytes(128, 128, False)
    for pos in (0, 7):
        assert bench.algorithmic_bytes(wl, pos) == 512 * 32 * (t + 8 + pos * ent + ent + io)
    assert bench.algorithmic_bytes(wl, 15) == 512 * 32 * (2 * t + 8 + 16 * ent + io)


def test_prefill_flops():
    # per token and head: 6 dk dv (three state products) + dk L + 2 dv (L + 1)
    assert bench.prefill_flops(1, 1, 128, 128) == 6 * 128 * 128 + 128 * 32 + 2 * 128 * 33 == 110848


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
