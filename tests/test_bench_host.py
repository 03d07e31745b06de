"""Host logic of the benchmark, on the CPU: the split-count model picks the
counts the decode figures are quoted at, a split covers whole 64-token pages
and no more of them than it needs, and a run on more than one GPU is refused
before anything touches a GPU."""
import math
import os
import subprocess
import sys

import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name,want", [("dsv3", 8), ("grouped", 32), ("long", 256), ("mtp", 3)])
def test_default_splits(name, want):
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, seed=0)  # the benchmark's inputs
    assert bench.default_splits(wl, inp["seq_lens"]) == want


def test_split_len_whole_pages():
    for T in (1, 63, 64, 65, 1000, 4096, 9373, 262144):
        for P in (1, 3, 7, 8, 256):
            L = bench.split_len(T, P)
            assert L % 64 == 0 and L >= 64
            assert L * P >= T                       # the splits cover the sequence
            assert L - 64 < math.ceil(T / P)        # with no page to spare


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
