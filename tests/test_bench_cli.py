"""bench.py's host logic on the CPU: the one-GPU refusal, the sparse FLOP count, and the
counter figures it reports only while they match the kernel source they were taken on."""

import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_sparse_flops_counts_kept_tokens():
    """4 d sum over query blocks i and kept blocks j of r_i c_j, with the short last block's
    token count on either side."""
    N, d, block = 150, 16, 64  # blocks of 64, 64 and 22 tokens
    r = [64, 64, 22]
    rng = np.random.default_rng(3)
    idx = np.sort(np.stack([[rng.choice(3, 2, replace=False) for _ in range(3)] for _ in range(4)]), -1)
    idx = idx.reshape(2, 2, 3, 2)
    want = 0
    for b in range(2):
        for h in range(2):
            for i in range(3):
                for j in idx[b, h, i]:
                    want += 4 * d * r[i] * r[j]
    got = bench.sparse_flops(torch.from_numpy(idx.astype(np.int32)), N, d, block)
    assert got == want


def test_traffic_only_for_the_measured_source():
    digest = bench.source_digest(bench.PAIR_SOURCES)
    assert bench.traffic_for("pair_kernel@video_s", "0" * 16) is None
    assert bench.traffic_for("no_such_kernel@video_s", digest) is None
    got = bench.traffic_for("pair_kernel@video_s", digest)
    # committed counters either match this source (a positive byte count) or are stale (None)
    assert got is None or got > 0
