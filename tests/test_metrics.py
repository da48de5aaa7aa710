"""The host-side useful-pair counter (closed form over residue classes) must
equal the oracle's explicit enumeration of N(i), bit for bit."""
import numpy as np
import pytest

import oracle
from sparse_long_sequence_lf_amd import metrics
from sparse_long_sequence_lf_amd import workloads as W


@pytest.mark.parametrize("seed", range(12))
def test_counter_matches_enumeration_random(seed):
    rng = np.random.default_rng(seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    T = int(rng.integers(1, 300))
    r = int(rng.integers(0, T + 3))
    dil = [int(x) for x in rng.integers(1, 6, size=H)]
    G = [int(x) for x in rng.integers(0, T, size=int(rng.integers(0, 7)))]
    pad = (rng.random((B, T)) < 0.2).astype(np.uint8) if seed % 2 else None
    want = oracle.count_pairs(B, H, T, r, dil, G, pad)
    assert metrics.useful_pairs(B, H, T, r, dil, G, pad) == want


@pytest.mark.parametrize("seed", range(10))
def test_counter_matches_enumeration_per_head_one_sided(seed):
    rng = np.random.default_rng(100 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 5))
    T = int(rng.integers(1, 300))
    rads = [int(x) for x in rng.integers(0, T + 3, size=H)]
    dil = [int(x) for x in rng.integers(1, 6, size=H)]
    G = [int(x) for x in rng.integers(0, T, size=int(rng.integers(0, 7)))]
    pad = (rng.random((B, T)) < 0.2).astype(np.uint8) if seed % 2 else None
    one = seed % 3 != 0
    want = oracle.count_pairs(B, H, T, rads, dil, G, pad, one_sided=one)
    assert metrics.useful_pairs(B, H, T, rads, dil, G, pad, one_sided=one) == want


@pytest.mark.parametrize("seed", range(10))
def test_counter_matches_enumeration_random_blocks(seed):
    rng = np.random.default_rng(200 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    T = int(rng.integers(1, 400))
    rads = [int(x) for x in rng.integers(0, 100, size=H)]
    G = [int(x) for x in rng.integers(0, T, size=int(rng.integers(0, 7)))]
    pad = (rng.random((B, T)) < 0.2).astype(np.uint8) if seed % 2 else None
    one = seed % 3 == 0
    nqb = (T + 63) // 64
    rb = rng.integers(0, nqb, size=(H, nqb, int(rng.integers(1, 4)))).astype(np.int32)
    want = oracle.count_pairs(B, H, T, rads, None, G, pad, one_sided=one, random_blocks=rb)
    assert metrics.useful_pairs(B, H, T, rads, None, G, pad, one_sided=one, random_blocks=rb) == want


@pytest.mark.parametrize("name", [w.name for w in W.WORKLOADS])
def test_counter_matches_enumeration_workloads(name):
    w = W.workload(name)
    kw = {}
    if w.T > 4096:
        kw = dict(T=4096, H=4)
    inp = W.make_inputs(w, **kw)
    B, H, T, d = inp.q.shape
    want = oracle.count_pairs(B, H, T, inp.r, inp.dilation, inp.global_idx, inp.key_padding_mask,
                              one_sided=inp.one_sided, random_blocks=inp.random_blocks)
    got = metrics.useful_pairs(B, H, T, inp.r, inp.dilation, inp.global_idx, inp.key_padding_mask,
                               one_sided=inp.one_sided, random_blocks=inp.random_blocks)
    assert got == want


def test_workload_counts_closed_form():
    # per-head closed forms of the window and the single global at 0
    assert metrics.useful_pairs(1, 2, 1024, 64, None, [0]) == 259708
    assert metrics.useful_pairs(1, 12, 4096, 256, None, [0]) == 24517608
    assert metrics.useful_pairs(1, 12, 4096, 128, [1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 4, 4], []) == 12136704


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: bench.py exits with status 2 and says why, before it
    # touches torch or the library
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""
