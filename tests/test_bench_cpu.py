"""Host logic of bench.py, on the CPU: the one-GPU guard, the useful-pair counts behind every
TFLOP/s figure, and the rule that committed hardware counters only describe the workload and
kernel sources they were taken on."""
from __future__ import annotations

import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


def _brute_pairs(layout, P, c, p, causal):
    """Unmasked (query, key) pairs of device p per round, counted element by element from the
    token positions of the two layouts (contiguous: block k holds tokens k c .. k c + c - 1;
    striped: row y of block k is token y P + k)."""
    def pos(k):
        return np.arange(c) + k * c if layout == "contiguous" else np.arange(c) * P + k
    out = []
    for r in range(P):
        k = (p - r) % P
        if not causal:
            out.append(c * c)
            continue
        out.append(int((pos(p)[:, None] >= pos(k)[None, :]).sum()))
    return out


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
@pytest.mark.parametrize("P,c", [(1, 5), (3, 7), (4, 16), (8, 9)])
def test_useful_pairs_match_brute_force(bench, layout, P, c):
    for p in range(P):
        for causal in (True, False):
            assert bench.useful_pairs(layout, P, c, p, causal) == _brute_pairs(layout, P, c, p, causal)


def test_headline_flop_count(bench):
    # device 7 of the 256K share: 8 blocks of c = 32768 rows, 32 heads, d = 128
    c, H, d = 32768, 32, 128
    pairs = sum(bench.useful_pairs("striped", 8, c, 7))
    assert pairs == 8 * c * (c + 1) // 2
    assert 4.0 * d * H * pairs == pytest.approx(7.0370891661312e13, rel=1e-12)
    pairs_c = sum(bench.useful_pairs("contiguous", 8, c, 7))
    assert pairs_c == 7 * c * c + c * (c + 1) // 2


def test_profile_traffic_only_for_its_workload(bench):
    with open(bench.PMC_FILE) as f:
        rec = json.load(f)
    assert rec["workload_name"] == "share_n256k"
    assert bench.traffic_from_profile("stress_n1m") is None
    assert bench.traffic_from_profile("seq_n8k") is None
    got = bench.traffic_from_profile("share_n256k")
    # None once the kernel sources differ from the ones the counters were taken on
    assert got is None or got == rec["hbm_bytes_per_launch"]
