"""The kernels' tile dealing, checked on the host: tests/tile_deal_check.cpp includes the same
csrc/tile_deal.h that the HIP kernels compile and replays, for every workgroup shape and for
block sizes 1..700 (plus the full-size shares), which tiles each wavefront fetches and computes.
Every fetch must start inside its block and every needed tile must be computed exactly once."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "tile_deal_check.cpp")


def _build(tmp_path, *defines):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / ("tdc" + "".join(d.replace("-D", "_") for d in defines))
    subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Werror", *defines,
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "striped_blockwise_amd", "csrc"),
                    SRC, "-o", str(exe)], check=True)
    return exe


def test_every_fetch_in_block_and_every_tile_once(tmp_path):
    exe = _build(tmp_path)
    out = subprocess.run([str(exe), "700"], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok "), out.stdout
    assert int(out.stdout.split()[1]) > 1_000_000


def test_check_rejects_the_former_unguarded_first_fetch(tmp_path):
    """Replaying the issue rule that once let a key split with no tile in a round fetch past the
    end of its block (non-causal, P = 64, c = 1) must fail the check."""
    exe = _build(tmp_path, "-DREPLAY_UNGUARDED_FIRST_ISSUE")
    out = subprocess.run([str(exe), "8"], capture_output=True, text=True, timeout=300)
    assert out.returncode != 0 and "past the block" in out.stdout, out.stdout
