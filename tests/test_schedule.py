"""The resident forward grid's work lists (csrc/fa_schedule.h) on the CPU.

The schedule header is plain integer arithmetic compiled for the host as well.
tests/sched_check.hip enumerates every order the launcher can pick (one item
per workgroup; XCD-grouped head-major and block-major snakes; flat head-major
and block-major snakes), over grids, head counts and query-block counts, with
and without the balanced schedule's pool, and checks that every (head, query
block) item is computed exactly once, and that the balanced kernel's smaller
XCD-only list function deals the same lists.  The page's causal rule (aiml.sh "Speed up long contexts
with FlashAttention", lab.py tiled_flash_attention: the key loop stops at the
diagonal) makes items unequal; the cost model's makespans are checked against
the page's worked example (S = 64 in 16 x 16 blocks visits 10 tiles,
run-output.txt equivalence_check, flash_tiles_visited).
"""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_online_softmax_causal_amd", "csrc")
SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sched_check.hip")


@pytest.fixture(scope="module")
def sched_check(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("sched") / "sched_check")
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    res = subprocess.run([hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return exe


def test_every_item_exactly_once(sched_check):
    res = subprocess.run([sched_check], capture_output=True, text=True, timeout=300)
    print(res.stdout[-3000:])
    assert res.returncode == 0, res.stdout[-3000:]
    last = res.stdout.strip().splitlines()[-1].split()
    assert last[0] == "plans" and int(last[1]) > 1000 and last[-1] == "0"
    page = [l for l in res.stdout.splitlines() if l.startswith("page_tiles")][0]
    assert float(page.split()[1]) == 10.0
