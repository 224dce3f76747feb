"""The committed counter summaries under profiles/ belong to the current
kernels: each records the sources it was taken from and their sha256, and
bench.py reports its traffic only while they match. A kernel source changed
without re-taking its summary fails here instead of turning the benchmark
line's traffic fields silently to null."""

import glob
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_pmc.txt")))


def test_every_traffic_summary_named_by_the_bench_exists():
    names = {os.path.basename(p) for p in SUMMARIES}
    for name in (bench.DECODE_PROFILE, bench.PREFILL_PROFILE, bench.VERIFY_PROFILE, bench.RAGGED_PROFILE,
                 bench.REUSE_PROFILE, bench.SWA_DECODE_PROFILE, bench.SWA_PREFILL_PROFILE):
        assert name in names, name


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_summary_matches_current_sources(path):
    assert bench.profile_traffic(os.path.basename(path)) is not None, (
        f"{os.path.basename(path)}: kernel sources changed since its counters were taken")
