"""The committed counter summaries bench.py reads agree with the forward's current sources.

bench.py reports roofline.traffic (measured HBM bytes per launch) from profiles/<kernel>__<workload>.txt
only while the hash recorded there matches the forward's device sources and build flags; after any change
to them the summaries must be taken again. This fails until they are, rather than letting the figure
silently turn null.
"""
import glob
import os

import bench

WORKLOADS = sorted(os.path.basename(p).split("__", 1)[1][:-4]
                   for p in glob.glob(os.path.join(bench.ROOT, "profiles", "fwd*__*.txt")))


def test_headline_workload_has_a_summary():
    assert "hvp" in WORKLOADS


def test_every_forward_summary_matches_the_sources():
    stale = [w for w in WORKLOADS if bench.measured_traffic(w) is None]
    assert not stale, f"counter summaries older than the forward's sources: {stale}"
