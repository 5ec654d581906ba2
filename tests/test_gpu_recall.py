"""The retrieval-quality harness (bench.py --recall) on the 32K layer: structural properties that
hold whatever the data (a diagnostic: the recall values themselves are not pinned)."""
import argparse
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

pytestmark = pytest.mark.gpu


def test_recall_harness_properties():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    rep = bench.recall_report(argparse.Namespace(workload="llama-32k"), quiet=True)
    rows = rep["rows"]
    assert rows
    for r in rows:
        assert 0.0 <= r["topk_recall"] <= r["topk_in_kept_pages"] <= 1.0
        if r["stages"] == "pages":      # every candidate is attended
            assert abs(r["topk_recall"] - r["topk_in_kept_pages"]) < 1e-9
        if r["stages"] == "codes":      # every page is a candidate
            assert r["topk_in_kept_pages"] == 1.0

    def series(stages, rot, nb, key, order):
        sel = [r for r in rows if r["stages"] == stages and r["rotation"] == rot
               and r["hash_bits"] == nb]
        return [r[key] for r in sorted(sel, key=lambda r: r[order] or 0)]

    # a larger budget selects a superset: recall never drops
    for rot, nb in (("random", 128), ("random", 256)):
        s = series("codes", rot, nb, "topk_recall", "token_budget")
        assert all(a <= b + 1e-12 for a, b in zip(s, s[1:])), s
        s = series("pages", rot, nb, "topk_in_kept_pages", "keep_ratio")
        assert all(a <= b + 1e-12 for a, b in zip(s, s[1:])), s
