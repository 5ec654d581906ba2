"""The retrieval-quality harness (bench.py --recall). On the 32K layer: structural properties that
hold whatever the data (the recall values themselves are a diagnostic). On a small layer: the
harness's rows from the GPU path's selections equal those from the oracle's, whose arithmetic is
pinned on the CPU (brute-force top-K, hand counts)."""
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


@pytest.mark.parametrize("stages,rho,k", [("both", 1 / 8, 128), ("pages", 1 / 8, 1),
                                          ("codes", 1.0, 128)])
def test_recall_rows_equal_the_oracles(stages, rho, k):
    """On a small ragged two-sequence layer (fp32 summary), the harness's row from the GPU path's
    selections equals the row from the oracle's selections, the decode being parity-checked
    first (its page sets may differ from the oracle's only by near-tie swaps; none is expected
    here, and the rows are compared only when there is none)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    import numpy as np
    from long_context_decode_gkr_amd import synth
    from oracle import hhr_oracle as orc
    from hhr_case import GpuLayer, check_decode, oracle_index
    lens = [2000, 1337]
    cfg = synth.CONFIGS[2].scaled(seq_len=2048, batch=2, lens=lens, n_plant=4)
    lay = GpuLayer(cfg, max_seq_len=2048, lens=lens)
    lay.build()
    print(f"recall rows: {stages} rho={rho} k={k} lens={lens}", flush=True)
    out, dbg = lay.decode(rho, k, stages=stages)
    idx = oracle_index(lay)
    stats = check_decode(lay, out, dbg, rho, k, ref_index=idx, stages=stages)
    assert stats["swaps"] == 0
    ref, planted = bench.recall_reference(lay.data, lens, cfg.group)
    sel_g, pages_g = bench.gpu_selections(dbg)
    sel_o, pages_o = {}, {}
    d, S, G = lay.data, cfg.page_size, cfg.group
    for (b, h) in ref:
        g = h // G
        r = orc.decode_head(d["q"][b, h], d["K"][b, g], d["V"][b, g], lens[b], idx["lo"][b, g],
                            idx["hi"][b, g], idx["codes"][b, g], d["R"][g], d["W"][g], S, rho, k,
                            orc.default_scale(128), stages=stages)
        sel_o[(b, h)] = set(int(t) for t in r["sel"])
        pages_o[(b, h)] = set(int(p) for p in r["pages"])
    assert sel_g == sel_o and pages_g == pages_o
    row_g = bench.recall_row(sel_g, pages_g, ref, planted, lens, S)
    row_o = bench.recall_row(sel_o, pages_o, ref, planted, lens, S)
    assert row_g == row_o
    assert 0.0 < row_g["topk_recall"] <= row_g["topk_in_kept_pages"] <= 1.0
    assert np.isclose(row_g["attended_frac"],
                      np.mean([len(sel_g[x]) / lens[x[0]] for x in ref]), atol=1e-4)
