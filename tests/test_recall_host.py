"""The recall harness's arithmetic (bench.recall_reference, bench.recall_row) pinned on the CPU:
the exact top-K against a pairwise-count definition, the row against hand counts, and the rows
of the oracle's own selections against the properties each stage variant fixes."""
import os
import sys
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_decode_gkr_amd import synth  # noqa: E402
from oracle import hhr_oracle as orc  # noqa: E402

LENS = [300, 171]


@pytest.fixture(scope="module")
def layer():
    cfg = synth.CONFIGS[2].scaled(seq_len=320, batch=2, lens=LENS, n_plant=3)
    return cfg, synth.make_layer(cfg, max_seq_len=320, lens=LENS)


def test_reference_is_the_pairwise_top_k(layer):
    """Token t is in the top-K iff fewer than K tokens beat it (a larger q.k, or an equal one at
    a lower position): counted pair by pair in exact rational arithmetic of the fp32 inputs."""
    cfg, data = layer
    ref, planted = bench.recall_reference(data, LENS, cfg.group)
    assert len(ref) == cfg.batch * cfg.num_q_heads
    for (b, h) in [(0, 0), (0, 13), (1, 31)]:
        L = LENS[b]
        kref = max(1, round(0.015 * L))
        q = [Fraction(float(x)) for x in data["q"][b, h]]
        K = data["K"][b, h // cfg.group]
        s = [sum(qi * Fraction(float(ki)) for qi, ki in zip(q, K[t])) for t in range(L)]
        top = {t for t in range(L)
               if sum(1 for u in range(L) if s[u] > s[t] or (s[u] == s[t] and u < t)) < kref}
        assert ref[(b, h)] == top, (b, h)
        assert planted[(b, h)] == {int(p) for p in data["planted"][b, h] if p >= 0}


def test_row_by_hand():
    """Two heads, page size 2: every share counted by hand."""
    ref = {(0, 0): {1, 2, 3, 4}, (0, 1): {0, 5}}
    planted = {(0, 0): {2}, (0, 1): set()}
    sel = {(0, 0): {1, 2, 9}, (0, 1): {0, 4, 5, 6}}
    pages = {(0, 0): {0, 4}, (0, 1): {0, 2, 3}}
    row = bench.recall_row(sel, pages, ref, planted, [10], 2)
    # head 0: {1,2} of 4 selected; {1} of 4 in pages 0 (tokens 0,1) and 4 (8,9); planted 1 of 1;
    # 3 of 10 attended. head 1: {0,5} of 2; both in pages 0 and 2; no planted key; 4 of 10
    assert row == {"attended_frac": 0.35, "topk_recall": 0.75, "topk_in_kept_pages": 0.625,
                   "planted_recall": 1.0}
    assert bench.recall_row(sel, pages, ref, {k: set() for k in ref}, [10], 2)[
        "planted_recall"] is None


def test_rows_of_the_oracles_selections(layer):
    """recall_row on the oracle's selections: each share recounted token by token, and the
    relations each stage variant fixes (the coarse stage alone attends to every candidate, the
    fine stage alone keeps every page, a budget and ratio covering the context attend to all)."""
    cfg, data = layer
    S, G = cfg.page_size, cfg.group
    ref, planted = bench.recall_reference(data, LENS, G)
    index = {}
    for b in range(cfg.batch):
        for g in range(cfg.num_kv_heads):
            index[(b, g)] = orc.build_head(data["K"][b, g], LENS[b], data["R"][g], data["W"][g],
                                           S)
    scale = orc.default_scale(cfg.head_dim)
    rows = {}
    for stages, rho, k in (("both", 1 / 8, 16), ("both", 0.5, 64), ("pages", 1 / 4, 1),
                           ("codes", 1.0, 32), ("both", 1.0, 512)):
        sel, pages = {}, {}
        for (b, h) in ref:
            g, L = h // G, LENS[b]
            lo, hi, kc = index[(b, g)]
            r = orc.decode_head(data["q"][b, h], data["K"][b, g], data["V"][b, g], L, lo, hi,
                                kc, data["R"][g], data["W"][g], S, rho, k, scale, stages=stages)
            sel[(b, h)] = set(int(t) for t in r["sel"])
            pages[(b, h)] = set(int(p) for p in r["pages"])
        row = bench.recall_row(sel, pages, ref, planted, LENS, S)
        # recount
        n = len(ref)
        hand_rec = sum(sum(1 for t in ref[x] if t in sel[x]) / len(ref[x]) for x in ref) / n
        hand_in = sum(sum(1 for t in ref[x] if (t // S) in pages[x]) / len(ref[x])
                      for x in ref) / n
        hand_att = sum(len(sel[x]) / LENS[x[0]] for x in ref) / n
        assert row["topk_recall"] == round(hand_rec, 4)
        assert row["topk_in_kept_pages"] == round(hand_in, 4)
        assert row["attended_frac"] == round(hand_att, 4)
        assert 0.0 <= row["topk_recall"] <= row["topk_in_kept_pages"] <= 1.0
        if stages == "pages":
            assert row["topk_recall"] == row["topk_in_kept_pages"]
        if stages == "codes" or rho == 1.0:
            assert row["topk_in_kept_pages"] == 1.0
        rows[(stages, rho, k)] = row
    assert rows[("both", 1.0, 512)] == {"attended_frac": 1.0, "topk_recall": 1.0,
                                        "topk_in_kept_pages": 1.0, "planted_recall": 1.0}
    # a larger ratio and budget select a superset of the candidates
    assert rows[("both", 0.5, 64)]["topk_in_kept_pages"] >= rows[("both", 1 / 8, 16)][
        "topk_in_kept_pages"]
