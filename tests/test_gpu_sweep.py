"""Seeded sweep over the decode path's configuration space against the oracle.

Each case draws, from its own seed, one combination of the axes the fixed cases cover one at a
time: key/value dtype, key distribution, page size and code length (from the five workload
shapes), group size 1/2/4/8, batch and ragged lengths (tiny ones included), keep ratio, token
budget, stage variant, per-head or group-shared selection, fp32 or bf16 page extrema, and the
MFMA or fp64 index build. Every output is checked as in the fixed cases: codes, distances and
indices bit-exact, page sets up to the documented near-tie swaps, attention within 2e-3.
"""
import numpy as np
import pytest

from long_context_decode_gkr_amd import synth

import hhr_case as hc

N_CASES = 48


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def draw_case(seed: int) -> dict:
    """The seed's configuration: plain draws from a seeded generator, nothing computed."""
    r = np.random.default_rng(1000 + seed)
    cfg_id = int(r.integers(1, 6))
    base = synth.CONFIGS[cfg_id]
    G = int(r.choice([1, 2, 4, 8]))
    hkv = int(r.choice([1, 2]))
    batch = int(r.integers(1, 4))
    S = base.page_size
    cap = int(r.integers(8, 48)) * 4 * S                      # capacity, whole groups of 4 pages
    lens = [int(x) for x in r.integers(1, cap + 1, size=batch)]
    if batch > 1 and r.random() < 0.5:
        lens[int(r.integers(0, batch))] = int(r.choice([1, 2, S - 1, S, S + 1]))
    stages = str(r.choice(["both", "both", "both", "pages", "codes"]))
    return dict(cfg_id=cfg_id, G=G, hkv=hkv, batch=batch, cap=cap, lens=lens,
                rho=float(r.choice([0.03, 0.1, 0.25, 0.5, 1.0])),
                k=int(r.choice([1, 7, 64, 200, 513, 5000])),
                stages=stages, shared=bool(r.random() < 0.3),
                summary=str(r.choice(["f32", "bf16"])),
                method=str(r.choice(["auto", "auto", "fp64"])))


def test_cases_cover_every_axis():
    """The drawn cases reach every value of the categorical axes (a host check of the sweep)."""
    cases = [draw_case(i) for i in range(N_CASES)]
    assert {c["cfg_id"] for c in cases} == {1, 2, 3, 4, 5}
    assert {c["G"] for c in cases} == {1, 2, 4, 8}
    assert {c["stages"] for c in cases} == {"both", "pages", "codes"}
    assert {c["shared"] for c in cases} == {False, True}
    assert {c["summary"] for c in cases} == {"f32", "bf16"}
    assert {c["method"] for c in cases} == {"auto", "fp64"}


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration_matches_oracle(seed):
    _torch()
    c = draw_case(seed)
    print(f"seed {seed}: {c}", flush=True)
    base = synth.CONFIGS[c["cfg_id"]]
    cfg = base.scaled(seq_len=c["cap"], batch=c["batch"], lens=c["lens"],
                      num_q_heads=c["G"] * c["hkv"], num_kv_heads=c["hkv"], n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=c["cap"], summary=c["summary"])
    lay.build(method=c["method"])
    ref = hc.oracle_index(lay)
    out, dbg = lay.decode(c["rho"], c["k"], stages=c["stages"], group_shared=c["shared"])
    if c["shared"]:
        st = hc.check_decode_shared(lay, out, dbg, c["rho"], c["k"], ref_index=ref,
                                    stages=c["stages"])
    else:
        st = hc.check_decode(lay, out, dbg, c["rho"], c["k"], ref_index=ref, stages=c["stages"])
    print(f"seed {seed}: max out rel err {st['max_out_rel']:.2e}", flush=True)
