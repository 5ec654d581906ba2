"""GPU parity at the workloads' full sizes, in the launch configuration the benchmark times
(MFMA index build, hhr_append_decode / hhr_decode with the workload's budgets). The oracle
checks sampled (sequence, head) pairs completely: key codes of their KV head, query code, bounds,
page set (swap rule), distances, selected indices and the attention output.
"""
import numpy as np
import pytest

from long_context_decode_gkr_amd import binding as hb
from long_context_decode_gkr_amd import synth

import hhr_case as hc

pytestmark = pytest.mark.gpu

MFMA_EXTREMA_SCALE = 20.0


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _check(lay, out, dbg, cfg, heads, kvs):
    ref = hc.oracle_index(lay, heads_kv=kvs)
    hc.check_index(lay, ref, pairs=kvs, extrema_atol_scale=MFMA_EXTREMA_SCALE)
    st = hc.check_decode(lay, out, dbg, cfg.keep_ratio, cfg.token_budget, heads=heads, ref_index=ref)
    print(f"cfg{cfg.cfg_id}: heads {len(heads)}, max out rel err {st['max_out_rel']:.2e}, "
          f"page swaps {st['swaps']}")


def test_fullsize_128k_append_decode():
    """128K context, 32q/8kv, keep 1/16, k = 4096: 16 appended tokens then a decode step."""
    torch = _torch()
    cfg = synth.CONFIGS[3]
    L0, n = 131072 - 16, 16
    lay = hc.GpuLayer(cfg, max_seq_len=131072, lens=[L0])
    lay.build()
    kn, vn = synth.append_tokens(cfg, n)
    dec = hb.Decoder(lay.dims, cfg.keep_ratio, cfg.token_budget)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    for i in range(n - 1):
        hb.append(lay.cache, hc.to_dev(kn[i], lay.tdt), hc.to_dev(vn[i], lay.tdt), lay.R, lay.W)
    dbg = hb.Debug(lay.dims, cfg.token_budget)
    dec(lay.cache, lay.q, lay.R, lay.W, out, dbg, k_new=hc.to_dev(kn[n - 1], lay.tdt),
        v_new=hc.to_dev(vn[n - 1], lay.tdt))
    torch.cuda.synchronize()
    d = lay.data
    d["K"][0, :, L0:L0 + n] = kn[:, 0].transpose(1, 0, 2)
    d["V"][0, :, L0:L0 + n] = vn[:, 0].transpose(1, 0, 2)
    d["seq_lens"][:] = L0 + n
    assert int(lay.cache.seq_lens[0]) == 131072
    heads = [(0, 0), (0, 13), (0, 31)]
    _check(lay, out, dbg, cfg, heads, [(0, 0), (0, 3), (0, 7)])


def test_fullsize_32k_all_heads():
    """32K context, 32q/8kv, keep 1/8, k = 2048: every head checked."""
    _torch()
    cfg = synth.CONFIGS[2]
    lay = hc.GpuLayer(cfg)
    lay.build()
    out, dbg = lay.decode(cfg.keep_ratio, cfg.token_budget)
    heads = [(0, h) for h in range(32)]
    _check(lay, out, dbg, cfg, heads, [(0, g) for g in range(8)])


@pytest.mark.parametrize("cfg_id,ctx", [(2, 16384), (3, 65536)])
def test_fullsize_context_sweep_points(cfg_id, ctx):
    """The batch-1 context sweep's other two points: 16K with the 32K layer's budgets (keep 1/8,
    k = 2048) and 64K with the 128K layer's (keep 1/16, k = 4096); sampled heads."""
    _torch()
    cfg = synth.CONFIGS[cfg_id].scaled(seq_len=ctx)
    lay = hc.GpuLayer(cfg)
    lay.build()
    out, dbg = lay.decode(cfg.keep_ratio, cfg.token_budget)
    heads = [(0, 0), (0, 6), (0, 17), (0, 31)]
    _check(lay, out, dbg, cfg, heads, sorted({(0, h // 4) for _, h in heads}))


def test_fullsize_varlen_batch():
    """8 sequences, lengths U[8K, 32K], keep 0.30, k = 2048."""
    _torch()
    cfg = synth.CONFIGS[4]
    lay = hc.GpuLayer(cfg)
    lay.build()
    out, dbg = lay.decode(cfg.keep_ratio, cfg.token_budget)
    heads = [(b, h) for b in (0, 3, 7) for h in (0, 21)]
    _check(lay, out, dbg, cfg, heads, sorted({(b, h // 4) for b, h in heads}))


def test_fullsize_qwen_64k_batch4():
    """Batch 4 x 64K, page 32, 256-bit codes, lognormal key scales, keep 1/8, k = 4096."""
    _torch()
    cfg = synth.CONFIGS[5]
    lay = hc.GpuLayer(cfg)
    lay.build()
    out, dbg = lay.decode(cfg.keep_ratio, cfg.token_budget)
    heads = [(0, 0), (3, 17), (2, 31)]
    _check(lay, out, dbg, cfg, heads, sorted({(b, h // 4) for b, h in heads}))


@pytest.mark.parametrize("stages", ["pages", "codes"])
def test_fullsize_128k_stage_variants(stages):
    """The stage-wise ablation variants at 128K (keep 1/16, k = 4096), sampled heads. The fine
    stage alone ranks all 131072 keys per head (more than the LDS distance cache holds: the
    selection recomputes distances while emitting)."""
    _torch()
    cfg = synth.CONFIGS[3]
    lay = hc.GpuLayer(cfg, max_seq_len=131072, lens=[131072 - 5])
    lay.build()
    out, dbg = lay.decode(cfg.keep_ratio, cfg.token_budget, stages=stages)
    heads = [(0, 2), (0, 30)]
    kvs = [(0, 0), (0, 7)]
    ref = hc.oracle_index(lay, heads_kv=kvs)
    hc.check_index(lay, ref, pairs=kvs, extrema_atol_scale=MFMA_EXTREMA_SCALE)
    st = hc.check_decode(lay, out, dbg, cfg.keep_ratio, cfg.token_budget, heads=heads,
                         ref_index=ref, stages=stages)
    print(f"{stages}: max out rel err {st['max_out_rel']:.2e}")


def test_fullsize_128k_dense_baseline():
    """Full attention over the 128K layer (the dense baseline), sampled heads against fp64."""
    torch = _torch()
    from oracle import hhr_oracle as orc
    cfg = synth.CONFIGS[3]
    lay = hc.GpuLayer(cfg, max_seq_len=131072, lens=[131072 - 3])
    dd = hb.DenseDecoder(lay.dims)
    out = torch.full((1, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    dd(lay.cache, lay.q, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    d = lay.data
    for h in (0, 11, 31):
        g = h // cfg.group
        ref = orc.dense_head(d["q"][0, h], d["K"][0, g], d["V"][0, g], 131072 - 3,
                             orc.default_scale(128))
        rel = np.abs(got[0, h] - ref).max() / np.abs(ref).max()
        assert rel <= hc.OUT_RTOL, (h, rel)
