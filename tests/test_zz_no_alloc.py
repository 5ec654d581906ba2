"""hhr_decode_scratch, the allocation-free decode (its workspace in the library's static device
scratch), against hhr_decode with a caller workspace: the same kernels, so identical outputs and
side outputs to the bit, on two calls in a row, the second on a smaller layer (the scratch then
holds the first call's leftovers, which the step must not depend on)."""
import numpy as np
import pytest

from long_context_decode_gkr_amd import binding as hb
from long_context_decode_gkr_amd import synth

import hhr_case as hc

pytestmark = pytest.mark.gpu


def _run_both(lay, rho, k, stages="both", group_shared=False):
    torch = hc.torch_mod()
    dec = hb.Decoder(lay.dims, rho, k, stages=stages, group_shared=group_shared)
    res = []
    for scratch in (False, True):
        out = torch.full((lay.cfg.batch, lay.cfg.num_q_heads, 128), float("nan"),
                         dtype=torch.float32, device="cuda")
        dbg = hb.Debug(lay.dims, k, rho, stages)
        if scratch:
            hb.hhr_decode_scratch(lay.dims, dec.params, lay.cache.struct(), lay.q.data_ptr(),
                                  lay.R.data_ptr(), lay.W.data_ptr(), out.data_ptr(),
                                  dbg.struct(), hb.current_stream())
        else:
            dec(lay.cache, lay.q, lay.R, lay.W, out, dbg)
        torch.cuda.synchronize()
        res.append((out, dbg))
    (o0, d0), (o1, d1) = res
    assert torch.equal(o0, o1)
    for name in ("q_rot", "q_code", "bounds", "page_ids", "page_count", "dist", "token_idx",
                 "token_count"):
        assert torch.equal(getattr(d0, name), getattr(d1, name)), name
    return o1, d1


def test_scratch_decode_equals_workspace_decode_twice_second_smaller():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = hc.GpuLayer(synth.CONFIGS[2].scaled(seq_len=9000, n_plant=8), max_seq_len=9088)
    big.build()
    o, d = _run_both(big, 0.125, 700)
    hc.check_decode(big, o, d, 0.125, 700)
    small = hc.GpuLayer(synth.CONFIGS[5].scaled(seq_len=2000, batch=2, lens=[2000, 777],
                                                 n_plant=4), max_seq_len=2048)
    small.build()
    o, d = _run_both(small, 0.25, 120)
    hc.check_decode(small, o, d, 0.25, 120)
