"""HHR_TRACE: with the variable set, the library logs each decode step's plan and byte counts
and every launch (kernel, grid, block, stream, status) to stderr. Checked in a child process:
the setting is read once per process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, %r)
import torch
from long_context_decode_gkr_amd import binding as hb
from long_context_decode_gkr_amd import synth
import hhr_case as hc
cfg = synth.CONFIGS[2].scaled(seq_len=3000, n_plant=4)
lay = hc.GpuLayer(cfg, max_seq_len=3072)
lay.build()
out, dbg = lay.decode(0.125, 256, debug=False)
print("done", flush=True)
"""


def test_trace_logs_plan_and_every_launch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, HHR_TRACE="1", PYTHONPATH=os.path.join(ROOT, "tests"))
    r = subprocess.run([sys.executable, "-c", SCRIPT % ROOT], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[hhr] ")]
    launches = [ln for ln in lines if ln.startswith("[hhr] launch ")]
    names = [ln.split()[2] for ln in launches]
    # the index build, then the step's kernels in order
    assert names[0] == "build_mfma_kernel"
    assert names[1:] == ["prep_kernel", "page_bound_kernel", "select_unit_kernel",
                         "attn_kernel", "combine_kernel"], names
    assert all(ln.endswith(": no error") for ln in launches), launches
    plan = [ln for ln in lines if ln.startswith("[hhr] decode ")]
    assert len(plan) == 1 and "selection one workgroup per unit" in plan[0], plan
    assert any(ln.startswith("[hhr] bytes at most: ") for ln in lines)
    # without the variable nothing is logged
    env.pop("HHR_TRACE")
    r = subprocess.run([sys.executable, "-c", SCRIPT % ROOT], capture_output=True, text=True,
                       timeout=300, env=env)
    assert r.returncode == 0 and "[hhr]" not in r.stderr
