"""Host-side checks of the benchmark script: argument contract and the byte model it reports."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from long_context_decode_gkr_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_workloads_name_existing_configs():
    assert bench.DEFAULT_WORKLOAD in bench.WORKLOADS
    for cfg_id, append, layers, desc in bench.WORKLOADS.values():
        assert cfg_id in synth.CONFIGS and layers >= 8 and desc
    assert [w for w, v in bench.WORKLOADS.items() if v[1]] == [bench.DEFAULT_WORKLOAD]


def test_byte_model_128k():
    """Counts for the 128K layer (8192 pages, keep 512, k = 4096), written out by hand."""
    a = bench.algorithmic_bytes(synth.CONFIGS[3], [131072], append=True)
    # extrema: 8 KV heads x 8192 pages x 128 channels x (min + max) x 4 B; U: 32 x 8192 x 4 B
    assert a["page_bound"] == 8 * 8192 * 128 * 8 + 32 * 8192 * 4 + 32 * 128 * 4
    # U row, query code, 512 pages x 16 codes of 16 B, 4096 indices, per query head
    assert a["select"] == 32 * (8192 * 4 + 16 + 512 * 16 * 16 + 4096 * 4)
    # 4096 K + V rows of 256 B each, indices, q, 32 partials of 130 floats, per query head
    assert a["sparse_attn"] == 32 * (4096 * 512 + 4096 * 4 + 256 + 32 * 130 * 4)
    assert a["combine"] == 32 * (32 * 130 * 4 + 128 * 4)
    # R and W (1 MiB) dominate the preparation; the append adds 1.28 KiB per KV head
    assert a["prep"] - bench.algorithmic_bytes(synth.CONFIGS[3], [131072], False)["prep"] \
        == 8 * (512 + 512 + 16 + 2048)


def test_byte_model_sums_over_sequences():
    cfg = synth.CONFIGS[4]
    one = [bench.algorithmic_bytes(cfg, [L], False) for L in (8192, 20000)]
    both = bench.algorithmic_bytes(cfg, [8192, 20000], False)
    for k in ("page_bound", "select", "sparse_attn", "combine"):
        assert both[k] == one[0][k] + one[1][k]
    # R and W are read once per KV head, not once per sequence
    assert both["prep"] < one[0]["prep"] + one[1]["prep"]


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_kernel_source_digest_is_stable(kernel):
    assert bench.kernel_source_digest(kernel) == bench.kernel_source_digest(kernel)
    assert len(bench.kernel_source_digest(kernel)) == 16


def test_byte_model_of_the_variants():
    cfg = synth.CONFIGS[3]
    base = bench.algorithmic_bytes(cfg, [131072], False, "hhr")
    pages = bench.algorithmic_bytes(cfg, [131072], False, "pages")
    codes = bench.algorithmic_bytes(cfg, [131072], False, "codes")
    # coarse stage alone: no codes read, all 512 x 16 candidates attended
    assert pages["select"] == 32 * (8192 * 4 + 8192 * 4)
    assert pages["sparse_attn"] > 2 * base["sparse_attn"] - 32 * 4096 * 8
    # fine stage alone: no bound kernel, every token's code read by the scan
    assert "page_bound" not in codes and "select" not in codes
    assert codes["hamming_scan"] == 32 * (16 + 131072 * 16 + 131072 + 32 * 129 * 4)
    assert codes["sparse_attn"] == base["sparse_attn"]
    dense = bench.algorithmic_bytes(cfg, [131072], False, "dense", 131072)
    # every K and V row once per KV head (512 MiB) dominates
    assert 8 * 131072 * 512 < dense["dense_attn"] < 1.01 * 8 * 131072 * 512
    assert set(bench.VARIANTS) == {"hhr", "identity-r", "pages", "codes", "dense",
                                   "bf16-extrema", "group-shared"}
    sh = bench.algorithmic_bytes(cfg, [131072], False, "group-shared")
    # one row set per KV head: a quarter of the K/V gather
    assert sh["sparse_attn"] < base["sparse_attn"] / 3
    half = bench.algorithmic_bytes(cfg, [131072], False, "bf16-extrema")
    assert half["page_bound"] == 8 * 8192 * 128 * 4 + 32 * 8192 * 4 + 32 * 128 * 4
    for v, ks in bench.VARIANTS.items():
        alg = bench.algorithmic_bytes(cfg, [131072], False, v, 131072)
        assert {n for n, _ in ks} == set(alg), v


def test_dense_split_rule():
    # 128K x 8 KV heads in sub-chunks of 128 tokens: 8 sub-chunks per workgroup, 128 splits
    assert bench.dense_splits(synth.CONFIGS[3], 131072) == 128
    assert bench.dense_splits(synth.CONFIGS[1], 4096) >= 1


@pytest.mark.skipif(not os.path.exists(os.path.join(ROOT, "long_context_decode_gkr_amd",
                                                    "libhhr.so")), reason="libhhr.so not built")
@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4, 5])
def test_dense_split_rule_matches_the_library(cfg_id):
    from long_context_decode_gkr_amd import binding as hb
    cfg = synth.CONFIGS[cfg_id]
    lmax = -(-cfg.seq_len // (4 * cfg.page_size)) * 4 * cfg.page_size
    dims = hb.make_dims(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.page_size,
                        cfg.hash_bits, lmax,
                        kv_dtype=hb.HHR_BF16 if cfg.dtype == "bf16" else hb.HHR_F32)
    assert hb.hhr_dense_workspace_bytes(dims) == \
        cfg.batch * cfg.num_q_heads * bench.dense_splits(cfg, lmax) * 130 * 4
