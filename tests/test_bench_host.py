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
    for name, (cfg_id, append, layers, desc, ctx) in bench.WORKLOADS.items():
        assert cfg_id in synth.CONFIGS and layers >= 8 and desc
        cfg = bench.workload_config(name)
        assert cfg.seq_len == (ctx or synth.CONFIGS[cfg_id].seq_len)
        # enough instances that a revisit is not served from the 256 MB last-level cache
        kv = cfg.batch * cfg.num_kv_heads * cfg.seq_len * 128 * 2 * 2
        assert layers * kv >= 4 * 256e6 or layers >= 16, name
    assert [w for w, v in bench.WORKLOADS.items() if v[1]] == [bench.DEFAULT_WORKLOAD]
    # the batch-1 context sweep: 16K, 32K, 64K, 128K
    sweep = sorted(bench.workload_config(w).seq_len for w in
                   ("llama-16k", "llama-32k", "llama-64k", "llama-128k"))
    assert sweep == [16384, 32768, 65536, 131072]


def test_layer_inputs_are_make_layers_draws():
    cfg = synth.CONFIGS[2].scaled(seq_len=200, n_plant=2)
    for layer in (0, 3):
        full = synth.make_layer(cfg, layer=layer)
        part = synth.layer_inputs(cfg, layer)
        for k in ("q", "R", "W"):
            assert (full[k] == part[k]).all(), (layer, k)
    a, b = synth.layer_inputs(cfg, 1), synth.layer_inputs(cfg, 2)
    assert not (a["q"] == b["q"]).all() and not (a["R"] == b["R"]).all()


def test_byte_model_128k():
    """Counts for the 128K layer (8192 pages, keep 512, k = 4096), written out by hand."""
    a = bench.algorithmic_bytes(synth.CONFIGS[3], [131072], append=True)
    # extrema: 8 KV heads x 8192 pages x 128 channels x (min + max) x 4 B; U: 32 x 8192 x 4 B
    assert a["page_bound"] == 8 * 8192 * 128 * 8 + 32 * 8192 * 4 + 32 * 128 * 4
    # per query head, one selection kernel: the U row, the query code, 512 pages x 16 codes of
    # 16 B read, 4096 indices written
    assert bench.unit_select("hhr", 512, 16)
    assert a["select"] == 32 * (8192 * 4 + 16 + 512 * 16 * 16 + 4096 * 4)
    # 4096 K + V rows of 256 B each, indices, q, 32 partials of 130 floats, per query head
    assert a["sparse_attn"] == 32 * (4096 * 512 + 4096 * 4 + 256 + 32 * 130 * 4)
    assert a["combine"] == 32 * (32 * 130 * 4 + 128 * 4)
    # R and W (1 MiB) dominate the preparation; the append adds 1.28 KiB per KV head
    assert a["prep"] - bench.algorithmic_bytes(synth.CONFIGS[3], [131072], False)["prep"] \
        == 8 * (512 + 512 + 16 + 2048)
    assert "select_emit" not in a


def test_byte_model_sums_over_sequences():
    cfg = synth.CONFIGS[4]
    one = [bench.algorithmic_bytes(cfg, [L], False, lmax=32768) for L in (8192, 20000)]
    both = bench.algorithmic_bytes(cfg, [8192, 20000], False, lmax=32768)
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
    assert pages["select"] == 32 * (8192 * 4 + 16 + 8192 * 4)
    assert pages["sparse_attn"] > 2 * base["sparse_attn"] - 32 * 4096 * 8
    # fine stage alone: no bound kernel; the sliced selection (8192 pages in 16 slices of 512
    # per query head) reads every token's code once and writes a distance byte per token, the
    # page ids and the histograms, which the emission reads back with the 4096 indices written
    assert "page_bound" not in codes
    assert not bench.unit_select("codes", 8192, 16)
    assert bench.select_slices(8192, 32, True) == 16
    inter = 131072 + 8192 * 4 + 16 * 129 * 4
    assert codes["select"] == 32 * (16 + 131072 * 16 + inter)
    assert codes["select_emit"] == 32 * (inter + 4096 * 4)
    assert codes["sparse_attn"] == base["sparse_attn"]
    dense = bench.algorithmic_bytes(cfg, [131072], False, "dense", 131072)
    # every K and V row once per KV head (512 MiB) dominates
    assert 8 * 131072 * 512 < dense["dense_attn"] < 1.01 * 8 * 131072 * 512
    assert set(bench.VARIANTS) == {"hhr", "identity-r", "pages", "codes", "dense",
                                   "bf16-extrema", "group-shared"}
    assert "prep" in codes and "prep" in base
    sh = bench.algorithmic_bytes(cfg, [131072], False, "group-shared")
    # one row set per KV head: a quarter of the K/V gather
    assert sh["sparse_attn"] < base["sparse_attn"] / 3
    half = bench.algorithmic_bytes(cfg, [131072], False, "bf16-extrema")
    assert half["page_bound"] == 8 * 8192 * 128 * 4 + 32 * 8192 * 4 + 32 * 128 * 4
    for v in bench.VARIANTS:
        alg = bench.algorithmic_bytes(cfg, [131072], False, v, 131072)
        unit = bench.unit_select(v, 8192 if v == "codes" else 512, 16)
        assert {n for n, _ in bench.timed_kernels(v, unit)} == set(alg), v


def test_hamming_scored_counts():
    cfg = synth.CONFIGS[3]
    # 128K: 32 query heads x 512 kept pages x 16 tokens
    assert bench.hamming_scored(cfg, [131072]) == 32 * 512 * 16
    # group-shared: 8 KV heads, each candidate against the group's 4 query codes
    assert bench.hamming_scored(cfg, [131072], "group-shared") == 8 * 4 * 512 * 16
    # fine stage alone: every token; coarse stage alone: none
    assert bench.hamming_scored(cfg, [131072], "codes") == 32 * 131072
    assert bench.hamming_scored(cfg, [131072], "pages") == 0
    # 40 tokens in 3 pages of 16, keep 1/4: one kept page of 16 tokens; with every page kept,
    # the partial last page holds only its 8 valid tokens
    assert bench.hamming_scored(synth.CONFIGS[1], [40]) == 16
    assert bench.hamming_scored(synth.CONFIGS[1], [40], "codes") == 40


def test_select_form_rule():
    # one workgroup per unit while the largest kept page set's tokens fit 32768 LDS slots
    assert bench.unit_select("hhr", 2048, 16) and not bench.unit_select("hhr", 2049, 16)
    assert bench.unit_select("pages", 1024, 32) and not bench.unit_select("codes", 4, 16)


def test_select_slice_rule():
    # about 256 workgroups with a page cut, 512 without; 8..512 kept pages per slice
    assert bench.select_slices(256, 32, False) == 8            # 32K, batch 1: 32 pages each
    assert bench.select_slices(512, 8, False) == 32            # 128K, group-shared
    assert bench.select_slices(615, 256, False) == 2           # 8 sequences: the 512-page cap
    assert bench.select_slices(4, 1, False) == 1               # tiny: at least 8 pages a slice
    assert bench.select_slices(16384, 1, True) == 512
    assert bench.select_slices(8192, 32, True) == 16           # 128K, fine stage alone


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
