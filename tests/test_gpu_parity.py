"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on seeded inputs.

Sizes span several kernel tiles and a ragged tail while the oracle still finishes in seconds;
the full-size workloads are checked on sampled heads in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

from long_context_decode_gkr_amd import binding as hb
from long_context_decode_gkr_amd import synth
from oracle import hhr_oracle as orc

import hhr_case as hc

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _cfg(i, L, **kw):
    return synth.CONFIGS[i].scaled(seq_len=L, **kw)


# ---------------------------------------------------------------------------------------------
# Index build (fp64 vector path): codes bit-exact, extrema within a few ulps
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg_id,L,batch", [(1, 4096, None), (1, 1000, None), (2, 3001, None),
                                            (5, 2085, 2)])
def test_build_fp64_matches_oracle(cfg_id, L, batch):
    _torch()
    cfg = _cfg(cfg_id, L, batch=batch, n_plant=8)
    lay = hc.GpuLayer(cfg, max_seq_len=L + 4 * cfg.page_size * 2)
    lay.build(method="fp64")
    hc.check_index(lay, hc.oracle_index(lay))


# ---------------------------------------------------------------------------------------------
# Decode step per workload shape (scaled-down contexts)
# ---------------------------------------------------------------------------------------------
DECODE_CASES = [
    # cfg, L, batch, lens, rho, k
    (1, 4096, None, None, 0.25, 256),        # workload 1 at full size
    (1, 1111, None, None, 0.25, 100),        # ragged tail, G = 1, fp32
    (2, 5003, None, None, 1 / 8, 300),       # Llama shape, bf16, ragged
    (3, 8192, None, None, 1 / 16, 256),      # 128K-workload budgets at 8K
    (4, 6000, 3, [5000, 6000, 2001], 0.30, 200),   # varlen batch
    (5, 4096, 2, None, 1 / 8, 257),          # page 32, 256-bit codes, lognormal keys
]


@pytest.mark.parametrize("cfg_id,L,batch,lens,rho,k", DECODE_CASES)
def test_decode_matches_oracle(cfg_id, L, batch, lens, rho, k):
    _torch()
    cfg = _cfg(cfg_id, L, batch=batch, lens=lens, n_plant=16)
    lay = hc.GpuLayer(cfg, max_seq_len=L + 64)
    lay.build(method="fp64")
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref)
    out, dbg = lay.decode(rho, k)
    st = hc.check_decode(lay, out, dbg, rho, k, ref_index=ref)
    print(f"cfg{cfg_id} L={L}: max out rel err {st['max_out_rel']:.2e}, page swaps {st['swaps']}")


def test_decode_full_budget_is_dense_attention():
    torch = _torch()
    cfg = _cfg(2, 777, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=1024)
    lay.build(method="fp64")
    out, dbg = lay.decode(1.0, 777)
    assert np.all(dbg.token_count.cpu().numpy() == 777)
    d = lay.data
    for h in (0, 13, 31):
        g = h // cfg.group
        qt = torch.tensor(d["q"][0, h], dtype=torch.float64)[None, None, None]
        kt = torch.tensor(d["K"][0, g, :777], dtype=torch.float64)[None, None]
        vt = torch.tensor(d["V"][0, g, :777], dtype=torch.float64)[None, None]
        dense = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=orc.default_scale(128))[0, 0, 0].numpy()
        rel = np.abs(out[0, h].cpu().numpy() - dense).max() / np.abs(dense).max()
        assert rel <= hc.OUT_RTOL


@pytest.mark.parametrize("k", [1, 5000])
def test_decode_budget_extremes(k):
    _torch()
    cfg = _cfg(2, 2048 + 7, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=2048 + 64)
    lay.build(method="fp64")
    out, dbg = lay.decode(0.2, k)
    hc.check_decode(lay, out, dbg, 0.2, k)


def test_decode_short_and_empty_sequences():
    _torch()
    cfg = _cfg(4, 64, batch=4, lens=[0, 1, 15, 17], n_plant=0)
    lay = hc.GpuLayer(cfg, max_seq_len=64)
    lay.build(method="fp64")
    out, dbg = lay.decode(0.3, 8)
    hc.check_decode(lay, out, dbg, 0.3, 8)
    assert np.all(out[0].cpu().numpy() == 0.0)


def test_decode_many_candidates_recompute_path():
    # more than 32768 candidate slots: distances are recomputed instead of cached in LDS
    _torch()
    cfg = _cfg(1, 40000, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=40064)
    lay.build(method="fp64")
    heads = [(0, 0)]
    out, dbg = lay.decode(1.0, 3000)
    hc.check_decode(lay, out, dbg, 1.0, 3000, heads=heads)


def test_kernel_events_time_the_six_kernels():
    """The optional start/stop events (12) are recorded around each of the step's six kernel
    slots (preparation, page bound, selection, second selection kernel, attention, merge), in
    launch order: here the selection is one kernel, so slot 3 gets its two events back to back.
    Timing does not change the result."""
    torch = _torch()
    cfg = _cfg(3, 4096 + 5, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=4096 + 64)
    lay.build()
    dec = hb.Decoder(lay.dims, 1 / 16, 256)
    outs = []
    ev = hb.HipEvents(12)
    try:
        for timed in (False, True):
            out = torch.full((1, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
            dbg = (hb.DebugStruct(None, None, None, None, None, None, None, None, ev.address(0))
                   if timed else None)
            hb.hhr_decode(lay.dims, dec.params, lay.cache.struct(), lay.q.data_ptr(),
                          lay.R.data_ptr(), lay.W.data_ptr(), dec.ws.data_ptr(), dec.ws_bytes,
                          out.data_ptr(), dbg, hb.current_stream())
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        ms = [ev.elapsed_ms(2 * j, 2 * j + 1) for j in range(6)]
        gaps = [ev.elapsed_ms(2 * j + 1, 2 * j + 2) for j in range(5)]
    finally:
        ev.close()
    assert np.array_equal(outs[0], outs[1])
    assert all(0.0 <= m < 50.0 for m in ms), ms
    assert all(ms[j] > 0.0 for j in (0, 1, 2, 4, 5)), ms
    assert all(g > -0.005 for g in gaps), gaps  # launch order


def test_decode_ties_all_bounds_equal():
    # identical keys: every page bound and every distance ties; lower indices must win
    torch = _torch()
    cfg = _cfg(2, 1024, n_plant=0)
    data = synth.make_layer(cfg)
    data["K"][:, :, :1024] = data["K"][:, :, :1][:, :, :1]
    lay = hc.GpuLayer(cfg, data=data)
    lay.build(method="fp64")
    out, dbg = lay.decode(0.25, 50)
    hc.check_decode(lay, out, dbg, 0.25, 50)
    pid = dbg.page_ids.cpu().numpy()[0, 0, :16]
    assert pid.tolist() == list(range(16))
    assert dbg.token_idx.cpu().numpy()[0, 0].tolist() == list(range(50))
    del torch


@pytest.mark.parametrize("mode", ["cluster", "equal"])
def test_decode_clustered_bounds(mode):
    """Page extrema written directly (lo = hi = c_p v), so U_p = c_p (q~ . v): a clear top group,
    then a cluster that straddles the n_keep cut. "cluster": 300 pages within 2e-6 of each
    other (several radix passes, then one wave ranks the threshold bin); "equal": 200 pages
    with exactly equal bounds (ties broken in page order by the scan)."""
    torch = _torch()
    cfg = _cfg(2, 16384, n_plant=0)
    lay = hc.GpuLayer(cfg, max_seq_len=16384)
    lay.build(method="fp64")
    ref = hc.oracle_index(lay)
    P, Hkv = 1024, cfg.num_kv_heads
    rng = np.random.default_rng(11)
    v = rng.choice([-1.0, 1.0], size=128).astype(np.float32)
    c = rng.uniform(0.0, 1.5, size=P)
    top = rng.choice(P, size=400, replace=False)
    c[top[:100]] = rng.uniform(2.5, 3.0, size=100)
    if mode == "cluster":
        c[top[100:]] = 2.0 * (1.0 + rng.uniform(0.0, 2e-6, size=300))
    else:
        c[top[100:300]] = 2.0
    ext = (c[:, None] * v[None, :]).astype(np.float32)          # [P][128]
    lo = np.broadcast_to(ext, (1, Hkv, P, 128)).copy()
    ref["lo"], ref["hi"] = lo, lo.copy()
    ref["lo32"], ref["hi32"] = ref["lo"], ref["hi"]
    dev = torch.from_numpy(lo).permute(0, 1, 3, 2).contiguous().cuda()
    lay.cache.page_min.copy_(dev)
    lay.cache.page_max.copy_(dev)
    out, dbg = lay.decode(1 / 8, 400)
    st = hc.check_decode(lay, out, dbg, 1 / 8, 400, ref_index=ref)
    print(f"{mode}: page swaps vs the oracle {st['swaps']}")


def test_decode_is_deterministic():
    torch = _torch()
    cfg = _cfg(2, 6000, n_plant=16)
    lay = hc.GpuLayer(cfg, max_seq_len=6016)
    lay.build(method="fp64")
    o1, d1 = lay.decode(0.125, 512)
    o2, d2 = lay.decode(0.125, 512)
    assert torch.equal(o1, o2)
    assert torch.equal(d1.token_idx, d2.token_idx) and torch.equal(d1.bounds, d2.bounds)


SELECT_FORM_CASES = [
    # cfg, L, batch, lens, rho, k, stages, group_shared, summary
    (2, 9000, None, None, 0.125, 700, "both", False, "f32"),
    (3, 20000, None, None, 1 / 16, 1024, "both", False, "f32"),
    (5, 4200, 2, [4200, 1777], 0.3, 600, "both", False, "f32"),      # page 32, 256-bit codes
    (2, 7000, None, None, 0.2, 900, "both", True, "f32"),
    (4, 6000, 3, [6000, 1, 2500], 0.3, 400, "pages", False, "f32"),
    (2, 5000, None, None, 0.125, 300, "both", False, "bf16"),
]


@pytest.mark.parametrize("cfg_id,L,batch,lens,rho,k,stages,group_shared,summary",
                         SELECT_FORM_CASES)
def test_selection_forms_agree_bit_for_bit(cfg_id, L, batch, lens, rho, k, stages,
                                           group_shared, summary, monkeypatch):
    """The two forms of the selection (one workgroup per unit, of 256, 512 or 1024 threads; the
    sliced pair of a 1024-thread scan and a 256-thread emission, at several slice counts)
    decompose the same work differently over workgroups, LDS and barriers: their kept pages,
    distances, selected tokens and outputs must be identical to the bit (a check for races in
    the LDS staging)."""
    torch = _torch()
    kw = dict(n_plant=8) if batch is None else dict(batch=batch, n_plant=8)
    cfg = _cfg(cfg_id, L, **kw)
    lay = hc.GpuLayer(cfg, max_seq_len=-(-L // 128) * 128, lens=lens, summary=summary)
    lay.build()
    runs = []
    for form, nsl in (("unit", None), ("unit256", None), ("unit512", None), ("unit1024", None),
                      ("sliced", None), ("sliced", 1), ("sliced", 3), ("sliced", 7)):
        for var in ("HHR_SELECT", "HHR_SELECT_SLICES", "HHR_SELECT_THREADS"):
            monkeypatch.delenv(var, raising=False)
        if form == "sliced":
            monkeypatch.setenv("HHR_SELECT", "sliced")
        if form in ("unit256", "unit512", "unit1024"):
            monkeypatch.setenv("HHR_SELECT_THREADS", form[4:])
        if nsl is not None:
            monkeypatch.setenv("HHR_SELECT_SLICES", str(nsl))
        out, dbg = lay.decode(rho, k, stages=stages, group_shared=group_shared)
        runs.append((form, nsl, out, dbg))
    _, _, out0, d0 = runs[0]
    for form, nsl, out, dbg in runs[1:]:
        for name in ("page_ids", "page_count", "dist", "token_idx", "token_count"):
            assert torch.equal(getattr(d0, name), getattr(dbg, name)), (form, nsl, name)
        assert torch.equal(out0, out), (form, nsl)
    # and the first run against the oracle
    if group_shared:
        hc.check_decode_shared(lay, out0, d0, rho, k, stages=stages)
    else:
        hc.check_decode(lay, out0, d0, rho, k, stages=stages)


BOUND_PAGE_CASES = [
    # cfg, L, batch, lens, rho, k, group_shared, summary
    (2, 9000, None, None, 0.125, 700, False, "f32"),
    (5, 4200, 2, [4200, 1777], 0.3, 600, False, "f32"),               # page 32, 256-bit codes
    (4, 6000, 3, [6000, 1, 2500], 0.3, 400, False, "f32"),            # ragged, one-token sequence
    (2, 7000, None, None, 0.2, 900, True, "f32"),
    (2, 5000, None, None, 0.125, 300, False, "bf16"),
]


@pytest.mark.parametrize("cfg_id,L,batch,lens,rho,k,group_shared,summary", BOUND_PAGE_CASES)
def test_bound_workgroup_sizes_agree_bit_for_bit(cfg_id, L, batch, lens, rho, k, group_shared,
                                                 summary, monkeypatch):
    """The page-bound kernel covers 64, 128 or 256 pages per workgroup (1, 2 or 4 per lane, the
    largest that still fills the chip unless HHR_BOUND_PAGES forces one): every choice runs the
    same sequence of operations per page, so bounds, kept pages, selected tokens and outputs
    must be identical to the bit (also a check of the partial-workgroup and early-exit paths,
    with lengths that end inside a workgroup's range)."""
    torch = _torch()
    kw = dict(n_plant=8) if batch is None else dict(batch=batch, n_plant=8)
    cfg = _cfg(cfg_id, L, **kw)
    lay = hc.GpuLayer(cfg, max_seq_len=-(-L // 128) * 128, lens=lens, summary=summary)
    lay.build()
    runs = []
    for pages in (None, "64", "128", "256"):
        monkeypatch.delenv("HHR_BOUND_PAGES", raising=False)
        if pages is not None:
            monkeypatch.setenv("HHR_BOUND_PAGES", pages)
        out, dbg = lay.decode(rho, k, group_shared=group_shared)
        runs.append((pages, out, dbg))
    _, out0, d0 = runs[0]
    for pages, out, dbg in runs[1:]:
        for name in ("bounds", "page_ids", "page_count", "token_idx", "token_count"):
            assert torch.equal(getattr(d0, name), getattr(dbg, name)), (pages, name)
        assert torch.equal(out0, out), pages
    if group_shared:
        hc.check_decode_shared(lay, out0, d0, rho, k)
    else:
        hc.check_decode(lay, out0, d0, rho, k)


@pytest.mark.parametrize("stages,group_shared", [("both", False), ("codes", False),
                                                 ("both", True)])
def test_decode_on_a_side_stream_and_in_a_replayed_graph(stages, group_shared):
    """The step enqueues everything on the stream it is given: the same output on a side
    stream, and from a captured HIP graph replayed several times with eager decodes and
    synchronisations in between (the library records no memset and allocates nothing)."""
    torch = _torch()
    cfg = _cfg(2, 3001, n_plant=8)
    lay = hc.GpuLayer(cfg, max_seq_len=3072)
    lay.build()
    dec = hb.Decoder(lay.dims, 1 / 8, 300, stages=stages, group_shared=group_shared)
    shape = (1, cfg.num_q_heads, 128)
    ref = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    dec(lay.cache, lay.q, lay.R, lay.W, ref)
    torch.cuda.synchronize()
    assert not torch.isnan(ref).any()
    side = torch.cuda.Stream()
    out_s = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        dec(lay.cache, lay.q, lay.R, lay.W, out_s, stream=side.cuda_stream)
    side.synchronize()
    assert torch.equal(out_s, ref)
    graph, gstream = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    out_g = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=gstream):
        dec(lay.cache, lay.q, lay.R, lay.W, out_g, stream=gstream.cuda_stream)
    for _ in range(4):
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref)
        eager = torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
        dec(lay.cache, lay.q, lay.R, lay.W, eager)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref)


def test_concurrent_decodes_on_two_streams():
    """Two layers (their own caches and workspaces) decoded at once on two streams, each step
    enqueued back to back several times: every output equals its layer's eager result."""
    torch = _torch()
    lays, decs, refs = [], [], []
    for layer, (cfg_id, L) in enumerate([(2, 3001), (3, 2500)]):
        cfg = _cfg(cfg_id, L, n_plant=8)
        lay = hc.GpuLayer(cfg, max_seq_len=3072, layer=layer)
        lay.build()
        dec = hb.Decoder(lay.dims, cfg.keep_ratio, 257)
        ref = torch.full((1, cfg.num_q_heads, 128), float("nan"), dtype=torch.float32,
                         device="cuda")
        dec(lay.cache, lay.q, lay.R, lay.W, ref)
        lays.append(lay), decs.append(dec), refs.append(ref)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.full_like(refs[i], float("nan")) for _ in range(3)] for i in range(2)]
    for r in range(3):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                decs[i](lays[i].cache, lays[i].q, lays[i].R, lays[i].W, outs[i][r],
                        stream=streams[i].cuda_stream)
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(3):
            assert torch.equal(outs[i][r], refs[i]), (i, r)


# ---------------------------------------------------------------------------------------------
# Append: one token per step; equals a rebuild; decode sees the new token
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("cfg_id", [1, 3, 5])
def test_append_matches_oracle_and_rebuild(cfg_id):
    torch = _torch()
    base = synth.CONFIGS[cfg_id]
    S = base.page_size
    L0, n = 3 * S - 5, 2 * S + 9          # crosses two page boundaries
    cfg = base.scaled(seq_len=L0, batch=min(base.batch, 2), n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=L0 + n + 4 * S)
    lay.build(method="fp64")
    kn, vn = synth.append_tokens(cfg, n)
    for i in range(n):
        hb.append(lay.cache, hc.to_dev(kn[i], lay.tdt), hc.to_dev(vn[i], lay.tdt), lay.R, lay.W)
    torch.cuda.synchronize()
    lens = lay.cache.seq_lens.cpu().numpy()
    assert np.all(lens == L0 + n)
    # oracle: the same appends on the host
    d = lay.data
    for b in range(cfg.batch):
        d["K"][b, :, L0:L0 + n] = kn[:, b].transpose(1, 0, 2)
        d["V"][b, :, L0:L0 + n] = vn[:, b].transpose(1, 0, 2)
    d["seq_lens"][:] = L0 + n
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref)
    np.testing.assert_array_equal(lay.cache.K.float().cpu().numpy(), d["K"])
    np.testing.assert_array_equal(lay.cache.V.float().cpu().numpy(), d["V"])
    assert np.all(lay.cache.append_ticket.cpu().numpy() == 0)
    out, dbg = lay.decode(cfg.keep_ratio, 40)
    hc.check_decode(lay, out, dbg, cfg.keep_ratio, 40, ref_index=ref)


def test_append_at_capacity_is_a_no_op():
    torch = _torch()
    cfg = _cfg(2, 64, n_plant=0)
    lay = hc.GpuLayer(cfg, max_seq_len=64)
    lay.build(method="fp64")
    before = lay.cache.codes.clone()
    kn, vn = synth.append_tokens(cfg, 1)
    hb.append(lay.cache, hc.to_dev(kn[0], lay.tdt), hc.to_dev(vn[0], lay.tdt), lay.R, lay.W)
    torch.cuda.synchronize()
    assert int(lay.cache.seq_lens[0]) == 64
    assert torch.equal(before, lay.cache.codes)


def test_append_decode_equals_append_then_decode():
    torch = _torch()
    cfg = _cfg(3, 4000, n_plant=8)
    a = hc.GpuLayer(cfg, max_seq_len=4096)
    a.build(method="fp64")
    b = hc.GpuLayer(cfg, data={k: (v.copy() if hasattr(v, "copy") else v) for k, v in a.data.items()})
    b.build(method="fp64")
    kn, vn = synth.append_tokens(cfg, 3)
    dec_a = hb.Decoder(a.dims, 1 / 16, 300)
    dec_b = hb.Decoder(b.dims, 1 / 16, 300)
    for i in range(3):
        k_i, v_i = hc.to_dev(kn[i], a.tdt), hc.to_dev(vn[i], a.tdt)
        oa = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
        ob = torch.empty_like(oa)
        da, db = hb.Debug(a.dims, 300), hb.Debug(b.dims, 300)
        hb.append(a.cache, k_i, v_i, a.R, a.W)
        dec_a(a.cache, a.q, a.R, a.W, oa, da)
        dec_b(b.cache, b.q, b.R, b.W, ob, db, k_new=k_i, v_new=v_i)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob)
        assert torch.equal(da.token_idx, db.token_idx) and torch.equal(da.q_code, db.q_code)
    for name in ("K", "V", "page_min", "page_max", "codes", "seq_lens", "append_ticket"):
        assert torch.equal(getattr(a.cache, name), getattr(b.cache, name)), name
    assert int(b.cache.seq_lens[0]) == 4003


# ---------------------------------------------------------------------------------------------
# Index build on the matrix cores (bf16 keys): codes bit-exact; page extrema carry fp32
# accumulation error of a 128-term dot product (tolerance 8e-6 |k|_2, ~20 fp32 ulps of |k|)
# ---------------------------------------------------------------------------------------------
MFMA_EXTREMA_SCALE = 20.0


@pytest.mark.parametrize("cfg_id,L,batch,lens", [(2, 5003, None, None), (3, 1500, None, None),
                                                 (4, 3000, 3, [3000, 1, 2049]),
                                                 (5, 2085, 2, None)])
def test_build_mfma_matches_oracle(cfg_id, L, batch, lens):
    _torch()
    cfg = _cfg(cfg_id, L, batch=batch, lens=lens, n_plant=8)
    lay = hc.GpuLayer(cfg, max_seq_len=L + 4 * cfg.page_size * 2)
    lay.build(method="auto")
    hc.check_index(lay, hc.oracle_index(lay), extrema_atol_scale=MFMA_EXTREMA_SCALE)


def test_build_mfma_balanced_chunk_list_across_sequence_groups():
    """70 sequences of ragged lengths (empty, one token, chunk and tile boundaries, the full
    capacity) in two groups of at most 64: each KV head's workgroups share out the group's
    list of 512-token chunks, so one workgroup builds chunks of several sequences in turn and
    its queued uncertain bits carry their own rows. Codes bit-exact and extrema admissible
    against the oracle on sampled (sequence, KV head) pairs of both groups; codes equal to the
    fp64 builder's on every pair."""
    _torch()
    r = np.random.default_rng(7)
    lens = [int(x) for x in r.integers(0, 1281, size=70)]
    lens[:6] = [0, 1, 512, 513, 1280, 127]
    lens[64:68] = [0, 1280, 640, 1]
    cfg = _cfg(3, 1280, batch=70, lens=lens, n_plant=0, num_q_heads=4, num_kv_heads=2)
    lay = hc.GpuLayer(cfg, max_seq_len=1280)
    lay.build(method="fp64")
    codes64 = lay.cache.codes.cpu().numpy().view(np.uint32).copy()
    lay.cache.codes.zero_()
    lay.cache.page_min.zero_()
    lay.cache.page_max.zero_()
    lay.build(method="auto")
    got = lay.cache.codes.cpu().numpy().view(np.uint32)
    for b, L in enumerate(lens):
        np.testing.assert_array_equal(got[b, :, :L], codes64[b, :, :L], err_msg=f"b={b}")
    pairs = [(b, g) for b in (1, 2, 3, 4, 5, 17, 63, 65, 66, 69) for g in (0, 1)]
    hc.check_index(lay, hc.oracle_index(lay, heads_kv=pairs), pairs=pairs,
                   extrema_atol_scale=MFMA_EXTREMA_SCALE)


@pytest.mark.parametrize("cfg_id,col0,nzero,ntiny", [(3, 0, 16, 8), (3, 0, 1, 0), (3, 0, 0, 1),
                                                    (5, 128, 16, 8), (5, 128, 1, 0)])
def test_build_mfma_exact_path_for_zero_and_tiny_projections(cfg_id, col0, nzero, ntiny):
    # code columns col0 + [0, nzero) give z = k0 - k1 = 0 exactly (k0 == k1), the next ntiny give
    # z = 2^-30 k2: all of them fall inside the certification band. 24 columns x 512 rows
    # overflow the queue segment of the code wave owning those columns (every word of the
    # 512-token chunk recomputed); one column's 512 fit (4 lanes per queued bit, z == 0 decided
    # by the exact accumulator). cfg 5 (256-bit codes, page 32) puts them in columns 128.., which
    # the second, code-only launch builds with two waves per code block.
    _torch()
    cfg = _cfg(cfg_id, 2048, n_plant=0, num_q_heads=4, num_kv_heads=1)
    data = synth.make_layer(cfg)
    data["K"][:, :, :, 1] = data["K"][:, :, :, 0]
    W = data["W"]
    nc = nzero + ntiny
    cols = slice(col0, col0 + nc)
    W[:, :, cols] = 0.0
    W[:, 0, cols] = 1.0
    W[:, 1, cols] = -1.0
    W[:, 2, col0 + nzero:col0 + nc] = np.float32(2.0 ** -30)
    lay = hc.GpuLayer(cfg, data=data)
    lay.build(method="auto")
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref, extrema_atol_scale=MFMA_EXTREMA_SCALE)
    bits0 = ref["codes"][0, :, :2048, col0 // 32]
    assert np.all(bits0 & ((1 << nzero) - 1) == 0)                         # z == 0 gives 0
    k2pos = (data["K"][0, :, :2048, 2] > 0).astype(np.uint32)
    assert np.array_equal((bits0 >> nzero) & ((1 << ntiny) - 1), k2pos * ((1 << ntiny) - 1))


def test_build_mfma_queue_drained_between_chunks():
    """Every workgroup builds 8 chunks of 512 tokens in turn (32 sequences x 8 KV heads: each KV
    head's 32 workgroups share out its 256 chunks): code column 0 is z = k0 - k1 with k0 == k1 on every
    other token, so about 270 uncertain bits a chunk reach the first code wave's queue segment;
    it is drained into the stored words every third chunk (at 3/4 of its 1024 entries) and the
    key tile staged before the drain is staged again. Codes bit-exact and extrema admissible on
    sampled heads; bit 0 of the tied tokens is 0."""
    _torch()
    cfg = _cfg(3, 4096, batch=32, n_plant=0)
    data = synth.make_layer(cfg)
    tied = np.arange(4096) % 2 == 0
    data["K"][:, :, tied, 1] = data["K"][:, :, tied, 0]
    W = data["W"]
    W[:, :, 0] = 0.0
    W[:, 0, 0] = 1.0
    W[:, 1, 0] = -1.0
    lay = hc.GpuLayer(cfg, data=data)
    lay.build(method="auto")
    pairs = [(0, 0), (13, 5), (31, 7)]
    ref = hc.oracle_index(lay, heads_kv=pairs)
    hc.check_index(lay, ref, pairs=pairs, extrema_atol_scale=MFMA_EXTREMA_SCALE)
    got = lay.index_host()["codes"]
    assert np.all(got[:, :, :4096, 0][:, :, tied] & 1 == 0)
    k0, k1 = data["K"][..., 0], data["K"][..., 1]
    want = (k0 - k1 > 0)[:, :, :4096][:, :, ~tied].astype(np.uint32)
    assert np.array_equal(got[:, :, :4096, 0][:, :, ~tied] & 1, want)


def test_step_codes_exact_for_zero_and_tiny_projections():
    """Codes computed in the decode step (queries) and by appends (keys) where the projection
    is exactly 0 (16 columns: x0 - x1 with x0 == x1) or tiny (8 columns: 2^-30 x2): the
    certified fp32 test must defer to the exact path and still match the oracle."""
    torch = _torch()
    cfg = _cfg(3, 2000, n_plant=0, num_q_heads=4, num_kv_heads=1)
    data = synth.make_layer(cfg, max_seq_len=2048)
    data["q"][..., 1] = data["q"][..., 0]
    W = data["W"]
    W[:, :, :24] = 0.0
    W[:, 0, :24] = 1.0
    W[:, 1, :24] = -1.0
    W[:, 2, 16:24] = np.float32(2.0 ** -30)
    lay = hc.GpuLayer(cfg, data=data)
    lay.build(method="fp64")
    kn, vn = synth.append_tokens(cfg, 4)
    kn[..., 1] = kn[..., 0]
    dec = hb.Decoder(lay.dims, cfg.keep_ratio, 200)
    out = torch.empty((1, 4, 128), dtype=torch.float32, device="cuda")
    for i in range(3):
        hb.append(lay.cache, hc.to_dev(kn[i], lay.tdt), hc.to_dev(vn[i], lay.tdt), lay.R, lay.W)
    dbg = hb.Debug(lay.dims, 200)
    dec(lay.cache, lay.q, lay.R, lay.W, out, dbg, k_new=hc.to_dev(kn[3], lay.tdt),
        v_new=hc.to_dev(vn[3], lay.tdt))
    torch.cuda.synchronize()
    d = lay.data
    d["K"][0, :, 2000:2004] = kn[:, 0].transpose(1, 0, 2)
    d["V"][0, :, 2000:2004] = vn[:, 0].transpose(1, 0, 2)
    d["seq_lens"][:] = 2004
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref)
    hc.check_decode(lay, out, dbg, cfg.keep_ratio, 200, ref_index=ref)
    qc = dbg.q_code.cpu().numpy().view(np.uint32)[0, :, 0]
    assert np.all(qc & 0xFFFF == 0)                                        # z == 0 gives 0


def test_decode_on_mfma_index_matches_oracle():
    _torch()
    cfg = _cfg(3, 9000, n_plant=16)
    lay = hc.GpuLayer(cfg, max_seq_len=9024)
    lay.build(method="auto")
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref, extrema_atol_scale=MFMA_EXTREMA_SCALE)
    out, dbg = lay.decode(1 / 16, 512)
    st = hc.check_decode(lay, out, dbg, 1 / 16, 512, ref_index=ref)
    print(f"mfma index: max out rel err {st['max_out_rel']:.2e}, page swaps {st['swaps']}")


# ---------------------------------------------------------------------------------------------
# Stage variants (Appendix C, Table 8) and the dense baseline (§4.3, Fig. 7)
# ---------------------------------------------------------------------------------------------
STAGE_CASES = [
    # stages, cfg, L, batch, lens, rho, k
    ("pages", 2, 3001, None, None, 1 / 8, 300),
    ("pages", 4, 3000, 3, [3000, 1777, 17], 0.30, 50),
    ("pages", 1, 2000, None, None, 0.25, 7),            # fp32, G = 1
    ("codes", 2, 3001, None, None, 1 / 8, 300),
    ("codes", 5, 2085, 2, None, 1 / 8, 257),            # page 32, 256-bit codes
    ("codes", 1, 2000, None, None, 0.25, 2000),         # k = L: dense
]


@pytest.mark.parametrize("stages,cfg_id,L,batch,lens,rho,k", STAGE_CASES)
def test_decode_stage_variants_match_oracle(stages, cfg_id, L, batch, lens, rho, k):
    _torch()
    cfg = _cfg(cfg_id, L, batch=batch, lens=lens, n_plant=8)
    lay = hc.GpuLayer(cfg, max_seq_len=L + 64)
    lay.build()
    ref = hc.oracle_index(lay)
    out, dbg = lay.decode(rho, k, stages=stages)
    st = hc.check_decode(lay, out, dbg, rho, k, ref_index=ref, stages=stages)
    print(f"{stages} cfg{cfg_id} L={L}: max out rel err {st['max_out_rel']:.2e}")


def test_codes_only_leaves_bounds_untouched_and_identity_rotation_works():
    torch = _torch()
    cfg = _cfg(2, 1500, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=1536)
    # R = I: the plain per-channel min/max page bound (the rotation is an input)
    lay.R = torch.eye(128, dtype=torch.float32, device="cuda").expand(8, 128, 128).contiguous()
    lay.data = dict(lay.data, R=np.stack([np.eye(128, dtype=np.float32)] * 8))
    lay.build()
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref)
    out, dbg = lay.decode(0.2, 100)
    hc.check_decode(lay, out, dbg, 0.2, 100, ref_index=ref)
    out2, dbg2 = lay.decode(0.2, 100, stages="codes", debug=True)
    assert torch.all(dbg2.bounds == 0.0)      # freshly allocated: never written
    hc.check_decode(lay, out2, dbg2, 0.2, 100, ref_index=ref, stages="codes")


DENSE_CASES = [
    # cfg, L, batch, lens
    (1, 4096, None, None),                  # fp32, G = 1
    (2, 5003, None, None),                  # bf16, G = 4, ragged
    (4, 3000, 3, [3000, 0, 1]),             # empty and one-token sequences
    (5, 4096, 2, [4096, 2049]),
]


@pytest.mark.parametrize("cfg_id,L,batch,lens", DENSE_CASES)
def test_dense_decode_matches_textbook_attention(cfg_id, L, batch, lens):
    torch = _torch()
    cfg = _cfg(cfg_id, L, batch=batch, lens=lens, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=L + 64)
    dd = hb.DenseDecoder(lay.dims)
    out = torch.full((cfg.batch, cfg.num_q_heads, 128), float("nan"), dtype=torch.float32,
                     device="cuda")
    dd(lay.cache, lay.q, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    d = lay.data
    for b in range(cfg.batch):
        Lb = int(d["seq_lens"][b])
        for h in range(cfg.num_q_heads):
            if Lb == 0:
                assert np.all(got[b, h] == 0.0)
                continue
            g = h // cfg.group
            ref = orc.dense_head(d["q"][b, h], d["K"][b, g], d["V"][b, g], Lb,
                                 orc.default_scale(128))
            rel = np.abs(got[b, h] - ref).max() / np.abs(ref).max()
            assert rel <= hc.OUT_RTOL, (b, h, rel)


def test_dense_decode_fp32_query_on_bf16_cache():
    """A fp32 query (not bf16-representable) against bf16 K/V: the matrix-core logits take the
    query as two bf16 pieces."""
    torch = _torch()
    cfg = _cfg(2, 3000, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=3072)
    dims = hb.make_dims(1, 32, 8, 16, 128, lay.data["max_seq_len"], kv_dtype=hb.HHR_BF16,
                        q_dtype=hb.HHR_F32)
    qf = np.random.default_rng(5).standard_normal((1, 32, 128)).astype(np.float32)
    dd = hb.DenseDecoder(dims)
    out = torch.full((1, 32, 128), float("nan"), dtype=torch.float32, device="cuda")
    dd(lay.cache, torch.from_numpy(qf).cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    d = lay.data
    for h in range(32):
        ref = orc.dense_head(qf[0, h], d["K"][0, h // 4], d["V"][0, h // 4], 3000,
                             orc.default_scale(128))
        rel = np.abs(got[0, h] - ref).max() / np.abs(ref).max()
        assert rel <= hc.OUT_RTOL, (h, rel)


# ---------------------------------------------------------------------------------------------
# Compressed page summaries: bf16 extrema rounded outward
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("method", ["fp64", "auto"])
@pytest.mark.parametrize("cfg_id,L,batch", [(2, 3001, None), (5, 2085, 2), (1, 1111, None)])
def test_bf16_extrema_build_and_decode(method, cfg_id, L, batch):
    _torch()
    cfg = _cfg(cfg_id, L, batch=batch, n_plant=8)
    lay = hc.GpuLayer(cfg, max_seq_len=L + 64, summary="bf16")
    lay.build(method=method)
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref, extrema_atol_scale=20.0 if method == "auto" else 1.0)
    if method == "fp64":   # the fp64 build rounds the oracle's own fp32 values: identical
        got = lay.index_host()
        for b in range(cfg.batch):
            P = -(-int(lay.data["seq_lens"][b]) // cfg.page_size)
            assert np.array_equal(got["lo"][b, :, :P], ref["lo"][b, :, :P])
            assert np.array_equal(got["hi"][b, :, :P], ref["hi"][b, :, :P])
    rho = cfg.keep_ratio
    out, dbg = lay.decode(rho, 200)
    hc.check_decode(lay, out, dbg, rho, 200, ref_index=ref)


def test_bf16_extrema_append_decode_equals_rebuild():
    torch = _torch()
    base = synth.CONFIGS[3]
    L0, n = 3 * 16 - 5, 2 * 16 + 9
    cfg = base.scaled(seq_len=L0, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=L0 + n + 64, summary="bf16")
    lay.build(method="fp64")
    kn, vn = synth.append_tokens(cfg, n)
    dec = hb.Decoder(lay.dims, cfg.keep_ratio, 40)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    for i in range(n):   # appends folded into decode steps
        dec(lay.cache, lay.q, lay.R, lay.W, out, k_new=hc.to_dev(kn[i], lay.tdt),
            v_new=hc.to_dev(vn[i], lay.tdt))
    torch.cuda.synchronize()
    d = lay.data
    d["K"][0, :, L0:L0 + n] = kn[:, 0].transpose(1, 0, 2)
    d["V"][0, :, L0:L0 + n] = vn[:, 0].transpose(1, 0, 2)
    d["seq_lens"][:] = L0 + n
    ref = hc.oracle_index(lay)
    got = lay.index_host()
    P = -(-(L0 + n) // 16)
    assert np.array_equal(got["lo"][0, :, :P], ref["lo"][0, :, :P])
    assert np.array_equal(got["hi"][0, :, :P], ref["hi"][0, :, :P])
    hc.check_index(lay, ref)
    out, dbg = lay.decode(cfg.keep_ratio, 40)
    hc.check_decode(lay, out, dbg, cfg.keep_ratio, 40, ref_index=ref)


# ---------------------------------------------------------------------------------------------
# Group-shared selection: one page and token set per KV head
# ---------------------------------------------------------------------------------------------
SHARED_CASES = [
    # stages, cfg, L, batch, lens, rho, k, summary
    ("both", 2, 3001, None, None, 1 / 8, 300, "f32"),
    ("both", 4, 3000, 3, [3000, 1777, 17], 0.30, 50, "f32"),
    ("both", 5, 2085, 2, None, 1 / 8, 257, "f32"),       # page 32, 256-bit codes
    ("both", 1, 1500, None, None, 0.25, 100, "f32"),     # G = 1: the per-head step
    ("pages", 2, 2000, None, None, 0.2, 1, "f32"),
    ("codes", 2, 2000, None, None, 0.2, 150, "f32"),
    ("both", 3, 4096, None, None, 1 / 16, 256, "bf16"),
]


@pytest.mark.parametrize("stages,cfg_id,L,batch,lens,rho,k,summary", SHARED_CASES)
def test_group_shared_selection_matches_oracle(stages, cfg_id, L, batch, lens, rho, k, summary):
    _torch()
    cfg = _cfg(cfg_id, L, batch=batch, lens=lens, n_plant=8)
    lay = hc.GpuLayer(cfg, max_seq_len=L + 64, summary=summary)
    lay.build()
    ref = hc.oracle_index(lay)
    out, dbg = lay.decode(rho, k, stages=stages, group_shared=True)
    st = hc.check_decode_shared(lay, out, dbg, rho, k, ref_index=ref, stages=stages)
    print(f"shared {stages} cfg{cfg_id}: max out rel err {st['max_out_rel']:.2e}, swaps {st['swaps']}")


# ---------------------------------------------------------------------------------------------
# Group sizes other than 4 and 1, and the page capacity
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4)])     # G = 2, G = 8
@pytest.mark.parametrize("group_shared", [False, True])
def test_decode_other_group_sizes(hq, hkv, group_shared):
    _torch()
    cfg = _cfg(2, 2500, num_q_heads=hq, num_kv_heads=hkv, n_plant=4)
    lay = hc.GpuLayer(cfg, max_seq_len=2560)
    lay.build()
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref, extrema_atol_scale=20.0)
    out, dbg = lay.decode(0.15, 150, group_shared=group_shared)
    if group_shared:
        hc.check_decode_shared(lay, out, dbg, 0.15, 150, ref_index=ref)
    else:
        hc.check_decode(lay, out, dbg, 0.15, 150, ref_index=ref)


@pytest.mark.parametrize("hq,hkv", [(16, 8), (32, 4)])
def test_dense_decode_other_group_sizes(hq, hkv):
    torch = _torch()
    cfg = _cfg(2, 1800, num_q_heads=hq, num_kv_heads=hkv, n_plant=2)
    lay = hc.GpuLayer(cfg, max_seq_len=1856)
    dd = hb.DenseDecoder(lay.dims)
    out = torch.full((1, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    dd(lay.cache, lay.q, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    d, G = lay.data, hq // hkv
    for h in range(hq):
        ref = orc.dense_head(d["q"][0, h], d["K"][0, h // G], d["V"][0, h // G], 1800,
                             orc.default_scale(128))
        assert np.abs(got[0, h] - ref).max() / np.abs(ref).max() <= hc.OUT_RTOL, h


def test_decode_at_the_page_capacity():
    """16384 pages (the documented maximum) of 16 tokens: 16 pages per selection thread."""
    _torch()
    L = hb.HHR_MAX_PAGES * 16
    cfg = _cfg(2, L, num_q_heads=2, num_kv_heads=1, n_plant=8)
    lay = hc.GpuLayer(cfg, max_seq_len=L, lens=[L - 11])
    lay.build()
    ref = hc.oracle_index(lay)
    hc.check_index(lay, ref, extrema_atol_scale=20.0)
    out, dbg = lay.decode(1 / 32, 2048)
    st = hc.check_decode(lay, out, dbg, 1 / 32, 2048, ref_index=ref)
    print(f"capacity: max out rel err {st['max_out_rel']:.2e}, swaps {st['swaps']}")


@pytest.mark.parametrize("nbytes", [16, 4096, 32768, 32768 * 3 + 48, 68 * 1000 * 1000])
def test_read_probe_sums_what_it_reads(nbytes):
    """The read-rate probe reads every byte once: its per-block sums match numpy's (fp64) over
    the same floats, including a ragged last block; a guard word past the end is not read."""
    torch = _torch()
    n = nbytes // 4
    rng = np.random.default_rng(nbytes)
    host = rng.standard_normal(n + 4).astype(np.float32)
    host[n:] = np.float32(1e30)          # beyond `nbytes`: would dominate any sum that read it
    x = torch.from_numpy(host).to("cuda")
    nb = hb.hhr_read_probe_blocks(nbytes)
    partial = torch.full((nb + 1,), -7.0, dtype=torch.float32, device="cuda")
    hb.hhr_read_probe(x.data_ptr(), nbytes, partial.data_ptr(),
                      torch.cuda.current_stream().cuda_stream)
    got = partial.cpu().numpy()
    assert got[nb] == -7.0
    blk = 32768 // 4
    want = np.array([host[i * blk:min((i + 1) * blk, n)].astype(np.float64).sum()
                     for i in range(nb)])
    mag = np.array([np.abs(host[i * blk:min((i + 1) * blk, n)]).astype(np.float64).sum()
                    for i in range(nb)])
    # fp32 sums of at most 8192 terms: error below 8192 * 2^-24 of the absolute sum
    assert np.all(np.abs(got[:nb] - want) <= 8192 * 2.0 ** -24 * mag + 1e-30)
