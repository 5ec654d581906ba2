"""The C-ABI library on the CPU: it loads, exports every symbol the header declares, and rejects
invalid calls with the documented status before touching the device. No kernel is launched."""
import ctypes
import os
import re

import pytest

from long_context_decode_gkr_amd import binding as hb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hhr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(hb.LIB_PATH), reason="libhhr.so not built")

FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hhr_status|size_t|const char\*)\s+(hhr_\w+)\s*\(", text,
                                 re.M)))


def test_library_exports_every_declared_symbol():
    lib = hb.load()
    names = declared_functions()
    assert set(names) == set(hb.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, text in hb.STATUS.items():
        assert hb.hhr_status_string(code) == text


def good_dims(**kw):
    d = dict(batch=1, num_q_heads=32, num_kv_heads=8, page_size=16, hash_bits=128,
             max_seq_len=4096, kv_dtype=hb.HHR_BF16)
    d.update(kw)
    return hb.make_dims(**d)


def fake_cache(**kw):
    c = hb.CacheStruct(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def decode_status(dims=None, params=None, cache=None, ws=FAKE * 256, ws_bytes=1 << 40, q=FAKE,
                  out=FAKE):
    lib = hb.load()
    dims = dims or good_dims()
    params = params or hb.Params(0.125, 2048, 0.0)
    cache = cache or fake_cache()
    return lib.hhr_decode(ctypes.byref(dims), ctypes.byref(params), ctypes.byref(cache), q, FAKE,
                          FAKE, ws, ws_bytes, out, None, None)


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, 2), ("page_size", 8, 2), ("hash_bits", 64, 2), ("num_q_heads", 12, 1),
    ("num_q_heads", 48, 2), ("batch", 0, 1), ("max_seq_len", 4104, 2), ("kv_dtype", 7, 1),
    ("q_dtype", -1, 1), ("max_seq_len", 16 * 16384 + 64, 3), ("max_seq_len", -64, 1),
])
def test_invalid_dims(field, value, status):
    d = good_dims()
    setattr(d, field, value)
    assert decode_status(dims=d) == status
    lib = hb.load()
    assert lib.hhr_build_pages(ctypes.byref(d), ctypes.byref(fake_cache()), FAKE, FAKE, None) == status
    assert lib.hhr_append(ctypes.byref(d), ctypes.byref(fake_cache()), FAKE, FAKE, FAKE, FAKE, None) == status


@pytest.mark.parametrize("rho,k,scale", [(0.0, 10, 0.0), (1.5, 10, 0.0), (float("nan"), 10, 0.0),
                                         (0.5, 0, 0.0), (0.5, -3, 0.0), (0.5, 4, float("inf"))])
def test_invalid_params(rho, k, scale):
    assert decode_status(params=hb.Params(rho, k, scale)) == 1
    assert hb.hhr_decode_workspace_bytes(good_dims(), hb.Params(rho, k, scale)) == 0


@pytest.mark.parametrize("field", ["K", "V", "page_min", "page_max", "codes", "seq_lens"])
def test_null_cache_pointer(field):
    assert decode_status(cache=fake_cache(**{field: None})) == 1


def test_null_ticket_only_matters_for_append():
    lib = hb.load()
    c = fake_cache(append_ticket=None)
    d = good_dims()
    assert lib.hhr_append(ctypes.byref(d), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, None) == 1


def test_null_io_pointers():
    assert decode_status(q=None) == 1
    assert decode_status(out=None) == 1


def test_workspace_checks():
    need = hb.hhr_decode_workspace_bytes(good_dims(), hb.Params(0.125, 2048, 0.0))
    assert need > 0
    assert decode_status(ws_bytes=need - 1) == 4
    assert decode_status(ws=FAKE * 256 + 64, ws_bytes=need) == 4
    assert decode_status(ws=None, ws_bytes=need) == 4


def test_workspace_size_grows_with_shapes():
    p = hb.Params(0.125, 2048, 0.0)
    a = hb.hhr_decode_workspace_bytes(good_dims(max_seq_len=4096), p)
    b = hb.hhr_decode_workspace_bytes(good_dims(max_seq_len=131072), p)
    c = hb.hhr_decode_workspace_bytes(good_dims(batch=4, max_seq_len=131072), p)
    assert 0 < a < b < c
    # U + indices + counters + split partials: at least the bounds and the token indices
    assert b >= 32 * (131072 // 16) * 4 + 32 * 2048 * 4


def test_append_decode_needs_new_token_and_ticket():
    lib = hb.load()
    d, p = good_dims(), hb.Params(0.125, 2048, 0.0)

    def call(cache, kn=FAKE, vn=FAKE):
        return lib.hhr_append_decode(ctypes.byref(d), ctypes.byref(p), ctypes.byref(cache), kn, vn,
                                     FAKE, FAKE, FAKE, FAKE * 256, 1 << 40, FAKE, None, None)
    assert call(fake_cache(), kn=None) == 1
    assert call(fake_cache(), vn=None) == 1
    assert call(fake_cache(append_ticket=None)) == 1


@pytest.mark.parametrize("stages", [-1, 3, 100])
def test_invalid_stages(stages):
    p = hb.Params(0.125, 2048, 0.0, stages)
    assert decode_status(params=p) == 1
    assert hb.hhr_decode_workspace_bytes(good_dims(), p) == 0


def _align256(x):
    return (x + 255) // 256 * 256


def expected_workspace(B, Hq, Hkv, S, nb, lmax, rho, k, stages, shared=False, bf16=True):
    """The decode workspace carve-up written out: q~, query codes, bounds, index rows (kcap
    rounded to 4 plus 64 trash entries), counts, attention partials, then the selection's kept
    page ids, candidate distances and per-slice histograms."""
    import math
    import bench
    pmax = lmax // S
    if stages == hb.HHR_STAGES_CODES_ONLY:
        rho = 1.0
    kpages = min(pmax, max(1, math.ceil(rho * pmax)))
    kcap = min(kpages * S, lmax) if stages == hb.HHR_STAGES_PAGES_ONLY else min(k, lmax)
    chunk = 128 if bf16 else 64       # rows per attention workgroup (both bf16 kernels: 128)
    nsplit = -(-kcap // chunk)
    BH, NU = B * Hq, B * (Hkv if shared else Hq)
    nsl = bench.select_slices(kpages, NU, stages == hb.HHR_STAGES_CODES_ONLY)
    dstride = (kpages * S + 15) // 16 * 16
    istride = (kcap + 3) // 4 * 4 + 64
    parts = [BH * 128 * 4, BH * (nb // 32) * 4, NU * pmax * 4, NU * istride * 4, NU * 4,
             BH * nsplit * 130 * 4, NU * kpages * 4, NU * dstride * (1 if nb == 128 else 2),
             NU * nsl * (nb + 1) * 4]
    return sum(_align256(x) for x in parts)


@pytest.mark.parametrize("lmax,S,nb,rho,k,shared", [
    (131072, 16, 128, 1 / 16, 4096, False), (32768, 16, 128, 1 / 8, 2048, False),
    (131072, 16, 128, 1 / 16, 4096, True), (65536, 32, 256, 1 / 8, 4096, False),
    (64, 16, 128, 0.3, 8, False), (262144, 16, 128, 1.0, 100, False)])
@pytest.mark.parametrize("stages", [hb.HHR_STAGES_BOTH, hb.HHR_STAGES_PAGES_ONLY,
                                    hb.HHR_STAGES_CODES_ONLY])
def test_workspace_size_matches_its_carve_up(lmax, S, nb, rho, k, shared, stages):
    d = hb.make_dims(1, 32, 8, S, nb, lmax)
    p = hb.Params(rho, k, 0.0, stages, int(shared))
    assert hb.hhr_decode_workspace_bytes(d, p) == \
        expected_workspace(1, 32, 8, S, nb, lmax, rho, k, stages, shared)


@pytest.mark.parametrize("lmax,S,rho,units,stages", [
    (2112, 16, 1.0, 1, hb.HHR_STAGES_CODES_ONLY),     # max_seq_len not a multiple of 4096
    (4160, 32, 0.3, 32, hb.HHR_STAGES_BOTH),
    (131072, 16, 1 / 16, 32, hb.HHR_STAGES_BOTH),
    (262144, 16, 1.0, 32, hb.HHR_STAGES_CODES_ONLY),
    (64, 16, 1.0, 3, hb.HHR_STAGES_PAGES_ONLY)])
def test_sliced_selection_reads_stay_in_its_rows(lmax, S, rho, units, stages):
    """The sliced selection's addressing, written out: for every sequence length, slice i of n
    owns kept-page ranks [i n_keep / n, (i + 1) n_keep / n); its emission reads its slots' one-
    or two-byte distances 16 at a time from a clamped start and one page id per 16 slots. Every
    read must stay within the unit's row of kpages * S distances (rounded up to 16), which is
    what the workspace holds per unit."""
    import math
    import bench
    pmax = lmax // S
    r = 1.0 if stages == hb.HHR_STAGES_CODES_ONLY else rho
    kpages = min(pmax, max(1, math.ceil(r * pmax)))
    nsl = bench.select_slices(kpages, units, stages == hb.HHR_STAGES_CODES_ONLY)
    dstride = (kpages * S + 15) // 16 * 16
    assert -(-kpages // nsl) <= 512                    # a slice's pages fit its LDS list
    for L in sorted({1, S - 1, S, S + 1, lmax // 2 + 7, lmax - 1, lmax}):
        P = -(-L // S)
        n_keep = min(P, max(1, math.ceil(r * P)))
        assert n_keep <= kpages
        for i in range(nsl):
            r0, r1 = i * n_keep // nsl, (i + 1) * n_keep // nsl
            nslots = (r1 - r0) * S
            if nslots == 0:
                continue
            assert nslots % 16 == 0
            for base in range(0, nslots, 256 * 16):
                for tid in (0, 1, 255):
                    s0 = min(base + 16 * tid, max(nslots - 16, 0))
                    assert 0 <= r0 * S + s0 and r0 * S + s0 + 16 <= dstride
                    assert r0 + s0 // S < r1                # its page id is in the slice
            # the scan writes 4 distances per unit of 4 slots
            assert r1 * S <= dstride


def test_scratch_decode_validates_before_touching_the_device():
    """The allocation-free decode validates like hhr_decode and refuses shapes whose workspace
    exceeds HHR_SCRATCH_BYTES, all before any device call (fake pointers, no GPU)."""
    lib = hb.load()
    p = hb.Params(0.125, 2048, 0.0)

    def call(dims, params=p, cache=None, q=FAKE, out=FAKE):
        return lib.hhr_decode_scratch(ctypes.byref(dims), ctypes.byref(params),
                                      ctypes.byref(cache or fake_cache()), q, FAKE, FAKE, out,
                                      None, None)
    assert call(good_dims(), q=None) == 1
    assert call(good_dims(), out=None) == 1
    assert call(good_dims(), params=hb.Params(0.0, 2048, 0.0)) == 1
    big = good_dims(batch=64, max_seq_len=131072)
    assert hb.hhr_decode_workspace_bytes(big, p) > hb.HHR_SCRATCH_BYTES
    assert call(big) == 3                                   # HHR_ERR_CAPACITY
    # the bench's workloads fit
    for B, L, S, nb, rho, k in ((1, 131072, 16, 128, 1 / 16, 4096), (8, 32768, 16, 128, 0.3, 2048),
                                (4, 65536, 32, 256, 1 / 8, 4096)):
        d = good_dims(batch=B, max_seq_len=L, page_size=S, hash_bits=nb)
        assert hb.hhr_decode_workspace_bytes(d, hb.Params(rho, k, 0.0)) <= hb.HHR_SCRATCH_BYTES


def test_pages_only_workspace_holds_every_kept_token():
    d = good_dims(max_seq_len=131072)
    both = hb.hhr_decode_workspace_bytes(d, hb.Params(1 / 16, 4096, 0.0, hb.HHR_STAGES_BOTH))
    pages = hb.hhr_decode_workspace_bytes(d, hb.Params(1 / 16, 4096, 0.0,
                                                       hb.HHR_STAGES_PAGES_ONLY))
    codes = hb.hhr_decode_workspace_bytes(d, hb.Params(1 / 16, 4096, 0.0,
                                                       hb.HHR_STAGES_CODES_ONLY))
    # pages only: 512 kept pages x 16 tokens = 8192 indices per head instead of 4096
    assert pages >= both + 32 * 4096 * 4
    # fine only: every token a candidate (a distance byte each) and every page kept
    assert codes >= both + 32 * (131072 - 8192) + 32 * (8192 - 512) * 4


def dense_status(dims=None, cache=None, q=FAKE, scale=0.0, ws=FAKE * 256, ws_bytes=1 << 40,
                 out=FAKE):
    lib = hb.load()
    dims = dims or good_dims()
    cache = cache or fake_cache()
    return lib.hhr_dense_decode(ctypes.byref(dims), ctypes.byref(cache), q, scale, ws, ws_bytes,
                                out, None, None)


def test_dense_decode_validation():
    d = good_dims()
    need = hb.hhr_dense_workspace_bytes(d)
    # one partial (128 + 2 floats) per (b, h) and split
    assert need > 0 and need % (32 * 130 * 4) == 0
    bad = good_dims(head_dim=64)
    assert hb.hhr_dense_workspace_bytes(bad) == 0
    assert dense_status(dims=bad) == 2
    for field in ("K", "V", "seq_lens"):
        assert dense_status(cache=fake_cache(**{field: None})) == 1
    # the index is not read: its pointers may be NULL (validation passes them; the call then
    # fails on the workspace check below, before anything is enqueued)
    assert dense_status(cache=fake_cache(page_min=None, page_max=None, codes=None),
                        ws_bytes=need - 1) == 4
    assert dense_status(q=None) == 1
    assert dense_status(out=None) == 1
    assert dense_status(scale=float("nan")) == 1
    assert dense_status(ws_bytes=need - 1) == 4
    assert dense_status(ws=FAKE * 256 + 4, ws_bytes=need) == 4


@pytest.mark.parametrize("value", [-1, 2, 9])
def test_invalid_summary_dtype(value):
    d = good_dims()
    d.summary_dtype = value
    assert decode_status(dims=d) == 1
    assert hb.hhr_dense_workspace_bytes(d) == 0


@pytest.mark.parametrize("value", [-1, 2])
def test_invalid_group_shared(value):
    p = hb.Params(0.125, 2048, 0.0, 0, value)
    assert decode_status(params=p) == 1


def test_group_shared_workspace_is_smaller():
    d = good_dims(max_seq_len=131072)
    per_head = hb.hhr_decode_workspace_bytes(d, hb.Params(1 / 16, 4096, 0.0, 0, 0))
    shared = hb.hhr_decode_workspace_bytes(d, hb.Params(1 / 16, 4096, 0.0, 0, 1))
    assert 0 < shared < per_head


def test_read_probe_blocks_and_validation():
    lib = hb.load()
    assert hb.hhr_read_probe_blocks(16) == 1
    assert hb.hhr_read_probe_blocks(32768) == 1
    assert hb.hhr_read_probe_blocks(32768 + 16) == 2
    assert hb.hhr_read_probe_blocks(68 * 1000 * 1000) == -(-68 * 1000 * 1000 // 32768)
    for src, nbytes, partial in [(None, 4096, FAKE), (FAKE, 4096, None), (FAKE, 0, FAKE),
                                 (FAKE, 4100, FAKE), (FAKE + 4, 4096, FAKE)]:
        assert lib.hhr_read_probe(src, nbytes, partial, None) == 1


def test_header_compiles_as_c_and_links(tmp_path):
    """include/hhr.h is plain C: a C11 translation unit (strict warnings) that takes the address
    of every declared entry point compiles, links against libhhr.so and loads."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    names = declared_functions()
    src = tmp_path / "use.c"
    src.write_text('#include "hhr.h"\ntypedef void (*fn)(void);\nint main(void) {\n  int n = 0;\n' +
                   "".join(f"  n += (fn)&{n} != (fn)0;\n" for n in names) +
                   f"  return n == {len(names)} ? 0 : 1;\n}}\n")
    exe = tmp_path / "use"
    lib_dir = os.path.dirname(hb.LIB_PATH)
    r = subprocess.run([cc, "-std=c11", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe),
                        f"-L{lib_dir}", "-l:libhhr.so", f"-Wl,-rpath,{lib_dir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True)   # resolves, calls nothing
    assert run.returncode == 0, run.stderr
