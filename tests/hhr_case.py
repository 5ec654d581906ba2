"""Shared test plumbing: put a seeded synthetic layer on the GPU, run the library through its C
ABI, run the CPU oracle on the same arrays, and compare them by the parity rules:

  * query codes, key codes, Hamming distances: bit-exact;
  * page extrema: inside their admissible sets (within the builder's fp32 error of the oracle's
    rotated keys; for bf16 summaries, rounded outward from such a value);
  * page bounds: within tau_p = 1e-5 * S_p (S_p = sum_j |q~_j| max(|l_j|, |u_j|)) plus, for
    bf16 summaries, the bound's spread over the admissible extrema, of the oracle's bound on its
    own extrema;
  * kept page sets: exact for the GPU's own bounds; against the oracle a page in the symmetric
    difference must have an oracle bound within tau_p + max(tau) of the oracle's cut value;
  * token indices: bit-exact against the oracle's fine stage run on the GPU's page set;
  * attention output: max |o - o*| / max |o*| <= 2e-3 against exact attention over those
    indices.
"""
from __future__ import annotations

import numpy as np

from long_context_decode_gkr_amd import binding as hb
from long_context_decode_gkr_amd import synth
from oracle import hhr_oracle as orc

OUT_RTOL = 2e-3
BOUND_RTOL = 1e-5
# The matrix-core index build rounds its fp32 accumulation of a 128-term dot product (bf16 pieces
# of R, fp32 sums): its page extrema may sit up to ~20 fp32 ulps of |k|_2 (8e-6 |k|_2) from the
# correctly rounded rotated keys, against the few ulps of the fp64 build and the append.
MFMA_EXTREMA_SCALE = 20.0


def torch_mod():
    import torch
    return torch


def to_dev(a, dtype):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device="cuda").to(dtype)


class GpuLayer:
    """A synthetic layer on the device plus its oracle view."""

    def __init__(self, cfg: synth.Config, max_seq_len=None, lens=None, layer=0, data=None,
                 summary="f32"):
        torch = torch_mod()
        self.cfg = cfg
        self.summary = summary
        self.data = data if data is not None else synth.make_layer(cfg, max_seq_len, layer, lens)
        d = self.data
        kv = hb.HHR_BF16 if cfg.dtype == "bf16" else hb.HHR_F32
        self.dims = hb.make_dims(cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.page_size,
                                 cfg.hash_bits, d["max_seq_len"], kv_dtype=kv,
                                 summary_dtype=hb.HHR_BF16 if summary == "bf16" else hb.HHR_F32)
        self.tdt = torch.bfloat16 if kv == hb.HHR_BF16 else torch.float32
        self.cache = hb.Cache(self.dims)
        self.cache.K.copy_(to_dev(d["K"], self.tdt))
        self.cache.V.copy_(to_dev(d["V"], self.tdt))
        self.cache.seq_lens.copy_(torch.from_numpy(d["seq_lens"]).cuda())
        self.q = to_dev(d["q"], self.tdt)
        self.R = to_dev(d["R"], torch.float32)
        self.W = to_dev(d["W"], torch.float32)

    def build(self, method="auto"):
        hb.build_pages(self.cache, self.R, self.W, method=method)
        torch_mod().cuda.synchronize()
        self.built = method

    def extrema_scale(self) -> float:
        """The extrema tolerance scale of the builder that made this index."""
        mfma = getattr(self, "built", "auto") == "auto" and self.cfg.dtype == "bf16"
        return MFMA_EXTREMA_SCALE if mfma else 1.0

    def decode(self, rho, k, scale=0.0, debug=True, stages="both", group_shared=False):
        torch = torch_mod()
        dec = hb.Decoder(self.dims, rho, k, scale, stages=stages, group_shared=group_shared)
        out = torch.full((self.cfg.batch, self.cfg.num_q_heads, 128), float("nan"),
                         dtype=torch.float32, device="cuda")
        dbg = hb.Debug(self.dims, k, rho, stages) if debug else None
        dec(self.cache, self.q, self.R, self.W, out, dbg)
        torch.cuda.synchronize()
        return out, dbg

    # -- host copies in the oracle's natural layouts
    def index_host(self):
        c = self.cache
        lo = c.page_min.float().permute(0, 1, 3, 2).contiguous().cpu().numpy()
        hi = c.page_max.float().permute(0, 1, 3, 2).contiguous().cpu().numpy()
        codes = c.codes.cpu().numpy().view(np.uint32)
        return dict(lo=lo, hi=hi, codes=codes)


def oracle_index(layer: GpuLayer, heads_kv=None):
    """The oracle's index of the layer: key codes, page extrema as stored (bf16 rounded outward
    for a bf16 summary) in lo / hi, and the fp32 extrema before that rounding in lo32 / hi32."""
    d, cfg = layer.data, layer.cfg
    B, Hkv, Lmax, dd = d["K"].shape
    Pmax = Lmax // cfg.page_size
    lo = np.zeros((B, Hkv, Pmax, dd), np.float32)
    hi = np.zeros_like(lo)
    kc = np.zeros((B, Hkv, Lmax, cfg.hash_bits // 32), np.uint32)
    pairs = heads_kv or [(b, g) for b in range(B) for g in range(Hkv)]
    for b, g in pairs:
        L = int(d["seq_lens"][b])
        l_, h_, c_ = orc.build_head(d["K"][b, g], L, d["R"][g], d["W"][g], cfg.page_size, "f32")
        lo[b, g, :len(l_)], hi[b, g, :len(h_)], kc[b, g, :L] = l_, h_, c_
    return summary_index(dict(lo32=lo, hi32=hi, codes=kc), layer.summary)


def summary_index(ref: dict, summary: str) -> dict:
    """lo / hi as the cache stores them, from the fp32 extrema lo32 / hi32."""
    if summary == "bf16":
        lo, hi = orc.extrema_bf16(ref["lo32"], ref["hi32"])
    else:
        lo, hi = ref["lo32"], ref["hi32"]
    return dict(ref, lo=lo, hi=hi)


def extrema_tolerance(K_bg: np.ndarray, L: int) -> float:
    """fp32 rounding of a 128-term dot product with an orthogonal R: a few ulps of |k|_2."""
    if L == 0:
        return 0.0
    return 4e-7 * float(np.linalg.norm(K_bg[:L].astype(np.float64), axis=1).max())


def bf16_down_up(x):
    """The bf16 grid values at or below and at or above each float64 x (the oracle's directed
    bf16 rounding, on float64 inputs)."""
    x = np.asarray(x, np.float64)
    e = np.frexp(x)[1].astype(np.float64) - 1.0
    ulp = np.exp2(np.maximum(e, -126.0) - 7.0)
    return np.floor(x / ulp) * ulp, np.ceil(x / ulp) * ulp


def admissible_extrema(lo32, hi32, tol, summary):
    """[min, max] of what a correct GPU may store for each extremum: the fp32 value within tol
    of the oracle's (the builders' rounding of the rotated keys), stored as is (fp32 summary)
    or, for a bf16 summary, the minimum rounded toward -inf and the maximum toward +inf."""
    lo32 = np.asarray(lo32, np.float64)
    hi32 = np.asarray(hi32, np.float64)
    if summary == "bf16":
        lmin, lmax = bf16_down_up(lo32 - tol)[0], bf16_down_up(lo32 + tol)[0]
        hmin, hmax = bf16_down_up(hi32 - tol)[1], bf16_down_up(hi32 + tol)[1]
        return (lmin, lmax), (hmin, hmax)
    return (lo32 - tol, lo32 + tol), (hi32 - tol, hi32 + tol)


def check_index(layer: GpuLayer, ref: dict, pairs=None, extrema_atol_scale=None):
    """Key codes bit-exact; each stored extremum inside its admissible set (admissible_extrema:
    within a few fp32 ulps of the oracle's, and for a bf16 summary a bf16 value rounded in the
    right direction from such an fp32 value)."""
    got = layer.index_host()
    d, S = layer.data, layer.cfg.page_size
    B, Hkv = d["K"].shape[:2]
    pairs = pairs or [(b, g) for b in range(B) for g in range(Hkv)]
    if extrema_atol_scale is None:
        extrema_atol_scale = layer.extrema_scale()
    for b, g in pairs:
        L = int(d["seq_lens"][b])
        P = orc.num_pages(L, S)
        np.testing.assert_array_equal(got["codes"][b, g, :L], ref["codes"][b, g, :L],
                                      err_msg=f"key codes differ at b={b} g={g}")
        tol = extrema_tolerance(d["K"][b, g], L) * extrema_atol_scale
        adm = admissible_extrema(ref["lo32"][b, g, :P], ref["hi32"][b, g, :P], tol, layer.summary)
        for name, (amin, amax) in zip(("lo", "hi"), adm):
            v = got[name][b, g, :P].astype(np.float64)
            assert np.all((amin <= v) & (v <= amax)), (name, b, g, float(np.max(amin - v)),
                                                        float(np.max(v - amax)), tol)
            if layer.summary == "bf16":   # a bf16 value (the storage is 16 bits wide)
                assert np.array_equal(bf16_down_up(v)[0], v), (name, b, g)


def bound_tolerance(qt, ref: dict, b: int, g: int, P: int, tol: float, summary: str):
    """Allowed |U_gpu - U_oracle| per page: 1e-5 S_p (S_p = sum_j |q~_j| max(|l_j|, |u_j|)),
    plus sum_j |q~_j| w_j with w_j the width of the admissible set of the extremum q~_j selects
    (u_j for q~_j >= 0, l_j otherwise): the GPU's stored extrema may be any admissible value."""
    qt = np.asarray(qt, np.float64)
    lo = ref["lo"][b, g, :P].astype(np.float64)
    hi = ref["hi"][b, g, :P].astype(np.float64)
    Sp = (np.abs(qt)[None, :] * np.maximum(np.abs(lo), np.abs(hi))).sum(axis=1)
    (lmin, lmax), (hmin, hmax) = admissible_extrema(ref["lo32"][b, g, :P], ref["hi32"][b, g, :P],
                                                    tol, summary)
    if summary == "bf16":
        width = np.where(qt[None, :] >= 0, hmax - hmin, lmax - lmin)
        dU = (np.abs(qt)[None, :] * width).sum(axis=1)
    else:
        dU = np.zeros(P)     # fp32 extrema: within the 1e-5 S_p of the bound's reading
    return BOUND_RTOL * Sp + dU


def check_page_set(gp, o_pages, U_orc, n_keep, tau, where):
    """The GPU's kept pages gp against the oracle's: a page in the symmetric difference must have
    an oracle bound within tau_p + max(tau over the difference) of the oracle's cut (a swapped
    pair p, c satisfies U(c) - U(p) <= tau_p + tau_c)."""
    cut = np.sort(U_orc)[::-1][n_keep - 1]
    sym = sorted(set(gp.tolist()) ^ set(o_pages.tolist()))
    if sym:
        tmax = max(tau[p] for p in sym)
        for p in sym:
            assert abs(U_orc[p] - cut) <= tau[p] + tmax, (where, p, U_orc[p], cut, tau[p])
    return len(sym) // 2


def check_decode(layer: GpuLayer, out, dbg, rho, k, scale=None, heads=None, ref_index=None,
                 stages="both", extrema_atol_scale=None):
    """Compare one decode step with the oracle on the listed (b, h) pairs (default: all).
    `stages`: "both", "pages" (coarse stage only) or "codes" (fine stage only)."""
    d, cfg = layer.data, layer.cfg
    S, G = cfg.page_size, cfg.group
    scale = orc.default_scale(128) if not scale else scale
    ref_index = ref_index or oracle_index(layer)
    if extrema_atol_scale is None:
        extrema_atol_scale = layer.extrema_scale()
    out_h = out.cpu().numpy()
    qr = dbg.q_rot.cpu().numpy()
    qc = dbg.q_code.cpu().numpy().view(np.uint32)
    U = dbg.bounds.cpu().numpy()
    pid = dbg.page_ids.cpu().numpy()
    pcnt = dbg.page_count.cpu().numpy()
    dist = dbg.dist.cpu().numpy().view(np.uint16)
    tidx = dbg.token_idx.cpu().numpy()
    tcnt = dbg.token_count.cpu().numpy()
    heads = heads or [(b, h) for b in range(cfg.batch) for h in range(cfg.num_q_heads)]
    stats = dict(max_out_rel=0.0, swaps=0)
    for b, h in heads:
        g = h // G
        L = int(d["seq_lens"][b])
        q = d["q"][b, h]
        if L == 0:
            assert tcnt[b, h] == 0 and np.all(out_h[b, h] == 0.0)
            continue
        o = orc.decode_head(q, d["K"][b, g], d["V"][b, g], L, ref_index["lo"][b, g],
                            ref_index["hi"][b, g], ref_index["codes"][b, g], d["R"][g], d["W"][g],
                            S, rho, k, scale, stages=stages)
        P, n_keep = orc.num_pages(L, S), o["n_keep"]
        # query rotation and code
        assert np.abs(qr[b, h] - o["q_rot"]).max() <= 1e-6 * np.linalg.norm(q), (b, h)
        np.testing.assert_array_equal(qc[b, h], o["q_code"], err_msg=f"q code b={b} h={h}")
        assert pcnt[b, h] == n_keep
        gp = pid[b, h, :n_keep]
        assert np.all(np.diff(gp) > 0)
        if stages == "codes":
            np.testing.assert_array_equal(gp, np.arange(P))   # every page is a candidate
        else:
            # bounds: GPU (own index, own q~) against the oracle's (its own extrema)
            tol = extrema_tolerance(d["K"][b, g], L) * extrema_atol_scale
            tau = bound_tolerance(o["q_rot"], ref_index, b, g, P, tol, layer.summary)
            assert np.all(np.abs(U[b, h, :P] - o["U"]) <= tau), (b, h)
            # page set: exact for the GPU's own bounds; swaps against the oracle only at
            # near-ties
            np.testing.assert_array_equal(gp, orc.select_pages(U[b, h, :P].astype(np.float64),
                                                               n_keep))
            stats["swaps"] += check_page_set(gp, o["pages"], o["U"], n_keep, tau, (b, h))
        # fine stage on the GPU's pages
        cand = orc.candidates(gp, L, S)
        if stages == "pages":
            sel = cand                                       # every candidate is attended
        else:
            Dref = orc.hamming(o["q_code"], ref_index["codes"][b, g][cand])
            slots = (gp[:, None] * S + np.arange(S)[None, :]).reshape(-1)
            dgot = dist[b, h, :n_keep * S]
            np.testing.assert_array_equal(dgot[slots < L], Dref, err_msg=f"distances b={b} h={h}")
            assert np.all(dgot[slots >= L] == 0xFFFF)
            sel = orc.select_tokens(cand, Dref, k)
        assert tcnt[b, h] == len(sel), (b, h)
        np.testing.assert_array_equal(tidx[b, h, :len(sel)], sel, err_msg=f"tokens b={b} h={h}")
        ref_out = orc.attend(q, d["K"][b, g][sel], d["V"][b, g][sel], scale)
        rel = np.abs(out_h[b, h] - ref_out).max() / np.abs(ref_out).max()
        assert rel <= OUT_RTOL, (b, h, rel)
        stats["max_out_rel"] = max(stats["max_out_rel"], float(rel))
    return stats


def check_decode_shared(layer: GpuLayer, out, dbg, rho, k, scale=None, ref_index=None,
                        stages="both", groups=None, extrema_atol_scale=None):
    """One selection per (b, KV head) (group_shared): per-head bounds and query codes as in
    check_decode; the group's page set on the GPU's own U (the largest head bound) and, against
    the oracle, swaps only at near-ties; distances (smallest over the group) and tokens
    bit-exact on the GPU's pages; each head's output within the tolerance."""
    d, cfg = layer.data, layer.cfg
    S, G, Hkv = cfg.page_size, cfg.group, cfg.num_kv_heads
    scale = orc.default_scale(128) if not scale else scale
    ref_index = ref_index or oracle_index(layer)
    if extrema_atol_scale is None:
        extrema_atol_scale = layer.extrema_scale()
    out_h = out.cpu().numpy()
    qr = dbg.q_rot.cpu().numpy()
    qc = dbg.q_code.cpu().numpy().view(np.uint32)
    U = dbg.bounds.cpu().numpy()
    pid = dbg.page_ids.cpu().numpy().reshape(-1, dbg.page_ids.shape[-1])
    pcnt = dbg.page_count.cpu().numpy().reshape(-1)
    dist = dbg.dist.cpu().numpy().view(np.uint16).reshape(-1, dbg.dist.shape[-1])
    tidx = dbg.token_idx.cpu().numpy().reshape(-1, dbg.token_idx.shape[-1])
    tcnt = dbg.token_count.cpu().numpy().reshape(-1)
    groups = groups or [(b, g) for b in range(cfg.batch) for g in range(Hkv)]
    stats = dict(max_out_rel=0.0, swaps=0)
    for b, g in groups:
        L = int(d["seq_lens"][b])
        row = b * Hkv + g
        heads = list(range(g * G, g * G + G))
        qs = d["q"][b, heads]
        if L == 0:
            assert tcnt[row] == 0 and np.all(out_h[b, heads] == 0.0)
            continue
        o = orc.decode_group(qs, d["K"][b, g], d["V"][b, g], L, ref_index["lo"][b, g],
                             ref_index["hi"][b, g], ref_index["codes"][b, g], d["R"][g],
                             d["W"][g], S, rho, k, scale, stages=stages)
        P, n_keep = orc.num_pages(L, S), o["n_keep"]
        for i, h in enumerate(heads):
            assert np.abs(qr[b, h] - o["q_rot"][i]).max() <= 1e-6 * np.linalg.norm(qs[i]), (b, h)
            np.testing.assert_array_equal(qc[b, h], o["q_code"][i], err_msg=f"q code b={b} h={h}")
        assert pcnt[row] == n_keep
        gp = pid[row, :n_keep]
        assert np.all(np.diff(gp) > 0)
        if stages == "codes":
            np.testing.assert_array_equal(gp, np.arange(P))
        else:
            tol = extrema_tolerance(d["K"][b, g], L) * extrema_atol_scale
            tau = np.zeros(P)
            for i, h in enumerate(heads):
                th = bound_tolerance(o["q_rot"][i], ref_index, b, g, P, tol, layer.summary)
                Uh = orc.page_bounds(o["q_rot"][i], ref_index["lo"][b, g, :P],
                                     ref_index["hi"][b, g, :P])
                assert np.all(np.abs(U[b, h, :P] - Uh) <= th), (b, h)
                tau = np.maximum(tau, th)
            Ug = U[b, heads, :P].astype(np.float64).max(axis=0)   # the GPU's group bound
            np.testing.assert_array_equal(gp, orc.select_pages(Ug, n_keep))
            stats["swaps"] += check_page_set(gp, o["pages"], o["U"], n_keep, tau, (b, g))
        cand = orc.candidates(gp, L, S)
        if stages == "pages":
            sel = cand
        else:
            Dref = np.stack([orc.hamming(o["q_code"][i], ref_index["codes"][b, g][cand])
                             for i in range(G)]).min(axis=0)
            slots = (gp[:, None] * S + np.arange(S)[None, :]).reshape(-1)
            dgot = dist[row, :n_keep * S]
            np.testing.assert_array_equal(dgot[slots < L], Dref, err_msg=f"distances b={b} g={g}")
            sel = orc.select_tokens(cand, Dref, k)
        assert tcnt[row] == len(sel), (b, g)
        np.testing.assert_array_equal(tidx[row, :len(sel)], sel, err_msg=f"tokens b={b} g={g}")
        for i, h in enumerate(heads):
            ref_out = orc.attend(qs[i], d["K"][b, g][sel], d["V"][b, g][sel], scale)
            rel = np.abs(out_h[b, h] - ref_out).max() / np.abs(ref_out).max()
            assert rel <= OUT_RTOL, (b, h, rel)
            stats["max_out_rel"] = max(stats["max_out_rel"], float(rel))
    return stats
