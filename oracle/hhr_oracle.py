"""CPU oracle of the HHR sparse-attention decode step.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import or run this module. The GPU library never calls it and shares no code
with it; the two meet only through the seeded input generator.

It is a plain, slow, obviously-correct restatement of the method in "HHR: Hierarchical Hash
Retrieval for Efficient LLM Generation" (arXiv 2610.01230):

* §3.3.1, Eq. (4): head-wise orthogonal rotation, q~ = q R and k~ = k R (row vectors).
* §3.3.1, text before Eq. (3): per-page, per-dimension minimum l and maximum u of the
  (rotated) keys of non-overlapping pages.
* §3.3.1, Eq. (3): page upper bound U = sum_j max(q~_j l_j, q~_j u_j); pages with U above a
  threshold survive.
* §3.1, Eq. (1), and §3.3.2, Eq. (10) with c = sign(z) at inference: z = x W, code bit = sign.
* §3.1, Eq. (2): Hamming distance = number of differing bits (XOR + popcount).
* §3.3.2 / §1: the surviving keys are ranked by Hamming distance and attention is computed
  exactly over the selected keys.
* Appendix A: defaults (30 % candidate budget, 128-bit codes).

Readings where the paper is silent (each one also listed in the design notes):
* Rotation and projection matrices are per KV head; selection is per query head.
* The hash input is the raw stored key / query (not the rotated one).
* A code bit is 1 iff the exact real value of z = x W (from the stored operands) is > 0.
  Bit c of a code sits in 32-bit word c // 32 at position c % 32.
* The threshold c_h keeps exactly n_keep = min(P, max(1, ceil(rho * P))) pages (the product
  rho * P evaluated as one IEEE double multiply); ties in U go to the lower page index.
* Token selection keeps the k_eff = min(k, #candidates) candidates of smallest (D, t).
* Attention uses the unrotated stored q and K with scale 1/sqrt(d) unless given, fp64 here.
* Page extrema are fp32 values of the fp32-rounded rotated keys; a partial last page covers
  only its valid tokens.

Precision: fp64 throughout, with an exact fallback (math.fsum of the exact fp64 products) for
code signs whose fp64 value is within its rounding-error bound of zero.
"""
from __future__ import annotations

import math
import numpy as np

U64 = 2.0 ** -53  # unit roundoff of IEEE double


# ----------------------------------------------------------------------------------------------
# §3.3.1 Eq. (4): rotation
# ----------------------------------------------------------------------------------------------
def rotate(x: np.ndarray, R: np.ndarray) -> np.ndarray:
    """x~ = x R for row vectors x (shape [n, d]); fp64 accumulate, one rounding to fp32."""
    return (np.asarray(x, np.float64) @ np.asarray(R, np.float64)).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# §3.3.1: page extrema of the rotated keys
# ----------------------------------------------------------------------------------------------
def num_pages(L: int, S: int) -> int:
    return -(-int(L) // int(S))


def page_extrema(kt: np.ndarray, L: int, S: int):
    """lo[p], hi[p]: per-dimension min / max of rows p*S .. min(L, p*S+S)-1 of kt."""
    P = num_pages(L, S)
    d = kt.shape[1]
    lo = np.zeros((P, d), np.float32)
    hi = np.zeros((P, d), np.float32)
    for p in range(P):
        rows = kt[p * S:min(L, p * S + S)]
        lo[p] = rows.min(axis=0)
        hi[p] = rows.max(axis=0)
    return lo, hi


def _bf16_neighbours(x: np.ndarray):
    """The bf16 values just below and just above each fp32 x (equal when x is one): bf16 has
    fp32's exponent range and 8 significant bits, so near x its spacing is 2^(e - 7) with
    e = floor(log2 |x|) (at least -126, the subnormal spacing below that)."""
    x64 = np.asarray(x, np.float32).astype(np.float64)
    e = np.frexp(x64)[1].astype(np.float64) - 1.0      # |x| in [2^e, 2^(e+1)); x = 0 gives -1
    ulp = np.exp2(np.maximum(e, -126.0) - 7.0)
    down = np.floor(x64 / ulp) * ulp
    up = np.ceil(x64 / ulp) * ulp
    return down, up


def extrema_bf16(lo: np.ndarray, hi: np.ndarray):
    """Page extrema stored as bf16 (returned as fp32 values): the minimum rounded toward -inf and
    the maximum toward +inf, so max(q l, q u) over the stored values is never below its value
    over the exact ones and Eq. (3) remains an upper bound."""
    return (_bf16_neighbours(lo)[0].astype(np.float32), _bf16_neighbours(hi)[1].astype(np.float32))


# ----------------------------------------------------------------------------------------------
# §3.1 Eq. (1), §3.3.2 Eq. (10): sign codes
# ----------------------------------------------------------------------------------------------
def _exact_positive(x_row: np.ndarray, w_col: np.ndarray) -> bool:
    """Is sum_j x_j w_j > 0 for the exact real value?

    Each product of two fp32 values is exact in fp64 (at most 48 significant bits, exponent
    within range), and math.fsum returns the correctly rounded value of the exact sum of its
    arguments, whose sign is the sign of the exact sum (0.0 exactly when the sum is 0).
    """
    return math.fsum(float(a) * float(b) for a, b in zip(x_row.tolist(), w_col.tolist())) > 0.0


def sign_bits(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """bits[i, c] = [ (x_i W)_c > 0 ] for the exact real dot product of the stored operands.

    fp64 products of fp32 (or bf16) operands are exact; the fp64 sum is within
    gamma_d * sum|products| of the true value, so any entry whose fp64 magnitude is not above
    twice that bound is recomputed exactly.
    """
    x64 = np.asarray(x, np.float64)
    W64 = np.asarray(W, np.float64)
    z = x64 @ W64
    s = np.abs(x64) @ np.abs(W64)
    n = x64.shape[1]
    gamma = n * U64 / (1.0 - n * U64)
    bits = z > 0.0
    unsure = np.abs(z) <= 2.0 * gamma * s
    for i, c in zip(*np.nonzero(unsure)):
        bits[i, c] = _exact_positive(x64[i], W64[:, c])
    return bits


def pack_bits(bits: np.ndarray) -> np.ndarray:
    """[n, nb] bool -> [n, ceil(nb/32)] uint32; bit c goes to word c // 32, position c % 32."""
    n, nb = bits.shape
    nw = -(-nb // 32)
    words = np.zeros((n, nw), np.uint64)
    for c in range(nb):
        words[:, c // 32] |= bits[:, c].astype(np.uint64) << np.uint64(c % 32)
    return words.astype(np.uint32)


def codes(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    return pack_bits(sign_bits(x, W))


# ----------------------------------------------------------------------------------------------
# §3.1 Eq. (2): Hamming distance
# ----------------------------------------------------------------------------------------------
def hamming(qcode: np.ndarray, kcodes: np.ndarray) -> np.ndarray:
    """D[t] = number of bit positions where qcode and kcodes[t] differ."""
    x = np.bitwise_xor(np.asarray(kcodes, np.uint32), np.asarray(qcode, np.uint32)[None, :])
    bits = np.unpackbits(x.view(np.uint8), axis=1)
    return bits.sum(axis=1).astype(np.int64)


# ----------------------------------------------------------------------------------------------
# §3.3.1 Eq. (3): page bound, and the page threshold
# ----------------------------------------------------------------------------------------------
def page_bounds(qt: np.ndarray, lo: np.ndarray, hi: np.ndarray) -> np.ndarray:
    """U[p] = sum_j max(q~_j lo[p, j], q~_j hi[p, j]) in fp64."""
    q = np.asarray(qt, np.float64)[None, :]
    a = np.asarray(lo, np.float64) * q
    b = np.asarray(hi, np.float64) * q
    return np.maximum(a, b).sum(axis=1)


def keep_count(P: int, rho: float) -> int:
    """Pages kept: ceil(rho * P) (one IEEE double multiply), at least 1, at most P."""
    return min(P, max(1, math.ceil(float(rho) * float(P))))


def select_pages(U: np.ndarray, n_keep: int) -> np.ndarray:
    """The n_keep pages of largest U (ties: lower page index), returned ascending."""
    P = len(U)
    order = np.lexsort((np.arange(P), -np.asarray(U, np.float64)))
    return np.sort(order[:n_keep])


def candidates(pages: np.ndarray, L: int, S: int) -> np.ndarray:
    """All token positions t < L of the given pages, ascending."""
    t = (np.asarray(pages, np.int64)[:, None] * S + np.arange(S)[None, :]).reshape(-1)
    return t[t < L]


def select_tokens(cand: np.ndarray, D: np.ndarray, k: int) -> np.ndarray:
    """The min(k, len(cand)) candidates of smallest (D, t), returned ascending."""
    order = np.lexsort((cand, D))
    return np.sort(cand[order[:min(int(k), len(cand))]])


# ----------------------------------------------------------------------------------------------
# Exact attention over the selected keys (§1, §3.3.2)
# ----------------------------------------------------------------------------------------------
def attend(q: np.ndarray, Ksel: np.ndarray, Vsel: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) weighted sum of V rows, fp64."""
    s = float(scale) * (np.asarray(Ksel, np.float64) @ np.asarray(q, np.float64))
    s = s - s.max()
    p = np.exp(s)
    return (p @ np.asarray(Vsel, np.float64)) / p.sum()


def default_scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))


# ----------------------------------------------------------------------------------------------
# Index build and append (one sequence, one KV head)
# ----------------------------------------------------------------------------------------------
def build_head(K: np.ndarray, L: int, R: np.ndarray, W: np.ndarray, S: int,
               summary: str = "f32"):
    """Page extrema of the rotated keys and the key codes for rows [0, L) of K; with
    summary="bf16" the extrema are the outward-rounded bf16 values."""
    kt = rotate(K[:L], R)
    lo, hi = page_extrema(kt, L, S)
    if summary == "bf16":
        lo, hi = extrema_bf16(lo, hi)
    return lo, hi, codes(K[:L], W)


def append_head(state: dict, k_new: np.ndarray, v_new: np.ndarray, R: np.ndarray,
                W: np.ndarray, S: int) -> None:
    """Write token t = L, extend (or open) page t // S, write its code, then L += 1.

    state: dict with K, V [Lmax, d], lo, hi [Pmax, d], codes [Lmax, nw], L, and optionally
    summary ("f32" or "bf16": the stored extrema rounded outward).
    """
    t = int(state["L"])
    state["K"][t] = k_new
    state["V"][t] = v_new
    kt = rotate(np.asarray(k_new)[None, :], R)[0]
    p = t // S
    if t % S == 0:
        lo, hi = kt, kt
    else:
        lo = np.minimum(state["lo"][p], kt)
        hi = np.maximum(state["hi"][p], kt)
    if state.get("summary", "f32") == "bf16":
        lo, hi = extrema_bf16(lo, hi)
    state["lo"][p] = lo
    state["hi"][p] = hi
    state["codes"][t] = codes(np.asarray(k_new)[None, :], W)[0]
    state["L"] = t + 1


# ----------------------------------------------------------------------------------------------
# One decode step for one (sequence, query head)
# ----------------------------------------------------------------------------------------------
STAGES = ("both", "pages", "codes")


def decode_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, L: int, lo: np.ndarray,
                hi: np.ndarray, kcodes: np.ndarray, R: np.ndarray, W: np.ndarray, S: int,
                rho: float, k: int, scale: float, pages: np.ndarray | None = None,
                stages: str = "both") -> dict:
    """Coarse stage (rotate q, bound every page, keep the top pages), fine stage (query code,
    Hamming distance of every candidate, keep the top-k tokens), then exact attention.

    If `pages` is given, the coarse stage's choice is replaced by it (used to run the fine
    stage on another implementation's page set).

    `stages` selects the variants of the stage-wise ablation (Appendix C, Table 8):
    "both" is the method; "pages" runs the coarse stage alone and attends to every candidate
    (no Hamming ranking, k unused); "codes" runs the fine stage alone over every token (every
    page is a candidate, rho unused; no bound is computed).
    """
    assert stages in STAGES
    P = num_pages(L, S)
    qt = rotate(np.asarray(q)[None, :], R)[0]
    if stages == "codes":
        U, n_keep = None, P
        if pages is None:
            pages = np.arange(P)
    else:
        U = page_bounds(qt, lo[:P], hi[:P])
        n_keep = keep_count(P, rho)
        if pages is None:
            pages = select_pages(U, n_keep)
    cand = candidates(pages, L, S)
    qc = codes(np.asarray(q)[None, :], W)[0]
    if stages == "pages":
        D, sel = None, cand
    else:
        D = hamming(qc, kcodes[cand])
        sel = select_tokens(cand, D, k)
    out = attend(q, K[sel], V[sel], scale)
    return dict(q_rot=qt, q_code=qc, U=U, n_keep=n_keep, pages=np.asarray(pages), cand=cand,
                D=D, sel=sel, out=out)


def decode_group(qs: np.ndarray, K: np.ndarray, V: np.ndarray, L: int, lo: np.ndarray,
                 hi: np.ndarray, kcodes: np.ndarray, R: np.ndarray, W: np.ndarray, S: int,
                 rho: float, k: int, scale: float, pages: np.ndarray | None = None,
                 stages: str = "both") -> dict:
    """One selection shared by the query heads `qs` [G][d] of a KV head (a reading of the
    group-shared variant; the pages select per head): a page's bound is the largest of the
    heads' Eq. (3) bounds, a token's distance the smallest of the heads' Eq. (2) distances; the
    coarse and fine stages then run once, and every head attends to the shared tokens.
    `pages` and `stages` as in decode_head."""
    assert stages in STAGES
    qs = np.asarray(qs)
    P = num_pages(L, S)
    qt = rotate(qs, R)
    if stages == "codes":
        U, n_keep = None, P
        if pages is None:
            pages = np.arange(P)
    else:
        Uh = np.stack([page_bounds(qt[i], lo[:P], hi[:P]) for i in range(len(qs))])
        U = Uh.max(axis=0)
        n_keep = keep_count(P, rho)
        if pages is None:
            pages = select_pages(U, n_keep)
    cand = candidates(pages, L, S)
    qc = codes(qs, W)
    if stages == "pages":
        D, sel = None, cand
    else:
        D = np.stack([hamming(qc[i], kcodes[cand]) for i in range(len(qs))]).min(axis=0)
        sel = select_tokens(cand, D, k)
    outs = np.stack([attend(qs[i], K[sel], V[sel], scale) for i in range(len(qs))])
    return dict(q_rot=qt, q_code=qc, U=U, n_keep=n_keep, pages=np.asarray(pages), cand=cand,
                D=D, sel=sel, out=outs)


def dense_head(q: np.ndarray, K: np.ndarray, V: np.ndarray, L: int, scale: float) -> np.ndarray:
    """Full attention over the first L keys: the baseline HHR is timed against (§4.3, Fig. 7)."""
    return attend(q, K[:L], V[:L], scale)


# ----------------------------------------------------------------------------------------------
# Whole layer (natural layouts: K, V [B][Hkv][Lmax][d], q [B][Hq][d])
# ----------------------------------------------------------------------------------------------
def build_layer(K: np.ndarray, seq_lens, R: np.ndarray, W: np.ndarray, S: int,
                summary: str = "f32") -> dict:
    B, Hkv, Lmax, d = K.shape
    nb = W.shape[2]
    Pmax = num_pages(Lmax, S)
    lo = np.zeros((B, Hkv, Pmax, d), np.float32)
    hi = np.zeros((B, Hkv, Pmax, d), np.float32)
    kc = np.zeros((B, Hkv, Lmax, -(-nb // 32)), np.uint32)
    for b in range(B):
        L = int(seq_lens[b])
        for g in range(Hkv):
            l_, h_, c_ = build_head(K[b, g], L, R[g], W[g], S, summary)
            P = l_.shape[0]
            lo[b, g, :P] = l_
            hi[b, g, :P] = h_
            kc[b, g, :L] = c_
    return dict(lo=lo, hi=hi, codes=kc)


def decode_layer(q: np.ndarray, K: np.ndarray, V: np.ndarray, seq_lens, index: dict,
                 R: np.ndarray, W: np.ndarray, S: int, rho: float, k: int,
                 scale: float | None = None, heads=None, stages: str = "both") -> dict:
    """Run decode_head for every (b, h) (or the listed (b, h) pairs); returns {(b, h): result}."""
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(d)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    res = {}
    for b, h in pairs:
        g = h // G
        res[(b, h)] = decode_head(q[b, h], K[b, g], V[b, g], int(seq_lens[b]),
                                  index["lo"][b, g], index["hi"][b, g], index["codes"][b, g],
                                  R[g], W[g], S, rho, k, scale, stages=stages)
    return res
