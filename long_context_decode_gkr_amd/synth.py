"""Seeded synthetic inputs for the HHR decode path.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests. It holds no step of the method itself (no rotation of the index, no
page bound, no hashing, no selection, no attention): it only draws keys,
values, queries, rotation and projection stand-ins and sequence lengths.

Workload shapes follow "HHR: Hierarchical Hash Retrieval for Efficient LLM
Generation", Appendix A, Table 3 (Llama-3.1-8B: 32 attention heads, 8 KV
heads, hidden 4096, so head dim 128, context up to 131072) and §4.3 (context
lengths 16K-128K). Default budgets: candidate budget 30 %, 128-bit codes
(Appendix A). The benchmark datasets of §4.1 are not available; these seeded
draws stand in for them.

Every array is drawn from its own counter-keyed stream
``PCG64(SeedSequence([cfg_id, b, g, purpose, layer]))`` so a slice of a large
workload can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

PURPOSE = {"K": 0, "V": 1, "q": 2, "outl": 3, "plant": 4, "R": 5, "W": 6,
           "lens": 7, "app": 8}


def rng(cfg_id: int, b: int, g: int, purpose: str, layer: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(cfg_id), int(b), int(g), PURPOSE[purpose], int(layer)])))


@dataclasses.dataclass(frozen=True)
class Config:
    cfg_id: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int            # fixed length, or the upper end when lens_range is set
    page_size: int
    hash_bits: int
    keep_ratio: float
    token_budget: int
    dtype: str              # "f32" or "bf16" for q, K and V
    key_dist: str           # "outlier" (N(0,1), 4 channels x10) or "lognormal"
    lens_range: Optional[tuple] = None   # (lo, hi) inclusive: per-sequence uniform lengths
    append: bool = False
    n_plant: int = 32

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def lengths(self) -> List[int]:
        if self.lens_range is None:
            return [self.seq_len] * self.batch
        lo, hi = self.lens_range
        r = rng(self.cfg_id, 0, 0, "lens")
        return [int(x) for x in r.integers(lo, hi, endpoint=True, size=self.batch)]

    def scaled(self, seq_len: int, batch: Optional[int] = None, lens: Optional[List[int]] = None,
               **kw) -> "Config":
        """Same head shape and budgets ratio, shorter context (for parity tests)."""
        d = dataclasses.asdict(self)
        d.update(seq_len=seq_len, lens_range=None)
        if batch is not None:
            d["batch"] = batch
        d.update(kw)
        c = Config(**d)
        if lens is not None:
            object.__setattr__(c, "_lens", list(lens))
        return c


def _lengths(cfg: Config) -> List[int]:
    return list(getattr(cfg, "_lens", None) or cfg.lengths())


CONFIGS = {
    1: Config(1, "single-head d128 fp32, 4096 keys", 1, 1, 1, 128, 4096, 16, 128, 0.25, 256,
              "f32", "outlier"),
    2: Config(2, "llama3.1-8b layer, 32K ctx", 1, 32, 8, 128, 32768, 16, 128, 1.0 / 8, 2048,
              "bf16", "outlier"),
    3: Config(3, "llama3.1-8b layer, 128K ctx, append+decode", 1, 32, 8, 128, 131072, 16, 128,
              1.0 / 16, 4096, "bf16", "outlier", append=True),
    4: Config(4, "llama3.1-8b layer, 8 seqs len U[8K,32K]", 8, 32, 8, 128, 32768, 16, 128, 0.30,
              2048, "bf16", "outlier", lens_range=(8192, 32768)),
    5: Config(5, "qwen3-8b layer, B4 x 64K, page 32, 256-bit codes", 4, 32, 8, 128, 65536, 32,
              256, 1.0 / 8, 4096, "bf16", "lognormal"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32 holding them."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def rotation(cfg_id: int, g: int, d: int, layer: int = 0) -> np.ndarray:
    """Seeded Haar-random orthogonal d x d matrix (QR of a Gaussian, sign-fixed), stored fp32."""
    a = rng(cfg_id, 0, g, "R", layer).standard_normal((d, d))
    q, r = np.linalg.qr(a)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


def projection(cfg_id: int, g: int, d: int, nb: int, layer: int = 0) -> np.ndarray:
    """Seeded Gaussian d x nb hash projection, stored fp32."""
    return rng(cfg_id, 0, g, "W", layer).standard_normal((d, nb), dtype=np.float32)


def _background_keys(cfg: Config, b: int, g: int, L: int, layer: int) -> np.ndarray:
    d = cfg.head_dim
    k = rng(cfg.cfg_id, b, g, "K", layer).standard_normal((L, d), dtype=np.float32)
    ro = rng(cfg.cfg_id, 0, g, "outl", layer)
    if cfg.key_dist == "outlier":
        ch = ro.choice(d, 4, replace=False)
        k[:, ch] *= np.float32(10.0)
    elif cfg.key_dist == "lognormal":
        s = np.exp(ro.standard_normal(d)).astype(np.float32)
        k *= s[None, :]
    else:
        raise ValueError(cfg.key_dist)
    return k


def make_layer(cfg: Config, max_seq_len: Optional[int] = None, layer: int = 0,
               lens: Optional[List[int]] = None) -> dict:
    """Draw one decode layer: K, V [B][Hkv][Lmax][d], q [B][Hq][d], R, W, seq_lens.

    Values are float32 arrays holding exactly the stored values (bf16-representable for bf16
    configs). Rows at or beyond a sequence's length are zero. `planted` [B][Hq][n_plant] holds
    the planted positions of each query head (-1 where a short sequence has fewer).
    Planted keys: for each query head, n_plant background keys at distinct positions are moved
    along q so that their logit is the background mean + 4 std of that head's logits.
    """
    B, Hq, Hkv, d, G = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.group
    lens = list(lens) if lens is not None else _lengths(cfg)
    S = cfg.page_size
    Lmax = max_seq_len or max(lens)
    Lmax = -(-Lmax // (4 * S)) * (4 * S)   # capacity in whole groups of four pages
    assert max(lens) <= Lmax
    K = np.zeros((B, Hkv, Lmax, d), np.float32)
    V = np.zeros((B, Hkv, Lmax, d), np.float32)
    q = np.zeros((B, Hq, d), np.float32)
    planted = np.full((B, Hq, cfg.n_plant), -1, np.int64)   # positions, -1 where none
    for b in range(B):
        L = lens[b]
        for h in range(Hq):
            q[b, h] = _storage(rng(cfg.cfg_id, b, h, "q", layer).standard_normal(d, dtype=np.float32),
                               cfg.dtype)
        for g in range(Hkv):
            k = _background_keys(cfg, b, g, L, layer)
            n_plant = min(cfg.n_plant, L // G)
            if n_plant > 0:
                pos = rng(cfg.cfg_id, b, g, "plant", layer).choice(L, n_plant * G, replace=False)
                pos = pos.reshape(G, n_plant)
                k64 = k.astype(np.float64)
                for i in range(G):
                    qh = q[b, g * G + i].astype(np.float64)
                    logits = k64 @ qh
                    mu, sd = logits.mean(), logits.std()
                    sel = pos[i]
                    planted[b, g * G + i, :n_plant] = sel
                    target = mu + 4.0 * sd
                    shift = (target - logits[sel]) / float(qh @ qh)
                    k[sel] = (k64[sel] + shift[:, None] * qh[None, :]).astype(np.float32)
            K[b, g, :L] = _storage(k, cfg.dtype)
            V[b, g, :L] = _storage(rng(cfg.cfg_id, b, g, "V", layer).standard_normal((L, d), dtype=np.float32),
                                   cfg.dtype)
    R = np.stack([rotation(cfg.cfg_id, g, d, layer) for g in range(Hkv)])
    W = np.stack([projection(cfg.cfg_id, g, d, cfg.hash_bits, layer) for g in range(Hkv)])
    return dict(K=K, V=V, q=q, R=R, W=W, seq_lens=np.asarray(lens, np.int32), max_seq_len=Lmax,
                planted=planted)


def layer_inputs(cfg: Config, layer: int) -> dict:
    """The per-layer inputs of make_layer alone: q [B][Hq][d] and the rotation and projection
    stand-ins R, W of layer `layer` (the same draws make_layer(cfg, layer=layer) makes)."""
    B, Hq, Hkv, d = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    q = np.zeros((B, Hq, d), np.float32)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = _storage(rng(cfg.cfg_id, b, h, "q", layer).standard_normal(d, dtype=np.float32),
                               cfg.dtype)
    R = np.stack([rotation(cfg.cfg_id, g, d, layer) for g in range(Hkv)])
    W = np.stack([projection(cfg.cfg_id, g, d, cfg.hash_bits, layer) for g in range(Hkv)])
    return dict(q=q, R=R, W=W)


def append_tokens(cfg: Config, n: int, layer: int = 0) -> tuple:
    """n fresh (k, v) tokens per (b, kv-head), same background key distribution; [n][B][Hkv][d]."""
    B, Hkv, d = cfg.batch, cfg.num_kv_heads, cfg.head_dim
    kn = np.zeros((n, B, Hkv, d), np.float32)
    vn = np.zeros((n, B, Hkv, d), np.float32)
    for b in range(B):
        for g in range(Hkv):
            r = rng(cfg.cfg_id, b, g, "app", layer)
            k = r.standard_normal((n, d), dtype=np.float32)
            ro = rng(cfg.cfg_id, 0, g, "outl", layer)
            if cfg.key_dist == "outlier":
                ch = ro.choice(d, 4, replace=False)
                k[:, ch] *= np.float32(10.0)
            else:
                k *= np.exp(ro.standard_normal(d)).astype(np.float32)[None, :]
            kn[:, b, g] = _storage(k, cfg.dtype)
            vn[:, b, g] = _storage(r.standard_normal((n, d), dtype=np.float32), cfg.dtype)
    return kn, vn


__all__ = ["Config", "CONFIGS", "make_layer", "layer_inputs", "append_tokens", "rotation",
           "projection", "round_to_bf16", "rng"]
