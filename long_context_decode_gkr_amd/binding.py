"""ctypes binding of libhhr.so (the C ABI in include/hhr.h).

Only argument marshalling lives here: every step of the method runs in the library's HIP
kernels. PyTorch supplies device memory and the stream. Loading fails loudly when the library
has not been built (`python -m long_context_decode_gkr_amd.build`).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhhr.so")

HHR_F32, HHR_BF16 = 0, 1
HHR_MAX_PAGES = 16384
HHR_STAGES_BOTH, HHR_STAGES_PAGES_ONLY, HHR_STAGES_CODES_ONLY = 0, 1, 2
STAGES = {"both": HHR_STAGES_BOTH, "pages": HHR_STAGES_PAGES_ONLY, "codes": HHR_STAGES_CODES_ONLY}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape or type",
          3: "size exceeds a documented maximum", 4: "workspace too small or misaligned",
          5: "HIP launch or runtime error"}

# Every exported symbol of include/hhr.h.
EXPORTS = ("hhr_build_pages", "hhr_build_pages_fp64", "hhr_append", "hhr_decode_workspace_bytes",
           "hhr_decode", "hhr_append_decode", "hhr_decode_scratch", "hhr_dense_workspace_bytes",
           "hhr_dense_decode", "hhr_read_probe_blocks", "hhr_read_probe", "hhr_status_string")
HHR_SCRATCH_BYTES = 16 * 1024 * 1024


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("hash_bits", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("summary_dtype", ctypes.c_int32)]


class Params(ctypes.Structure):
    _fields_ = [("page_keep_ratio", ctypes.c_double), ("token_budget", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("stages", ctypes.c_int32),
                ("group_shared", ctypes.c_int32)]


class CacheStruct(ctypes.Structure):
    _fields_ = [("K", ctypes.c_void_p), ("V", ctypes.c_void_p), ("page_min", ctypes.c_void_p),
                ("page_max", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("append_ticket", ctypes.c_void_p)]


class DebugStruct(ctypes.Structure):
    _fields_ = [("q_rot", ctypes.c_void_p), ("q_code", ctypes.c_void_p),
                ("bounds", ctypes.c_void_p), ("page_ids", ctypes.c_void_p),
                ("page_count", ctypes.c_void_p), ("dist", ctypes.c_void_p),
                ("token_idx", ctypes.c_void_p), ("token_count", ctypes.c_void_p),
                ("kernel_events", ctypes.c_void_p)]


class HHRError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({STATUS.get(status, 'unknown')})")
        self.status = status


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libhhr.so; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m long_context_decode_gkr_amd.build`")
    # torch first: the library then binds to the HIP runtime torch already loaded (same
    # SONAME), so device pointers and streams are shared by a single runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.hhr_build_pages.argtypes = [P(Dims), P(CacheStruct), vp, vp, vp]
    lib.hhr_build_pages_fp64.argtypes = [P(Dims), P(CacheStruct), vp, vp, vp]
    lib.hhr_append.argtypes = [P(Dims), P(CacheStruct), vp, vp, vp, vp, vp]
    lib.hhr_decode_workspace_bytes.argtypes = [P(Dims), P(Params)]
    lib.hhr_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.hhr_decode.argtypes = [P(Dims), P(Params), P(CacheStruct), vp, vp, vp, vp, ctypes.c_size_t,
                               vp, P(DebugStruct), vp]
    lib.hhr_append_decode.argtypes = [P(Dims), P(Params), P(CacheStruct), vp, vp, vp, vp, vp, vp,
                                      ctypes.c_size_t, vp, P(DebugStruct), vp]
    lib.hhr_decode_scratch.argtypes = [P(Dims), P(Params), P(CacheStruct), vp, vp, vp, vp,
                                       P(DebugStruct), vp]
    lib.hhr_dense_workspace_bytes.argtypes = [P(Dims)]
    lib.hhr_dense_workspace_bytes.restype = ctypes.c_size_t
    lib.hhr_dense_decode.argtypes = [P(Dims), P(CacheStruct), vp, ctypes.c_float, vp,
                                     ctypes.c_size_t, vp, P(DebugStruct), vp]
    lib.hhr_read_probe_blocks.argtypes = [ctypes.c_size_t]
    lib.hhr_read_probe_blocks.restype = ctypes.c_size_t
    lib.hhr_read_probe.argtypes = [vp, ctypes.c_size_t, vp, vp]
    lib.hhr_status_string.argtypes = [ctypes.c_int]
    lib.hhr_status_string.restype = ctypes.c_char_p
    for fn in ("hhr_build_pages", "hhr_build_pages_fp64", "hhr_append", "hhr_decode",
               "hhr_append_decode", "hhr_decode_scratch", "hhr_dense_decode", "hhr_read_probe"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise HHRError(fn, status)


# ---- raw entry points (pointers as ints; None = NULL) -----------------------------------------
def hhr_build_pages(dims: Dims, cache: CacheStruct, R: int, W: int, stream: int = 0,
                    method: str = "auto") -> None:
    fn = "hhr_build_pages" if method == "auto" else "hhr_build_pages_fp64"
    _check(fn, getattr(load(), fn)(ctypes.byref(dims), ctypes.byref(cache), R, W, stream))


def hhr_append(dims: Dims, cache: CacheStruct, k_new: int, v_new: int, R: int, W: int,
               stream: int = 0) -> None:
    _check("hhr_append", load().hhr_append(ctypes.byref(dims), ctypes.byref(cache), k_new, v_new,
                                           R, W, stream))


def hhr_decode_workspace_bytes(dims: Dims, params: Params) -> int:
    return int(load().hhr_decode_workspace_bytes(ctypes.byref(dims), ctypes.byref(params)))


def hhr_decode(dims: Dims, params: Params, cache: CacheStruct, q: int, R: int, W: int, ws: int,
               ws_bytes: int, out: int, dbg: Optional[DebugStruct] = None, stream: int = 0) -> None:
    _check("hhr_decode", load().hhr_decode(
        ctypes.byref(dims), ctypes.byref(params), ctypes.byref(cache), q, R, W, ws, ws_bytes, out,
        ctypes.byref(dbg) if dbg is not None else None, stream))


def hhr_append_decode(dims: Dims, params: Params, cache: CacheStruct, k_new: int, v_new: int,
                      q: int, R: int, W: int, ws: int, ws_bytes: int, out: int,
                      dbg: Optional[DebugStruct] = None, stream: int = 0) -> None:
    _check("hhr_append_decode", load().hhr_append_decode(
        ctypes.byref(dims), ctypes.byref(params), ctypes.byref(cache), k_new, v_new, q, R, W, ws,
        ws_bytes, out, ctypes.byref(dbg) if dbg is not None else None, stream))


def hhr_decode_scratch(dims: Dims, params: Params, cache: CacheStruct, q: int, R: int, W: int,
                       out: int, dbg: Optional[DebugStruct] = None, stream: int = 0) -> None:
    _check("hhr_decode_scratch", load().hhr_decode_scratch(
        ctypes.byref(dims), ctypes.byref(params), ctypes.byref(cache), q, R, W, out,
        ctypes.byref(dbg) if dbg is not None else None, stream))


def hhr_read_probe_blocks(nbytes: int) -> int:
    return int(load().hhr_read_probe_blocks(nbytes))


def hhr_read_probe(src: int, nbytes: int, partial: int, stream: int = 0) -> None:
    _check("hhr_read_probe", load().hhr_read_probe(src, nbytes, partial, stream))


def hhr_dense_workspace_bytes(dims: Dims) -> int:
    return int(load().hhr_dense_workspace_bytes(ctypes.byref(dims)))


def hhr_dense_decode(dims: Dims, cache: CacheStruct, q: int, softmax_scale: float, ws: int,
                     ws_bytes: int, out: int, dbg: Optional[DebugStruct] = None,
                     stream: int = 0) -> None:
    _check("hhr_dense_decode", load().hhr_dense_decode(
        ctypes.byref(dims), ctypes.byref(cache), q, softmax_scale, ws, ws_bytes, out,
        ctypes.byref(dbg) if dbg is not None else None, stream))


def hhr_status_string(status: int) -> str:
    return load().hhr_status_string(status).decode()


# ---- torch-owned buffers ----------------------------------------------------------------------
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_dims(batch, num_q_heads, num_kv_heads, page_size, hash_bits, max_seq_len,
              kv_dtype=HHR_BF16, q_dtype=None, head_dim=128, summary_dtype=HHR_F32) -> Dims:
    return Dims(batch, num_q_heads, num_kv_heads, head_dim, page_size, hash_bits, max_seq_len,
                kv_dtype, kv_dtype if q_dtype is None else q_dtype, summary_dtype)


class Cache:
    """Device buffers of one layer's KV cache and its index, allocated through torch."""

    def __init__(self, dims: Dims, device="cuda"):
        import torch
        self.dims = dims
        B, Hkv, L, d = dims.batch, dims.num_kv_heads, dims.max_seq_len, dims.head_dim
        P = L // dims.page_size
        kvt = torch.bfloat16 if dims.kv_dtype == HHR_BF16 else torch.float32
        self.K = torch.zeros((B, Hkv, L, d), dtype=kvt, device=device)
        self.V = torch.zeros((B, Hkv, L, d), dtype=kvt, device=device)
        st = torch.bfloat16 if dims.summary_dtype == HHR_BF16 else torch.float32
        self.page_min = torch.zeros((B, Hkv, d, P), dtype=st, device=device)
        self.page_max = torch.zeros((B, Hkv, d, P), dtype=st, device=device)
        self.codes = torch.zeros((B, Hkv, L, dims.hash_bits // 32), dtype=torch.int32, device=device)
        self.seq_lens = torch.zeros((B,), dtype=torch.int32, device=device)
        self.append_ticket = torch.zeros((B,), dtype=torch.int32, device=device)

    def struct(self) -> CacheStruct:
        return CacheStruct(_ptr(self.K), _ptr(self.V), _ptr(self.page_min), _ptr(self.page_max),
                           _ptr(self.codes), _ptr(self.seq_lens), _ptr(self.append_ticket))


def index_capacity(dims: Dims, keep_ratio: float, token_budget: int, stages: str = "both") -> int:
    """Entries per (b, h) of the selected-token list (hhr_debug.token_idx): the token budget
    clamped to max_seq_len, or, with the coarse stage alone, every token of the largest kept page
    set, min(max(1, ceil(rho * Pmax)) * page_size, max_seq_len)."""
    import math
    if STAGES[stages] == HHR_STAGES_PAGES_ONLY:
        keep = max(1, math.ceil(keep_ratio * (dims.max_seq_len // dims.page_size)))
        return min(keep * dims.page_size, dims.max_seq_len)
    return min(token_budget, dims.max_seq_len)


class Debug:
    """Optional side outputs of hhr_decode (all allocated)."""

    def __init__(self, dims: Dims, token_budget: int, keep_ratio: float = 1.0,
                 stages: str = "both", device="cuda"):
        import torch
        B, H, d = dims.batch, dims.num_q_heads, dims.head_dim
        P = dims.max_seq_len // dims.page_size
        k = index_capacity(dims, keep_ratio, token_budget, stages)
        i32 = torch.int32
        self.q_rot = torch.zeros((B, H, d), dtype=torch.float32, device=device)
        self.q_code = torch.zeros((B, H, dims.hash_bits // 32), dtype=i32, device=device)
        self.bounds = torch.zeros((B, H, P), dtype=torch.float32, device=device)
        self.page_ids = torch.full((B, H, P), -1, dtype=i32, device=device)
        self.page_count = torch.zeros((B, H), dtype=i32, device=device)
        self.dist = torch.zeros((B, H, dims.max_seq_len), dtype=torch.int16, device=device)
        self.token_idx = torch.full((B, H, k), -1, dtype=i32, device=device)
        self.token_count = torch.zeros((B, H), dtype=i32, device=device)

    def struct(self) -> DebugStruct:
        return DebugStruct(_ptr(self.q_rot), _ptr(self.q_code), _ptr(self.bounds),
                           _ptr(self.page_ids), _ptr(self.page_count), _ptr(self.dist),
                           _ptr(self.token_idx), _ptr(self.token_count), None)


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


class Decoder:
    """Holds the workspace for hhr_decode at fixed shapes and budgets."""

    def __init__(self, dims: Dims, keep_ratio: float, token_budget: int, softmax_scale: float = 0.0,
                 device="cuda", stages: str = "both", group_shared: bool = False):
        import torch
        self.dims = dims
        self.params = Params(keep_ratio, token_budget, softmax_scale, STAGES[stages],
                             int(group_shared))
        self.ws_bytes = hhr_decode_workspace_bytes(dims, self.params)
        if self.ws_bytes == 0:
            raise HHRError("hhr_decode_workspace_bytes", 1)
        self.ws = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=device)

    def __call__(self, cache: Cache, q, R, W, out, dbg: Optional[Debug] = None,
                 stream: Optional[int] = None, k_new=None, v_new=None) -> None:
        """hhr_decode, or hhr_append_decode when k_new / v_new are given."""
        st = current_stream() if stream is None else stream
        d = dbg.struct() if dbg is not None else None
        if k_new is None:
            hhr_decode(self.dims, self.params, cache.struct(), _ptr(q), _ptr(R), _ptr(W),
                       _ptr(self.ws), self.ws_bytes, _ptr(out), d, st)
        else:
            hhr_append_decode(self.dims, self.params, cache.struct(), _ptr(k_new), _ptr(v_new),
                              _ptr(q), _ptr(R), _ptr(W), _ptr(self.ws), self.ws_bytes, _ptr(out),
                              d, st)


class DenseDecoder:
    """Holds the workspace of hhr_dense_decode (full attention over every cached token)."""

    def __init__(self, dims: Dims, softmax_scale: float = 0.0, device="cuda"):
        import torch
        self.dims = dims
        self.softmax_scale = softmax_scale
        self.ws_bytes = hhr_dense_workspace_bytes(dims)
        if self.ws_bytes == 0:
            raise HHRError("hhr_dense_workspace_bytes", 1)
        self.ws = torch.empty((self.ws_bytes,), dtype=torch.uint8, device=device)

    def __call__(self, cache: Cache, q, out, stream: Optional[int] = None) -> None:
        st = current_stream() if stream is None else stream
        hhr_dense_decode(self.dims, cache.struct(), _ptr(q), self.softmax_scale, _ptr(self.ws),
                         self.ws_bytes, _ptr(out), None, st)


def build_pages(cache: Cache, R, W, method: str = "auto", stream: Optional[int] = None) -> None:
    hhr_build_pages(cache.dims, cache.struct(), _ptr(R), _ptr(W),
                    current_stream() if stream is None else stream, method)


def append(cache: Cache, k_new, v_new, R, W, stream: Optional[int] = None) -> None:
    hhr_append(cache.dims, cache.struct(), _ptr(k_new), _ptr(v_new), _ptr(R), _ptr(W),
               current_stream() if stream is None else stream)


# ---- raw HIP events (the runtime torch loaded) ------------------------------------------------
class HipEvents:
    """A pool of hipEvent_t handles for per-kernel timing on the decode stream."""

    def __init__(self, n: int):
        import torch  # noqa: F401  (loads the runtime)
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles[i] = h.value

    def address(self, i: int) -> int:
        """Address of handles[i] (a hipEvent_t* for hhr_debug.kernel_events)."""
        return ctypes.addressof(self.handles) + i * ctypes.sizeof(ctypes.c_void_p)

    def record(self, i: int, stream: int) -> None:
        if self.rt.hipEventRecord(self.handles[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self) -> None:
        for h in self.handles:
            self.rt.hipEventDestroy(h)
