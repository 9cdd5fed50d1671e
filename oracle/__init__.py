"""kv4 oracle: TEST INFRASTRUCTURE ONLY.

A ctypes front end to ``kv4_oracle.c``, the plain CPU implementation of the
sparse-MLA-over-NVFP4 hot path (quantized row write, dedup compaction, page
translation, dequantizing gather, softmax attention, (o, lse) merge).  Only
the tests, the smoke check and the benchmark's CPU baseline use it; the HIP
library never imports, links or calls anything here.

Sources are the web pages cited in ``kv4_oracle.c``'s header: the README
"60+ inference optimizations & kernels" (section "4-bit KV cache": the 352-byte
NVFP4 row, E2M1 values, one E4M3 scale per 16 values; section "Parallelism and
disaggregation": (o, lse) merge) and the sgl-amd-mono GLM-5.3 monokernel PR
(section "Modifications": 64-token page table and its stride, exact top-2048).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kv4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ERR_PAGE = 1
ERR_SLOT = 2


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off",
                               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


class _AttnArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("n_rows", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_latent", ctypes.c_int32), ("n_rope", ctypes.c_int32),
        ("pool", ctypes.c_void_p), ("n_slots", ctypes.c_int64),
        ("page_table", ctypes.c_void_p), ("pt_row_stride", ctypes.c_int64),
        ("pt_n_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("row_req", ctypes.c_void_p),
        ("topk", ctypes.c_void_p), ("topk_row_stride", ctypes.c_int64), ("k", ctypes.c_int32),
        ("sm_scale", ctypes.c_double),
    ]


def _load(path: str):
    L = ctypes.CDLL(path)
    u8, i32, i64, f32, dbl, vp = (ctypes.c_uint8, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_double, ctypes.c_void_p)
    L.o_e4m3_value.argtypes, L.o_e4m3_value.restype = [u8], dbl
    L.o_e2m1_value.argtypes, L.o_e2m1_value.restype = [u8], dbl
    L.o_e4m3_encode.argtypes, L.o_e4m3_encode.restype = [f32], u8
    L.o_e2m1_encode.argtypes, L.o_e2m1_encode.restype = [f32], u8
    L.o_row_bytes.argtypes, L.o_row_bytes.restype = [ctypes.c_int, ctypes.c_int], ctypes.c_int
    L.o_quantize_row.argtypes, L.o_quantize_row.restype = [vp, ctypes.c_int, ctypes.c_int, vp], None
    L.o_dequantize_row.argtypes, L.o_dequantize_row.restype = [vp, ctypes.c_int, ctypes.c_int, vp], None
    L.o_quant_write.argtypes = [vp, i64, vp, i64, ctypes.c_int, ctypes.c_int, vp, i64, vp]
    L.o_quant_write.restype = None
    L.o_quantize_row_mse.argtypes, L.o_quantize_row_mse.restype = [vp, ctypes.c_int, ctypes.c_int, vp], None
    L.o_quant_write_mse.argtypes = [vp, i64, vp, i64, ctypes.c_int, ctypes.c_int, vp, i64, vp]
    L.o_quant_write_mse.restype = None
    L.o_dedup_compact.argtypes, L.o_dedup_compact.restype = [vp, i64, i32, i64, vp, vp], None
    L.o_translate.argtypes, L.o_translate.restype = [i32, vp, i32, i32, i64, vp], i64
    L.o_sparse_mla.argtypes, L.o_sparse_mla.restype = [ctypes.POINTER(_AttnArgs), vp, vp, vp, vp], None
    L.o_global_compact.argtypes = [vp, i32, i32, i64, vp, i64, i32, i32, i32, vp, vp, i64, ctypes.c_int, vp, vp, vp]
    L.o_global_compact.restype = i64
    L.o_merge_states.argtypes = [vp, vp, ctypes.c_int, i64, ctypes.c_int, vp, vp]
    L.o_merge_states.restype = None
    L.o_num_threads.argtypes, L.o_num_threads.restype = [], ctypes.c_int
    L.o_set_num_threads.argtypes, L.o_set_num_threads.restype = [ctypes.c_int], None
    return L


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = _load(_LIB)
    return _lib


@contextlib.contextmanager
def using_library(path: str):
    """Run the wrappers against another build of the oracle source (the
    mutation tests plant mistakes in a copy and check that the pins fail)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return lib().o_num_threads()


def set_num_threads(n: int) -> None:
    lib().o_set_num_threads(int(n))


# ------------------------------------------------------------------ codecs
def e4m3_value(code: int) -> float:
    return lib().o_e4m3_value(int(code) & 0xFF)


def e2m1_value(code: int) -> float:
    return lib().o_e2m1_value(int(code) & 0xF)


def e4m3_encode(x: float) -> int:
    return lib().o_e4m3_encode(float(np.float32(x)))


def e2m1_encode(y: float) -> int:
    return lib().o_e2m1_encode(float(np.float32(y)))


def row_bytes(n_latent: int = 512, n_rope: int = 64) -> int:
    return lib().o_row_bytes(n_latent, n_rope)


def quantize_row(x, n_latent: int = 512, n_rope: int = 64, mse: bool = False) -> np.ndarray:
    """One row's bytes; mse=True takes the MSE-searched block scales."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.shape == (n_latent + n_rope,)
    out = np.zeros(row_bytes(n_latent, n_rope), dtype=np.uint8)
    (lib().o_quantize_row_mse if mse else lib().o_quantize_row)(_ptr(x), n_latent, n_rope, _ptr(out))
    return out


def dequantize_row(row, n_latent: int = 512, n_rope: int = 64) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    assert row.shape == (row_bytes(n_latent, n_rope),)
    out = np.zeros(n_latent + n_rope, dtype=np.float64)
    lib().o_dequantize_row(_ptr(row), n_latent, n_rope, _ptr(out))
    return out


def dequantize_rows(rows, n_latent: int = 512, n_rope: int = 64) -> np.ndarray:
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    return np.stack([dequantize_row(r, n_latent, n_rope) for r in rows]) if len(rows) else \
        np.zeros((0, n_latent + n_rope))


# ----------------------------------------------------------- quantized write
def quant_write(kv, slots, pool, n_latent: int = 512, n_rope: int = 64, mse: bool = False) -> int:
    """Quantize kv[n] into pool[slots[n]] in place; returns the error bits.
    mse=True takes the MSE-searched block scales."""
    kv = np.ascontiguousarray(kv, dtype=np.float32)
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    assert pool.dtype == np.uint8 and pool.flags.c_contiguous
    rb = row_bytes(n_latent, n_rope)
    assert pool.ndim == 2 and pool.shape[1] == rb
    assert kv.ndim == 2 and kv.shape[1] == n_latent + n_rope and kv.shape[0] == slots.shape[0]
    err = np.zeros(1, dtype=np.uint32)
    (lib().o_quant_write_mse if mse else lib().o_quant_write)(_ptr(kv), kv.shape[1], _ptr(slots), kv.shape[0],
                                                              n_latent, n_rope, _ptr(pool), pool.shape[0], _ptr(err))
    return int(err[0])


# ----------------------------------------------------------------- dedup
def dedup_compact(idx):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n, k = idx.shape
    out = np.empty((n, k), dtype=np.int32)
    cnt = np.empty(n, dtype=np.int32)
    lib().o_dedup_compact(_ptr(idx), n, k, k, _ptr(out), _ptr(cnt))
    return out, cnt


# --------------------------------------------------------- page translate
def translate(pos: int, pt_row=None, page_size: int = 64, n_slots: int = 1 << 62):
    """Returns (slot or -1, error bits)."""
    err = np.zeros(1, dtype=np.uint32)
    if pt_row is not None:
        pt_row = np.ascontiguousarray(pt_row, dtype=np.int32)
    s = lib().o_translate(int(pos), _ptr(pt_row), 0 if pt_row is None else pt_row.shape[0],
                          page_size, n_slots, _ptr(err))
    return int(s), int(err[0])


# ------------------------------------------------- global dedup across lists
def global_compact(topk, pool, page_table=None, row_req=None, page_size: int = 64):
    """The compacted pool: (cpool [|U|, row_bytes] u8, out_idx [R, k] int32, |U|, err bits).
    U = the distinct valid translated slots of all lists, increasing; out_idx holds
    each entry's index in U (-1 when skipped)."""
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    pool = np.ascontiguousarray(pool, dtype=np.uint8)
    R, k = topk.shape
    rb = pool.shape[1]
    if page_table is not None:
        page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    if row_req is not None:
        row_req = np.ascontiguousarray(row_req, dtype=np.int32)
    cap = min(pool.shape[0], R * k)
    cpool = np.zeros((max(cap, 1), rb), dtype=np.uint8)
    out_idx = np.zeros((R, k), dtype=np.int32)
    err = np.zeros(1, dtype=np.uint32)
    n = lib().o_global_compact(_ptr(topk), R, k, k, _ptr(page_table),
                               0 if page_table is None else page_table.shape[1],
                               0 if page_table is None else page_table.shape[0],
                               0 if page_table is None else page_table.shape[1], page_size, _ptr(row_req),
                               _ptr(pool), pool.shape[0], rb, _ptr(cpool), _ptr(out_idx), _ptr(err))
    return cpool[:n], out_idx, int(n), int(err[0])


# --------------------------------------------------------------- attention
def sparse_mla(q, pool, topk, sm_scale, page_table=None, row_req=None, page_size: int = 64,
               n_latent: int = 512, n_rope: int = 64, want_probs: bool = False):
    """q: [R, H, n_latent + n_rope] (float32; widen bf16 first); pool: [n_slots, row_bytes] u8;
    topk: [R, k] int32; page_table: [n_req, n_pages] int32 or None.
    Returns (out [R, H, n_latent] f64, lse [R, H] f64, err bits[, probs [R, H, k]])."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    pool = np.ascontiguousarray(pool, dtype=np.uint8)
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    R, H, D = q.shape
    assert D == n_latent + n_rope and topk.shape[0] == R
    assert pool.ndim == 2 and pool.shape[1] == row_bytes(n_latent, n_rope)
    if page_table is not None:
        page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    if row_req is not None:
        row_req = np.ascontiguousarray(row_req, dtype=np.int32)
    a = _AttnArgs()
    a.q = q.ctypes.data
    a.q_row_stride, a.q_head_stride = H * D, D
    a.n_rows, a.n_heads, a.n_latent, a.n_rope = R, H, n_latent, n_rope
    a.pool, a.n_slots = pool.ctypes.data, pool.shape[0]
    a.page_table = None if page_table is None else page_table.ctypes.data
    a.pt_row_stride = 0 if page_table is None else page_table.shape[1]
    a.pt_n_pages = 0 if page_table is None else page_table.shape[1]
    a.page_size = page_size
    a.row_req = None if row_req is None else row_req.ctypes.data
    a.topk, a.topk_row_stride, a.k = topk.ctypes.data, topk.shape[1], topk.shape[1]
    a.sm_scale = float(np.float32(sm_scale))
    out = np.zeros((R, H, n_latent), dtype=np.float64)
    lse = np.zeros((R, H), dtype=np.float64)
    probs = np.zeros((R, H, topk.shape[1]), dtype=np.float64) if want_probs else None
    err = np.zeros(1, dtype=np.uint32)
    lib().o_sparse_mla(ctypes.byref(a), _ptr(out), _ptr(lse), _ptr(probs), _ptr(err))
    if want_probs:
        return out, lse, int(err[0]), probs
    return out, lse, int(err[0])


def merge_states(part_o, part_lse):
    """part_o: [S, T, dim], part_lse: [S, T] -> (o [T, dim], lse [T])."""
    part_o = np.ascontiguousarray(part_o, dtype=np.float64)
    part_lse = np.ascontiguousarray(part_lse, dtype=np.float64)
    S, T, dim = part_o.shape
    out = np.zeros((T, dim), dtype=np.float64)
    lse = np.zeros(T, dtype=np.float64)
    lib().o_merge_states(_ptr(part_o), _ptr(part_lse), S, T, dim, _ptr(out), _ptr(lse))
    return out, lse
