"""bit_kv_cache_kv4_amd: sparse MLA attention over a 4-bit NVFP4 KV cache on
AMD Instinct MI355X (gfx950).

A thin ctypes binding over libkv4.so, whose C ABI is include/kv4.h.  The
functions here have the ABI's names and only marshal arguments (torch tensors
to device pointers, strides and the current HIP stream); every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or fails to load, every call raises.

Row format and operations: README "60+ inference optimizations & kernels",
section "4-bit KV cache" (352-byte NVFP4 rows: E2M1 values, one E4M3 scale per
16, FP8 rope; quantized write, dequantizing gather, dedup compaction) and
section "AMD MI355X" (HIP sparse MLA decode, split-K decode, prefill).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Kv4Error", "ROW_BYTES", "ROW_BYTES_ROPE_FREE", "LATENT", "ROPE", "DIM", "ERRBIT_PAGE", "ERRBIT_SLOT",
    "library_path", "load", "version", "last_error",
    "quant_write", "quant_write_mse", "dedup_compact", "write_and_dedup", "global_compact",
    "global_compact_workspace", "sparse_mla_decode", "sparse_mla_decode_noalloc", "noalloc_scratch_bytes",
    "sparse_mla_decode_partial", "sparse_mla_decode_splits",
    "sparse_mla_decode_workspace", "merge_states", "sparse_mla_prefill", "gather_dequant",
]

LATENT, ROPE, DIM, ROW_BYTES = 512, 64, 576, 352
ROW_BYTES_ROPE_FREE = 288           # the rope-free row: codes and block scales only
ERRBIT_PAGE, ERRBIT_SLOT = 1, 2
MAX_DEDUP_K, MAX_SPLITS = 4096, 64
_F32, _BF16 = 0, 1
_ROW_ROPE, _ROW_ROPE_FREE = 0, 1
_STATUS = {0: "KV4_OK", 1: "KV4_ERR_NULL", 2: "KV4_ERR_SHAPE", 3: "KV4_ERR_ALIGN", 4: "KV4_ERR_UNSUPPORTED",
           5: "KV4_ERR_WORKSPACE", 6: "KV4_ERR_HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libkv4.so")


class Kv4Error(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__("%s: %s" % (_STATUS.get(status, str(status)), text))
        self.status = status


class AttnArgs(ctypes.Structure):
    """Mirror of kv4_attn_args."""
    _fields_ = [
        ("struct_size", ctypes.c_uint32), ("q_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("q_row_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
        ("n_rows", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("pool", ctypes.c_void_p), ("n_slots", ctypes.c_int64),
        ("page_table", ctypes.c_void_p), ("pt_row_stride", ctypes.c_int64),
        ("pt_n_rows", ctypes.c_int32), ("pt_n_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("row_req", ctypes.c_void_p),
        ("topk", ctypes.c_void_p), ("topk_row_stride", ctypes.c_int64), ("k", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p), ("out_row_stride", ctypes.c_int64),
        ("lse", ctypes.c_void_p), ("err_word", ctypes.c_void_p),
        ("row_format", ctypes.c_int32),
    ]


_lib = None


def load():
    """Load libkv4.so (built by bit_kv_cache_kv4_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise Kv4Error(6, "libkv4.so not found at %s; run `python -m bit_kv_cache_kv4_amd.build` "
                          "(or __graft_entry__.build())" % path)
    L = ctypes.CDLL(path)
    vp, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    pa = ctypes.POINTER(AttnArgs)
    L.kv4_version.argtypes, L.kv4_version.restype = [], ctypes.c_char_p
    L.kv4_last_error.argtypes, L.kv4_last_error.restype = [], ctypes.c_char_p
    L.kv4_attn_args_size.argtypes, L.kv4_attn_args_size.restype = [], sz
    L.kv4_quant_write.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp]
    L.kv4_quant_write_rope_free.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp]
    L.kv4_quant_write_mse.argtypes = [vp, i64, vp, i64, vp, i64, i32, vp, vp]
    L.kv4_dedup_compact.argtypes = [vp, i64, i32, i64, vp, vp, vp]
    L.kv4_write_and_dedup.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, i64, i32, i64, vp, vp, vp]
    L.kv4_global_compact_workspace.argtypes, L.kv4_global_compact_workspace.restype = [pa], sz
    L.kv4_global_compact.argtypes = [pa, vp, i64, vp, vp, vp, sz, vp]
    L.kv4_sparse_mla_decode_splits.argtypes, L.kv4_sparse_mla_decode_splits.restype = [pa], i32
    L.kv4_sparse_mla_decode_workspace.argtypes, L.kv4_sparse_mla_decode_workspace.restype = [pa, i32], sz
    L.kv4_sparse_mla_decode.argtypes = [pa, i32, vp, sz, vp]
    L.kv4_sparse_mla_decode_noalloc.argtypes = [pa, i32, vp]
    L.kv4_noalloc_scratch_bytes.argtypes, L.kv4_noalloc_scratch_bytes.restype = [], sz
    L.kv4_sparse_mla_decode_partial.argtypes = [pa, i32, vp, vp, vp]
    L.kv4_sparse_mla_decode_partial_f16.argtypes = [pa, i32, vp, vp, vp]
    L.kv4_merge_states.argtypes = [vp, vp, i32, i64, i32, vp, i64, vp, vp]
    L.kv4_merge_states_f16.argtypes = [vp, vp, i32, i64, i32, vp, i64, vp, vp]
    L.kv4_sparse_mla_prefill.argtypes = [pa, vp]
    L.kv4_gather_dequant.argtypes = [pa, vp, vp, vp]
    for f in ("kv4_quant_write", "kv4_dedup_compact", "kv4_sparse_mla_decode", "kv4_sparse_mla_decode_partial",
              "kv4_sparse_mla_decode_partial_f16", "kv4_merge_states", "kv4_merge_states_f16",
              "kv4_sparse_mla_prefill", "kv4_gather_dequant", "kv4_sparse_mla_decode_noalloc"):
        getattr(L, f).restype = ctypes.c_int
    if L.kv4_attn_args_size() != ctypes.sizeof(AttnArgs):
        raise Kv4Error(2, "kv4_attn_args layout mismatch: library %d bytes, binding %d"
                       % (L.kv4_attn_args_size(), ctypes.sizeof(AttnArgs)))
    _lib = L
    return L


def version() -> str:
    return load().kv4_version().decode()


def last_error() -> str:
    return load().kv4_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise Kv4Error(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


# ------------------------------------------------------------------ write
def _check_write_args(kv, slots, pool, err_word, rope_free=False):
    _need(kv, "kv", torch.float32)
    _need(slots, "slots", torch.int32, kv.device)
    _need(pool, "pool", torch.uint8, kv.device)
    if err_word is not None:
        _need(err_word, "err_word", torch.int32, kv.device)
    if kv.dim() != 2 or slots.dim() != 1 or slots.numel() != kv.shape[0] or (
            kv.shape[0] > 0 and (kv.stride(1) != 1 or (slots.shape[0] > 1 and slots.stride(0) != 1))):
        raise ValueError("kv must be [N, >=576] with unit inner stride and slots [N] contiguous")
    dim, row = (LATENT, ROW_BYTES_ROPE_FREE) if rope_free else (DIM, ROW_BYTES)
    if kv.shape[1] < dim:
        raise ValueError("kv rows need at least %d values" % dim)
    if pool.dim() != 2 or pool.shape[1] != row or not pool.is_contiguous():
        raise ValueError("pool must be a contiguous [n_slots, %d] uint8 tensor" % row)


def quant_write(kv, slots, pool, err_word=None, stream=None) -> None:
    """kv4_quant_write: quantize kv[n] (fp32 [N, >=576] rows) into pool[slots[n]]; with a
    rope-free pool ([n_slots, 288]) kv4_quant_write_rope_free of fp32 [N, >=512] rows."""
    if pool.dim() == 2 and pool.shape[1] == ROW_BYTES_ROPE_FREE:
        _check_write_args(kv, slots, pool, err_word, rope_free=True)
        _check(load().kv4_quant_write_rope_free(_ptr(kv), _stride(kv, 0), _ptr(slots), kv.shape[0], _ptr(pool),
                                                pool.shape[0], _ptr(err_word), _stream(stream, kv.device)))
        return
    _check_write_args(kv, slots, pool, err_word)
    _check(load().kv4_quant_write(_ptr(kv), _stride(kv, 0), _ptr(slots), kv.shape[0], _ptr(pool), pool.shape[0],
                                  _ptr(err_word), _stream(stream, kv.device)))


def quant_write_mse(kv, slots, pool, err_word=None, stream=None) -> None:
    """kv4_quant_write_mse: quant_write with MSE-searched block scales; the row format
    (352-byte rows from 576 values, or 288-byte rope-free rows from 512) follows the pool."""
    rope_free = pool.dim() == 2 and pool.shape[1] == ROW_BYTES_ROPE_FREE
    _check_write_args(kv, slots, pool, err_word, rope_free=rope_free)
    _check(load().kv4_quant_write_mse(_ptr(kv), _stride(kv, 0), _ptr(slots), kv.shape[0], _ptr(pool), pool.shape[0],
                                      _ROW_ROPE_FREE if rope_free else _ROW_ROPE, _ptr(err_word),
                                      _stream(stream, kv.device)))


# ------------------------------------------------------------------ dedup
def _dedup_outputs(idx, k, out_idx, out_count):
    _need(idx, "idx", torch.int32)
    if idx.dim() != 2 or (idx.shape[0] > 0 and idx.stride(1) != 1):
        raise ValueError("idx must be [n_lists, >=k] with unit inner stride")
    n, k = idx.shape[0], idx.shape[1] if k is None else int(k)
    if out_idx is None:
        out_idx = torch.empty((n, k), dtype=torch.int32, device=idx.device)
    if out_count is None:
        out_count = torch.empty((n,), dtype=torch.int32, device=idx.device)
    _need(out_idx, "out_idx", torch.int32, idx.device)
    _need(out_count, "out_count", torch.int32, idx.device)
    if not out_idx.is_contiguous() or tuple(out_idx.shape) != (n, k) or not out_count.is_contiguous():
        raise ValueError("out_idx must be contiguous [n_lists, k], out_count contiguous [n_lists]")
    return n, k, out_idx, out_count


def dedup_compact(idx, k=None, out_idx=None, out_count=None, stream=None):
    """kv4_dedup_compact: per list, first occurrences of values >= 0 in order, -1 fill, counts."""
    n, k, out_idx, out_count = _dedup_outputs(idx, k, out_idx, out_count)
    _check(load().kv4_dedup_compact(_ptr(idx), n, k, _stride(idx, 0), _ptr(out_idx), _ptr(out_count),
                                    _stream(stream, idx.device)))
    return out_idx, out_count


def write_and_dedup(kv, slots, pool, idx, k=None, out_idx=None, out_count=None, err_word=None, stream=None):
    """kv4_write_and_dedup: quant_write(kv, slots, pool) and dedup_compact(idx) as one call
    (one kernel with fewer than 256 lists); returns (out_idx, out_count)."""
    _check_write_args(kv, slots, pool, err_word)
    if idx.device != kv.device:
        raise ValueError("idx must be on the device of kv")
    n, k, out_idx, out_count = _dedup_outputs(idx, k, out_idx, out_count)
    _check(load().kv4_write_and_dedup(_ptr(kv), _stride(kv, 0), _ptr(slots), kv.shape[0], _ptr(pool), pool.shape[0],
                                      _ptr(err_word), _ptr(idx), n, k, _stride(idx, 0), _ptr(out_idx),
                                      _ptr(out_count), _stream(stream, kv.device)))
    return out_idx, out_count


# -------------------------------------------------------------- attention
def _stride(t, d):
    """Element stride of dimension d; a dimension of size 1 is never stepped
    over, and its stride (which torch and numpy leave arbitrary, often 0) is
    reported as the size of the dimensions inside it."""
    if t.shape[d] == 1:
        n = 1
        for x in t.shape[d + 1:]:
            n *= x
        return n
    return t.stride(d)


def _attn_args(q, pool, topk, sm_scale, page_table, row_req, page_size, out, lse, err_word, k=None):
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("q must be bfloat16 or float32")
    _need(q, "q", q.dtype)
    dev = q.device
    _need(pool, "pool", torch.uint8, dev)
    _need(topk, "topk", torch.int32, dev)
    # the pool's row width names the format: 352-byte rows (q of 576 dims) or
    # 288-byte rope-free rows (q of 512)
    if pool.dim() != 2 or pool.shape[1] not in (ROW_BYTES, ROW_BYTES_ROPE_FREE) or not pool.is_contiguous():
        raise ValueError("pool must be a contiguous [n_slots, 352] or [n_slots, 288] uint8 tensor")
    rope_free = pool.shape[1] == ROW_BYTES_ROPE_FREE
    dim = LATENT if rope_free else DIM
    if q.dim() != 3 or q.shape[2] != dim or q.stride(2) != 1:
        raise ValueError("q must be [n_rows, n_heads, %d] with unit inner stride for a %d-byte pool"
                         % (dim, pool.shape[1]))
    if topk.dim() != 2 or topk.shape[0] != q.shape[0] or (topk.numel() > 0 and topk.stride(1) != 1):
        raise ValueError("topk must be [n_rows, k] with unit inner stride")
    a = AttnArgs()
    a.struct_size = ctypes.sizeof(AttnArgs)
    a.q_dtype = _BF16 if q.dtype == torch.bfloat16 else _F32
    a.q, a.q_row_stride, a.q_head_stride = q.data_ptr(), _stride(q, 0), _stride(q, 1)
    a.n_rows, a.n_heads = q.shape[0], q.shape[1]
    a.pool, a.n_slots = pool.data_ptr(), pool.shape[0]
    a.row_format = _ROW_ROPE_FREE if rope_free else _ROW_ROPE
    if page_table is not None:
        _need(page_table, "page_table", torch.int32, dev)
        if page_table.dim() != 2 or page_table.stride(1) != 1:
            raise ValueError("page_table must be [n_req, n_pages] with unit inner stride")
        a.page_table, a.pt_row_stride = page_table.data_ptr(), _stride(page_table, 0)
        a.pt_n_rows, a.pt_n_pages = page_table.shape[0], page_table.shape[1]
    a.page_size = page_size
    if row_req is not None:
        _need(row_req, "row_req", torch.int32, dev)
        if row_req.dim() != 1 or row_req.numel() != q.shape[0] or not row_req.is_contiguous():
            raise ValueError("row_req must be contiguous [n_rows]")
        a.row_req = row_req.data_ptr()
    a.topk, a.topk_row_stride = topk.data_ptr(), _stride(topk, 0)
    a.k = topk.shape[1] if k is None else int(k)
    a.sm_scale = float(sm_scale)
    if out is not None:
        _need(out, "out", torch.float32, dev)
        if out.dim() != 3 or tuple(out.shape) != (q.shape[0], q.shape[1], LATENT) or out.stride(2) != 1 \
                or out.stride(1) != LATENT:
            raise ValueError("out must be [n_rows, n_heads, 512] fp32 with heads packed")
        a.out, a.out_row_stride = out.data_ptr(), _stride(out, 0)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev)
        if tuple(lse.shape) != (q.shape[0], q.shape[1]) or not lse.is_contiguous():
            raise ValueError("lse must be contiguous [n_rows, n_heads] fp32")
        a.lse = lse.data_ptr()
    if err_word is not None:
        _need(err_word, "err_word", torch.int32, dev)
        a.err_word = err_word.data_ptr()
    return a


def _alloc_out(q, out, lse):
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], LATENT), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    return out, lse


def sparse_mla_decode_splits(q, pool, topk, page_table=None, row_req=None, page_size=64) -> int:
    a = _attn_args(q, pool, topk, 1.0, page_table, row_req, page_size, None, None, None)
    s = load().kv4_sparse_mla_decode_splits(ctypes.byref(a))
    if s < 0:
        raise Kv4Error(-s, last_error())
    return s


def sparse_mla_decode_workspace(q, pool, topk, num_splits=0, page_table=None, row_req=None, page_size=64) -> int:
    a = _attn_args(q, pool, topk, 1.0, page_table, row_req, page_size, None, None, None)
    return int(load().kv4_sparse_mla_decode_workspace(ctypes.byref(a), int(num_splits)))


def sparse_mla_decode(q, pool, topk, sm_scale, page_table=None, row_req=None, page_size=64, out=None, lse=None,
                      err_word=None, num_splits=0, workspace=None, stream=None):
    """kv4_sparse_mla_decode; returns (out [R, H, 512] fp32, lse [R, H] fp32).  A workspace is
    allocated with torch when none is given (callers that cannot allocate pass their own)."""
    out, lse = _alloc_out(q, out, lse)
    a = _attn_args(q, pool, topk, sm_scale, page_table, row_req, page_size, out, lse, err_word)
    L = load()
    need = int(L.kv4_sparse_mla_decode_workspace(ctypes.byref(a), int(num_splits)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, q.device)
    _check(L.kv4_sparse_mla_decode(ctypes.byref(a), int(num_splits), _ptr(workspace),
                                   0 if workspace is None else workspace.numel(), _stream(stream, q.device)))
    return out, lse


def sparse_mla_decode_noalloc(q, pool, topk, sm_scale, page_table=None, row_req=None, page_size=64, out=None,
                              lse=None, err_word=None, num_splits=0, stream=None):
    """kv4_sparse_mla_decode_noalloc: decode with the split parts in the library's own scratch array
    (no workspace; out / lse are allocated here only when not given)."""
    out, lse = _alloc_out(q, out, lse)
    a = _attn_args(q, pool, topk, sm_scale, page_table, row_req, page_size, out, lse, err_word)
    _check(load().kv4_sparse_mla_decode_noalloc(ctypes.byref(a), int(num_splits), _stream(stream, q.device)))
    return out, lse


def noalloc_scratch_bytes() -> int:
    """kv4_noalloc_scratch_bytes."""
    return int(load().kv4_noalloc_scratch_bytes())


def sparse_mla_decode_partial(q, pool, topk, sm_scale, num_splits, page_table=None, row_req=None, page_size=64,
                              part_o=None, part_lse=None, err_word=None, stream=None, parts_dtype=torch.float32):
    """kv4_sparse_mla_decode_partial (fp32 parts) or kv4_sparse_mla_decode_partial_f16 (fp16 parts, chosen by
    part_o's dtype, else by parts_dtype); returns (part_o [S, R, H, 512], part_lse [S, R, H])."""
    R, H = q.shape[0], q.shape[1]
    if part_o is None:
        part_o = torch.empty((num_splits, R, H, LATENT), dtype=parts_dtype, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((num_splits, R, H), dtype=torch.float32, device=q.device)
    f16 = part_o.dtype == torch.float16
    _need(part_o, "part_o", torch.float16 if f16 else torch.float32, q.device)
    _need(part_lse, "part_lse", torch.float32, q.device)
    if tuple(part_o.shape) != (num_splits, R, H, LATENT) or not part_o.is_contiguous() or \
            tuple(part_lse.shape) != (num_splits, R, H) or not part_lse.is_contiguous():
        raise ValueError("part_o must be contiguous [S, R, H, 512] and part_lse [S, R, H]")
    a = _attn_args(q, pool, topk, sm_scale, page_table, row_req, page_size, None, None, err_word)
    fn = load().kv4_sparse_mla_decode_partial_f16 if f16 else load().kv4_sparse_mla_decode_partial
    _check(fn(ctypes.byref(a), int(num_splits), _ptr(part_o), _ptr(part_lse), _stream(stream, q.device)))
    return part_o, part_lse


def merge_states(part_o, part_lse, out=None, lse=None, stream=None):
    """kv4_merge_states (fp32 part_o) or kv4_merge_states_f16 (fp16 part_o) over the leading axis:
    part_o [S, ..., dim], part_lse [S, ...]."""
    f16 = part_o.dtype == torch.float16
    _need(part_o, "part_o", torch.float16 if f16 else torch.float32)
    _need(part_lse, "part_lse", torch.float32, part_o.device)
    if not part_o.is_contiguous() or not part_lse.is_contiguous() or part_o.shape[:-1] != part_lse.shape:
        raise ValueError("part_o [S, ..., dim] and part_lse [S, ...] must be contiguous and agree")
    S, dim = part_o.shape[0], part_o.shape[-1]
    n_states = part_lse[0].numel()
    if out is None:
        out = torch.empty(part_o.shape[1:], dtype=torch.float32, device=part_o.device)
    if lse is None:
        lse = torch.empty(part_lse.shape[1:], dtype=torch.float32, device=part_o.device)
    _need(out, "out", torch.float32, part_o.device)
    _need(lse, "lse", torch.float32, part_o.device)
    if out.is_contiguous() and out.numel() == n_states * dim:
        state_stride = dim
    elif out.dim() == 2 and tuple(out.shape) == (n_states, dim) and out.stride(1) == 1 and out.stride(0) >= dim:
        state_stride = out.stride(0)                 # rows of a wider array
    else:
        raise ValueError("out must be contiguous with the parts' shape, or [n_states, dim] with unit inner stride")
    if not lse.is_contiguous() or lse.numel() != n_states:
        raise ValueError("lse must be contiguous with one value per state")
    fn = load().kv4_merge_states_f16 if f16 else load().kv4_merge_states
    _check(fn(_ptr(part_o), _ptr(part_lse), S, n_states, dim, _ptr(out), state_stride, _ptr(lse),
              _stream(stream, part_o.device)))
    return out, lse


def sparse_mla_prefill(q, pool, topk, sm_scale, page_table=None, row_req=None, page_size=64, out=None, lse=None,
                       err_word=None, stream=None):
    """kv4_sparse_mla_prefill; returns (out [R, H, 512] fp32, lse [R, H] fp32)."""
    out, lse = _alloc_out(q, out, lse)
    a = _attn_args(q, pool, topk, sm_scale, page_table, row_req, page_size, out, lse, err_word)
    _check(load().kv4_sparse_mla_prefill(ctypes.byref(a), _stream(stream, q.device)))
    return out, lse


def _unread_q(pool, topk):
    """A stand-in q for the entry points that do not read it (one row of 16
    heads, broadcast over the list rows, so nothing of q's size is allocated)."""
    rope_free = pool.dim() == 2 and pool.shape[1] == ROW_BYTES_ROPE_FREE
    return torch.empty((1, 16, LATENT if rope_free else DIM), dtype=torch.bfloat16,
                       device=topk.device).expand(topk.shape[0], 16, -1)


def _compact_args(pool, topk, page_table, row_req, page_size, err_word):
    return _attn_args(_unread_q(pool, topk), pool, topk, 1.0, page_table, row_req, page_size, None, None, err_word)


def global_compact_workspace(pool, topk, page_table=None, row_req=None, page_size=64) -> int:
    """kv4_global_compact_workspace: bytes of the compaction's workspace for these arguments."""
    a = _compact_args(pool, topk, page_table, row_req, page_size, None)
    return int(load().kv4_global_compact_workspace(ctypes.byref(a)))


def global_compact(pool, topk, page_table=None, row_req=None, page_size=64, err_word=None, cpool=None, out_idx=None,
                   out_count=None, workspace=None, stream=None):
    """kv4_global_compact: the distinct valid slots U of all lists, in increasing order; returns
    (cpool [min(n_slots, R*k), row bytes] with rows U in its first |U| rows, out_idx [R, k] int32
    with each entry's index in U or -1, out_count [1] int32 = |U|) (device tensors; nothing is
    synchronized)."""
    R, k = topk.shape[0], topk.shape[1]
    a = _compact_args(pool, topk, page_table, row_req, page_size, err_word)
    L = load()
    cap = min(pool.shape[0], R * k)
    if cpool is None:
        cpool = torch.empty((max(cap, 1), pool.shape[1]), dtype=torch.uint8, device=pool.device)
    if out_idx is None:
        out_idx = torch.empty((R, k), dtype=torch.int32, device=pool.device)
    if out_count is None:
        out_count = torch.empty((1,), dtype=torch.int32, device=pool.device)
    if workspace is None:
        workspace = torch.empty(max(1, int(L.kv4_global_compact_workspace(ctypes.byref(a)))), dtype=torch.uint8,
                                device=pool.device)
    _need(cpool, "cpool", torch.uint8, pool.device)
    _need(out_idx, "out_idx", torch.int32, pool.device)
    _need(out_count, "out_count", torch.int32, pool.device)
    _need(workspace, "workspace", torch.uint8, pool.device)
    if not cpool.is_contiguous() or cpool.dim() != 2 or cpool.shape[1] != pool.shape[1]:
        raise ValueError("cpool must be contiguous [rows, %d]" % pool.shape[1])
    if not out_idx.is_contiguous() or tuple(out_idx.shape) != (R, k):
        raise ValueError("out_idx must be contiguous [n_rows, k]")
    _check(L.kv4_global_compact(ctypes.byref(a), _ptr(cpool), cpool.shape[0], _ptr(out_idx), _ptr(out_count),
                                _ptr(workspace), workspace.numel(), _stream(stream, pool.device)))
    return cpool, out_idx, out_count


def gather_dequant(pool, topk, page_table=None, row_req=None, page_size=64, err_word=None, stream=None):
    """kv4_gather_dequant; returns (rows [R, k, D] float16, slots [R, k] int32), D = 576, or 512
    for a rope-free (288-byte) pool.  Within each chunk of 2048 entries the valid ones come first, in
    list order (as the attention kernels hold them); the rest are zero rows with slot -1."""
    R, k = topk.shape[0], topk.shape[1]
    dim = LATENT if pool.dim() == 2 and pool.shape[1] == ROW_BYTES_ROPE_FREE else DIM
    a = _attn_args(_unread_q(pool, topk), pool, topk, 1.0, page_table, row_req, page_size, None, None, err_word)
    out = torch.empty((R, k, dim), dtype=torch.float16, device=topk.device)
    slots = torch.empty((R, k), dtype=torch.int32, device=topk.device)
    _check(load().kv4_gather_dequant(ctypes.byref(a), _ptr(out), _ptr(slots), _stream(stream, topk.device)))
    return out, slots
