"""The C ABI on the CPU: the library loads, exports every symbol include/kv4.h
declares, agrees with the binding's struct layout, and rejects bad arguments
on the host before anything is enqueued.  No call here reaches the GPU: every
case fails argument checks first (or has nothing to do)."""
import ctypes
import os
import re
import subprocess

import pytest

import bit_kv_cache_kv4_amd as kv4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kv4.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kv4_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_operations():
    names = _declared_functions()
    for f in ("kv4_quant_write", "kv4_dedup_compact", "kv4_sparse_mla_decode", "kv4_sparse_mla_prefill"):
        assert f in names


def test_library_exports_every_declared_symbol():
    lib = kv4.load()
    out = subprocess.run(["nm", "-D", "--defined-only", kv4.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kv4_\w+)", out))
    missing = [f for f in _declared_functions() if f not in exported]
    assert not missing, missing
    for f in _declared_functions():
        assert hasattr(lib, f)


def test_version_and_struct_layout():
    assert kv4.version().startswith("kv4 ") and "gfx950" in kv4.version()
    assert kv4.load().kv4_attn_args_size() == ctypes.sizeof(kv4.AttnArgs)
    # the ABI constants the binding uses match the header
    src = open(HEADER).read()
    for name, val in (("KV4_ROW_BYTES", kv4.ROW_BYTES), ("KV4_LATENT", kv4.LATENT), ("KV4_DIM", kv4.DIM),
                      ("KV4_MAX_DEDUP_K", kv4.MAX_DEDUP_K), ("KV4_MAX_SPLITS", kv4.MAX_SPLITS)):
        assert re.search(r"#define %s\s+%d\b" % (name, val), src), name
    assert re.search(r"#define KV4_ERRBIT_PAGE 1u", src) and re.search(r"#define KV4_ERRBIT_SLOT 2u", src)


def _args(**kw):
    a = kv4.AttnArgs()
    a.struct_size = ctypes.sizeof(kv4.AttnArgs)
    a.q_dtype = 1
    a.q = 0x1000
    a.q_row_stride, a.q_head_stride = 64 * 576, 576
    a.n_rows, a.n_heads = 2, 64
    a.pool, a.n_slots = 0x2000, 100
    a.page_size = 64
    a.topk, a.topk_row_stride, a.k = 0x3000, 16, 16
    a.sm_scale = 0.04
    a.out, a.out_row_stride = 0x4000, 64 * 512
    for key, v in kw.items():
        setattr(a, key, v)
    return a


BAD_ARGS = [
    (dict(struct_size=8), 2, "struct_size"),
    (dict(q_dtype=7), 2, "q_dtype"),
    (dict(n_heads=20), 4, "n_heads"),
    (dict(n_heads=256), 4, "n_heads"),
    (dict(k=-1), 2, "k"),
    (dict(k=(1 << 30) + 1, topk_row_stride=(1 << 30) + 1), 4, "k"),
    (dict(q=None), 1, "q is NULL"),
    (dict(topk=None), 1, "topk"),
    (dict(out=None), 1, "out"),
    (dict(q=0x1008), 3, "q must be 16-byte aligned"),
    (dict(q_head_stride=500), 3, "q_head_stride"),
    (dict(q_head_stride=580), 3, "q_head_stride"),
    (dict(q_row_stride=576), 3, "q_row_stride"),
    (dict(pool=0x2004), 3, "pool"),
    (dict(topk_row_stride=8), 2, "topk_row_stride"),
    (dict(page_table=0x5000, page_size=48, pt_n_rows=2), 2, "page_size"),
    (dict(page_table=0x5000, pt_n_rows=0), 2, "pt_n_rows"),
    (dict(page_table=0x5000, pt_n_rows=1), 2, "pt_n_rows"),
    (dict(out=0x4004), 3, "out"),
    (dict(out_row_stride=100), 3, "out_row_stride"),
    (dict(n_slots=1 << 31), 4, "n_slots"),           # slots are 32-bit inside the kernels
    (dict(n_slots=(1 << 31) + 5), 4, "n_slots"),
    (dict(sm_scale=float("nan")), 2, "sm_scale"),
    (dict(sm_scale=float("inf")), 2, "sm_scale"),
    (dict(sm_scale=float("-inf")), 2, "sm_scale"),
]


@pytest.mark.parametrize("kw,status,text", BAD_ARGS)
def test_attention_argument_checks(kw, status, text):
    lib = kv4.load()
    a = _args(**kw)
    st = lib.kv4_sparse_mla_prefill(ctypes.byref(a), None)
    assert st == status and text in kv4.last_error()
    st = lib.kv4_sparse_mla_decode(ctypes.byref(a), 1, None, 0, None)
    assert st == status


def test_decode_split_and_workspace_checks():
    lib = kv4.load()
    a = _args()
    assert lib.kv4_sparse_mla_decode(ctypes.byref(a), -1, None, 0, None) == 2
    assert lib.kv4_sparse_mla_decode(ctypes.byref(a), 65, None, 0, None) == 2
    # 2 splits need a workspace; none given
    assert lib.kv4_sparse_mla_decode(ctypes.byref(a), 2, None, 0, None) == 5
    need = lib.kv4_sparse_mla_decode_workspace(ctypes.byref(a), 2)
    assert need == 2 * 2 * 64 * 512 * 2 + 2 * 2 * 64 * 4   # fp16 o of each part, fp32 lse
    assert lib.kv4_sparse_mla_decode(ctypes.byref(a), 2, ctypes.c_void_p(0x100000), need - 1, None) == 5
    assert lib.kv4_sparse_mla_decode(ctypes.byref(a), 2, ctypes.c_void_p(0x100010), need, None) == 3
    assert lib.kv4_sparse_mla_decode_workspace(ctypes.byref(a), 1) == 0
    assert lib.kv4_sparse_mla_decode_partial(ctypes.byref(a), 0, None, None, None) == 2
    assert lib.kv4_sparse_mla_decode_partial(ctypes.byref(a), 2, None, None, None) == 1
    # fp16 parts: the same checks, 8-byte alignment of part_o
    V = ctypes.c_void_p
    assert lib.kv4_sparse_mla_decode_partial_f16(ctypes.byref(a), 0, None, None, None) == 2
    assert lib.kv4_sparse_mla_decode_partial_f16(ctypes.byref(a), 2, None, V(0x100000), None) == 1
    assert lib.kv4_sparse_mla_decode_partial_f16(ctypes.byref(a), 2, V(0x100004), V(0x200000), None) == 3
    assert lib.kv4_sparse_mla_decode_partial(ctypes.byref(a), 2, V(0x100008), V(0x200000), None) == 3


def test_merge_states_argument_checks():
    lib = kv4.load()
    V = ctypes.c_void_p
    for f, bad_align in ((lib.kv4_merge_states, 0x1008), (lib.kv4_merge_states_f16, 0x1004)):
        assert f(V(0x1000), V(0x2000), 0, 4, 512, V(0x3000), 512, None, None) == 2     # n_parts
        assert f(V(0x1000), V(0x2000), 65, 4, 512, V(0x3000), 512, None, None) == 2
        assert f(V(0x1000), V(0x2000), 2, 4, 510, V(0x3000), 512, None, None) == 2     # dim % 4
        assert f(V(0x1000), V(0x2000), 2, 0, 512, V(0x3000), 512, None, None) == 0     # nothing to do
        assert f(None, V(0x2000), 2, 4, 512, V(0x3000), 512, None, None) == 1
        assert f(V(0x1000), V(0x2000), 2, 4, 512, None, 512, None, None) == 1
        assert f(V(bad_align), V(0x2000), 2, 4, 512, V(0x3000), 512, None, None) == 3
        assert f(V(0x1000), V(0x2000), 2, 4, 512, V(0x3008), 512, None, None) == 3
        assert f(V(0x1000), V(0x2000), 2, 4, 512, V(0x3000), 508, None, None) == 3     # stride < dim


def test_zero_rows_is_a_no_op():
    lib = kv4.load()
    a = _args(n_rows=0, q=None, out=None, topk=None)
    assert lib.kv4_sparse_mla_prefill(ctypes.byref(a), None) == 0
    assert lib.kv4_sparse_mla_decode(ctypes.byref(a), 0, None, 0, None) == 0


def test_quant_write_argument_checks():
    lib = kv4.load()
    f = lib.kv4_quant_write
    V = ctypes.c_void_p
    assert f(None, 576, None, 0, None, 0, None, None) == 0                 # nothing to do
    assert f(None, 576, V(0x10), 4, V(0x20), 8, None, None) == 1
    assert f(V(0x10), 576, V(0x10), -1, V(0x20), 8, None, None) == 2
    assert f(V(0x10), 575, V(0x10), 4, V(0x20), 8, None, None) == 3
    assert f(V(0x10), 578, V(0x10), 4, V(0x20), 8, None, None) == 3
    assert f(V(0x18), 576, V(0x10), 4, V(0x20), 8, None, None) == 3
    assert f(V(0x10), 576, V(0x10), 4, V(0x28), 8, None, None) == 3
    assert f(V(0x10), 576, V(0x10), 4, None, 8, None, None) == 1


def test_quant_write_mse_argument_checks():
    lib = kv4.load()
    f = lib.kv4_quant_write_mse
    V = ctypes.c_void_p
    assert f(None, 576, None, 0, None, 0, 0, None, None) == 0              # nothing to do
    assert f(V(0x10), 576, V(0x10), 4, V(0x20), 8, 2, None, None) == 2    # unknown row format
    assert f(V(0x10), 576, V(0x10), 4, V(0x20), 8, -1, None, None) == 2
    assert f(V(0x10), 575, V(0x10), 4, V(0x20), 8, 0, None, None) == 3
    assert f(V(0x10), 512, V(0x10), 4, V(0x20), 8, 0, None, None) == 3    # 352-byte rows need 576 values
    assert f(V(0x10), 511, V(0x10), 4, V(0x20), 8, 1, None, None) == 3
    assert f(V(0x18), 512, V(0x10), 4, V(0x20), 8, 1, None, None) == 3
    assert f(None, 576, V(0x10), 4, V(0x20), 8, 0, None, None) == 1
    assert f(V(0x10), 576, V(0x10), 4, V(0x20), 8, 9, None, None) == 2
    assert b"row_format" in lib.kv4_last_error()


def test_dedup_argument_checks():
    lib = kv4.load()
    f = lib.kv4_dedup_compact
    V = ctypes.c_void_p
    assert f(None, 0, 16, 16, None, None, None) == 0
    assert f(V(0x10), 4, 4097, 4097, V(0x100000), V(0x200000), None) == 4
    assert f(V(0x10), 4, 16, 8, V(0x100000), V(0x200000), None) == 2
    assert f(V(0x1000), 4, 16, 16, V(0x1010), V(0x200000), None) == 2      # overlap
    assert "overlap" in kv4.last_error()
    assert f(V(0x1000), 4, 16, 16, None, V(0x200000), None) == 1


def test_write_and_dedup_argument_checks():
    """The combined call checks both halves exactly as the two calls do and
    launches nothing when both are empty (no GPU needed for any of these)."""
    lib = kv4.load()
    f = lib.kv4_write_and_dedup
    V = ctypes.c_void_p
    w_ok = (V(0x10), 576, V(0x10), 4, V(0x20), 8, None)
    d_ok = (V(0x100000), 4, 16, 16, V(0x200000), V(0x300000))
    assert f(None, 576, None, 0, None, 0, None, None, 0, 16, 16, None, None, None) == 0     # nothing to do
    assert f(None, 576, V(0x10), 4, V(0x20), 8, None, *d_ok, None) == 1                    # write half: kv NULL
    assert f(V(0x10), 575, V(0x10), 4, V(0x20), 8, None, *d_ok, None) == 3                  # write half: stride
    assert f(*w_ok, V(0x100000), 4, 4097, 4097, V(0x200000), V(0x300000), None) == 4        # dedup half: k
    assert f(*w_ok, V(0x1000), 4, 16, 16, V(0x1010), V(0x300000), None) == 2                # dedup half: overlap
    assert "overlap" in kv4.last_error()
    assert f(*w_ok, V(0x1000), 4, 16, 16, None, V(0x300000), None) == 1


def test_global_compact_argument_checks():
    """Workspace and output sizing of the compaction (no launch)."""
    lib = kv4.load()
    a = _args()                                          # 2 rows x 16 entries over 100 slots
    need = lib.kv4_global_compact_workspace(ctypes.byref(a))
    assert need > 0
    V = ctypes.c_void_p
    f = lib.kv4_global_compact
    assert f(ctypes.byref(a), V(0x10000), 32, V(0x20000), V(0x30000), V(0x100000), need - 1, None) == 5
    assert f(ctypes.byref(a), V(0x10000), 31, V(0x20000), V(0x30000), V(0x100000), need, None) == 2   # cpool rows
    assert "cpool" in kv4.last_error()
    assert f(ctypes.byref(a), V(0x10000), 32, None, V(0x30000), V(0x100000), need, None) == 1           # out_idx
    assert f(ctypes.byref(a), V(0x10000), 32, V(0x20000), None, V(0x100000), need, None) == 1           # out_count
    assert f(ctypes.byref(a), V(0x10008), 32, V(0x20000), V(0x30000), V(0x100000), need, None) == 3     # cpool align
    assert f(ctypes.byref(a), V(0x10000), 32, V(0x20000), V(0x30000), V(0x100010), need, None) == 3     # workspace align
    a2 = _args(row_format=1, q_head_stride=576)                  # rope-free: 512-dim queries suffice
    assert lib.kv4_global_compact_workspace(ctypes.byref(a2)) == need
    a3 = _args(row_format=2)
    assert lib.kv4_global_compact_workspace(ctypes.byref(a3)) == 0
    # q, its strides and n_heads are not read by the compaction or the gather
    a4 = _args(q=None, q_row_stride=0, q_head_stride=0, n_heads=0)
    assert lib.kv4_global_compact_workspace(ctypes.byref(a4)) == need
    assert f(ctypes.byref(a4), V(0x10000), 32, V(0x20000), None, V(0x100000), need, None) == 1
    assert "out_count" in kv4.last_error()
    assert lib.kv4_gather_dequant(ctypes.byref(a4), None, None, None) == 1
    assert "out" in kv4.last_error()
    assert lib.kv4_sparse_mla_decode_splits(ctypes.byref(a4)) < 0      # attention still needs q


def test_merge_argument_checks():
    lib = kv4.load()
    f = lib.kv4_merge_states
    V = ctypes.c_void_p
    assert f(V(0x10), V(0x20), 0, 4, 512, V(0x30), 512, None, None) == 2
    assert f(V(0x10), V(0x20), 65, 4, 512, V(0x30), 512, None, None) == 2
    assert f(V(0x10), V(0x20), 2, 4, 510, V(0x30), 512, None, None) == 2
    assert f(V(0x10), V(0x20), 2, 4, 512, V(0x30), 500, None, None) == 3
    assert f(V(0x18), V(0x20), 2, 4, 512, V(0x30), 512, None, None) == 3
    assert f(V(0x10), V(0x20), 2, 0, 512, V(0x30), 512, None, None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        kv4.quant_write(torch.zeros(4, 576), torch.zeros(4, dtype=torch.int32), torch.zeros(8, 352, dtype=torch.uint8))
