"""GPU parity of the dequantizing gather, through the attention kernel's own
front end: kv4_gather_dequant translates each chunk of 2048 list entries with
the same device functions as the attention kernel (positions, page-table
entries, the ballot packing of valid slots) and dequantizes each tile with the
same gather and FP4/FP8 conversion code into the same LDS tile, then copies
that tile out.  The translated slots and every dequantized fp16 value are
compared bit for bit with the oracle's page arithmetic and row decoding.

Entry j of a chunk's output is the j-th valid entry of the chunk, in list
order; the entries past the valid count get slot -1 and zero rows."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, build_pools, to_dev

pytestmark = pytest.mark.gpu

CHUNK = 2048


def _expected(pool_h, topk, pt, row_req=None, page_size=64, n_rope=64):
    """Oracle: translate every entry, then pack each chunk's valid entries to
    its front (list order); returns (rows [R, k, D] float64, slots, err)."""
    R, k = topk.shape
    D = 512 + n_rope
    rows = np.zeros((R, k, D), dtype=np.float64)
    slots = np.full((R, k), -1, dtype=np.int64)
    err = 0
    n_slots = pool_h.shape[0]
    for r in range(R):
        req = r if row_req is None else int(row_req[r])
        for c_lo in range(0, k, CHUNK):
            j_out = c_lo
            for j in range(c_lo, min(k, c_lo + CHUNK)):
                if pt is not None and not (0 <= req < pt.shape[0]):
                    err |= kv4.ERRBIT_PAGE if topk[r, j] >= 0 else 0
                    continue
                s, e = oracle.translate(int(topk[r, j]), None if pt is None else pt[req], page_size, n_slots)
                err |= e
                if s >= 0:
                    slots[r, j_out] = s
                    rows[r, j_out] = oracle.dequantize_row(pool_h[s], n_rope=n_rope)
                    j_out += 1
    return rows, slots, err


def _compare(rows_d, slots_d, rows_h, slots_h):
    assert (slots_d.cpu().numpy() == slots_h).all(), "translated slots differ"
    got = rows_d.cpu().numpy()
    valid = slots_h >= 0
    want = rows_h.astype(np.float16)
    nan = np.isnan(rows_h)
    assert ((want.astype(np.float64) == rows_h) | nan).all()            # every value is exact in fp16
    g, w = got[valid], want[valid]
    gn, wn = np.isnan(g), np.isnan(w)
    assert (gn == wn).all(), "NaN positions differ"
    assert (g.view(np.uint16)[~gn] == w.view(np.uint16)[~wn]).all(), "dequantized values differ bitwise"
    assert (got[~valid] == 0).all(), "padding entries are not zero"


def _check(spec, topk, pt, err_expect=0, row_req=None, pools=None):
    pool_d, pool_h = build_pools(spec) if pools is None else pools
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rows_d, slots_d = kv4.gather_dequant(pool_d, to_dev(topk), page_table=None if pt is None else to_dev(pt),
                                         row_req=None if row_req is None else to_dev(row_req), err_word=err)
    torch.cuda.synchronize()
    n_rope = 64 if pool_h.shape[1] == 352 else 0
    rows_h, slots_h, err_h = _expected(pool_h, topk, pt, row_req, n_rope=n_rope)
    _compare(rows_d, slots_d, rows_h, slots_h)
    assert int(err.item()) == err_h == err_expect


def test_gather_c1_bit_exact():
    spec = W.C1
    _check(spec, W.topk_lists(spec), W.page_table(spec))


def test_gather_invalid_entries_and_outliers():
    spec = W.scaled(W.C2, n_req=2, ctx=4096, n_pool_pages=160, k=300, seed=2100)
    pools = build_pools(spec)
    topk, pt = W.topk_lists(spec).copy(), W.page_table(spec).copy()
    topk[0, :3] = [-1, spec.ctx + 64, 5]            # pad, past the table, valid
    pt[1, 2] = -1                                    # an unmapped page
    topk[1, :2] = [2 * 64 + 7, 64]
    topk[0, 100:140] = -1                            # a run of pads in the middle
    _check(spec, topk, pt, err_expect=kv4.ERRBIT_PAGE, pools=pools)
    slots = np.int32([[0, 1, spec.n_slots, -4] + list(range(10, 306))] * 2)
    _check(spec, slots, None, err_expect=kv4.ERRBIT_SLOT, pools=pools)
    _check(spec, W.topk_lists(spec), W.page_table(spec), row_req=np.int32([1, 1]), pools=pools)
    _check(spec, W.topk_lists(spec), W.page_table(spec), row_req=np.int32([1, 7]), err_expect=kv4.ERRBIT_PAGE,
           pools=pools)                              # a request outside the table


def test_gather_all_invalid_and_single_entries():
    spec = W.scaled(W.C1, seed=1100)
    pools = build_pools(spec)
    _check(spec, np.full((1, 64), -1, dtype=np.int32), W.page_table(spec), pools=pools)
    _check(spec, np.int32([[spec.ctx - 1]]), W.page_table(spec), pools=pools)
    _check(spec, np.int32([[3, -1, 3, 3]]), W.page_table(spec), pools=pools)   # repeats kept as given


def test_gather_lists_longer_than_a_chunk():
    """2500 entries: two chunks, each packed on its own."""
    spec = W.scaled(W.C2, n_req=1, ctx=8192, n_pool_pages=160, k=2500, seed=2200)
    pools = build_pools(spec)
    topk = W.topk_lists(spec).copy()
    topk[0, ::7] = -1
    topk[0, 2040:2060] = -1                          # pads across the chunk boundary
    _check(spec, topk, W.page_table(spec), pools=pools)


@pytest.mark.parametrize("n_pages", [4096, 4097])
def test_gather_long_page_table_rows(n_pages):
    """Page-table rows of 4096 and 4097 entries naming pool pages more than
    once; entries in both chunks of a 2100-entry list."""
    spec = W.scaled(W.C2, n_req=2, ctx=64 * n_pages, n_pool_pages=160, k=2100, seed=2300)
    pools = build_pools(spec)
    g = np.random.default_rng(n_pages)
    pt = g.integers(0, spec.n_pool_pages, size=(spec.n_req, n_pages)).astype(np.int32)
    topk = W.topk_lists(spec).copy()
    topk[0, 0] = spec.ctx - 1
    _check(spec, topk, pt, pools=pools)
    topk[1, 2049] = spec.ctx                         # past the table, in the second chunk
    _check(spec, topk, pt, err_expect=kv4.ERRBIT_PAGE, pools=pools)


def _code_pool(n_rope):
    """Eight rows holding every (E2M1 code, E4M3 scale byte) pair once: block b
    of row i has scale byte 32 i + b (all 256, NaN bytes and negative scales
    included) and codes 0..15 (both signs); rows 0..3 hold the 256 rope codes
    in order, rows 4..7 the same permuted."""
    rb = 352 if n_rope else 288
    pool = np.zeros((8, rb), dtype=np.uint8)
    codes = np.array([(2 * k) | ((2 * k + 1) << 4) for k in range(8)], dtype=np.uint8)
    for i in range(8):
        for b in range(32):
            pool[i, 8 * b:8 * b + 8] = codes
            pool[i, 256 + b] = 32 * i + b
        if n_rope:
            pool[i, 288:352] = (np.arange(64) + 64 * (i % 4)) ^ (0x5A if i >= 4 else 0)
    return pool


@pytest.mark.parametrize("n_rope", [64, 0])
def test_gather_every_code_and_scale(n_rope):
    """Every E2M1 code under every E4M3 scale byte, and every rope code, through
    a permuted page table, bit-exact."""
    code_rows = _code_pool(n_rope)
    n_slots = 64 * 6
    rng = np.random.default_rng(31)
    pool_h = rng.integers(0, 256, size=(n_slots, code_rows.shape[1]), dtype=np.uint8)
    place = rng.choice(n_slots, size=8, replace=False)
    pool_h[place] = code_rows
    pool_d = to_dev(pool_h)
    pt = rng.permutation(6).astype(np.int32)[None, :]
    inv = np.empty(6, dtype=np.int64)
    inv[pt[0]] = np.arange(6)
    pos = (inv[place // 64] * 64 + place % 64).astype(np.int32)     # request-local positions of the code rows
    lst = np.concatenate([pos, pos[::-1], [-1, 6 * 64 + 3], pos[:3]]).astype(np.int32)[None, :]
    _check(None, lst, pt, err_expect=kv4.ERRBIT_PAGE, pools=(pool_d, pool_h))
    _check(None, place.astype(np.int32)[None, :], None, pools=(pool_d, pool_h))   # physical slots


def test_gather_rope_free_bit_exact():
    spec = W.C1
    kv = W.kv_rows_host(spec, 0, spec.n_slots)[:, :512].copy()
    pool_h = np.zeros((spec.n_slots, 288), dtype=np.uint8)
    oracle.quant_write(kv, np.arange(spec.n_slots, dtype=np.int32), pool_h, n_rope=0)
    pool_d = torch.zeros((spec.n_slots, 288), dtype=torch.uint8, device=DEV)
    kv4.quant_write(to_dev(kv), torch.arange(spec.n_slots, dtype=torch.int32, device=DEV), pool_d)
    topk = W.topk_lists(spec).copy()
    topk[0, 5] = -1
    topk[0, 77] = spec.ctx + 1
    _check(spec, topk, W.page_table(spec), err_expect=kv4.ERRBIT_PAGE, pools=(pool_d, pool_h))
