"""GPU parity of the dequantizing gather: translated slots and dequantized
fp16 rows bit-exact against the oracle's page arithmetic and row decoding."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, build_pools, to_dev

pytestmark = pytest.mark.gpu


def _oracle_gather(pool_h, topk, pt, row_req=None, page_size=64):
    R, k = topk.shape
    rows = np.zeros((R, k, 576), dtype=np.float64)
    slots = np.full((R, k), -1, dtype=np.int64)
    err = 0
    n_slots = pool_h.shape[0]
    for r in range(R):
        req = r if row_req is None else int(row_req[r])
        for j in range(k):
            s, e = oracle.translate(int(topk[r, j]), None if pt is None else pt[req], page_size, n_slots)
            err |= e
            slots[r, j] = s
            if s >= 0:
                rows[r, j] = oracle.dequantize_row(pool_h[s])
    return rows, slots, err


def _check(spec, topk, pt, err_expect=0, row_req=None):
    pool_d, pool_h = build_pools(spec)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    rows_d, slots_d = kv4.gather_dequant(pool_d, to_dev(topk), page_table=None if pt is None else to_dev(pt),
                                         row_req=None if row_req is None else to_dev(row_req), err_word=err)
    torch.cuda.synchronize()
    rows_h, slots_h, err_h = _oracle_gather(pool_h, topk, pt, row_req)
    assert (slots_d.cpu().numpy() == slots_h).all()
    want = rows_h.astype(np.float16)
    assert (want.astype(np.float64) == rows_h).all()            # exact in fp16
    got = rows_d.cpu().numpy()
    assert (got.view(np.uint16) == want.view(np.uint16)).all()
    assert int(err.item()) == err_h == err_expect


def test_gather_c1_bit_exact():
    spec = W.C1
    _check(spec, W.topk_lists(spec), W.page_table(spec))


def test_gather_invalid_entries_and_outliers():
    spec = W.scaled(W.C2, n_req=2, ctx=4096, n_pool_pages=160, k=300, seed=2100)
    topk, pt = W.topk_lists(spec).copy(), W.page_table(spec).copy()
    topk[0, :3] = [-1, spec.ctx + 64, 5]            # pad, past the table, valid
    pt[1, 2] = -1                                    # an unmapped page
    topk[1, :2] = [2 * 64 + 7, 64]
    _check(spec, topk, pt, err_expect=kv4.ERRBIT_PAGE)
    slots = np.int32([[0, 1, spec.n_slots, -4] + list(range(10, 306))] * 2)
    _check(spec, slots, None, err_expect=kv4.ERRBIT_SLOT)
    _check(spec, W.topk_lists(spec), W.page_table(spec), row_req=np.int32([1, 1]))
