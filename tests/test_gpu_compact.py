"""GPU parity of the global dedup across lists (the compacted pool): bytes,
rewritten lists and counts bit-exact against the oracle, and attention over
the compacted pool equal, bit for bit, to attention over the original."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, to_dev

pytestmark = pytest.mark.gpu


def _both(pool_h, topk, pt=None, row_req=None, pool_d=None):
    cp_h, idx_h, n_h, err_h = oracle.global_compact(topk, pool_h, pt, row_req)
    pool_d = to_dev(pool_h) if pool_d is None else pool_d
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    cp_d, idx_d, n_d = kv4.global_compact(pool_d, to_dev(topk), page_table=None if pt is None else to_dev(pt),
                                          row_req=None if row_req is None else to_dev(row_req), err_word=err)
    torch.cuda.synchronize()
    n = int(n_d.item())
    assert n == n_h
    assert int(err.item()) == err_h
    assert (idx_d.cpu().numpy() == idx_h).all()
    assert (cp_d[:n].cpu().numpy() == cp_h).all()
    return cp_d, idx_d, n


@pytest.mark.parametrize("row_bytes", [352, 288])
def test_compact_invalid_entries_and_missing_requests(row_bytes):
    g = np.random.default_rng(60 + row_bytes)
    n_req, n_pages, R, k = 3, 6, 5, 300
    n_slots = 20 * 64 - 7
    pool = g.integers(0, 256, size=(n_slots, row_bytes)).astype(np.uint8)
    pt = g.permutation(20)[:n_req * n_pages].reshape(n_req, n_pages).astype(np.int32)
    pt[1, 2] = -1
    row_req = np.array([0, 1, 2, 2, 7], np.int32)
    topk = g.integers(-3, n_pages * 64 + 30, size=(R, k)).astype(np.int32)
    _both(pool, topk, pt, row_req)


@pytest.mark.parametrize("n_slots,R,k", [(1000, 1, 5), (1000, 3, 0), (70000, 40, 2048), (1 << 21, 64, 2048),
                                         (400000, 17, 3000), (1000, 1100, 64), (262144, 3, 100)])
def test_compact_physical_slots(n_slots, R, k):
    """Lists of physical slots.  2^21 slots take the global-atomic marking;
    the others the LDS marking, with the rewrite's word table in LDS up to
    262,144 slots (400,000 slots: marking in LDS, rewrite from global memory);
    1100 rows give several rows to each of the 512 marking workgroups."""
    g = np.random.default_rng(n_slots + R)
    pool_d = torch.randint(0, 256, (n_slots, 352), dtype=torch.uint8, device=DEV)
    pool_h = pool_d.cpu().numpy()
    topk = g.integers(-1, n_slots + 3, size=(R, k)).astype(np.int32)   # a few past the pool
    _both(pool_h, topk, pool_d=pool_d)


def test_compact_pool_past_the_inline_scan():
    """A pool of 140M slots: more than 1024 scan blocks of 4096 bitmap words,
    so the block totals get a scan launch of their own before the rewrite
    (smaller pools scan them inside it).  The compaction depends only on the
    order of the distinct slots, so the oracle runs on the same lists with
    their slots renumbered in order onto a small pool holding the same rows;
    entries past the pool map past the small one (flagged by both)."""
    n_slots = 140_000_000
    g = np.random.default_rng(140)
    R, k = 3, 700
    used = np.unique(g.integers(0, n_slots, size=1500))
    used = np.union1d(used, [0, 134_217_727, 134_217_728, n_slots - 1])   # both sides of block 1024, the ends
    topk = g.choice(used, size=(R, k)).astype(np.int64)
    topk[0, :6] = [n_slots - 1, n_slots, n_slots + 7, -1, 134_217_728, 0]
    topk[2] = -1
    valid = (topk >= 0) & (topk < n_slots)
    small = np.where(valid, np.searchsorted(used, np.clip(topk, 0, n_slots - 1)),
                     np.where(topk >= n_slots, len(used) + (topk - n_slots), topk)).astype(np.int32)
    rows = g.integers(0, 256, size=(len(used), 352)).astype(np.uint8)
    cp_h, idx_h, n_h, err_h = oracle.global_compact(small, rows)
    pool_d = torch.empty((n_slots, 352), dtype=torch.uint8, device=DEV)
    pool_d[torch.from_numpy(used).to(DEV)] = to_dev(rows)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    cp_d, idx_d, n_d = kv4.global_compact(pool_d, to_dev(topk.astype(np.int32)), err_word=err)
    torch.cuda.synchronize()
    n = int(n_d.item())
    try:
        assert n == n_h and int(err.item()) == err_h
        assert (idx_d.cpu().numpy() == idx_h).all()
        assert (cp_d[:n].cpu().numpy() == cp_h).all()
    finally:
        del pool_d, cp_d
        torch.cuda.empty_cache()


def test_compact_all_invalid():
    pool = np.zeros((100, 352), np.uint8)
    topk = np.full((4, 16), -1, np.int32)
    _, idx, n = _both(pool, topk)
    assert n == 0


def test_attention_over_the_compacted_pool_is_unchanged():
    """Decode and prefill over (compacted pool, rewritten lists, no page
    table) equal decode and prefill over the original arguments bit for bit."""
    spec = W.C2
    kv = W.kv_rows_host(spec, 0, spec.n_slots)
    pool_d = torch.zeros((spec.n_slots, 352), dtype=torch.uint8, device=DEV)
    kv4.quant_write(to_dev(kv), to_dev(np.arange(spec.n_slots, dtype=np.int32)), pool_d)
    q, topk, pt = to_dev(W.queries(spec)), W.topk_lists(spec), W.page_table(spec)
    topk[0, 3] = -1
    topk[1, 7] = topk[1, 8]
    cp, idx, n = kv4.global_compact(pool_d, to_dev(topk), page_table=to_dev(pt))
    torch.cuda.synchronize()
    cnt = int(n.item())
    assert cnt == len(set((pt[np.arange(topk.shape[0])[:, None], np.maximum(topk, 0) >> 6] * 64
                           + (np.maximum(topk, 0) & 63))[topk >= 0].tolist()))
    cpool = cp[:cnt].contiguous()
    for s in (1, 4):
        a = kv4.sparse_mla_decode(q, pool_d, to_dev(topk), spec.sm_scale, page_table=to_dev(pt), num_splits=s)
        b = kv4.sparse_mla_decode(q, cpool, idx, spec.sm_scale, num_splits=s)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), "splits=%d" % s
    a = kv4.sparse_mla_prefill(q, pool_d, to_dev(topk), spec.sm_scale, page_table=to_dev(pt))
    b = kv4.sparse_mla_prefill(q, cpool, idx, spec.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
