"""The full-size workloads in the launch configuration bench.py times, every
output compared with the oracle: the long-context decode pool (64 requests x
204,800 tokens, 4.6 GB of rows; all 64 requests, automatic split count, fp16
split parts and their merge) and the 4096-query prefill (every query row, one
launch)."""
import numpy as np
import pytest
import torch

import bench
import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, compare_attention, q_for_oracle

pytestmark = pytest.mark.gpu


def test_c3_long_context_decode_every_request():
    spec = W.C3
    dev = torch.device(DEV)
    wl = bench.build_decode_workload(spec, dev, n_sets=1)
    st, pool, pt = wl["sets"][0], wl["pool"], wl["pt"]
    S = kv4.sparse_mla_decode_splits(st["q"], pool, st["topk"], page_table=pt)
    lists, counts = kv4.dedup_compact(st["topk"])
    # the launch configuration the benchmark times: fp16 parts, then their merge
    po, pl = kv4.sparse_mla_decode_partial(st["q"], pool, lists, spec.sm_scale, S, page_table=pt,
                                           parts_dtype=torch.float16)
    out, lse = kv4.merge_states(po, pl)
    torch.cuda.synchronize()
    assert (counts.cpu().numpy() == spec.k).all()
    rows_all = np.arange(spec.n_req)
    uniq, rows, slots = bench.gathered_rows_host(spec, wl["pt_h"][rows_all], st["topk_h"][rows_all], dev)
    pool_h = np.zeros((uniq.size, 352), dtype=np.uint8)
    oracle.quant_write(rows, np.arange(uniq.size, dtype=np.int32), pool_h)
    got_rows = pool.index_select(0, torch.from_numpy(uniq).to(dev)).cpu().numpy()
    assert (got_rows == pool_h).all(), "gathered pool rows differ from the oracle's bytes"
    compact = np.searchsorted(uniq, slots).astype(np.int32)
    o_ref, lse_ref, err = oracle.sparse_mla(q_for_oracle(st["q"]), pool_h, compact, spec.sm_scale)
    assert err == 0
    rel, lerr = compare_attention(out, lse, o_ref, lse_ref)
    print("c3 all %d requests (splits=%d): max rel err %.2e, lse err %.2e" % (spec.n_req, S, rel, lerr))


def test_c5_prefill_every_row():
    spec = W.C5
    dev = torch.device(DEV)
    kv = W.kv_rows_host(spec, 0, spec.n_slots)
    pool_h = np.zeros((spec.n_slots, 352), dtype=np.uint8)
    oracle.quant_write(kv, np.arange(spec.n_slots, dtype=np.int32), pool_h)
    pool = torch.empty((spec.n_slots, 352), dtype=torch.uint8, device=dev)
    kv4.quant_write(torch.from_numpy(kv).to(dev), torch.arange(spec.n_slots, dtype=torch.int32, device=dev), pool)
    q = W.queries(spec)
    topk = W.topk_lists(spec)
    pt = W.page_table(spec)
    rr = W.row_req(spec)
    out, lse = kv4.sparse_mla_prefill(q.to(dev), pool, torch.from_numpy(topk).to(dev), spec.sm_scale,
                                      page_table=torch.from_numpy(pt).to(dev), row_req=torch.from_numpy(rr).to(dev))
    torch.cuda.synchronize()
    assert (pool.cpu().numpy() == pool_h).all()
    o_ref, lse_ref, err = oracle.sparse_mla(q.float().numpy(), pool_h, topk, spec.sm_scale, page_table=pt, row_req=rr)
    assert err == 0
    rel, lerr = compare_attention(out, lse, o_ref, lse_ref)
    print("c5 all %d rows: max rel err %.2e, lse err %.2e" % (spec.rows, rel, lerr))
