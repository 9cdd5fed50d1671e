"""The full-size workloads in the launch configuration bench.py times, checked
on sampled outputs the oracle computes one by one: the long-context decode
pool (64 x 204,800 tokens, 4.6 GB of rows) and the 4096-query prefill."""
import numpy as np
import pytest
import torch

import bench
import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, compare_attention, q_for_oracle

pytestmark = pytest.mark.gpu


def test_c3_long_context_decode_sampled():
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
    sample = np.array([0, 21, 42, 63])
    uniq, rows, slots = bench.gathered_rows_host(spec, wl["pt_h"][sample], st["topk_h"][sample], dev)
    pool_h = np.zeros((uniq.size, 352), dtype=np.uint8)
    oracle.quant_write(rows, np.arange(uniq.size, dtype=np.int32), pool_h)
    got_rows = pool.index_select(0, torch.from_numpy(uniq).to(dev)).cpu().numpy()
    assert (got_rows == pool_h).all(), "sampled pool rows differ from the oracle's bytes"
    compact = np.searchsorted(uniq, slots).astype(np.int32)
    q = q_for_oracle(st["q"])[sample]
    o_ref, lse_ref, err = oracle.sparse_mla(q, pool_h, compact, spec.sm_scale)
    assert err == 0
    rel, lerr = compare_attention(out[sample], lse[sample], o_ref, lse_ref)
    print("c3 sampled (splits=%d) max rel err %.2e, lse err %.2e" % (S, rel, lerr))


def test_c5_prefill_full_size_sampled():
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
    sample = np.unique(np.concatenate([[0, 1, spec.rows - 1], np.random.default_rng(1).choice(spec.rows, 21)]))
    o_ref, lse_ref, err = oracle.sparse_mla(q.float().numpy()[sample], pool_h, topk[sample], spec.sm_scale,
                                            page_table=pt, row_req=rr[sample])
    assert err == 0
    rel, lerr = compare_attention(out[sample], lse[sample], o_ref, lse_ref)
    print("c5 full-size sampled max rel err %.2e, lse err %.2e" % (rel, lerr))
