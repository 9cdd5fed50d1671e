"""kv4_sparse_mla_decode_noalloc (the split parts in the library's scratch array,
for callers that cannot allocate) against kv4_sparse_mla_decode with a
workspace: the same kernels, so the results are equal bit for bit.  Two calls
in a row, the second on a smaller input, each checked; and a call needing more
than the array holds is refused before anything runs."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import workloads as W
from gpu_harness import DEV, build_pools, to_dev

pytestmark = pytest.mark.gpu


def _case(spec):
    pool_d, _ = build_pools(spec)
    return pool_d, to_dev(W.queries(spec)), to_dev(W.topk_lists(spec)), to_dev(W.page_table(spec))


def _both(spec, case, num_splits):
    pool_d, q, topk, pt = case
    err_a = torch.zeros(1, dtype=torch.int32, device=DEV)
    err_b = torch.zeros(1, dtype=torch.int32, device=DEV)
    out_a, lse_a = kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=num_splits,
                                         err_word=err_a)
    out_b, lse_b = kv4.sparse_mla_decode_noalloc(q, pool_d, topk, spec.sm_scale, page_table=pt,
                                                 num_splits=num_splits, err_word=err_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    assert int(err_a.item()) == int(err_b.item())
    assert torch.isfinite(out_b).all()


def test_noalloc_matches_decode_on_two_calls():
    big = W.scaled(W.C2, n_req=8, ctx=8192, n_pool_pages=1100, k=2048, seed=7600)
    small = W.scaled(W.C1, n_req=2, ctx=2048, n_pool_pages=70, n_heads=16, k=300, seed=7601)
    case_big, case_small = _case(big), _case(small)
    S = kv4.sparse_mla_decode_splits(case_big[1], case_big[0], case_big[2], page_table=case_big[3])
    assert S > 1                                   # the scratch array is in use
    _both(big, case_big, 0)
    _both(small, case_small, 0)                    # smaller parts over the first call's leftovers
    _both(small, case_small, 3)
    _both(big, case_big, 16)


def test_noalloc_refuses_more_than_its_scratch():
    """64 rows x 64 heads x 64 splits of fp16 parts (268 MB) exceed the array:
    refused on the host, nothing enqueued, the output left as it was."""
    spec = W.scaled(W.C2, n_req=8, ctx=8192, n_pool_pages=1100, k=2048, seed=7600)
    pool_d, q, topk, pt = _case(spec)
    q64, topk64 = torch.cat([q] * 8), torch.cat([topk] * 8)
    rr = torch.arange(64, dtype=torch.int32, device=DEV) % 8
    assert kv4.MAX_SPLITS * 64 * 64 * 512 * 2 > kv4.noalloc_scratch_bytes()
    out = torch.full((64, 64, 512), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(kv4.Kv4Error) as e:
        kv4.sparse_mla_decode_noalloc(q64, pool_d, topk64, spec.sm_scale, page_table=pt, row_req=rr, out=out,
                                      num_splits=kv4.MAX_SPLITS)
    assert e.value.status == 5 and "noalloc" in str(e.value)
    torch.cuda.synchronize()
    assert (out == 3.0).all()
