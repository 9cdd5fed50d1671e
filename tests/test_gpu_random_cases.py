"""Seeded random attention cases against the oracle: row format, page size,
requests and their page counts, a page-table entry beyond the pool, head
count, list length, decode or prefill (with a request per query row), query
dtype and magnitude, softmax scale and split count are all drawn per case;
lists hold invalid positions (negative, past the request's pages) and
repeats.  Each case checks the pool bytes, the error word, the outputs
within the tolerance, and (split decode) the fp16-part halves bit for bit
against the decode call."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
from gpu_harness import DEV, compare_attention, q_for_oracle

pytestmark = pytest.mark.gpu

SEED = 777


def _case(case):
    g = np.random.default_rng([SEED, case])
    rope = bool(g.integers(0, 2))
    n_rope = 64 if rope else 0
    D = 512 + n_rope
    ps = int(g.choice([16, 64, 128]))
    n_req = int(g.integers(1, 5))
    pages = [int(g.integers(1, 40)) for _ in range(n_req)]
    pool_pages = sum(pages) + int(g.integers(0, 8))
    perm = g.permutation(pool_pages)
    pt = np.full((n_req, max(pages)), -1, dtype=np.int32)
    o = 0
    for r in range(n_req):
        pt[r, :pages[r]] = perm[o:o + pages[r]]
        o += pages[r]
    if g.random() < 0.3:
        pt[0, int(g.integers(0, pages[0]))] = pool_pages + 3      # a page beyond the pool
    H = int(g.choice([16, 32, 48, 64, 80, 96, 112, 128]))
    k = int(g.integers(1, 1500))
    prefill = bool(g.integers(0, 2))
    if prefill:
        rows = int(g.integers(1, 7))
        row_req = g.integers(0, n_req, size=rows).astype(np.int32)
    else:
        rows, row_req = n_req, None
    ctx = [pages[row_req[i] if prefill else i] * ps for i in range(rows)]
    topk = np.stack([g.integers(-3, ctx[i] + 5, size=k) for i in range(rows)]).astype(np.int32)
    n_slots = pool_pages * ps
    kv = (g.standard_normal((n_slots, D)) * np.exp(g.uniform(-3, 3, size=(n_slots, 1)))).astype(np.float32)
    kv[g.random((n_slots, D)) < 0.01] *= 20
    q32 = (g.standard_normal((rows, H, D)) * np.exp(g.uniform(-4, 3))).astype(np.float32)
    qdt = torch.bfloat16 if g.integers(0, 2) else torch.float32
    scale = float(g.uniform(0.5, 4.0) / np.sqrt(D))
    splits = int(g.choice([0, 1, 2, 3, 5, 8, 13, 16]))
    return dict(n_rope=n_rope, ps=ps, pt=pt, topk=topk, row_req=row_req, kv=kv, q32=q32, qdt=qdt, scale=scale,
                splits=splits, prefill=prefill)


@pytest.mark.parametrize("case", range(24))
def test_random_case(case):
    c = _case(case)
    n_rope, ps = c["n_rope"], c["ps"]
    kv = c["kv"]
    n_slots = kv.shape[0]
    pool_h = np.zeros((n_slots, oracle.row_bytes(512, n_rope)), dtype=np.uint8)
    oracle.quant_write(kv, np.arange(n_slots, dtype=np.int32), pool_h, 512, n_rope)
    pool = torch.zeros(pool_h.shape, dtype=torch.uint8, device=DEV)
    kv4.quant_write(torch.from_numpy(kv).to(DEV), torch.arange(n_slots, dtype=torch.int32, device=DEV), pool)
    q = torch.from_numpy(c["q32"]).to(DEV, c["qdt"])
    pt, topk, rr = c["pt"], c["topk"], c["row_req"]
    o_ref, l_ref, e_ref = oracle.sparse_mla(q_for_oracle(q), pool_h, topk, c["scale"], page_table=pt, row_req=rr,
                                            page_size=ps, n_latent=512, n_rope=n_rope)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ptd, td = torch.from_numpy(pt).to(DEV), torch.from_numpy(topk).to(DEV)
    rrd = None if rr is None else torch.from_numpy(rr).to(DEV)
    if c["prefill"]:
        out, lse = kv4.sparse_mla_prefill(q, pool, td, c["scale"], page_table=ptd, row_req=rrd, page_size=ps,
                                          err_word=err)
    else:
        out, lse = kv4.sparse_mla_decode(q, pool, td, c["scale"], page_table=ptd, page_size=ps, err_word=err,
                                         num_splits=c["splits"])
    torch.cuda.synchronize()
    assert (pool.cpu().numpy() == pool_h).all(), "pool bytes differ from the oracle's"
    assert int(err.item()) == e_ref
    compare_attention(out, lse, o_ref, l_ref)
    if not c["prefill"]:
        S = c["splits"] or kv4.sparse_mla_decode_splits(q, pool, td, page_table=ptd, page_size=ps)
        if S > 1:
            ph, pl = kv4.sparse_mla_decode_partial(q, pool, td, c["scale"], S, page_table=ptd, page_size=ps,
                                                   parts_dtype=torch.float16)
            o2, l2 = kv4.merge_states(ph, pl)
            torch.cuda.synchronize()
            assert torch.equal(o2, out) and torch.equal(l2, lse)
