"""GPU parity of the 288-byte rope-free row (README "60+ inference
optimizations & kernels", section "4-bit KV cache": GLM-5.3-Flash's rope-free
row): the write and the dequantizing gather bit-exact against the oracle with
n_rope = 0, attention within the tolerance of gpu_harness."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, compare_attention, q_for_oracle, to_dev

pytestmark = pytest.mark.gpu

RB = kv4.ROW_BYTES_ROPE_FREE
SCALE = 1.0 / np.sqrt(512.0)


def _pools_rope_free(kv):
    """Rope-free pools of the rows kv[:, :512], written by both sides."""
    kv = np.ascontiguousarray(kv[:, :512])
    slots = np.arange(kv.shape[0], dtype=np.int32)
    pool_h = np.zeros((kv.shape[0], RB), dtype=np.uint8)
    oracle.quant_write(kv, slots, pool_h, n_rope=0)
    pool_d = torch.zeros((kv.shape[0], RB), dtype=torch.uint8, device=DEV)
    kv4.quant_write(to_dev(kv), to_dev(slots), pool_d)
    torch.cuda.synchronize()
    return pool_d, pool_h


_CACHE = {}


def _spec_pools(spec):
    key = (spec.name, spec.n_slots, spec.seed)
    if key not in _CACHE:
        _CACHE[key] = _pools_rope_free(W.kv_rows_host(spec, 0, spec.n_slots))
    return _CACHE[key]


def test_rope_free_write_bit_exact():
    g = np.random.default_rng(21)
    n, n_slots = 700, 1000
    kv = (g.standard_normal((n, 512)) * 10.0 ** g.uniform(-2, 2, (n, 1))).astype(np.float32)
    kv[5] = 0.0
    kv[6, ::3] = 3e38
    kv[7] = np.float32(1e-40)
    slots = g.permutation(n_slots)[:n].astype(np.int32)
    slots[10] = -1
    slots[11] = n_slots + 2
    pool_h = np.full((n_slots, RB), 0xA5, np.uint8)
    err_h = oracle.quant_write(kv, slots, pool_h, n_rope=0)
    pool_d = torch.full((n_slots, RB), 0xA5, dtype=torch.uint8, device=DEV)
    err_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    wide = torch.zeros((n, 520), dtype=torch.float32, device=DEV)     # row stride 520 >= 512
    wide[:, :512] = to_dev(kv)
    kv4.quant_write(wide, to_dev(slots), pool_d, err_d)
    torch.cuda.synchronize()
    got = pool_d.cpu().numpy()
    bad = np.nonzero((got != pool_h).any(axis=1))[0]
    assert bad.size == 0, "rows differ: %s" % bad[:8].tolist()
    assert int(err_d.item()) == err_h == kv4.ERRBIT_SLOT


def test_rope_free_rows_are_the_rope_rows_without_their_rope():
    """The same values written in both formats: the first 288 bytes agree."""
    kv = W.kv_rows_host(W.C1, 0, 512)
    slots = to_dev(np.arange(512, dtype=np.int32))
    full = torch.zeros((512, kv4.ROW_BYTES), dtype=torch.uint8, device=DEV)
    free = torch.zeros((512, RB), dtype=torch.uint8, device=DEV)
    kv4.quant_write(to_dev(kv), slots, full)
    kv4.quant_write(to_dev(np.ascontiguousarray(kv[:, :512])), slots, free)
    torch.cuda.synchronize()
    assert torch.equal(full[:, :RB], free)


def test_rope_free_gather_bit_exact():
    spec = W.C1
    pool_d, pool_h = _spec_pools(spec)
    topk, pt = W.topk_lists(spec), W.page_table(spec)
    topk[0, 5] = -1
    rows, slots = kv4.gather_dequant(pool_d, to_dev(topk), page_table=to_dev(pt))
    torch.cuda.synchronize()
    assert rows.shape == (1, topk.shape[1], 512)
    got = rows.float().cpu().numpy()
    for j in range(topk.shape[1]):
        s = int(slots[0, j].item())
        want = np.zeros(512) if s < 0 else oracle.dequantize_row(pool_h[s], n_rope=0)
        assert (got[0, j] == want).all(), "entry %d" % j


def _attn(spec, q, topk, pt, *, num_splits=0, prefill=False, row_req=None):
    pool_d, pool_h = _spec_pools(spec)
    args = dict(page_table=to_dev(pt), row_req=None if row_req is None else to_dev(row_req))
    if prefill:
        out, lse = kv4.sparse_mla_prefill(to_dev(q), pool_d, to_dev(topk), SCALE, **args)
    else:
        out, lse = kv4.sparse_mla_decode(to_dev(q), pool_d, to_dev(topk), SCALE, num_splits=num_splits, **args)
    torch.cuda.synchronize()
    o_ref, lse_ref, _ = oracle.sparse_mla(q_for_oracle(q), pool_h, topk, SCALE, page_table=pt, row_req=row_req,
                                          n_rope=0)
    return compare_attention(out, lse, o_ref, lse_ref), (out, lse)


def _q512(spec):
    """The workload's queries without their rope dims."""
    return W.queries(spec)[:, :, :512].contiguous()


@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 8])
def test_rope_free_c1_decode(num_splits):
    spec = W.C1
    _attn(spec, _q512(spec), W.topk_lists(spec), W.page_table(spec), num_splits=num_splits)


def test_rope_free_c2_decode_full():
    spec = W.C2
    (rel, lerr), _ = _attn(spec, _q512(spec), W.topk_lists(spec), W.page_table(spec))
    print("rope-free c2 max rel err %.2e, lse err %.2e" % (rel, lerr))


def test_rope_free_prefill_rows_and_bitwise_single_split():
    spec = W.scaled(W.C5, n_query_rows=24, first_query_pos=W.C5.ctx - 24)
    q, topk, pt, rr = _q512(spec), W.topk_lists(spec), W.page_table(spec), W.row_req(spec)
    _, (a_out, a_lse) = _attn(spec, q, topk, pt, prefill=True, row_req=rr)
    _, (b_out, b_lse) = _attn(spec, q, topk, pt, num_splits=1, row_req=rr)
    assert torch.equal(a_out, b_out) and torch.equal(a_lse, b_lse)


@pytest.mark.parametrize("k", [1, 33, 100, 2051])
def test_rope_free_ragged_lengths(k):
    spec = W.scaled(W.C1, n_req=4, ctx=8192, n_pool_pages=160 * 4 + 8, n_heads=64, q_dtype="bf16", k=k, seed=7100)
    for s in (1, 3):
        _attn(spec, _q512(spec), W.topk_lists(spec), W.page_table(spec), num_splits=s)


def test_rope_free_fp32_queries_and_head_counts():
    spec = W.scaled(W.C1, n_heads=48, q_dtype="f32", seed=7200)
    _attn(spec, _q512(spec), W.topk_lists(spec), W.page_table(spec), num_splits=2)
    spec = W.scaled(W.C1, n_heads=128, q_dtype="bf16", seed=7300)
    _attn(spec, _q512(spec), W.topk_lists(spec), W.page_table(spec))


def test_rope_free_partial_plus_merge_equals_decode_bitwise():
    spec = W.C2
    pool_d, _ = _spec_pools(spec)
    q, topk, pt = to_dev(_q512(spec)), to_dev(W.topk_lists(spec)), to_dev(W.page_table(spec))
    for s in (2, 5):
        out, lse = kv4.sparse_mla_decode(q, pool_d, topk, SCALE, page_table=pt, num_splits=s)
        po, pl = kv4.sparse_mla_decode_partial(q, pool_d, topk, SCALE, s, page_table=pt)
        o2, l2 = kv4.merge_states(po.half().float(), pl)   # decode's workspace holds the parts' o as fp16
        torch.cuda.synchronize()
        assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_rope_free_needs_512_dim_queries():
    spec = W.C1
    pool_d, _ = _spec_pools(spec)
    with pytest.raises(ValueError):
        kv4.sparse_mla_decode(to_dev(W.queries(spec)), pool_d, to_dev(W.topk_lists(spec)), SCALE,
                              page_table=to_dev(W.page_table(spec)))
