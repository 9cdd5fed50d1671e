"""GPU parity of sparse MLA decode and prefill against the oracle.

The pool is quantized independently on both sides from the same seeded fp32
rows (the bytes are checked bit-exact first); the kernel's (o, lse) must match
the oracle's at the tolerance in gpu_harness."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, build_pools, compare_attention, q_for_oracle, to_dev

pytestmark = pytest.mark.gpu

_POOLS = {}


def pools(spec):
    """Device and host pools of a (small) workload, built once per module."""
    key = (spec.name, spec.n_slots, spec.seed)
    if key not in _POOLS:
        pool_d, pool_h = build_pools(spec)
        torch.cuda.synchronize()
        got = pool_d.cpu().numpy()
        assert (got == pool_h).all(), "pool bytes differ before any attention check"
        _POOLS[key] = (pool_d, pool_h)
    return _POOLS[key]


def _run(spec, q, topk, pt, *, row_req=None, num_splits=0, prefill=False, pool_pair=None, page_size=64,
         err_expect=0, o_tol=None, lse_tol=None):
    pool_d, pool_h = pool_pair if pool_pair is not None else pools(spec)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    args = dict(page_table=None if pt is None else to_dev(pt), row_req=None if row_req is None else to_dev(row_req),
                page_size=page_size, err_word=err)
    if prefill:
        out, lse = kv4.sparse_mla_prefill(to_dev(q), pool_d, to_dev(topk), spec.sm_scale, **args)
    else:
        out, lse = kv4.sparse_mla_decode(to_dev(q), pool_d, to_dev(topk), spec.sm_scale, num_splits=num_splits, **args)
    torch.cuda.synchronize()
    o_ref, lse_ref, err_ref = oracle.sparse_mla(q_for_oracle(q), pool_h, topk, spec.sm_scale, page_table=pt,
                                                row_req=row_req, page_size=page_size)
    assert int(err.item()) == err_ref == err_expect
    kw = {} if o_tol is None else {"o_tol": o_tol}
    if lse_tol is not None:
        kw["lse_tol"] = lse_tol
    return compare_attention(out, lse, o_ref, lse_ref, **kw), (out, lse)


# ------------------------------------------------------------ the configs
@pytest.mark.parametrize("num_splits", [0, 1, 2, 3, 8])
def test_c1_tiny_decode(num_splits):
    spec = W.C1
    (rel, lerr), _ = _run(spec, W.queries(spec), W.topk_lists(spec), W.page_table(spec), num_splits=num_splits)
    print("c1 splits=%d max rel err %.2e, lse err %.2e" % (num_splits, rel, lerr))


def test_c2_decode_head_share_full():
    spec = W.C2
    (rel, lerr), _ = _run(spec, W.queries(spec), W.topk_lists(spec), W.page_table(spec))
    print("c2 max rel err %.2e, lse err %.2e" % (rel, lerr))


def test_c5_prefill_rows_subset():
    spec = W.scaled(W.C5, n_query_rows=48, first_query_pos=W.C5.ctx - 48)
    q, topk, pt, rr = W.queries(spec), W.topk_lists(spec), W.page_table(spec), W.row_req(spec)
    pos = W.query_positions(spec)
    assert (topk < pos[:, None]).all()
    (rel, lerr), _ = _run(spec, q, topk, pt, row_req=rr, prefill=True)
    print("c5 subset max rel err %.2e, lse err %.2e" % (rel, lerr))


# ----------------------------------------------------- equalities of paths
def test_partial_plus_merge_equals_decode_bitwise():
    """Decode equals its two exposed halves bit for bit once the parts' o are
    rounded to fp16 (the workspace holds them so), for several split counts
    (16 and 17 included) run on one workspace, some twice in a row."""
    spec = W.C2
    pool_d, _ = pools(spec)
    q, topk, pt = to_dev(W.queries(spec)), to_dev(W.topk_lists(spec)), to_dev(W.page_table(spec))
    splits = (2, 5, 16, 16, 17, 3, 3)
    need = max(kv4.sparse_mla_decode_workspace(q, pool_d, topk, s, page_table=pt) for s in splits)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for s in splits:
        out, lse = kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=s, workspace=ws)
        po, pl = kv4.sparse_mla_decode_partial(q, pool_d, topk, spec.sm_scale, s, page_table=pt)
        ph, plh = kv4.sparse_mla_decode_partial(q, pool_d, topk, spec.sm_scale, s, page_table=pt,
                                                parts_dtype=torch.float16)
        o2, l2 = kv4.merge_states(po.half().float(), pl)
        o3, l3 = kv4.merge_states(ph, plh)
        torch.cuda.synchronize()
        # the fp16 parts are the fp32 parts rounded to nearest even (torch's rounding)
        assert torch.equal(ph, po.half()) and torch.equal(plh, pl), "splits=%d" % s
        assert torch.equal(out, o2) and torch.equal(lse, l2), "splits=%d" % s
        assert torch.equal(out, o3) and torch.equal(lse, l3), "splits=%d" % s


def test_fp16_parts_stay_within_their_rounding_bound():
    """Decode with fp16 parts differs from the merge of the fp32 parts by at
    most the fp16 rounding of the largest part, elementwise: the merged o is a
    convex combination of the parts, and rounding to nearest even moves each
    part's o by at most 2^-11 |o_s| (fp16's unit roundoff; |o_s| <= 2688) or,
    in fp16's subnormal range, 2^-25; the two merges' own fp32 roundings add
    a few fp32 ulp of the largest part."""
    spec = W.C2
    pool_d, _ = pools(spec)
    q, topk, pt = to_dev(W.queries(spec)), to_dev(W.topk_lists(spec)), to_dev(W.page_table(spec))
    for s in (2, 4, 8):
        o16, _ = kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=s)
        po, pl = kv4.sparse_mla_decode_partial(q, pool_d, topk, spec.sm_scale, s, page_table=pt)
        o32, _ = kv4.merge_states(po, pl)
        torch.cuda.synchronize()
        part_max = po.abs().amax(dim=0).double()                        # max_s |o_s| per element
        bound = 2.0 ** -11 * part_max + 2.0 ** -25 + 16 * 2.0 ** -24 * part_max
        diff = (o16.double() - o32.double()).abs()
        assert (diff <= bound).all(), "splits=%d: worst excess %.3g" % (s, float((diff - bound).max()))
        assert float(diff.max()) > 0.0          # the fp16 parts are in use


def test_prefill_equals_single_split_decode_bitwise():
    spec = W.scaled(W.C5, n_query_rows=16, first_query_pos=W.C5.ctx - 16)
    pool_d, _ = pools(spec)
    q, topk, pt, rr = (to_dev(W.queries(spec)), to_dev(W.topk_lists(spec)), to_dev(W.page_table(spec)),
                       to_dev(W.row_req(spec)))
    a = kv4.sparse_mla_prefill(q, pool_d, topk, spec.sm_scale, page_table=pt, row_req=rr)
    b = kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, row_req=rr, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_split_counts_agree():
    spec = W.C2
    pool_d, _ = pools(spec)
    q, topk, pt = to_dev(W.queries(spec)), to_dev(W.topk_lists(spec)), to_dev(W.page_table(spec))
    ref = kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=1)
    for s in (2, 4, 7, 64):
        out = kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=s)
        compare_attention(out[0], out[1], ref[0].double().cpu().numpy(), ref[1].double().cpu().numpy())


# ----------------------------------------------------------- shapes, edges
SMALL = W.scaled(W.C1, n_req=4, ctx=2048, n_pool_pages=160, n_heads=64, q_dtype="bf16", k=256, seed=7000)


@pytest.mark.parametrize("k", [1, 2, 31, 32, 33, 100, 2051, 4500])
def test_ragged_list_lengths(k):
    spec = W.scaled(SMALL, ctx=8192, n_pool_pages=160 * 4 + 8, k=k)
    q, topk, pt = W.queries(spec), W.topk_lists(spec), W.page_table(spec)
    for s in (1, 0, 3):
        _run(spec, q, topk, pt, num_splits=s)


@pytest.mark.parametrize("h", [16, 32, 48, 80, 128])
def test_head_counts(h):
    spec = W.scaled(SMALL, n_heads=h)
    _run(spec, W.queries(spec), W.topk_lists(spec), W.page_table(spec))
    _run(spec, W.queries(spec), W.topk_lists(spec), W.page_table(spec), prefill=True)


# Rows a multiple of 8: the decode's merge takes each row on the XCD that
# wrote its parts (a reordering of its work only); 48 and 80 heads give
# groups of states that are not powers of two, 128 heads two head blocks.
@pytest.mark.parametrize("h", [48, 80, 128])
@pytest.mark.parametrize("rows", [8, 16])
def test_decode_rows_multiple_of_eight(h, rows):
    spec = W.scaled(SMALL, n_req=rows, n_heads=h, n_pool_pages=rows * 40)
    q, topk, pt = W.queries(spec), W.topk_lists(spec), W.page_table(spec)
    for s in (0, 3, 5):
        _run(spec, q, topk, pt, num_splits=s)


def test_fp32_queries():
    spec = W.scaled(SMALL, q_dtype="f32")
    q = W.queries(spec)
    assert q.dtype == torch.float32
    (rel, _), _ = _run(spec, q, W.topk_lists(spec), W.page_table(spec), num_splits=2)
    print("fp32 q max rel err %.2e" % rel)


def test_query_scale_extremes():
    """Queries far from N(0, 1) scale: tiny, large, one dominant head."""
    spec = SMALL
    base = W.queries(spec).float()
    for mul in (1e-30, 1e-6, 1e4):
        q = (base * mul).to(torch.bfloat16)
        _run(spec, q, W.topk_lists(spec), W.page_table(spec), num_splits=2)
    q = base.clone()
    q[:, 3] *= 1e5
    q[:, 5] = 0
    _run(spec, q.to(torch.bfloat16), W.topk_lists(spec), W.page_table(spec))


def test_invalid_entries_are_skipped_and_flagged():
    spec = SMALL
    q, topk, pt = W.queries(spec), W.topk_lists(spec).copy(), W.page_table(spec).copy()
    topk[0, 5] = -1
    topk[0, 9] = -77
    _run(spec, q, topk, pt)
    t2 = topk.copy()
    t2[1, 7] = spec.ctx + 5                      # past this request's table
    _run(spec, q, t2, pt, err_expect=kv4.ERRBIT_PAGE)
    pt3 = pt.copy()
    pt3[2, 0] = -1                               # unmapped page
    t3 = topk.copy()
    t3[2, :4] = [0, 1, 2, 63]
    _run(spec, q, t3, pt3, err_expect=kv4.ERRBIT_PAGE)
    t4 = topk.copy()
    t4[3, 0] = spec.n_slots + 3                  # physical slot past the pool (no page table)
    t4[3, 1:] = np.arange(spec.k - 1) * 3
    _run(spec, q, t4, None, err_expect=kv4.ERRBIT_SLOT)


def test_empty_and_duplicate_lists():
    spec = SMALL
    q, topk, pt = W.queries(spec), W.topk_lists(spec).copy(), W.page_table(spec)
    topk[0] = -1                                 # empty list
    topk[1, :] = topk[1, 0]                      # one key repeated k times
    topk[2, 100:] = topk[2, :100].repeat(2)[: spec.k - 100]
    for s in (1, 4):
        (_, _), (out, lse) = _run(spec, q, topk, pt, num_splits=s)
        assert (out[0] == 0).all() and torch.isneginf(lse[0]).all()


def test_physical_slots_and_shared_table():
    spec = SMALL
    q, topk, pt = W.queries(spec), W.topk_lists(spec), W.page_table(spec)
    slots = (pt[np.arange(spec.n_req)[:, None], topk >> 6] * 64 + (topk & 63)).astype(np.int32)
    _run(spec, q, slots, None)
    rr = np.int32([2, 2, 0, 1])
    _run(spec, q, topk, pt, row_req=rr)


@pytest.mark.parametrize("page_size", [16, 128])
def test_other_page_sizes(page_size):
    spec = SMALL
    n_pages = spec.n_slots // page_size
    g = np.random.default_rng(page_size)
    per = spec.ctx // page_size
    pt = g.permutation(n_pages)[: spec.n_req * per].astype(np.int32).reshape(spec.n_req, per)
    _run(spec, W.queries(spec), W.topk_lists(spec), pt, page_size=page_size)


@pytest.mark.parametrize("n_pages", [4096, 4097, 9000])
def test_long_page_table_rows(n_pages):
    """Page-table rows of 4096 to 9000 entries over 16-token pages, naming
    physical pages more than once; the last position of the table and one past
    it; decode with bf16 and fp32 queries, and prefill."""
    spec = W.scaled(SMALL, n_req=2, ctx=16 * n_pages, k=300)
    g = np.random.default_rng(n_pages)
    pt = g.integers(0, spec.n_slots // 16, size=(spec.n_req, n_pages)).astype(np.int32)
    q, topk = W.queries(spec), W.topk_lists(spec).copy()
    topk[0, 0] = spec.ctx - 1
    _run(spec, q, topk, pt, page_size=16)
    _run(spec, q, topk, pt, page_size=16, num_splits=2)
    _run(W.scaled(spec, q_dtype="f32"), W.queries(W.scaled(spec, q_dtype="f32")), topk, pt, page_size=16)
    _run(spec, q, topk, pt, page_size=16, prefill=True, row_req=np.int32([1, 0]))
    topk[1, 3] = spec.ctx
    _run(spec, q, topk, pt, page_size=16, err_expect=kv4.ERRBIT_PAGE)


# ------------------------------------------------- the path is exercised
def test_unselected_rows_do_not_matter_selected_rows_do():
    spec = SMALL
    pool_d, pool_h = pools(spec)
    q, topk, pt = to_dev(W.queries(spec)), W.topk_lists(spec), W.page_table(spec)
    sel = set((pt[r, topk[r] >> 6] * 64 + (topk[r] & 63)).tolist()[i] for r in range(spec.n_req)
              for i in range(spec.k))
    unsel = np.setdiff1d(np.arange(spec.n_slots), np.array(sorted(sel)))
    base = kv4.sparse_mla_decode(q, pool_d, to_dev(topk), spec.sm_scale, page_table=to_dev(pt), num_splits=2)
    p2 = pool_d.clone()
    p2[to_dev(unsel.astype(np.int64))] ^= 0x5A
    a = kv4.sparse_mla_decode(q, p2, to_dev(topk), spec.sm_scale, page_table=to_dev(pt), num_splits=2)
    p3 = pool_d.clone()
    one = int(pt[0, topk[0, 17] >> 6] * 64 + (topk[0, 17] & 63))
    p3[one, 40] ^= 0x11                           # one code byte of one selected row
    b = kv4.sparse_mla_decode(q, p3, to_dev(topk), spec.sm_scale, page_table=to_dev(pt), num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(base[0], a[0]) and torch.equal(base[1], a[1])
    changed = (base[0] != b[0]).any(dim=-1)
    assert changed[0].sum() > 0 and not changed[1:].any()


def test_negative_controls_fail_parity():
    """Planted on the CPU side: an oracle fed a doubled scale, swapped nibbles,
    an off-by-one page or a dropped rope must disagree with the kernel."""
    spec = SMALL
    pool_d, pool_h = pools(spec)
    q, topk, pt = W.queries(spec), W.topk_lists(spec), W.page_table(spec)
    out, lse = kv4.sparse_mla_decode(to_dev(q), pool_d, to_dev(topk), spec.sm_scale, page_table=to_dev(pt))
    torch.cuda.synchronize()
    rows = (pt[np.arange(spec.n_req)[:, None], topk >> 6] * 64 + (topk & 63)).reshape(-1)
    bad_scale = pool_h.copy()
    bad_scale[rows, 256:288] = np.where(bad_scale[rows, 256:288] > 0, bad_scale[rows, 256:288] + 8, 0)
    bad_nibble = pool_h.copy()
    bad_nibble[rows, :256] = (bad_nibble[rows, :256] >> 4) | (bad_nibble[rows, :256] << 4)
    no_rope = pool_h.copy()
    no_rope[rows, 288:] = 0
    cases = {"doubled scale": (bad_scale, pt), "swapped nibbles": (bad_nibble, pt), "dropped rope": (no_rope, pt),
             "off-by-one page": (pool_h, (pt + 1) % (spec.n_slots // 64))}
    for name, (ph, ptx) in cases.items():
        o_ref, lse_ref, _ = oracle.sparse_mla(q_for_oracle(q), ph, topk, spec.sm_scale, page_table=ptx)
        with pytest.raises(AssertionError):
            compare_attention(out, lse, o_ref, lse_ref)


def test_graph_replay_matches_eager_bitwise():
    spec = W.C2
    pool_d, _ = pools(spec)
    q, topk, pt = to_dev(W.queries(spec)), to_dev(W.topk_lists(spec)), to_dev(W.page_table(spec))
    s = kv4.sparse_mla_decode_splits(q, pool_d, topk, page_table=pt)
    ws = torch.empty(kv4.sparse_mla_decode_workspace(q, pool_d, topk, s, page_table=pt), dtype=torch.uint8, device=DEV)
    out = torch.empty((spec.n_req, spec.n_heads, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((spec.n_req, spec.n_heads), dtype=torch.float32, device=DEV)
    ref = kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=s, workspace=ws)
    ref = (ref[0].clone(), ref[1].clone())
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=s, workspace=ws,
                              out=out, lse=lse)              # warm-up outside capture
        with torch.cuda.graph(graph, stream=stream):
            kv4.sparse_mla_decode(q, pool_d, topk, spec.sm_scale, page_table=pt, num_splits=s, workspace=ws,
                                  out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(stream)
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), "replay %d differs" % i


@pytest.mark.parametrize("num_splits", [1, 3])
def test_rising_scores_take_the_exact_second_pass(num_splits):
    """Lists ordered by increasing score with large queries: the first tile's
    maximum sits far below later scores (P would overflow fp16 against it), so
    the kernel must fall back to its second pass with the exact maximum."""
    spec = W.scaled(SMALL, k=512, ctx=2048)
    pool_d, pool_h = pools(spec)
    q = (W.queries(spec).float() * 40.0).to(torch.bfloat16)
    topk, pt = W.topk_lists(spec), W.page_table(spec)
    _, _, _, probs = oracle.sparse_mla(q_for_oracle(q), pool_h, topk, spec.sm_scale, page_table=pt, want_probs=True)
    order = np.argsort(np.log(probs[:, 0, :] + 1e-300), axis=1)          # head 0's scores, ascending
    rising = np.take_along_axis(topk, order, axis=1).astype(np.int32)
    _run(spec, q, rising, pt, num_splits=num_splits)


def _rising_lists(spec, q, pool_h, topk, pt):
    """The lists reordered by head 0's score, ascending, and the largest log2
    gap (over rows) between head 0's best score in the first 32 entries and its
    best score in the whole list."""
    _, _, _, probs = oracle.sparse_mla(q_for_oracle(q), pool_h, topk, spec.sm_scale, page_table=pt, want_probs=True)
    order = np.argsort(np.log(probs[:, 0, :] + 1e-300), axis=1)
    rising = np.take_along_axis(topk, order, axis=1).astype(np.int32)
    p = np.take_along_axis(probs[:, 0, :], order, axis=1)
    gap = np.log2(p.max(axis=1) / p[:, :32].max(axis=1))
    return rising, float(gap.max())


@pytest.mark.parametrize("mode", ["decode_one_split", "prefill"])
def test_rising_scores_redo_across_chunks(mode):
    """Lists of 4096 entries (two translation chunks of 2048) ordered by rising
    score: head 0's best score lies more than 16 (log2) above the first tile's,
    so P against the first tile's reference would overflow fp16 (max 65504 <
    2^16) and the output would be inf/NaN.  Matching the oracle therefore
    shows the exact second pass ran, re-translating the first chunk."""
    spec = W.scaled(SMALL, ctx=8192, n_pool_pages=160 * 4 + 8, k=4096, seed=7300)
    pool_d, pool_h = pools(spec)
    q = (W.queries(spec).float() * 40.0).to(torch.bfloat16)
    topk, pt = W.topk_lists(spec), W.page_table(spec)
    rising, gap = _rising_lists(spec, q, pool_h, topk, pt)
    assert gap > 16.0, "the case does not force the second pass (gap %.1f)" % gap
    if mode == "prefill":
        _run(spec, q, rising, pt, prefill=True, row_req=np.arange(spec.n_req, dtype=np.int32),
             pool_pair=(pool_d, pool_h))
    else:
        _run(spec, q, rising, pt, num_splits=1, pool_pair=(pool_d, pool_h))


def test_rising_scores_force_the_second_pass_within_a_chunk():
    """k = 2048 in one chunk, decode with one split and with the automatic
    split count; the same overflow argument as above."""
    spec = W.scaled(SMALL, ctx=8192, n_pool_pages=160 * 4 + 8, k=2048, seed=7400)
    pool_d, pool_h = pools(spec)
    q = (W.queries(spec).float() * 40.0).to(torch.bfloat16)
    topk, pt = W.topk_lists(spec), W.page_table(spec)
    rising, gap = _rising_lists(spec, q, pool_h, topk, pt)
    assert gap > 16.0, "the case does not force the second pass (gap %.1f)" % gap
    _run(spec, q, rising, pt, num_splits=1, pool_pair=(pool_d, pool_h))
    _run(spec, q, rising, pt, num_splits=0, pool_pair=(pool_d, pool_h))


@pytest.mark.parametrize("sm_scale", [-1.0 / 24.0, 0.0, 3.0])
def test_softmax_scale_of_any_sign(sm_scale):
    """The softmax scale is any finite number: negative scales reverse the
    order of the scores (the reference comes from the scaled scores, not the
    raw ones), zero makes every weight equal."""
    spec = W.scaled(SMALL, k=300, seed=7500, softmax_scale=sm_scale)
    q, topk, pt = W.queries(spec), W.topk_lists(spec), W.page_table(spec)
    _run(spec, q, topk, pt, num_splits=0)
    _run(spec, q, topk, pt, prefill=True, row_req=np.arange(spec.n_req, dtype=np.int32))
