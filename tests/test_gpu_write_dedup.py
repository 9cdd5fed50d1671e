"""GPU parity of the quantized row write and dedup compaction: bit-exact
against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, to_dev

pytestmark = pytest.mark.gpu


def _write_both(kv, slots, n_slots, sentinel=0xA5, stride=None):
    pool_h = np.full((n_slots, 352), sentinel, np.uint8)
    err_h = oracle.quant_write(kv, slots, pool_h)
    pool_d = torch.full((n_slots, 352), sentinel, dtype=torch.uint8, device=DEV)
    err_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_d = to_dev(kv)
    if stride is not None:
        wide = torch.zeros((kv.shape[0], stride), dtype=torch.float32, device=DEV)
        wide[:, :576] = kv_d
        kv_d = wide[:, :576]
    kv4.quant_write(kv_d, to_dev(slots), pool_d, err_d)
    torch.cuda.synchronize()
    return pool_d.cpu().numpy(), pool_h, int(err_d.item()), err_h


def _assert_same_bytes(got, want):
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, "rows differ: %s; first row bytes differ at %s" % (
        bad[:8].tolist(), np.nonzero(got[bad[0]] != want[bad[0]])[0][:16].tolist())


def test_write_c4_full_size_bit_exact():
    spec = W.C4
    kv, slots = W.write_tokens(spec), W.write_slots(spec)
    got, want, e_d, e_h = _write_both(kv, slots, spec.n_slots)
    _assert_same_bytes(got, want)
    assert e_d == e_h == 0
    untouched = np.setdiff1d(np.arange(spec.n_slots), slots)
    assert (got[untouched] == 0xA5).all()


def _adversarial_rows():
    g = np.random.default_rng(99)
    rows = []
    z = np.zeros(576, np.float32)
    rows.append(z.copy())                                           # all zero
    rows.append(-z)                                                 # all -0.0
    rows.append(np.full(576, 1e-30, np.float32))                    # below every scale
    rows.append(np.full(576, -1e-40, np.float32))                   # fp32 subnormal
    rows.append(np.full(576, 3e38, np.float32) * g.choice([-1, 1], 576))   # saturation
    rows.append(np.float32(np.linspace(-1e5, 1e5, 576)))
    r = g.standard_normal(576).astype(np.float32)
    r[::7] = 0
    rows.append(r)
    # E4M3 scale midpoints (amax = 6 x midpoint, +-2 ulps) in every block
    v = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    base = (mids * np.float32(6.0)).astype(np.float32).view(np.int32)
    amax = np.concatenate([(base + k).view(np.float32) for k in range(-2, 3)])
    for i in range(0, amax.size, 32):
        r = (g.standard_normal(576) * 0.1).astype(np.float32)
        a = amax[i:i + 32]
        for b in range(a.size):
            r[16 * b:16 * b + 16] *= a[b]
            r[16 * b + (b % 16)] = a[b] * (1 if b % 2 else -1)
        r[512:] = np.resize(mids, 64) * g.choice([-1, 1], 64)            # rope at E4M3 midpoints
        rows.append(r.astype(np.float32))
    # E2M1 ties: amax = 6d exactly, other entries at d * {0.25, 0.75, ..., 5}
    # and up to 8 ulps either side (quotients at and next to every rounding
    # midpoint, where a quotient formed without dividing could round apart)
    ties = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for k in (-8, -4, -3, -2, -1, 0, 1, 2, 3, 4, 8):
        r = np.zeros(576, np.float32)
        for b in range(32):
            d = np.float32(oracle.e4m3_value(int(g.integers(1, 0x7F))))
            r[16 * b] = np.float32(6) * d
            t = (ties * d).astype(np.float32).view(np.int32) + k
            r[16 * b + 1:16 * b + 8] = t.view(np.float32) * g.choice([-1, 1], 7)
            r[16 * b + 8:16 * b + 16] = g.uniform(-6, 6, 8).astype(np.float32) * d
        rows.append(r)
    # NaN and infinity among ordinary values (a NaN is no block's maximum and
    # codes as zero; an infinite maximum saturates the scale)
    r = g.standard_normal(576).astype(np.float32)
    r[[3, 40, 77, 300, 515, 570]] = np.nan
    r[[100, 200]] = np.inf
    r[201] = -np.inf
    rows.append(r)
    return np.stack(rows).astype(np.float32)


def test_write_adversarial_rows_bit_exact():
    kv = _adversarial_rows()
    n = kv.shape[0]
    slots = np.arange(n, dtype=np.int32)[::-1].copy()
    got, want, e_d, e_h = _write_both(kv, slots, n + 3)
    _assert_same_bytes(got, want)
    assert e_d == e_h == 0


def test_write_pads_out_of_range_and_strided_rows():
    g = np.random.default_rng(5)
    kv = (g.standard_normal((70, 576)) * 3).astype(np.float32)
    slots = g.permutation(100)[:70].astype(np.int32)
    slots[3] = -1
    slots[10] = -100
    slots[20] = 100            # == n_slots: out of range, flagged
    slots[21] = 1 << 30
    got, want, e_d, e_h = _write_both(kv, slots, 100, stride=640)
    _assert_same_bytes(got, want)
    assert e_d == e_h == kv4.ERRBIT_SLOT


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1023])
def test_write_ragged_token_counts(n):
    g = np.random.default_rng(n)
    kv = g.standard_normal((n, 576)).astype(np.float32)
    slots = g.permutation(2 * n + 1)[:n].astype(np.int32)
    got, want, e_d, e_h = _write_both(kv, slots, 2 * n + 1)
    _assert_same_bytes(got, want)


def _dedup_both(idx, k=None):
    out_h, cnt_h = oracle.dedup_compact(idx[:, :k] if k is not None else idx)
    out_d, cnt_d = kv4.dedup_compact(to_dev(idx), k=k)
    torch.cuda.synchronize()
    return out_d.cpu().numpy(), cnt_d.cpu().numpy(), out_h, cnt_h


def test_dedup_c4_full_size_bit_exact():
    idx = W.dup_lists(W.C4)
    out_d, cnt_d, out_h, cnt_h = _dedup_both(idx)
    assert (cnt_d == cnt_h).all() and (cnt_h == W.C4.n_distinct).all()
    assert (out_d == out_h).all()


# 37 lists take the wide (1024-lane) workgroups for k > 512, 300 lists the
# 256- and 512-lane ones
@pytest.mark.parametrize("L", [37, 300])
@pytest.mark.parametrize("k", [1, 2, 5, 64, 255, 256, 257, 511, 512, 1000, 2048, 2051, 3000, 4096])
def test_dedup_lengths_and_edge_lists(k, L):
    g = np.random.default_rng(k)
    idx = g.integers(-4, max(3, k // 2), size=(L, k)).astype(np.int32)
    idx[0] = -1                                       # all padding
    idx[1] = 7                                        # one value
    idx[2] = np.arange(k, dtype=np.int32)             # all distinct
    idx[3] = g.integers(0, 2**31 - 1, size=k)         # large values
    idx[4, ::2] = 2**31 - 1
    out_d, cnt_d, out_h, cnt_h = _dedup_both(idx)
    assert (cnt_d == cnt_h).all()
    assert (out_d == out_h).all()


# More lists than workgroups fit on the chip at once: each workgroup compacts
# several lists in turn, loading the next while it works and clearing only
# the table slots the last one used.  Neighbouring lists differ in length of
# distinct runs, so a slot left set would show in the next list's output.
# (k, row width): each thread's entries come straight from aligned rows when k
# is a whole number of them (5, 300, 1000, 2048, 4096), through LDS otherwise
# (1002 and 3000 are not; rows of 1001 are not aligned to 16 bytes)
@pytest.mark.parametrize("k,width", [(5, 5), (300, 300), (1000, 1000), (1002, 1002), (1000, 1001), (2048, 2048),
                                     (3000, 3000), (4096, 4096)])
def test_dedup_many_lists(k, width):
    g = np.random.default_rng(50 + k + width)
    L = 4100
    idx = g.integers(-4, max(3, k // 2), size=(L, width)).astype(np.int32)
    idx[0] = -1                                       # all padding
    idx[1] = 7                                        # one value
    idx[2, :k] = np.arange(k, dtype=np.int32)         # all distinct
    idx[3, :k] = idx[2, :k][::-1]
    idx[L - 1] = g.integers(0, 2**31 - 1, size=width)  # large values, in the last (ragged) round
    idx[L - 2] = -1
    idx[1000::97, :k] = np.arange(k, dtype=np.int32) % 3   # three values
    out_d, cnt_d, out_h, cnt_h = _dedup_both(idx, k=k if width != k else None)
    assert (cnt_d == cnt_h).all()
    assert (out_d == out_h).all()


def test_dedup_strided_rows_and_prefix_k():
    g = np.random.default_rng(3)
    idx = g.integers(-2, 300, size=(50, 1000)).astype(np.int32)
    out_d, cnt_d, out_h, cnt_h = _dedup_both(idx, k=700)      # row stride 1000, k 700
    assert (cnt_d == cnt_h).all() and (out_d == out_h).all()


def test_dedup_empty_calls():
    idx = torch.zeros((0, 16), dtype=torch.int32, device=DEV)
    out, cnt = kv4.dedup_compact(idx)
    assert out.shape == (0, 16)
    idx = torch.zeros((5, 0), dtype=torch.int32, device=DEV)
    out, cnt = kv4.dedup_compact(idx)
    torch.cuda.synchronize()
    assert (cnt.cpu() == 0).all()


# ------------------------------------------- the write and the compaction in one call
def _write_and_dedup_both(kv, slots, n_slots, idx, k=None):
    """The combined call on the GPU against the oracle's write and dedup."""
    pool_h = np.full((n_slots, 352), 0xA5, np.uint8)
    err_h = oracle.quant_write(kv, slots, pool_h) if kv.shape[0] else 0
    out_h, cnt_h = oracle.dedup_compact(idx[:, :k] if k is not None else idx)
    pool_d = torch.full((n_slots, 352), 0xA5, dtype=torch.uint8, device=DEV)
    err_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    out_d, cnt_d = kv4.write_and_dedup(to_dev(kv), to_dev(slots), pool_d, to_dev(idx), k=k, err_word=err_d)
    torch.cuda.synchronize()
    return (pool_d.cpu().numpy(), pool_h, int(err_d.item()), err_h, out_d.cpu().numpy(), cnt_d.cpu().numpy(),
            out_h, cnt_h)


@pytest.mark.parametrize("n_tokens,n_lists,k", [
    (64, 64, 2048),      # the decode step: one kernel, lists of 2048
    (1, 1, 5),
    (0, 37, 1000),       # compaction only
    (70, 0, 16),         # write only
    (33, 5, 4096),       # longest lists
    (17, 300, 700),      # enough lists for the two separate kernels
    (9, 20, 1025),       # two entries a thread, k odd: staged through LDS
    (9, 20, 2051),       # four entries a thread, k not a multiple of four
])
def test_write_and_dedup_equals_oracle(n_tokens, n_lists, k):
    g = np.random.default_rng(1000 + n_tokens + n_lists + k)
    kv = (g.standard_normal((n_tokens, 576)) * 2).astype(np.float32)
    n_slots = 4 * n_tokens + 8
    slots = g.permutation(n_slots)[:n_tokens].astype(np.int32)
    if n_tokens > 4:
        slots[1] = -1                   # pad: nothing written
        slots[3] = n_slots + 5          # out of range: flagged
    idx = g.integers(-3, max(3, k // 3), size=(n_lists, k)).astype(np.int32)
    got, want, e_d, e_h, out_d, cnt_d, out_h, cnt_h = _write_and_dedup_both(kv, slots, n_slots, idx)
    _assert_same_bytes(got, want)
    assert e_d == e_h
    assert (cnt_d == cnt_h).all() and (out_d == out_h).all()


@pytest.mark.parametrize("k", [700, 1500, 3000])
def test_write_and_dedup_unaligned_lists(k):
    """Lists that start one entry into a device buffer, so that a thread's
    entries are not one aligned vector: the staged load path."""
    g = np.random.default_rng(77 + k)
    kv = g.standard_normal((12, 576)).astype(np.float32)
    slots = g.permutation(64)[:12].astype(np.int32)
    idx = g.integers(-2, k // 4, size=(9, k)).astype(np.int32)
    pool_h = np.full((64, 352), 0xA5, np.uint8)
    oracle.quant_write(kv, slots, pool_h)
    out_h, cnt_h = oracle.dedup_compact(idx)
    wide = torch.zeros((9, k + 1), dtype=torch.int32, device=DEV)
    wide[:, 1:] = to_dev(idx)
    pool_d = torch.full((64, 352), 0xA5, dtype=torch.uint8, device=DEV)
    out_d, cnt_d = kv4.write_and_dedup(to_dev(kv), to_dev(slots), pool_d, wide[:, 1:])
    torch.cuda.synchronize()
    _assert_same_bytes(pool_d.cpu().numpy(), pool_h)
    assert (cnt_d.cpu().numpy() == cnt_h).all() and (out_d.cpu().numpy() == out_h).all()


def test_write_and_dedup_prefix_k_and_step_inputs():
    """The decode step's own inputs (the long-context pool's new rows and
    lists) with a prefix k of a wider list buffer."""
    spec = W.C3
    g = np.random.default_rng(11)
    kv = g.standard_normal((spec.n_req, 576)).astype(np.float32)
    slots = g.permutation(4096)[:spec.n_req].astype(np.int32)
    idx = W.topk_lists(spec)
    wide = np.full((idx.shape[0], idx.shape[1] + 64), -7, np.int32)
    wide[:, :idx.shape[1]] = idx
    got, want, e_d, e_h, out_d, cnt_d, out_h, cnt_h = _write_and_dedup_both(kv, slots, 4096, wide, k=idx.shape[1])
    _assert_same_bytes(got, want)
    assert e_d == e_h == 0
    assert (cnt_d == cnt_h).all() and (out_d == out_h).all()
