"""GPU parity of the quantized write with MSE-searched block scales: every
byte equal to the oracle's on the same seeded inputs, in both row formats."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W
from gpu_harness import DEV, to_dev
from test_gpu_write_dedup import _adversarial_rows

pytestmark = pytest.mark.gpu


def _write_both(kv, slots, n_slots, rope_free=False, stride=None):
    dim, rb = (512, 288) if rope_free else (576, 352)
    pool_h = np.full((n_slots, rb), 0xA5, np.uint8)
    err_h = oracle.quant_write(kv, slots, pool_h, n_rope=0 if rope_free else 64, mse=True)
    pool_d = torch.full((n_slots, rb), 0xA5, dtype=torch.uint8, device=DEV)
    err_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    kv_d = to_dev(kv)
    if stride is not None:
        wide = torch.zeros((kv.shape[0], stride), dtype=torch.float32, device=DEV)
        wide[:, :dim] = kv_d
        kv_d = wide[:, :dim]
    kv4.quant_write_mse(kv_d, to_dev(slots), pool_d, err_d)
    torch.cuda.synchronize()
    return pool_d.cpu().numpy(), pool_h, int(err_d.item()), err_h


def _assert_same_bytes(got, want):
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, "rows differ: %s; first row bytes differ at %s" % (
        bad[:8].tolist(), np.nonzero(got[bad[0]] != want[bad[0]])[0][:16].tolist())


def _mse_rows(seed):
    """Blocks that exercise the search: exact fits at scales other than
    amax/6, single values, all-equal blocks, outliers, heavy tails, tiny and
    huge magnitudes (subnormal scales, the largest scale, denormal squares),
    sparse blocks, and values on E2M1 thresholds of neighbouring scales."""
    g = np.random.default_rng(seed)
    rows = []
    for kind in range(12):
        x = g.standard_normal(576)
        if kind == 0:                                     # exact fits, largest code below 6
            for b in range(32):
                d = oracle.e4m3_value(int(g.integers(1, 0x7F)))
                top = int(g.integers(1, 8))
                c = g.integers(0, top + 1, 16) | (g.integers(0, 2, 16) << 3)
                c[g.integers(0, 16)] = top
                x[16 * b:16 * b + 16] = [oracle.e2m1_value(int(v)) * d for v in c]
        elif kind == 1:                                   # one value per block
            x[:512] = 0
            x[:512:16] = g.uniform(-100, 100, 32)
        elif kind == 2:                                   # all equal within a block
            x[:512] = np.repeat(g.uniform(-5, 5, 32), 16)
        elif kind == 3:
            x[g.random(576) < 0.05] *= 50.0
        elif kind == 4:
            x = g.standard_cauchy(576)
        elif kind == 5:
            x *= 1e-3
        elif kind == 6:
            x *= 1e-20                                    # squares in the fp32 denormal range
        elif kind == 7:
            x *= 600.0
        elif kind == 8:
            x[g.random(576) < 0.85] = 0.0
        elif kind == 9:                                   # on thresholds of scale 2d and d/2
            for b in range(32):
                d = oracle.e4m3_value(int(g.integers(0x20, 0x60)))
                t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
                x[16 * b:16 * b + 16] = g.choice(np.concatenate([t * d, t * 2 * d, t * d / 2, [6 * d]]), 16)
                x[16 * b] = 6 * d
        elif kind == 10:
            x *= np.power(10.0, g.uniform(-6, 6, 576))
        elif kind == 11:                                  # values near the largest scale's range
            x *= 448.0 * 6.0 / 3.0
        rows.append(x.astype(np.float32))
    return np.stack(rows)


def test_mse_write_c4_full_size_bit_exact():
    spec = W.C4
    kv, slots = W.write_tokens(spec), W.write_slots(spec)
    got, want, e_d, e_h = _write_both(kv, slots, spec.n_slots)
    _assert_same_bytes(got, want)
    assert e_d == e_h == 0
    untouched = np.setdiff1d(np.arange(spec.n_slots), slots)
    assert (got[untouched] == 0xA5).all()
    # the search changed many scales, and none for the worse
    base = np.full_like(want, 0xA5)
    oracle.quant_write(kv, slots, base)
    assert (want[slots, 256:288] != base[slots, 256:288]).mean() > 0.3


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mse_write_search_cases_bit_exact(seed):
    kv = _mse_rows(seed)
    slots = np.arange(kv.shape[0], dtype=np.int32)
    got, want, e_d, e_h = _write_both(kv, slots, kv.shape[0])
    _assert_same_bytes(got, want)


def test_mse_write_adversarial_rows_bit_exact():
    kv = _adversarial_rows()
    n = kv.shape[0]
    slots = np.arange(n, dtype=np.int32)[::-1].copy()
    got, want, e_d, e_h = _write_both(kv, slots, n + 3)
    _assert_same_bytes(got, want)
    assert e_d == e_h == 0


def test_mse_write_pads_out_of_range_and_strided_rows():
    g = np.random.default_rng(5)
    kv = (g.standard_normal((70, 576)) * 3).astype(np.float32)
    slots = g.permutation(100)[:70].astype(np.int32)
    slots[3] = -1
    slots[20] = 100
    slots[21] = 1 << 30
    got, want, e_d, e_h = _write_both(kv, slots, 100, stride=640)
    _assert_same_bytes(got, want)
    assert e_d == e_h == kv4.ERRBIT_SLOT


@pytest.mark.parametrize("n", [1, 3, 7, 8, 9, 1023])
def test_mse_write_ragged_token_counts(n):
    g = np.random.default_rng(100 + n)
    kv = (g.standard_normal((n, 576)) * np.power(10.0, g.uniform(-2, 2, (n, 1)))).astype(np.float32)
    slots = g.permutation(2 * n + 1)[:n].astype(np.int32)
    got, want, e_d, e_h = _write_both(kv, slots, 2 * n + 1)
    _assert_same_bytes(got, want)


def test_mse_write_rope_free_bit_exact():
    g = np.random.default_rng(17)
    kv = np.concatenate([_mse_rows(7)[:, :512],
                         (g.standard_normal((300, 512)) * np.power(10.0, g.uniform(-2, 2, (300, 1))))]).astype(
                             np.float32)
    n = kv.shape[0]
    slots = g.permutation(n + 10)[:n].astype(np.int32)
    slots[5] = -1
    slots[6] = n + 10
    got, want, e_d, e_h = _write_both(kv, slots, n + 10, rope_free=True, stride=520)
    _assert_same_bytes(got, want)
    assert e_d == e_h == kv4.ERRBIT_SLOT


def test_mse_write_empty_call():
    pool = torch.zeros((4, 352), dtype=torch.uint8, device=DEV)
    kv4.quant_write_mse(torch.zeros((0, 576), device=DEV), torch.zeros((0,), dtype=torch.int32, device=DEV), pool)
    torch.cuda.synchronize()
    assert (pool.cpu() == 0).all()
