"""Seeded random cases for the bit-exact kernels against the oracle: the row
write with amax/6 and with MSE-searched scales (both row formats) over rows
whose magnitudes span e^-40..e^40 with per-block factors e^-12..e^12, values
placed exactly on E2M1 rounding thresholds of representable scales, and
zeros, -0, infinities, NaN, the smallest denormal and 3.4e38 sprinkled in,
written to permuted slots with pads; and the per-list dedup over random list
counts, lengths (1..4096) and value ranges."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
from gpu_harness import DEV

pytestmark = pytest.mark.gpu

SEED = 99


def _rows(g):
    n_rope = 64 if g.integers(0, 2) else 0
    D = 512 + n_rope
    n = int(g.integers(1, 700))
    x = g.standard_normal((n, D)) * np.exp(g.uniform(-40, 40, size=(n, 1)))
    x[:, :512] *= np.repeat(np.exp(g.uniform(-12, 12, size=(n, 32))), 16, axis=1)
    d = 2.0 ** g.integers(-8, 8, size=(n, D)) * (1 + g.integers(0, 8, size=(n, D)) / 8)
    thr = g.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], size=(n, D)) * d * g.choice([-1, 1], size=(n, D))
    x = np.where(g.random((n, D)) < 0.05, thr, x)
    special = g.choice([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, 3.4e38], size=(n, D))
    x = np.where(g.random((n, D)) < 0.002, special, x).astype(np.float32)
    n_slots = n + int(g.integers(0, 50))
    slots = g.permutation(n_slots)[:n].astype(np.int32)
    slots[g.random(n) < 0.05] = -1
    return x, slots, n_slots, n_rope


@pytest.mark.parametrize("case", range(12))
@pytest.mark.parametrize("mse", [False, True])
def test_random_rows_write_bit_exact(case, mse):
    x, slots, n_slots, n_rope = _rows(np.random.default_rng([SEED, case]))
    ph = np.zeros((n_slots, oracle.row_bytes(512, n_rope)), dtype=np.uint8)
    e_ref = oracle.quant_write(x, slots, ph, 512, n_rope, mse=mse)
    pd = torch.zeros(ph.shape, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    write = kv4.quant_write_mse if mse else kv4.quant_write
    write(torch.from_numpy(x).to(DEV), torch.from_numpy(slots).to(DEV), pd, err_word=err)
    torch.cuda.synchronize()
    got = pd.cpu().numpy()
    assert (got == ph).all(), "%d bytes differ, first at %s" % ((got != ph).sum(), np.argwhere(got != ph)[0])
    assert int(err.item()) == e_ref


@pytest.mark.parametrize("case", range(12))
def test_random_lists_dedup_bit_exact(case):
    g = np.random.default_rng([SEED, 1000 + case])
    L, k = int(g.integers(1, 300)), int(g.integers(1, 4097))
    vr = int(g.choice([8, 100, 5000, 1 << 20, (1 << 31) - 1]))
    idx = g.integers(-2, vr, size=(L, k)).astype(np.int32)
    o_ref, c_ref = oracle.dedup_compact(idx)
    o, c = kv4.dedup_compact(torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    assert (o.cpu().numpy() == o_ref).all() and (c.cpu().numpy() == c_ref).all()
