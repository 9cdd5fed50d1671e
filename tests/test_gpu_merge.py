"""GPU parity of the exported (o, lse) merge, kv4_merge_states and its fp16-part
form, against the oracle's merge (README "60+ inference optimizations &
kernels", section "Parallelism and disaggregation": each rank returns (o, lse)
for a cross-rank merge).  Parts are arbitrary, not produced by this library:
any count from 1 to 64, any dim from 4 to 4096, lse spread over +-80 with
empty (-inf) parts mixed in.

Tolerance: the merge is fp32 arithmetic on the given parts (weights exp(lse_s -
M) by the fp32 exponential, their sum, and a weighted sum of at most 64 terms),
so its error is a few units of fp32 rounding per term: below 64 * 2^-22 of the
state's largest |o| and of |lse| plus 2^-20 absolute; the test allows 2e-5 of
the ∞-norm and 2e-5 + 2^-20 |lse|."""
import numpy as np
import pytest
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
from gpu_harness import DEV

pytestmark = pytest.mark.gpu

O_TOL = 2e-5
LSE_TOL = 2e-5


def _parts(n_parts, n_states, dim, seed, empty_frac=0.15):
    g = np.random.default_rng(seed)
    o = (g.standard_normal((n_parts, n_states, dim)) * np.exp(g.uniform(-3, 3, (n_parts, n_states, 1)))).astype(np.float32)
    lse = g.uniform(-80.0, 80.0, (n_parts, n_states)).astype(np.float32)
    lse[g.random((n_parts, n_states)) < empty_frac] = -np.inf
    lse[:, :3] = -np.inf                                     # states whose parts are all empty
    if n_parts > 1:
        lse[0, 3:6] = 80.0                                   # one part dominating by a wide margin
        lse[1:, 3:6] = -80.0
    return o, lse


def _compare(out, lse, o_ref, lse_ref):
    o = out.cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert (np.isneginf(l) == empty).all()
    assert (o[empty] == 0).all()
    norm = np.abs(o_ref).max(axis=-1)
    err = np.abs(o - o_ref).max(axis=-1)
    rel = np.where(empty, 0.0, err / np.maximum(norm, 1e-300))
    assert rel.max() <= O_TOL, "o rel err %.3g" % rel.max()
    safe = np.where(empty, 0.0, lse_ref)
    lerr = np.where(empty, 0.0, np.abs(l - safe) - 2.0 ** -20 * np.abs(safe))
    assert lerr.max() <= LSE_TOL, "lse err %.3g" % lerr.max()
    return float(rel.max())


@pytest.mark.parametrize("n_parts", [1, 2, 8, 9, 16, 17, 33, 64])
@pytest.mark.parametrize("dim", [4, 64, 260, 512, 576, 4096])
def test_merge_matches_oracle(n_parts, dim):
    n_states = 37 if dim >= 4096 else 301
    o, lse = _parts(n_parts, n_states, dim, seed=7000 + 131 * n_parts + dim)
    o_ref, lse_ref = oracle.merge_states(o.astype(np.float64), lse.astype(np.float64))
    out, l = kv4.merge_states(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV))
    torch.cuda.synchronize()
    _compare(out, l, o_ref, lse_ref)
    # fp16 parts: the same merge of the parts rounded to fp16, widened exactly
    o16 = o.astype(np.float16)
    o_ref16, lse_ref16 = oracle.merge_states(o16.astype(np.float64), lse.astype(np.float64))
    out16, l16 = kv4.merge_states(torch.from_numpy(o16).to(DEV), torch.from_numpy(lse).to(DEV))
    torch.cuda.synchronize()
    _compare(out16, l16, o_ref16, lse_ref16)


@pytest.mark.parametrize("n_parts", [1, 4, 5, 8])
@pytest.mark.parametrize("n_states,dim", [(2100, 264), (2048, 512), (900, 1032), (1100, 1028)])
def test_merge_many_states_two_pieces_per_lane(n_parts, n_states, dim):
    """At least 4096 tasks of 256 dims and at most 8 parts: each lane merges
    two 4-dim pieces (512 dims per wavefront) when dim is a multiple of 8,
    including segments that end inside a wavefront; dim 1028 keeps one piece
    per lane."""
    o, lse = _parts(n_parts, n_states, dim, seed=7300 + 17 * n_parts + dim)
    o_ref, lse_ref = oracle.merge_states(o.astype(np.float64), lse.astype(np.float64))
    out, l = kv4.merge_states(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV))
    torch.cuda.synchronize()
    _compare(out, l, o_ref, lse_ref)
    o16 = o.astype(np.float16)
    o_ref16, lse_ref16 = oracle.merge_states(o16.astype(np.float64), lse.astype(np.float64))
    out16, l16 = kv4.merge_states(torch.from_numpy(o16).to(DEV), torch.from_numpy(lse).to(DEV))
    torch.cuda.synchronize()
    _compare(out16, l16, o_ref16, lse_ref16)


def test_merge_into_strided_output_rows():
    """States written into rows of a wider output (out_state_stride > dim)."""
    n_parts, n_states, dim = 5, 64, 512
    o, lse = _parts(n_parts, n_states, dim, seed=7100)
    o_ref, lse_ref = oracle.merge_states(o.astype(np.float64), lse.astype(np.float64))
    wide = torch.full((n_states, dim + 64), 7.0, dtype=torch.float32, device=DEV)
    out = wide[:, :dim]
    l = torch.empty(n_states, dtype=torch.float32, device=DEV)
    kv4.merge_states(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV), out=out, lse=l)
    torch.cuda.synchronize()
    _compare(out, l, o_ref, lse_ref)
    assert (wide[:, dim:] == 7.0).all(), "the merge wrote outside its rows"


def test_merge_millions_of_states():
    """4.3M states of 4 dims: more wavefront tasks than one launch has
    wavefronts, so wavefronts take several states each."""
    n_parts, n_states, dim = 2, 4_300_000, 4
    o, lse = _parts(n_parts, n_states, dim, seed=7200)
    o_ref, lse_ref = oracle.merge_states(o.astype(np.float64), lse.astype(np.float64))
    out, l = kv4.merge_states(torch.from_numpy(o).to(DEV), torch.from_numpy(lse).to(DEV))
    torch.cuda.synchronize()
    _compare(out, l, o_ref, lse_ref)
