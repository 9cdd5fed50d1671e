"""Host checks of the arithmetic identities the MSE-scale write relies on
(CPU only, exact integer arithmetic)."""
import numpy as np
import pytest


def _rne_shift(n, k):
    """Round n / 2^k to the nearest integer, ties to even (n >= 0, int64)."""
    q = n >> k
    r = n - (q << k)
    half = np.int64(1) << np.int64(k - 1)
    up = (r > half) | ((r == half) & (q & 1 == 1))
    return q + up


@pytest.mark.parametrize("m", range(1, 8))
def test_reciprocal_quotient_is_correctly_rounded(m):
    """For mult = 1 + m/8 and r = the fp32 reciprocal of mult, q0 = RN(x r),
    res = x - q0 mult (exact) and RN(q0 + res r) equal the IEEE quotient
    RN(x / mult) for every float x in [1, 2); every step commutes with
    scaling by powers of two, so this covers every normal x."""
    M = 8 + m
    r = np.float32(1.0) / np.float32(M / 8)
    R = np.int64(round(float(r) * 2.0 ** 24))          # r = R 2^-24, r in (0.5, 1)
    assert float(R) * 2.0 ** -24 == float(r)
    X = np.arange(1 << 23, 1 << 24, dtype=np.int64)     # x = X 2^-23
    P = X * R                                            # x r = P 2^-47
    big = P >= (np.int64(1) << 47)
    # q0 = Q0 2^-s, s = 23 when x r >= 1 else 24
    Q0 = np.where(big, _rne_shift(P, 24), _rne_shift(P, 23))
    s = np.where(big, 23, 24)
    rem = np.where(big, X * 8, X * 16) - Q0 * M         # residual in units 2^-(s + 3)
    assert (np.abs(rem) < (1 << 24)).all()               # exact in fp32
    N = Q0 * (np.int64(1) << 27) + rem * R              # q0 + rem r = N 2^-(s + 27)
    assert (N > 0).all()
    # round N 2^-(s + 27) to fp32: unit 2^-23 at or above 1, else 2^-24
    one = np.where(big, np.int64(1) << 50, np.int64(1) << 51)
    hi = N >= one
    shift = np.where(hi, s + 4, s + 3)
    Q1 = np.empty_like(N)
    for sh in np.unique(shift):
        sel = shift == sh
        Q1[sel] = _rne_shift(N[sel], int(sh))
    q1 = (Q1.astype(np.float64) * np.where(hi, 2.0 ** -23, 2.0 ** -24)).astype(np.float32)
    x = (X.astype(np.float64) * 2.0 ** -23).astype(np.float32)
    ieee = x / np.float32(M / 8)
    bad = np.nonzero(q1.view(np.int32) != ieee.view(np.int32))[0]
    assert bad.size == 0, (m, x[bad[:5]], q1[bad[:5]], ieee[bad[:5]])
