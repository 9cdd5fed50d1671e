"""Helpers for the GPU parity tests: build the same pool on both sides from the
same seeded fp32 rows (the oracle quantizes on the host, the library on the
device), and compare attention outputs at the stated tolerance.

Tolerance (attention): per (query row, head), max_d |o - o_ref| <= 2e-3 *
max_d |o_ref|; |lse - lse_ref| <= 1e-3 + 2^-20 |lse_ref| (an fp32 lse holds
about 2^-24 relative, so large scores need the relative term).  The kernel's
only roundings are the fp32 accumulation of exact fp16 products and P rounded
to fp16 (relative 2^-11) before the P.V product; both are far inside that
bound.
"""
from __future__ import annotations

import numpy as np
import torch

import bit_kv_cache_kv4_amd as kv4
import oracle
import workloads as W

O_TOL = 2e-3
LSE_TOL = 1e-3
LSE_REL = 2.0 ** -20
DEV = "cuda:0"


def host_kv(spec, n_slots=None):
    """fp32 pre-quantization rows of every slot (host-generated pools)."""
    n = spec.n_slots if n_slots is None else n_slots
    return W.kv_rows_host(spec, 0, n)


def build_pools(spec, kv=None):
    """(device pool written by kv4_quant_write, host pool written by the oracle)."""
    kv = host_kv(spec) if kv is None else kv
    slots = np.arange(kv.shape[0], dtype=np.int32)
    pool_h = np.zeros((kv.shape[0], oracle.row_bytes()), dtype=np.uint8)
    oracle.quant_write(kv, slots, pool_h)
    pool_d = torch.zeros((kv.shape[0], 352), dtype=torch.uint8, device=DEV)
    kv4.quant_write(torch.from_numpy(kv).to(DEV), torch.from_numpy(slots).to(DEV), pool_d)
    return pool_d, pool_h


def q_for_oracle(q):
    """The query exactly as the kernel sees it, widened to fp32."""
    return q.float().cpu().numpy()


def compare_attention(out, lse, o_ref, lse_ref, o_tol=O_TOL, lse_tol=LSE_TOL):
    """Returns (worst relative error, worst lse error); asserts the bound."""
    o = out.detach().float().cpu().numpy().astype(np.float64)
    l = lse.detach().float().cpu().numpy().astype(np.float64)
    assert o.shape == o_ref.shape and l.shape == lse_ref.shape
    empty = np.isneginf(lse_ref)
    assert (np.isneginf(l) == empty).all(), "empty-list rows disagree"
    assert (o[empty] == 0).all()
    ref_norm = np.abs(o_ref).max(axis=-1)
    err = np.abs(o - o_ref).max(axis=-1)
    rel = np.where(ref_norm > 0, err / np.maximum(ref_norm, 1e-300), err)
    rel = np.where(empty, 0.0, rel)
    worst = float(rel.max()) if rel.size else 0.0
    safe_ref = np.where(empty, 0.0, lse_ref)
    lerr = np.where(empty, 0.0, np.abs(l - safe_ref) / (1.0 + LSE_REL / lse_tol * np.abs(safe_ref)))
    lworst = float(lerr.max()) if lerr.size else 0.0
    assert worst <= o_tol, "max rel error %.3g > %.3g at %s" % (worst, o_tol, np.unravel_index(rel.argmax(), rel.shape))
    assert lworst <= lse_tol, "max lse error %.3g > %.3g (scaled by 1 + 2^-20 |lse| / tol)" % (lworst, lse_tol)
    return worst, lworst


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    return t.to(DEV) if dtype is None else t.to(DEV, dtype)
