"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and lays them out: page tables, top-k
index lists, queries and pre-quantization KV rows.  It holds none of the
method's arithmetic (no quantization, translation or attention) and is shared
by the tests, the benchmark and the smoke check.

Shapes follow the pages: 352-byte rows of 512 latent + 64 rope dims, a 64-token
page table, exact top-2048 lists, 64 sessions at 204,800 tokens of context
("60+ inference optimizations & kernels", section "Headline results" and
"4-bit KV cache"; sgl-amd-mono GLM-5.3 monokernel PR, "Modifications").

Seeds: 1000 * config number + stream id.
"""
from __future__ import annotations

import dataclasses
from typing import Optional
import math

import numpy as np

N_LATENT = 512
N_ROPE = 64
DIM = N_LATENT + N_ROPE
PAGE = 64


@dataclasses.dataclass
class DecodeSpec:
    """A paged-pool attention workload (decode or prefill)."""
    name: str
    n_req: int            # requests (page-table rows)
    ctx: int              # tokens of context per request
    n_heads: int
    k: int                # top-k entries per query row
    q_dtype: str          # "f32" or "bf16"
    n_pool_pages: int     # physical pages in the pool
    outlier_p: float = 0.0
    outlier_mul: float = 1.0
    n_query_rows: int = 0  # prefill: query rows (all in request 0); 0 = one row per request
    first_query_pos: int = 0
    seed: int = 0
    softmax_scale: Optional[float] = None   # None: 1/sqrt(576)

    @property
    def n_slots(self) -> int:
        return self.n_pool_pages * PAGE

    @property
    def pages_per_req(self) -> int:
        return self.ctx // PAGE

    @property
    def rows(self) -> int:
        return self.n_query_rows if self.n_query_rows else self.n_req

    @property
    def sm_scale(self) -> float:
        if self.softmax_scale is not None:
            return float(np.float32(self.softmax_scale))
        return float(np.float32(1.0 / math.sqrt(DIM)))


# The five workloads.  C1..C3 decode, C5 prefill; C4 (write + compaction) has
# its own generator below.
C1 = DecodeSpec("c1_tiny_decode", n_req=1, ctx=4096, n_heads=16, k=256, q_dtype="f32",
                n_pool_pages=64, seed=1000)
C2 = DecodeSpec("c2_decode_head_share", n_req=8, ctx=32768, n_heads=64, k=2048, q_dtype="bf16",
                n_pool_pages=4096, outlier_p=0.01, outlier_mul=20.0, seed=2000)
C3 = DecodeSpec("c3_long_context_decode", n_req=64, ctx=204800, n_heads=64, k=2048, q_dtype="bf16",
                n_pool_pages=204800, seed=3000)
C5 = DecodeSpec("c5_sparse_prefill", n_req=1, ctx=65536, n_heads=64, k=2048, q_dtype="bf16",
                n_pool_pages=1024, n_query_rows=4096, first_query_pos=61440, seed=5000)

SPECS = {s.name: s for s in (C1, C2, C3, C5)}


def scaled(spec: DecodeSpec, **kw) -> DecodeSpec:
    """A copy of spec with some fields replaced (smaller parity cases)."""
    return dataclasses.replace(spec, **kw)


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def page_table(spec: DecodeSpec) -> np.ndarray:
    """[n_req, pages_per_req] int32: a random permutation of physical pages."""
    need = spec.n_req * spec.pages_per_req
    assert need <= spec.n_pool_pages
    perm = rng(spec.seed, 1).permutation(spec.n_pool_pages)[:need].astype(np.int32)
    return perm.reshape(spec.n_req, spec.pages_per_req)


def query_positions(spec: DecodeSpec) -> np.ndarray:
    """Position of each query row (decode: the last token; prefill: a run)."""
    if spec.n_query_rows:
        return np.arange(spec.first_query_pos, spec.first_query_pos + spec.n_query_rows,
                         dtype=np.int64)
    return np.full(spec.n_req, spec.ctx, dtype=np.int64)


def topk_lists(spec: DecodeSpec, stream: int = 2) -> np.ndarray:
    """[rows, k] int32 request-local positions, distinct within a row, drawn
    uniformly without replacement from [0, position) (prefill) or [0, ctx)."""
    g = rng(spec.seed, stream)
    pos = query_positions(spec)
    out = np.empty((spec.rows, spec.k), dtype=np.int32)
    for r in range(spec.rows):
        hi = int(min(pos[r], spec.ctx))
        out[r] = g.choice(hi, size=spec.k, replace=False).astype(np.int32)
    return out


def row_req(spec: DecodeSpec) -> np.ndarray | None:
    if spec.n_query_rows:
        return np.zeros(spec.n_query_rows, dtype=np.int32)
    return None


def queries(spec: DecodeSpec, stream: int = 3):
    """[rows, n_heads, 576] torch tensor on the CPU: float32 N(0, 1), or its
    bfloat16 rounding for bf16 workloads."""
    import torch
    g = torch.Generator().manual_seed(spec.seed * 16 + stream)
    q = torch.randn(spec.rows, spec.n_heads, DIM, generator=g, dtype=torch.float32)
    return q.to(torch.bfloat16) if spec.q_dtype == "bf16" else q


def kv_rows_host(spec: DecodeSpec, slot_lo: int, n: int, stream: int = 4) -> np.ndarray:
    """Pre-quantization fp32 KV rows for slots [slot_lo, slot_lo + n) drawn on
    the host (small pools): N(0, 1), with outlier entries multiplied."""
    g = rng(spec.seed, stream * 1_000_003 + slot_lo)
    x = g.standard_normal((n, DIM), dtype=np.float32)
    if spec.outlier_p > 0:
        m = g.random((n, DIM)) < spec.outlier_p
        x[m] *= np.float32(spec.outlier_mul)
    return x


KV_CHUNK = 1 << 20  # rows per device-generated chunk


def kv_chunk_device(spec: DecodeSpec, chunk: int, device, stream: int = 4):
    """Pre-quantization fp32 KV rows of slots [chunk * KV_CHUNK, ...) drawn on
    the device with torch's generator (large pools).  Same chunk, same rows."""
    import torch
    lo = chunk * KV_CHUNK
    n = min(KV_CHUNK, spec.n_slots - lo)
    g = torch.Generator(device=device).manual_seed(spec.seed * 1_000_003 + stream * 4096 + chunk)
    x = torch.randn(n, DIM, generator=g, device=device, dtype=torch.float32)
    if spec.outlier_p > 0:
        m = torch.rand(n, DIM, generator=g, device=device) < spec.outlier_p
        x = torch.where(m, x * spec.outlier_mul, x)
    return x


# ----------------------------------------------------- write + compaction
@dataclasses.dataclass
class WriteSpec:
    name: str = "c4_write_compaction"
    n_tokens: int = 16384
    n_pool_pages: int = 1024
    n_lists: int = 4096
    list_len: int = 2048
    n_distinct: int = 1536
    value_range: int = 65536
    seed: int = 4000

    @property
    def n_slots(self) -> int:
        return self.n_pool_pages * PAGE


C4 = WriteSpec()


def write_tokens(spec: WriteSpec, stream: int = 1) -> np.ndarray:
    """[n_tokens, 576] fp32: N(0, 1) times a per-row scale log-uniform in
    [1e-2, 1e2]."""
    g = rng(spec.seed, stream)
    z = g.standard_normal((spec.n_tokens, DIM), dtype=np.float32)
    u = g.uniform(-2.0, 2.0, size=(spec.n_tokens, 1))
    return (z * np.power(10.0, u)).astype(np.float32)


def write_slots(spec: WriteSpec, stream: int = 2) -> np.ndarray:
    """[n_tokens] int32: free slots = whole pages drawn without replacement
    from the pool, filled in order."""
    g = rng(spec.seed, stream)
    n_pages = -(-spec.n_tokens // PAGE)
    pages = g.choice(spec.n_pool_pages, size=n_pages, replace=False)
    slots = (pages[:, None] * PAGE + np.arange(PAGE)[None, :]).reshape(-1)[: spec.n_tokens]
    return slots.astype(np.int32)


def dup_lists(spec: WriteSpec, stream: int = 3, n_lists: int | None = None) -> np.ndarray:
    """[n_lists, list_len] int32: each list holds n_distinct distinct values
    from [0, value_range) plus repeats of them, shuffled (~25% duplicates)."""
    g = rng(spec.seed, stream)
    n_lists = spec.n_lists if n_lists is None else n_lists
    out = np.empty((n_lists, spec.list_len), dtype=np.int32)
    for i in range(n_lists):
        base = g.choice(spec.value_range, size=spec.n_distinct, replace=False)
        rep = g.choice(base, size=spec.list_len - spec.n_distinct, replace=True)
        row = np.concatenate([base, rep])
        g.shuffle(row)
        out[i] = row
    return out
