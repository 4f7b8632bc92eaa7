"""Seeded synthetic inputs for one paged grouped-query-attention decode step.

This module only *creates* inputs: context lengths, block tables, a paged K/V
pool and queries.  It holds none of the attention arithmetic, so both the fp64
oracle (``oracle/``) and the HIP path consume the very same bits without
sharing any of the method's code.

Workloads follow the problem statement of the PersistentKV summary
(aissential.tech, "PersistentKV: Page-Aware Decode Scheduling ...", Summary:
FP16, page size 16, Hq=32, Hkv=8, d=128, B1 / B8 bimodal, uniform and
Zipf-like workloads) plus two extra cases: a tiny hand-checkable case and a
batched prefix-sharing case (GrowPage abstract: paged KV that keeps prefix
caching).

Recipe (per workload, ``seed`` given):

* ``rng = numpy.random.default_rng(seed)``; draw order is context lengths,
  then the physical-page permutation, then q.
* K and V pools are filled in fixed chunks of ``_CHUNK`` elements, chunk ``i``
  of pool ``tag`` (0 = K, 1 = V) from ``default_rng([seed, tag, i])``, so the
  bits do not depend on how many threads generate them.
* Values are N(0, 1) drawn in float32 and rounded to the storage type
  (float16 by numpy's cast, bfloat16 by round-to-nearest-even on the bits).
* Sequence ``b`` owns ``ceil(ctx_b / P)`` logical pages; physical ids are
  taken from the permutation in (sequence, logical page) order.  Block-table
  slots past a sequence's last page hold an id that no sequence references.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

F16 = "f16"
BF16 = "bf16"
_CHUNK = 1 << 22

__all__ = [
    "F16", "BF16", "Workload", "make", "NAMES", "f32_to_bf16_bits",
    "poison_unused", "draw_queries", "kv_bytes", "custom", "k_tiles_from_rows",
    "k_rows_from_tiles",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return x32.astype(np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _nan_bits(dtype: str):
    return np.float16(np.nan) if dtype == F16 else np.uint16(0x7FC0)


@dataclasses.dataclass
class Workload:
    """One decode step's inputs.  Arrays are host numpy arrays.

    ``q``: [B, Hq, d]; ``k_pool``: [num_pages, Hkv, d/8, P, 8] (each tile's
    keys as 16-byte chunks, chunk c of every slot together); ``v_pool``:
    [num_pages, Hkv, P, d]; float16
    arrays for ``f16`` or uint16 bfloat16 bit patterns for ``bf16``.
    ``block_tables``: int32 [B, max_pages]; ``ctx_lens``: int32 [B].
    ``s_prev``: float32 [2, B, Hkv, d] query-summary state (fast, slow).
    """

    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    d: int
    page_size: int
    split_tokens: int
    dtype: str
    num_pages: int
    ctx_lens: np.ndarray
    block_tables: np.ndarray
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    s_prev: np.ndarray
    scale: float
    alpha_fast: float = 0.5
    alpha_slow: float = 0.05
    steps: int = 1
    shared_prefix_pages: int = 0
    rng: np.random.Generator | None = dataclasses.field(default=None, repr=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_pages(self) -> int:
        return int(self.block_tables.shape[1])

    def pages_of(self, b: int) -> int:
        return -(-int(self.ctx_lens[b]) // self.page_size)

    def referenced_pages(self) -> np.ndarray:
        ids = [self.block_tables[b, : self.pages_of(b)] for b in range(self.B)]
        return np.unique(np.concatenate(ids)) if ids else np.zeros(0, np.int32)

    def shares_pages(self) -> bool:
        """True if some physical page is in the used part of two sequences' tables."""
        n = sum(self.pages_of(b) for b in range(self.B))
        return len(self.referenced_pages()) < n


def shared_leading_pages(wl: Workload) -> np.ndarray:
    """Per sequence, the leading table pages that other sequences share."""
    pages = (wl.ctx_lens.astype(np.int64) + wl.page_size - 1) // wl.page_size
    return np.minimum(pages, wl.shared_prefix_pages).astype(np.int32)


def kv_bytes(wl: Workload, unique: bool = False) -> int:
    """Algorithmic K+V bytes one decode step must read.

    Logical: every (sequence, token, KV head) row of K and of V once.  With
    ``unique`` a physical page shared by several sequences counts once.
    """
    elem = 2
    if unique:
        return int(len(wl.referenced_pages())) * wl.Hkv * wl.page_size * wl.d * 2 * elem
    return int(np.sum(wl.ctx_lens, dtype=np.int64)) * wl.Hkv * wl.d * 2 * elem


def _fill_pool(seed: int, tag: int, shape, dtype: str, threads: int) -> np.ndarray:
    total = int(np.prod(shape))
    out_dtype = np.float16 if dtype == F16 else np.uint16
    flat = np.empty(total, dtype=out_dtype)
    nchunks = -(-total // _CHUNK)

    def work(i):
        lo = i * _CHUNK
        hi = min(total, lo + _CHUNK)
        g = np.random.default_rng([seed, tag, i])
        flat[lo:hi] = _store(g.standard_normal(hi - lo, dtype=np.float32), dtype)

    if nchunks <= 1 or threads <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(work, range(nchunks)))
    return flat.reshape(shape)


def _assemble(name, seed, rng, ctx, Hq, Hkv, d, P, S, dtype, num_pages,
              shared_prefix_pages=0, max_pages=None, steps=1, threads=None,
              fill_pools=True) -> Workload:
    ctx = np.asarray(ctx, dtype=np.int64)
    if np.any(ctx < 0):
        raise ValueError("negative context length")
    B = len(ctx)
    pages = [-(-int(c) // P) for c in ctx]
    need_max = max(pages) if pages else 0
    max_pages = need_max if max_pages is None else int(max_pages)
    if max_pages < need_max:
        raise ValueError("max_pages smaller than the longest sequence")
    own = [max(0, p - shared_prefix_pages) for p in pages]
    distinct = (shared_prefix_pages if shared_prefix_pages else 0) + sum(own)
    if num_pages is None:
        raise ValueError("num_pages required")
    if num_pages <= distinct:
        raise ValueError("pool must hold at least one unreferenced page")
    perm = rng.permutation(num_pages).astype(np.int32)
    spare = perm[-1]
    bt = np.full((B, max(1, max_pages)), spare, dtype=np.int32)
    shared = perm[:shared_prefix_pages]
    cur = shared_prefix_pages
    for b in range(B):
        ns = min(pages[b], shared_prefix_pages)
        bt[b, :ns] = shared[:ns]
        bt[b, ns:pages[b]] = perm[cur:cur + own[b]]
        cur += own[b]
    q32 = rng.standard_normal((B, Hq, d), dtype=np.float32)
    q = _store(q32, dtype)
    threads = threads or min(16, os.cpu_count() or 1)
    kshape, vshape = (num_pages, Hkv, d // 8, P, 8), (num_pages, Hkv, P, d)
    if fill_pools:
        k_pool = _fill_pool(seed, 0, kshape, dtype, threads)
        v_pool = _fill_pool(seed, 1, vshape, dtype, threads)
    else:  # lengths and tables only (queue-level checks): empty placeholder pools
        dt = np.float16 if dtype == F16 else np.uint16
        k_pool = np.zeros((0, Hkv, d // 8, P, 8), dtype=dt)
        v_pool = np.zeros((0, Hkv, P, d), dtype=dt)
    return Workload(
        name=name, seed=seed, B=B, Hq=Hq, Hkv=Hkv, d=d, page_size=P, split_tokens=S,
        dtype=dtype, num_pages=num_pages, ctx_lens=ctx.astype(np.int32), block_tables=bt,
        q=q, k_pool=k_pool, v_pool=v_pool,
        s_prev=np.zeros((2, B, Hkv, d), dtype=np.float32),
        scale=1.0 / math.sqrt(d), steps=steps, shared_prefix_pages=shared_prefix_pages,
        rng=rng)


def draw_queries(wl: Workload) -> np.ndarray:
    """Next step's q, drawn from the workload's own stream (after its pools)."""
    return _store(wl.rng.standard_normal((wl.B, wl.Hq, wl.d), dtype=np.float32), wl.dtype)


def _ctx_scale(ctx, divisor: int, P: int):
    """Shrink lengths for oracle-sized parity runs while keeping ragged tails."""
    if divisor == 1:
        return ctx
    return [max(1, int(c) // divisor) for c in ctx]


def make(name: str, seed: int | None = None, ctx_divisor: int = 1, threads=None,
         split_tokens: int = 256, fill_pools: bool = True) -> Workload:
    """Build a named workload.

    ``ctx_divisor`` > 1 divides every context length (oracle-sized variants
    with the same head shape, dtype, page structure and length mix).
    """
    base = {"tiny": 1000, "b1": 1001, "b8_bimodal": 1002, "b8_uniform": 1102,
            "b8_zipf": 1003, "b64_prefix": 1004, "b4_bimodal": 1005}
    if name not in base:
        raise KeyError(name)
    seed = base[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    kw = dict(threads=threads, fill_pools=fill_pools)
    if name == "tiny":
        # B=2, contexts 37 and 100, P=16, Hq=4, Hkv=1, d=64, 32-page pool.
        ctx = [37, 100]
        return _assemble(name, seed, rng, ctx, 4, 1, 64, 16, split_tokens, F16, 32, **kw)
    if name == "b1":
        # B=1, context 32768, 2048 pages scattered over a 4096-page pool.
        ctx = _ctx_scale([32768], ctx_divisor, 16)
        return _assemble(name, seed, rng, ctx, 32, 8, 128, 16, split_tokens, F16,
                         max(4096 // ctx_divisor, -(-ctx[0] // 16) + 1), **kw)
    if name in ("b8_bimodal", "b8_uniform", "b4_bimodal"):
        if name == "b8_bimodal":
            ctx = np.concatenate([rng.integers(512, 2048 + 1, 4), rng.integers(24576, 65536 + 1, 4)])
        elif name == "b4_bimodal":
            # The B4 bimodal mix: 2 short and 2 long sequences.
            ctx = np.concatenate([rng.integers(512, 2048 + 1, 2), rng.integers(24576, 65536 + 1, 2)])
        else:
            ctx = rng.integers(512, 65536 + 1, 8)
        ctx = _ctx_scale(ctx, ctx_divisor, 16)
        distinct = sum(-(-int(c) // 16) for c in ctx)
        return _assemble(name, seed, rng, ctx, 32, 8, 128, 16, split_tokens, F16,
                         math.ceil(1.25 * distinct) + (1 if ctx_divisor > 1 else 0), **kw)
    if name == "b8_zipf":
        z = rng.zipf(1.1, 8)
        ctx = [min(131072, max(256, 256 * int(min(v, 1 << 20)))) for v in z]
        ctx = _ctx_scale(ctx, ctx_divisor, 16)
        distinct = sum(-(-int(c) // 16) for c in ctx)
        return _assemble(name, seed, rng, ctx, 32, 8, 128, 16, split_tokens, F16,
                         math.ceil(1.25 * distinct) + (1 if ctx_divisor > 1 else 0), steps=16, **kw)
    # b64_prefix: B=64, U[4096,16384], Hq=64, Hkv=8, bf16, first 128 pages shared.
    ctx = rng.integers(4096, 16384 + 1, 64)
    shared = 128
    if ctx_divisor > 1:
        ctx = _ctx_scale(ctx, ctx_divisor, 16)
        shared = max(1, shared // ctx_divisor)
        ctx = [max(c, shared * 16 + 1) for c in ctx]
    pages = [-(-int(c) // 16) for c in ctx]
    distinct = shared + sum(p - shared for p in pages)
    return _assemble(name, seed, rng, ctx, 64, 8, 128, 16, split_tokens, BF16,
                     math.ceil(1.1 * distinct) + (1 if ctx_divisor > 1 else 0),
                     shared_prefix_pages=shared, **kw)


NAMES = ("tiny", "b1", "b8_bimodal", "b8_uniform", "b8_zipf", "b64_prefix", "b4_bimodal")


def custom(ctx, Hq, Hkv, d, page_size=16, split_tokens=256, dtype=F16, seed=7,
           pool_factor=1.5, max_pages=None, shared_prefix_pages=0,
           fill_pools=True) -> Workload:
    """Free-form workload for edge cases (empty, one-token, ragged contexts)."""
    rng = np.random.default_rng(seed)
    pages = [-(-int(c) // page_size) for c in ctx]
    distinct = shared_prefix_pages + sum(max(0, p - shared_prefix_pages) for p in pages)
    num_pages = max(distinct + 1, math.ceil(pool_factor * max(1, distinct)))
    return _assemble(f"custom{list(ctx)[:4]}", seed, rng, ctx, Hq, Hkv, d, page_size,
                     split_tokens, dtype, num_pages, shared_prefix_pages=shared_prefix_pages,
                     max_pages=max_pages, fill_pools=fill_pools)


def k_tiles_from_rows(rows: np.ndarray) -> np.ndarray:
    """K pool tiles from key rows: [..., P, d] -> [..., d/8, P, 8]."""
    r = np.asarray(rows)
    *lead, P, d = r.shape
    return np.ascontiguousarray(np.swapaxes(r.reshape(*lead, P, d // 8, 8), -3, -2))


def k_rows_from_tiles(tiles: np.ndarray) -> np.ndarray:
    """Key rows from K pool tiles: [..., d/8, P, 8] -> [..., P, d]."""
    t = np.asarray(tiles)
    *lead, nch, P, _ = t.shape
    return np.ascontiguousarray(np.swapaxes(t, -3, -2).reshape(*lead, P, nch * 8))


def poison_unused(wl: Workload) -> Workload:
    """Copy of ``wl`` whose unreferenced pages and slots past each context are NaN."""
    k = wl.k_pool.copy()
    v = wl.v_pool.copy()
    nan = _nan_bits(wl.dtype)
    used = np.zeros(wl.num_pages, dtype=bool)
    used[wl.referenced_pages()] = True
    k[~used] = nan
    v[~used] = nan
    P = wl.page_size
    for b in range(wl.B):
        c = int(wl.ctx_lens[b])
        if c % P:
            last = wl.block_tables[b, c // P]
            # A shared page is never a partial last page in these workloads.
            k[last, :, :, c % P:, :] = nan
            v[last, :, c % P:, :] = nan
    return dataclasses.replace(wl, k_pool=k, v_pool=v)
