"""fp64 CPU oracle for one paged GQA decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it and it
never calls the HIP library: the two share no code.

What is computed, and where it comes from:

* Work queue -- the PersistentKV summary (aissential.tech, "PersistentKV:
  Page-Aware Decode Scheduling ...", Summary and Method) says the engine runs
  a compact workqueue holding only non-empty (sequence, KV head, sequence
  split) tasks.  ``build_queue`` enumerates them in (sequence, KV head, split)
  order with fixed ``split_tokens``-token splits.
* Page-table gather -- same page (Summary: native page tables; Method: work
  mapped by KV-head group).  Logical token ``t`` of sequence ``b`` lives in
  physical page ``block_tables[b, t // P]`` at slot ``t % P``.  The V pool is
  ``[num_pages, Hkv, P, d]`` (row-major tiles); the K pool is
  ``[num_pages, Hkv, d/8, P, 8]``: each (page, KV head) tile keeps its keys as
  16-byte chunks, chunk ``c`` of every slot together, so key element ``i``
  of slot ``s`` is ``k_pool[page, g, i // 8, s, i % 8]``.
* Attention -- grouped-query attention: query head ``h`` reads KV head
  ``h // (Hq // Hkv)``.  The oracle evaluates the plain softmax definition
  over the whole context (no splitting, no online softmax): split-KV with a
  log-sum-exp merge reaches the same value up to rounding.
* Page mass -- the per-page sum of the softmax weights of the step, the
  page-level attention signal that GrowPage's page budgeting consumes
  (mlsanity.com GrowPage entry, Abstract: page-level KV abstraction).
* KV append -- the step before attention: each sequence's new token goes to
  slot ``ctx % P`` of its last page; a sequence at a page boundary first takes
  a physical page from the pool's integer free list (GrowPage, aitrending.vip
  article, Technical Details: a page is acquired at a capacity boundary;
  "Elastic KV Cache for LLM Serving", 2 Background and Motivation: the paged
  pool is fixed-size blocks handed out from an integer free list).
* Input checks -- what the decode step assumes of its integer inputs, as
  plain definitions: lengths within the table row, the table entries a
  sequence uses inside the pool, and a queue equal to ``build_queue`` of the
  lengths (each clamped into the row first).
* Query summaries -- GrowPage (Abstract; aitrending.vip article, Technical
  Details) keeps dual-timescale query summaries.  Here: per (sequence, KV
  group) a fast and a slow exponential moving average of the group-mean query,
  ``s <- (1 - a) * s + a * qbar``, and per page the largest scaled dot product
  of each updated summary with the page's keys.
* Budgeting decision -- GrowPage (mlsanity.com entry, Abstract; aitrending.vip
  article, Technical Details: on-demand page allocation) compares the two
  summaries' attention working sets and, at each capacity boundary, either
  compresses within the allocation or acquires a page.  The pages give no
  formula; the reading implemented: a working set is the smallest top set of
  pages (by summary page score, equal scores entering together) holding at
  least ``tau`` of the scores' softmax weight; F and S are the unions over KV
  heads of the fast and slow sets; a sequence whose last page is full
  acquires when ``|F| > |S|`` or no page lies outside both, else compresses
  the page outside both with the lowest slow score (largest slow page max
  over the KV heads; ties to the lowest page).

Everything is float64.  Inputs keep the exact stored bits: float16 arrays, or
uint16 arrays holding bfloat16 bit patterns, are widened exactly.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "widen", "build_queue", "gather_offsets", "logical_rows", "logical_key_rows", "attention",
    "update_summaries", "summary_page_max", "decode_step", "append_kv",
    "APPEND_FULL", "APPEND_NO_PAGE", "APPEND_BAD_PAGE",
    "check_inputs", "CHECK_LENGTH", "CHECK_PAGE", "CHECK_QUEUE",
    "working_set", "budget_decision", "DECIDE_NONE", "DECIDE_ACQUIRE", "DECIDE_COMPRESS",
]

APPEND_FULL = 1      # status bit: a sequence had no room left in its block-table row
APPEND_NO_PAGE = 2   # status bit: the free list ran out
APPEND_BAD_PAGE = 4  # status bit: a page id outside the pool (free list or table)

DECIDE_NONE = 0      # decision: the sequence is not at a capacity boundary
DECIDE_ACQUIRE = 1   # decision: take one more physical page
DECIDE_COMPRESS = 2  # decision: stay within the allocation, compress the victim page

CHECK_LENGTH = 1     # status bit: a length outside [0, max_pages * P]
CHECK_PAGE = 2       # status bit: a table entry a sequence uses outside the pool
CHECK_QUEUE = 4      # status bit: the queue is not build_queue of the (clamped) lengths


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored float16 / bfloat16 (uint16 bits) data."""
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def build_queue(ctx_lens, Hkv: int, split_tokens: int):
    """Compact task queue (PersistentKV summary, Summary and Method).

    Returns ``tasks`` int32 [n, 4] with rows (seq, kv_head, tok_begin,
    tok_end), ``group_offsets`` int32 [B*Hkv + 1] (first task of each
    (seq, kv_head) pair; the last entry is n) and ``n``.
    A sequence with no tokens contributes no task.
    """
    tasks = []
    offsets = []
    for b, ctx in enumerate(int(c) for c in ctx_lens):
        for g in range(Hkv):
            offsets.append(len(tasks))
            begin = 0
            while begin < ctx:
                end = min(ctx, begin + split_tokens)
                tasks.append((b, g, begin, end))
                begin = end
    offsets.append(len(tasks))
    arr = np.array(tasks, dtype=np.int32).reshape(-1, 4)
    return arr, np.array(offsets, dtype=np.int32), len(tasks)


def gather_offsets(block_tables, tasks, Hkv: int, page_size: int, d: int, split_tokens: int):
    """Element offsets into the K and V pools of every token a task reads.

    Entry ``[i, j]`` is, for token ``tok_begin + j`` of task ``i``, the
    offset of its first key element in the K pool ``[num_pages, Hkv, d/8, P,
    8]`` (``[..., 0]``) and of its value row in the V pool ``[num_pages, Hkv,
    P, d]`` (``[..., 1]``); -1 when the token is past ``tok_end``.
    """
    n = len(tasks)
    out = np.full((n, split_tokens, 2), -1, dtype=np.int64)
    for i in range(n):
        b, g, t0, t1 = (int(v) for v in tasks[i])
        for j in range(t1 - t0):
            t = t0 + j
            page = int(block_tables[b, t // page_size])
            tile = (page * Hkv + g) * page_size * d
            out[i, j, 0] = tile + (t % page_size) * 8
            out[i, j, 1] = tile + (t % page_size) * d
    return out


def logical_rows(pool, block_tables, b: int, g: int, ctx: int, page_size: int, dtype: str):
    """The ``ctx`` V rows of (sequence b, KV head g) in logical order, fp64."""
    npages = -(-ctx // page_size)
    pages = np.asarray(block_tables[b, :npages], dtype=np.int64)
    tiles = pool[pages, g]                      # [npages, P, d], stored type
    d = tiles.shape[-1]
    return widen(tiles.reshape(npages * page_size, d)[:ctx], dtype)


def logical_key_rows(k_pool, block_tables, b: int, g: int, ctx: int, page_size: int, dtype: str):
    """The ``ctx`` K rows of (sequence b, KV head g) in logical order, fp64.

    A K tile ``[d/8, P, 8]`` holds slot ``s``'s key as chunks ``[:, s, :]``.
    """
    npages = -(-ctx // page_size)
    pages = np.asarray(block_tables[b, :npages], dtype=np.int64)
    tiles = k_pool[pages, g]                    # [npages, d/8, P, 8], stored type
    nch = tiles.shape[1]
    rows = tiles.transpose(0, 2, 1, 3).reshape(npages * page_size, nch * 8)
    return widen(rows[:ctx], dtype)


def attention(q, k_pool, v_pool, block_tables, ctx_lens, page_size: int, scale: float,
              dtype: str, rows=None):
    """Softmax attention of each query head over its sequence's cached tokens.

    Returns ``out`` [B, Hq, d], ``lse`` [B, Hq] (natural log of the sum of
    exp(scaled score)), ``mass`` [B, Hq, max_pages] (softmax weight summed
    over each logical page; 0 past the last page).  ``rows``: optional
    iterable of (b, h) to compute; other entries stay NaN.
    A sequence with no tokens gets out = 0, lse = -inf, mass = 0.
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    max_pages = block_tables.shape[1]
    out = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    mass = np.full((B, Hq, max_pages), np.nan)
    want = {}
    for b, h in (rows if rows is not None else ((b, h) for b in range(B) for h in range(Hq))):
        want.setdefault((int(b), int(h) // G), []).append(int(h))
    for (b, g), heads in sorted(want.items()):
        ctx = int(ctx_lens[b])
        npages = -(-ctx // page_size)
        if ctx == 0:
            for h in heads:
                out[b, h] = 0.0
                lse[b, h] = -np.inf
                mass[b, h] = 0.0
            continue
        K = logical_key_rows(k_pool, block_tables, b, g, ctx, page_size, dtype)
        V = logical_rows(v_pool, block_tables, b, g, ctx, page_size, dtype)
        for h in heads:
            qh = widen(q[b, h], dtype)
            x = scale * (K @ qh)                 # scaled scores, [ctx]
            M = np.max(x)
            w = np.exp(x - M)
            L = np.sum(w)
            out[b, h] = (w @ V) / L
            lse[b, h] = M + math.log(L)
            p = np.zeros(npages * page_size)
            p[:ctx] = w / L
            mass[b, h] = 0.0
            mass[b, h, :npages] = p.reshape(npages, page_size).sum(axis=1)
    return out, lse, mass


def update_summaries(q, s_prev, Hkv: int, alpha_fast: float, alpha_slow: float, dtype: str):
    """One EMA step of the fast and slow query summaries (GrowPage, Abstract).

    ``qbar`` is the mean of the raw query vectors of the G heads sharing a KV
    head; each summary moves ``s <- (1 - a) * s + a * qbar``.  ``s_prev`` is
    [2, B, Hkv, d] (0 = fast, 1 = slow); returns float64 of the same shape.
    """
    B, Hq, d = q.shape
    G = Hq // Hkv
    qbar = widen(q, dtype).reshape(B, Hkv, G, d).mean(axis=2)
    s = np.asarray(s_prev, dtype=np.float64)
    a = np.array([float(np.float32(alpha_fast)), float(np.float32(alpha_slow))], dtype=np.float64)
    return (1.0 - a)[:, None, None, None] * s + a[:, None, None, None] * qbar[None]


def summary_page_max(s_next, k_pool, block_tables, ctx_lens, page_size: int, scale: float,
                     dtype: str, groups=None):
    """Per logical page, max over its valid keys of ``scale * (s . k)``.

    For both summaries (fast, slow).  Returns [2, B, Hkv, max_pages]; pages
    past the sequence's last page hold -inf.  ``groups``: optional iterable
    of (b, g) to compute; others stay NaN.
    """
    _, B, Hkv, d = s_next.shape
    max_pages = block_tables.shape[1]
    pm = np.full((2, B, Hkv, max_pages), np.nan)
    sel = groups if groups is not None else ((b, g) for b in range(B) for g in range(Hkv))
    for b, g in sel:
        ctx = int(ctx_lens[b])
        npages = -(-ctx // page_size)
        pm[:, b, g] = -np.inf
        if ctx == 0:
            continue
        K = logical_key_rows(k_pool, block_tables, b, g, ctx, page_size, dtype)
        for k in range(2):
            x = np.full(npages * page_size, -np.inf)
            x[:ctx] = scale * (K @ s_next[k, b, g])
            pm[k, b, g, :npages] = x.reshape(npages, page_size).max(axis=1)
    return pm


def decode_step(wl, rows=None, q=None, s_prev=None):
    """Every output of one decode step for a workload-like object.

    ``wl`` needs attributes q, k_pool, v_pool, block_tables, ctx_lens,
    page_size, scale, dtype, Hkv, split_tokens, d, alpha_fast, alpha_slow,
    s_prev.  ``rows`` restricts attention/mass to (b, h) pairs and the page
    max to their (b, g) groups.
    """
    q = wl.q if q is None else q
    s_prev = wl.s_prev if s_prev is None else s_prev
    tasks, offsets, n = build_queue(wl.ctx_lens, wl.Hkv, wl.split_tokens)
    out, lse, mass = attention(q, wl.k_pool, wl.v_pool, wl.block_tables, wl.ctx_lens,
                               wl.page_size, wl.scale, wl.dtype, rows=rows)
    s_next = update_summaries(q, s_prev, wl.Hkv, wl.alpha_fast, wl.alpha_slow, wl.dtype)
    G = q.shape[1] // wl.Hkv
    groups = None if rows is None else sorted({(int(b), int(h) // G) for b, h in rows})
    pm = summary_page_max(s_next, wl.k_pool, wl.block_tables, wl.ctx_lens, wl.page_size,
                          wl.scale, wl.dtype, groups=groups)
    return {"tasks": tasks, "group_offsets": offsets, "n_tasks": n, "out": out,
            "lse": lse, "mass": mass, "s_next": s_next, "page_max": pm}


def append_kv(k_pool, v_pool, block_tables, ctx_lens, k_new, v_new, free_pages, free_count,
              page_size: int):
    """Append one token per sequence to the paged cache (see the header).

    Sequences are taken in order.  Sequence ``b`` with ``t = ctx_lens[b]``:

    * ``t == max_pages * P``: its row is full; nothing changes for it and the
      status gets ``APPEND_FULL``.
    * ``t % P == 0``: it needs a new page.  The k-th sequence (in order)
      needing one takes ``free_pages[free_count - 1 - k]`` (the top of the
      stack) and records it at ``block_tables[b, t // P]``; if ``k >=
      free_count`` the list is exhausted: nothing changes for it and the
      status gets ``APPEND_NO_PAGE``.
    * Otherwise its page is ``block_tables[b, t // P]``.
    * A page id outside ``[0, num_pages)`` leaves the sequence unchanged (a
      free-list entry it came from is still used up) and sets
      ``APPEND_BAD_PAGE``.

    Then ``k_new[b, g]`` / ``v_new[b, g]`` are written to slot ``t % P`` of
    that page for every KV head ``g`` (the key as the slot's chunks of the K
    tile), and its length becomes ``t + 1``.

    Returns new copies ``(k_pool, v_pool, block_tables, ctx_lens, free_count,
    status)``; inputs are not modified.  Pure integer and copy work: the
    pools keep their dtype and bits.
    """
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    bt = np.array(block_tables, dtype=np.int32, copy=True)
    ctx = np.array(ctx_lens, dtype=np.int32, copy=True)
    max_pages = bt.shape[1]
    taken, status = 0, 0
    for b in range(len(ctx)):
        t = int(ctx[b])
        if t >= max_pages * page_size:
            status |= APPEND_FULL
            continue
        new_page = t % page_size == 0
        if new_page:
            if taken >= free_count:
                status |= APPEND_NO_PAGE
                continue
            page = int(free_pages[free_count - 1 - taken])
            taken += 1
        else:
            page = int(bt[b, t // page_size])
        if not 0 <= page < k_pool.shape[0]:
            status |= APPEND_BAD_PAGE
            continue
        if new_page:
            bt[b, t // page_size] = page
        Hkv, nch = k_pool.shape[1], k_pool.shape[2]
        k_pool[page, :, :, t % page_size, :] = np.asarray(k_new[b]).reshape(Hkv, nch, 8)
        v_pool[page, :, t % page_size, :] = v_new[b]
        ctx[b] = t + 1
    return k_pool, v_pool, bt, ctx, free_count - taken, status


def check_inputs(ctx_lens, block_tables, num_pages: int, page_size: int, Hkv: int,
                 split_tokens: int, capacity=None, tasks=None, group_offsets=None, n_tasks=None):
    """Status bits for the integer inputs of a decode step (see the header).

    * ``CHECK_LENGTH``: some length outside ``[0, max_pages * P]``.
    * ``CHECK_PAGE``: for some sequence ``b`` and page ``p`` with
      ``p * P < ctx_b`` (``ctx_b`` clamped into ``[0, max_pages * P]``), the
      table entry ``block_tables[b, p]`` is outside ``[0, num_pages)``.
    * ``CHECK_QUEUE`` (only when a queue is given): ``n_tasks`` is outside
      ``[0, capacity]``, or ``n_tasks``, ``group_offsets`` or the first
      ``n_tasks`` rows of ``tasks`` differ from ``build_queue`` of the
      clamped lengths.
    """
    bt = np.asarray(block_tables, dtype=np.int64)
    max_pages = bt.shape[1]
    status = 0
    ctx = [int(c) for c in ctx_lens]
    clamped = []
    for c in ctx:
        if c < 0 or c > max_pages * page_size:
            status |= CHECK_LENGTH
        clamped.append(min(max(c, 0), max_pages * page_size))
    for b, c in enumerate(clamped):
        for p in range(max_pages):
            if p * page_size < c and not 0 <= bt[b, p] < num_pages:
                status |= CHECK_PAGE
    if tasks is not None:
        want_tasks, want_offsets, want_n = build_queue(clamped, Hkv, split_tokens)
        n = int(np.asarray(n_tasks).reshape(-1)[0])
        given = np.asarray(tasks, dtype=np.int64).reshape(-1, 4)
        if (not 0 <= n <= capacity or n != want_n
                or not np.array_equal(np.asarray(group_offsets, dtype=np.int64), want_offsets)
                or not np.array_equal(given[:n], want_tasks)):
            status |= CHECK_QUEUE
    return status


def working_set(scores, tau: float):
    """Attention working set of one summary over one sequence's pages.

    ``scores``: the page scores (summary page maxima) of the sequence's
    pages.  Their softmax gives page weights; the working set is every page
    whose score is at or above the highest score level whose at-or-above
    pages hold at least ``tau`` of the weight, i.e. the smallest top set by
    score covering ``tau``, pages of equal score entering together.  Scores
    of -inf weigh 0 (all -inf: they all tie).  Returns ``(size, level)``;
    ``(0, inf)`` for no pages.
    """
    x = np.asarray(scores, dtype=np.float64)
    if x.size == 0:
        return 0, math.inf
    M = np.max(x)
    with np.errstate(invalid="ignore"):
        w = np.where(x == M, 1.0, np.exp(x - M))
    pi = w / np.sum(w)
    order = np.argsort(-x, kind="stable")          # pages by score, highest first
    xs = x[order]
    cum = np.cumsum(pi[order])
    ends = np.flatnonzero(np.r_[xs[1:] != xs[:-1], True])   # last page of each score level
    hit = np.flatnonzero(cum[ends] >= tau)
    j = ends[hit[0]] if hit.size else ends[-1]
    return int(j + 1), float(xs[j])


def budget_decision(page_max, ctx_lens, page_size: int, tau: float, ws_size=None):
    """Compress-or-acquire decision of every sequence (see the header).

    ``page_max``: [2, B, Hkv, max_pages] summary page maxima (0 fast, 1 slow)
    as the step writes them; only each sequence's first ``ceil(ctx/P)``
    pages are read.  ``ws_size`` (optional [2, B, Hkv]): take these working
    sets (the given number of top pages by score) instead of computing them,
    to decide from another implementation's sets.  Returns a dict with
    ``ws_size`` and ``ws_level`` [2, B, Hkv], ``ws_union`` [2, B] (sizes of
    F and S), ``decision`` [B] and ``victim`` [B] (-1 unless compressing).
    """
    pm = np.asarray(page_max, dtype=np.float64)
    _, B, Hkv, _ = pm.shape
    size = np.zeros((2, B, Hkv), dtype=np.int64)
    level = np.full((2, B, Hkv), np.inf)
    union = np.zeros((2, B), dtype=np.int64)
    decision = np.full(B, DECIDE_NONE, dtype=np.int64)
    victim = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        ctx = int(ctx_lens[b])
        npg = -(-ctx // page_size)
        member = np.zeros((2, npg), dtype=bool)
        for k in range(2):
            for g in range(Hkv):
                x = pm[k, b, g, :npg]
                if ws_size is None:
                    size[k, b, g], level[k, b, g] = working_set(x, tau)
                else:
                    n = int(ws_size[k, b, g])
                    size[k, b, g] = n
                    level[k, b, g] = np.sort(x)[::-1][n - 1] if n > 0 else np.inf
                member[k] |= x >= level[k, b, g]
        union[:, b] = member.sum(axis=1)
        if ctx == 0 or ctx % page_size != 0:
            continue
        outside = np.flatnonzero(~(member[0] | member[1]))
        if union[0, b] > union[1, b] or outside.size == 0:
            decision[b] = DECIDE_ACQUIRE
            continue
        decision[b] = DECIDE_COMPRESS
        slow = pm[1, b, :, :npg].max(axis=0)       # a page's best slow score over KV heads
        victim[b] = min(outside, key=lambda p: (slow[p], p))
    return {"ws_size": size, "ws_level": level, "ws_union": union,
            "decision": decision, "victim": victim}
