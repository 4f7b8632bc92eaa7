"""Pins for the fp64 oracle: each check comes from outside the oracle itself.

Hand-worked fixtures (tests/golden), closed forms, a library routine
(torch's scaled_dot_product_attention in float64 on the CPU), invariants and
pure-Python brute force on tiny inputs.  CPU only.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import kvref
from paged_kv_cache_07_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_queue_golden():
    cases = {}
    cur = None
    with open(os.path.join(GOLDEN, "tiny_queue.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            if parts[0] == "split":
                cur = int(parts[1])
                cases[cur] = {"tasks": [], "offsets": None}
            elif parts[0] == "offsets":
                cases[cur]["offsets"] = [int(v) for v in parts[1:]]
            else:
                cases[cur]["tasks"].append(tuple(int(v) for v in parts))
    return cases


# ---------------------------------------------------------------- queue ---

def test_queue_matches_hand_worked_tiny_case():
    cases = _read_queue_golden()
    assert sorted(cases) == [16, 32, 256]
    for split, want in cases.items():
        tasks, offsets, n = kvref.build_queue([37, 100], 1, split)
        assert [tuple(r) for r in tasks.tolist()] == want["tasks"]
        assert offsets.tolist() == want["offsets"]
        assert n == len(want["tasks"])


@pytest.mark.parametrize("seed", range(5))
def test_queue_closed_form_and_tiling(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 9))
    Hkv = int(rng.integers(1, 5))
    split = int(rng.choice([16, 32, 48, 256]))
    ctx = rng.integers(0, 1200, B)
    ctx[rng.integers(0, B)] = 0
    tasks, offsets, n = kvref.build_queue(ctx, Hkv, split)
    assert n == Hkv * sum(-(-int(c) // split) for c in ctx)
    assert offsets[-1] == n and len(offsets) == B * Hkv + 1
    assert np.all(np.diff(offsets) >= 0)
    for b in range(B):
        for g in range(Hkv):
            rows = tasks[offsets[b * Hkv + g]: offsets[b * Hkv + g + 1]]
            assert np.all(rows[:, 0] == b) and np.all(rows[:, 1] == g)
            if ctx[b] == 0:
                assert len(rows) == 0
                continue
            assert rows[0, 2] == 0 and rows[-1, 3] == ctx[b]
            assert np.all(rows[1:, 2] == rows[:-1, 3])            # contiguous
            lens = rows[:, 3] - rows[:, 2]
            assert np.all(lens[:-1] == split) and 0 < lens[-1] <= split


# ------------------------------------------------------------- indexing ---

def test_gather_offsets_decode_to_layout_coordinates():
    wl = W.custom([37, 0, 100, 16, 1], Hq=6, Hkv=3, d=16, page_size=4, split_tokens=12, seed=3)
    tasks, _, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, wl.split_tokens)
    offs = kvref.gather_offsets(wl.block_tables, tasks, wl.Hkv, wl.page_size, wl.d, wl.split_tokens)
    for i in range(n):
        b, g, t0, t1 = tasks[i]
        for j in range(wl.split_tokens):
            t = t0 + j
            if t >= t1:
                assert np.all(offs[i, j] == -1)
                continue
            page, slot = int(wl.block_tables[b, t // wl.page_size]), int(t % wl.page_size)
            kc = np.unravel_index(offs[i, j, 0], wl.k_pool.shape)     # [pages, Hkv, d/8, P, 8]
            vc = np.unravel_index(offs[i, j, 1], wl.v_pool.shape)     # [pages, Hkv, P, d]
            assert tuple(int(c) for c in kc) == (page, int(g), 0, slot, 0)
            assert tuple(int(c) for c in vc) == (page, int(g), slot, 0)


def test_attention_reads_the_tables_physical_rows():
    """V rows carry their own (page, head, slot) address; a query that singles
    out one logical token must return that token's physical address."""
    wl = W.custom([37, 100], Hq=4, Hkv=2, d=8, page_size=16, seed=11)
    P = wl.page_size
    v = np.zeros(wl.v_pool.shape, dtype=np.float16)
    pg, hd, sl = np.meshgrid(np.arange(wl.num_pages), np.arange(wl.Hkv), np.arange(P), indexing="ij")
    v[..., 0], v[..., 1], v[..., 2] = pg, hd, sl
    rng = np.random.default_rng(0)
    for b, c in enumerate(wl.ctx_lens):
        for g in range(wl.Hkv):
            t = int(rng.integers(0, c))
            k = np.zeros(wl.k_pool.shape, dtype=np.float16)
            page = wl.block_tables[b, t // P]
            k[page, g, 0, t % P, 0] = 8.0                 # key element 0 of slot t % P
            q = np.zeros(wl.q.shape, dtype=np.float16)
            q[b, :, 0] = 8.0 * math.sqrt(wl.d)          # scaled score 64 vs 0
            out, _, _ = kvref.attention(q, k, v, wl.block_tables, wl.ctx_lens, P, wl.scale, "f16")
            for h in range(g * wl.G, (g + 1) * wl.G):
                np.testing.assert_allclose(out[b, h, :3], [page, g, t % P], rtol=0, atol=1e-12)


# ------------------------------------------------------------ attention ---

def _identity_table_workload(ctx, Hq, Hkv, d, P, seed):
    wl = W.custom(ctx, Hq=Hq, Hkv=Hkv, d=d, page_size=P, seed=seed)
    B, mp = wl.block_tables.shape
    num_pages = B * mp + 1
    rng = np.random.default_rng(seed + 1)
    k = W.k_tiles_from_rows(rng.standard_normal((num_pages, Hkv, P, d)).astype(np.float16))
    v = rng.standard_normal((num_pages, Hkv, P, d)).astype(np.float16)
    bt = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    wl.k_pool, wl.v_pool, wl.block_tables, wl.num_pages = k, v, bt, num_pages
    return wl


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 2), (6, 6)])
def test_attention_matches_torch_sdpa_on_contiguous_pages(Hq, Hkv):
    wl = _identity_table_workload([37, 100, 1, 64], Hq, Hkv, 16, 16, seed=Hq * 10 + Hkv)
    out, lse, mass = kvref.attention(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.ctx_lens,
                                     wl.page_size, wl.scale, "f16")
    B, mp = wl.block_tables.shape
    P, d = wl.page_size, wl.d
    dense = lambda pool: torch.from_numpy(
        pool[: B * mp].astype(np.float64).reshape(B, mp, Hkv, P, d).transpose(0, 2, 1, 3, 4)
        .reshape(B, Hkv, mp * P, d))
    mask = torch.zeros(B, 1, 1, mp * P, dtype=torch.bool)
    for b, c in enumerate(wl.ctx_lens):
        mask[b, 0, 0, :c] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(wl.q.astype(np.float64))[:, :, None, :], dense(W.k_rows_from_tiles(wl.k_pool)),
        dense(wl.v_pool), attn_mask=mask, scale=wl.scale, enable_gqa=True)[:, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(mass.sum(axis=2), 1.0, rtol=0, atol=1e-12)


def test_attention_invariant_to_physical_page_relabelling():
    wl = W.make("tiny")
    base = kvref.decode_step(wl)
    rng = np.random.default_rng(5)
    pi = rng.permutation(wl.num_pages)                 # new id of old page p is pi[p]
    k = np.empty_like(wl.k_pool)
    v = np.empty_like(wl.v_pool)
    k[pi] = wl.k_pool
    v[pi] = wl.v_pool
    wl2 = W.make("tiny")
    wl2.k_pool, wl2.v_pool, wl2.block_tables = k, v, pi[wl.block_tables].astype(np.int32)
    moved = kvref.decode_step(wl2)
    for key in ("out", "lse", "mass", "s_next", "page_max"):
        assert np.array_equal(base[key], moved[key]), key


def test_uniform_scores_closed_forms():
    """q = 0: every weight is 1/ctx, so out is the mean of the cached V rows,
    lse = ln(ctx), and page mass is (valid tokens on the page)/ctx."""
    wl = W.make("tiny")
    q = np.zeros_like(wl.q)
    out, lse, mass = kvref.attention(q, wl.k_pool, wl.v_pool, wl.block_tables, wl.ctx_lens,
                                     wl.page_size, wl.scale, "f16")
    golden = {}
    with open(os.path.join(GOLDEN, "tiny_uniform_mass.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                parts = line.split()
                golden[int(parts[0])] = [float(Fraction(p)) for p in parts[1:]]
    for b, c in enumerate(wl.ctx_lens):
        V = np.stack([wl.v_pool[wl.block_tables[b, t // 16], 0, t % 16] for t in range(c)])
        want = golden[int(c)]
        for h in range(wl.Hq):
            np.testing.assert_allclose(out[b, h], V.astype(np.float64).mean(axis=0), rtol=1e-12, atol=1e-14)
            assert abs(lse[b, h] - math.log(c)) < 1e-13
            np.testing.assert_allclose(mass[b, h, :len(want)], want, rtol=0, atol=1e-15)
            assert np.all(mass[b, h, len(want):] == 0)


def test_constant_values_and_single_token_closed_forms():
    wl = W.custom([1, 5, 33], Hq=4, Hkv=2, d=16, page_size=16, seed=2)
    v = np.full_like(wl.v_pool, np.float16(0.75))
    out, _, _ = kvref.attention(wl.q, wl.k_pool, v, wl.block_tables, wl.ctx_lens, 16, wl.scale, "f16")
    np.testing.assert_allclose(out, 0.75, rtol=1e-14)
    out, lse, mass = kvref.attention(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.ctx_lens,
                                     16, wl.scale, "f16")
    b = 0                                                # ctx = 1
    for h in range(wl.Hq):
        g = h // wl.G
        page = wl.block_tables[b, 0]
        assert np.array_equal(out[b, h], wl.v_pool[page, g, 0].astype(np.float64))
        krow = W.k_rows_from_tiles(wl.k_pool[page, g])[0]
        x0 = wl.scale * float(np.dot(wl.q[b, h].astype(np.float64), krow.astype(np.float64)))
        assert abs(lse[b, h] - x0) < 1e-13
        assert mass[b, h, 0] == 1.0


def test_lse_consistent_with_prefix_mass():
    """Softmax over a prefix and the whole context: the prefix's share of the
    total exp-mass is exp(lse_prefix - lse_total), which is also the sum of the
    page masses of the prefix pages."""
    wl = W.custom([160, 100], Hq=4, Hkv=1, d=32, page_size=16, seed=9)
    full = kvref.attention(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.ctx_lens, 16, wl.scale, "f16")
    pref_ctx = np.array([64, 48], dtype=np.int32)
    pre = kvref.attention(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, pref_ctx, 16, wl.scale, "f16")
    for b in range(2):
        npre = pref_ctx[b] // 16
        share = np.exp(pre[1][b] - full[1][b])
        np.testing.assert_allclose(full[2][b, :, :npre].sum(axis=1), share, rtol=1e-12)


def test_empty_sequence_outputs():
    wl = W.custom([0, 20], Hq=2, Hkv=1, d=8, page_size=16, seed=4)
    step = kvref.decode_step(wl)
    assert np.all(step["out"][0] == 0) and np.all(step["lse"][0] == -np.inf)
    assert np.all(step["mass"][0] == 0) and np.all(step["page_max"][:, 0] == -np.inf)
    assert np.all(np.isfinite(step["s_next"]))


def _brute(wl):
    """Pure-Python loops: one token at a time through the block table."""
    B, Hq, d = wl.q.shape
    G = Hq // wl.Hkv
    P = wl.page_size
    f = lambda x: float(x)
    res = {}
    for b in range(B):
        c = int(wl.ctx_lens[b])
        for h in range(Hq):
            g = h // G
            xs = []
            for t in range(c):
                krow = wl.k_pool[wl.block_tables[b, t // P], g, :, t % P, :].reshape(-1)
                xs.append(wl.scale * math.fsum(f(wl.q[b, h, i]) * f(krow[i]) for i in range(d)))
            M = max(xs)
            ws = [math.exp(x - M) for x in xs]
            L = math.fsum(ws)
            o = []
            for i in range(d):
                o.append(math.fsum(ws[t] * f(wl.v_pool[wl.block_tables[b, t // P], g, t % P, i])
                                   for t in range(c)) / L)
            mass = [math.fsum(ws[t] for t in range(c) if t // P == p) / L for p in range(-(-c // P))]
            res[b, h] = (o, M + math.log(L), mass)
    return res


def test_matches_pure_python_brute_force_on_tiny():
    wl = W.make("tiny")
    step = kvref.decode_step(wl)
    for (b, h), (o, lse, mass) in _brute(wl).items():
        np.testing.assert_allclose(step["out"][b, h], o, rtol=1e-12, atol=1e-14)
        assert abs(step["lse"][b, h] - lse) < 1e-12
        np.testing.assert_allclose(step["mass"][b, h, :len(mass)], mass, rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ summaries ---

@pytest.mark.parametrize("alpha", [0.5, 0.05])
def test_ema_closed_form_from_zero_state(alpha):
    """Constant group mean x from a zero state: s_n = (1 - (1 - a)^n) x."""
    x = np.array([1.0, -2.0, 0.5, 3.25], dtype=np.float16)
    G, Hkv = 4, 2
    q = np.empty((1, G * Hkv, 4), dtype=np.float16)
    for h in range(G * Hkv):
        # Heads of a group differ but average to x exactly.
        q[0, h] = x + np.float16(0.25 * ((h % G) - 1.5))
    s = np.zeros((2, 1, Hkv, 4))
    a = float(np.float32(alpha))
    for n in range(1, 40):
        s = kvref.update_summaries(q, s, Hkv, alpha, alpha, "f16")
        want = (1.0 - (1.0 - a) ** n) * x.astype(np.float64)
        np.testing.assert_allclose(s[0, 0, 0], want, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(s[1, 0, 1], want, rtol=1e-13, atol=1e-15)


def test_page_max_zero_state_zero_query():
    wl = W.make("tiny")
    step = kvref.decode_step(wl, q=np.zeros_like(wl.q))
    pm = step["page_max"]
    for b in range(wl.B):
        n = wl.pages_of(b)
        assert np.all(pm[:, b, :, :n] == 0.0)
        assert np.all(pm[:, b, :, n:] == -np.inf)


def test_page_max_brackets_page_mass_at_summary_fixed_point():
    """With one head per KV group and both summaries already equal to q (an
    EMA fixed point), a page's max scaled score m_p satisfies
    exp(m_p - lse) <= mass_p <= n_valid(p) * exp(m_p - lse)."""
    wl = W.custom([37, 100, 16], Hq=2, Hkv=2, d=32, page_size=16, seed=21)
    s_prev = np.stack([wl.q.astype(np.float32).reshape(wl.B, wl.Hkv, wl.d)] * 2)
    step = kvref.decode_step(wl, s_prev=s_prev)
    for b in range(wl.B):
        c = int(wl.ctx_lens[b])
        for g in range(wl.Hkv):
            for p in range(wl.pages_of(b)):
                nv = min(16, c - 16 * p)
                for k in range(2):
                    lo = math.exp(step["page_max"][k, b, g, p] - step["lse"][b, g])
                    m = step["mass"][b, g, p]
                    assert lo * (1 - 1e-9) <= m <= nv * lo * (1 + 1e-9)


def test_page_max_matches_brute_force():
    wl = W.make("tiny")
    wl.s_prev = np.random.default_rng(3).standard_normal(wl.s_prev.shape).astype(np.float32)
    step = kvref.decode_step(wl)
    s = step["s_next"]
    P = wl.page_size
    for b in range(wl.B):
        c = int(wl.ctx_lens[b])
        for k in range(2):
            for p in range(wl.max_pages):
                toks = [t for t in range(c) if t // P == p]
                if not toks:
                    assert step["page_max"][k, b, 0, p] == -np.inf
                    continue
                best = max(wl.scale * math.fsum(
                    float(s[k, b, 0, i]) * float(wl.k_pool[wl.block_tables[b, t // P], 0, i // 8, t % P, i % 8])
                    for i in range(wl.d)) for t in toks)
                assert abs(step["page_max"][k, b, 0, p] - best) < 1e-12


# ----------------------------------------------------------- workloads ---

def test_workload_shapes_and_structure():
    wl = W.make("tiny")
    assert wl.ctx_lens.tolist() == [37, 100] and wl.num_pages == 32
    assert len(wl.referenced_pages()) == 10
    wl = W.make("b64_prefix", ctx_divisor=16)
    assert wl.dtype == "bf16" and wl.G == 8
    shared = wl.block_tables[:, : wl.shared_prefix_pages]
    assert np.all(shared == shared[0])
    rest = np.concatenate([wl.block_tables[b, wl.shared_prefix_pages: wl.pages_of(b)] for b in range(wl.B)])
    assert len(np.unique(rest)) == len(rest) and not np.isin(rest, shared[0]).any()


def test_bf16_widening_is_exact():
    x = np.array([1.0, -3.5, 1e-3, 65504.0, 3.0e38], dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    back = kvref.widen(bits, "bf16")
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)
    assert kvref.widen(np.array([0x3F80], dtype=np.uint16), "bf16")[0] == 1.0


# ------------------------------------------------------------- KV append ---

def _read_append_golden():
    kv = {}
    for line in open(os.path.join(GOLDEN, "append_small.txt")):
        if line.strip() and not line.startswith("#"):
            key, *vals = line.split()
            kv[key] = vals
    rows = lambda v: np.array([[int(x) for x in r.split(",")] for r in v], dtype=np.int32)
    ints = lambda v: np.array([int(x) for x in v], dtype=np.int32)
    return kv, rows, ints


def test_append_golden_hand_worked():
    kv, rows, ints = _read_append_golden()
    P, npages, Hkv, d = int(kv["page_size"][0]), int(kv["num_pages"][0]), 2, 8
    table = rows(kv["table"])
    ctx = ints(kv["ctx_in"])
    B = len(ctx)
    k_pool = np.zeros((npages, Hkv, d // 8, P, 8), np.float16)   # chunk-major key tiles
    v_pool = np.zeros((npages, Hkv, P, d), np.float16)
    k_new = (1 + np.arange(B * Hkv * d, dtype=np.float16).reshape(B, Hkv, d))
    v_new = -k_new
    k2, v2, t2, c2, fc2, st = kvref.append_kv(k_pool, v_pool, table, ctx, k_new, v_new,
                                               ints(kv["free_pages"]), int(kv["free_count"][0]), P)
    assert np.array_equal(c2, ints(kv["ctx_out"]))
    assert fc2 == int(kv["free_count_out"][0])
    assert st == int(kv["status"][0]) == kvref.APPEND_FULL | kvref.APPEND_NO_PAGE
    assert np.array_equal(t2, rows(kv["table_out"]))
    want_k = np.zeros_like(k_pool)
    want_v = np.zeros_like(v_pool)
    for w in kv["written"]:
        b, page, slot = (int(x) for x in w.split(":"))
        for g in range(Hkv):
            for i in range(d):                       # key element i: chunk i // 8, lane i % 8
                want_k[page, g, i // 8, slot, i % 8] = k_new[b, g, i]
        want_v[page, :, slot, :] = v_new[b]
    assert np.array_equal(k2, want_k) and np.array_equal(v2, want_v)
    # inputs untouched
    assert np.array_equal(table, rows(kv["table"])) and not k_pool.any()


def test_append_then_gather_reads_the_new_token():
    """On a random paged cache: after the append, logical token ctx_b of every
    appended sequence is the new K/V (read back through the pinned gather), all
    earlier tokens are unchanged, and the pages taken are the top of the free
    list in sequence order, each used once."""
    wl = W.custom([0, 16, 17, 31, 32, 90, 47, 64], Hq=4, Hkv=2, d=16, seed=3, max_pages=6)
    rng = np.random.default_rng(9)
    free = np.setdiff1d(np.arange(wl.num_pages), wl.block_tables[wl.block_tables < wl.num_pages])
    free = rng.permutation(free).astype(np.int32)
    k_new = rng.standard_normal((wl.B, wl.Hkv, wl.d)).astype(np.float16)
    v_new = rng.standard_normal((wl.B, wl.Hkv, wl.d)).astype(np.float16)
    k2, v2, bt2, c2, fc2, st = kvref.append_kv(wl.k_pool, wl.v_pool, wl.block_tables, wl.ctx_lens,
                                                k_new, v_new, free, len(free), wl.page_size)
    need = [b for b, c in enumerate(wl.ctx_lens) if c % 16 == 0 and c < 6 * 16]
    assert st == 0 and fc2 == len(free) - len(need)
    for k, b in enumerate(need):
        assert bt2[b, wl.ctx_lens[b] // 16] == free[len(free) - 1 - k]
    assert np.array_equal(c2, wl.ctx_lens + 1)
    for b in range(wl.B):
        for g in range(wl.Hkv):
            old = kvref.logical_key_rows(wl.k_pool, wl.block_tables, b, g, int(wl.ctx_lens[b]), 16, "f16")
            new = kvref.logical_key_rows(k2, bt2, b, g, int(c2[b]), 16, "f16")
            assert np.array_equal(new[:-1], old) and np.array_equal(new[-1], k_new[b, g].astype(np.float64))
            newv = kvref.logical_rows(v2, bt2, b, g, int(c2[b]), 16, "f16")
            assert np.array_equal(newv[-1], v_new[b, g].astype(np.float64))
    # Only the appended slots changed in the pools.
    changed = np.argwhere(np.any(v2 != wl.v_pool, axis=-1))
    assert len(changed) <= wl.B * wl.Hkv
    changed_k = np.argwhere(np.any(k2 != wl.k_pool, axis=(2, 4)))   # (page, head, slot)
    assert len(changed_k) <= wl.B * wl.Hkv


def test_append_bad_page_ids_change_nothing_for_that_sequence():
    kv, rows, ints = _read_append_golden()
    P = 16
    k_pool = np.zeros((16, 1, 1, P, 8), np.float16)            # d = 8: one chunk
    v_pool = np.zeros((16, 1, P, 8), np.float16)
    table = np.array([[3, 15], [99, 15], [4, 15]], np.int32)   # row 1 points outside the pool
    ctx = np.array([5, 7, 16], np.int32)
    free = np.array([-1], np.int32)                             # seq 2 would take page -1
    k_new = np.ones((3, 1, 8), np.float16)
    k2, v2, t2, c2, fc2, st = kvref.append_kv(k_pool, v_pool, table, ctx, k_new, k_new, free, 1, P)
    assert st == kvref.APPEND_BAD_PAGE
    assert np.array_equal(c2, [6, 7, 16]) and fc2 == 0 and np.array_equal(t2, table)
    assert k2[3, 0, 0, 5].all() and k2.sum() == 8
    assert v2[3, 0, 5].all() and v2.sum() == 8


@pytest.mark.parametrize("split", [16, 32, 64, 256, 1 << 20])
def test_split_partials_merged_by_lse_equal_the_full_softmax(split):
    """The method reaches the plain softmax only up to rounding: per queue
    task (split) a partial max m, sum l and weighted V sum o, merged with the
    log-sum-exp rule, must give the oracle's out and lse to ~1e-12 (the
    pages' split-KV decode over the compact queue; the merge is the textbook
    one).  Computed here from the gathered rows, independently of
    ``kvref.attention``'s single pass."""
    wl = W.custom([37, 100, 1, 0, 300], Hq=6, Hkv=2, d=16, seed=17)
    out, lse, _ = kvref.attention(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.ctx_lens,
                                  wl.page_size, wl.scale, wl.dtype)
    tasks, offs, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, split)
    parts = {}
    for b, g, t0, t1 in tasks:
        K = kvref.logical_key_rows(wl.k_pool, wl.block_tables, b, g, int(wl.ctx_lens[b]), 16, wl.dtype)[t0:t1]
        V = kvref.logical_rows(wl.v_pool, wl.block_tables, b, g, int(wl.ctx_lens[b]), 16, wl.dtype)[t0:t1]
        for h in range(g * wl.G, (g + 1) * wl.G):
            x = wl.scale * (K @ kvref.widen(wl.q[b, h], wl.dtype))
            m = x.max()
            w = np.exp(x - m)
            parts.setdefault((b, h), []).append((m, w.sum(), w @ V))
    for b in range(wl.B):
        for h in range(wl.Hq):
            if wl.ctx_lens[b] == 0:
                assert (b, h) not in parts and lse[b, h] == -np.inf and not out[b, h].any()
                continue
            ps = parts[(b, h)]
            M = max(p[0] for p in ps)
            L = sum(np.exp(p[0] - M) * p[1] for p in ps)
            O = sum(np.exp(p[0] - M) * p[2] for p in ps) / L
            np.testing.assert_allclose(O, out[b, h], rtol=1e-12, atol=1e-14)
            assert abs(M + np.log(L) - lse[b, h]) <= 1e-12 * max(1.0, abs(lse[b, h]))


# ---------------------------------------------------------- input checks ---

def _tiny_check_case():
    # Two sequences of 37 and 0 tokens, rows of 4 pages, pool of 10 pages,
    # one KV head, 16-token splits.  The queue written out by hand.
    ctx = [37, 0]
    bt = np.array([[3, 7, 1, -1], [-1, 99, -1, -1]], dtype=np.int32)   # unused cells hold junk
    tasks = np.array([[0, 0, 0, 16], [0, 0, 16, 32], [0, 0, 32, 37], [9, 9, 9, 9]], dtype=np.int32)
    go = np.array([0, 3, 3], dtype=np.int32)
    return ctx, bt, tasks, go


def test_check_inputs_hand_worked_clean_case():
    """Junk in table cells no sequence uses and queue rows past n_tasks is
    allowed: the status is 0."""
    ctx, bt, tasks, go = _tiny_check_case()
    assert kvref.check_inputs(ctx, bt, 10, 16, 1, 16) == 0
    assert kvref.check_inputs(ctx, bt, 10, 16, 1, 16, capacity=8, tasks=tasks, group_offsets=go,
                              n_tasks=[3]) == 0


@pytest.mark.parametrize("case,want", [
    ("negative length", kvref.CHECK_LENGTH),
    ("length past the row", kvref.CHECK_LENGTH | kvref.CHECK_QUEUE),
    ("used page id = num_pages", kvref.CHECK_PAGE),
    ("used page id negative", kvref.CHECK_PAGE),
    ("task end off by one", kvref.CHECK_QUEUE),
    ("tasks swapped", kvref.CHECK_QUEUE),
    ("n_tasks one more", kvref.CHECK_QUEUE),
    ("n_tasks past capacity", kvref.CHECK_QUEUE),
    ("group offset moved", kvref.CHECK_QUEUE),
])
def test_check_inputs_flags_each_violation(case, want):
    """Each kind of violation sets its own bit (a length past the row is
    clamped, so the hand-written queue no longer matches either)."""
    ctx, bt, tasks, go = _tiny_check_case()
    n = [3]
    cap = 8
    if case == "negative length":
        ctx = [37, -1]
    elif case == "length past the row":
        ctx = [65, 0]
        bt[0, 3] = 5   # clamped to 64 tokens, the row's fourth page is now used
    elif case == "used page id = num_pages":
        bt[0, 2] = 10
    elif case == "used page id negative":
        bt[0, 0] = -1
    elif case == "task end off by one":
        tasks[2, 3] = 36
    elif case == "tasks swapped":
        tasks[[0, 1]] = tasks[[1, 0]]
    elif case == "n_tasks one more":
        n = [4]
    elif case == "n_tasks past capacity":
        cap = 2
    elif case == "group offset moved":
        go[1] = 2
    got = kvref.check_inputs(ctx, bt, 10, 16, 1, 16, capacity=cap, tasks=tasks, group_offsets=go,
                             n_tasks=n)
    assert got == want, (case, got)


def test_check_inputs_accepts_every_workload_queue():
    """The queue build_queue gives for a workload's own lengths, with its
    tables, passes every check."""
    for name, div in (("tiny", 1), ("b8_bimodal", 64), ("b64_prefix", 32)):
        wl = W.make(name, ctx_divisor=div) if div > 1 else W.make(name)
        tasks, go, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, wl.split_tokens)
        assert kvref.check_inputs(wl.ctx_lens, wl.block_tables, wl.num_pages, wl.page_size, wl.Hkv,
                                  wl.split_tokens, capacity=max(n, 1), tasks=tasks,
                                  group_offsets=go, n_tasks=[n]) == 0


# ------------------------------------------------ compress-or-acquire decision ---
# GrowPage (mlsanity.com entry, Abstract; aitrending.vip article, Technical
# Details): working sets of the fast and slow summaries, compared at each
# capacity boundary.  Reading and hand-worked cases: tests/golden/growpage_decision.txt.

import itertools  # noqa: E402

import decision_cases  # noqa: E402


@pytest.mark.parametrize("case", decision_cases.load(), ids=lambda c: c["name"])
def test_decision_hand_worked_cases(case):
    r = kvref.budget_decision(case["page_max"], [case["ctx"]], 16, case["tau"])
    assert np.array_equal(r["ws_size"][:, 0], case["ws_size"])
    assert np.array_equal(r["ws_union"][:, 0], case["union"])
    assert r["decision"][0] == case["decision"]
    assert r["victim"][0] == case["victim"]


def _brute_working_set(x, tau):
    """Smallest set of pages that is closed upward in score (a page in it
    brings every page scoring at least as high) and holds >= tau of the
    softmax weight, found by trying every subset."""
    n = len(x)
    w = [math.exp(v - max(x)) for v in x]
    Z = sum(w)
    best = None
    for mask in range(1, 1 << n):
        s = [i for i in range(n) if mask >> i & 1]
        if any(x[j] >= x[i] and j not in s for i in s for j in range(n)):
            continue
        if sum(w[i] for i in s) / Z >= tau and (best is None or len(s) < len(best)):
            best = s
    return best


@pytest.mark.parametrize("seed", range(40))
def test_working_set_matches_brute_force(seed):
    """Scores from a few integer levels (many ties); tau drawn away from every
    achievable covered fraction so rounding cannot decide."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 8))
    x = [float(v) for v in rng.integers(-3, 3, n) * 0.7]
    w = np.exp(np.array(x) - max(x))
    fracs = sorted({float(w[np.array(x) >= lv].sum() / w.sum()) for lv in x})
    while True:
        tau = float(rng.uniform(0.05, 1.0))
        if all(abs(tau - f) > 1e-9 for f in fracs):
            break
    size, level = kvref.working_set(x, tau)
    want = _brute_working_set(x, tau)
    assert size == len(want)
    assert level == min(x[i] for i in want)
    assert sorted(i for i in range(n) if x[i] >= level) == sorted(want)


def test_working_set_depends_only_on_score_differences():
    """The weights are a softmax: shifting every score of a set by a constant
    changes no working set (a fixed threshold on raw scores would)."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = rng.standard_normal(30) * 3
        for c in (-50.0, 7.5, 300.0):
            assert kvref.working_set(x + c, 0.9)[0] == kvref.working_set(x, 0.9)[0]


def test_working_set_geometric_weights_closed_form():
    """Scores -p ln 2 give weights 2^-p / (1 - 2^-n): the top k pages hold
    (1 - 2^-k) / (1 - 2^-n), so the set for tau is the smallest such k."""
    n = 12
    x = [-p * math.log(2.0) for p in range(n)]
    for tau in (0.3, 0.5001, 0.74, 0.76, 0.9, 0.97, 0.999):
        k = next(k for k in range(1, n + 1)
                 if Fraction(2 ** k - 1, 2 ** k) / Fraction(2 ** n - 1, 2 ** n) >= Fraction(tau))
        assert kvref.working_set(x, tau)[0] == k, tau


def test_working_set_ties_and_extremes():
    assert kvref.working_set([1.0] * 5, 1e-6) == (5, 1.0)            # one level: all
    assert kvref.working_set([2.0, 1.0, 1.0], 1.0)[0] == 3            # tau 1: every page
    assert kvref.working_set([50.0, 0.0, 0.0], 0.5)[0] == 1           # a dominant page
    assert kvref.working_set([-np.inf, 0.0, -np.inf], 0.99)[0] == 1   # -inf weighs 0
    assert kvref.working_set([-np.inf, -np.inf], 0.5)[0] == 2         # all -inf tie
    assert kvref.working_set([], 0.9) == (0, math.inf)


def test_decision_from_given_working_sets_is_the_same():
    """Deciding from the sets' sizes (another implementation's sets) gives
    the oracle's own decision when the sizes agree."""
    rng = np.random.default_rng(5)
    pm = rng.standard_normal((2, 6, 3, 40)) * 2
    ctx = np.array([640, 0, 16, 300, 48, 17])
    a = kvref.budget_decision(pm, ctx, 16, 0.8)
    b = kvref.budget_decision(pm, ctx, 16, 0.8, ws_size=a["ws_size"])
    for key in ("ws_size", "ws_level", "ws_union", "decision", "victim"):
        assert np.array_equal(a[key], b[key]), key


def test_decision_rules_on_random_sequences():
    """Every decision follows its rule: none off a boundary; acquire exactly
    when |F| > |S| or F and S cover every page; otherwise the victim lies
    outside both sets and no page outside them has a lower best slow score
    (or an equal one and a lower index).  F and S are checked against the
    union of per-head brute-force sets."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        B, Hkv = 4, int(rng.integers(1, 4))
        npg_max = 7
        pm = np.round(rng.standard_normal((2, B, Hkv, npg_max)) * 1.5, 1)
        ctx = rng.integers(0, npg_max * 16 + 1, B)
        ctx[rng.random(B) < 0.5] = rng.integers(0, npg_max + 1) * 16
        tau = float(rng.choice([0.5, 0.62, 0.83, 0.95]))
        r = kvref.budget_decision(pm, ctx, 16, tau)
        for b in range(B):
            npg = -(-int(ctx[b]) // 16)
            sets, near_tie = [], False
            for k in range(2):
                u = set()
                for g in range(Hkv):
                    x = np.array(pm[k, b, g, :npg])
                    if npg == 0:
                        continue
                    w = np.exp(x - x.max())
                    if any(abs(w[x >= lv].sum() / w.sum() - tau) < 1e-9 for lv in x):
                        near_tie = True
                    u |= set(_brute_working_set(list(x), tau))
                sets.append(u)
            F, S = (set().union(set(), *[set(np.flatnonzero(pm[k, b, g, :npg] >= r["ws_level"][k, b, g]))
                                         for g in range(Hkv)]) for k in (0, 1))
            if not near_tie:
                assert sets == [F, S]
            assert r["ws_union"][0, b] == len(F) and r["ws_union"][1, b] == len(S)
            outside = [p for p in range(npg) if p not in F and p not in S]
            d, v = r["decision"][b], r["victim"][b]
            if ctx[b] == 0 or ctx[b] % 16:
                assert d == kvref.DECIDE_NONE and v == -1
            elif len(F) > len(S) or not outside:
                assert d == kvref.DECIDE_ACQUIRE and v == -1
            else:
                assert d == kvref.DECIDE_COMPRESS and v in outside
                slow = pm[1, b, :, :npg].max(axis=0)
                assert all((slow[v], v) <= (slow[p], p) for p in outside)
