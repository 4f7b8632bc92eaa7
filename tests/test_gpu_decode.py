"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Queue, group offsets and gather offsets bit for bit; attention outputs, page
mass, summaries and page maxima within the tolerances in gpu_util.  Oracle-
sized runs compare every output; full-size runs (in the launch configuration
the benchmark times) compare one query head of every (sequence, KV head)
group plus sampled rows, and check properties of every row.  Every buffer
the library writes starts filled with NaN or junk (DecodeStep.scribble), so
an entry a kernel skips cannot pass as a leftover zero.
"""

import dataclasses

import numpy as np
import pytest

from gpu_util import assert_close, compare_step, group_rows, oracle_step, sample_rows, say
from oracle import kvref
from paged_kv_cache_07_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_07_amd import binding
    binding.lib()


def _run(wl, budget=True, split_tokens=None, label="", one_call=False, stream_kv=False):
    """Separate calls (queue, attention + merge, page-mass finish), or with
    one_call the single kvpage_decode_step call bench.py times."""
    from paged_kv_cache_07_amd.device import DecodeStep
    say("run", label or wl.name, "ctx", wl.ctx_lens.tolist()[:8], "G", wl.G, "d", wl.d,
        wl.dtype, "split", split_tokens or wl.split_tokens, "budget", budget, "one_call", one_call,
        "stream_kv", stream_kv)
    ds = DecodeStep(wl, budget=budget, split_tokens=split_tokens, stream_kv=stream_kv)
    if one_call:
        ds.step()
    else:
        ds.run()
    return ds, ds.results()


# ------------------------------------------------------------------ queue ---

@pytest.mark.parametrize("name", W.NAMES)
def test_queue_bit_exact_full_size(name):
    wl = W.make(name, fill_pools=False)
    wl = dataclasses.replace(wl, k_pool=np.zeros((1, wl.Hkv, 16, wl.d), np.float16),
                             v_pool=np.zeros((1, wl.Hkv, 16, wl.d), np.float16), num_pages=1,
                             q=np.zeros((wl.B, wl.Hq, wl.d), np.float16), dtype="f16")
    from paged_kv_cache_07_amd.device import DecodeStep
    for split in (256, 16, 128):
        say("queue", name, split)
        ds = DecodeStep(wl, budget=False, split_tokens=split)
        ds.build_queue()
        torch.cuda.synchronize()
        tasks, offs, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, split)
        assert int(ds.n_tasks.item()) == n
        assert np.array_equal(ds.tasks[:n].cpu().numpy(), tasks)
        assert np.array_equal(ds.group_offsets.cpu().numpy(), offs)


@pytest.mark.parametrize("ctx", [[0], [1], [0, 0, 5], [15, 16, 17], [255, 256, 257, 0, 512],
                                 [4096, 1, 0, 33]])
def test_queue_edge_lengths(ctx):
    wl = W.custom(ctx, Hq=8, Hkv=4, d=64, split_tokens=256)
    from paged_kv_cache_07_amd.device import DecodeStep
    for split in (16, 32, 256):
        say("queue-edge", ctx, split)
        ds = DecodeStep(wl, budget=False, split_tokens=split)
        ds.build_queue()
        torch.cuda.synchronize()
        tasks, offs, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, split)
        assert int(ds.n_tasks.item()) == n
        assert np.array_equal(ds.tasks[:n].cpu().numpy(), tasks)
        assert np.array_equal(ds.group_offsets.cpu().numpy(), offs)


# ----------------------------------------------------------- page gather ---

@pytest.mark.parametrize("case", ["tiny16", "tiny256", "edge", "b8_bimodal_small", "b8_zipf_full"])
def test_gather_offsets_bit_exact(case):
    from paged_kv_cache_07_amd.device import DecodeStep
    split = 256
    if case.startswith("tiny"):
        wl, split = W.make("tiny"), int(case[4:])
    elif case == "edge":
        wl = W.custom([1, 17, 255, 256, 257, 0], Hq=4, Hkv=2, d=64)
    elif case == "b8_bimodal_small":
        wl = W.make("b8_bimodal", ctx_divisor=16)
    else:
        wl = W.make("b8_zipf", fill_pools=False)
        kp = np.zeros((1, 8, 16, 128), np.float16)
        wl = dataclasses.replace(wl, k_pool=kp, v_pool=kp, q=np.zeros((wl.B, wl.Hq, wl.d), np.float16))
    say("gather", case)
    ds = DecodeStep(wl, budget=False, split_tokens=split)
    ds.build_queue()
    offs = ds.gather_offsets().cpu().numpy()
    n = int(ds.n_tasks.item())
    tasks = ds.tasks[:n].cpu().numpy()
    rows = np.arange(n) if n <= 4096 else np.random.default_rng(1).choice(n, 256, replace=False)
    want = kvref.gather_offsets(wl.block_tables, tasks[rows], wl.Hkv, wl.page_size, wl.d, split)
    assert np.array_equal(offs[rows], want)


def test_one_hot_query_returns_the_physical_address():
    """V rows hold their own (page, head, slot); a query singling out one
    logical token must return that token's physical address through out."""
    wl = W.custom([37, 100, 300], Hq=8, Hkv=2, d=64, seed=11)
    P = wl.page_size
    v = np.zeros(wl.v_pool.shape, dtype=np.float16)
    pg, hd, sl = np.meshgrid(np.arange(wl.num_pages), np.arange(wl.Hkv), np.arange(P), indexing="ij")
    v[..., 0], v[..., 1], v[..., 2] = pg, hd, sl
    rng = np.random.default_rng(0)
    k = np.zeros(wl.k_pool.shape, dtype=np.float16)
    q = np.zeros(wl.q.shape, dtype=np.float16)
    want = {}
    for b, c in enumerate(wl.ctx_lens):
        for g in range(wl.Hkv):
            t = int(rng.integers(0, c))
            page = wl.block_tables[b, t // P]
            k[page, g, g // 8, t % P, g % 8] = 8.0     # key element g of slot t % P
            q[b, g * wl.G:(g + 1) * wl.G, g] = 8.0 * np.sqrt(wl.d)
            want[b, g] = (page, g, t % P)
    wl2 = dataclasses.replace(wl, k_pool=k, v_pool=v, q=q)
    _, res = _run(wl2, budget=False, label="one-hot")
    for (b, g), addr in want.items():
        for h in range(g * wl.G, (g + 1) * wl.G):
            np.testing.assert_allclose(res["out"][b, h, :3], addr, rtol=0, atol=0.5)


# -------------------------------------------------------------- attention ---

@pytest.mark.parametrize("split", [16, 32, 256])
def test_tiny_all_outputs(split):
    wl = W.make("tiny")
    wl.s_prev = np.random.default_rng(2).standard_normal(wl.s_prev.shape).astype(np.float32)
    _, res = _run(wl, split_tokens=split, label=f"tiny-S{split}")
    compare_step(res, oracle_step(wl, split_tokens=split))


@pytest.mark.parametrize("name,div", [("b1", 16), ("b8_bimodal", 32), ("b8_uniform", 32),
                                      ("b8_zipf", 64), ("b64_prefix", 16), ("b4_bimodal", 32)])
def test_oracle_sized_configs_all_outputs(name, div):
    wl = W.make(name, ctx_divisor=div)
    _, res = _run(wl, label=f"{name}/{div}")
    compare_step(res, oracle_step(wl), label=name)


@pytest.mark.parametrize("name,split", [("b1", 256), ("b8_bimodal", 256), ("b8_uniform", 256),
                                        ("b8_zipf", 256), ("b64_prefix", 256), ("b4_bimodal", 256),
                                        ("b8_bimodal", 1024), ("b8_zipf", 2048),
                                        ("b4_bimodal", 1024), ("b8_uniform", 1024)])
def test_full_size_sampled_rows(name, split):
    """Full-size workloads in the launch configurations bench.py times (one
    kvpage_decode_step call, streaming tile loads except a shared prefix's;
    the B8 and B4 workloads also at the splits the policy picks for them,
    run as 16-page pieces): one query head of
    every (sequence, KV head) group, plus sampled rows, against the oracle."""
    wl = dataclasses.replace(W.make(name), split_tokens=split)
    if wl.shares_pages():   # streaming except the shared prefix pages, as the benchmark runs it
        from paged_kv_cache_07_amd.device import DecodeStep
        say("run", name, "full", "split", split, "shared prefix loads")
        ds = DecodeStep(wl, stream_kv=True, shared_pages=W.shared_leading_pages(wl))
        ds.step()
        res = ds.results()
    else:
        _, res = _run(wl, label=f"{name}-full-S{split}", one_call=True, stream_kv=True)
    tasks, offs, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, wl.split_tokens)
    assert res["n_tasks"] == n
    assert np.array_equal(res["tasks"], tasks) and np.array_equal(res["group_offsets"], offs)
    rows = group_rows(wl, extra=6, seed=3)
    ref = oracle_step(wl, rows=rows)
    compare_step(res, ref, label=name)
    # Properties that hold for every row at any size.
    mass = res["mass"]
    for b in range(wl.B):
        npg = wl.pages_of(b)
        np.testing.assert_allclose(mass[b, :, :npg].sum(axis=1), 1.0, atol=1e-4)
        assert np.all(mass[b, :, npg:] == 0)
        assert np.all(res["page_max"][:, b, :, npg:] == -np.inf)
        assert np.all(np.isfinite(res["page_max"][:, b, :, :npg]))
    assert np.all(np.isfinite(res["out"])) and np.all(np.isfinite(res["lse"]))


@pytest.mark.parametrize("one_call", [True, False])
def test_wave_merge_several_page_slices(one_call):
    """16 sequences x 32 heads = 512 rows take the one-wavefront-per-row
    merge, and a 2200-page table row splits each row's page mass and page-max
    tails into three slices of 1024 pages (slices past the first recompute
    the row's lse).  Contexts cross slice boundaries (16385, 17000, 18001,
    20000 tokens) next to short and empty ones.  Every row and every output
    against the oracle, on the one-call step (merge fused with the finish)
    and on the separate calls (merge, then the finish kernel's slices)."""
    ctx = [20000, 517, 0, 17000, 300, 16, 1, 4096, 33, 18001, 1025, 255, 700, 16385, 2, 9000]
    wl = W.custom(ctx, Hq=32, Hkv=8, d=128, seed=71, max_pages=2200)
    wl.s_prev = np.random.default_rng(14).standard_normal(wl.s_prev.shape).astype(np.float32)
    assert wl.B * wl.Hq >= 512 and wl.max_pages > 2 * 1024
    _, res = _run(wl, label="wave-merge-slices", one_call=one_call, stream_kv=True)
    compare_step(res, oracle_step(wl), label=f"wave merge, one_call={one_call}")


def test_zipf_chained_steps_with_summary_state():
    """Sixteen decode steps: fresh queries each step, s_next fed back as s_prev."""
    from paged_kv_cache_07_amd.device import DecodeStep
    wl = W.make("b8_zipf", ctx_divisor=64)
    ds = DecodeStep(wl)
    s_prev = wl.s_prev.astype(np.float64)
    q = wl.q
    for step in range(wl.steps):
        say("zipf-chain step", step)
        if step:
            q = W.draw_queries(wl)
            ds.set_query(q)
            ds.swap_summaries()
            ds.scribble()
        ds.run()
        res = ds.results()
        ref = oracle_step(wl, q=q, s_prev=s_prev)
        compare_step(res, ref, label=f"step {step}")
        s_prev = ref["s_next"]


@pytest.mark.parametrize("G,d,dtype", [(1, 128, "f16"), (2, 64, "bf16"), (4, 64, "f16"),
                                       (8, 128, "bf16"), (8, 64, "f16"), (3, 128, "f16"),
                                       (5, 128, "bf16")])
def test_edge_lengths_all_outputs(G, d, dtype):
    ctx = [0, 1, 15, 16, 17, 255, 256, 257, 1000]
    wl = W.custom(ctx, Hq=2 * G, Hkv=2, d=d, dtype=dtype, seed=G * 100 + d)
    wl.s_prev = np.random.default_rng(5).standard_normal(wl.s_prev.shape).astype(np.float32)
    for split in (16, 256):
        _, res = _run(wl, split_tokens=split, label=f"edge G{G} d{d} {dtype} S{split}")
        compare_step(res, oracle_step(wl, split_tokens=split))


def test_longest_table_row_is_fully_used():
    """Context equal to max_pages * P: the last table column is read."""
    wl = W.custom([16 * 40, 3], Hq=4, Hkv=1, d=128, max_pages=40)
    _, res = _run(wl, label="max-ctx")
    compare_step(res, oracle_step(wl))


def test_all_sequences_empty():
    wl = W.custom([0, 0, 0], Hq=4, Hkv=2, d=64)
    _, res = _run(wl, label="empty")
    assert res["n_tasks"] == 0
    assert np.all(res["out"] == 0) and np.all(res["lse"] == -np.inf)
    assert np.all(res["mass"] == 0) and np.all(res["page_max"] == -np.inf)
    ref = oracle_step(wl)
    assert_close("s_next", res["s_next"], ref["s_next"])


# -------------------------------------------------------------- robustness ---

def test_nan_poison_in_unreferenced_memory_changes_nothing():
    for name, div in (("tiny", 1), ("b8_bimodal", 32), ("b64_prefix", 16)):
        wl = W.make(name, ctx_divisor=div) if div > 1 else W.make(name)
        _, clean = _run(wl, label=f"{name}-clean")
        _, dirty = _run(W.poison_unused(wl), label=f"{name}-poisoned")
        for key in ("out_bits", "lse", "mass", "page_max", "s_next"):
            assert np.array_equal(clean[key], dirty[key]), (name, key)


def test_physical_page_permutation_is_bitwise_invariant():
    wl = W.make("b8_uniform", ctx_divisor=32)
    _, base = _run(wl, label="perm-base")
    pi = np.random.default_rng(9).permutation(wl.num_pages)
    k = np.empty_like(wl.k_pool)
    v = np.empty_like(wl.v_pool)
    k[pi] = wl.k_pool
    v[pi] = wl.v_pool
    wl2 = dataclasses.replace(wl, k_pool=k, v_pool=v, block_tables=pi[wl.block_tables].astype(np.int32))
    _, moved = _run(wl2, label="perm-moved")
    for key in ("out_bits", "lse", "mass", "page_max", "s_next"):
        assert np.array_equal(base[key], moved[key]), key


def test_repeat_runs_are_bitwise_identical_and_split_calls_match():
    from paged_kv_cache_07_amd.device import DecodeStep
    wl = W.make("b8_bimodal", ctx_divisor=16)
    say("determinism")
    ds = DecodeStep(wl)
    ds.run()
    first = ds.results()
    ds.run()
    second = ds.results()
    for key in ("out_bits", "lse", "mass", "page_max", "s_next"):
        assert np.array_equal(first[key], second[key]), key
    # decode_attn == split_attn followed by merge_splits
    ds.out.zero_()
    ds.lse.zero_()
    ds.build_queue()
    ds.split_attn()
    ds.merge_splits()
    ds.page_mass_finish()
    third = ds.results()
    for key in ("out_bits", "lse", "mass", "page_max", "s_next"):
        assert np.array_equal(first[key], third[key]), key


@pytest.mark.parametrize("budget", [True, False])
def test_one_call_step_equals_separate_calls(budget):
    """kvpage_decode_step (fused merge + finish, timed attention launch) gives
    the same bits as kvpage_build_queue + kvpage_decode_attn + kvpage_page_mass
    where both run the same schedule.  Where the one-call step runs one class
    of KV heads per XCD (several sequences, Hkv a multiple of 8) its run
    partials differ from the separate calls' linear schedule: the queue, page
    maxima and summaries still agree bit for bit, out, lse and page mass to
    rounding (and both match the oracle)."""
    from paged_kv_cache_07_amd import binding
    from paged_kv_cache_07_amd.device import DecodeStep
    for name, div in (("tiny", 1), ("b8_bimodal", 32), ("b64_prefix", 16), ("b8_zipf", 64)):
        wl = W.make(name, ctx_divisor=div) if div > 1 else W.make(name)
        wl.s_prev = np.random.default_rng(4).standard_normal(wl.s_prev.shape).astype(np.float32)
        say("one-call", name, budget)
        a = DecodeStep(wl, budget=budget)
        a.run()
        ra = a.results()
        b = DecodeStep(wl, budget=budget)
        start, stop = binding.HipEvent(), binding.HipEvent()
        b.step(opts=binding.make_opts(start, stop))
        rb = b.results()
        stop.synchronize()
        assert start.elapsed_ms(stop) > 0
        same = b.schedule_classes() == a.schedule_classes() == 1
        assert b.schedule_classes() == (8 if wl.B >= 2 and wl.Hkv % 8 == 0 else 1), name
        keys = ["tasks", "group_offsets"] + (["page_max", "s_next"] if budget else [])
        keys += (["out_bits", "lse"] + (["mass"] if budget else [])) if same else []
        for key in keys:
            assert np.array_equal(ra[key], rb[key]), (name, key)
        if not same:
            for key in ("out", "lse") + (("mass",) if budget else ()):
                assert_close(key, rb[key], ra[key])
        ref = oracle_step(wl)
        compare_step(rb, ref, budget=budget, label=name)
        if not same:
            compare_step(ra, ref, budget=budget, label=name)


@pytest.mark.parametrize("max_wg,split", [(1, 256), (3, 256), (1, 64), (3, 32), (2, 128),
                                          (8, 256), (16, 64), (8, 1024)])
def test_long_wave_runs_fold_consecutive_tasks(max_wg, split):
    """Few workgroups: each wavefront walks a long stretch of the queue,
    folding consecutive tasks of one (sequence, KV head) into one partial and
    crossing group boundaries inside its stretch.  Splits shorter than 16
    pages put several short tasks in one run, whose staged page values must
    land on the right logical pages.  With 8 or 16 workgroups the one-call
    step of the Hkv = 8 batches runs one class of KV heads per XCD, so run
    starts sit at class-chunk offsets the merge must recompute."""
    from paged_kv_cache_07_amd import binding
    from paged_kv_cache_07_amd.device import DecodeStep
    cases = [W.make("b8_bimodal", ctx_divisor=32), W.make("b64_prefix", ctx_divisor=16),
             W.custom([0, 1, 300, 17, 1000, 256, 0, 513], Hq=8, Hkv=2, d=128, seed=12),
             W.custom([700, 33, 2049], Hq=16, Hkv=2, d=64, dtype="bf16", seed=13)]
    for wl in cases:
        wl.s_prev = np.random.default_rng(8).standard_normal(wl.s_prev.shape).astype(np.float32)
        for budget in (True, False):
            say("long-runs", wl.name, "max_wg", max_wg, "split", split, "budget", budget)
            ds = DecodeStep(wl, budget=budget, split_tokens=split)
            ds.step(opts=binding.make_opts(max_workgroups=max_wg))
            res = ds.results()
            classes = 8 if (max_wg % 8 == 0 and wl.B >= 2 and wl.Hkv % 8 == 0) else 1
            assert ds.schedule_classes() == classes, (wl.name, max_wg)
            compare_step(res, oracle_step(wl, split_tokens=split), budget=budget,
                         label=f"{wl.name} wg{max_wg} S{split}")


@pytest.mark.parametrize("split,max_wg", [(512, 0), (1024, 0), (4096, 0), (512, 1), (1024, 3),
                                           (2048, 2), (4096, 1)])
def test_long_splits_run_as_pieces(split, max_wg):
    """Splits of 32 to 256 pages run as consecutive 16-page pieces of one
    task.  Contexts on both sides of piece and split boundaries; with few
    workgroups a wavefront folds several multi-piece tasks (and group
    changes) into its runs, whose staged page values cover more than one
    piece.  Every output against the oracle, on the one-call step and on the
    separate calls, with and without the budgeting outputs."""
    from paged_kv_cache_07_amd import binding
    from paged_kv_cache_07_amd.device import DecodeStep
    ctx = [0, 1, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 4095, 4096, 4097, 9000]
    cases = [W.custom(ctx, Hq=16, Hkv=4, d=128, seed=31, max_pages=600),
             W.custom([3000, 17, 8200, 700], Hq=16, Hkv=2, d=64, dtype="bf16", seed=32),
             W.make("b8_bimodal", ctx_divisor=16)]
    opts = binding.make_opts(max_workgroups=max_wg) if max_wg else None
    for wl in cases:
        wl.s_prev = np.random.default_rng(6).standard_normal(wl.s_prev.shape).astype(np.float32)
        ref = oracle_step(wl, split_tokens=split)
        for budget, one_call, stream_kv in ((True, True, True), (True, False, False),
                                            (False, True, False)):
            say("pieces", wl.name, "split", split, "max_wg", max_wg, "budget", budget,
                "one_call", one_call, "stream", stream_kv)
            ds = DecodeStep(wl, budget=budget, split_tokens=split, stream_kv=stream_kv)
            if one_call:
                ds.step(opts=opts)
            else:
                ds.run()
            res = ds.results()
            tasks, offs, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, split)
            assert res["n_tasks"] == n
            assert np.array_equal(res["tasks"], tasks) and np.array_equal(res["group_offsets"], offs)
            compare_step(res, ref, budget=budget,
                         label=f"{wl.name} S{split} wg{max_wg} one_call={one_call}")


@pytest.mark.parametrize("ctx,extra_pages,split,max_wg", [
    (32768, 0, 256, 0),    # context fills the table row (the headline shape)
    (32768, 0, 256, 3),    # the same with long wavefront runs (chunks of 15 tasks)
    (4000, 6, 256, 0),     # table wider by less than a split
    (4000, 40, 256, 0),    # table wider by more than a split
    (1, 0, 256, 0), (17, 3, 64, 0), (257, 0, 128, 0), (5000, 0, 16, 0), (3000, 1, 32, 2)])
def test_one_sequence_table_widths(ctx, extra_pages, split, max_wg):
    """One sequence in the one-call step (fused queue build), with a table
    exactly fitting the context, wider by less than a split and wider by more
    than a split: the bits equal the separate calls and match the oracle."""
    from paged_kv_cache_07_amd import binding
    from paged_kv_cache_07_amd.device import DecodeStep
    max_pages = -(-ctx // 16) + extra_pages
    wl = W.custom([ctx], Hq=32, Hkv=8, d=128, seed=40 + ctx % 97, max_pages=max_pages)
    wl.s_prev = np.random.default_rng(9).standard_normal(wl.s_prev.shape).astype(np.float32)
    ref = oracle_step(wl, split_tokens=split)
    for budget, stream_kv in ((True, True), (False, False)):
        say("one-seq", ctx, "table", max_pages, "split", split, "max_wg", max_wg,
            "budget", budget, "stream", stream_kv)
        a = DecodeStep(wl, budget=budget, split_tokens=split, stream_kv=stream_kv)
        a.run()
        ra = a.results()
        b = DecodeStep(wl, budget=budget, split_tokens=split, stream_kv=stream_kv)
        b.step(opts=binding.make_opts(max_workgroups=max_wg) if max_wg else None)
        rb = b.results()
        keys = ["out_bits", "lse", "tasks", "group_offsets"] + (
            ["mass", "page_max", "s_next"] if budget else [])
        # A different grid folds tasks into different runs: then the values
        # agree to rounding only, the queue still bit for bit.
        for key in keys if not max_wg else ["tasks", "group_offsets"]:
            assert np.array_equal(ra[key], rb[key]), key
        compare_step(rb, ref, budget=budget, label=f"ctx{ctx} table{max_pages} S{split}")


@pytest.mark.parametrize("ctx", [[8192], [4096] * 4, [100, 3000, 0, 700], [32768]])
def test_chosen_split_all_outputs(ctx):
    """The split the policy picks for this device (short splits for short
    batches) gives the oracle's outputs, and its queue has a task per
    resident wavefront unless even page-sized splits cannot."""
    from paged_kv_cache_07_amd import binding as K
    wl = W.custom(ctx, Hq=32, Hkv=8, d=128, seed=21)
    wl.s_prev = np.random.default_rng(5).standard_normal(wl.s_prev.shape).astype(np.float32)
    shape = K.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.page_size, 256, wl.max_pages,
                         wl.num_pages, wl.dtype, wl.scale)
    split = K.kvpage_choose_split(shape, wl.ctx_lens.tolist())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert split == K.kvpage_choose_split(shape, wl.ctx_lens.tolist(), 4 * cus)
    tasks = wl.Hkv * sum(-(-int(c) // split) for c in ctx)
    assert split == 16 or tasks >= 4 * cus
    ds, res = _run(wl, split_tokens=split, label=f"policy S{split}")
    assert int(ds.n_tasks.item()) == tasks
    compare_step(res, oracle_step(wl, split_tokens=split), label=f"policy S{split}")


@pytest.mark.parametrize("budget", [True, False])
def test_one_call_step_beyond_64_sequences(budget):
    """More than 64 sequences: kvpage_decode_step builds the queue with its
    own kernel before the attention kernel (the fused build covers up to 64);
    100 x 32 rows also take the one-wavefront-per-row merge."""
    rng = np.random.default_rng(12)
    ctx = rng.integers(0, 700, 100)
    ctx[::9] = 0
    wl = W.custom(ctx.tolist(), Hq=32, Hkv=8, d=128, seed=51)
    wl.s_prev = rng.standard_normal(wl.s_prev.shape).astype(np.float32)
    ds, res = _run(wl, budget=budget, label="B100", one_call=True)
    tasks, offs, n = kvref.build_queue(wl.ctx_lens, wl.Hkv, wl.split_tokens)
    assert res["n_tasks"] == n and np.array_equal(res["tasks"], tasks)
    assert np.array_equal(res["group_offsets"], offs)
    compare_step(res, oracle_step(wl), budget=budget, label="B100")


@pytest.mark.parametrize("gain", [6.0, 24.0])
def test_peaky_queries_exercise_run_rescales(gain):
    """Queries scaled up (scores with standard deviation ~gain): the softmax
    is dominated by a few tokens, a run's reference max moves often between
    its tasks, and weights span many orders of magnitude.  Few workgroups so
    runs are long; both dtypes."""
    from paged_kv_cache_07_amd import binding
    from paged_kv_cache_07_amd.device import DecodeStep
    for dtype, d in (("f16", 128), ("bf16", 64)):
        wl = W.custom([3000, 517, 1024, 40], Hq=16, Hkv=4, d=d, dtype=dtype, seed=61)
        q = wl.q.astype(np.float32) if dtype == "f16" else \
            (wl.q.astype(np.uint32) << 16).view(np.float32)
        q = q * gain
        wl.q = q.astype(np.float16) if dtype == "f16" else W.f32_to_bf16_bits(q)
        for max_wg in (0, 2):
            say("peaky", gain, dtype, "max_wg", max_wg)
            ds = DecodeStep(wl, budget=True)
            ds.step(opts=binding.make_opts(max_workgroups=max_wg))
            compare_step(ds.results(), oracle_step(wl), label=f"peaky x{gain} {dtype} wg{max_wg}")


@pytest.mark.parametrize("path", ["one_call", "caller_queue"])
def test_bad_caller_data_stays_in_its_rows(path):
    """Page ids outside the pool (sequence 1), a length past the table row
    (sequence 2), a negative length (sequence 4) and, for a caller's queue,
    garbage entries in sequence 1's tasks: every kernel clamps what it reads
    into the shape, so sequences 0 and 3 still match the oracle on the clean
    data, and the summaries (which need no table) match everywhere."""
    from paged_kv_cache_07_amd.device import DecodeStep
    wl = W.custom([300, 200, 500, 77, 1000], Hq=8, Hkv=2, d=64, max_pages=70, seed=23)
    good = [0, 3]
    rows = [(b, h) for b in good for h in range(wl.Hq)]
    ref = oracle_step(wl, rows=rows)
    bt = wl.block_tables.copy()
    bt[1, 0:13:2] = wl.num_pages + 7
    bt[1, 1:13:2] = -5
    ctx = wl.ctx_lens.copy()
    ctx[2] = np.iinfo(np.int32).max
    ctx[4] = -50
    say("bad-data", path, "num_pages", wl.num_pages, "max_pages", wl.max_pages)
    ds = DecodeStep(wl)
    ds.block_tables.copy_(torch.from_numpy(bt))
    ds.ctx_lens.copy_(torch.from_numpy(ctx))
    if path == "one_call":
        ds.step()
    else:
        ds.build_queue()
        n = int(ds.n_tasks.item())
        tasks = ds.tasks[:n].cpu().numpy().copy()
        bad = np.flatnonzero(tasks[:, 0] == 1)
        assert bad.size
        tasks[bad[0::3]] = [99, -4, -100, 10**9]
        tasks[bad[1::3]] = [-3, 7, 5000, 4000]
        tasks[bad[2::3]] = [1, 1, 40, 2**31 - 1]
        ds.tasks[:n].copy_(torch.from_numpy(tasks))
        ds.decode_attn()
        ds.page_mass_finish()
        ds.gather_offsets()
    torch.cuda.synchronize()
    res = ds.results()
    for b in good:
        assert_close("out", res["out"][b], ref["out"][b])
        assert_close("lse", res["lse"][b], ref["lse"][b])
        assert_close("mass", res["mass"][b], ref["mass"][b])
        assert_close("page_max", res["page_max"][:, b], ref["page_max"][:, b])
    assert_close("s_next", res["s_next"], ref["s_next"])


@pytest.mark.parametrize("case", ["tiny", "edge", "b8_bimodal_small", "b64_prefix_small"])
@pytest.mark.parametrize("one_call", [True, False])
def test_stream_kv_changes_no_bits(case, one_call):
    """KVPAGE_FLAG_STREAM_KV only marks the tile loads non-temporal: every
    output is bit-identical to the cached loads (and matches the oracle)."""
    if case == "tiny":
        wl = W.make("tiny")
    elif case == "edge":
        wl = W.custom([0, 1, 15, 16, 17, 255, 256, 257, 1000], Hq=8, Hkv=2, d=64, dtype="bf16", seed=31)
    elif case == "b8_bimodal_small":
        wl = W.make("b8_bimodal", ctx_divisor=32)
    else:
        wl = W.make("b64_prefix", ctx_divisor=16)
    outs = []
    for stream_kv in (False, True):
        _, res = _run(wl, label=f"{case}-stream{int(stream_kv)}", one_call=one_call, stream_kv=stream_kv)
        outs.append(res)
    a, b = outs
    for key in ("tasks", "group_offsets", "out_bits", "lse", "mass", "page_max", "s_next"):
        assert np.array_equal(a[key], b[key]), key
    compare_step(b, oracle_step(wl), label=case)


@pytest.mark.parametrize("case,split", [("b64_prefix_small", 256), ("b64_prefix_small", 1024),
                                        ("edge", 256), ("edge", 512), ("edge", 64),
                                        ("many", 256)])
def test_shared_prefix_loads_change_no_bits(case, split):
    """KVPAGE_FLAG_STREAM_KV with kvpage_launch_opts.shared_pages: pieces of
    work that start on one of a sequence's shared leading pages load through
    the caches, the rest stream.  Every output is bit-identical to all loads
    cached (same schedule), and matches the oracle.  The edge case gives
    every sequence its own count: none, one page, mid-split, mid-piece, past
    the end of the context, and the whole table row; "many" has 70 sequences,
    past the fused queue build (separate queue kernel, linear schedule)."""
    from paged_kv_cache_07_amd.device import DecodeStep
    if case == "many":
        rng = np.random.default_rng(34)
        ctx = rng.integers(0, 3000, size=70).tolist()
        wl = W.custom(ctx, Hq=16, Hkv=8, d=64, dtype="f16", seed=34, max_pages=200)
        shared = rng.integers(0, 200, size=70).astype(np.int32)
    elif case == "edge":
        ctx = [0, 1, 300, 17, 4100, 2048, 9000, 513, 6000, 700, 4096, 15000]
        wl = W.custom(ctx, Hq=16, Hkv=8, d=128, dtype="bf16", seed=33, max_pages=1000)
        shared = np.array([0, 1, 0, 2, 40, 128, 100, 3, 5, 1000, 256, 937], dtype=np.int32)
    else:
        wl = W.make("b64_prefix", ctx_divisor=16)
        shared = W.shared_leading_pages(wl)
    wl.s_prev = np.random.default_rng(15).standard_normal(wl.s_prev.shape).astype(np.float32)
    say("shared-prefix loads", case, "split", split)
    a = DecodeStep(wl, split_tokens=split)
    a.step()
    ra = a.results()
    b = DecodeStep(wl, split_tokens=split, stream_kv=True, shared_pages=shared)
    b.step()
    rb = b.results()
    assert a.schedule_classes() == b.schedule_classes()
    for key in ("tasks", "group_offsets", "out_bits", "lse", "mass", "page_max", "s_next"):
        assert np.array_equal(ra[key], rb[key]), key
    compare_step(rb, oracle_step(wl, split_tokens=split), label=f"{case} S{split}")


@pytest.mark.parametrize("Hq,Hkv,d,dtype,ctx,extra_pages,split", [
    (64, 8, 128, "bf16", 5000, 0, 256),   # G = 8, bf16
    (8, 2, 64, "f16", 3000, 2, 128),      # d = 64, table wider by less than a split
    (8, 8, 64, "bf16", 700, 0, 64),       # G = 1, 4-page instance
    (16, 2, 128, "f16", 2000, 20, 32),    # table wider by more than a split
])
def test_one_sequence_across_instances(Hq, Hkv, d, dtype, ctx, extra_pages, split):
    """One sequence in the one-call step for other head groupings, head
    sizes, dtypes and split lengths: bit for bit against the separate calls
    and within tolerance of the oracle, with and without budgeting and
    streaming."""
    from paged_kv_cache_07_amd.device import DecodeStep
    max_pages = -(-ctx // 16) + extra_pages
    wl = W.custom([ctx], Hq=Hq, Hkv=Hkv, d=d, dtype=dtype, seed=60 + ctx % 89, max_pages=max_pages)
    wl.s_prev = np.random.default_rng(10).standard_normal(wl.s_prev.shape).astype(np.float32)
    ref = oracle_step(wl, split_tokens=split)
    for budget, stream_kv in ((True, True), (False, True), (True, False)):
        say("one-seq-inst", Hq, Hkv, d, dtype, ctx, "table", max_pages, "split", split,
            "budget", budget, "stream", stream_kv)
        a = DecodeStep(wl, budget=budget, split_tokens=split, stream_kv=stream_kv)
        a.run()
        ra = a.results()
        b = DecodeStep(wl, budget=budget, split_tokens=split, stream_kv=stream_kv)
        b.step()
        rb = b.results()
        keys = ["out_bits", "lse", "tasks", "group_offsets"] + (
            ["mass", "page_max", "s_next"] if budget else [])
        for key in keys:
            assert np.array_equal(ra[key], rb[key]), key
        compare_step(rb, ref, budget=budget, label=f"{Hq}/{Hkv} d{d} {dtype} ctx{ctx} S{split}")
