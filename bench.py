"""Benchmark one paged GQA decode step on one MI355X.

A step is the whole hot path on one batch, one kvpage_decode_step call:
build the task queue, split attention (with the page-mass and query-summary
budgeting outputs), then the log-sum-exp merge fused with the page-mass /
summary finish -- three kernels on one stream.  Inputs are seeded synthetic tensors already resident in HBM.  Before
every timed step the caches are flushed by reading a 1 GiB buffer (outside
the step's events), so KV bytes come from HBM.

The headline workload is the B1 long-context step (B=1, context 32768,
Hq=32, Hkv=8, d=128, page 16, fp16, 2048 pages in a 4096-page pool, 256-token
splits); B8 workloads are reported beside it.

Prints ONE JSON line.  ``value`` is KV bytes read per second over the whole
step; ``roofline`` rates the split-attention kernel alone (timed with HIP
events on the stream it runs on) against MI355X's 8 TB/s HBM peak.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "split_attn_traffic.txt")
ATTN_SRC = os.path.join(ROOT, "paged_kv_cache_07_amd", "csrc", "attn.hip")


def kernel_source_hash() -> str:
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(config: str):
    """HBM bytes per split-attention launch from rocprofv3 counters (FETCH_SIZE
    + WRITE_SIZE, scaled by a plain copy), if they were taken on the current
    kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [l.split() for l in f if l.strip() and not l.startswith("#")]
    except OSError:
        return None
    for parts in lines:
        if parts[0] != config:
            continue
        kv = dict(x.split("=", 1) for x in parts[1:])
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return float(kv["bytes_per_launch"])
    return None


def workload_title(name, r) -> str:
    if name == "b1":
        return "B1 long-context paged GQA decode step"
    return f"{name} paged GQA decode step ({r['B']} sequences, {r['ctx_total']} tokens)"


def kernel_title(r) -> str:
    loads = ("streaming loads, shared prefix cached" if r["shared_prefix_cached"]
             else "streaming loads" if r["stream_kv"] else "cached loads")
    queue = "fused queue" if r["B"] <= 64 else "queue kernel"
    return f"kvpage::split_attn_kernel<{r['d']}, {r['dtype']}, budget, {queue}, {loads}>"


_SPIN_CYCLES_PER_MS = None


def hold_stream(ms: float):
    """Keep the launch stream busy for about `ms` milliseconds (a device-side
    spin) while the host enqueues a timed loop behind it.  The per-step
    events then see the device's time only: a host slower to launch than the
    device is to run never shows up as gaps between the timed steps.  The
    spin's clock rate is calibrated once with events."""
    import torch

    from paged_kv_cache_07_amd import binding

    global _SPIN_CYCLES_PER_MS
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is None:   # no device spin in this torch: the loop runs unheld
        return
    if _SPIN_CYCLES_PER_MS is None:
        spin(1000)     # first launch (code load) outside the calibration
        a, b = binding.HipEvent(), binding.HipEvent()
        torch.cuda.synchronize()
        a.record()
        spin(2_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN_CYCLES_PER_MS = 2_000_000 / max(a.elapsed_ms(b), 1e-3)
    spin(int(min(ms, 500.0) * _SPIN_CYCLES_PER_MS))


def host_ms_per_iter(fn, iters: int) -> float:
    """Host time to enqueue one iteration of `fn` (no synchronisation)."""
    t0 = time.perf_counter()
    for _ in range(iters):
        fn()
    return (time.perf_counter() - t0) * 1e3 / max(iters, 1)


def time_config(name: str, steps: int, warmup: int, flush: bool, budget: bool = True,
                stream_kv=None):
    """Time workload `name`: one kvpage_decode_step call per step.

    Two timed regions of `steps` steps each, both with the cache flush before
    every step (outside the timed events):
      * steps: HIP events (timing-only, no system fence) on the launch stream
        around each whole step -> step time;
      * roofline: the split-attention kernel's own dispatch records its start
        and end (hipExtLaunchKernelGGL events) -> that kernel's duration.
    They are separate because kernel-level timestamps add a few microseconds
    to a step.  stream_kv (KVPAGE_FLAG_STREAM_KV) defaults to on; where the
    tables share a prefix, its pages are named in kvpage_launch_opts
    .shared_pages and load through the caches while the rest streams.
    """
    import torch

    from paged_kv_cache_07_amd import binding, workloads as W
    from paged_kv_cache_07_amd.device import DecodeStep

    if isinstance(name, tuple) and name[0] == "custom":     # ("custom", contexts, split)
        _, ctx, split = name
        wl = W.custom(ctx, Hq=32, Hkv=8, d=128, seed=21)
        split_tokens = split
        name = f"{len(ctx)}x{ctx[0]}/S{split}"
    elif isinstance(name, tuple):                            # ("named", workload, split)
        _, base, split = name
        wl = W.make(base)
        split_tokens = split
        name = f"{base}/S{split}"
    else:
        wl = W.make(name)
        split_tokens = None
    if stream_kv is None:
        stream_kv = True
    shared = W.shared_leading_pages(wl) if (stream_kv and wl.shares_pages()) else None
    ds = DecodeStep(wl, budget=budget, split_tokens=split_tokens, stream_kv=stream_kv,
                    shared_pages=shared)
    kv = W.kv_bytes(wl)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")

    def flush_caches():
        if flush:
            torch.sum(flush_buf, dim=0, out=sink[0])

    def one():
        flush_caches()
        ds.step()

    host_ms = host_ms_per_iter(one, max(warmup, 1))
    torch.cuda.synchronize()

    # Region 1: whole steps, enqueued behind a spin that outlasts the host's
    # launches.
    ev = [(binding.HipEvent(), binding.HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    hold_stream(2.0 * steps * host_ms + 2.0)
    t0 = time.perf_counter()
    for a, b in ev:
        flush_caches()
        a.record()
        ds.step()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_ms(b) for a, b in ev])

    # Region 2: the split-attention kernel's own timestamps.
    kev = [(binding.HipEvent(), binding.HipEvent()) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in kev:
        flush_caches()
        ds.step(opts=binding.make_opts(a, b))
    torch.cuda.synchronize()
    attn_ms = np.array([a.elapsed_ms(b) for a, b in kev])

    n_tasks = int(ds.n_tasks.item())
    return {
        "workload": name, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "d": wl.d,
        "page_size": wl.page_size, "split_tokens": split_tokens or wl.split_tokens,
        "dtype": wl.dtype, "num_pages": wl.num_pages, "max_ctx": int(wl.ctx_lens.max()),
        "ctx_total": int(wl.ctx_lens.sum()), "n_tasks": n_tasks, "kv_bytes": kv,
        "kv_bytes_unique": W.kv_bytes(wl, unique=True), "stream_kv": stream_kv,
        "shared_prefix_cached": shared is not None,
        "step_ms_mean": float(step_ms.mean()), "step_ms_p50": float(np.median(step_ms)),
        "step_ms_p10": float(np.percentile(step_ms, 10)), "step_ms_p90": float(np.percentile(step_ms, 90)),
        "attn_ms_mean": float(attn_ms.mean()), "attn_ms_p50": float(np.median(attn_ms)),
        "wall_s": wall, "cold_cache": flush, "host_enqueue_ms_per_step": host_ms,
    }


def time_append(name: str, calls: int, flush: bool):
    """kvpage_append_kv on workload `name`: one token per sequence per call,
    pages taken from the pool's unreferenced pages; HIP events around each
    call, caches flushed before it.  The lengths grow by one per call (a
    sequence whose table row is full is left as it is and flagged in
    `status`, as the call defines)."""
    import torch

    from paged_kv_cache_07_amd import binding, workloads as W
    from paged_kv_cache_07_amd.device import DecodeStep, host_to_device

    wl = W.make(name)
    ds = DecodeStep(wl, budget=False)
    used = np.zeros(wl.num_pages, dtype=bool)
    used[wl.referenced_pages()] = True
    ds.set_free_list(np.flatnonzero(~used).astype(np.int32))
    rng = np.random.default_rng(7)
    rows = (wl.B, wl.Hkv, wl.d)
    x = rng.standard_normal(rows).astype(np.float32)
    k_new = host_to_device(W.f32_to_bf16_bits(x) if wl.dtype == "bf16" else x.astype(np.float16),
                           wl.dtype, ds.device)
    v_new = k_new.clone()
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    ev = [(binding.HipEvent(), binding.HipEvent()) for _ in range(calls + 3)]
    torch.cuda.synchronize()
    hold_stream(2.0 * len(ev) * 0.5 + 2.0)   # ~0.5 ms of host work per call at most
    for a, b in ev:       # the first three calls are warm-up
        if flush:
            torch.sum(flush_buf, dim=0, out=sink[0])
        a.record()
        binding.kvpage_append_kv(ds.shape, k_new, v_new, ds.k_pool, ds.v_pool, ds.block_tables,
                                 ds.ctx_lens, ds.ctx_next, ds.free_pages, ds.free_count,
                                 ds.free_count_next, ds.append_status)
        b.record()
        ds.ctx_lens, ds.ctx_next = ds.ctx_next, ds.ctx_lens
        ds.free_count, ds.free_count_next = ds.free_count_next, ds.free_count
    torch.cuda.synchronize()
    us = np.array([a.elapsed_ms(b) for a, b in ev[3:]]) * 1e3
    return {"calls": calls, "us_mean": float(us.mean()), "us_p50": float(np.median(us)),
            "bytes_written": wl.B * wl.Hkv * wl.d * 2 * 2,
            "status": int(ds.append_status.item()), "B": wl.B}


def time_decide(name: str, calls: int, flush: bool, tau: float = 0.9):
    """kvpage_budget_decide where it runs in a serving step: right after the
    budgeting decode step that wrote its page maxima (workload `name`, every
    length cut back to a page boundary so that every sequence gets a
    decision).  Per call: cache flush, the decode step, then HIP events
    around the decision alone (both kernels)."""
    import torch

    from paged_kv_cache_07_amd import binding, workloads as W
    from paged_kv_cache_07_amd.device import DecodeStep

    wl = W.make(name)
    ds = DecodeStep(wl, stream_kv=not wl.shares_pages())
    ds.step()
    dev = ds.device
    ctx = torch.from_numpy((wl.ctx_lens // 16 * 16).astype(np.int32)).to(dev)
    size = torch.empty((2, wl.B, wl.Hkv), dtype=torch.int32, device=dev)
    level = torch.empty((2, wl.B, wl.Hkv), dtype=torch.float32, device=dev)
    union = torch.empty((2, wl.B), dtype=torch.int32, device=dev)
    dec = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    vic = torch.empty((wl.B,), dtype=torch.int32, device=dev)
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    ev = [(binding.HipEvent(), binding.HipEvent()) for _ in range(calls + 3)]
    torch.cuda.synchronize()
    hold_stream(2.0 * len(ev) * 0.5 + 2.0)
    for a, b in ev:       # the first three calls are warm-up
        if flush:
            torch.sum(flush_buf, dim=0, out=sink[0])
        ds.step()
        a.record()
        binding.kvpage_budget_decide(ds.shape, ds.page_max, ctx, tau, size, level, union, dec, vic)
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_ms(b) for a, b in ev[3:]]) * 1e3
    d = dec.cpu().numpy()
    return {"calls": calls, "us_mean": float(us.mean()), "us_p50": float(np.median(us)),
            "tau": tau, "B": wl.B, "Hkv": wl.Hkv, "max_pages": wl.max_pages,
            "pages_read": int(2 * wl.Hkv * (wl.ctx_lens // 16).sum()),
            "acquire": int((d == 1).sum()), "compress": int((d == 2).sum())}


# The oracle baseline spreads whole (sequence, KV head) groups over worker
# processes; each worker builds the same seeded workload once and runs the
# oracle unchanged on the groups it is handed.
_ORACLE_WL = None


def _oracle_worker_init(name: str):
    global _ORACLE_WL
    from threadpoolctl import threadpool_limits

    from paged_kv_cache_07_amd import workloads as W
    threadpool_limits(limits=1)
    _ORACLE_WL = W.make(name)


def _oracle_groups(groups):
    """The oracle's step for the query heads of ``groups`` [(b, g), ...]:
    their attention rows, page mass and summary page maxima."""
    from oracle import kvref
    wl = _ORACLE_WL
    rows = [(b, g * wl.G + i) for b, g in groups for i in range(wl.G)]
    r = kvref.decode_step(wl, rows=rows)
    return [(b, g, r["out"][b, g * wl.G:(g + 1) * wl.G], r["lse"][b, g * wl.G:(g + 1) * wl.G],
             r["mass"][b, g * wl.G:(g + 1) * wl.G], r["page_max"][:, b, g]) for b, g in groups]


def cpu_baseline(seconds: float = 12.0):
    """The fp64 oracle on the host: full B1 steps repeated for ~``seconds``.

    Multi-core: the step's (sequence, KV head) groups are spread over worker
    processes (one BLAS thread each; as many processes as groups, at most the
    host's share of cores), the queue is built in the parent and every
    group's rows are gathered back into whole-step arrays.  Then the same
    steps in one process on one thread."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    from oracle import kvref
    from paged_kv_cache_07_amd import workloads as W

    name = "b1"
    wl = W.make(name)
    kv = W.kv_bytes(wl)
    groups = [(b, g) for b in range(wl.B) for g in range(wl.Hkv)]
    share = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count() or 1
    nproc = max(1, min(share, len(groups)))
    items = [groups[i::nproc] for i in range(nproc)]

    def whole_step(pool):
        kvref.build_queue(wl.ctx_lens, wl.Hkv, wl.split_tokens)
        out = np.empty((wl.B, wl.Hq, wl.d))
        lse = np.empty((wl.B, wl.Hq))
        mass = np.empty((wl.B, wl.Hq, wl.max_pages))
        pmax = np.empty((2, wl.B, wl.Hkv, wl.max_pages))
        for part in pool.map(_oracle_groups, items):
            for b, g, o, l, m, pm in part:
                out[b, g * wl.G:(g + 1) * wl.G] = o
                lse[b, g * wl.G:(g + 1) * wl.G] = l
                mass[b, g * wl.G:(g + 1) * wl.G] = m
                pmax[:, b, g] = pm
        kvref.update_summaries(wl.q, wl.s_prev, wl.Hkv, wl.alpha_fast, wl.alpha_slow, wl.dtype)
        return out

    with mp.get_context("spawn").Pool(nproc, initializer=_oracle_worker_init,
                                      initargs=(name,)) as pool:
        whole_step(pool)                       # warm-up: workers have built the inputs
        n = 0
        t0 = time.perf_counter()
        while True:
            whole_step(pool)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break

    n1 = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            kvref.decode_step(wl)
            n1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= seconds:
                break
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": kv * n / el / 1e9, "unit": "GB/s", "cores": nproc, "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"{n} full B1 steps (ctx 32768, Hq 32, Hkv 8, d 128: queue, attention, "
                      f"page mass, summaries, page max) in {el:.1f} s, numpy fp64, "
                      f"{nproc} worker processes x 1 BLAS thread, (sequence, KV head) groups "
                      f"spread over them",
            "steps_per_s": n / el,
            "single_thread": {"value": kv * n1 / el1 / 1e9, "unit": "GB/s", "cores": 1,
                              "steps_per_s": n1 / el1,
                              "sample": f"{n1} full B1 steps in {el1:.1f} s, one process, "
                                        f"one BLAS thread"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="b1")
    ap.add_argument("--also", default="b8_bimodal,b8_uniform,b8_zipf,b64_prefix,b4_bimodal",
                    help="comma-separated extra workloads reported beside the headline one")
    ap.add_argument("--warm", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the KV append (one token per sequence) on B8 and B64")
    ap.add_argument("--decide", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the compress-or-acquire decision on B1, B8 Zipf and B64")
    ap.add_argument("--policy", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the split policy on short batches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for counter calibration)")
    ap.add_argument("--floor", action="store_true",
                    help="only time a trivial kernel (a 4-byte fill) behind the same cache flush")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: this decode "
              "step is built and timed on a single MI355X (see the sharding design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from paged_kv_cache_07_amd import binding
    binding.lib()   # fail loudly if the HIP library is missing

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4}))
        return

    if args.floor:
        # What any kernel launched behind the 1 GiB flush costs when timed by
        # HIP events around it, as the step is timed (kernel-trace durations
        # of the same launches come from the profiler).
        flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.zeros(1, dtype=torch.float32, device="cuda")
        tiny = torch.zeros(1, dtype=torch.int32, device="cuda")
        ev = [(binding.HipEvent(), binding.HipEvent()) for _ in range(args.steps)]
        for a, b in ev:
            torch.sum(flush_buf, dim=0, out=sink[0])
            a.record()
            tiny.fill_(1)
            b.record()
        torch.cuda.synchronize()
        us = np.array([a.elapsed_ms(b) for a, b in ev]) * 1e3
        print(json.dumps({"floor_kernel": "4-byte fill behind the 1 GiB flush", "us_mean": float(us.mean()),
                          "us_p50": float(np.median(us)), "launches": args.steps}))
        return

    flush = not args.warm
    head = time_config(args.config, args.steps, args.warmup, flush)
    # The same steps back to back (no cache flush): KV partly served from MALL.
    warm = time_config(args.config, max(20, args.steps // 4), 5, False) if flush else head
    also = {}
    for name in [x for x in args.also.split(",") if x and x != args.config]:
        k = max(10, args.steps // 4)
        r = time_config(name, k, max(3, args.warmup // 4), flush)
        also[name] = {
            "kv_gbs_step": r["kv_bytes"] / r["step_ms_mean"] / 1e6,
            "kv_gbs_attn_kernel": r["kv_bytes"] / r["attn_ms_mean"] / 1e6,
            "frac_hbm_peak_attn": r["kv_bytes"] / r["attn_ms_mean"] / 1e6 / HBM_PEAK_GBS,
            # Distinct pages only (a page shared by several sequences counted once):
            # the bytes HBM has to deliver at least.
            "frac_hbm_peak_attn_unique": r["kv_bytes_unique"] / r["attn_ms_mean"] / 1e6 / HBM_PEAK_GBS,
            "steps_per_s": 1e3 / r["step_ms_mean"],
            "step_ms_mean": r["step_ms_mean"], "attn_ms_mean": r["attn_ms_mean"],
            "kv_bytes": r["kv_bytes"], "kv_bytes_unique": r["kv_bytes_unique"],
            "n_tasks": r["n_tasks"], "B": r["B"], "Hq": r["Hq"], "Hkv": r["Hkv"],
            "dtype": r["dtype"], "stream_kv": r["stream_kv"],
            "shared_prefix_cached": r["shared_prefix_cached"], "steps": k,
        }

    # The split policy (kvpage_choose_split) beside the fixed 256-token split,
    # both in the same load mode: three short batches, where the fixed split
    # leaves wavefronts idle, with cached tile loads (streaming loads slow
    # such a step by ~6%, which would flatter the policy); and the B8
    # bimodal, B8 Zipf and B4 bimodal lengths with streaming loads, where the
    # policy takes longer splits (fewer, longer tasks).
    policy = {}
    if args.policy:
        from paged_kv_cache_07_amd import binding as K
        from paged_kv_cache_07_amd import workloads as W
        cases = [(("custom", ctx), f"{len(ctx)}x{ctx[0]}", False)
                 for ctx in ([8192], [4096] * 4, [16384])]
        cases += [(("named", n), n, True) for n in ("b8_bimodal", "b8_zipf", "b4_bimodal")]
        for spec, label, stream_kv in cases:
            if spec[0] == "custom":
                wl = W.custom(spec[1], Hq=32, Hkv=8, d=128, seed=21, fill_pools=False)
            else:
                wl = W.make(spec[1], fill_pools=False)
            shape = K.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.page_size, 256, wl.max_pages,
                                 wl.num_pages, wl.dtype, wl.scale,
                                 K.KVPAGE_FLAG_STREAM_KV if stream_kv else 0)
            split = K.kvpage_choose_split(shape, wl.ctx_lens.tolist())
            k = max(10, args.steps // 4)
            fixed = time_config((*spec, 256), k, 3, flush, stream_kv=stream_kv)
            chosen = time_config((*spec, split), k, 3, flush, stream_kv=stream_kv)
            policy[label] = {
                "split_chosen": split, "stream_kv": stream_kv,
                "step_ms_split256": fixed["step_ms_mean"], "step_ms_chosen": chosen["step_ms_mean"],
                "attn_ms_split256": fixed["attn_ms_mean"], "attn_ms_chosen": chosen["attn_ms_mean"],
                "speedup": fixed["step_ms_mean"] / chosen["step_ms_mean"],
                "kv_gbs_step_chosen": chosen["kv_bytes"] / chosen["step_ms_mean"] / 1e6}

    append = {}
    if args.append:
        for name in ("b8_bimodal", "b64_prefix"):
            append[name] = time_append(name, 40, flush)
    decide = {}
    if args.decide:
        for name in ("b1", "b8_zipf", "b64_prefix"):
            decide[name] = time_decide(name, 40, flush)

    kv = head["kv_bytes"]
    achieved = kv / head["attn_ms_mean"] / 1e6
    traffic = measured_traffic(args.config)
    result = {
        "metric": "KV GB/s read per decode step (% of HBM peak); decode steps/s at B1 & B8",
        "value": kv / head["step_ms_mean"] / 1e6,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms_mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": f"synthetic: seeded N(0,1) {head['dtype']} q/K/V, pages scattered by a seeded permutation",
        "config": {"workload": workload_title(args.config, head), "B": head["B"],
                   "context": head["max_ctx"] if head["B"] == 1 else None,
                   "tokens": head["ctx_total"], "Hq": head["Hq"], "Hkv": head["Hkv"],
                   "d": head["d"], "page_size": head["page_size"],
                   "split_tokens": head["split_tokens"], "pool_pages": head["num_pages"],
                   "budgeting_outputs": True, "cold_cache": flush,
                   "stream_kv": head["stream_kv"],
                   "shared_prefix_cached": head["shared_prefix_cached"]},
        "steps_per_s": 1e3 / head["step_ms_mean"],
        "frac_hbm_peak_step": kv / head["step_ms_mean"] / 1e6 / HBM_PEAK_GBS,
        "step_ms_p50": head["step_ms_p50"], "step_ms_p10": head["step_ms_p10"],
        "step_ms_p90": head["step_ms_p90"], "n_tasks": head["n_tasks"], "kv_bytes": kv,
        "host_enqueue_ms_per_step": head["host_enqueue_ms_per_step"],
        "warm_step_ms_mean": warm["step_ms_mean"], "warm_steps_per_s": 1e3 / warm["step_ms_mean"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel_title(head),
                     "attn_ms_mean": head["attn_ms_mean"],
                     "algorithmic_bytes_per_launch": kv},
        "also": also,
    }
    if policy:
        result["split_policy"] = policy
    if append:
        result["kv_append"] = append
    if decide:
        result["budget_decide"] = decide
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
