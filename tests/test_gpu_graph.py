"""The one-call decode step captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed: every replay must reproduce the eager step bit for bit.

The library enqueues kernels only (no memset, copy or allocation), so the
whole step -- queue, split attention, merge and finish -- can be captured.
Between replays the outputs are overwritten and the query changed by eager
work, so each replay has to recompute everything from its inputs.
"""

import numpy as np
import pytest

from gpu_util import compare_step, oracle_step, say
from paged_kv_cache_07_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_07_amd import binding
    binding.lib()


def _scribble(ds):
    """Eager work between replays: overwrite every output."""
    for t in (ds.out, ds.lse, ds.tasks, ds.group_offsets, ds.n_tasks):
        t.fill_(7)
    if ds.use_budget:
        for t in (ds.page_mass, ds.page_max, ds.s_next):
            t.fill_(7)


KEYS = ("n_tasks", "tasks", "group_offsets", "out_bits", "lse", "mass", "page_max", "s_next")


@pytest.mark.parametrize("case", ["b8_bimodal_small", "b64_prefix_small", "b100"])
def test_graph_replays_match_eager(case):
    from paged_kv_cache_07_amd.device import DecodeStep
    if case == "b8_bimodal_small":
        wl = W.make("b8_bimodal", ctx_divisor=32)
    elif case == "b64_prefix_small":
        wl = W.make("b64_prefix", ctx_divisor=16)
    else:   # more than 64 sequences: separate queue kernel, wavefront merge
        ctx = np.random.default_rng(5).integers(0, 700, size=100).tolist()
        wl = W.custom(ctx, Hq=32, Hkv=8, d=128, seed=55)
    say("graph", case, "B", wl.B)
    ds = DecodeStep(wl, budget=True, stream_kv=not wl.shares_pages())
    queries = [wl.q, W.draw_queries(wl), W.draw_queries(wl)]

    # Eager reference for each query.
    eager = []
    for q in queries:
        ds.set_query(q)
        ds.step()
        eager.append(ds.results())

    # Capture (after the eager calls, so the library's one-time device
    # queries are done), then replay with eager work in between.
    ds.set_query(queries[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ds.step()
    torch.cuda.synchronize()
    for rep in range(6):
        k = rep % len(queries)
        say("graph replay", case, rep)
        _scribble(ds)
        ds.set_query(queries[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = ds.results()
        for key in KEYS:
            assert np.array_equal(np.asarray(got[key]), np.asarray(eager[k][key])), (case, rep, key)
    # And the replayed result is the step the oracle defines.
    compare_step(got, oracle_step(wl, q=queries[(6 - 1) % len(queries)]), label=case)
