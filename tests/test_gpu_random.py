"""Seeded random configurations through the C ABI against the fp64 oracle.

Each case draws its own shape (batch size on both sides of the 64-sequence
limit of the fused queue, KV heads, group size, head dim, dtype, split
length, table width, shared prefix pages), context lengths (empty, short,
page-aligned and ragged mixed), the call path (one call or separate calls),
budgeting on or off and, for tables without shared pages, the streaming tile
loads.  Every output is compared: queue bit for bit, floating point within
the tolerances in gpu_util.
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


def _draw(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 3, 7, 33, 64, 65, 90]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 9))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f16", "bf16"]))
    split = int(rng.choice([16, 32, 64, 128, 256]))
    kind = rng.integers(0, 4, size=B)
    ctx = np.where(kind == 0, 0,
          np.where(kind == 1, rng.integers(1, 40, size=B),
          np.where(kind == 2, 16 * rng.integers(1, 40, size=B), rng.integers(1, 1500, size=B))))
    shared = 0
    if rng.integers(0, 4) == 0:          # a shared prefix of 3 pages in every sequence
        shared = 3
        ctx = np.maximum(ctx, 3 * 16 + rng.integers(1, 200, size=B))
    extra = int(rng.integers(0, 5))
    need = max(1, -(-int(ctx.max()) // 16))
    wl = W.custom(ctx.tolist(), Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, split_tokens=split,
                  seed=seed, max_pages=need + extra, shared_prefix_pages=shared)
    one_call = bool(rng.integers(0, 2))
    budget = bool(rng.integers(0, 2))
    stream_kv = bool(rng.integers(0, 2)) and not wl.shares_pages()
    return wl, one_call, budget, stream_kv


# 5039, 5075 and 5148: bfloat16 with 16-token splits, where a weight rounded
# once to bfloat16 had put 1-3 outputs past the tolerance.
@pytest.mark.parametrize("seed", list(range(4000, 4024)) + [5039, 5075, 5148])
def test_random_config_matches_oracle(seed):
    from paged_kv_cache_07_amd.device import DecodeStep
    wl, one_call, budget, stream_kv = _draw(seed)
    say("random", seed, "B", wl.B, "Hkv", wl.Hkv, "G", wl.G, "d", wl.d, wl.dtype,
        "split", wl.split_tokens, "max_pages", wl.max_pages, "one_call", one_call,
        "budget", budget, "stream_kv", stream_kv, "ctx", wl.ctx_lens.tolist()[:6])
    ds = DecodeStep(wl, budget=budget, stream_kv=stream_kv)
    if one_call:
        ds.step()
    else:
        ds.run()
    compare_step(ds.results(), oracle_step(wl), budget=budget, label=f"seed {seed}")
