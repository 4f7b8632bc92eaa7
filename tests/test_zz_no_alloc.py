"""kvpage_decode_step_noalloc (static device workspace) against
kvpage_decode_step (caller's workspace) through the C ABI: the same kernels,
so the outputs must agree bit for bit; two calls in a row, the second with a
smaller input, so the shared static workspace holds the first call's
partials when the second runs.  Plus the refusal of a workspace past the
static size."""

import numpy as np
import pytest

from gpu_util import compare_step, oracle_step, say
from paged_kv_cache_07_amd import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

KEYS = ("tasks", "group_offsets", "out_bits", "lse", "mass", "page_max", "s_next")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_cache_07_amd import binding
    binding.lib()


def _both(wl, stream_kv):
    from paged_kv_cache_07_amd import binding as K
    from paged_kv_cache_07_amd.device import DecodeStep
    a = DecodeStep(wl, stream_kv=stream_kv)
    a.step()
    ra = a.results()
    b = DecodeStep(wl, stream_kv=stream_kv)
    assert K.kvpage_workspace_bytes(b.shape, b.capacity) <= K.KVPAGE_NOALLOC_WORKSPACE_BYTES
    K.kvpage_decode_step_noalloc(b.shape, b.q, b.k_pool, b.v_pool, b.block_tables, b.ctx_lens,
                                 b.tasks, b.group_offsets, b.n_tasks, b.capacity, b.budget,
                                 b.out, b.lse)
    return ra, b.results()


def test_noalloc_matches_caller_workspace_two_calls():
    first = W.make("b8_bimodal")                        # full size: ~34 MB of workspace
    second = W.custom([3000, 0, 17, 700], Hq=16, Hkv=4, d=64, dtype="bf16", seed=81)
    second.s_prev = np.random.default_rng(3).standard_normal(second.s_prev.shape).astype(np.float32)
    for i, (wl, stream_kv) in enumerate(((first, True), (second, False))):
        say("noalloc call", i, wl.name, "B", wl.B, "max_pages", wl.max_pages)
        ra, rb = _both(wl, stream_kv)
        assert ra["n_tasks"] == rb["n_tasks"]
        for key in KEYS:
            assert np.array_equal(ra[key], rb[key]), (wl.name, key)
        if i == 1:
            compare_step(rb, oracle_step(wl), label="noalloc, second call")


def test_noalloc_refuses_a_workspace_past_the_static_size():
    from paged_kv_cache_07_amd import binding as K
    # 64 sequences x 8 KV heads x 64 splits x G 8 x 130 floats: 136 MB.
    shape = K.make_shape(64, 64, 8, 128, 16, 256, 1024, 100000, "bf16", 128 ** -0.5, 0)
    cap = K.kvpage_queue_capacity(shape)
    assert K.kvpage_workspace_bytes(shape, cap) > K.KVPAGE_NOALLOC_WORKSPACE_BYTES
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    say("noalloc refusal")
    with pytest.raises(K.KvpageError) as e:
        K.kvpage_decode_step_noalloc(shape, dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                     dummy, cap, None, dummy, dummy)
    assert e.value.status == K.KVPAGE_ERR_SCRATCH
