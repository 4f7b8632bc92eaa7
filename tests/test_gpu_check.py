"""kvpage_check_inputs (debug checks of the integer preconditions) against
the oracle's check_inputs, bit for bit, on clean inputs and on each kind of
violation planted in the device buffers."""
import numpy as np
import pytest

from gpu_util import say
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


def _workload(case):
    if case == "tiny":
        return W.make("tiny")
    if case == "edge":
        return W.custom([0, 1, 15, 16, 17, 255, 256, 257, 1000], Hq=8, Hkv=2, d=64, seed=51,
                        max_pages=70)
    if case == "b8_bimodal_small":
        return W.make("b8_bimodal", ctx_divisor=32)
    return W.make("b64_prefix", ctx_divisor=16)


def _both(ds, wl, with_queue):
    """Library status and oracle status for the device buffers as they are."""
    from paged_kv_cache_07_amd import binding as K
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    if with_queue:
        K.kvpage_check_inputs(ds.shape, ds.ctx_lens, ds.block_tables, ds.tasks, ds.group_offsets,
                              ds.n_tasks, ds.capacity, status)
    else:
        K.kvpage_check_inputs(ds.shape, ds.ctx_lens, ds.block_tables, None, None, None, 0, status)
    torch.cuda.synchronize()
    got = int(status.item())
    ctx = ds.ctx_lens.cpu().numpy()
    bt = ds.block_tables.cpu().numpy()
    if with_queue:
        want = kvref.check_inputs(ctx, bt, wl.num_pages, wl.page_size, wl.Hkv, ds.split_tokens,
                                  capacity=ds.capacity, tasks=ds.tasks.cpu().numpy(),
                                  group_offsets=ds.group_offsets.cpu().numpy(),
                                  n_tasks=ds.n_tasks.cpu().numpy())
    else:
        want = kvref.check_inputs(ctx, bt, wl.num_pages, wl.page_size, wl.Hkv, ds.split_tokens)
    return got, want


@pytest.mark.parametrize("case", ["tiny", "edge", "b8_bimodal_small", "b64_prefix_small"])
def test_check_inputs_matches_oracle(case):
    from paged_kv_cache_07_amd.device import DecodeStep
    wl = _workload(case)
    ds = DecodeStep(wl)
    ds.build_queue()
    torch.cuda.synchronize()
    say("check", case, "clean")
    for with_queue in (False, True):
        got, want = _both(ds, wl, with_queue)
        assert got == want == 0, (case, with_queue, got, want)

    ctx0 = ds.ctx_lens.clone()
    bt0 = ds.block_tables.clone()
    tasks0 = ds.tasks.clone()
    go0 = ds.group_offsets.clone()
    n0 = ds.n_tasks.clone()
    n = int(n0.item())
    B, max_pages = wl.B, wl.max_pages
    b_long = int(np.argmax(wl.ctx_lens))
    used = int(-(-int(wl.ctx_lens[b_long]) // wl.page_size))

    def restore():
        ds.ctx_lens.copy_(ctx0)
        ds.block_tables.copy_(bt0)
        ds.tasks.copy_(tasks0)
        ds.group_offsets.copy_(go0)
        ds.n_tasks.copy_(n0)

    plants = {
        "negative length": lambda: ds.ctx_lens.__setitem__(0, -3),
        "length past the row": lambda: ds.ctx_lens.__setitem__(B - 1, max_pages * wl.page_size + 1),
        "used page = num_pages": lambda: ds.block_tables.__setitem__((b_long, used - 1), wl.num_pages),
        "used page negative": lambda: ds.block_tables.__setitem__((b_long, 0), -7),
        "task end off by one": lambda: ds.tasks.__setitem__((n // 2, 3), int(tasks0[n // 2, 3]) - 1),
        "task head changed": lambda: ds.tasks.__setitem__((n - 1, 1), int(tasks0[n - 1, 1]) + 1),
        "n_tasks one less": lambda: ds.n_tasks.__setitem__(0, n - 1),
        "group offset moved": lambda: ds.group_offsets.__setitem__(1, int(go0[1]) + 1),
        "junk past n_tasks": lambda: ds.tasks[n:].fill_(-5),
    }
    if used < max_pages:
        plants["junk in an unused cell"] = lambda: ds.block_tables.__setitem__((b_long, used), -1)
    for name, plant in plants.items():
        restore()
        plant()
        torch.cuda.synchronize()
        say("check", case, name)
        for with_queue in (False, True):
            got, want = _both(ds, wl, with_queue)
            assert got == want, (case, name, with_queue, got, want)
        if name.startswith("junk"):
            assert want == 0, name
        else:
            assert want != 0, name
    restore()


def test_check_inputs_empty_batch_writes_zero():
    from paged_kv_cache_07_amd import binding as K
    shape = K.make_shape(0, 8, 2, 64, 16, 256, 4, 10, "f16", 0.125)
    ctx = torch.zeros(1, dtype=torch.int32, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    status = torch.full((1,), 123, dtype=torch.int32, device="cuda")
    K.kvpage_check_inputs(shape, ctx, bt, None, None, None, 0, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
