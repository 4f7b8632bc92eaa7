"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a device.  No GPU needed: each call
here fails validation (or is pure host arithmetic) before any HIP call."""

import ctypes
import os
import re

import pytest

from paged_kv_cache_07_amd import binding as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvpage.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvpage_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert {"kvpage_build_queue", "kvpage_decode_attn", "kvpage_page_mass"} <= set(names)
    lib = ctypes.CDLL(K.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(K._SIGS), "binding signatures out of step with the header"


def _shape(**kw):
    base = dict(B=2, Hq=32, Hkv=8, d=128, page_size=16, split_tokens=256, max_pages=2048,
                num_pages=4096, dtype="f16", scale=128 ** -0.5)
    base.update(kw)
    return K.make_shape(**base)


def test_capacity_and_workspace_arithmetic():
    s = _shape(B=1)
    assert K.kvpage_queue_capacity(s) == 1 * 8 * (2048 * 16 // 256)
    s = _shape(B=3, max_pages=7, split_tokens=32)
    assert K.kvpage_queue_capacity(s) == 3 * 8 * 4          # ceil(112 / 32) = 4
    cap = K.kvpage_queue_capacity(s)
    assert K.kvpage_workspace_bytes(s, cap) == (64 + cap * 4 * (128 + 2)) * 4


def test_stream_flag_is_accepted():
    """KVPAGE_FLAG_STREAM_KV changes no size: same capacity and workspace."""
    s, plain = _shape(flags=K.KVPAGE_FLAG_STREAM_KV), _shape()
    cap = K.kvpage_queue_capacity(s)
    assert cap == K.kvpage_queue_capacity(plain) > 0
    assert K.kvpage_workspace_bytes(s, cap) == K.kvpage_workspace_bytes(plain, cap) > 0


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=30), K.KVPAGE_ERR_INVALID_ARG),          # Hq % Hkv != 0
    (dict(split_tokens=40), K.KVPAGE_ERR_INVALID_ARG),  # split not a page multiple
    (dict(scale=0.0), K.KVPAGE_ERR_INVALID_ARG),
    (dict(scale=float("inf")), K.KVPAGE_ERR_INVALID_ARG),
    (dict(dtype=7), K.KVPAGE_ERR_INVALID_ARG),
    (dict(max_pages=0), K.KVPAGE_ERR_INVALID_ARG),
    (dict(B=-1), K.KVPAGE_ERR_INVALID_ARG),
    (dict(max_pages=(1 << 27)), K.KVPAGE_ERR_INVALID_ARG),  # tokens overflow int32
    (dict(flags=2), K.KVPAGE_ERR_INVALID_ARG),          # only KVPAGE_FLAG_STREAM_KV is defined
    (dict(flags=K.KVPAGE_FLAG_STREAM_KV | 4), K.KVPAGE_ERR_INVALID_ARG),
])
def test_invalid_shapes_are_rejected(kw, status):
    s = _shape(**kw)
    assert K.lib().kvpage_queue_capacity(ctypes.byref(s)) == status
    rc = K.lib().kvpage_build_queue(ctypes.byref(s), ctypes.c_void_p(16), ctypes.c_void_p(16),
                                    1 << 20, ctypes.c_void_p(16), ctypes.c_void_p(16), None)
    assert rc == status


@pytest.mark.parametrize("kw", [dict(d=96), dict(page_size=8, split_tokens=256),
                                dict(Hq=80, Hkv=8),
                                # past 16 pages only whole multiples of 16 pages, up to 256
                                dict(split_tokens=272), dict(split_tokens=768 + 16),
                                dict(split_tokens=8192)])
def test_unsupported_shapes_report_unsupported(kw):
    s = _shape(**kw)
    cap = K.kvpage_queue_capacity(s)
    dummy = ctypes.c_void_p(256)
    rc = K.lib().kvpage_split_attn(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, dummy,
                                   dummy, cap, dummy, None, None)
    assert rc == K.KVPAGE_ERR_UNSUPPORTED
    assert K.lib().kvpage_workspace_bytes(ctypes.byref(s), cap) == K.KVPAGE_ERR_UNSUPPORTED


def test_capacity_too_small_and_null_pointers():
    s = _shape()
    cap = K.kvpage_queue_capacity(s)
    dummy = ctypes.c_void_p(256)
    lib = K.lib()
    assert lib.kvpage_build_queue(ctypes.byref(s), dummy, dummy, cap - 1, dummy, dummy, None) \
        == K.KVPAGE_ERR_CAPACITY
    assert lib.kvpage_build_queue(ctypes.byref(s), None, dummy, cap, dummy, dummy, None) \
        == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_decode_attn(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                  dummy, cap, dummy, None, None, dummy, None) == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_page_mass(ctypes.byref(s), None, dummy, dummy, dummy, dummy, cap, dummy, None) \
        == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_merge_splits(ctypes.byref(s), dummy, cap, dummy, None, dummy, None) \
        == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_debug_gather_offsets(ctypes.byref(s), dummy, dummy, dummy, cap, None, None) \
        == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_queue_capacity(None) == K.KVPAGE_ERR_INVALID_ARG


def test_budget_validation():
    s = _shape()
    cap = K.kvpage_queue_capacity(s)
    dummy = ctypes.c_void_p(256)
    lib = K.lib()
    same = K.kvpage_budget(dummy, dummy, dummy, 0.5, 0.05, dummy)            # s_prev aliases s_next
    bad_alpha = K.kvpage_budget(dummy, dummy, ctypes.c_void_p(512), 1.5, 0.05, dummy)
    missing = K.kvpage_budget(None, dummy, ctypes.c_void_p(512), 0.5, 0.05, dummy)
    for bud in (same, bad_alpha, missing):
        rc = lib.kvpage_split_attn(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                   cap, dummy, ctypes.byref(bud), None)
        assert rc == K.KVPAGE_ERR_INVALID_ARG
        rc = lib.kvpage_page_mass(ctypes.byref(s), ctypes.byref(bud), dummy, dummy, dummy, dummy,
                                  cap, dummy, None)
        assert rc == K.KVPAGE_ERR_INVALID_ARG


def test_status_strings():
    for code in (0, -1, -2, -3, -4, 99):
        assert isinstance(K.status_string(code), str) and K.status_string(code)


def test_choose_split_fills_the_resident_wavefronts():
    """Among the splits whose queue has a task per resident wavefront
    (Hkv * sum ceil(ctx / S) >= W), the least simulated time: each
    wavefront's pages plus a fixed cost per queue position under the
    kernel's schedule, finished by water filling (every unfinished
    wavefront streams at min(1.43, W / unfinished) pages per unit); the page
    size if none qualifies, 256 for an all-empty batch.  Pure host
    arithmetic with W given."""
    def pick(ctx, W=1024, **kw):
        return K.kvpage_choose_split(_shape(B=len(ctx), **kw), ctx, W)
    assert pick([32768]) == 256          # 8 * 128 tasks = 1024
    assert pick([32767]) == 256          # still 128 splits of 256 per KV head
    assert pick([32512]) == 128          # 8 * 127 = 1016 at 256; 8 * 254 at 128
    assert pick([16384]) == 128          # 8 * 64 = 512 at 256, 8 * 128 = 1024 at 128
    assert pick([8192]) == 64
    assert pick([4096]) == 32
    assert pick([100]) == 16             # even 16-token splits leave wavefronts idle
    assert pick([4096] * 4) == 128
    assert pick([0, 0]) == 256
    assert pick([1000], W=1) == 256
    assert pick([16384], W=2048) == 64
    assert pick([16384], Hq=16, Hkv=4) == 64   # half the KV heads, half the tasks
    for S in (16, 32, 64, 128, 256):
        assert pick([8192] * 3, W=3 * 8 * 8192 // S) >= S
    stream = K.KVPAGE_FLAG_STREAM_KV
    # Worked by hand: one KV head, 4 wavefronts (linear schedule), contexts
    # 2048, 256, 256, 256 tokens (128 + 3 * 16 pages), streaming (1/2 page
    # per position).  Loads per wavefront, then water filling:
    #   S = 4096 and 2048: 4 tasks, one each: 128.5, 16.5, 16.5, 16.5
    #     -> 16.5 + 112 / 1.43 = 94.82
    #   S = 1024: 5 tasks, chunks of 2: 129, 33, 16.5, 0
    #     -> 16.5 / (4/3) + 16.5 / 1.43 + 96 / 1.43 = 91.05
    #   S = 512: 7 tasks, chunks of 2: 65, 65, 33, 16.5
    #     -> 16.5 + 16.5 / (4/3) + 32 / 1.43 = 51.25
    #   S = 256: 11 tasks, chunks of 3: 49.5, 49.5, 49.5, 33
    #     -> 33 + 16.5 / (4/3) = 45.375
    #   S = 128: 22 tasks, chunks of 6: 51, 51, 51, 34 -> 46.75
    #   S = 64: 44 tasks, chunks of 11: 49.5 each -> 49.5
    # so 256.  (Pricing only the busiest wavefront against the mean would take
    # 512: the many loaded wavefronts of 512 are what water filling sees.)
    assert pick([2048, 256, 256, 256], W=4, Hq=8, Hkv=1, flags=stream) == 256
    # Full-size shapes (per-XCD classes: several sequences, Hkv = 8).
    # Streaming: four 53248-token sequences take 1024 (4096 and 2048 leave
    # wavefronts idle); cached loads stop at 256.
    assert pick([53248] * 4, max_pages=8192, flags=stream) == 1024
    assert pick([53248] * 4, max_pages=8192) == 256
    assert pick([73728] * 4, max_pages=8192, flags=stream) == 1024
    # One position per chunk at 4096 tokens: 8 x 262144 tokens on 2048
    # wavefronts, 4096 tasks in two even rounds.
    assert pick([2097152 // 8] * 8, max_pages=16384, flags=stream, W=2048) == 4096


def test_choose_split_on_the_reference_workloads():
    """With the load mode the benchmark uses (streaming unless pages are
    shared), as measured on MI355X against 256-token splits: B8 bimodal and
    B4 bimodal take 1024 (2.3% and 2.8% faster attention), Zipf lengths 2048
    (4.1%), B8 uniform 1024 (no difference measured); one long sequence and
    the shared-prefix batch keep 256.  The B64 lengths without their shared
    prefix (private pages, streaming) keep 256 too: measured 366.9 us
    against 392.0 us at 1024, where many wavefronts carry six 64-page tasks
    against a mean of 264 pages."""
    from paged_kv_cache_07_amd import workloads as W
    want = {"b1": 256, "b8_bimodal": 1024, "b8_uniform": 1024, "b8_zipf": 2048,
            "b4_bimodal": 1024, "b64_prefix": 256}
    for name, split in want.items():
        wl = W.make(name, fill_pools=False)
        flags = 0 if wl.shares_pages() else K.KVPAGE_FLAG_STREAM_KV
        shape = K.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.page_size, 256, wl.max_pages,
                             wl.num_pages, wl.dtype, wl.scale, flags)
        assert K.kvpage_choose_split(shape, wl.ctx_lens.tolist(), 1024) == split, name
    wl = W.make("b64_prefix", fill_pools=False)
    private = (wl.ctx_lens - wl.shared_prefix_pages * wl.page_size).tolist()
    shape = K.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.page_size, 256, wl.max_pages,
                         wl.num_pages, wl.dtype, wl.scale, K.KVPAGE_FLAG_STREAM_KV)
    assert K.kvpage_choose_split(shape, private, 1024) == 256


def test_choose_split_rejects_bad_lengths():
    lib = K.lib()
    s = _shape(B=2, max_pages=8)
    for ctx in ([-1, 4], [0, 8 * 16 + 1]):
        arr = (ctypes.c_int32 * 2)(*ctx)
        assert lib.kvpage_choose_split(ctypes.byref(s), arr, 1024) == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_choose_split(ctypes.byref(s), None, 1024) == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_choose_split(None, None, 1024) == K.KVPAGE_ERR_INVALID_ARG
    bad = _shape(B=1, d=96)
    arr = (ctypes.c_int32 * 1)(16)
    assert lib.kvpage_choose_split(ctypes.byref(bad), arr, 1024) == K.KVPAGE_ERR_UNSUPPORTED


def test_append_rejects_bad_arguments():
    """Null pointers, in/out buffers that overlap and misaligned rows are
    refused on the host (nothing enqueued, no device needed)."""
    lib = K.lib()
    s = _shape(B=4)
    p = [ctypes.c_void_p(256 * (i + 1)) for i in range(11)]
    ok = lambda args: lib.kvpage_append_kv(ctypes.byref(s), *args, None)
    for i in range(11):
        args = list(p)
        args[i] = None
        assert ok(args) == K.KVPAGE_ERR_INVALID_ARG, i
    args = list(p)
    args[6] = args[5]                      # ctx_lens_out == ctx_lens
    assert ok(args) == K.KVPAGE_ERR_INVALID_ARG
    args = list(p)
    args[9] = args[8]                      # free_count_out == free_count
    assert ok(args) == K.KVPAGE_ERR_INVALID_ARG
    args = list(p)
    args[0] = ctypes.c_void_p(256 + 8)     # k_new not 16-byte aligned
    assert ok(args) == K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_append_kv(ctypes.byref(_shape(B=4, d=96)), *p, None) == K.KVPAGE_ERR_UNSUPPORTED


def test_misaligned_buffers_are_rejected():
    """Vector loads need 16-byte aligned q, pools and workspace and 8-byte
    aligned out; misaligned pointers are refused on the host."""
    s = _shape()
    cap = K.kvpage_queue_capacity(s)
    lib = K.lib()
    good = ctypes.c_void_p(4096)
    for i, bad in ((0, 4096 + 8), (1, 4096 + 4), (2, 4096 + 2), (8, 4096 + 8)):
        args = [good] * 12
        args[i] = ctypes.c_void_p(bad)       # q, k_pool, v_pool, workspace
        rc = lib.kvpage_decode_step(ctypes.byref(s), args[0], args[1], args[2], good, good, good,
                                    good, good, cap, args[8], None, good, good, None, None)
        assert rc == K.KVPAGE_ERR_INVALID_ARG, i
    rc = lib.kvpage_decode_step(ctypes.byref(s), good, good, good, good, good, good, good, good,
                                cap, good, None, ctypes.c_void_p(4096 + 4), good, None, None)
    assert rc == K.KVPAGE_ERR_INVALID_ARG           # out
    assert lib.kvpage_merge_splits(ctypes.byref(s), good, cap, ctypes.c_void_p(4096 + 8), good,
                                   good, None) == K.KVPAGE_ERR_INVALID_ARG


def test_check_inputs_rejects_bad_arguments():
    """Null buffers, a queue given in part, or a capacity below the queue
    capacity are refused before anything is enqueued (no GPU needed)."""
    lib = K.lib()
    s = K.make_shape(2, 8, 2, 64, 16, 64, 4, 10, "f16", 0.125)
    cap = K.kvpage_queue_capacity(s)
    d = ctypes.c_void_p(16)
    bad = K.KVPAGE_ERR_INVALID_ARG
    assert lib.kvpage_check_inputs(ctypes.byref(s), None, d, None, None, None, 0, d, None) == bad
    assert lib.kvpage_check_inputs(ctypes.byref(s), d, None, None, None, None, 0, d, None) == bad
    assert lib.kvpage_check_inputs(ctypes.byref(s), d, d, None, None, None, 0, None, None) == bad
    assert lib.kvpage_check_inputs(ctypes.byref(s), d, d, d, None, d, cap, d, None) == bad
    assert lib.kvpage_check_inputs(ctypes.byref(s), d, d, d, d, d, cap - 1, d, None) \
        == K.KVPAGE_ERR_CAPACITY
    assert lib.kvpage_check_inputs(None, d, d, None, None, None, 0, d, None) == bad


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits non-zero with a message
    and starts no work (no GPU needed to check this)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=root)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_noalloc_step_refuses_a_workspace_past_its_static_size():
    """kvpage_decode_step_noalloc checks the workspace size against its
    static array before touching the device: 64 x 8 heads x 64 splits x G 8
    needs 136 MB, past the 64 MiB array."""
    lib = K.lib()
    s = K.make_shape(64, 64, 8, 128, 16, 256, 1024, 100000, "bf16", 128 ** -0.5, 0)
    cap = K.kvpage_queue_capacity(s)
    assert K.kvpage_workspace_bytes(s, cap) > K.KVPAGE_NOALLOC_WORKSPACE_BYTES
    dummy = ctypes.c_void_p(256)
    rc = lib.kvpage_decode_step_noalloc(ctypes.byref(s), dummy, dummy, dummy, dummy, dummy, dummy,
                                        dummy, dummy, cap, None, dummy, dummy, None, None)
    assert rc == K.KVPAGE_ERR_SCRATCH
    assert "static" in K.status_string(rc)
    small = K.make_shape(1, 32, 8, 128, 16, 256, 2048, 4096, "f16", 128 ** -0.5, 0)
    assert K.kvpage_workspace_bytes(small, K.kvpage_queue_capacity(small)) \
        <= K.KVPAGE_NOALLOC_WORKSPACE_BYTES
