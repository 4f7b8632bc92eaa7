"""Device-resident buffers for one decode step, driven through the C ABI.

Plumbing only: torch allocates device memory and provides the stream; every
computation is a libkvpage.so kernel called through ``binding``.
"""

from __future__ import annotations

import numpy as np

from . import binding as K


def _torch():
    import torch
    return torch


def host_to_device(arr: np.ndarray, dtype: str, device):
    """Upload f16 arrays or bf16 bit patterns (uint16) without changing bits."""
    torch = _torch()
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def device_to_bits(t) -> np.ndarray:
    """Download an f16/bf16 tensor as its raw uint16 bits."""
    torch = _torch()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class DecodeStep:
    """Inputs, queue, workspace and outputs of one paged GQA decode step.

    ``run()`` enqueues build_queue -> decode_attn (split attention + merge)
    -> page_mass on torch's current stream.  Summary state double-buffers:
    each run reads ``s_prev`` and writes ``s_next``; ``swap_summaries()``
    flips them for the next step.
    """

    def __init__(self, wl, device="cuda", budget=True, split_tokens=None, stream_kv=False,
                 shared_pages=None):
        torch = _torch()
        self.wl = wl
        self.device = torch.device(device)
        self.split_tokens = split_tokens or wl.split_tokens
        # stream_kv: the caller's promise that no page is shared between
        # sequences (KVPAGE_FLAG_STREAM_KV); it changes no result.
        self.shape = K.make_shape(wl.B, wl.Hq, wl.Hkv, wl.d, wl.page_size, self.split_tokens,
                                  wl.max_pages, wl.num_pages, wl.dtype, wl.scale,
                                  K.KVPAGE_FLAG_STREAM_KV if stream_kv else 0)
        self.capacity = K.kvpage_queue_capacity(self.shape)
        ws = K.kvpage_workspace_bytes(self.shape, self.capacity)
        dev = self.device
        self.q = host_to_device(wl.q, wl.dtype, dev)
        self.k_pool = host_to_device(wl.k_pool, wl.dtype, dev)
        self.v_pool = host_to_device(wl.v_pool, wl.dtype, dev)
        self.block_tables = torch.from_numpy(np.ascontiguousarray(wl.block_tables)).to(dev)
        self.ctx_lens = torch.from_numpy(np.ascontiguousarray(wl.ctx_lens)).to(dev)
        self.tasks = torch.zeros((max(1, self.capacity), 4), dtype=torch.int32, device=dev)
        self.group_offsets = torch.zeros(wl.B * wl.Hkv + 1, dtype=torch.int32, device=dev)
        self.n_tasks = torch.zeros(1, dtype=torch.int32, device=dev)
        self.workspace = torch.zeros(max(256, ws), dtype=torch.uint8, device=dev)
        out_dtype = torch.float16 if wl.dtype == "f16" else torch.bfloat16
        self.out = torch.zeros((wl.B, wl.Hq, wl.d), dtype=out_dtype, device=dev)
        self.lse = torch.zeros((wl.B, wl.Hq), dtype=torch.float32, device=dev)
        # shared_pages: None, or per sequence the leading table pages other
        # sequences may share (kvpage_launch_opts.shared_pages; with stream_kv
        # those pages load through the caches, the rest stream).
        self.shared_pages = None if shared_pages is None else torch.from_numpy(
            np.ascontiguousarray(shared_pages, dtype=np.int32)).to(dev)
        self.use_budget = budget
        if budget:
            self.page_mass = torch.zeros((wl.B, wl.Hq, wl.max_pages), dtype=torch.float32, device=dev)
            self.page_max = torch.zeros((2, wl.B, wl.Hkv, wl.max_pages), dtype=torch.float32, device=dev)
            self.s_prev = torch.from_numpy(np.ascontiguousarray(wl.s_prev)).to(dev)
            self.s_next = torch.zeros_like(self.s_prev)
            self._make_budget()
        else:
            self.budget = None
        self.scribble()

    def scribble(self):
        """Fill every buffer the library writes (queue, workspace, outputs)
        with NaN or junk, so that an entry a kernel fails to write cannot pass
        a comparison as a leftover zero."""
        torch = _torch()
        self.tasks.fill_(-7)
        self.group_offsets.fill_(-7)
        self.n_tasks.fill_(-7)
        self.workspace.fill_(0xFF)          # NaN floats, header word -1
        self.out.fill_(float("nan"))
        self.lse.fill_(float("nan"))
        if self.use_budget:
            self.page_mass.fill_(float("nan"))
            self.page_max.fill_(float("nan"))
            self.s_next.fill_(float("nan"))
        torch.cuda.synchronize(self.device)

    def _make_budget(self):
        self.budget = K.make_budget(self.page_mass, self.s_prev, self.s_next, self.page_max,
                                    self.wl.alpha_fast, self.wl.alpha_slow)

    def swap_summaries(self):
        self.s_prev, self.s_next = self.s_next, self.s_prev
        self._make_budget()

    def set_query(self, q_host: np.ndarray):
        self.q.copy_(host_to_device(q_host, self.wl.dtype, self.device))

    def schedule_classes(self) -> int:
        """Schedule classes the last attention launch used (workspace header
        word 1): 8 when each KV head's tasks ran on one XCD, else 1.  Run
        partials, and so the rounding of out, lse and page mass, follow the
        schedule."""
        torch = _torch()
        torch.cuda.synchronize(self.device)
        return int(self.workspace[4:8].view(torch.int32).item())

    # -- the three calls of a step --------------------------------------
    def build_queue(self, stream=None):
        K.kvpage_build_queue(self.shape, self.ctx_lens, self.tasks, self.capacity,
                             self.group_offsets, self.n_tasks, stream)

    def decode_attn(self, stream=None):
        K.kvpage_decode_attn(self.shape, self.q, self.k_pool, self.v_pool, self.block_tables,
                             self.ctx_lens, self.tasks, self.group_offsets, self.n_tasks,
                             self.capacity, self.workspace, self.budget, self.out, self.lse, stream)

    def split_attn(self, stream=None):
        K.kvpage_split_attn(self.shape, self.q, self.k_pool, self.v_pool, self.block_tables,
                            self.ctx_lens, self.tasks, self.n_tasks, self.capacity,
                            self.workspace, self.budget, stream)

    def merge_splits(self, stream=None):
        K.kvpage_merge_splits(self.shape, self.group_offsets, self.capacity, self.workspace,
                              self.out, self.lse, stream)

    def page_mass_finish(self, stream=None):
        K.kvpage_page_mass(self.shape, self.budget, self.q, self.lse, self.ctx_lens,
                           self.group_offsets, self.capacity, self.workspace, stream)

    def run(self, stream=None):
        self.build_queue(stream)
        self.decode_attn(stream)
        if self.use_budget:
            self.page_mass_finish(stream)

    def launch_opts(self, opts=None):
        """opts with this step's shared_pages filled in (a new one if None)."""
        if self.shared_pages is None:
            return opts
        if opts is None:
            opts = K.make_opts()
        opts.shared_pages = self.shared_pages.data_ptr()
        return opts

    def step(self, opts=None, stream=None):
        """The whole step in one call (queue, split attention, fused merge+finish)."""
        K.kvpage_decode_step(self.shape, self.q, self.k_pool, self.v_pool, self.block_tables,
                             self.ctx_lens, self.tasks, self.group_offsets, self.n_tasks,
                             self.capacity, self.workspace, self.budget, self.out, self.lse,
                             self.launch_opts(opts), stream)

    # -- KV append (the step before attention) ----------------------------
    def set_free_list(self, free_pages: np.ndarray):
        """Physical pages the appends may take (a stack: the last entry goes first)."""
        torch = _torch()
        dev = self.device
        fp = np.ascontiguousarray(free_pages, dtype=np.int32)
        self.free_pages = torch.from_numpy(fp if len(fp) else np.zeros(1, np.int32)).to(dev)
        self.free_count = torch.tensor([len(fp)], dtype=torch.int32, device=dev)
        self.free_count_next = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ctx_next = torch.zeros_like(self.ctx_lens)
        self.append_status = torch.zeros(1, dtype=torch.int32, device=dev)

    def append_kv(self, k_new_host: np.ndarray, v_new_host: np.ndarray, stream=None):
        """Append one token per sequence; the new lengths and free count become current."""
        k_new = host_to_device(k_new_host, self.wl.dtype, self.device)
        v_new = host_to_device(v_new_host, self.wl.dtype, self.device)
        K.kvpage_append_kv(self.shape, k_new, v_new, self.k_pool, self.v_pool, self.block_tables,
                           self.ctx_lens, self.ctx_next, self.free_pages, self.free_count,
                           self.free_count_next, self.append_status, stream)
        self.ctx_lens, self.ctx_next = self.ctx_next, self.ctx_lens
        self.free_count, self.free_count_next = self.free_count_next, self.free_count
        self._keep = (k_new, v_new)   # alive until the stream has used them

    def gather_offsets(self, stream=None):
        torch = _torch()
        offs = torch.full((max(1, self.capacity), self.split_tokens, 2), -7, dtype=torch.int64,
                          device=self.device)
        K.kvpage_debug_gather_offsets(self.shape, self.block_tables, self.tasks, self.n_tasks,
                                      self.capacity, offs, stream)
        return offs

    def results(self) -> dict:
        torch = _torch()
        torch.cuda.synchronize(self.device)
        n = int(self.n_tasks.item())
        res = {
            "n_tasks": n,
            "tasks": self.tasks[:n].cpu().numpy(),
            "group_offsets": self.group_offsets.cpu().numpy(),
            "out_bits": device_to_bits(self.out),
            "out": self.out.float().cpu().numpy().astype(np.float64),
            "lse": self.lse.cpu().numpy().astype(np.float64),
        }
        if self.use_budget:
            res["mass"] = self.page_mass.cpu().numpy().astype(np.float64)
            res["page_max"] = self.page_max.cpu().numpy().astype(np.float64)
            res["s_next"] = self.s_next.cpu().numpy().astype(np.float64)
        return res
