"""Host block manager and decoding-step loop over the paged kernels.

:class:`BlockManager` wraps the C++ manager of ``include/pa_manager.h``
(free blocks, reference counts, per-sequence block lists; copy-on-write
of a shared last block).  :class:`DecodeStepper` runs one decoding step of a
batch the way the PagedAttention pages describe it: the manager reserves
each sequence's next slot (a fresh block when the last one is full, a
private copy when it is shared), then the GPU copies the shared blocks
(``pa_copy_blocks``), then stores the new tokens' K/V and attends over the
whole context in one launch (``pa_decode_append``).  Argument marshalling and
bookkeeping only; all device work runs in the HIP kernels.
"""
from __future__ import annotations

import ctypes
import time

import numpy as np

from . import PAError, library, pa_copy_blocks, pa_decode_append, pa_decode_workspace_bytes, \
    pa_status_string, pa_swap_blocks

PA_ERR_NO_SEQUENCE = -6
PA_ERR_EXISTS = -7
PA_ERR_NO_BLOCKS = -8
PA_ERR_SWAPPED = -9


class OutOfBlocks(PAError):
    """pa_manager_append found too few free blocks; nothing was changed."""


def _bind(lib):
    if getattr(lib, "_pa_manager_bound", False):
        return lib
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.pa_manager_create.argtypes = [i32, i32, i32, vp]
    lib.pa_manager_create.restype = vp
    lib.pa_manager_destroy.argtypes = [vp]
    lib.pa_manager_destroy.restype = None
    lib.pa_manager_add.argtypes = [vp, i64]
    lib.pa_manager_fork.argtypes = [vp, i64, i64]
    lib.pa_manager_append.argtypes = [vp, vp, i32, vp, vp, i32, vp]
    lib.pa_manager_free.argtypes = [vp, i64]
    lib.pa_manager_tables.argtypes = [vp, vp, i32, vp, i32, vp]
    lib.pa_manager_num_free.argtypes = [vp]
    lib.pa_manager_num_sequences.argtypes = [vp]
    lib.pa_manager_refcount.argtypes = [vp, i32]
    lib.pa_manager_length.argtypes = [vp, i64]
    lib.pa_manager_check.argtypes = [vp]
    lib.pa_manager_swap_out.argtypes = [vp, vp, i32, vp, i32, vp]
    lib.pa_manager_swap_in.argtypes = [vp, vp, i32, vp, i32, vp]
    lib.pa_manager_num_free_host.argtypes = [vp]
    lib.pa_manager_is_swapped.argtypes = [vp, i64]
    for f in ("add", "fork", "append", "free", "tables", "num_free", "num_sequences",
              "refcount", "length", "check", "swap_out", "swap_in", "num_free_host",
              "is_swapped"):
        getattr(lib, "pa_manager_" + f).restype = i32
    lib._pa_manager_bound = True
    return lib


def _check(rc, what):
    if rc == PA_ERR_NO_BLOCKS:
        raise OutOfBlocks(f"{what}: {pa_status_string(rc)}")
    if rc < 0:
        raise PAError(f"{what}: {pa_status_string(rc)} ({rc})")
    return rc


class BlockManager:
    """GPU blocks 0..num_blocks-1 of block_size tokens and a CPU swap space
    of num_host_blocks blocks (host state only).

    ``lib`` is the ctypes library exporting the ``pa_manager_*`` functions
    (default: this package's libpa.so)."""

    def __init__(self, num_blocks, block_size, alloc_order=None, num_host_blocks=0, lib=None):
        self._lib = _bind(lib if lib is not None else library())
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.num_host_blocks = int(num_host_blocks)
        order = None
        if alloc_order is not None:
            order = np.ascontiguousarray(alloc_order, dtype=np.int32)
            if order.shape != (self.num_blocks,):
                raise PAError("alloc_order must list every block once")
        self._h = self._lib.pa_manager_create(self.num_blocks, self.block_size,
                                              self.num_host_blocks,
                                              None if order is None else order.ctypes.data)
        if not self._h:
            raise PAError("pa_manager_create: bad arguments")

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h:
            self._lib.pa_manager_destroy(h)

    def add(self, seq):
        _check(self._lib.pa_manager_add(self._h, int(seq)), "add")

    def fork(self, parent, child):
        _check(self._lib.pa_manager_fork(self._h, int(parent), int(child)), "fork")

    def free(self, seq):
        _check(self._lib.pa_manager_free(self._h, int(seq)), "free")

    def append(self, seqs):
        """Slots (int64 [n]) for the next token of each sequence, and the
        copy-on-write pairs (int64 [P][2]) to execute before writing them."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        n = len(ids)
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int64)
        npairs = ctypes.c_int(0)
        _check(self._lib.pa_manager_append(self._h, ids.ctypes.data, n, slots.ctypes.data,
                                           pairs.ctypes.data, pairs.shape[0],
                                           ctypes.byref(npairs)), "append")
        return slots, pairs[:npairs.value].copy()

    def _move(self, fn, seqs, what):
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        cap = max(self.num_blocks, self.num_host_blocks, 1)
        pairs = np.empty((cap, 2), dtype=np.int64)
        npairs = ctypes.c_int(0)
        _check(fn(self._h, ids.ctypes.data, len(ids), pairs.ctypes.data, cap,
                  ctypes.byref(npairs)), what)
        return pairs[:npairs.value].copy()

    def swap_out(self, seqs):
        """Evict a group of sequences to the swap space: (gpu, host) pairs."""
        return self._move(self._lib.pa_manager_swap_out, seqs, "swap_out")

    def swap_in(self, seqs):
        """Bring a swapped-out group back: (host, gpu) pairs."""
        return self._move(self._lib.pa_manager_swap_in, seqs, "swap_in")

    @property
    def num_free_host(self):
        return _check(self._lib.pa_manager_num_free_host(self._h), "num_free_host")

    def is_swapped(self, seq):
        return bool(_check(self._lib.pa_manager_is_swapped(self._h, int(seq)), "is_swapped"))

    def tables(self, seqs, max_blocks):
        """Block tables (int32 [n][max_blocks], -1 padded) and context lengths."""
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        tables = np.empty((len(ids), int(max_blocks)), dtype=np.int32)
        ctx = np.empty(len(ids), dtype=np.int32)
        _check(self._lib.pa_manager_tables(self._h, ids.ctypes.data, len(ids),
                                           tables.ctypes.data, int(max_blocks), ctx.ctypes.data),
               "tables")
        return tables, ctx

    @property
    def num_free(self):
        return _check(self._lib.pa_manager_num_free(self._h), "num_free")

    @property
    def num_sequences(self):
        return _check(self._lib.pa_manager_num_sequences(self._h), "num_sequences")

    def refcount(self, block):
        return _check(self._lib.pa_manager_refcount(self._h, int(block)), "refcount")

    def length(self, seq):
        return _check(self._lib.pa_manager_length(self._h, int(seq)), "length")

    def check(self):
        _check(self._lib.pa_manager_check(self._h), "check")


class StepPlan:
    """The host decisions of one decoding step and their device copies:
    slots (int64 [n]), copy pairs (int64 [P][2]), block tables (int32
    [n][max_blocks]) and context lengths (int32 [n]).  Every layer of the
    step uses the same plan."""

    __slots__ = ("seqs", "slots", "pairs", "tables", "context_lens", "max_context_len",
                 "d_slots", "d_pairs", "d_tables", "d_context_lens", "host_seconds")


class DecodeStepper:
    """Decoding steps of a batch over one or more layers' K/V pools that a
    single BlockManager manages (every layer of a model shares the block
    tables; only the pool contents differ).

    ``pools`` is one (k_pool, v_pool) pair or a list of them, one per layer;
    ``host_pools`` (optional, same form, pinned host tensors of
    manager.num_host_blocks blocks) is the swap space.  :meth:`plan` makes
    the step's host decisions and uploads them with one host-to-device copy
    from pinned memory; :meth:`layer` runs the step's device work on one
    layer: copy-on-write copies (pa_copy_blocks), then the new tokens' K/V
    and the decode attention in one launch (pa_decode_append).  :meth:`swap_out` and
    :meth:`swap_in` move a preempted group's blocks to the swap space and
    back, on every layer (pa_swap_blocks).  All device work goes to torch's
    current stream, so a swap-out's copies finish before the freed blocks
    are written again.
    """

    def __init__(self, manager: BlockManager, pools, max_blocks, partition_size=0,
                 host_pools=None):
        import torch
        self._torch = torch

        def as_list(p):
            if isinstance(p, tuple) and len(p) == 2 and hasattr(p[0], "shape"):
                return [p]
            return list(p)

        self.pools = as_list(pools)
        self.host_pools = as_list(host_pools) if host_pools is not None else None
        if self.host_pools is not None:
            if len(self.host_pools) != len(self.pools):
                raise PAError("one host pool pair per layer")
            for (k, v), (hk, hv) in zip(self.pools, self.host_pools):
                if (hk.shape[0] != manager.num_host_blocks or hk.shape[1:] != k.shape[1:]
                        or hv.shape != hk.shape or hk.dtype != k.dtype or hv.dtype != k.dtype):
                    raise PAError("host pools do not match the manager and the device pools")
        self.manager = manager
        self.max_blocks, self.partition_size = int(max_blocks), int(partition_size)
        self.device = self.pools[0][0].device
        for k, v in self.pools:
            NB, H, B, D = k.shape
            if (NB, B) != (manager.num_blocks, manager.block_size) or v.shape != k.shape:
                raise PAError("pools do not match the manager")
        self._ws = None
        # two pinned staging buffers, each reused only after its copy finished
        self._staging = [None, None]
        self._staged = [None, None]
        self._turn = 0

    @property
    def k_pool(self):
        return self.pools[0][0]

    @property
    def v_pool(self):
        return self.pools[0][1]

    def _upload(self, arrays):
        torch = self._torch
        offs, size = [], 0
        for a in arrays:
            offs.append(size)
            size += -(-a.nbytes // 256) * 256
        size = max(size, 256)
        t = self._turn
        self._turn ^= 1
        if self._staged[t] is not None:
            self._staged[t].synchronize()
        if self._staging[t] is None or self._staging[t].numel() < size:
            self._staging[t] = torch.empty(max(size, 1 << 16), dtype=torch.uint8, pin_memory=True)
        host = self._staging[t].numpy()
        for a, o in zip(arrays, offs):
            host[o:o + a.nbytes] = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
        dbuf = torch.empty(size, dtype=torch.uint8, device=self.device)
        dbuf.copy_(self._staging[t][:size], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record()
        self._staged[t] = ev
        tdt = {np.dtype(np.int32): torch.int32, np.dtype(np.int64): torch.int64}
        return [dbuf[o:o + a.nbytes].view(tdt[a.dtype]).view(a.shape) for a, o in zip(arrays, offs)]

    def _workspace(self, n, H, D, maxctx):
        # an explicit partition size, or else the smallest partition the
        # host-planned launch picks (256 tokens; it never needs more)
        need = pa_decode_workspace_bytes(n, H, D, maxctx, self.partition_size or 256)
        if self._ws is None or self._ws.numel() < need:
            self._ws = self._torch.empty(max(need, 256), dtype=self._torch.uint8,
                                         device=self.device)
        return self._ws

    def plan(self, seqs) -> StepPlan:
        """Reserve every sequence's next slot (allocation and copy-on-write
        decisions), build the tables and upload them.  Each sequence appears
        at most once: a step adds one token per sequence."""
        t = time.perf_counter()
        p = StepPlan()
        p.seqs = list(seqs)
        if len(set(p.seqs)) != len(p.seqs):
            raise PAError("a decoding step lists each sequence once")
        p.slots, p.pairs = self.manager.append(p.seqs)
        p.tables, p.context_lens = self.manager.tables(p.seqs, self.max_blocks)
        p.max_context_len = int(p.context_lens.max()) if len(p.seqs) else 0
        p.host_seconds = time.perf_counter() - t   # the manager's decisions alone
        p.d_slots, p.d_pairs, p.d_tables, p.d_context_lens = self._upload(
            [p.slots, p.pairs, p.tables, p.context_lens])
        return p

    def layer(self, plan: StepPlan, layer, new_key, new_value, q, scale, out=None):
        """The step's device work on one layer's pools: the copy-on-write
        copies, then one fused launch that stores the new tokens and decodes
        (pa_decode_append); returns out [n][H][D]."""
        k, v = self.pools[layer]
        if len(plan.pairs):
            pa_copy_blocks(k, v, plan.d_pairs)
        if out is None:
            out = self._torch.empty_like(q)
        n, H, D = q.shape
        ws = self._workspace(n, H, D, plan.max_context_len)
        pa_decode_append(out, q, new_key, new_value, k, v, plan.d_tables, plan.d_context_lens,
                         plan.d_slots, scale, plan.max_context_len, self.partition_size, ws,
                         host_context_lens=plan.context_lens)
        return out

    def _swap(self, pairs, out):
        if self.host_pools is None:
            raise PAError("no swap space: pass host_pools")
        if len(pairs):
            (d_pairs,) = self._upload([pairs])
            for (k, v), (hk, hv) in zip(self.pools, self.host_pools):
                if out:
                    pa_swap_blocks(hk, hv, k, v, d_pairs)
                else:
                    pa_swap_blocks(k, v, hk, hv, d_pairs)
        return pairs

    def swap_out(self, seqs):
        """Preempt a group: its blocks go to the swap space on every layer.
        Returns the (gpu, host) pairs."""
        return self._swap(self.manager.swap_out(seqs), True)

    def swap_in(self, seqs):
        """Resume a swapped-out group on fresh GPU blocks, every layer.
        Returns the (host, gpu) pairs."""
        return self._swap(self.manager.swap_in(seqs), False)

    def step(self, seqs, new_key, new_value, q, scale, out=None):
        """One step on the first (or only) layer: append one token
        (new_key/new_value [n][H][D] device tensors) to each sequence and
        return (decode attention of q over each context, new token included,
        the plan)."""
        plan = self.plan(seqs)
        return self.layer(plan, 0, new_key, new_value, q, scale, out), plan
