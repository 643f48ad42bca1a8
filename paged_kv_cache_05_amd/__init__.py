"""Paged decode attention for MI355X: Python binding of ``libpa.so``.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/pa.h``.  Tensors are torch
device tensors (torch supplies device memory and streams); the functions
carry the C names:

* :func:`pa_decode` -- single-query decode attention over block pools
  addressed through per-sequence block tables,
* :func:`pa_decode_noalloc` -- pa_decode without a workspace (static device
  scratch), for callers that cannot allocate,
* :func:`pa_decode_append` -- one fused step: store each new token's K/V and
  decode over the context that includes it,
* :func:`pa_prefill` -- causal attention of a chunk of query tokens per
  sequence over its paged context (the prompt phase),
* :func:`pa_swap_blocks` -- whole blocks between device and pinned host pools,
* :func:`pa_write_kv` -- store the new tokens' K/V rows in their slots,
* :func:`pa_copy_blocks` -- copy-on-write copy of whole physical blocks,
* :func:`pa_decode_workspace_bytes`, :func:`pa_decode_partition_size`,
  :func:`pa_status_string`;

and :mod:`paged_kv_cache_05_amd.manager` wraps the host block manager
(``include/pa_manager.h``) and a decoding-step loop.

If ``libpa.so`` has not been built, every call raises :class:`PAError`;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libpa.so")

PA_OK = 0
PA_ERR_HIP = -5
PA_F16 = 0
PA_F32 = 1
PA_DEFAULT_PARTITION = 1024
PA_LONG_PARTITION = 4096
PA_LONG_CONTEXT = 8192
PA_NOALLOC_SCRATCH_BYTES = 16 << 20


def default_partition(max_context_len: int) -> int:
    """The partition length pa_decode uses when given partition_size 0."""
    return PA_LONG_PARTITION if max_context_len > PA_LONG_CONTEXT else PA_DEFAULT_PARTITION

# Every symbol include/pa.h and include/pa_manager.h declare.
EXPORTS = ("pa_decode", "pa_decode_append", "pa_decode_noalloc", "pa_decode_workspace_bytes", "pa_decode_partition_size", "pa_write_kv",
           "pa_copy_blocks", "pa_swap_blocks", "pa_prefill", "pa_prefill_workspace_bytes",
           "pa_status_string", "pa_last_error",
           "pa_manager_create", "pa_manager_destroy", "pa_manager_add", "pa_manager_fork",
           "pa_manager_append", "pa_manager_free", "pa_manager_tables", "pa_manager_num_free",
           "pa_manager_num_sequences", "pa_manager_refcount", "pa_manager_length",
           "pa_manager_check", "pa_manager_swap_out", "pa_manager_swap_in",
           "pa_manager_num_free_host", "pa_manager_is_swapped")


class PAError(RuntimeError):
    """A C-ABI call returned an error, or the library is missing."""


_lib = None


def hip_runtimes() -> list:
    """Paths of the HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return []
    return sorted(os.path.realpath(p) for p in paths)


def library() -> ctypes.CDLL:
    """Load libpa.so (built in-tree by ``python -m paged_kv_cache_05_amd._build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        raise PAError(f"{LIBRARY} is not built; run `python -m paged_kv_cache_05_amd._build` "
                      "(there is no fallback path)")
    # torch ships its own HIP runtime under the same soname.  Loaded first, it
    # is the one libpa.so binds to; loaded after libpa.so, a second runtime
    # would be mapped and the two would not share devices, memory or streams.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIBRARY)
    runtimes = hip_runtimes()
    if len(runtimes) > 1:
        raise PAError(f"two HIP runtimes are loaded in this process: {runtimes}; load torch "
                      "before any other HIP library")
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    lib.pa_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                              f32, i32, i32, vp, vp, sz, vp]
    lib.pa_decode.restype = i32
    lib.pa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                      f32, i32, i32, vp, vp]
    lib.pa_decode_noalloc.restype = i32
    lib.pa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                     i32, i32, f32, i32, i32, vp, vp, sz, vp]
    lib.pa_decode_append.restype = i32
    lib.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.pa_decode_workspace_bytes.restype = sz
    lib.pa_decode_partition_size.argtypes = [vp, i32, i32, i32, i32, i32, sz]
    lib.pa_decode_partition_size.restype = i32
    lib.pa_write_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_write_kv.restype = i32
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_copy_blocks.restype = i32
    lib.pa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                               i32, i32, f32, i32, vp, vp, vp, sz, vp]
    lib.pa_prefill.restype = i32
    lib.pa_prefill_workspace_bytes.argtypes = [i32, i32, i32]
    lib.pa_prefill_workspace_bytes.restype = sz
    lib.pa_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.pa_swap_blocks.restype = i32
    lib.pa_status_string.argtypes = [i32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def pa_status_string(status: int) -> str:
    return library().pa_status_string(int(status)).decode()


def pa_last_error() -> str:
    """The library's description of the last HIP runtime error it saw on
    this thread ("" if none)."""
    return library().pa_last_error().decode()


def _check(rc: int, what: str):
    if rc != PA_OK:
        detail = f" [{pa_last_error()}]" if rc == PA_ERR_HIP else ""
        raise PAError(f"{what}: {pa_status_string(rc)} ({rc}){detail}")


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.float32:
        return PA_F32
    raise PAError(f"unsupported element type {t.dtype}")


def _dev(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise PAError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise PAError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PAError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len,
                              partition_size=0) -> int:
    n = library().pa_decode_workspace_bytes(int(num_seqs), int(num_heads), int(head_dim),
                                            int(max_context_len), int(partition_size))
    if n == ctypes.c_size_t(-1).value:
        raise PAError("pa_decode_workspace_bytes: invalid arguments")
    return int(n)


def pa_decode_partition_size(num_seqs, num_heads, head_dim, max_context_len, partition_size=0,
                             host_context_lens=None, workspace_bytes=0) -> int:
    """The partition length pa_decode will use for these arguments."""
    import numpy as np
    host = None
    if host_context_lens is not None:
        host = np.ascontiguousarray(host_context_lens, dtype=np.int32)
    n = library().pa_decode_partition_size(None if host is None else host.ctypes.data,
                                           int(num_seqs), int(num_heads), int(head_dim),
                                           int(max_context_len), int(partition_size),
                                           int(workspace_bytes))
    if n < 0:
        raise PAError(f"pa_decode_partition_size: {pa_status_string(n)} ({n})")
    return int(n)


def pa_prefill_workspace_bytes(num_heads, head_dim, slots) -> int:
    """Bytes of a pa_prefill workspace with `slots` partial-result slots."""
    n = library().pa_prefill_workspace_bytes(int(num_heads), int(head_dim), int(slots))
    if n == 0:
        raise PAError("pa_prefill_workspace_bytes: invalid arguments")
    return int(n)


def new_prefill_workspace(num_heads, head_dim, slots=64, device="cuda"):
    """A pa_prefill workspace of `slots` partial-result slots."""
    import torch
    return torch.empty(pa_prefill_workspace_bytes(num_heads, head_dim, slots), dtype=torch.uint8,
                       device=device)


def new_workspace(num_seqs, num_heads, head_dim, max_context_len, partition_size=0,
                  device="cuda"):
    """A workspace of the size pa_decode needs (None when none is needed)."""
    import torch
    n = pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def _decode_common(q, out, k_pool, v_pool, block_tables, context_lens, host_context_lens):
    import numpy as np
    host = None
    if host_context_lens is not None:
        host = np.ascontiguousarray(host_context_lens, dtype=np.int32)
        if host.shape != (q.shape[0],):
            raise PAError("host_context_lens must have one entry per sequence")
    N, H, D = q.shape
    NB, H2, B, D2 = k_pool.shape
    if (H2, D2) != (H, D) or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise PAError("pool shape does not match q")
    if tuple(out.shape) != (N, H, D) or out.dtype != q.dtype:
        raise PAError("out must match q in shape and type")
    if k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise PAError("q and pools must share one element type")
    if block_tables.dim() != 2 or block_tables.shape[0] != N or tuple(context_lens.shape) != (N,):
        raise PAError("block_tables / context_lens do not match the batch")
    return host, (N, H, D, B, NB)


def pa_decode(out, q, k_pool, v_pool, block_tables, context_lens, scale, max_context_len,
              partition_size=0, workspace=None, stream=None, host_context_lens=None):
    """out[N][H][D] = paged decode attention of q[N][H][D] over the pools.

    k_pool/v_pool: [num_blocks][H][block_size][D]; block_tables int32
    [N][max_blocks_per_seq]; context_lens int32 [N]; max_context_len: host
    int >= every context length; workspace: from :func:`new_workspace`;
    host_context_lens: optional host copy of context_lens (numpy int32 or a
    sequence of ints), used only to plan the launch.
    """
    import torch
    host, (N, H, D, B, NB) = _decode_common(q, out, k_pool, v_pool, block_tables, context_lens,
                                            host_context_lens)
    ws_ptr = _dev(workspace, "workspace", torch.uint8)
    ws_bytes = workspace.numel() if workspace is not None else 0
    rc = library().pa_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        N, H, D, B, NB, block_tables.shape[1], int(max_context_len), float(scale), _dtype_code(q),
        int(partition_size), None if host is None else host.ctypes.data, ws_ptr, ws_bytes,
        _stream(stream))
    _check(rc, "pa_decode")
    return out


def pa_decode_noalloc(out, q, k_pool, v_pool, block_tables, context_lens, scale,
                      max_context_len, partition_size=0, stream=None, host_context_lens=None):
    """pa_decode without a workspace: partial results go to the library's
    static device scratch (PA_NOALLOC_SCRATCH_BYTES per GPU), so the call
    allocates nothing.  Calls that overlap on one GPU race on that scratch."""
    import torch
    host, (N, H, D, B, NB) = _decode_common(q, out, k_pool, v_pool, block_tables, context_lens,
                                            host_context_lens)
    rc = library().pa_decode_noalloc(
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        N, H, D, B, NB, block_tables.shape[1], int(max_context_len), float(scale), _dtype_code(q),
        int(partition_size), None if host is None else host.ctypes.data, _stream(stream))
    _check(rc, "pa_decode_noalloc")
    return out


def pa_decode_append(out, q, new_key, new_value, k_pool, v_pool, block_tables, context_lens,
                     slot_mapping, scale, max_context_len, partition_size=0, workspace=None,
                     stream=None, host_context_lens=None):
    """One fused decoding step: store new_key/new_value [N][H][D] at
    slot_mapping (int64 [N], the slot of each sequence's position
    context_lens - 1) and attend q over every context, the new token
    included.  Bit for bit pa_write_kv followed by pa_decode."""
    import torch
    host, (N, H, D, B, NB) = _decode_common(q, out, k_pool, v_pool, block_tables, context_lens,
                                            host_context_lens)
    for t, name in ((new_key, "new_key"), (new_value, "new_value")):
        if tuple(t.shape) != (N, H, D) or t.dtype != q.dtype:
            raise PAError(f"{name} must match q in shape and type")
    if tuple(slot_mapping.shape) != (N,):
        raise PAError("slot_mapping must have one entry per sequence")
    ws_ptr = _dev(workspace, "workspace", torch.uint8)
    ws_bytes = workspace.numel() if workspace is not None else 0
    rc = library().pa_decode_append(
        _dev(out, "out"), _dev(q, "q"), _dev(new_key, "new_key"), _dev(new_value, "new_value"),
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32), _dev(context_lens, "context_lens", torch.int32),
        _dev(slot_mapping, "slot_mapping", torch.int64),
        N, H, D, B, NB, block_tables.shape[1], int(max_context_len), float(scale), _dtype_code(q),
        int(partition_size), None if host is None else host.ctypes.data, ws_ptr, ws_bytes,
        _stream(stream))
    _check(rc, "pa_decode_append")
    return out


def pa_write_kv(key, value, k_pool, v_pool, slot_mapping, stream=None):
    """Store key/value [T][H][D] rows at slot_mapping (int64 [T]) in the pools."""
    import torch
    T, H, D = key.shape
    NB, H2, B, D2 = k_pool.shape
    if (H2, D2) != (H, D) or tuple(value.shape) != tuple(key.shape) or \
            tuple(v_pool.shape) != tuple(k_pool.shape) or tuple(slot_mapping.shape) != (T,):
        raise PAError("pa_write_kv: shapes do not match")
    if not (key.dtype == value.dtype == k_pool.dtype == v_pool.dtype):
        raise PAError("pa_write_kv: key, value and pools must share one element type")
    rc = library().pa_write_kv(
        _dev(key, "key"), _dev(value, "value"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(slot_mapping, "slot_mapping", torch.int64), T, H, D, B, NB, _dtype_code(key),
        _stream(stream))
    _check(rc, "pa_write_kv")


def pa_copy_blocks(k_pool, v_pool, block_mapping, stream=None):
    """Copy whole blocks (src, dst) = block_mapping[i] (int64 [P][2]) in both pools."""
    import torch
    NB, H, B, D = k_pool.shape
    if tuple(v_pool.shape) != tuple(k_pool.shape) or v_pool.dtype != k_pool.dtype:
        raise PAError("pa_copy_blocks: pools differ")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise PAError("pa_copy_blocks: block_mapping must be [P][2]")
    rc = library().pa_copy_blocks(
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_mapping, "block_mapping", torch.int64), block_mapping.shape[0], H, D, B, NB,
        _dtype_code(k_pool), _stream(stream))
    _check(rc, "pa_copy_blocks")


def _reachable(t, name, dtype=None):
    """Pointer of a device tensor or of a pinned host tensor."""
    if not t.is_cuda and not t.is_pinned():
        raise PAError(f"{name} must be a device tensor or a pinned host tensor")
    if not t.is_contiguous():
        raise PAError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise PAError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def pa_swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping, stream=None):
    """Copy block src of (src_k, src_v) onto block dst of (dst_k, dst_v) for
    every (src, dst) = block_mapping[i] (int64 [P][2]).  Each tensor is a
    device tensor or a pinned host tensor (swap out: device pools -> pinned
    host pools; swap in: the reverse)."""
    import torch
    sNB, H, B, D = src_k.shape
    dNB = dst_k.shape[0]
    if (tuple(dst_k.shape[1:]) != (H, B, D) or tuple(src_v.shape) != tuple(src_k.shape)
            or tuple(dst_v.shape) != tuple(dst_k.shape)):
        raise PAError("pa_swap_blocks: pools differ in block shape")
    if len({t.dtype for t in (dst_k, dst_v, src_k, src_v)}) != 1:
        raise PAError("pa_swap_blocks: pools differ in element type")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise PAError("pa_swap_blocks: block_mapping must be [P][2]")
    rc = library().pa_swap_blocks(
        _reachable(dst_k, "dst_k"), _reachable(dst_v, "dst_v"), _reachable(src_k, "src_k"),
        _reachable(src_v, "src_v"), _reachable(block_mapping, "block_mapping", torch.int64),
        block_mapping.shape[0], H, D, B, sNB, dNB, _dtype_code(src_k), _stream(stream))
    _check(rc, "pa_swap_blocks")


def pa_prefill(out, q, k_pool, v_pool, block_tables, context_lens, query_start, scale,
               max_context_len, max_query_len, stream=None, host_query_start=None,
               host_context_lens=None, workspace=None):
    """out[T][H][D] = causal paged prefill attention of q[T][H][D]: sequence
    b's rows query_start[b] .. query_start[b+1]-1 are the last tokens of its
    context_lens[b]-token context (int32 device tensors; query_start [N+1]).
    max_context_len and max_query_len are host-side bounds; host copies of
    query_start (and context_lens) let the library launch only the tiles
    that exist, grouped by sequence, heaviest first.  workspace (optional,
    a device uint8 tensor, see new_prefill_workspace) lets that launch split
    the key range of its heaviest tiles when they alone would set its
    length."""
    import numpy as np
    import torch
    NB, H, B, D = k_pool.shape
    T = q.shape[0]
    N = context_lens.shape[0]
    if tuple(q.shape) != (T, H, D) or tuple(out.shape) != (T, H, D):
        raise PAError("pa_prefill: q / out must be [T][H][D] matching the pools")
    if tuple(query_start.shape) != (N + 1,):
        raise PAError("pa_prefill: query_start must be [num_seqs + 1]")
    if block_tables.dim() != 2 or block_tables.shape[0] != N:
        raise PAError("pa_prefill: block_tables must be [num_seqs][max_blocks]")
    for t, name in ((q, "q"), (out, "out"), (v_pool, "v_pool")):
        if t.dtype != k_pool.dtype:
            raise PAError(f"pa_prefill: {name} must be {k_pool.dtype}")
    hqs = _host_i32(host_query_start, N + 1, "host_query_start")
    hctx = _host_i32(host_context_lens, N, "host_context_lens")
    rc = library().pa_prefill(
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _dev(block_tables, "block_tables", torch.int32),
        _dev(context_lens, "context_lens", torch.int32),
        _dev(query_start, "query_start", torch.int32), N, T, H, D, B, NB,
        block_tables.shape[1], int(max_context_len), int(max_query_len), float(scale),
        _dtype_code(q), None if hqs is None else hqs.ctypes.data,
        None if hctx is None else hctx.ctypes.data,
        None if workspace is None else _dev(workspace, "workspace", torch.uint8),
        0 if workspace is None else workspace.numel(), _stream(stream))
    _check(rc, "pa_prefill")



def _host_i32(a, n, name):
    """A contiguous int32 host copy (kept alive by the caller for the call)."""
    import numpy as np
    if a is None:
        return None
    arr = np.ascontiguousarray(a, dtype=np.int32)
    if arr.shape != (n,):
        raise PAError(f"{name} must have {n} entries")
    return arr
