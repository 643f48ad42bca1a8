"""Plain fp64 CPU oracle for paged decode attention, its KV write and its
copy-on-write block copy.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline are the only callers.  The product path never imports this package,
and this package imports nothing from the product path.  The arithmetic lives
in ``oracle.c`` (plain C, gcc, OpenMP over (sequence, head) pairs); this file
only builds it and marshals numpy arrays.

What each function follows on the pages (Kwon et al., PagedAttention):

* :func:`decode` -- zhaifeiyue.github.io summary, "method" paragraph, the
  block-wise equation for ``A_ij`` and ``o_i``; block tables per wywy.jp
  Keyword "Block table" and ricepunchb.github.io section 3.2.
* :func:`write_kv` -- wywy.jp Keyword "autoregressive generation phase" and
  "KV cache manager" (next free position of the last block).
* :func:`copy_blocks` -- wywy.jp WHERE, parallel-sampling copy-on-write
  example; zhaifeiyue memory-management table, "Copy-on-Write".
* :func:`prefill` -- wywy.jp Keyword "prompt phase" and WHERE, shared prefix
  (a cached prefix's KV is reused; only the new tokens are queries); each
  query attends causally over the context up to its own position.
* :func:`swap_blocks` -- wywy.jp Keyword "Swapping" and Overview,
  scheduling and preemption (every block of an evicted sequence goes to CPU
  memory and comes back whole); zhaifeiyue "Scheduling & Preemption" table,
  row "Swap".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

F16 = 0
F32 = 1

_STATUS = {0: "ok", -1: "bad argument", -2: "block table entry out of range",
           -3: "bad or repeated slot", -4: "bad copy pairs"}


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` with gcc (no fast-math, no intrinsics)."""
    if not force and os.path.exists(LIBRARY):
        return LIBRARY
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
           "-o", tmp, SOURCE, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def _bind(lib):
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_half_to_double_array.argtypes = [vp, vp, i64]
    lib.oracle_half_to_double_array.restype = None
    lib.oracle_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                  f32, i32, vp, i32, vp, i32, i32]
    lib.oracle_decode.restype = i32
    lib.oracle_write_kv.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32]
    lib.oracle_write_kv.restype = i32
    lib.oracle_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32]
    lib.oracle_copy_blocks.restype = i32
    lib.oracle_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                   f32, i32, i32]
    lib.oracle_prefill.restype = i32
    lib.oracle_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32]
    lib.oracle_swap_blocks.restype = i32
    lib.oracle_threads_available.argtypes = []
    lib.oracle_threads_available.restype = i32
    return lib


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            build()
        _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float16:
        return F16
    if arr.dtype == np.float32:
        return F32
    raise OracleError(f"unsupported element type {arr.dtype}")


def _ptr(arr):
    return None if arr is None else arr.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {_STATUS.get(rc, rc)}")


def threads_available(_lib_=None) -> int:
    return int((_lib_ or _load()).oracle_threads_available())


def half_to_double(bits: np.ndarray, _lib_=None) -> np.ndarray:
    """Decode uint16 binary16 bit patterns to float64 with the oracle's own decoder."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    (_lib_ or _load()).oracle_half_to_double_array(_ptr(bits), _ptr(out), bits.size)
    return out


def decode(q, k_pool, v_pool, block_tables, context_lens, scale, *,
           pairs=None, return_weights=False, threads=0, _lib_=None):
    """fp64 paged decode attention.

    q: [N][H][D]; pools: [NB][H][B][D] (float16 or float32, same type as q);
    block_tables: int32 [N][MB]; context_lens: int32 [N]; scale: fp32 value.
    pairs: optional int array [P][2] of (b, h) to compute; other rows of the
    result stay NaN.  Returns float64 [N][H][D] (and weights [N][H][max ctx]
    when asked, NaN past each context).
    """
    q = np.ascontiguousarray(q)
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    dt = _dtype_code(q)
    if _dtype_code(k_pool) != dt or _dtype_code(v_pool) != dt:
        raise OracleError("q, k_pool and v_pool must share one element type")
    N, H, D = q.shape
    NB, H2, B, D2 = k_pool.shape
    if (H2, D2) != (H, D) or v_pool.shape != k_pool.shape:
        raise OracleError("pool shape does not match q")
    MB = tables.shape[1] if tables.ndim == 2 else 0
    if tables.shape[0] != N or ctx.shape != (N,):
        raise OracleError("block_tables / context_lens do not match the batch")
    out = np.full((N, H, D), np.nan, dtype=np.float64)
    pair_arr = None
    npairs = 0
    if pairs is not None:
        pair_arr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        npairs = pair_arr.shape[0]
    w = None
    wstride = 0
    if return_weights:
        wstride = max(int(ctx.max()) if N else 0, 1)
        w = np.full((N, H, wstride), np.nan, dtype=np.float64)
    rc = (_lib_ or _load()).oracle_decode(_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(tables),
                               _ptr(ctx), N, H, D, B, NB, MB, float(np.float32(scale)), dt,
                               _ptr(pair_arr), npairs, _ptr(w), wstride, int(threads))
    _check(rc, "oracle decode")
    return (out, w) if return_weights else out


def write_kv(key, value, k_pool, v_pool, slot_mapping, _lib_=None):
    """Scatter key/value [T][H][D] into the pools in place (bit copies)."""
    key = np.ascontiguousarray(key)
    value = np.ascontiguousarray(value)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    for p in (k_pool, v_pool):
        if not p.flags.c_contiguous:
            raise OracleError("pools must be C-contiguous (written in place)")
    dt = _dtype_code(key)
    T, H, D = key.shape
    NB, _, B, _ = k_pool.shape
    rc = (_lib_ or _load()).oracle_write_kv(_ptr(key), _ptr(value), _ptr(k_pool), _ptr(v_pool), _ptr(slots),
                                 T, H, D, B, NB, dt)
    _check(rc, "oracle write_kv")


def copy_blocks(k_pool, v_pool, block_mapping, _lib_=None):
    """Copy whole physical blocks src -> dst in both pools, in place."""
    pairs = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
    for p in (k_pool, v_pool):
        if not p.flags.c_contiguous:
            raise OracleError("pools must be C-contiguous (written in place)")
    NB, H, B, D = k_pool.shape
    rc = (_lib_ or _load()).oracle_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(pairs), pairs.shape[0],
                                    H, D, B, NB, _dtype_code(k_pool))
    _check(rc, "oracle copy_blocks")


def prefill(q, k_pool, v_pool, block_tables, context_lens, query_start, scale, *, threads=0,
            _lib_=None):
    """fp64 paged prefill attention (causal).

    q: [T][H][D] query rows of all sequences back to back; query_start: int
    [N+1] row offsets; sequence b's rows are the last query_start[b+1] -
    query_start[b] tokens of its context_lens[b]-token context.  Returns
    float64 [T][H][D].
    """
    q = np.ascontiguousarray(q)
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    dt = _dtype_code(q)
    if _dtype_code(k_pool) != dt or _dtype_code(v_pool) != dt:
        raise OracleError("q, k_pool and v_pool must share one element type")
    T, H, D = q.shape
    NB, H2, B, D2 = k_pool.shape
    N = ctx.shape[0]
    if (H2, D2) != (H, D) or v_pool.shape != k_pool.shape:
        raise OracleError("pool shape does not match q")
    if qs.shape != (N + 1,) or int(qs[-1]) != T or tables.shape[0] != N:
        raise OracleError("query_start / block_tables do not match the batch")
    MB = tables.shape[1] if tables.ndim == 2 else 0
    out = np.full((T, H, D), np.nan, dtype=np.float64)
    rc = (_lib_ or _load()).oracle_prefill(_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                           _ptr(tables), _ptr(ctx), _ptr(qs), N, H, D, B, NB,
                                           MB, float(np.float32(scale)), dt, int(threads))
    _check(rc, "oracle prefill")
    return out


def swap_blocks(dst_k, dst_v, src_k, src_v, block_mapping, _lib_=None):
    """Copy block src of the source pools onto block dst of the destination
    pools for every (src, dst) pair, K and V (swap out or in)."""
    pairs = np.ascontiguousarray(np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2))
    for p in (dst_k, dst_v):
        if not p.flags.c_contiguous:
            raise OracleError("destination pools must be C-contiguous (written in place)")
    src_k = np.ascontiguousarray(src_k)
    src_v = np.ascontiguousarray(src_v)
    sNB, H, B, D = src_k.shape
    dNB = dst_k.shape[0]
    if dst_k.shape[1:] != (H, B, D) or src_v.shape != src_k.shape or dst_v.shape != dst_k.shape:
        raise OracleError("pools differ in block shape")
    dt = _dtype_code(src_k)
    if _dtype_code(dst_k) != dt:
        raise OracleError("pools differ in element type")
    rc = (_lib_ or _load()).oracle_swap_blocks(_ptr(dst_k), _ptr(dst_v), _ptr(src_k), _ptr(src_v),
                                               _ptr(pairs), pairs.shape[0], H, D, B, sNB, dNB, dt)
    _check(rc, "oracle swap_blocks")


class Oracle:
    """The same functions bound to another build of the oracle source (the
    tests use it to check that their pins catch planted mistakes)."""

    OracleError = OracleError

    def __init__(self, library_path: str):
        self._lib = _bind(ctypes.CDLL(library_path))

    def half_to_double(self, bits):
        return half_to_double(bits, _lib_=self._lib)

    def decode(self, *args, **kw):
        return decode(*args, _lib_=self._lib, **kw)

    def write_kv(self, *args):
        return write_kv(*args, _lib_=self._lib)

    def copy_blocks(self, *args):
        return copy_blocks(*args, _lib_=self._lib)

    def swap_blocks(self, *args):
        return swap_blocks(*args, _lib_=self._lib)

    def prefill(self, *args, **kw):
        return prefill(*args, _lib_=self._lib, **kw)

    def threads_available(self):
        return threads_available(_lib_=self._lib)
