"""pa_decode_noalloc against pa_decode, through the C ABI.

pa_decode_noalloc keeps the partial results of rows that span several
partitions in the library's static device scratch instead of a caller's
workspace.  With the same arguments and partition length it must give the
same output as pa_decode bit for bit, and both must meet the oracle within
the decode tolerance (|gpu - oracle| <= 2e-3 + 1e-2 |oracle| for fp16,
<= 1e-5 for fp32).  Two calls in a row, the second on a smaller batch,
check that the scratch left by the first does not matter; a batch too
large for the scratch is refused before any launch.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


def close(got, ref, dtype):
    got = got.astype(np.float64)
    if dtype == W.F16:
        return bool(np.all(np.abs(got - ref) <= 2e-3 + 1e-2 * np.abs(ref)))
    return bool(np.all(np.abs(got - ref) <= 1e-5))


def c_call(pa, name, wl, out, q, k, v, tables, ctx, part, host, ws=None):
    """One call of pa_decode / pa_decode_noalloc through the C ABI."""
    lib = pa.library()
    N, H, D = wl.q.shape
    dt = pa.PA_F16 if wl.dtype == W.F16 else pa.PA_F32
    h = None if host is None else np.ascontiguousarray(host, dtype=np.int32)
    args = [out.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(), tables.data_ptr(),
            ctx.data_ptr(), N, H, D, wl.block_size, wl.num_blocks, wl.max_blocks_per_seq,
            wl.max_context_len, ctypes.c_float(float(wl.scale)), dt, part,
            None if h is None else h.ctypes.data]
    stream = torch.cuda.current_stream().cuda_stream
    if name == "pa_decode":
        args += [None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel()]
    rc = getattr(lib, name)(*args, stream)
    return rc


def run_pair(pa, oracle_lib, device, wl, part, host):
    """(noalloc output, pa_decode output) on the same inputs."""
    k, v = dev(wl.k_pool, device), dev(wl.v_pool, device)
    q, tables, ctx = dev(wl.q, device), dev(wl.block_tables, device), dev(wl.context_lens, device)
    N, H, D = wl.q.shape
    out_a = torch.full_like(q, float("nan"))
    out_b = torch.full_like(q, float("nan"))
    host_ctx = wl.context_lens if host else None
    rc = c_call(pa, "pa_decode_noalloc", wl, out_a, q, k, v, tables, ctx, part, host_ctx)
    assert rc == pa.PA_OK, (rc, pa.pa_last_error())
    # pa_decode with a workspace of the scratch's size plans the same
    # partition (the planner bounds it by the workspace size)
    ws = torch.empty(pa.PA_NOALLOC_SCRATCH_BYTES, dtype=torch.uint8, device=device)
    ws.fill_(0x7F)
    rc = c_call(pa, "pa_decode", wl, out_b, q, k, v, tables, ctx, part, host_ctx, ws)
    assert rc == pa.PA_OK, (rc, pa.pa_last_error())
    torch.cuda.synchronize()
    return out_a.cpu().numpy(), out_b.cpu().numpy()


CASES = [
    # (workload, kwargs, partition, host lengths): the first of each pair
    # is the larger batch; every case spans several partitions somewhere
    (("opt13b", {"num_seqs": 24, "num_heads": 8}), 64, False),
    (("short", {"num_seqs": 12, "num_heads": 4, "block_size": 16}), 32, False),
    (("opt13b", {"num_seqs": 40, "num_heads": 8}), 0, True),
    (("tiny", {}), 16, True),
]


@pytest.mark.parametrize("first,second", [(0, 1), (2, 3)], ids=["grid", "host-planned"])
def test_noalloc_matches_pa_decode_twice(pa, oracle_lib, device, first, second):
    for i in (first, second):
        (name, kw), part, host = CASES[i]
        wl = W.make(name, **kw)
        announce(f"noalloc {wl.name} N={wl.num_seqs} H={wl.num_heads} partition={part} "
                 f"host={host}")
        got, ref_gpu = run_pair(pa, oracle_lib, device, wl, part, host)
        np_parts = pa.pa_decode_partition_size(
            wl.num_seqs, wl.num_heads, wl.head_dim, wl.max_context_len, part,
            wl.context_lens if host else None, pa.PA_NOALLOC_SCRATCH_BYTES)
        assert -(-wl.max_context_len // np_parts) > 1, "the case must use the scratch"
        assert np.array_equal(bits(got), bits(ref_gpu)), f"{wl.name}: noalloc differs from pa_decode"
        ref = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                                wl.scale)
        assert close(got, ref, wl.dtype), f"{wl.name}: noalloc outside the oracle tolerance"


def test_noalloc_refuses_batches_beyond_the_scratch(pa, device):
    """A batch whose partial results exceed the scratch returns
    PA_ERR_WORKSPACE before any launch, and pa_last_error gives the sizes.
    The output keeps its contents (nothing ran)."""
    wl = W.make("opt13b", num_seqs=24, num_heads=8)
    H, D = wl.num_heads, wl.head_dim
    # 1000 sequences x 8 heads x 32 partitions of 64 tokens: 256,000 rows
    N = 1000
    tables = np.full((N, wl.max_blocks_per_seq), -1, np.int32)
    ctx = np.full(N, 2048, np.int32)
    need_tables = np.resize(np.arange(wl.num_blocks, dtype=np.int32), (N, 128))
    tables[:, :128] = need_tables
    q = torch.zeros((N, H, D), dtype=torch.float16, device=device)
    out = torch.full_like(q, 3.0)
    k, v = dev(wl.k_pool, device), dev(wl.v_pool, device)
    lib = pa.library()
    announce("noalloc over the scratch size")
    rc = lib.pa_decode_noalloc(out.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               dev(tables, device).data_ptr(), dev(ctx, device).data_ptr(), N, H,
                               D, 16, wl.num_blocks, wl.max_blocks_per_seq, 2048,
                               ctypes.c_float(0.088), pa.PA_F16, 64, None,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == -4, rc                                    # PA_ERR_WORKSPACE
    assert "static scratch holds" in pa.pa_last_error()
    torch.cuda.synchronize()
    assert bool((out == 3.0).all().item())


def test_noalloc_replayed_from_a_hip_graph(pa, oracle_lib, device):
    """The callers it is for: pa_decode_noalloc captured into a HIP graph
    (no allocation inside the capture) and replayed three times, with eager
    work and synchronisation between replays; every replay reproduces the
    eager output bit for bit.  The batch spans several partitions, so the
    static scratch carries the partial results."""
    wl = W.make("opt13b", num_seqs=24, num_heads=8)
    k, v = dev(wl.k_pool, device), dev(wl.v_pool, device)
    q, tables, ctx = dev(wl.q, device), dev(wl.block_tables, device), dev(wl.context_lens, device)
    out = torch.full_like(q, float("nan"))

    def call():
        pa.pa_decode_noalloc(out, q, k, v, tables, ctx, float(wl.scale), wl.max_context_len,
                             partition_size=64)

    announce("noalloc eager call before capture")
    call()
    torch.cuda.synchronize()
    eager = out.cpu().numpy()
    ref = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens, wl.scale)
    assert close(eager, ref, wl.dtype)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce("noalloc capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))               # eager work between replays
        torch.cuda.synchronize()
        announce(f"noalloc replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out.cpu().numpy()), bits(eager)), f"replay {r} differs"
