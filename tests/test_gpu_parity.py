"""GPU parity: the HIP kernels behind the C ABI against the CPU oracle on the
same seeded inputs.

Bars: bit-exact for pa_write_kv, pa_copy_blocks and every address (pools
compared as raw bits); pa_decode elementwise within
|gpu - oracle| <= 2e-3 + 1e-2 |oracle| for fp16 K/V and <= 1e-5 for fp32.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

F16_ABS, F16_REL, F32_ABS = 2e-3, 1e-2, 1e-5


def announce(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


def tbits(t):
    return bits(t.cpu().numpy())


def assert_close(gpu, ref, dtype, where=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    if dtype == W.F16:
        bound = F16_ABS + F16_REL * np.abs(ref)
    else:
        bound = np.full_like(ref, F32_ABS)
    bad = ~(err <= bound)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {bad.sum()} elements out of tolerance; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} oracle={ref[tuple(i)]!r}")


def gpu_decode(pa, wl, k, v, device, partition_size=0, ctx=None, tables=None, workspace=None,
               host_ctx=None):
    ctx = wl.context_lens if ctx is None else ctx
    tables = wl.block_tables if tables is None else tables
    N, H, D = wl.q.shape
    q = dev(wl.q, device)
    out = torch.empty_like(q)
    maxctx = int(max(int(np.max(ctx)) if len(ctx) else 0, 1))
    if workspace is None:
        workspace = pa.new_workspace(N, H, D, maxctx, partition_size, device=device)
    if host_ctx is not None:
        maxctx = max(maxctx, int(np.max(host_ctx)))
        workspace = pa.new_workspace(N, H, D, maxctx, partition_size, device=device)
    pa.pa_decode(out, q, k, v, dev(tables, device), dev(ctx, device), float(wl.scale), maxctx,
                 partition_size=partition_size, workspace=workspace, host_context_lens=host_ctx)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_decode(oracle, wl, k=None, v=None, **kw):
    k = wl.k_pool if k is None else k
    v = wl.v_pool if v is None else v
    return oracle.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale, **kw)


@functools.lru_cache(maxsize=None)
def cached(key):
    name, kw = key[0], dict(key[1:])
    return W.make(name, **kw)


def workload(name, **kw):
    return cached((name,) + tuple(sorted(kw.items())))


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def step_on_gpu(pa, wl, device):
    """Pools before the step -> copy-on-write copies -> token writes, on the GPU."""
    k = dev(wl.k_pool_pre, device)
    v = dev(wl.v_pool_pre, device)
    if len(wl.block_mapping):
        pa.pa_copy_blocks(k, v, dev(wl.block_mapping, device))
    pa.pa_write_kv(dev(wl.new_key, device), dev(wl.new_value, device), k, v,
                   dev(wl.slot_mapping, device))
    torch.cuda.synchronize()
    return k, v


def step_on_oracle(oracle, wl):
    k, v = wl.k_pool_pre.copy(), wl.v_pool_pre.copy()
    oracle.copy_blocks(k, v, wl.block_mapping)
    oracle.write_kv(wl.new_key, wl.new_value, k, v, wl.slot_mapping)
    return k, v


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("opt13b", {}),
    ("short", {"block_size": 16}),
    ("cow", {}),
], ids=["tiny-fp32", "opt13b", "short", "cow"])
def test_step_then_decode(pa, oracle_lib, device, name, kw):
    wl = workload(name, **kw)
    announce(f"{wl.name}: N={wl.num_seqs} H={wl.num_heads} D={wl.head_dim} B={wl.block_size} "
             f"NB={wl.num_blocks} pairs={len(wl.block_mapping)} tokens={len(wl.slot_mapping)}")
    k, v = step_on_gpu(pa, wl, device)
    ok, ov = step_on_oracle(oracle_lib, wl)
    assert np.array_equal(tbits(k), bits(ok)), "K pool after copy+write differs"
    assert np.array_equal(tbits(v), bits(ov)), "V pool after copy+write differs"
    announce(f"{wl.name}: pa_decode")
    got = gpu_decode(pa, wl, k, v, device)
    ref = oracle_decode(oracle_lib, wl, ok, ov)
    assert_close(got, ref, wl.dtype, wl.name)
    one = np.flatnonzero(wl.context_lens == 1)
    for b in one:  # a single token returns its V row exactly
        assert np.array_equal(bits(got[b]), bits(wl.logical_v[b][0]))


@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_block_size_sweep(pa, oracle_lib, device, B):
    """The short-row sweep: same sequences and logical K/V for B = 8..64; every B
    matches the oracle and the GPU output is bit-identical across B (the
    kernel's summation order depends on logical positions only)."""
    wl = workload("short", block_size=B)
    announce(f"{wl.name}: N={wl.num_seqs} B={B}")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device)
    assert_close(got, oracle_decode(oracle_lib, wl), wl.dtype, wl.name)
    base = workload("short", block_size=16)
    if B != 16:
        ref = gpu_decode(pa, base, dev(base.k_pool, device), dev(base.v_pool, device), device)
        assert np.array_equal(bits(got), bits(ref))


def test_long_context_every_row(pa, oracle_lib, device):
    """OPT-175B layer shape, all 96 heads, contexts 4K-16K (device-filled
    pools): every (sequence, head) row of four launches against the oracle --
    the bench's fused step (pa_decode_append, host-planned), then pa_decode
    on the pools it wrote through the grid launch (default partition 4096,
    merged), the host-planned list (partition planned from the lengths) and
    the grid at partition 1024.  The oracle runs per sequence on that
    sequence's blocks, copied to the host one sequence at a time."""
    wl = W.long_context(host=False)
    N, H, D = wl.q.shape
    announce(f"{wl.name}: N={N} H={H} NB={wl.num_blocks} filling pools")
    k, v = W.device_pools(wl, device)
    q, tables, ctx = dev(wl.q, device), dev(wl.block_tables, device), dev(wl.context_lens, device)
    maxctx = wl.max_context_len
    scale = float(wl.scale)
    outs = {}
    announce(f"{wl.name}: fused step, host-planned")
    ws = pa.new_workspace(N, H, D, maxctx, 256, device=device)
    o = torch.empty_like(q)
    pa.pa_decode_append(o, q, dev(wl.new_key, device), dev(wl.new_value, device), k, v, tables,
                        ctx, dev(wl.slot_mapping, device), scale, maxctx, 0, ws,
                        host_context_lens=wl.context_lens)
    outs["fused listed"] = o
    for name, part, host in (("grid default", 0, None), ("listed", 0, wl.context_lens),
                             ("grid 1024", 1024, None)):
        announce(f"{wl.name}: pa_decode {name}")
        o = torch.empty_like(q)
        w = pa.new_workspace(N, H, D, maxctx, part if host is None else 256, device=device)
        pa.pa_decode(o, q, k, v, tables, ctx, scale, maxctx, partition_size=part, workspace=w,
                     host_context_lens=host)
        outs[name] = o
    torch.cuda.synchronize()
    got = {name: o.cpu().numpy() for name, o in outs.items()}
    for b in range(N):
        n = int(wl.context_lens[b])
        nblk = -(-n // wl.block_size)
        idx = torch.as_tensor(wl.block_tables[b, :nblk].astype(np.int64), device=device)
        kb, vb = k[idx].cpu().numpy(), v[idx].cpu().numpy()
        ref = oracle_lib.decode(wl.q[b:b + 1], kb, vb, np.arange(nblk, dtype=np.int32)[None],
                                wl.context_lens[b:b + 1], wl.scale)
        for name, g in got.items():
            assert_close(g[b:b + 1], ref, wl.dtype, f"{wl.name} {name} sequence {b} ctx={n}")
        if b % 8 == 7:
            announce(f"{wl.name}: {b + 1} of {N} sequences match the oracle on every head")
    del k, v
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# partitions, invariances, edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("part", [16, 48, 128, 256, 512, 1024, 4096])
def test_partition_sizes(pa, oracle_lib, device, part):
    wl = workload("opt13b", num_seqs=24, num_heads=8)
    announce(f"{wl.name} small: partition {part}")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device,
                     partition_size=part)
    assert_close(got, oracle_decode(oracle_lib, wl), wl.dtype, f"partition {part}")


def test_placement_invariance_bit_identical(pa, device):
    wl = workload("opt13b", num_seqs=24, num_heads=8)
    ref = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device)
    for s in range(2):
        r = W.relayout(wl, s)
        announce(f"relayout {s}")
        got = gpu_decode(pa, r, dev(r.k_pool, device), dev(r.v_pool, device), device)
        assert np.array_equal(bits(got), bits(ref))


def test_shared_prefix_bit_identical_to_private_copies(pa, device):
    wl = workload("cow", num_prompts=6, samples=6, num_heads=4)
    ref = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device)
    r = W.relayout(wl, 9)
    got = gpu_decode(pa, r, dev(r.k_pool, device), dev(r.v_pool, device), device)
    assert np.array_equal(bits(got), bits(ref))


EDGE_CTX = [1, 2, 3, 4, 5, 15, 16, 17, 31, 33, 63, 64, 65, 255, 256, 257, 511, 777]


@pytest.mark.parametrize("dtype,D,B", [(W.F16, 128, 16), (W.F16, 128, 8), (W.F16, 64, 64),
                                       (W.F16, 64, 8), (W.F32, 64, 16), (W.F32, 128, 32),
                                       (W.F32, 128, 8), (W.F16, 128, 32)])
@pytest.mark.parametrize("part", [0, 64])
def test_edge_contexts(pa, oracle_lib, device, dtype, D, B, part):
    H = 3
    wl = W._simple(f"edge-{dtype}-D{D}-B{B}", 77, dtype, H, D, B, EDGE_CTX)
    announce(f"{wl.name} part={part}")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device,
                     partition_size=part)
    ref = oracle_decode(oracle_lib, wl)
    assert_close(got, ref, dtype, wl.name)
    assert np.array_equal(bits(got[0]), bits(wl.logical_v[0][0]))  # ctx 1 -> V exactly
    assert np.isfinite(got).all()                                     # NaN in unused slots never leaks


def test_zero_context_and_max_context(pa, oracle_lib, device):
    B, MB = 16, 6
    wl = W._simple("zero-max", 5, W.F16, 2, 128, B, [5, MB * B, 1, MB * B], MB=MB)
    ctx = wl.context_lens.copy()
    ctx[2] = 0
    announce("zero and max contexts")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device, ctx=ctx,
                     partition_size=32)
    ref = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, ctx, wl.scale)
    assert np.array_equal(got[2], np.zeros_like(got[2]))
    assert_close(got, ref, W.F16, "zero/max")


def test_out_of_range_table_entry_poisons_only_its_row(pa, oracle_lib, device):
    wl = workload("opt13b", num_seqs=24, num_heads=8)
    tables = wl.block_tables.copy()
    victim = int(np.argmax(wl.context_lens))
    tables[victim, 1] = wl.num_blocks + 1000  # outside the pool: the kernel must not read it
    announce("out-of-range table entry")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device, tables=tables,
                     partition_size=64)
    assert np.isnan(got[victim].astype(np.float32)).all()
    others = [b for b in range(wl.num_seqs) if b != victim]
    ref = oracle_decode(oracle_lib, wl)
    assert_close(got[others], ref[others], wl.dtype, "other rows")


def test_workspace_contents_ignored_and_reused(pa, oracle_lib, device):
    """Workspace contents on entry do not matter: one buffer, filled with NaN
    bit patterns between calls, serves calls of different batch shapes."""
    big = workload("opt13b", num_seqs=24, num_heads=8)
    small = workload("short", block_size=16, num_seqs=12, num_heads=4)
    n = pa.pa_decode_workspace_bytes(big.num_seqs, big.num_heads, 128, big.max_context_len, 32)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    kb, vb = dev(big.k_pool, device), dev(big.v_pool, device)
    ks, vs = dev(small.k_pool, device), dev(small.v_pool, device)
    ref_big, ref_small = oracle_decode(oracle_lib, big), oracle_decode(oracle_lib, small)
    announce("workspace contents ignored")
    for fill in (0xFF, 0x7F, 0x00):
        ws.fill_(fill)
        a = gpu_decode(pa, big, kb, vb, device, partition_size=32, workspace=ws)
        assert_close(a, ref_big, big.dtype, f"big after fill {fill:#x}")
        b = gpu_decode(pa, small, ks, vs, device, partition_size=32, workspace=ws)
        assert_close(b, ref_small, small.dtype, f"small after fill {fill:#x}")


def test_large_batch(pa, oracle_lib, device):
    """A batch of 1100 short sequences."""
    ctx = np.random.default_rng(8).integers(1, 90, size=1100)
    wl = W._simple("many-seqs", 8, W.F16, 2, 64, 16, ctx)
    announce(f"large batch: N={wl.num_seqs}")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device,
                     partition_size=32)
    assert_close(got, oracle_decode(oracle_lib, wl), wl.dtype, "large batch")


@pytest.mark.parametrize("dtype,D,B", [(W.F16, 128, 16), (W.F32, 64, 8), (W.F16, 64, 64),
                                       (W.F32, 128, 32)])
def test_write_and_copy_random_bits(pa, oracle_lib, device, dtype, D, B):
    """Pools and rows of random bit patterns (NaN payloads, -0, infinities):
    writes (with padding slots) and copies move bits exactly."""
    rng = np.random.default_rng(D + B)
    H, NB, T = 3, 40, 25
    u = np.uint16 if dtype == W.F16 else np.uint32
    npd = W.NP_DTYPES[dtype]
    info = np.iinfo(u)
    rb = lambda shape: rng.integers(0, info.max, size=shape, dtype=u, endpoint=True).view(npd)
    k0, v0 = rb((NB, H, B, D)), rb((NB, H, B, D))
    key, val = rb((T, H, D)), rb((T, H, D))
    slots = rng.choice(NB * B, size=T, replace=False).astype(np.int64)
    slots[::7] = -1                                   # padding tokens are skipped
    pairs = np.array([[3, 10], [3, 11], [5, 12], [39, 0]], np.int64)
    announce(f"write/copy random bits {dtype} D{D} B{B}")
    k, v = dev(k0, device), dev(v0, device)
    pa.pa_copy_blocks(k, v, dev(pairs, device))
    pa.pa_write_kv(dev(key, device), dev(val, device), k, v, dev(slots, device))
    torch.cuda.synchronize()
    ok, ov = k0.copy(), v0.copy()
    oracle_lib.copy_blocks(ok, ov, pairs)
    oracle_lib.write_kv(key, val, ok, ov, slots)
    assert np.array_equal(tbits(k), bits(ok))
    assert np.array_equal(tbits(v), bits(ov))


def test_write_skips_slots_outside_pool(pa, oracle_lib, device):
    H, D, B, NB = 2, 128, 16, 8
    rng = np.random.default_rng(4)
    k0 = rng.standard_normal((NB, H, B, D)).astype(np.float16)
    key = rng.standard_normal((3, H, D)).astype(np.float16)
    slots = np.array([5, NB * B, 7], np.int64)        # the middle one is outside the pool
    k, v = dev(k0, device), dev(k0, device)
    announce("write with an out-of-pool slot")
    pa.pa_write_kv(dev(key, device), dev(key, device), k, v, dev(slots, device))
    torch.cuda.synchronize()
    ok, ov = k0.copy(), k0.copy()
    oracle_lib.write_kv(key[[0, 2]], key[[0, 2]], ok, ov, slots[[0, 2]])
    assert np.array_equal(tbits(k), bits(ok)) and np.array_equal(tbits(v), bits(ov))


def planned_waves(ctx, part, block_size):
    """The planner's waves per workgroup: 4 when the mean (sequence,
    partition) item is shorter than 12 tiles of 16 tokens, else 8."""
    items = sum(1 if c == 0 else -(-int(c) // part) for c in ctx)
    return 8 if items * 12 * 16 <= int(np.sum(ctx)) else 4


def grid_waves(wl):
    """The unplanned grid launch's waves per workgroup: 4 when the bound
    max_context_len that gpu_decode passes (the longest row) is at most 256
    tokens, else 8."""
    return 4 if int(np.max(wl.context_lens)) <= 256 else 8


@pytest.mark.parametrize("name,kw,part", [
    ("tiny", {}, 16), ("tiny", {}, 0), ("opt13b", {}, 0), ("opt13b", {}, 256), ("opt13b", {}, 1024), ("short", {"block_size": 8}, 0),
    ("short", {"block_size": 32}, 64), ("cow", {}, 0), ("cow", {}, 128),
    ("opt13b", {"num_seqs": 24, "num_heads": 8}, 48), ("opt13b", {"num_seqs": 3, "num_heads": 2}, 0),
], ids=["tiny-p16", "tiny-auto", "opt13b-auto", "opt13b-p256", "opt13b-p1024", "short-b8-auto",
        "short-b32-p64", "cow-auto", "cow-p128", "opt13b-small-p48", "opt13b-tiny-auto"])
def test_host_planned_launch(pa, oracle_lib, device, name, kw, part):
    """With host-side context lengths the library launches only the non-empty
    (sequence, partition) items, long ones first.  With an explicit partition
    size and 8-wave workgroups on both sides (the plan keeps 8, and the
    unplanned grid keeps 8 because some row is longer than 256 tokens) the
    results are bit-identical to the unplanned launch (same per-partition
    reduction order); with partition_size 0 the library also picks the
    partition size from the lengths."""
    wl = workload(name, **kw)
    k, v = dev(wl.k_pool, device), dev(wl.v_pool, device)
    announce(f"{wl.name}: planned vs unplanned, partition {part}")
    plain = gpu_decode(pa, wl, k, v, device, partition_size=part)
    planned = gpu_decode(pa, wl, k, v, device, partition_size=part, host_ctx=wl.context_lens)
    if part and planned_waves(wl.context_lens, part, wl.block_size) == 8 and grid_waves(wl) == 8:
        assert np.array_equal(bits(planned), bits(plain))
    assert_close(planned, oracle_decode(oracle_lib, wl), wl.dtype, wl.name)


@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_short_rows_use_fewer_waves(pa, oracle_lib, device, B):
    """Batches of short rows (mean item under 192 tokens) run the planned
    launch with 4 waves per workgroup: oracle parity at every
    block size, fp16 and fp32, including one-token rows and ragged tails."""
    for dtype in (W.F16, W.F32):
        ctx = np.random.default_rng(40 + B).integers(1, 180, size=96)
        ctx[:3] = (1, 2, 17)
        wl = W._simple(f"short-rows-b{B}", 40 + B, dtype, 8, 128 if dtype == W.F16 else 64, B, ctx)
        assert planned_waves(ctx, 4096, B) == 4
        announce(f"{wl.name} {dtype}: planned short-row launch")
        got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device,
                         host_ctx=wl.context_lens)
        assert_close(got, oracle_decode(oracle_lib, wl), wl.dtype, wl.name)


def test_host_lengths_as_upper_bound(pa, oracle_lib, device):
    """Host lengths may exceed the device ones (the extra items find nothing
    to do); empty sequences still get zero rows."""
    wl = workload("opt13b", num_seqs=24, num_heads=8)
    ctx = wl.context_lens.copy()
    ctx[[3, 7]] = 0
    host = np.minimum(ctx + np.random.default_rng(2).integers(0, 300, size=len(ctx)),
                      wl.max_blocks_per_seq * wl.block_size).astype(np.int32)
    announce("host lengths as upper bound")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device, ctx=ctx,
                     partition_size=64, host_ctx=host)
    ref = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, ctx, wl.scale)
    assert np.array_equal(got[[3, 7]], np.zeros_like(got[[3, 7]]))
    assert_close(got, ref, wl.dtype, "upper-bound host lengths")


def test_host_plan_over_capacity_falls_back(pa, oracle_lib, device):
    """More work items than one launch can list (960) use the unplanned grid."""
    ctx = np.random.default_rng(9).integers(1, 90, size=1100)
    wl = W._simple("many-seqs-planned", 9, W.F16, 2, 64, 16, ctx)
    announce("planned launch over capacity")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device,
                     partition_size=32, host_ctx=wl.context_lens)
    assert_close(got, oracle_decode(oracle_lib, wl), wl.dtype, "over capacity")


def test_nondefault_stream(pa, oracle_lib, device):
    wl = workload("tiny")
    s = torch.cuda.Stream()
    k, v = dev(wl.k_pool, device), dev(wl.v_pool, device)
    q = dev(wl.q, device)
    out = torch.empty_like(q)
    tabs, ctx = dev(wl.block_tables, device), dev(wl.context_lens, device)
    ws = pa.new_workspace(wl.num_seqs, wl.num_heads, wl.head_dim, wl.max_context_len,
                          device=device)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        pa.pa_decode(out, q, k, v, tabs, ctx, float(wl.scale), wl.max_context_len, workspace=ws)
    s.synchronize()
    assert_close(out.cpu().numpy(), oracle_decode(oracle_lib, wl), wl.dtype, "stream")


def test_pending_runtime_error_is_not_taken_for_the_launch(pa, oracle_lib, device):
    """An error an earlier HIP call left pending on the thread (here
    hipGetDevice(NULL): hipErrorInvalidValue, no side effect) does not make
    the next launch report failure; pa_last_error names it.  The C entry
    point is called directly so that no other HIP call comes in between."""
    import ctypes
    runtimes = pa.hip_runtimes()
    assert len(runtimes) == 1
    hip = ctypes.CDLL(runtimes[0])
    hip.hipGetDevice.argtypes = [ctypes.c_void_p]
    wl = workload("tiny")
    k, v = dev(wl.k_pool_pre, device), dev(wl.v_pool_pre, device)
    key, val = dev(wl.new_key, device), dev(wl.new_value, device)
    slots = dev(wl.slot_mapping, device)
    stream = torch.cuda.current_stream().cuda_stream
    T, H, D = wl.new_key.shape
    NB, _, B, _ = wl.k_pool_pre.shape
    dt = pa.PA_F16 if wl.dtype == W.F16 else pa.PA_F32
    lib = pa.library()
    torch.cuda.synchronize()
    assert hip.hipGetDevice(None) != 0          # leaves the error pending
    rc = lib.pa_write_kv(key.data_ptr(), val.data_ptr(), k.data_ptr(), v.data_ptr(),
                         slots.data_ptr(), T, H, D, B, NB, dt, stream)
    assert rc == pa.PA_OK, pa.pa_last_error()
    assert "hipErrorInvalidValue" in pa.pa_last_error()
    torch.cuda.synchronize()
    ref_k, ref_v = wl.k_pool_pre.copy(), wl.v_pool_pre.copy()
    oracle_lib.write_kv(wl.new_key, wl.new_value, ref_k, ref_v, wl.slot_mapping)
    assert np.array_equal(tbits(k), bits(ref_k)) and np.array_equal(tbits(v), bits(ref_v))


# ---------------------------------------------------------------------------
# pa_decode_append: the fused step, bit for bit pa_write_kv + pa_decode
# ---------------------------------------------------------------------------

def fused_and_split(pa, wl, device, partition_size=0, host=False, ctx=None, slots=None):
    """(fused pools, fused out, split pools, split out) after the step's
    copies, from the same pools before the step."""
    ctx = wl.context_lens if ctx is None else ctx
    slots = wl.slot_mapping if slots is None else slots
    N, H, D = wl.q.shape
    maxctx = max(int(np.max(ctx)), 1)
    host_ctx = ctx if host else None
    res = []
    for fused in (True, False):
        k, v = dev(wl.k_pool_pre, device), dev(wl.v_pool_pre, device)
        if len(wl.block_mapping):
            pa.pa_copy_blocks(k, v, dev(wl.block_mapping, device))
        q, out = dev(wl.q, device), torch.full((N, H, D), float("nan"), device=device,
                                                dtype=k.dtype)
        ws = pa.new_workspace(N, H, D, maxctx, partition_size or 256, device=device)
        args = (dev(wl.block_tables, device), dev(ctx, device))
        nk, nv, sl = dev(wl.new_key, device), dev(wl.new_value, device), dev(slots, device)
        if fused:
            pa.pa_decode_append(out, q, nk, nv, k, v, *args, sl, float(wl.scale), maxctx,
                                partition_size, ws, host_context_lens=host_ctx)
        else:
            pa.pa_write_kv(nk, nv, k, v, sl)
            pa.pa_decode(out, q, k, v, *args, float(wl.scale), maxctx, partition_size, ws,
                         host_context_lens=host_ctx)
        torch.cuda.synchronize()
        res += [(tbits(k), tbits(v)), tbits(out)]
    return res


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("opt13b", {}), ("short", {"block_size": 8}),
                                       ("short", {"block_size": 64})],
                         ids=["tiny", "opt13b", "short-b8", "short-b64"])
@pytest.mark.parametrize("part,host", [(0, False), (0, True), (64, False), (64, True), (16, True)])
def test_decode_append_equals_write_then_decode(pa, oracle_lib, device, name, kw, part, host):
    """The fused step gives the same pools and the same outputs, bit for
    bit, as the write followed by the decode -- with the new token in a
    split partition (64, 16) and in either launch form."""
    wl = workload(name, **kw)
    announce(f"decode_append {wl.name} part={part} host={host}")
    (fk, fv), fo, (sk, sv), so = fused_and_split(pa, wl, device, part, host)
    assert np.array_equal(fk, sk) and np.array_equal(fv, sv)
    assert np.array_equal(fo, so)
    if part == 0 and not host:
        ok, ov = step_on_oracle(oracle_lib, wl)
        assert np.array_equal(fk, bits(ok)) and np.array_equal(fv, bits(ov))
        assert_close(fo.view(wl.q.dtype), oracle_decode(oracle_lib, wl, ok, ov), wl.dtype,
                     "fused vs oracle")


@pytest.mark.parametrize("part,host", [(0, False), (0, True), (16, True), (64, False)])
def test_decode_append_full_last_tile(pa, device, part, host):
    """Contexts that end exactly on a 16-token tile: the tile holding the new
    token is full, and the fused step must still match the write followed by
    the decode bit for bit (pools and outputs)."""
    wl = workload("opt13b")
    ctx = wl.context_lens.copy()
    ctx = np.where(ctx >= 16, ctx // 16 * 16, ctx).astype(ctx.dtype)
    assert np.sum(ctx % 16 == 0) > len(ctx) // 2
    B = wl.block_size
    last = ctx - 1
    slots = (wl.block_tables[np.arange(len(ctx)), last // B].astype(np.int64) * B
             + last % B).astype(np.int64)
    announce(f"decode_append full last tile part={part} host={host}")
    (fk, fv), fo, (sk, sv), so = fused_and_split(pa, wl, device, part, host, ctx=ctx,
                                                 slots=slots)
    assert np.array_equal(fk, sk) and np.array_equal(fv, sv)
    assert np.array_equal(fo, so)


@pytest.mark.parametrize("name,kw", [("opt13b", {"num_seqs": 100}), ("short", {"num_seqs": 70})],
                         ids=["opt13b-100seqs", "short-70seqs"])
def test_decode_append_partial_writer_row(pa, device, name, kw):
    """Batches that do not fill the last writer workgroup of the listed
    launch (100 sequences at 8 waves: 64 + 36; 70 short rows at 4 waves:
    32 + 32 + 6): every new row is still stored, bit for bit as the write
    followed by the decode, and so are the outputs."""
    wl = workload(name, **kw)
    announce(f"decode_append partial writer row {wl.name} N={wl.num_seqs}")
    (fk, fv), fo, (sk, sv), so = fused_and_split(pa, wl, device, host=True)
    assert np.array_equal(fk, sk) and np.array_equal(fv, sv)
    assert np.array_equal(fo, so)


def test_decode_append_over_capacity(pa, device):
    """With more items than one launch can list, the fused step falls back to
    the grid launch, whose owning workgroups store the new rows: still bit
    for bit the write followed by the decode."""
    ctx = np.random.default_rng(19).integers(1, 90, size=1100)
    wl = W._simple("many-seqs-append", 19, W.F16, 2, 64, 16, ctx)
    announce("decode_append over list capacity")
    (fk, fv), fo, (sk, sv), so = fused_and_split(pa, wl, device, partition_size=32, host=True)
    assert np.array_equal(fk, sk) and np.array_equal(fv, sv)
    assert np.array_equal(fo, so)


@pytest.mark.parametrize("host", [True, False], ids=["listed", "grid"])
def test_decode_append_empty_context_still_writes(pa, device, host):
    """A sequence with context 0 gets a zero row and its new token is still
    stored (as pa_write_kv would), in either launch form."""
    announce(f"decode_append empty context host={host}")
    wl = workload("tiny")
    ctx = wl.context_lens.copy()
    ctx[0] = 0
    (fk, fv), fo, (sk, sv), so = fused_and_split(pa, wl, device, host=host, ctx=ctx)
    assert np.array_equal(fk, sk) and np.array_equal(fv, sv)
    assert np.array_equal(fo, so)
    assert not np.any(fo[0].view(wl.q.dtype))


def test_decode_append_skips_slots_outside_pool(pa, device):
    """A slot outside the pool is not written; the attention still uses the
    new row for the last position, which equals the normal step's output."""
    announce("decode_append slot outside pool")
    wl = workload("tiny")
    slots = wl.slot_mapping.copy()
    slots[2] = -1
    (fk, fv), fo, _, _ = fused_and_split(pa, wl, device, slots=slots)
    _, normal, _, _ = fused_and_split(pa, wl, device)
    before_k = tbits(dev(wl.k_pool_pre, device))
    blk, off = divmod(int(wl.slot_mapping[2]), wl.block_size)
    assert np.array_equal(fk[blk, :, off], before_k[blk, :, off])   # not written
    assert np.array_equal(fo, normal)
