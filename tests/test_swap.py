"""Swapping under memory pressure: a group of parallel samples is preempted
all or nothing when the GPU pool runs out, its blocks go to a CPU swap pool
and come back whole when blocks free up (the wywy.jp notes, Keyword
"Swapping", "All-or-nothing eviction", "FCFS" and Overview, scheduling and
preemption; the zhaifeiyue.github.io "Scheduling & Preemption" table).

The driver here is the plainest scheduler those passages describe: groups run
in arrival order; when an append finds too few blocks the latest-arrived
running group is swapped out; at the start of every step the earliest
swapped-out group is swapped back in if its blocks fit.

CPU: the manager decides, the oracle copies, swaps, writes and decodes; every
generated token's output equals fp64 dense attention over its sequence's
history, and equals the output of a run whose pool is large enough never to
preempt.

GPU: the same program through DecodeStepper over two layers (pa_swap_blocks
between device pools and pinned host pools): every output bit-identical to
the never-preempting GPU run at the same partition size, within the decode
tolerance of the oracle, and layer 1 (negated values) the exact negation of
layer 0.  Also pa_swap_blocks alone, bit-exact against the oracle's swap in
both directions, and its refusal of pageable host memory.
"""
import sys

import numpy as np
import pytest

import workloads as W
from test_step_loop import dense_attention

F16_ABS, F16_REL, F32_ABS = 2e-3, 1e-2, 1e-5


@pytest.fixture(scope="module")
def M(pa):
    from paged_kv_cache_05_amd import manager
    return manager


def token_batch(g, seqs, produced):
    parts = [W.token_inputs(g.seed, s, produced[s], g.num_heads, g.head_dim, g.dtype)
             for s in seqs]
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))


def drive(ex, M, m, g):
    """Run every sequence to its length; returns ({(seq, t): out row},
    [("out"|"in", group)])."""
    for gi, ids in enumerate(g.groups):
        p = ids[0]
        m.add(p)
        slots, pairs = m.append([p] * len(g.prompt_keys[gi]))
        assert len(pairs) == 0
        ex.prompt(slots, g.prompt_keys[gi], g.prompt_values[gi])
        for s in ids[1:]:
            m.fork(p, s)
    produced = {s: 0 for ids in g.groups for s in ids}

    def live(gi):
        return [s for s in g.groups[gi] if produced[s] < g.gen_lens[s]]

    running, swapped = list(range(len(g.groups))), []
    record, events = {}, []
    while running or swapped:
        while swapped:
            gi = swapped[0]
            try:
                ex.swap_in(live(gi))
            except M.OutOfBlocks:
                assert running, "nothing runs, yet the earliest swapped group does not fit"
                break
            swapped.pop(0)
            running = sorted(running + [gi])
            events.append(("in", gi))
        while True:
            batch = [s for gi in running for s in live(gi)]
            try:
                plan = ex.plan(batch)
                break
            except M.OutOfBlocks:
                assert len(running) > 1, "the earliest group alone must fit the pool"
                victim = running.pop()
                ex.swap_out(live(victim))
                swapped = sorted(swapped + [victim])
                events.append(("out", victim))
        key, value, q = token_batch(g, batch, produced)
        out = ex.run(plan, key, value, q)
        for j, s in enumerate(batch):
            record[(s, produced[s])] = out[j]
            produced[s] += 1
            if produced[s] == g.gen_lens[s]:
                m.free(s)
        running = [gi for gi in running if live(gi)]
        m.check()
    assert m.num_free == m.num_blocks and m.num_free_host == m.num_host_blocks
    return record, events


class OracleExec:
    """Device work done by the oracle on numpy pools."""

    def __init__(self, oracle, m, g):
        self.o, self.m, self.g = oracle, m, g
        dt = W.NP_DTYPES[g.dtype]
        shape = (g.num_heads, g.block_size, g.head_dim)
        self.k = np.full((m.num_blocks,) + shape, np.nan, dt)
        self.v = np.full((m.num_blocks,) + shape, np.nan, dt)
        self.hk = np.full((max(m.num_host_blocks, 1),) + shape, np.nan, dt)
        self.hv = np.full((max(m.num_host_blocks, 1),) + shape, np.nan, dt)

    def prompt(self, slots, key, value):
        self.o.write_kv(key, value, self.k, self.v, slots)

    def plan(self, seqs):
        slots, pairs = self.m.append(seqs)
        tables, ctx = self.m.tables(seqs, self.g.max_blocks)
        return slots, pairs, tables, ctx

    def run(self, plan, key, value, q):
        slots, pairs, tables, ctx = plan
        self.o.copy_blocks(self.k, self.v, pairs)
        self.o.write_kv(key, value, self.k, self.v, slots)
        return self.o.decode(q, self.k, self.v, tables, ctx, self.g.scale)

    def swap_out(self, seqs):
        self.o.swap_blocks(self.hk, self.hv, self.k, self.v, self.m.swap_out(seqs))

    def swap_in(self, seqs):
        self.o.swap_blocks(self.k, self.v, self.hk, self.hv, self.m.swap_in(seqs))


def history(g, s):
    """Prompt K/V of s's group, then s's generated tokens, as [T][H][D]."""
    gi = next(i for i, ids in enumerate(g.groups) if s in ids)
    ks, vs = [g.prompt_keys[gi]], [g.prompt_values[gi]]
    for t in range(g.gen_lens[s]):
        k, v, _ = W.token_inputs(g.seed, s, t, g.num_heads, g.head_dim, g.dtype)
        ks.append(k[None])
        vs.append(v[None])
    return np.concatenate(ks), np.concatenate(vs)


PROGRAMS = [
    dict(dtype=W.F32, num_heads=2, head_dim=16, block_size=4, prompt_lens=(9, 14, 5, 18),
         samples=2, gen=(6, 20)),
    dict(dtype=W.F16, num_heads=2, head_dim=32, block_size=16),
    dict(dtype=W.F16, num_heads=2, head_dim=16, block_size=8, samples=4, squeeze=0.4, seed=3),
]


@pytest.mark.parametrize("kw", PROGRAMS)
def test_preempted_run_equals_dense_and_unpressed_run(oracle_lib, M, kw):
    g = W.pressure(**kw)
    m = M.BlockManager(g.num_blocks, g.block_size, num_host_blocks=g.num_host_blocks)
    record, events = drive(OracleExec(oracle_lib, m, g), M, m, g)
    assert any(e[0] == "out" for e in events) and any(e[0] == "in" for e in events)
    big = M.BlockManager(4 * g.num_blocks, g.block_size)
    free_run, no_events = drive(OracleExec(oracle_lib, big, g), M, big, g)
    assert no_events == []
    assert record.keys() == free_run.keys()
    for key in record:
        assert np.array_equal(record[key], free_run[key]), key
    prompt_len = {s: len(g.prompt_keys[gi]) for gi, ids in enumerate(g.groups) for s in ids}
    for s in g.gen_lens:
        K, V = history(g, s)
        for t in range(g.gen_lens[s]):
            _, _, q = W.token_inputs(g.seed, s, t, g.num_heads, g.head_dim, g.dtype)
            n = prompt_len[s] + t + 1
            ref = dense_attention(q, K[:n], V[:n], g.scale)
            np.testing.assert_allclose(record[(s, t)], ref, rtol=1e-10, atol=1e-12,
                                       err_msg=f"sequence {s}, token {t}")


# ---------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------

class GpuExec:
    """DecodeStepper over two layers (layer 1: same keys, negated values),
    device pools and pinned host pools, fixed partition size."""

    def __init__(self, pa, M, m, g, device, part):
        import torch
        self.torch, self.pa, self.g, self.device = torch, pa, g, device
        tdt = torch.float16 if g.dtype == W.F16 else torch.float32
        shape = (g.num_heads, g.block_size, g.head_dim)
        pools = [tuple(torch.full((m.num_blocks,) + shape, float("nan"), dtype=tdt,
                                  device=device) for _ in range(2)) for _ in range(2)]
        host = None
        if m.num_host_blocks:
            host = [tuple(torch.full((m.num_host_blocks,) + shape, float("nan"),
                                     dtype=tdt).pin_memory() for _ in range(2))
                    for _ in range(2)]
        self.st = M.DecodeStepper(m, pools, g.max_blocks, part, host_pools=host)

    def to(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a)).to(self.device)

    def prompt(self, slots, key, value):
        d_slots = self.to(slots)
        for sign, (k, v) in zip((1, -1), self.st.pools):
            self.pa.pa_write_kv(self.to(key), self.to(sign * value), k, v, d_slots)

    def plan(self, seqs):
        return self.st.plan(seqs)

    def run(self, plan, key, value, q):
        dq, dk = self.to(q), self.to(key)
        out0 = self.st.layer(plan, 0, dk, self.to(value), dq, float(self.g.scale))
        out1 = self.st.layer(plan, 1, dk, self.to(-value), dq, float(self.g.scale))
        assert self.torch.equal(out1, -out0), "layer 1 is not the negation of layer 0"
        return out0.cpu().numpy()

    def swap_out(self, seqs):
        self.st.swap_out(seqs)

    def swap_in(self, seqs):
        self.st.swap_in(seqs)


# the GPU kernels take head_dim 64 or 128 and block sizes 8..64
GPU_PROGRAMS = [
    dict(dtype=W.F32, num_heads=2, head_dim=64, block_size=8, prompt_lens=(9, 14, 5, 18),
         samples=2, gen=(6, 20)),
    dict(dtype=W.F16, num_heads=2, head_dim=64, block_size=16),
    dict(dtype=W.F16, num_heads=2, head_dim=128, block_size=8, samples=4, squeeze=0.4, seed=3),
    dict(dtype=W.F16, num_heads=8, head_dim=128, block_size=16, prompt_lens=(120, 300, 64, 200),
         samples=3, gen=(30, 90)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("kw", GPU_PROGRAMS)
def test_gpu_preempted_run(oracle_lib, M, pa, device, kw):
    print(f"[gpu] preemption program {kw}", flush=True)
    sys.stdout.flush()
    g = W.pressure(**kw)
    part = 64
    m = M.BlockManager(g.num_blocks, g.block_size, num_host_blocks=g.num_host_blocks)
    record, events = drive(GpuExec(pa, M, m, g, device, part), M, m, g)
    assert any(e[0] == "out" for e in events)
    big = M.BlockManager(4 * g.num_blocks, g.block_size)
    free_run, _ = drive(GpuExec(pa, M, big, g, device, part), M, big, g)
    m2 = M.BlockManager(g.num_blocks, g.block_size, num_host_blocks=g.num_host_blocks)
    ref, ref_events = drive(OracleExec(oracle_lib, m2, g), M, m2, g)
    assert ref_events == events
    view = np.uint16 if g.dtype == W.F16 else np.uint32
    for key in record:
        assert np.array_equal(record[key].view(view), free_run[key].view(view)), key
        want = ref[key]
        bound = F16_ABS + F16_REL * np.abs(want) if g.dtype == W.F16 else F32_ABS
        assert np.all(np.abs(record[key].astype(np.float64) - want) <= bound), key


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,H,B,D", [(W.F16, 40, 16, 128), (W.F32, 2, 8, 64), (W.F16, 4, 1, 64),
                                         (W.F16, 8, 64, 128)])
def test_gpu_swap_blocks_bit_exact(oracle_lib, pa, device, dtype, H, B, D):
    """Device -> pinned host -> device against the oracle's swap, on random
    bit patterns (NaN payloads included); a source listed twice; pairs
    outside either pool are skipped."""
    import torch
    print(f"[gpu] swap blocks {dtype} H{H} B{B} D{D}", flush=True)
    rng = np.random.default_rng(H * 1000 + B)
    NB, HNB = 37, 23
    shape = (H, B, D)
    bits = np.uint16 if dtype == W.F16 else np.uint32
    npdt = W.NP_DTYPES[dtype]

    def randbits(n):
        return rng.integers(0, np.iinfo(bits).max, size=(n,) + shape, dtype=bits,
                            endpoint=True).view(npdt)

    k, v = randbits(NB), randbits(NB)
    hk0, hv0 = randbits(HNB), randbits(HNB)
    out_pairs = np.stack([rng.permutation(NB)[:15], rng.permutation(HNB)[:15]], axis=1)
    out_pairs = np.concatenate([out_pairs, [[out_pairs[0, 0], (out_pairs[:, 1].max() + 1) % HNB]]])
    out_pairs = out_pairs[np.unique(out_pairs[:, 1], return_index=True)[1]]
    tdt = torch.float16 if dtype == W.F16 else torch.float32
    to_dev = lambda a: torch.from_numpy(a).to(device)
    dk, dv = to_dev(k), to_dev(v)
    hk = torch.from_numpy(hk0.copy()).pin_memory()
    hv = torch.from_numpy(hv0.copy()).pin_memory()
    with_skips = np.concatenate([out_pairs, [[NB, 0], [-1, 1], [0, HNB]]])
    pa.pa_swap_blocks(hk, hv, dk, dv, to_dev(with_skips.astype(np.int64)))
    torch.cuda.synchronize()
    ek, ev = hk0.copy(), hv0.copy()
    oracle_lib.swap_blocks(ek, ev, k, v, out_pairs)
    assert np.array_equal(hk.numpy().view(bits), ek.view(bits))
    assert np.array_equal(hv.numpy().view(bits), ev.view(bits))
    # back in, to other device blocks; the mapping itself in pinned memory
    in_pairs = np.stack([out_pairs[:, 1], rng.permutation(NB)[:len(out_pairs)]], axis=1)
    d2k, d2v = to_dev(randbits(NB)), to_dev(randbits(NB))
    before_k, before_v = d2k.cpu().numpy(), d2v.cpu().numpy()
    pa.pa_swap_blocks(d2k, d2v, hk, hv, torch.from_numpy(in_pairs.astype(np.int64)).pin_memory())
    torch.cuda.synchronize()
    oracle_lib.swap_blocks(before_k, before_v, ek, ev, in_pairs)
    assert np.array_equal(d2k.cpu().numpy().view(bits), before_k.view(bits))
    assert np.array_equal(d2v.cpu().numpy().view(bits), before_v.view(bits))
    assert tdt == dk.dtype


@pytest.mark.gpu
def test_gpu_swap_refuses_pageable_memory(pa, device):
    """Pools in pageable host memory are refused before any launch.  The
    mapping lists only pairs outside every pool, so even a launch would
    touch no pool memory."""
    import ctypes
    import torch
    H, B, D, NB = 2, 16, 64, 4
    dk = torch.zeros((NB, H, B, D), dtype=torch.float16, device=device)
    dv = torch.zeros_like(dk)
    host = np.zeros((2, NB, H, B, D), np.float16)       # pageable
    pairs = torch.tensor([[-1, -1]], dtype=torch.int64, device=device)
    lib = pa.library()
    torch.cuda.synchronize()
    rc = lib.pa_swap_blocks(host[0].ctypes.data, host[1].ctypes.data, dk.data_ptr(),
                            dv.data_ptr(), pairs.data_ptr(), 1, H, D, B, NB, NB, pa.PA_F16,
                            torch.cuda.current_stream().cuda_stream)
    assert rc == -3, (rc, pa.pa_last_error())
    assert "dst_k" in pa.pa_last_error()
    with pytest.raises(pa.PAError):
        pa.pa_swap_blocks(torch.from_numpy(host[0]), torch.from_numpy(host[1]), dk, dv, pairs)
    torch.cuda.synchronize()
    del ctypes
