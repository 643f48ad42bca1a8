"""Multi-step generation through the host block manager: parallel sampling
with occasional pruning (workloads.generation) and beam search that forks
and prunes every step (workloads.beam_search).

CPU (no GPU): the manager's slots and copy pairs, executed by the oracle's
copy/write and read by the oracle's decode, give at every step the dense
attention of each sequence's own logical history (prompt + its tokens),
in fp64 -- pins the manager end to end (a missed copy-on-write, a wrong
slot or a block reused while still referenced all change some sequence's
history).  Pools start all-NaN, so a read of a slot that was never written
shows up.

GPU: DecodeStepper (pa_copy_blocks -> pa_write_kv -> pa_decode through the
C ABI) on the same program over two layers' pools: identical slots and
copies, layer-0 pools bit-identical to the oracle's after the run, every
step's layer-0 output within the decode tolerance of the oracle's, and
layer 1 (same keys, negated values) the exact negation of layer 0.
"""
import sys

import numpy as np
import pytest

import workloads as W

F16_ABS, F16_REL, F32_ABS = 2e-3, 1e-2, 1e-5


def nan_pools(g):
    shape = (g.num_blocks, g.num_heads, g.block_size, g.head_dim)
    dt = W.NP_DTYPES[g.dtype]
    return np.full(shape, np.nan, dtype=dt), np.full(shape, np.nan, dtype=dt)


def dense_attention(q, keys, values, scale):
    """softmax(scale * K q) V per head, fp64, over one logical history.
    q [H][D]; keys/values [T][H][D]."""
    q = q.astype(np.float64)
    K = keys.astype(np.float64)
    V = values.astype(np.float64)
    s = np.einsum("thd,hd->ht", K, q) * np.float64(scale)
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=1, keepdims=True)
    return np.einsum("ht,thd->hd", w, V)


def run_oracle(oracle, M, g, dense=True):
    """The program on the CPU: manager decisions, oracle execution."""
    m = M.BlockManager(g.num_blocks, g.block_size)
    k, v = nan_pools(g)
    hist = {}
    for p, (pk, pv) in enumerate(zip(g.prompt_keys, g.prompt_values)):
        m.add(p)
        slots, pairs = m.append([p] * len(pk))
        assert len(pairs) == 0
        oracle.write_kv(pk, pv, k, v, slots)
        hist[p] = (list(pk), list(pv))
    record = []
    for i, st in enumerate(g.steps):
        for s in st.frees:
            m.free(s)
            del hist[s]
        for parent, child in st.forks:
            m.fork(parent, child)
            hist[child] = (list(hist[parent][0]), list(hist[parent][1]))
        slots, pairs = m.append(st.seqs)
        tables, ctx = m.tables(st.seqs, g.max_blocks)
        oracle.copy_blocks(k, v, pairs)
        oracle.write_kv(st.key, st.value, k, v, slots)
        for j, s in enumerate(st.seqs):
            hist[s][0].append(st.key[j])
            hist[s][1].append(st.value[j])
        out = oracle.decode(st.q, k, v, tables, ctx, g.scale)
        assert np.isfinite(out).all(), f"step {i}: a never-written slot was read"
        if dense:
            for j, s in enumerate(st.seqs):
                ref = dense_attention(st.q[j], np.stack(hist[s][0]), np.stack(hist[s][1]),
                                      g.scale)
                np.testing.assert_allclose(out[j], ref, rtol=1e-10, atol=1e-12,
                                           err_msg=f"step {i}, sequence {s}")
        record.append((slots, pairs, tables, ctx, out))
        m.check()
    return record, k, v, m


@pytest.fixture(scope="module")
def M(pa):
    from paged_kv_cache_05_amd import manager
    return manager


@pytest.mark.parametrize("make,kw", [
    ("generation", dict(dtype=W.F32, num_heads=2, head_dim=16, block_size=4)),
    ("generation", dict(dtype=W.F16, num_heads=2, head_dim=32, block_size=16)),
    ("generation", dict(dtype=W.F32, num_heads=1, head_dim=8, block_size=1, steps=12)),
    ("generation", dict(dtype=W.F16, num_heads=2, head_dim=16, block_size=8, churn=0.9, seed=5)),
    ("beam_search", dict(dtype=W.F32, num_heads=2, head_dim=16, block_size=4)),
    ("beam_search", dict(dtype=W.F16, num_heads=2, head_dim=16, block_size=16, width=6,
                         steps=40, spread=2.0, seed=3)),
    ("beam_search", dict(dtype=W.F32, num_heads=1, head_dim=8, block_size=1, width=3, steps=10)),
])
def test_managed_steps_equal_dense_attention(oracle_lib, M, make, kw):
    """Also the beam-search workload: every step each request's beams are
    drawn again from their parents, pruned beams freed, repeated parents
    forked (the wywy.jp notes, WHERE beam search)."""
    g = getattr(W, make)(**kw)
    record, _, _, m = run_oracle(oracle_lib, M, g)
    copies = sum(len(r[1]) for r in record)
    # with B > 1 forks share partly filled blocks, so copy-on-write happens;
    # with B = 1 no block is ever partly filled
    assert (copies > 0) == (g.block_size > 1)
    # sharing only saves: blocks in use <= what private copies would hold
    B = g.block_size
    assert g.num_blocks - m.num_free <= sum(-(-int(c) // B) for c in record[-1][3])


@pytest.mark.gpu
@pytest.mark.parametrize("make,kw", [
    ("generation", dict(dtype=W.F16, num_heads=4, head_dim=128, block_size=16)),
    ("generation", dict(dtype=W.F16, num_heads=4, head_dim=128, block_size=8, churn=0.6, seed=7,
                        steps=40)),
    ("generation", dict(dtype=W.F32, num_heads=2, head_dim=64, block_size=16, seed=9)),
    ("generation", dict(dtype=W.F16, num_heads=8, head_dim=64, block_size=32,
                        prompt_lens=(300, 1, 2, 31, 33), samples=4, steps=20)),
    ("beam_search", dict(dtype=W.F16, num_heads=4, head_dim=128, block_size=16, width=4,
                         steps=48)),
    ("beam_search", dict(dtype=W.F16, num_heads=4, head_dim=64, block_size=8, width=8,
                         steps=40, spread=3.0, seed=4)),
    ("beam_search", dict(dtype=W.F32, num_heads=2, head_dim=128, block_size=32, width=5,
                         prompt_lens=(200, 17, 64), steps=30, seed=6)),
])
def test_decode_stepper_matches_oracle(oracle_lib, M, pa, device, make, kw):
    import torch
    print(f"[gpu] step loop {make} {kw}", flush=True)
    sys.stdout.flush()
    g = getattr(W, make)(**kw)
    record, k_ref, v_ref, _ = run_oracle(oracle_lib, M, g, dense=False)
    tdt = torch.float16 if g.dtype == W.F16 else torch.float32
    shape = (g.num_blocks, g.num_heads, g.block_size, g.head_dim)
    # layer 1 holds the same keys and negated values: its output must be the
    # exact negation of layer 0's (every layer shares the plan, copies included)
    pools = [tuple(torch.full(shape, float("nan"), dtype=tdt, device=device) for _ in range(2))
             for _ in range(2)]
    m = M.BlockManager(g.num_blocks, g.block_size)
    stepper = M.DecodeStepper(m, pools, g.max_blocks)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    for p, (pk, pv) in enumerate(zip(g.prompt_keys, g.prompt_values)):
        m.add(p)
        slots, _ = m.append([p] * len(pk))
        for sign, (kp, vp) in zip((1, -1), pools):
            pa.pa_write_kv(to(pk), to(sign * pv), kp, vp, to(slots))
    for i, (st, ref) in enumerate(zip(g.steps, record)):
        for s in st.frees:
            m.free(s)
        for parent, child in st.forks:
            m.fork(parent, child)
        plan = stepper.plan(st.seqs)
        assert np.array_equal(plan.slots, ref[0]) and np.array_equal(plan.pairs, ref[1])
        q, key = to(st.q), to(st.key)
        out0 = stepper.layer(plan, 0, key, to(st.value), q, float(g.scale))
        out1 = stepper.layer(plan, 1, key, to(-st.value), q, float(g.scale))
        got = out0.cpu().numpy().astype(np.float64)
        want = ref[4]
        if g.dtype == W.F16:
            bound = F16_ABS + F16_REL * np.abs(want)
        else:
            bound = F32_ABS
        bad = ~(np.abs(got - want) <= bound)
        assert not bad.any(), f"step {i}: {bad.sum()} outputs out of tolerance"
        assert torch.equal(out1, -out0), f"step {i}: layer 1 is not the negation of layer 0"
    torch.cuda.synchronize()
    view = np.uint16 if g.dtype == W.F16 else np.uint32
    (k0, v0), (k1, v1) = [(a.cpu().numpy(), b.cpu().numpy()) for a, b in pools]
    assert np.array_equal(k0.view(view), k_ref.view(view))
    assert np.array_equal(v0.view(view), v_ref.view(view))
    assert np.array_equal(k1.view(view), k_ref.view(view))
    assert np.array_equal(v1, -v_ref, equal_nan=True)
