"""GPU parity of pa_prefill (paged causal prefill on MFMA) against the
oracle's prefill, on the same seeded inputs, through the C ABI.

Bar: elementwise |gpu - oracle| <= 2e-3 + 1e-2 |oracle| (fp16 K/V/q; the
attention weights are rounded to fp16 for the product with V, an error of
at most 2^-11 relative per weight, far inside the bar).
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

ABS, REL = 2e-3, 1e-2


def announce(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def run_gpu(pa, wl, device, q=None, query_start=None, context_lens=None, tables=None,
            max_query_len=None, k_pool=None, listed=False):
    q = wl.q if q is None else q
    qs = wl.query_start if query_start is None else query_start
    ctx = wl.context_lens if context_lens is None else context_lens
    tables = wl.block_tables if tables is None else tables
    dq = dev(q, device)
    out = torch.full_like(dq, float("nan"))
    mq = int(np.diff(qs).max()) if len(qs) > 1 else 0
    pa.pa_prefill(out, dq, dev(wl.k_pool if k_pool is None else k_pool, device),
                  dev(wl.v_pool, device), dev(tables, device), dev(ctx, device), dev(qs, device),
                  float(wl.scale), max(int(np.max(ctx)) if len(ctx) else 0, 1),
                  mq if max_query_len is None else max_query_len,
                  host_query_start=qs if listed else None,
                  host_context_lens=ctx if listed else None)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(gpu, ref, where):
    gpu = gpu.astype(np.float64)
    bad = ~(np.abs(gpu - ref) <= ABS + REL * np.abs(ref))
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{where}: {bad.sum()} of {bad.size} out of tolerance; first {i}: "
                             f"gpu {gpu[i]!r} oracle {ref[i]!r}")


CASES = {
    "small-b16-d64": lambda: W.prefill_small(),
    "small-b8-d128": lambda: W.prefill_small(seed=5, head_dim=128, block_size=8),
    "small-b32-d64": lambda: W.prefill_small(seed=6, block_size=32,
                                             groups=((0, [130]), (33, [2, 97]), (64, [64]))),
    "small-b64-d128": lambda: W.prefill_small(seed=7, head_dim=128, block_size=64,
                                              groups=((0, [129]), (100, [1, 28]), (0, [2]))),
    # every block size at both head sizes, so each way the tile fetch picks
    # a row's table entry (one per tile, one per thread, inside one block)
    # meets the oracle
    "small-b8-d64": lambda: W.prefill_small(seed=12, block_size=8),
    "small-b64-d64": lambda: W.prefill_small(seed=13, block_size=64,
                                             groups=((0, [150]), (70, [3, 40]))),
    "small-b32-d128": lambda: W.prefill_small(seed=14, head_dim=128, block_size=32,
                                              groups=((0, [97]), (40, [70]), (64, [1, 9]))),
    "mix": lambda: W.prefill_mix(seed=8, num_heads=4, num_seqs=6, hi=700),
    "shared": lambda: W.prefill_shared(seed=9, num_heads=3, groups=2, members=4,
                                       prefix=(100, 400), suffix=(1, 200)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_matches_oracle(pa, oracle_lib, device, name):
    announce(f"prefill parity {name}")
    wl = CASES[name]()
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(run_gpu(pa, wl, device), ref, name)


@pytest.mark.parametrize("name", ["mix", "shared", "small-b8-d128", "small-b64-d128"])
def test_prefill_listed_launch(pa, oracle_lib, device, name):
    """With host copies of query_start and context_lens the library launches
    the existing tiles grouped by sequence: same oracle parity, and bit for bit
    the grid launch's output."""
    announce(f"prefill listed launch {name}")
    wl = CASES[name]()
    listed = run_gpu(pa, wl, device, listed=True)
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(listed, ref, name)
    grid = run_gpu(pa, wl, device)
    assert np.array_equal(listed.view(np.uint16), grid.view(np.uint16))


def test_prefill_edges(pa, oracle_lib, device):
    """Sequences with no queries beside one-token chunks and chunks around
    the 32-query wave and 256-query workgroup boundaries; rows of empty
    chunks are never written."""
    announce("prefill edges")
    wl = W.prefill_small(seed=11, head_dim=128,
                         groups=((0, [127]), (5, [0]), (0, [128]), (200, [0, 129]), (0, [1]),
                                 (0, [255]), (3, [256]), (0, [257]), (40, [33])))
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(run_gpu(pa, wl, device), ref, "edges")


def with_score_patterns(wl, patterns):
    """wl with q = 1 everywhere and every K row of head h at position t set to
    patterns[h](t) in each element, so that every query's score against key
    t is D * patterns[h](t): a pattern the lazy reference of the online
    softmax has to follow (slots past each context keep their NaN)."""
    q = np.ones_like(wl.q)
    kp = wl.k_pool.copy()
    B = wl.block_size
    for b, n in enumerate(wl.context_lens):
        t = np.arange(int(n))
        blk, off = wl.block_tables[b, t // B], t % B
        for h, f in enumerate(patterns):
            kp[blk, h, off, :] = f(t).astype(np.float32)[:, None]
    return q, kp


def test_prefill_lazy_reference_paths(pa, oracle_lib, device):
    """Scores that move the softmax reference on every 32-key tile (rising by
    about 21 log2 units per tile), never after the first (falling), and in
    jumps of about 200 log2 units at sparse spikes: the rescale branch runs
    often, with factors that underflow to 0, and the weights of keys far
    below the reference underflow.  Three more heads hold every score near
    one level, about -49, +16 and -7.3 log2 units: the first tile's
    reference is then its maximum (below -8 or above 11) or 0 (inside; the
    largest weight is 2^-7.3).  A reference of 0 at -49 would round every
    weight to 0 in fp16 and the rows to NaN.  Grid and listed launches
    against the oracle in fp64."""
    announce("prefill lazy reference paths")
    wl = W.prefill_small(seed=21, head_dim=128, num_heads=6, block_size=16,
                         groups=((0, [600]), (300, [1, 90]), (0, [33])))
    patterns = [lambda t: 0.04 * t,
                lambda t: -0.04 * t,
                lambda t: np.where(t % 97 == 0, 6.0, -6.0),
                lambda t: -3.0 + 0.05 * np.sin(t),
                lambda t: 1.0 + 0.05 * np.sin(t),
                lambda t: -0.45 + 0.02 * np.cos(t)]
    q, kp = with_score_patterns(wl, patterns)
    ref = oracle_lib.prefill(q, kp, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    assert np.isfinite(ref).all()
    for listed in (False, True):
        got = run_gpu(pa, wl, device, q=q, k_pool=kp, listed=listed)
        check(got, ref, f"lazy reference, listed={listed}")


def test_prefill_poisons_rows_that_see_a_bad_block(pa, oracle_lib, device):
    """A table entry outside the pool: rows whose context reaches that
    block are NaN, every other row is still right."""
    announce("prefill bad table entry")
    wl = W.prefill_small(seed=12, groups=((0, [70]), (0, [40])))
    B = wl.block_size
    tables = wl.block_tables.copy()
    tables[0, 2] = wl.num_blocks + 3            # keys 32..47 of sequence 0
    got = run_gpu(pa, wl, device, tables=tables)
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    n0 = int(wl.context_lens[0])
    pos = np.arange(n0)                          # sequence 0 is a full prefill
    sees = pos >= 2 * B
    assert np.isnan(got[:n0][sees]).all()
    check(got[:n0][~sees], ref[:n0][~sees], "rows before the bad block")
    check(got[n0:], ref[n0:], "other sequence")


def test_prefill_chunk_longer_than_context_is_nan(pa, oracle_lib, device):
    announce("prefill bad chunk")
    wl = W.prefill_small(seed=13, groups=((10, [5]), (0, [9])))
    ctx = wl.context_lens.copy()
    ctx[0] = 3                                   # 5 queries, 3 tokens: invalid
    got = run_gpu(pa, wl, device, context_lens=ctx)
    assert np.isnan(got[:5]).all()
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(got[5:], ref[5:], "valid sequence")


def test_prefill_rows_before_zero_are_not_written(pa, oracle_lib, device):
    """A sequence whose device query_start is negative is invalid: its rows
    that fall inside [0, num_query_rows) become NaN and the rows before row
    0 are not written.  out is a view into a larger buffer, so a write
    before it would land in the sentinel rows in front of it."""
    announce("prefill negative query start")
    import torch
    wl = W.prefill_small(seed=15, groups=((0, [20]), (0, [9])))
    qs = wl.query_start.copy()
    qs[0] = -4                                   # sequence 0: rows -4 .. 19
    T, H, D = wl.q.shape
    pad = 8
    big = torch.full((pad + T, H, D), 7.0, dtype=torch.float16, device=device)
    out = big[pad:]
    pa.pa_prefill(out, dev(wl.q, device), dev(wl.k_pool, device), dev(wl.v_pool, device),
                  dev(wl.block_tables, device), dev(wl.context_lens, device), dev(qs, device),
                  float(wl.scale), int(np.diff(qs).max()), int(np.diff(qs).max()))
    torch.cuda.synchronize()
    got = big.cpu().numpy()
    assert (got[:pad] == 7.0).all(), "rows before row 0 were written"
    n0 = int(wl.query_start[1])
    assert np.isnan(got[pad:pad + n0]).all()
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(got[pad + n0:], ref[n0:], "other sequence")


def run_split(pa, wl, device, slots, tables=None, context_lens=None):
    """The listed launch with a workspace of `slots` partial-result slots,
    pre-filled with a byte pattern; also says whether the launch wrote to it
    (the split form ran)."""
    T, H, D = wl.q.shape
    ctx = wl.context_lens if context_lens is None else context_lens
    ws = torch.full((pa.pa_prefill_workspace_bytes(H, D, slots),), 0x5A, dtype=torch.uint8,
                    device=device)
    dq = dev(wl.q, device)
    out = torch.full_like(dq, float("nan"))
    pa.pa_prefill(out, dq, dev(wl.k_pool, device), dev(wl.v_pool, device),
                  dev(wl.block_tables if tables is None else tables, device), dev(ctx, device),
                  dev(wl.query_start, device), float(wl.scale), max(int(np.max(ctx)), 1),
                  int(np.diff(wl.query_start).max()), host_query_start=wl.query_start,
                  host_context_lens=ctx, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), bool((ws != 0x5A).any().item())


SPLIT_CASES = {
    # few heads and query tiles of at least 48 key tiles (1536 keys), so the
    # planner splits the heaviest tiles over the idle GPU
    "one-prompt-b16-d128": lambda: W.prefill_small(seed=21, head_dim=128,
                                                   groups=((0, [1700]),)),
    "suffix-b16-d64": lambda: W.prefill_small(seed=22, groups=((1700, [100]), (0, [5]))),
    "one-prompt-b8-d128": lambda: W.prefill_small(seed=23, head_dim=128, block_size=8,
                                                  groups=((0, [1600]),)),
    "one-prompt-b64-d64": lambda: W.prefill_small(seed=24, block_size=64,
                                                  groups=((0, [1650]),)),
    "suffixes-b32-d128": lambda: W.prefill_small(seed=25, head_dim=128, block_size=32,
                                                 groups=((1600, [1, 300]), (0, [40]))),
}


@pytest.mark.parametrize("name", sorted(SPLIT_CASES))
def test_prefill_split_matches_oracle(pa, oracle_lib, device, name):
    """With a workspace the heaviest query tiles are split into key chunks
    and merged: oracle parity, and the workspace was used."""
    announce(f"prefill split {name}")
    wl = SPLIT_CASES[name]()
    got, used = run_split(pa, wl, device, slots=64)
    assert used, "the split form did not run"
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(got, ref, name)


def test_prefill_split_with_few_slots(pa, oracle_lib, device):
    """Two slots: only the heaviest tile is split, the rest run whole."""
    announce("prefill split, two slots")
    wl = SPLIT_CASES["one-prompt-b16-d128"]()
    got, used = run_split(pa, wl, device, slots=2)
    assert used
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(got, ref, "two slots")


def test_prefill_split_poisons_rows_that_see_a_bad_block(pa, oracle_lib, device):
    """A bad table entry inside a split tile's key range: exactly the rows
    that see it are NaN after the merge."""
    announce("prefill split, bad table entry")
    wl = SPLIT_CASES["one-prompt-b16-d128"]()
    B = wl.block_size
    tables = wl.block_tables.copy()
    tables[0, 20] = -7                           # keys 320..335
    got, used = run_split(pa, wl, device, slots=64, tables=tables)
    assert used
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    n0 = int(wl.context_lens[0])
    sees = np.arange(n0) >= 20 * B
    assert np.isnan(got[:n0][sees]).all()
    check(got[:n0][~sees], ref[:n0][~sees], "rows before the bad block")


def test_prefill_split_invalid_chunk_is_nan(pa, oracle_lib, device):
    """A sequence with more queries than context tokens gets NaN rows in the
    split form too; the other sequence is unaffected."""
    announce("prefill split, invalid chunk")
    wl = SPLIT_CASES["suffix-b16-d64"]()
    ctx = wl.context_lens.copy()
    ctx[1] = 2                                   # 5 queries over 2 tokens
    got, used = run_split(pa, wl, device, slots=64, context_lens=ctx)
    assert used
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    n0 = int(wl.query_start[1])
    check(got[:n0], ref[:n0], "valid sequence")
    assert np.isnan(got[n0:]).all()


def test_prefill_split_with_empty_chunks(pa, oracle_lib, device):
    """Host context lengths are upper bounds: planned from a 1740-token
    context, the device one is 50, so the tile's key range (2 tiles) is
    shorter than its chunk count and some chunks are empty (max -inf, sum
    0); the merge still gives the oracle's rows."""
    announce("prefill split, empty chunks")
    wl = W.prefill_small(seed=26, head_dim=128, groups=((1700, [40]),))
    T, H, D = wl.q.shape
    host_ctx = wl.context_lens.copy()
    ctx = wl.context_lens.copy()
    ctx[0] = 50                                  # the 40 queries sit at positions 10..49
    ws = torch.full((pa.pa_prefill_workspace_bytes(H, D, 64),), 0x5A, dtype=torch.uint8,
                    device=device)
    dq = dev(wl.q, device)
    out = torch.full_like(dq, float("nan"))
    pa.pa_prefill(out, dq, dev(wl.k_pool, device), dev(wl.v_pool, device),
                  dev(wl.block_tables, device), dev(ctx, device), dev(wl.query_start, device),
                  float(wl.scale), int(host_ctx.max()), 40, host_query_start=wl.query_start,
                  host_context_lens=host_ctx, workspace=ws)
    torch.cuda.synchronize()
    assert bool((ws != 0x5A).any().item()), "the split form did not run"
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, ctx,
                             wl.query_start, wl.scale)
    check(out.cpu().numpy(), ref, "empty chunks")


def test_prefill_no_split_when_balanced(pa, oracle_lib, device):
    """A batch whose work spreads over the GPU is not split even with a
    workspace: the output is bit for bit the listed launch's."""
    announce("prefill no split when balanced")
    wl = W.prefill_mix(seed=8, num_heads=40, num_seqs=24, hi=300)
    got, used = run_split(pa, wl, device, slots=64)
    assert not used
    listed = run_gpu(pa, wl, device, listed=True)
    assert np.array_equal(got.view(np.uint16), listed.view(np.uint16))


@pytest.mark.parametrize("which", ["mix", "shared"])
def test_prefill_full_size_every_row(pa, oracle_lib, device, which):
    """The OPT-13B-shaped workloads (40 heads x 128, B 16) in one launch:
    every query row of every head against the oracle."""
    announce(f"prefill full size {which}")
    wl = W.prefill_mix() if which == "mix" else W.prefill_shared()
    got = run_gpu(pa, wl, device, listed=True)
    announce(f"prefill full size {which}: oracle over {int(wl.query_start[-1])} query rows")
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(got, ref, f"prefill {which}")


@pytest.mark.parametrize("split", [False, True], ids=["listed", "split"])
def test_prefill_replayed_from_a_hip_graph(pa, oracle_lib, device, split):
    """pa_prefill (listed, and split with its merge pass) captured once and
    replayed three times, with eager work and synchronisation between
    replays: every replay reproduces the eager result bit for bit."""
    wl = SPLIT_CASES["suffix-b16-d64"]()
    T, H, D = wl.q.shape
    q, kp, vp = dev(wl.q, device), dev(wl.k_pool, device), dev(wl.v_pool, device)
    tb, cx, qs = dev(wl.block_tables, device), dev(wl.context_lens, device), dev(wl.query_start, device)
    ws = (torch.empty(pa.pa_prefill_workspace_bytes(H, D, 64), dtype=torch.uint8, device=device)
          if split else None)
    out = torch.empty_like(q)

    def call():
        pa.pa_prefill(out, q, kp, vp, tb, cx, qs, float(wl.scale), wl.max_context_len,
                      wl.max_query_len, host_query_start=wl.query_start,
                      host_context_lens=wl.context_lens, workspace=ws)

    announce(f"prefill eager ({'split' if split else 'listed'})")
    call()
    torch.cuda.synchronize()
    eager = out.cpu().numpy()
    ref = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    check(eager, ref, "eager")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    announce("prefill capture")
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))          # eager work between replays
        if ws is not None:
            ws.fill_(0x5A)
        torch.cuda.synchronize()
        announce(f"prefill replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager.view(np.uint16)), \
            f"replay {r}: output differs"
