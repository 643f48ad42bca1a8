"""The seeded input generators: determinism, the configurations' recipes,
valid placements, NaN in unused slots, and the byte counter's closed forms.
No GPU."""
import json
import math
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def live_entries(wl):
    out = []
    for b, n in enumerate(wl.context_lens):
        nb = -(-int(n) // wl.block_size)
        row = wl.block_tables[b]
        assert np.all(row[nb:] == -1)
        out.append(row[:nb])
    return out


def test_deterministic():
    a, b = W.opt13b_layer(num_seqs=8, num_heads=2), W.opt13b_layer(num_seqs=8, num_heads=2)
    assert np.array_equal(a.context_lens, b.context_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    assert np.array_equal(a.q.view(np.uint16), b.q.view(np.uint16))
    assert np.array_equal(a.k_pool.view(np.uint16), b.k_pool.view(np.uint16))
    c = W.opt13b_layer(seed=99, num_seqs=8, num_heads=2)
    assert not np.array_equal(a.context_lens, c.context_lens)


def test_config1_recipe():
    wl = W.tiny_fp32()
    assert list(wl.context_lens) == [1, 17, 33, 50, 50]          # 4 sequences + the fork of the 4th
    assert (wl.num_heads, wl.head_dim, wl.block_size, wl.num_blocks) == (2, 64, 16, 32)
    assert wl.dtype == W.F32 and wl.scale == np.float32(1 / 8)
    assert wl.max_blocks_per_seq == 4
    # the fork shares every block of sequence 3 but the copied last one
    assert np.array_equal(wl.block_tables[4, :3], wl.block_tables[3, :3])
    assert wl.block_mapping.tolist() == [[wl.block_tables[3, 3], wl.block_tables[4, 3]]]
    # all five rows append at position ctx - 1; the fork into the copy
    assert wl.slot_mapping[4] == wl.block_tables[4, 3] * 16 + 49 % 16
    assert wl.slot_mapping[3] == wl.block_tables[3, 3] * 16 + 49 % 16


@pytest.mark.parametrize("make", [lambda: W.opt13b_layer(num_seqs=16, num_heads=2),
                                  lambda: W.short_rows(block_size=8, num_seqs=16, num_heads=2),
                                  lambda: W.long_context(num_seqs=4, num_heads=2)],
                         ids=["opt13b", "short-b8", "long-meta"])
def test_scattered_unique_placement(make):
    wl = make()
    live = np.concatenate(live_entries(wl))
    assert live.min() >= 0 and live.max() < wl.num_blocks
    assert len(np.unique(live)) == len(live)        # no sharing outside the shared-prompt workload
    assert wl.num_blocks == math.ceil(1.5 * len(live))
    assert len(np.unique(wl.slot_mapping)) == len(wl.slot_mapping)


def test_config2_lengths():
    wl = W.opt13b_layer(num_heads=1)
    ctx = wl.context_lens
    assert ctx.min() >= 1 and ctx.max() <= 2048 and len(ctx) == 64
    big = W.lognormal_lengths(np.random.default_rng(0), 200000)
    assert abs(np.median(big) - 300) < 3          # median 300
    assert abs(np.std(np.log(big[(big > 1) & (big < 2048)])) - 0.9) < 0.05


def test_config3_same_logical_values_for_every_block_size():
    ref = W.short_rows(block_size=16, num_seqs=6, num_heads=2)
    assert ref.context_lens.min() >= 20 and ref.context_lens.max() <= 200
    for B in (8, 32, 64):
        wl = W.short_rows(block_size=B, num_seqs=6, num_heads=2)
        assert np.array_equal(wl.context_lens, ref.context_lens)
        assert all(np.array_equal(a.view(np.uint16), b.view(np.uint16))
                   for a, b in zip(wl.logical_k, ref.logical_k))
        assert wl.max_blocks_per_seq == -(-200 // B)


def test_config4_sharing_structure():
    wl = W.shared_prompts(num_prompts=5, samples=6, num_heads=2)
    P, T = wl.extra["prompt_lens"], wl.extra["tail_lens"]
    assert wl.num_seqs == 30
    refcount = {}
    for row in live_entries(wl):
        for blk in row:
            refcount[int(blk)] = refcount.get(int(blk), 0) + 1
    pairs = wl.block_mapping.tolist()
    for p in range(5):
        rows = wl.block_tables[p * 6:(p + 1) * 6]
        full = int(P[p]) // 16
        for j in range(full):                       # full prompt blocks: refcount 6
            assert len(set(rows[:, j])) == 1 and refcount[int(rows[0, j])] == 6
        if P[p] % 16:                               # partial last prompt block
            last = rows[:, full]
            assert len(set(last)) == 6              # 5 copies + the original
            orig = last[5]
            assert sorted([d for s, d in pairs if s == orig]) == sorted(last[:5])
    assert len(np.unique([d for _, d in pairs])) == len(pairs)
    assert np.all(wl.context_lens == (P[:, None] + T).reshape(-1))
    assert len(wl.slot_mapping) == T.sum()


def test_unused_slots_hold_nan():
    wl = W.opt13b_layer(num_seqs=6, num_heads=2)
    rows_finite = np.isfinite(wl.k_pool).all(axis=-1)        # [NB][H][B]
    assert rows_finite.sum() == wl.context_lens.sum() * wl.num_heads
    assert np.isnan(wl.k_pool_pre).sum() > np.isnan(wl.k_pool).sum()


def test_byte_counter_closed_forms():
    """zhaifeiyue summary: OPT-13B's KV cache is 800 KB per token; 12 GB of KV
    cache holds 15.7K slots (OPT-13B, 1xA100-40GB) and 264 GB holds 60.1K
    (OPT-175B, 8xA100-80GB)."""
    with open(os.path.join(GOLDEN, "kv_capacity.json")) as f:
        g = json.load(f)["models"]
    m = g["opt13b"]
    per_tok = W.kv_bytes_per_token(m["heads"], m["head_dim"], m["elem_bytes"], m["layers"])
    assert per_tok == m["kv_bytes_per_token"] == 800 * 1024
    for name in ("opt13b", "opt175b"):
        m = g[name]
        per_tok = W.kv_bytes_per_token(m["heads"], m["head_dim"], m["elem_bytes"], m["layers"])
        slots = m["kv_cache_gib"] * 2**30 / per_tok
        assert round(slots / 1000, 1) == m["max_slots_thousands"]
    # the per-call counter: one layer's K+V rows for every context token, plus
    # one 4-byte table entry per block in use
    ctx = np.array([1, 16, 17])
    assert W.algorithmic_bytes(ctx, 40, 128, 16, 2) == 34 * 40 * 128 * 2 * 2 + 4 * (1 + 1 + 2)


@pytest.mark.parametrize("make", [lambda: W.prefill_small(),
                                  lambda: W.prefill_shared(num_heads=2, head_dim=64, groups=2,
                                                           members=3, prefix=(17, 70),
                                                           suffix=(1, 40))])
def test_prefill_pools_hold_the_logical_tokens(make):
    """Gathering each sequence's tokens through its table gives its logical
    K/V; a group's full prefix blocks are shared; no other slot holds data."""
    wl = make()
    B = wl.block_size
    filled = np.zeros(wl.k_pool.shape[:1] + (B,), bool)
    for b in range(wl.num_seqs):
        n = int(wl.context_lens[b])
        for t in range(n):
            blk = int(wl.block_tables[b, t // B])
            assert np.array_equal(wl.k_pool[blk, :, t % B].view(np.uint16 if wl.dtype == W.F16 else np.uint32),
                                  wl.logical_k[b][t].view(np.uint16 if wl.dtype == W.F16 else np.uint32))
            assert np.array_equal(wl.v_pool[blk, :, t % B], wl.logical_v[b][t])
            filled[blk, t % B] = True
    by_slot = lambda pool: pool.transpose(0, 2, 1, 3)          # [NB][B][H][D]
    assert np.isnan(by_slot(wl.k_pool)[~filled]).all()
    assert np.isnan(by_slot(wl.v_pool)[~filled]).all()
    b = 0
    for P, sufs in wl.extra["groups"]:
        rows = wl.block_tables[b:b + len(sufs), :P // B]
        assert (rows == rows[0]).all()
        b += len(sufs)
    assert int(wl.query_start[-1]) == len(wl.q)
