"""The host block manager (include/pa_manager.h), on the CPU: the pages'
copy-on-write example and sharing diagram replayed through it, on-demand
allocation, reference counts, free at zero, all-or-nothing appends, and
random operation sequences checked against its own consistency check and
against lengths, slots and counts tracked independently in the test."""
import json
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def M(pa):
    from paged_kv_cache_05_amd import manager
    return manager


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_cow_worked_example(M):
    """wywy.jp WHERE, parallel sampling: A1's write into shared block 1 takes
    a new block (3), copies 1 into it and drops block 1's count to 1; A2 then
    writes into block 1 in place."""
    g = load("cow_example.json")
    B, NB, P = g["block_size"], g["num_blocks"], g["prompt_len"]
    # the page names blocks 1 and 3; the allocation order reads them in
    m = M.BlockManager(NB, B, alloc_order=[0, 1, 3, 2])
    A1, A2 = 1, 2
    m.add(A1)
    slots, pairs = m.append([A1] * P)
    assert list(slots) == list(range(P)) and len(pairs) == 0
    m.fork(A1, A2)
    assert {str(b): m.refcount(b) for b in (0, 1)} == g["refcount_before"]
    for ev, seq in zip(g["events"], (A1, A2)):
        assert m.refcount(ev["target_block"]) == ev["target_refcount"]
        slots, pairs = m.append([seq])
        assert int(slots[0]) == ev["slot"]
        assert (pairs.tolist()[0] if len(pairs) else None) == ev["copy"]
        tables, ctx = m.tables([seq], 2)
        assert tables[0].tolist() == ev["table_after"] and ctx[0] == P + 1
        got = {str(b): m.refcount(b) for b in range(NB) if m.refcount(b)}
        assert got == ev["refcount_after"]
        m.check()


def test_sharing_diagram(M):
    """ricepunchb 5.1: A -> [7, 3, 12], B -> [7, 3, 9] after a fork at 8
    tokens (block size 4) and 2 private tokens each."""
    g = load("sharing_diagram.json")
    B, NB = g["block_size"], g["num_blocks"]
    order = [7, 3, 12, 9] + [b for b in range(NB) if b not in (7, 3, 12, 9)]
    m = M.BlockManager(NB, B, alloc_order=order)
    A, Bs = 10, 11
    m.add(A)
    m.append([A] * g["shared_tokens"])
    m.fork(A, Bs)
    for _ in range(g["context_len"] - g["shared_tokens"]):
        _, pairs = m.append([A, Bs])
        assert len(pairs) == 0          # the shared blocks are full: no copy needed
    tables, ctx = m.tables([A, Bs], 3)
    assert tables.tolist() == [g["tables"]["A"], g["tables"]["B"]]
    assert ctx.tolist() == [g["context_len"]] * 2
    assert [m.refcount(b) for b in g["shared"]] == [2, 2]
    m.check()


def test_allocation_on_demand_and_waste(M):
    """A block is taken only when the previous one is full; every sequence
    wastes less than one block ([zhai] memory table 'Allocate'; ricepunchb 4)."""
    B = 16
    m = M.BlockManager(64, B)
    m.add(1)
    for t in range(100):
        free_before = m.num_free
        m.append([1])
        assert m.num_free == free_before - (1 if t % B == 0 else 0)
        nblk = -(-(t + 1) // B)
        assert 0 <= nblk * B - (t + 1) < B
    m.check()


def test_free_at_zero_and_reuse(M):
    m = M.BlockManager(8, 4)
    m.add(1)
    m.append([1] * 6)                   # blocks 0, 1 (1 partly filled)
    m.fork(1, 2)
    assert m.refcount(0) == m.refcount(1) == 2
    m.free(1)                           # pruned candidate (wywy WHERE beam search)
    assert m.refcount(0) == m.refcount(1) == 1 and m.num_free == 6
    m.free(2)
    assert m.num_free == 8 and m.refcount(0) == 0
    m.add(3)
    slots, _ = m.append([3])
    assert slots[0] // 4 == 0           # most recently freed block first
    m.check()


def test_append_is_all_or_nothing(M):
    m = M.BlockManager(3, 4)
    for s in (1, 2):
        m.add(s)
        m.append([s] * 4)               # each fills one block
    before = m.tables([1, 2], 4), m.num_free
    with pytest.raises(M.OutOfBlocks):
        m.append([1, 2])                # needs two fresh blocks, one is free
    after = m.tables([1, 2], 4), m.num_free
    assert np.array_equal(before[0][0], after[0][0]) and before[1] == after[1]
    m.append([1])                       # one fits
    m.check()


def test_errors(M):
    m = M.BlockManager(4, 4)
    m.add(1)
    with pytest.raises(M.PAError):
        m.add(1)
    with pytest.raises(M.PAError):
        m.fork(9, 2)
    with pytest.raises(M.PAError):
        m.append([5])
    with pytest.raises(M.PAError):
        M.BlockManager(4, 4, alloc_order=[0, 1, 1, 2])
    m.append([1] * 5)
    with pytest.raises(M.PAError):
        m.tables([1], 1)                # two blocks do not fit one column


def test_parallel_sampling_saves_memory(M):
    """Six samples of one 500-token prompt share its 32 blocks; each keeps a
    private copy of the partial last block once it writes."""
    B, prompt, samples, gen = 16, 500, 6, 40
    m = M.BlockManager(400, B)
    m.add(0)
    m.append([0] * prompt)
    for s in range(1, samples):
        m.fork(0, s)
    ids = list(range(samples))
    copies = 0
    for _ in range(gen):
        _, pairs = m.append(ids)
        copies += len(pairs)
    assert copies == samples - 1        # the last sharer writes in place
    used = 400 - m.num_free
    private = samples * -(-(prompt + gen) // B)
    assert used == prompt // B + samples * (-(-(prompt + gen) // B) - prompt // B)
    assert used < private
    m.check()


def test_swap_out_and_in_keep_sharing(M):
    """A group (prompt + 2 samples) is evicted whole: each distinct block
    it holds goes to the swap space once, its GPU blocks are freed, and it
    comes back with its sharing intact (wywy.jp Keyword "Swapping",
    "All-or-nothing eviction")."""
    B = 4
    m = M.BlockManager(16, B, num_host_blocks=16)
    m.add(0)
    m.append([0] * 10)                  # blocks 0, 1 full; 2 holds 2 tokens
    m.fork(0, 1)
    m.fork(0, 2)
    m.append([0, 1, 2])                 # 0 and 1 copy block 2; 2 writes in place
    tables, _ = m.tables([0, 1, 2], 4)
    distinct = {int(b) for b in tables[:, :3].ravel()}
    assert len(distinct) == 5           # 2 shared + 3 private last blocks
    free_before = m.num_free
    pairs = m.swap_out([0, 1, 2])
    assert len(pairs) == 5 and {int(a) for a, _ in pairs} == distinct
    assert len({int(b) for _, b in pairs}) == 5
    assert m.num_free == free_before + 5 and m.num_free_host == 16 - 5
    assert all(m.is_swapped(s) for s in (0, 1, 2))
    for call in (lambda: m.append([1]), lambda: m.tables([1], 4), lambda: m.fork(1, 9),
                 lambda: m.swap_out([1])):
        with pytest.raises(M.PAError):
            call()
    back = m.swap_in([2, 0, 1])
    assert len(back) == 5 and sorted(int(a) for a, _ in back) == sorted(int(b) for _, b in pairs)
    tables2, ctx = m.tables([0, 1, 2], 4)
    assert ctx.tolist() == [11, 11, 11]
    assert tables2[0, 0] == tables2[1, 0] == tables2[2, 0]       # still shared
    assert tables2[0, 1] == tables2[1, 1] == tables2[2, 1]
    assert len({int(x) for x in tables2[:, 2]}) == 3
    assert m.refcount(int(tables2[0, 0])) == 3 and m.num_free_host == 16
    m.check()


def test_swap_out_part_of_a_group(M):
    """Swapping out one of two sequences that share a block leaves the block
    on the GPU for the other; the swapped one keeps a host copy."""
    m = M.BlockManager(8, 4, num_host_blocks=8)
    m.add(0)
    m.append([0] * 8)                   # two full blocks
    m.fork(0, 1)
    pairs = m.swap_out([1])
    assert len(pairs) == 2
    assert m.refcount(0) == 1 and m.refcount(1) == 1 and m.num_free == 6
    m.free(1)                           # a swapped sequence frees host blocks
    assert m.num_free_host == 8
    m.check()


def test_swap_is_all_or_nothing(M):
    m = M.BlockManager(8, 4, num_host_blocks=2)
    m.add(0)
    m.append([0] * 12)                  # three blocks
    with pytest.raises(M.OutOfBlocks):
        m.swap_out([0])                 # the swap space holds two
    assert not m.is_swapped(0) and m.num_free == 5 and m.num_free_host == 2
    m2 = M.BlockManager(4, 4, num_host_blocks=4)
    for s in (0, 1):
        m2.add(s)
        m2.append([s] * 8)
    m2.swap_out([1])
    m2.add(2)
    m2.append([2] * 5)                  # takes both freed blocks
    with pytest.raises(M.OutOfBlocks):
        m2.swap_in([1])
    assert m2.is_swapped(1) and m2.num_free_host == 2
    m2.free(2)
    assert len(m2.swap_in([1])) == 2
    m2.check()


@st.composite
def programs(draw):
    ops = []
    live = []
    next_id = 0
    for _ in range(draw(st.integers(5, 40))):
        kind = draw(st.sampled_from(["add", "append", "append", "fork", "free", "swap"]))
        if kind == "add" or not live:
            ops.append(("add", next_id))
            live.append(next_id)
            next_id += 1
        elif kind == "swap":
            k = draw(st.integers(1, min(3, len(live))))
            ops.append(("swap", draw(st.permutations(live))[:k]))
        elif kind == "append":
            k = draw(st.integers(1, 6))
            ops.append(("append", [draw(st.sampled_from(live)) for _ in range(k)]))
        elif kind == "fork":
            ops.append(("fork", draw(st.sampled_from(live)), next_id))
            live.append(next_id)
            next_id += 1
        else:
            s = draw(st.sampled_from(live))
            live.remove(s)
            ops.append(("free", s))
    return ops


@settings(max_examples=150, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(programs(), st.sampled_from([1, 2, 4, 16]), st.integers(4, 40), st.integers(0, 40))
def test_random_programs_keep_invariants(M, ops, B, nb, hnb):
    """Random add / fork / append / free / swap programs.  A "swap" op
    swaps its sequences out if all are resident, in if all are out."""
    m = M.BlockManager(nb, B, num_host_blocks=hnb)
    lengths = {}
    for op in ops:
        # ids named by ops that failed earlier (a fork of a swapped-out
        # sequence) do not exist: skip what names them
        named = op[1] if op[0] in ("append", "swap") else [op[1]]
        if op[0] != "add" and any(i not in lengths for i in named):
            continue
        if op[0] == "swap":
            state = {m.is_swapped(i) for i in op[1]}
            if len(state) != 1:
                continue
            fn = m.swap_in if state.pop() else m.swap_out
            free = (m.num_free, m.num_free_host)
            try:
                pairs = fn(op[1])
            except M.OutOfBlocks:
                assert (m.num_free, m.num_free_host) == free
                continue
            assert len({int(b) for _, b in pairs}) == len(pairs)
            m.check()
            continue
        if op[0] == "append" and any(m.is_swapped(i) for i in op[1]):
            with pytest.raises(M.PAError):
                m.append(op[1])
            continue
        if op[0] == "fork" and m.is_swapped(op[1]):
            with pytest.raises(M.PAError):
                m.fork(op[1], op[2])
            continue
        if op[0] == "add":
            m.add(op[1])
            lengths[op[1]] = 0
        elif op[0] == "fork":
            m.fork(op[1], op[2])
            lengths[op[2]] = lengths[op[1]]
        elif op[0] == "free":
            m.free(op[1])
            del lengths[op[1]]
        else:
            free_before = m.num_free
            try:
                slots, pairs = m.append(op[1])
            except M.OutOfBlocks:
                assert m.num_free == free_before   # nothing changed
                continue
            # slots are distinct, in range, and at the next position of each sequence
            assert len(set(slots.tolist())) == len(slots)
            assert all(0 <= s < nb * B for s in slots)
            seen = {}
            for s, slot in zip(op[1], slots):
                pos = lengths[s] + seen.get(s, 0)
                seen[s] = seen.get(s, 0) + 1
                assert slot % B == pos % B
            for s, c in seen.items():
                lengths[s] += c
            for src, dst in pairs:
                assert src != dst
        m.check()
        ids = sorted(s for s in lengths if not m.is_swapped(s))
        if ids:
            tables, ctx = m.tables(ids, max(1, max(-(-lengths[i] // B) for i in ids)))
            assert ctx.tolist() == [lengths[i] for i in ids]
            # every block held by a sequence is counted once per holder
            held = {}
            for row, i in zip(tables, ids):
                for b in row[:-(-lengths[i] // B)]:
                    held[int(b)] = held.get(int(b), 0) + 1
            assert all(m.refcount(b) == c for b, c in held.items())
            # swapped-out sequences hold host blocks only
            assert m.num_free == nb - len(held)
