"""Pins of the CPU oracle to facts outside itself: the pages' printed examples,
library routines, closed forms, a literal high-precision evaluation of the
block-wise equation, and invariances the method guarantees.  No GPU.

Each test names the passage it follows (Kwon et al., PagedAttention, as
summarised by the wywy.jp notes, the zhaifeiyue.github.io summary and the
ricepunchb.github.io notes).
"""
import decimal
import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def run_decode(oracle, wl, **kw):
    return oracle.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens, wl.scale, **kw)


def sdpa_dense(wl):
    """Standard softmax attention of each query over its own logical K/V rows,
    by torch's scaled_dot_product_attention in float64 on the CPU."""
    N, H, D = wl.q.shape
    out = np.zeros((N, H, D))
    for b in range(N):
        n = int(wl.context_lens[b])
        if n == 0:
            continue
        q = torch.from_numpy(wl.q[b].astype(np.float64)).reshape(1, H, 1, D)
        k = torch.from_numpy(wl.logical_k[b].astype(np.float64)).permute(1, 0, 2).reshape(1, H, n, D)
        v = torch.from_numpy(wl.logical_v[b].astype(np.float64)).permute(1, 0, 2).reshape(1, H, n, D)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=float(wl.scale))
        out[b] = o.reshape(H, D).numpy()
    return out


# --------------------------------------------------------------------------
# binary16 widening
# --------------------------------------------------------------------------

def test_half_decoder_exhaustive(oracle_lib):
    """All 65,536 binary16 patterns decode exactly as numpy's float16 -> float64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle_lib.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))  # -0 stays -0


# --------------------------------------------------------------------------
# attention value: library routine, brute force, closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("make", [
    lambda: W.tiny_fp32(),
    lambda: W.opt13b_layer(num_seqs=6, num_heads=3),
    lambda: W.short_rows(block_size=8, num_seqs=8, num_heads=2),
    lambda: W.short_rows(block_size=64, num_seqs=8, num_heads=2),
    lambda: W.shared_prompts(num_prompts=2, samples=3, num_heads=2),
], ids=["tiny", "opt13b-small", "short-b8-small", "short-b64-small", "cow-small"])
def test_dense_attention_after_gather(oracle_lib, make):
    """The block-wise form equals standard attention (zhaifeiyue summary: the
    rewrite is mathematically equivalent because the softmax denominator
    runs over all blocks).  Reference: torch SDPA, fp64, on the logical rows
    the generator drew before scattering them."""
    wl = make()
    got = run_decode(oracle_lib, wl)
    ref = sdpa_dense(wl)
    assert np.all(np.abs(got - ref) <= 1e-12 * np.maximum(1.0, np.abs(ref)))


def literal_blockwise(q, keys, values, B, scale):
    """zhaifeiyue summary, method paragraph: A_ij = exp(q.K_j/sqrt d) over
    sum_t exp(q.K_t 1/sqrt d) (1: sum over the block's entries), o = sum_j
    V_j A_ij^T -- evaluated literally in 40-digit decimal, no max
    subtraction, block by block."""
    ctx = decimal.Context(prec=40)
    dec = lambda x: decimal.Decimal(float(x))
    n, D = keys.shape
    sc = dec(scale)
    blocks = [list(range(j, min(j + B, n))) for j in range(0, n, B)]
    num = [[ctx.exp(ctx.multiply(sc, sum((dec(q[d]) * dec(keys[t][d]) for d in range(D)), decimal.Decimal(0))))
            for t in blk] for blk in blocks]
    denom = sum((sum(row, decimal.Decimal(0)) for row in num), decimal.Decimal(0))
    out = []
    for d in range(D):
        acc = decimal.Decimal(0)
        for blk, row in zip(blocks, num):
            for t, e in zip(blk, row):
                acc += dec(values[t][d]) * ctx.divide(e, denom)
        out.append(float(acc))
    return np.array(out)


@pytest.mark.parametrize("seed", range(6))
def test_decimal_brute_force(oracle_lib, seed):
    rng = np.random.default_rng(seed)
    B = 2
    D = int(rng.integers(1, 5))
    n = int(rng.integers(1, 7))
    H = 2
    nb = -(-n // B)
    NB = nb + 3
    phys = rng.permutation(NB)[:nb]
    dtype = np.float16 if seed % 2 else np.float32
    keys = rng.standard_normal((n, H, D)).astype(dtype) * dtype(2)
    values = rng.standard_normal((n, H, D)).astype(dtype)
    q = rng.standard_normal((1, H, D)).astype(dtype)
    kp = np.full((NB, H, B, D), np.nan, dtype)
    vp = np.full((NB, H, B, D), np.nan, dtype)
    W._place(kp, keys, phys, B)
    W._place(vp, values, phys, B)
    table = np.full((1, nb + 1), -1, np.int32)
    table[0, :nb] = phys
    scale = np.float32(1 / math.sqrt(D))
    got = oracle_lib.decode(q, kp, vp, table, np.array([n], np.int32), scale)
    for h in range(H):
        ref = literal_blockwise(q[0, h], keys[:, h], values[:, h], B, scale)
        assert np.all(np.abs(got[0, h] - ref) <= 1e-14 * np.maximum(1.0, np.abs(ref)))


def test_single_token_returns_v_exactly(oracle_lib):
    wl = W.tiny_fp32()
    out = run_decode(oracle_lib, wl)
    b = int(np.flatnonzero(wl.context_lens == 1)[0])
    assert np.array_equal(out[b], wl.logical_v[b][0].astype(np.float64))


def test_weights_sum_to_one(oracle_lib):
    wl = W.short_rows(block_size=16, num_seqs=5, num_heads=3)
    _, w = run_decode(oracle_lib, wl, return_weights=True)
    for b in range(wl.num_seqs):
        n = int(wl.context_lens[b])
        assert np.all(np.abs(w[b, :, :n].sum(axis=1) - 1.0) <= 1e-14)
        assert np.all(w[b, :, :n] > 0)


def test_zero_query_gives_mean_of_values(oracle_lib):
    wl = W.short_rows(block_size=32, num_seqs=4, num_heads=2)
    wl.q = np.zeros_like(wl.q)
    out = run_decode(oracle_lib, wl)
    for b in range(wl.num_seqs):
        ref = wl.logical_v[b].astype(np.float64).mean(axis=0)
        assert np.allclose(out[b], ref, rtol=0, atol=1e-14)


def test_equal_keys_give_mean_of_values(oracle_lib):
    wl = W.tiny_fp32()
    k = wl.k_pool.copy()
    k[np.isfinite(k)] = 0.75  # every stored key row identical
    out = oracle_lib.decode(wl.q, k, wl.v_pool, wl.block_tables, wl.context_lens, wl.scale)
    for b in range(wl.num_seqs):
        ref = wl.logical_v[b].astype(np.float64).mean(axis=0)
        assert np.allclose(out[b], ref, rtol=0, atol=1e-14)


def test_two_tokens_logistic(oracle_lib):
    """n = 2: out = sigma(s1 - s2) v1 + sigma(s2 - s1) v2."""
    rng = np.random.default_rng(11)
    H, D, B = 3, 64, 16
    keys = rng.standard_normal((2, H, D)).astype(np.float32)
    values = rng.standard_normal((2, H, D)).astype(np.float32)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    kp = np.full((4, H, B, D), np.nan, np.float32)
    vp = kp.copy()
    W._place(kp, keys, [2], B)
    W._place(vp, values, [2], B)
    scale = np.float32(0.125)
    out = oracle_lib.decode(q, kp, vp, np.array([[2]], np.int32), np.array([2], np.int32), scale)
    for h in range(H):
        s = float(scale) * (keys[:, h].astype(np.float64) @ q[0, h].astype(np.float64))
        sig = 1.0 / (1.0 + math.exp(-(s[0] - s[1])))
        ref = sig * values[0, h].astype(np.float64) + (1 - sig) * values[1, h].astype(np.float64)
        assert np.allclose(out[0, h], ref, rtol=0, atol=1e-14)


def test_empty_context_is_zero(oracle_lib):
    wl = W.tiny_fp32()
    ctx = wl.context_lens.copy()
    ctx[2] = 0
    out = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, ctx, wl.scale)
    assert np.array_equal(out[2], np.zeros_like(out[2]))


def test_unused_slots_never_read(oracle_lib):
    """Slots past the filled count hold NaN in every workload; the oracle
    output is finite, and stays bit-identical when those slots change."""
    wl = W.short_rows(block_size=64, num_seqs=6, num_heads=2)
    a = run_decode(oracle_lib, wl)
    assert np.isfinite(a).all()
    k, v = wl.k_pool.copy(), wl.v_pool.copy()
    k[np.isnan(k)] = 1e4
    v[np.isnan(v)] = -3e4
    b = oracle_lib.decode(wl.q, k, v, wl.block_tables, wl.context_lens, wl.scale)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------

def test_placement_invariance(oracle_lib):
    """Any placement of the same logical blocks gives bit-identical results
    (the kernel only ever sees physical block ids: wywy.jp WHY)."""
    wl = W.opt13b_layer(num_seqs=5, num_heads=2)
    ref = run_decode(oracle_lib, wl)
    for s in range(3):
        r = W.relayout(wl, s)
        assert not np.array_equal(r.block_tables, wl.block_tables)
        assert np.array_equal(run_decode(oracle_lib, r), ref)


def test_block_size_invariance(oracle_lib):
    """Same logical K/V stored with B = 8, 16, 32, 64: bit-identical output
    (sums run in logical token order whatever the block size)."""
    base = W.short_rows(block_size=16, num_seqs=6, num_heads=2)
    ref = run_decode(oracle_lib, base)
    for B in (8, 32, 64):
        r = W.relayout(base, 100 + B, block_size=B)
        assert r.block_size == B
        assert np.array_equal(run_decode(oracle_lib, r), ref)


def test_shared_versus_copied_prefix(oracle_lib):
    """The shared prompts' blocks (refcount 6) and copy-on-write copies
    give bit-identical results to every sequence owning private copies."""
    wl = W.shared_prompts(num_prompts=3, samples=6, num_heads=2)
    ref = run_decode(oracle_lib, wl)
    private = W.relayout(wl, 5)
    assert np.array_equal(run_decode(oracle_lib, private), ref)
    # and the shared layout really shares: the same physical block in several rows
    live = np.concatenate([wl.block_tables[b, :-(-int(n) // 16)] for b, n in enumerate(wl.context_lens)])
    assert len(np.unique(live)) < len(live)


# --------------------------------------------------------------------------
# address translation
# --------------------------------------------------------------------------

def append_process(table_row, n, B):
    """Token-by-token placement as the KV cache manager does it: each token
    goes to the next free position of the sequence's last block; when that
    block is full the next physical block from the table is taken (wywy.jp
    Keyword "KV cache manager"; zhaifeiyue memory-management table,
    "Allocate").  Returns the (physical block, position) of every token."""
    where = []
    blocks_taken, fill = 0, B
    for _ in range(n):
        if fill == B:
            blocks_taken += 1
            fill = 0
        where.append((int(table_row[blocks_taken - 1]), fill))
        fill += 1
    return where


def tagged_probe(oracle, table, n, B, NB, H, target, dtype=np.float32):
    """Decode with a one-hot score on the slot `target` = (block, pos): its K
    row is 1000*e0 and every other K row 0, q = e0, scale 1, so exp of the
    other scores underflows to exactly 0 and the output is exactly the V row
    of whatever slot the oracle read for that score.  V rows carry their own
    (block, pos, head) as tags."""
    D = 64
    kp = np.zeros((NB, H, B, D), dtype)
    kp[target[0], :, target[1], 0] = 1000
    vp = np.zeros((NB, H, B, D), dtype)
    vp[:, :, :, 0] = np.arange(NB)[:, None, None]
    vp[:, :, :, 1] = np.arange(B)[None, None, :]
    vp[:, :, :, 2] = np.arange(H)[None, :, None]
    q = np.zeros((1, H, D), dtype)
    q[..., 0] = 1
    out = oracle.decode(q, kp, vp, table[None, :], np.array([n], np.int32), np.float32(1))
    return out[0]


@pytest.mark.parametrize("B", [1, 4, 8, 16])
def test_translation_matches_append_process(oracle_lib, B):
    rng = np.random.default_rng(B)
    H, n = 2, 37
    nb = -(-n // B)
    NB = nb + 5
    table = rng.permutation(NB)[:nb].astype(np.int32)
    for (blk, pos) in append_process(table, n, B):
        out = tagged_probe(oracle_lib, table, n, B, NB, H, (blk, pos))
        for h in range(H):
            assert tuple(out[h, :3]) == (blk, pos, h)


def test_sharing_diagram(oracle_lib):
    """ricepunchb section 5.1: A -> [7, 3, 12], B -> [7, 3, 9]; the shared
    blocks hold the shared prompt, each sequence's third block its own
    tokens."""
    g = load_golden("sharing_diagram.json")
    B, NB, n = g["block_size"], g["num_blocks"], g["context_len"]
    H, D = 2, 64
    rng = np.random.default_rng(0)
    prompt_k = rng.standard_normal((g["shared_tokens"], H, D)).astype(np.float32)
    prompt_v = rng.standard_normal((g["shared_tokens"], H, D)).astype(np.float32)
    kp = np.full((NB, H, B, D), np.nan, np.float32)
    vp = kp.copy()
    seqs = {}
    for name in ("A", "B"):
        tk = rng.standard_normal((n - g["shared_tokens"], H, D)).astype(np.float32)
        tv = rng.standard_normal((n - g["shared_tokens"], H, D)).astype(np.float32)
        lk, lv = np.concatenate([prompt_k, tk]), np.concatenate([prompt_v, tv])
        W._place(kp, lk, g["tables"][name], B)
        W._place(vp, lv, g["tables"][name], B)
        seqs[name] = (lk, lv)
    tables = np.array([g["tables"]["A"], g["tables"]["B"]], np.int32)
    q = rng.standard_normal((2, H, D)).astype(np.float32)
    scale = np.float32(1 / 8)
    out = oracle_lib.decode(q, kp, vp, tables, np.array([n, n], np.int32), scale)
    for i, name in enumerate(("A", "B")):
        lk, lv = seqs[name]
        qq = torch.from_numpy(q[i].astype(np.float64)).reshape(1, H, 1, D)
        kk = torch.from_numpy(lk.astype(np.float64)).permute(1, 0, 2).reshape(1, H, n, D)
        vv = torch.from_numpy(lv.astype(np.float64)).permute(1, 0, 2).reshape(1, H, n, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=float(scale))
        assert np.allclose(out[i], ref.reshape(H, D).numpy(), rtol=0, atol=1e-13)
    # B's private block changing leaves A untouched, bit for bit
    kp2 = kp.copy()
    kp2[g["private"]["B"]] = 5.0
    out2 = oracle_lib.decode(q, kp2, vp, tables, np.array([n, n], np.int32), scale)
    assert np.array_equal(out2[0], out[0])
    assert not np.array_equal(out2[1], out[1])


# --------------------------------------------------------------------------
# write and copy-on-write
# --------------------------------------------------------------------------

class RefcountManager:
    """Just enough of the pages' KV cache manager to replay the
    copy-on-write example: reference counts, allocate-on-write, copy orders."""

    def __init__(self, B, free):
        self.B, self.free, self.ref = B, list(free), {}

    def share(self, blocks, count):
        for b in blocks:
            self.ref[b] = self.ref.get(b, 0) + count

    def append(self, table, position):
        """Returns (slot, copy pair or None) for writing token `position`."""
        j, off = divmod(position, self.B)
        target = table[j]
        copy = None
        if self.ref[target] > 1:
            new = self.free.pop(0)
            copy = (target, new)
            self.ref[target] -= 1
            self.ref[new] = 1
            table[j] = new
            target = new
        return target * self.B + off, copy


def test_cow_worked_example(oracle_lib):
    """wywy.jp WHERE, parallel sampling: A1 writes first -> block 3 is
    allocated, block 1 copied into it, refcount(1) = 1; A2 then writes into
    block 1 in place.  Replayed through the oracle's copy and write."""
    g = load_golden("cow_example.json")
    B, NB, P = g["block_size"], g["num_blocks"], g["prompt_len"]
    H, D = 2, 64
    rng = np.random.default_rng(1)
    prompt_k = rng.standard_normal((P, H, D)).astype(np.float32)
    prompt_v = rng.standard_normal((P, H, D)).astype(np.float32)
    kp = np.full((NB, H, B, D), np.nan, np.float32)
    vp = kp.copy()
    W._place(kp, prompt_k, g["shared_table"], B)
    W._place(vp, prompt_v, g["shared_table"], B)
    mgr = RefcountManager(B, free=[3, 2])
    mgr.share(g["shared_table"], 2)
    assert {str(k): v for k, v in mgr.ref.items()} == g["refcount_before"]
    tables = {"A1": list(g["shared_table"]), "A2": list(g["shared_table"])}
    new_tok = {}
    for ev in g["events"]:
        name = ev["sample"]
        assert mgr.ref[tables[name][ev["position"] // B]] == ev["target_refcount"]
        slot, copy = mgr.append(tables[name], ev["position"])
        assert slot == ev["slot"]
        assert (list(copy) if copy else None) == ev["copy"]
        assert tables[name] == ev["table_after"]
        assert {str(k): v for k, v in mgr.ref.items()} == ev["refcount_after"]
        if copy:
            oracle_lib.copy_blocks(kp, vp, np.array([copy]))
        key = rng.standard_normal((1, H, D)).astype(np.float32)
        val = rng.standard_normal((1, H, D)).astype(np.float32)
        oracle_lib.write_kv(key, val, kp, vp, np.array([slot]))
        new_tok[name] = (key, val)
    # block 1 holds the prompt's second block + A2's token, block 3 the same
    # prompt part + A1's token, block 0 is untouched
    for name, blk in (("A1", 3), ("A2", 1)):
        assert np.array_equal(kp[blk, :, :P - B], prompt_k[B:].transpose(1, 0, 2))
        assert np.array_equal(kp[blk, :, P - B], new_tok[name][0][0])
        assert np.array_equal(vp[blk, :, P - B], new_tok[name][1][0])
    assert np.array_equal(kp[0], prompt_k[:B].transpose(1, 0, 2))
    # each sample decodes its own history
    tabs = np.array([tables["A1"], tables["A2"]], np.int32)
    q = rng.standard_normal((2, H, D)).astype(np.float32)
    out = oracle_lib.decode(q, kp, vp, tabs, np.array([P + 1, P + 1], np.int32), np.float32(0.125))
    for i, name in enumerate(("A1", "A2")):
        lk = np.concatenate([prompt_k, new_tok[name][0]])
        lv = np.concatenate([prompt_v, new_tok[name][1]])
        qq = torch.from_numpy(q[i].astype(np.float64)).reshape(1, H, 1, D)
        kk = torch.from_numpy(lk.astype(np.float64)).permute(1, 0, 2).reshape(1, H, P + 1, D)
        vv = torch.from_numpy(lv.astype(np.float64)).permute(1, 0, 2).reshape(1, H, P + 1, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.125)
        assert np.allclose(out[i], ref.reshape(H, D).numpy(), rtol=0, atol=1e-13)


@pytest.mark.parametrize("make", [lambda: W.tiny_fp32(),
                                  lambda: W.shared_prompts(num_prompts=4, samples=6, num_heads=2),
                                  lambda: W.short_rows(block_size=8, num_seqs=10, num_heads=2)],
                         ids=["tiny", "cow-small", "short-b8-small"])
def test_step_reproduces_placement(oracle_lib, make):
    """Pools before the step + the step's copies and writes (oracle) equal, bit
    for bit, the generator's own block-granular placement of the full
    sequences."""
    wl = make()
    k, v = wl.k_pool_pre.copy(), wl.v_pool_pre.copy()
    oracle_lib.copy_blocks(k, v, wl.block_mapping)
    oracle_lib.write_kv(wl.new_key, wl.new_value, k, v, wl.slot_mapping)
    u = np.uint32 if wl.dtype == W.F32 else np.uint16
    assert np.array_equal(k.view(u), wl.k_pool.view(u))
    assert np.array_equal(v.view(u), wl.v_pool.view(u))


def test_write_then_read_back(oracle_lib):
    """A token written by write_kv at the manager's next free position is the
    token decode reads as the newest one (one-hot probe)."""
    rng = np.random.default_rng(3)
    B, H, D, NB = 8, 2, 64, 12
    for n_before in (0, 5, 7, 8, 15):
        nb = -(-(n_before + 1) // B)
        table = rng.permutation(NB)[:nb].astype(np.int32)
        blk, pos = append_process(table, n_before + 1, B)[-1]
        kp = np.zeros((NB, H, B, D), np.float32)
        vp = np.zeros((NB, H, B, D), np.float32)
        key = np.zeros((1, H, D), np.float32)
        key[..., 0] = 1000
        val = rng.standard_normal((1, H, D)).astype(np.float32)
        oracle_lib.write_kv(key, val, kp, vp, np.array([blk * B + pos]))
        q = np.zeros((1, H, D), np.float32)
        q[..., 0] = 1
        out = oracle_lib.decode(q, kp, vp, table[None], np.array([n_before + 1], np.int32),
                                np.float32(1))
        assert np.array_equal(out[0], val[0].astype(np.float64))


def test_write_rejects_repeated_slots(oracle_lib):
    kp = np.zeros((4, 1, 8, 64), np.float16)
    key = np.zeros((2, 1, 64), np.float16)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.write_kv(key, key, kp, kp.copy(), np.array([3, 3]))


def test_copy_rejects_conflicting_pairs(oracle_lib):
    kp = np.zeros((6, 1, 8, 64), np.float16)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.copy_blocks(kp, kp.copy(), np.array([[0, 2], [1, 2]]))  # dst twice
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.copy_blocks(kp, kp.copy(), np.array([[0, 2], [2, 3]]))  # dst is a src
    oracle_lib.copy_blocks(kp, kp.copy(), np.array([[0, 2], [0, 3]]))      # fan-out is fine


def test_bad_table_entry_reported(oracle_lib):
    wl = W.tiny_fp32()
    t = wl.block_tables.copy()
    t[3, 1] = wl.num_blocks
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, t, wl.context_lens, wl.scale)


# --------------------------------------------------------------------------
# split-context merge (the GPU's partitioning) versus the unsplit definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("part", [16, 48, 256])
def test_split_merge_identity(oracle_lib, part):
    """Partition the context, keep (max, sum, unnormalised output) per
    partition, merge with exp(m_p - M) weights: equals the unsplit result
    (ricepunchb 3.3: per-block scores, softmax completed by a final
    reduction).  Written independently here in fp64 numpy."""
    wl = W.opt13b_layer(num_seqs=4, num_heads=2)
    ref = run_decode(oracle_lib, wl)
    for b in range(wl.num_seqs):
        n = int(wl.context_lens[b])
        for h in range(wl.num_heads):
            k = wl.logical_k[b][:, h].astype(np.float64)
            v = wl.logical_v[b][:, h].astype(np.float64)
            s = float(wl.scale) * (k @ wl.q[b, h].astype(np.float64))
            ms, ls, os_ = [], [], []
            for p0 in range(0, n, part):
                sp = s[p0:p0 + part]
                m = sp.max()
                e = np.exp(sp - m)
                ms.append(m)
                ls.append(e.sum())
                os_.append(e @ v[p0:p0 + part])
            M = max(ms)
            w = np.exp(np.array(ms) - M)
            merged = (w[:, None] * np.array(os_)).sum(0) / (w * np.array(ls)).sum()
            assert np.allclose(merged, ref[b, h], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# swapping (wywy.jp Keyword "Swapping", Overview scheduling and preemption;
# zhaifeiyue "Scheduling & Preemption" table, row "Swap")
# --------------------------------------------------------------------------

def swap_workload(seed=12):
    """Config-1 sequences with a host pool of another size to swap into."""
    wl = W.tiny_fp32(seed=seed)
    NB = wl.num_blocks
    nb = [-(-int(c) // wl.block_size) for c in wl.context_lens]
    return wl, NB, nb


def test_swap_round_trip_leaves_decode_unchanged(oracle_lib):
    """Every block of every sequence goes to a host pool (other ids, other
    pool size) and back to fresh device blocks; with the tables rewritten
    the decode is exactly the one before (fp64, same order of sums), and the
    host-pool decode with the host tables is too."""
    wl, NB, nb = swap_workload()
    before = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                               wl.scale)
    rng = np.random.default_rng(5)
    used = sorted({int(b) for r, n in zip(wl.block_tables, nb) for b in r[:n]})
    HNB = len(used) + 3
    host_ids = rng.permutation(HNB)[:len(used)]
    to_host = dict(zip(used, host_ids.tolist()))
    shape = (HNB,) + wl.k_pool.shape[1:]
    hk = np.full(shape, np.nan, wl.k_pool.dtype)
    hv = np.full(shape, np.nan, wl.v_pool.dtype)
    oracle_lib.swap_blocks(hk, hv, wl.k_pool, wl.v_pool, [[b, to_host[b]] for b in used])
    host_tables = wl.block_tables.copy()
    for r, n in zip(host_tables, nb):
        r[:n] = [to_host[int(b)] for b in r[:n]]
    on_host = oracle_lib.decode(wl.q, hk, hv, host_tables, wl.context_lens, wl.scale)
    assert np.array_equal(on_host, before)
    # back in: to device blocks other than the ones they came from
    free = [b for b in rng.permutation(NB).tolist()]
    back = dict(zip(host_ids.tolist(), free[:len(used)]))
    dk = np.full(wl.k_pool.shape, np.nan, wl.k_pool.dtype)
    dv = np.full(wl.v_pool.shape, np.nan, wl.v_pool.dtype)
    oracle_lib.swap_blocks(dk, dv, hk, hv, [[h, back[h]] for h in host_ids.tolist()])
    dev_tables = host_tables.copy()
    for r, n in zip(dev_tables, nb):
        r[:n] = [back[int(b)] for b in r[:n]]
    after = oracle_lib.decode(wl.q, dk, dv, dev_tables, wl.context_lens, wl.scale)
    assert np.array_equal(after, before)


def test_swap_equals_whole_block_slices(oracle_lib):
    """Each destination block equals its source block bit for bit (numpy
    whole-block indexing); every other destination block is untouched."""
    rng = np.random.default_rng(8)
    for dtype, (H, B, D) in ((np.float16, (3, 8, 64)), (np.float32, (2, 16, 32))):
        sk = rng.standard_normal((9, H, B, D)).astype(dtype)
        sv = rng.standard_normal((9, H, B, D)).astype(dtype)
        dk = rng.standard_normal((5, H, B, D)).astype(dtype)
        dv = rng.standard_normal((5, H, B, D)).astype(dtype)
        pairs = np.array([[7, 2], [0, 4], [7, 0]])     # one source to two places
        ek, ev = dk.copy(), dv.copy()
        for s, d in pairs:
            ek[d] = sk[s]
            ev[d] = sv[s]
        oracle_lib.swap_blocks(dk, dv, sk, sv, pairs)
        view = np.uint16 if dtype == np.float16 else np.uint32
        assert np.array_equal(dk.view(view), ek.view(view))
        assert np.array_equal(dv.view(view), ev.view(view))


def test_swap_within_one_pool_is_copy_blocks(oracle_lib):
    """With the source pools as destination the swap is the copy-on-write
    block copy (pinned by the worked example)."""
    rng = np.random.default_rng(9)
    k = rng.standard_normal((8, 2, 4, 16)).astype(np.float32)
    v = rng.standard_normal((8, 2, 4, 16)).astype(np.float32)
    pairs = np.array([[1, 3], [1, 6], [2, 0]])
    k2, v2 = k.copy(), v.copy()
    oracle_lib.copy_blocks(k2, v2, pairs)
    oracle_lib.swap_blocks(k, v, k.copy(), v.copy(), pairs)
    assert np.array_equal(k, k2) and np.array_equal(v, v2)


def test_swap_rejects(oracle_lib):
    src = np.zeros((6, 1, 4, 8), np.float32)
    dst = np.zeros((3, 1, 4, 8), np.float32)
    with pytest.raises(oracle_lib.OracleError):          # valid source, no such destination
        oracle_lib.swap_blocks(dst, dst.copy(), src, src, [[5, 3]])
    with pytest.raises(oracle_lib.OracleError):          # no such source
        oracle_lib.swap_blocks(dst, dst.copy(), src, src, [[6, 0]])
    with pytest.raises(oracle_lib.OracleError):          # one destination twice
        oracle_lib.swap_blocks(dst, dst.copy(), src, src, [[0, 1], [2, 1]])


# --------------------------------------------------------------------------
# prefill (wywy.jp Keyword "prompt phase"; WHERE, shared prefix)
# --------------------------------------------------------------------------

def causal_sdpa(k, v, q, scale):
    """torch's causal scaled-dot-product attention in fp64 over one
    sequence: q, k, v [n][H][D] -> [n][H][D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float64)).permute(1, 0, 2)
    kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float64)).permute(1, 0, 2)
    vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64)).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                         scale=float(scale))
    return o.permute(1, 0, 2).numpy()


def small_prefill_cases():
    return [W.prefill_small(),
            W.prefill_small(seed=7, dtype=W.F32, block_size=8,
                            groups=((0, [3]), (16, [16, 1]), (5, [30]), (0, [64]))),
            W.prefill_mix(seed=3, num_heads=2, head_dim=64, num_seqs=4, hi=200)]


@pytest.mark.parametrize("case", [0, 1, 2])
def test_prefill_equals_causal_sdpa(oracle_lib, case):
    """Every query row equals the matching row of torch's causal attention
    over the whole sequence (the query at position p sees tokens 0..p);
    for a suffix over a cached prefix, the rows are the last ones of that
    full causal attention, whatever the prefix's own queries would be --
    the prefix is reused, not recomputed (wywy.jp WHERE, shared prefix)."""
    wl = small_prefill_cases()[case]
    out = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    rng = np.random.default_rng(case)
    for b in range(wl.num_seqs):
        n, m = int(wl.context_lens[b]), int(wl.query_lens[b])
        qs = int(wl.query_start[b])
        q_full = rng.standard_normal((n, wl.num_heads, wl.head_dim))   # prefix queries: any
        q_full[n - m:] = wl.q[qs:qs + m]
        ref = causal_sdpa(wl.logical_k[b], wl.logical_v[b], q_full, wl.scale)[n - m:]
        np.testing.assert_allclose(out[qs:qs + m], ref, rtol=1e-10, atol=1e-12,
                                   err_msg=f"sequence {b}")


def test_prefill_of_one_token_is_decode(oracle_lib):
    """With one query per sequence (its last token) prefill is decode."""
    wl = W.prefill_small(groups=((0, [1]), (9, [1]), (32, [1]), (47, [1])))
    out = oracle_lib.prefill(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                             wl.query_start, wl.scale)
    ref = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens,
                            wl.scale)
    assert np.array_equal(out, ref)


def test_prefill_rejects(oracle_lib):
    wl = W.prefill_small()
    bad = wl.query_start.copy()
    bad[2] = bad[1] + int(wl.context_lens[1]) + 1      # more queries than context
    bad[3:] += bad[2] - wl.query_start[2]
    q = np.zeros((int(bad[-1]), wl.num_heads, wl.head_dim), wl.q.dtype)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.prefill(q, wl.k_pool, wl.v_pool, wl.block_tables, wl.context_lens, bad,
                           wl.scale)
