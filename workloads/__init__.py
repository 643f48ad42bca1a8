"""Seeded synthetic inputs shaped like the PagedAttention pages' workloads.

This module draws context lengths, block placements and K/V/q values, and
lays the values out in block pools.  It holds none of the attention
arithmetic and imports neither the oracle nor the GPU library; both sides of
every parity test take their inputs from here.

Shapes and value recipe
-----------------------
* K, V and q are standard normal, drawn in fp32 and rounded to the element
  type (round to nearest even).  K/V are drawn per sequence in logical token
  order, so the same logical values exist for every block size and every
  placement.
* Pools are [num_blocks][num_heads][block_size][head_dim]; K and V live in
  two separate pools indexed by one block table (the wywy.jp notes, Keyword
  "PagedAttention", say the paper keeps K and V in separate blocks).
* Physical blocks are a seeded random permutation of a pool 1.5x the size of
  the blocks in use ("randomly scattered"); sequences take consecutive slices
  of the permutation in logical-block order.
* Every slot that holds no token (unused blocks, the tail of each last block)
  is NaN, so a kernel that reads an unused slot shows it.
* Block-table entries past a sequence's last block are -1.

Each workload describes one decoding step: first the copy-on-write block
copies (``block_mapping``), then the write of new tokens (``slot_mapping``,
``new_key``, ``new_value``), then the decode over ``context_lens``.  With
host fill it also carries the pools before the step (``k_pool_pre``) and
after it (``k_pool``).

The configurations
------------------
1. tiny fp32: 4 sequences, contexts {1, 17, 33, 50}, 2 heads, head_dim 64,
   B = 16, 32 physical blocks, scale 1/sqrt(64); the step also forks the
   fourth sequence (one copy-on-write copy of its last block), so the decode
   batch holds 5 rows.
2. OPT-13B layer: 64 sequences, 40 heads, head_dim 128, fp16, B = 16,
   contexts lognormal (median 300, sigma 0.9) clipped to [1, 2048].
3. short requests: 256 sequences, contexts uniform in [20, 200], B in
   {8, 16, 32, 64} with the same sequences and logical K/V for every B.
4. shared prefix / copy-on-write: 32 prompts (length uniform [64, 512]) with
   6 samples each (refcount 6 on the prompt's blocks) and private tails of
   uniform [1, 256] tokens; the partial last prompt block is copied for 5 of
   the 6 samples, the 6th keeps the original.
5. long context: 32 sequences, 96 heads, head_dim 128, fp16, B = 16,
   contexts uniform in [4096, 16384].

These stand in for the ShareGPT (long, high-variance) and Alpaca (short)
request mixes the pages evaluate on; no dataset is read.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F16 = "f16"
F32 = "f32"
NP_DTYPES = {F16: np.float16, F32: np.float32}
ELEM_BYTES = {F16: 2, F32: 4}


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [N]
    block_tables: np.ndarray          # int32 [N][MB], -1 past the live entries
    scale: np.float32
    q: np.ndarray                     # [N][H][D] in the element type
    block_mapping: np.ndarray         # int64 [P][2] copy-on-write (src, dst)
    new_key: np.ndarray               # [T][H][D] tokens written by the step
    new_value: np.ndarray
    slot_mapping: np.ndarray          # int64 [T]
    logical_k: list | None = None          # host fill: per sequence [ctx][H][D]
    logical_v: list | None = None
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def np_dtype(self):
        return NP_DTYPES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def pool_shape(self):
        return (self.num_blocks, self.num_heads, self.block_size, self.head_dim)

    def algorithmic_bytes(self) -> int:
        return algorithmic_bytes(self.context_lens, self.num_heads, self.head_dim,
                                 self.block_size, self.elem_bytes)


def algorithmic_bytes(context_lens, num_heads, head_dim, block_size, elem_bytes) -> int:
    """Bytes a decode call must move at minimum: every context token's K and V
    row for every head, plus one 4-byte table entry per block in use."""
    ctx = np.asarray(context_lens, dtype=np.int64)
    blocks = (ctx + block_size - 1) // block_size
    return int(ctx.sum() * num_heads * head_dim * 2 * elem_bytes + 4 * blocks.sum())


def kv_bytes_per_token(num_heads, head_dim, elem_bytes, num_layers=1) -> int:
    """K plus V bytes one token occupies across `num_layers` layers."""
    return 2 * num_heads * head_dim * elem_bytes * num_layers


def _blocks_for(n: int, B: int) -> int:
    return -(-int(n) // B)


def _normal(rng, shape, dtype):
    return rng.standard_normal(shape, dtype=np.float32).astype(dtype)


def _draw_kv(seed_seqs, lengths, H, D, dtype):
    """K then V, [n][H][D] each, from one child stream per entry.  Streams
    are independent, so drawing them on worker threads is deterministic."""
    def one(i):
        r = np.random.default_rng(seed_seqs[i])
        return _normal(r, (int(lengths[i]), H, D), dtype), _normal(r, (int(lengths[i]), H, D), dtype)
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(one, range(len(lengths))))
    return [r[0] for r in res], [r[1] for r in res]


def _place(pool, seq_vals, phys_blocks, B):
    """Lay a sequence's logical rows [n][H][D] into its physical blocks,
    block-granular: logical rows are grouped B at a time (the last group
    padded with NaN) and each group is stored as one block."""
    n, H, D = seq_vals.shape
    nblk = len(phys_blocks)
    padded = np.full((nblk * B, H, D), np.nan, dtype=pool.dtype)
    padded[:n] = seq_vals
    pool[np.asarray(phys_blocks, dtype=np.int64)] = padded.reshape(nblk, B, H, D).transpose(0, 2, 1, 3)


def _next_slot(table_row, tokens_stored, B):
    """Where the manager stores the next token of a sequence that already
    holds `tokens_stored` tokens: the next free position of its last block,
    or position 0 of its next block when the last one is full."""
    blocks_used = _blocks_for(tokens_stored, B)
    if tokens_stored % B == 0:
        return int(table_row[blocks_used]) * B
    return int(table_row[blocks_used - 1]) * B + (tokens_stored - (blocks_used - 1) * B)


def _empty_tables(N, MB):
    return np.full((N, MB), -1, dtype=np.int32)


def _assemble(name, seed, dtype, H, D, B, NB, ctx, tables, q, logical_k, logical_v,
              pre_k_vals, pre_v_vals, seq_blocks, pre_blocks, block_mapping,
              new_key, new_value, slots, host, extra=None):
    wl = Workload(name=name, seed=seed, dtype=dtype, num_heads=H, head_dim=D, block_size=B,
                  num_blocks=NB, context_lens=ctx.astype(np.int32), block_tables=tables,
                  scale=np.float32(1.0 / math.sqrt(D)), q=q,
                  block_mapping=np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2),
                  new_key=new_key, new_value=new_value,
                  slot_mapping=np.asarray(slots, dtype=np.int64), extra=extra or {})
    if host:
        wl.logical_k, wl.logical_v = logical_k, logical_v
        wl.extra["_place_after"] = (logical_k, logical_v, seq_blocks)
        wl.extra["_place_before"] = (pre_k_vals, pre_v_vals, pre_blocks)
    return wl


def _build_pools(wl, key):
    ks, vs, blocks = wl.extra[key]
    k = np.full(wl.pool_shape, np.nan, dtype=wl.np_dtype)
    v = np.full(wl.pool_shape, np.nan, dtype=wl.np_dtype)
    for kv_vals, vv_vals, bl in zip(ks, vs, blocks):
        _place(k, kv_vals, bl, wl.block_size)
        _place(v, vv_vals, bl, wl.block_size)
    return k, v


def _lazy_pool(which, key):
    attr = "_" + which

    def get(self):
        cached = self.__dict__.get(attr)
        if cached is None:
            if key not in self.extra:
                return None
            k, v = _build_pools(self, key)
            self.__dict__["_" + which.replace("v_", "k_", 1)] = k
            self.__dict__["_" + which.replace("k_", "v_", 1)] = v
            cached = self.__dict__[attr]
        return cached

    def put(self, value):
        self.__dict__[attr] = value

    return property(get, put)


def _simple(name, seed, dtype, H, D, B, ctx, NB=None, MB=None, host=True, fork_last=False):
    """Independent sequences with scattered blocks; the step writes each
    sequence's last token (position ctx-1).  With fork_last, the last
    sequence is forked before the step and both copies append a token."""
    ss = np.random.SeedSequence(seed)
    c_place, c_q, c_kv, c_fork = ss.spawn(4)
    npd = NP_DTYPES[dtype]
    ctx = np.asarray(ctx, dtype=np.int64)
    N = len(ctx)
    rows = N + (1 if fork_last else 0)
    q = _normal(np.random.default_rng(c_q), (rows, H, D), npd)
    if host:
        logical_k, logical_v = _draw_kv(c_kv.spawn(N), ctx, H, D, npd)
    else:
        # device fill draws the pools on the GPU; only the written tokens are
        # drawn here (from the same per-sequence streams, first row only)
        logical_k, logical_v = _draw_kv(c_kv.spawn(N), np.ones(N, np.int64), H, D, npd)
    return _place_sequences(name, seed, dtype, H, D, B, ctx, q, logical_k, logical_v,
                            np.random.default_rng(c_place), NB=NB, MB=MB, host=host,
                            fork_rng=np.random.default_rng(c_fork) if fork_last else None)


def _place_sequences(name, seed, dtype, H, D, B, ctx, q, logical_k, logical_v, rng_place,
                     NB=None, MB=None, host=True, fork_rng=None):
    npd = NP_DTYPES[dtype]
    fork_last = fork_rng is not None
    N = len(ctx)
    nblks = [_blocks_for(n, B) for n in ctx]
    used = sum(nblks) + (1 if fork_last else 0)
    if NB is None:
        NB = int(math.ceil(1.5 * used))
    if MB is None:
        MB = max(max(nblks), 1)
    perm = rng_place.permutation(NB)
    if used > NB:
        raise ValueError("pool too small for the blocks in use")
    rows = N + (1 if fork_last else 0)
    tables = _empty_tables(rows, MB)
    seq_blocks = []
    cursor = 0
    for b, nb in enumerate(nblks):
        blocks = perm[cursor:cursor + nb]
        cursor += nb
        tables[b, :nb] = blocks
        seq_blocks.append(list(blocks))
    logical_k, logical_v = list(logical_k), list(logical_v)

    # The step: every sequence appends its token at position ctx-1.
    slots = [_next_slot(tables[b], int(ctx[b]) - 1, B) for b in range(N)]
    new_key = np.stack([logical_k[b][-1] for b in range(N)]) if N else np.zeros((0, H, D), npd)
    new_value = np.stack([logical_v[b][-1] for b in range(N)]) if N else np.zeros((0, H, D), npd)
    pre_k = [lk[:-1] for lk in logical_k]
    pre_v = [lv[:-1] for lv in logical_v]
    pre_blocks = [list(bl) for bl in seq_blocks]
    block_mapping = np.zeros((0, 2), dtype=np.int64)
    all_ctx = np.asarray(ctx, dtype=np.int64)
    extra = {}
    if fork_last:
        # The fork shares every block of the last sequence (refcount 2).  Its
        # append hits the shared, partially filled last block, so that block
        # is copied to a fresh block first and the fork writes into the copy;
        # the original sequence then writes into its own block in place.
        src = int(tables[N - 1, nblks[-1] - 1])
        dst = int(perm[cursor])
        cursor += 1
        tables[N] = tables[N - 1]
        tables[N, nblks[-1] - 1] = dst
        fork_key = _normal(fork_rng, (1, H, D), npd)
        fork_val = _normal(fork_rng, (1, H, D), npd)
        logical_k.append(np.concatenate([logical_k[-1][:-1], fork_key]))
        logical_v.append(np.concatenate([logical_v[-1][:-1], fork_val]))
        seq_blocks.append(list(tables[N, :nblks[-1]]))
        slots.append(_next_slot(tables[N], int(ctx[-1]) - 1, B))
        new_key = np.concatenate([new_key, fork_key])
        new_value = np.concatenate([new_value, fork_val])
        block_mapping = np.array([[src, dst]], dtype=np.int64)
        all_ctx = np.concatenate([all_ctx, all_ctx[-1:]])
        extra["fork_of"] = N - 1
    return _assemble(name, seed, dtype, H, D, B, NB, all_ctx, tables, q, logical_k, logical_v,
                     pre_k, pre_v, seq_blocks, pre_blocks, block_mapping, new_key, new_value,
                     slots, host, extra)


def relayout(wl: Workload, place_seed: int, block_size: int | None = None) -> Workload:
    """The same sequences, query and logical K/V placed afresh: a new random
    permutation, no block shared between sequences, optionally another
    block size.  Host fill only."""
    if wl.logical_k is None:
        raise ValueError("relayout needs a host-filled workload")
    B = block_size or wl.block_size
    return _place_sequences(wl.name + f"-relayout{place_seed}", wl.seed, wl.dtype, wl.num_heads,
                            wl.head_dim, B, wl.context_lens.astype(np.int64), wl.q,
                            wl.logical_k, wl.logical_v,
                            np.random.default_rng(np.random.SeedSequence([wl.seed, 7, place_seed])))


def tiny_fp32(seed=1, host=True):
    return _simple("tiny-fp32", seed, F32, H=2, D=64, B=16, ctx=[1, 17, 33, 50], NB=32, MB=4,
                   host=host, fork_last=True)


def lognormal_lengths(rng, n, median=300.0, sigma=0.9, lo=1, hi=2048):
    z = rng.standard_normal(n)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)


def opt13b_layer(seed=2, host=True, num_seqs=64, num_heads=40):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0]))
    ctx = lognormal_lengths(rng, num_seqs)
    return _simple("opt13b-layer", seed, F16, H=num_heads, D=128, B=16, ctx=ctx, MB=2048 // 16,
                   host=host)


def short_rows(seed=3, block_size=16, host=True, num_seqs=256, num_heads=40):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0]))
    ctx = rng.integers(20, 200, size=num_seqs, endpoint=True)
    return _simple(f"short-b{block_size}", seed, F16, H=num_heads, D=128, B=block_size, ctx=ctx,
                   MB=_blocks_for(200, block_size), host=host)


def long_context(seed=5, host=False, num_seqs=32, num_heads=96, lo=4096, hi=16384):
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0]))
    ctx = rng.integers(lo, hi, size=num_seqs, endpoint=True)
    return _simple("long-opt175b-layer", seed, F16, H=num_heads, D=128, B=16, ctx=ctx,
                   MB=_blocks_for(hi, 16), host=host)


def shared_prompts(seed=4, host=True, num_prompts=32, samples=6, num_heads=40,
            prompt_range=(64, 512), tail_range=(1, 256)):
    """Shared prompts with `samples` parallel samples each.  Before the step
    the pool holds only the prompts (their blocks shared by all samples); the
    step copies the partial last prompt block for all samples but the last
    and then writes every tail token of every sample."""
    H, D, B = num_heads, 128, 16
    ss = np.random.SeedSequence(seed)
    c_len, c_place, c_q, c_kv = ss.spawn(4)
    rl = np.random.default_rng(c_len)
    P = rl.integers(prompt_range[0], prompt_range[1], size=num_prompts, endpoint=True)
    T = rl.integers(tail_range[0], tail_range[1], size=(num_prompts, samples), endpoint=True)
    N = num_prompts * samples
    ctx = (P[:, None] + T).reshape(-1)
    unique = 0
    for p in range(num_prompts):
        pb = _blocks_for(P[p], B)
        unique += pb + (samples - 1 if P[p] % B else 0)
        for s in range(samples):
            unique += _blocks_for(P[p] + T[p, s], B) - pb
    NB = int(math.ceil(1.5 * unique))
    perm = np.random.default_rng(c_place).permutation(NB)
    MB = _blocks_for(prompt_range[1] + tail_range[1], B)
    tables = _empty_tables(N, MB)
    npd = np.float16
    q = _normal(np.random.default_rng(c_q), (N, H, D), npd)
    streams = [c.spawn(1 + samples) for c in c_kv.spawn(num_prompts)]
    prompt_k, prompt_v = _draw_kv([s[0] for s in streams], P, H, D, npd)
    tail_k, tail_v = _draw_kv([t for s in streams for t in s[1:]], T.reshape(-1), H, D, npd)
    cursor = 0
    logical_k, logical_v, seq_blocks = [], [], []
    pre_k, pre_v, pre_blocks = [], [], []
    pairs, slots, nk, nv = [], [], [], []
    for p in range(num_prompts):
        pk, pv = prompt_k[p], prompt_v[p]
        pb = _blocks_for(P[p], B)
        shared = list(perm[cursor:cursor + pb])
        cursor += pb
        pre_k.append(pk)
        pre_v.append(pv)
        pre_blocks.append(shared)
        for s in range(samples):
            b = p * samples + s
            blocks = list(shared)
            if P[p] % B and s < samples - 1:
                dst = int(perm[cursor])
                cursor += 1
                pairs.append((int(shared[-1]), dst))
                blocks[-1] = dst
            extra_blocks = _blocks_for(P[p] + T[p, s], B) - pb
            blocks += list(perm[cursor:cursor + extra_blocks])
            cursor += extra_blocks
            tables[b, :len(blocks)] = blocks
            tk, tv = tail_k[b], tail_v[b]
            logical_k.append(np.concatenate([pk, tk]))
            logical_v.append(np.concatenate([pv, tv]))
            seq_blocks.append(blocks)
            for i in range(int(T[p, s])):
                slots.append(_next_slot(tables[b], int(P[p]) + i, B))
            nk.append(tk)
            nv.append(tv)
    assert cursor == unique
    extra = {"prompt_lens": P, "tail_lens": T, "samples": samples, "unique_blocks": unique}
    return _assemble("shared-prefix-cow", seed, F16, H, D, B, NB, ctx, tables, q,
                     logical_k, logical_v, pre_k, pre_v, seq_blocks, pre_blocks,
                     np.array(pairs, dtype=np.int64).reshape(-1, 2),
                     np.concatenate(nk), np.concatenate(nv), slots, host, extra)


# Host fill: pools before the step (k_pool_pre, v_pool_pre) and after it
# (k_pool, v_pool), [NB][H][B][D], built on first use.
Workload.k_pool_pre = _lazy_pool("k_pool_pre", "_place_before")
Workload.v_pool_pre = _lazy_pool("v_pool_pre", "_place_before")
Workload.k_pool = _lazy_pool("k_pool", "_place_after")
Workload.v_pool = _lazy_pool("v_pool", "_place_after")


def make(name: str, **kw) -> Workload:
    return {"tiny": tiny_fp32, "opt13b": opt13b_layer, "short": short_rows, "cow": shared_prompts,
            "long": long_context}[name](**kw)


# ---------------------------------------------------------------------------
# Device fill: the same metadata, with pool contents drawn on the GPU by
# torch's seeded generator (for sizes where drawing on the host is too slow).
# Logical order is not preserved; every live slot holds N(0,1), every other
# slot NaN.
# ---------------------------------------------------------------------------

def live_rows(wl: Workload):
    """(block ids, number of filled rows) for every block in use."""
    ids, filled = [], []
    B = wl.block_size
    for b in range(wl.num_seqs):
        n = int(wl.context_lens[b])
        nb = _blocks_for(n, B)
        ids.append(wl.block_tables[b, :nb].astype(np.int64))
        f = np.full(nb, B, dtype=np.int64)
        if nb:
            f[-1] = n - (nb - 1) * B
        filled.append(f)
    ids = np.concatenate(ids) if ids else np.zeros(0, np.int64)
    filled = np.concatenate(filled) if filled else np.zeros(0, np.int64)
    # blocks shared by several sequences appear once
    uniq, first = np.unique(ids, return_index=True)
    return uniq, filled[first]


def device_pools(wl: Workload, device, seed_offset=0, chunk_blocks=2048):
    """Allocate and fill (k_pool, v_pool) on `device` with torch's RNG."""
    import torch
    tdt = torch.float16 if wl.dtype == F16 else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(int(wl.seed) * 1000003 + seed_offset)
    shape = wl.pool_shape
    pools = []
    ids, filled = live_rows(wl)
    ids_t = torch.as_tensor(ids, device=device)
    filled_t = torch.as_tensor(filled, device=device)
    row = torch.arange(wl.block_size, device=device)
    for _ in range(2):
        pool = torch.full(shape, float("nan"), dtype=tdt, device=device)
        for c0 in range(0, len(ids), chunk_blocks):
            sel = ids_t[c0:c0 + chunk_blocks]
            vals = torch.randn((len(sel),) + shape[1:], generator=gen, device=device,
                               dtype=torch.float32).to(tdt)
            keep = (row[None, :] < filled_t[c0:c0 + chunk_blocks, None])  # [n][B]
            vals = torch.where(keep[:, None, :, None], vals, torch.full_like(vals, float("nan")))
            pool[sel] = vals
        pools.append(pool)
    return pools[0], pools[1]


# ---------------------------------------------------------------------------
# Multi-step generation: the input program of a decoding loop driven by a
# block manager.  Only ids, events and values are drawn here; where each
# token lands is the manager's decision.
# ---------------------------------------------------------------------------

@dataclass
class GenStep:
    frees: list                      # sequence ids dropped before the step (pruned)
    forks: list                      # (parent, child) pairs made before the step
    seqs: list                       # the step's batch, in order
    key: np.ndarray                  # [n][H][D] the new token of each sequence
    value: np.ndarray
    q: np.ndarray                    # [n][H][D]


@dataclass
class Generation:
    name: str
    seed: int
    dtype: str
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks: int                  # block-table width that fits every sequence
    scale: np.float32
    prompt_keys: list                # per prompt, [L][H][D]; prompt p is sequence p
    prompt_values: list
    steps: list                      # GenStep per decoding step


def generation(seed=11, dtype=F16, num_heads=4, head_dim=128, block_size=16,
               prompt_lens=(37, 5, 64, 100, 1), samples=3, steps=24, churn=0.25):
    """Parallel sampling with beam-like pruning.

    Each prompt is written, then forked into ``samples`` sequences that share
    its blocks (the prompt's own id is the first sample).  Every decoding
    step appends one token to every live sequence.  Before a step, with
    probability ``churn`` one live sequence is dropped and another live
    sequence of the same prompt is forked in its place (a beam candidate
    replaced by a copy of a better one), so forks also happen from sequences
    whose last block is partly filled and both sides then write into it.
    """
    rng = np.random.default_rng(seed)
    dt = NP_DTYPES[dtype]
    H, D, B = num_heads, head_dim, block_size
    P = len(prompt_lens)
    prompt_keys = [_normal(rng, (int(L), H, D), dt) for L in prompt_lens]
    prompt_values = [_normal(rng, (int(L), H, D), dt) for L in prompt_lens]
    group = {p: p for p in range(P)}           # sequence id -> prompt
    live = list(range(P))
    next_id = P
    length = {p: int(L) for p, L in enumerate(prompt_lens)}
    peak_blocks = 0
    out = []
    for t in range(steps):
        frees, forks = [], []
        if t == 0:
            for p in range(P):
                for _ in range(samples - 1):
                    forks.append((p, next_id))
                    group[next_id] = p
                    length[next_id] = length[p]
                    live.append(next_id)
                    next_id += 1
        elif rng.random() < churn:
            victim = live[int(rng.integers(len(live)))]
            mates = [s for s in live if group[s] == group[victim] and s != victim]
            if mates:
                parent = mates[int(rng.integers(len(mates)))]
                live.remove(victim)
                frees.append(victim)
                forks.append((parent, next_id))
                group[next_id] = group[parent]
                length[next_id] = length[parent]
                live.append(next_id)
                next_id += 1
        n = len(live)
        out.append(GenStep(frees=frees, forks=forks, seqs=list(live),
                           key=_normal(rng, (n, H, D), dt), value=_normal(rng, (n, H, D), dt),
                           q=_normal(rng, (n, H, D), dt)))
        for s in live:
            length[s] += 1
        # upper bound on blocks in use: every sequence privately owning its blocks
        peak_blocks = max(peak_blocks, sum(_blocks_for(length[s], B) for s in live))
    max_len = max(length.values())
    return Generation(name="generation", seed=seed, dtype=dtype, num_heads=H, head_dim=D,
                      block_size=B, num_blocks=peak_blocks + P + 4,
                      max_blocks=_blocks_for(max_len, B), scale=np.float32(1.0 / math.sqrt(D)),
                      prompt_keys=prompt_keys, prompt_values=prompt_values, steps=out)


def beam_search(seed=17, dtype=F16, num_heads=4, head_dim=128, block_size=16,
                prompt_lens=(37, 5, 64, 100, 1), width=4, steps=24, spread=1.0):
    """Beam search with fork and prune every step.

    Each prompt is written, then forked into ``width`` beams sharing its
    blocks.  Before every later step each request draws ``width`` parents
    from its ``width`` live beams, with replacement, with probabilities
    softmax(spread * N(0,1)) (a stand-in for the candidates' scores: no
    model is run).  A beam drawn by no one is pruned (freed); a beam drawn
    c times continues as one candidate and is forked c - 1 times, so the
    candidates share its blocks, and the partly filled last block is copied
    when they append (the wywy.jp notes, WHERE beam search: candidates share
    blocks, a pruned candidate's blocks lose a reference, copy-on-write on
    the shared partial block).  Every live beam then appends one token.
    """
    rng = np.random.default_rng(seed)
    dt = NP_DTYPES[dtype]
    H, D, B = num_heads, head_dim, block_size
    P = len(prompt_lens)
    prompt_keys = [_normal(rng, (int(L), H, D), dt) for L in prompt_lens]
    prompt_values = [_normal(rng, (int(L), H, D), dt) for L in prompt_lens]
    beams = [[p] for p in range(P)]           # per request, its live beam ids
    next_id = P
    length = {p: int(L) for p, L in enumerate(prompt_lens)}
    peak_blocks = 0
    out = []
    for t in range(steps):
        frees, forks = [], []
        for r in range(P):
            cur = beams[r]
            if t == 0:
                parents = [cur[0]] * width
            else:
                logits = spread * rng.standard_normal(len(cur))
                prob = np.exp(logits - logits.max())
                prob /= prob.sum()
                parents = [cur[i] for i in rng.choice(len(cur), size=width, p=prob)]
            counts = {b: parents.count(b) for b in cur}
            new = []
            for b in cur:
                if counts[b] == 0:
                    frees.append(b)
                    continue
                new.append(b)
                for _ in range(counts[b] - 1):
                    forks.append((b, next_id))
                    length[next_id] = length[b]
                    new.append(next_id)
                    next_id += 1
            beams[r] = new
        live = [b for r in range(P) for b in beams[r]]
        n = len(live)
        out.append(GenStep(frees=frees, forks=forks, seqs=live,
                           key=_normal(rng, (n, H, D), dt), value=_normal(rng, (n, H, D), dt),
                           q=_normal(rng, (n, H, D), dt)))
        for b in live:
            length[b] += 1
        peak_blocks = max(peak_blocks, sum(_blocks_for(length[b], B) for b in live))
    max_len = max(length.values())
    return Generation(name="beam-search", seed=seed, dtype=dtype, num_heads=H, head_dim=D,
                      block_size=B, num_blocks=peak_blocks + P + 4,
                      max_blocks=_blocks_for(max_len, B), scale=np.float32(1.0 / math.sqrt(D)),
                      prompt_keys=prompt_keys, prompt_values=prompt_values, steps=out)


# ---------------------------------------------------------------------------
# Generation under memory pressure: groups of parallel samples that outgrow
# the GPU pool, so that some group must be preempted (and swapped out) for
# others to go on.  Inputs are keyed by (sequence, token index), not by step,
# so a run that preempts and a run that does not feed every sequence the same
# tokens.
# ---------------------------------------------------------------------------

def token_inputs(seed, seq, t, num_heads, head_dim, dtype):
    """(key, value, q), [H][D] each, of generated token t of sequence seq."""
    r = np.random.default_rng([int(seed), int(seq), int(t)])
    dt = NP_DTYPES[dtype]
    return tuple(_normal(r, (num_heads, head_dim), dt) for _ in range(3))


@dataclass
class Pressure:
    name: str
    seed: int
    dtype: str
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int                 # GPU pool: too small for every group at once
    num_host_blocks: int            # swap space: as many blocks as the GPU pool
    max_blocks: int
    scale: np.float32
    groups: list                    # per group (arrival order), its sequence ids; the first is the prompt's
    gen_lens: dict                  # sequence id -> tokens it generates
    prompt_keys: list               # per group, [L][H][D]
    prompt_values: list


def pressure(seed=13, dtype=F16, num_heads=4, head_dim=64, block_size=16,
             prompt_lens=(40, 70, 25, 90, 33), samples=3, gen=(20, 60), squeeze=0.55):
    """Groups of `samples` sequences forked from one prompt each generate a
    uniform [gen] number of tokens.  The GPU pool holds `squeeze` times the
    blocks every group would need at its longest, but never less than one
    group's worst case plus one block (so the earliest group can always
    finish).  The swap space has as many blocks as the GPU pool (the pages'
    bound on CPU swap space)."""
    rng = np.random.default_rng(seed)
    dt = NP_DTYPES[dtype]
    H, D, B = num_heads, head_dim, block_size
    groups, gen_lens, pk, pv = [], {}, [], []
    sid = 0
    need_all, need_max = 0, 0
    for L in prompt_lens:
        ids = list(range(sid, sid + samples))
        sid += samples
        groups.append(ids)
        pk.append(_normal(rng, (int(L), H, D), dt))
        pv.append(_normal(rng, (int(L), H, D), dt))
        lens = [int(x) for x in rng.integers(gen[0], gen[1] + 1, size=samples)]
        gen_lens.update(zip(ids, lens))
        # the prompt's full blocks stay shared; each sample ends up with
        # private blocks from the prompt's partial block on
        need = int(L) // B + sum(_blocks_for(int(L) + n, B) - int(L) // B for n in lens)
        need_all += need
        need_max = max(need_max, need)
    num_blocks = max(int(squeeze * need_all), need_max + 1)
    max_len = max(prompt_lens) + gen[1]
    return Pressure(name="pressure", seed=seed, dtype=dtype, num_heads=H, head_dim=D,
                    block_size=B, num_blocks=num_blocks, num_host_blocks=num_blocks,
                    max_blocks=_blocks_for(max_len, B), scale=np.float32(1.0 / math.sqrt(D)),
                    groups=groups, gen_lens=gen_lens, prompt_keys=pk, prompt_values=pv)


# ---------------------------------------------------------------------------
# Prefill (prompt phase): every sequence's last tokens are queries over its
# whole context, causally.  A group's members share a cached prefix (its
# full blocks shared in their tables; the partial prefix block copied per
# member, as copy-on-write leaves it) and each has its own suffix; a full
# prefill is a group of one with an empty prefix.
# ---------------------------------------------------------------------------

@dataclass
class PrefillWorkload:
    name: str
    seed: int
    dtype: str
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray       # int32 [N]
    query_start: np.ndarray        # int32 [N+1]: rows of q / out per sequence
    block_tables: np.ndarray       # int32 [N][MB], -1 past the live entries
    scale: np.float32
    q: np.ndarray                  # [T][H][D]
    k_pool: np.ndarray             # [NB][H][B][D]; NaN in every slot that holds no token
    v_pool: np.ndarray
    logical_k: list                # per sequence, [n][H][D]
    logical_v: list
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self):
        return len(self.context_lens)

    @property
    def query_lens(self):
        return np.diff(self.query_start)

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self):
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self):
        return ELEM_BYTES[self.dtype]

    def visible_tokens(self) -> int:
        """Sum over query tokens of the keys each one attends to (p + 1)."""
        tot = 0
        for n, m in zip(self.context_lens.tolist(), self.query_lens.tolist()):
            tot += m * (n - m) + m * (m + 1) // 2
        return tot

    def algorithmic_flops(self) -> int:
        """2 D flops for q.k and 2 D for p.v per (query, visible key, head)."""
        return 4 * self.head_dim * self.num_heads * self.visible_tokens()

    def algorithmic_bytes(self) -> int:
        """q and out once, each sequence's K and V once."""
        H, D, s = self.num_heads, self.head_dim, self.elem_bytes
        T = int(self.query_start[-1])
        return 2 * T * H * D * s + 2 * int(self.context_lens.sum()) * H * D * s


def _prefill_build(name, seed, dtype, H, D, B, groups, host=True):
    """groups: list of (prefix_len, [suffix_len, ...])."""
    npd = NP_DTYPES[dtype]
    ss = np.random.SeedSequence(seed)
    c_place, c_vals = ss.spawn(2)
    g_streams = c_vals.spawn(len(groups))
    ctx, qlen, plan = [], [], []
    used = 0
    for (P, sufs) in groups:
        used += P // B
        for S in sufs:
            ctx.append(P + S)
            qlen.append(S)
            used += _blocks_for(P + S, B) - P // B
    N = len(ctx)
    NB = max(int(math.ceil(1.5 * used)), 1)
    MB = max(max(_blocks_for(n, B) for n in ctx), 1)
    perm = np.random.default_rng(c_place).permutation(NB)
    tables = _empty_tables(N, MB)
    kp = np.full((NB, H, B, D), np.nan, npd)
    vp = np.full((NB, H, B, D), np.nan, npd)
    logical_k, logical_v, qs = [], [], []
    cursor, b = 0, 0
    for gi, (P, sufs) in enumerate(groups):
        streams = g_streams[gi].spawn(1 + len(sufs))
        r = np.random.default_rng(streams[0])
        pk, pv = _normal(r, (P, H, D), npd), _normal(r, (P, H, D), npd)
        shared = perm[cursor:cursor + P // B]
        cursor += P // B
        for j, blk in enumerate(shared):
            kp[blk] = pk[j * B:(j + 1) * B].transpose(1, 0, 2)
            vp[blk] = pv[j * B:(j + 1) * B].transpose(1, 0, 2)
        for si, S in enumerate(sufs):
            r = np.random.default_rng(streams[1 + si])
            sk, sv = _normal(r, (S, H, D), npd), _normal(r, (S, H, D), npd)
            qs.append(_normal(r, (S, H, D), npd))
            k = np.concatenate([pk, sk])
            v = np.concatenate([pv, sv])
            n = P + S
            own = perm[cursor:cursor + _blocks_for(n, B) - P // B]
            cursor += len(own)
            row = list(shared) + list(own)
            tables[b, :len(row)] = row
            for j in range(P // B, len(row)):
                lo, hi = j * B, min((j + 1) * B, n)
                kp[row[j], :, :hi - lo] = k[lo:hi].transpose(1, 0, 2)
                vp[row[j], :, :hi - lo] = v[lo:hi].transpose(1, 0, 2)
            logical_k.append(k)
            logical_v.append(v)
            b += 1
    q = np.concatenate(qs) if qs else np.zeros((0, H, D), npd)
    query_start = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    return PrefillWorkload(name=name, seed=seed, dtype=dtype, num_heads=H, head_dim=D,
                           block_size=B, num_blocks=NB,
                           context_lens=np.asarray(ctx, dtype=np.int32), query_start=query_start,
                           block_tables=tables, scale=np.float32(1.0 / math.sqrt(D)), q=q,
                           k_pool=kp, v_pool=vp, logical_k=logical_k, logical_v=logical_v,
                           extra={"groups": [(P, list(s)) for P, s in groups]})


def prefill_mix(seed=41, dtype=F16, num_heads=40, head_dim=128, block_size=16, num_seqs=16,
                median=300.0, sigma=0.9, lo=1, hi=2048):
    """Full prefills of num_seqs prompts, lengths lognormal (median 300,
    sigma 0.9, clipped to [1, 2048]: the long, varied request mix)."""
    rng = np.random.default_rng(seed)
    lens = lognormal_lengths(rng, num_seqs, median, sigma, lo, hi)
    return _prefill_build("prefill-mix", seed, dtype, num_heads, head_dim, block_size,
                          [(0, [int(n)]) for n in lens])


def prefill_shared(seed=42, dtype=F16, num_heads=40, head_dim=128, block_size=16, groups=4,
                   members=8, prefix=(256, 1024), suffix=(16, 256)):
    """Shared prefixes (a long system prompt or few-shot examples) cached
    once per group; each member's own suffix tokens are the queries."""
    rng = np.random.default_rng(seed)
    spec = []
    for _ in range(groups):
        P = int(rng.integers(prefix[0], prefix[1] + 1))
        spec.append((P, [int(x) for x in rng.integers(suffix[0], suffix[1] + 1, size=members)]))
    return _prefill_build("prefill-shared", seed, dtype, num_heads, head_dim, block_size, spec)


def prefill_small(seed=43, dtype=F16, num_heads=2, head_dim=64, block_size=16,
                  groups=((0, [1]), (0, [17]), (0, [40]), (21, [1, 5]), (48, [33]))):
    """A few short cases: one token, ragged tails, a prefix ending mid-block
    shared by two members, a prefix on a block boundary."""
    return _prefill_build("prefill-small", seed, dtype, num_heads, head_dim, block_size,
                          [(P, list(s)) for P, s in groups])
