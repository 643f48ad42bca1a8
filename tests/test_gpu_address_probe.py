"""Bit-exact GPU address probe of pa_decode and pa_decode_append.

The decode's attention output hides a one-token addressing mistake inside
the floating-point tolerance once contexts are long (one wrong row of ten
thousand moves the output by about |dv| / 10^4).  This probe makes the
output *be* the row the kernel read, so every address is checked bit for
bit: for every (sequence b, head h) the test picks one target position t,
stores K = 64 q[b][h] at t's slot and K = 0 in every other live slot, so
that t's score exceeds all others by hundreds (its weight is 1 and every
other weight underflows to exactly 0, in fp32 as in fp16).  Each V row holds
a tag of its own (slot, head), c = (phys * H + h) * B + offset, written as
small nonzero integers that fp16 holds exactly (c mod 2048, c div 2048,
then a nonlinear pattern of c and d, so that no mix of rows is another row).  The output
row must then equal, bit for bit, the V row at the slot that the pages'
address translation gives for t (the ricepunchb.github.io notes, section
3.2: block index t / B, offset t % B, physical block from the block table;
the zhaifeiyue.github.io summary, method paragraph, block-wise equation):

* reading any other slot for t (wrong table entry, offset, head or pool)
  yields another tag, or NaN (every slot that holds no token is NaN, K and
  V), or the mean of the V rows when t's slot is never read;
* rounds move the target through every logical position of every sequence
  (position (round * H + h) mod ctx_b for head h), across block sizes 8 to
  64, head_dim 64 and 128, partition boundaries (partitions of 64 tokens,
  merged by the second pass), the ragged last tile, a row above 8192 tokens,
  both launch forms (the grid without host lengths; the host-planned list,
  4-wave and 8-wave), and the fused append's last token, which is read from
  the new rows and stored to its slot.

The expected row comes from the test's own table lookup; the fp64 oracle on
the same pools, rounded to the element type, is checked to give the same
bits on the first and last round of every case.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

GAIN = 64.0   # K row of the target = GAIN * q: exact in fp32 and fp16 (a power of two)


def announce(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def tag_rows(code, D, npd):
    """Rows [..., D] naming integer codes (< 2^22) in values fp16 holds
    exactly, none of them 0 (so no sign of zero can differ): 1 + code mod
    2048, 1 + code div 2048, then 1 + a nonlinear pattern of (c, d) with
    c = code mod 2039, so that a weighted mix of tag rows is not itself a
    tag row: ((c + 1)(d + 3) mod 2039 * 7919 + c^2 mod 1009 + 13 d^2) mod
    2039."""
    code = np.asarray(code, dtype=np.int32)
    d = np.arange(D, dtype=np.int32)
    c = code[..., None] % 2039
    rows = ((c + 1) * (d + 3) % 2039 * 7919 + c * c % 1009 + 13 * d * d) % 2039
    rows[..., 0] = code % 2048
    rows[..., 1] = code // 2048
    return (rows + 1).astype(npd)


def tag_code(row):
    """The code a tag row names (NaN rows: None)."""
    r = np.asarray(row, dtype=np.float64)
    if not np.isfinite(r[:2]).all():
        return None
    return int(abs(r[0])) - 1 + 2048 * (int(abs(r[1])) - 1)


class Probe:
    """Pools, tables and the per-round targets of one probe case."""

    def __init__(self, name, seed, dtype, H, D, B, ctx, device):
        # placement and tables from the seeded generator (no pool values drawn there)
        self.wl = W._simple(name, seed, dtype, H, D, B, ctx, host=False)
        wl = self.wl
        self.H, self.D, self.B = H, D, B
        self.N = wl.num_seqs
        self.npd = W.NP_DTYPES[dtype]
        self.ctx = wl.context_lens.astype(np.int64)
        self.tables = wl.block_tables
        NB = wl.num_blocks
        ids, filled = W.live_rows(wl)
        live = np.zeros((NB, B), bool)
        for p, f in zip(ids.tolist(), filled.tolist()):
            live[p, :f] = True
        self.live = live
        # V tags of each (slot, head); NaN where no token is stored
        code = (np.arange(NB, dtype=np.int32)[:, None, None] * H
                + np.arange(H, dtype=np.int32)[None, :, None]) * B \
            + np.arange(B, dtype=np.int32)[None, None, :]
        self.v_host = tag_rows(code, D, self.npd)
        mask = np.broadcast_to(live[:, None, :, None], self.v_host.shape)
        self.v_host[~mask] = np.nan
        self.k_host = np.zeros(self.v_host.shape, self.npd)
        self.k_host[~mask] = np.nan
        qrng = np.random.default_rng(seed + 1000)
        self.q_host = qrng.standard_normal((self.N, H, D), dtype=np.float32).astype(self.npd)
        self.scale = np.float32(1.0 / np.sqrt(D))
        self.device = device
        self.q = dev(self.q_host, device)
        self.k = dev(self.k_host, device)
        self.v = dev(self.v_host, device)
        self.t_tables = dev(self.tables, device)
        self.t_ctx = dev(wl.context_lens, device)
        self.hot = dev((GAIN * self.q_host.astype(np.float32)).astype(self.npd), device)
        self.rounds = int(-(-int(self.ctx.max()) // H))
        self.prev = None

    def targets(self, rnd):
        """Target position per (b, h) of round `rnd`: (rnd * H + h) mod ctx_b."""
        t = (rnd * self.H + np.arange(self.H)[None, :]) % np.maximum(self.ctx, 1)[:, None]
        return t.astype(np.int64)

    def slots_of(self, t):
        """(phys, offset) of logical position t for every (b, h), by table lookup."""
        b = np.arange(self.N)[:, None]
        phys = self.tables[b, t // self.B].astype(np.int64)
        return phys, t % self.B

    def set_targets(self, t, skip=None):
        """K = GAIN q at each (b, h)'s target slot, 0 at the previous round's."""
        hh = np.broadcast_to(np.arange(self.H)[None, :], t.shape)
        bb = np.broadcast_to(np.arange(self.N)[:, None], t.shape)
        if self.prev is not None:
            pp, ph, po = self.prev
            self.k[pp, ph, po] = 0
        phys, off = self.slots_of(t)
        keep = np.ones(t.shape, bool) if skip is None else ~skip
        sel = (torch.as_tensor(phys[keep], device=self.device),
               torch.as_tensor(hh[keep], device=self.device),
               torch.as_tensor(off[keep], device=self.device))
        self.k[sel] = self.hot[torch.as_tensor(bb[keep], device=self.device),
                               torch.as_tensor(hh[keep], device=self.device)]
        self.prev = sel
        return phys, off

    def expected(self, phys, off):
        hh = np.arange(self.H)[None, :]
        return self.v_host[phys, hh, off]            # [N][H][D]

    def host_pools(self, phys, off, skip=None):
        """The pools of this round on the host (for the oracle cross-check)."""
        k = self.k_host.copy()
        hh = np.broadcast_to(np.arange(self.H)[None, :], phys.shape)
        bb = np.broadcast_to(np.arange(self.N)[:, None], phys.shape)
        keep = np.ones(phys.shape, bool) if skip is None else ~skip
        k[phys[keep], hh[keep], off[keep]] = (GAIN * self.q_host[bb[keep], hh[keep]]
                                              .astype(np.float32)).astype(self.npd)
        return k, self.v_host.copy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16 if a.dtype == np.float16 else np.uint32)


def describe_mismatch(probe, got, want, t, rnd, where, new_rows=None):
    """Fail with the first few differing (sequence, head) rows: the target,
    the expected slot, the raw output values, and the pool slots (or new
    rows) holding exactly the output row, if any."""
    bad = np.argwhere(np.any(bits(got) != bits(want), axis=-1))
    hb = probe.H * probe.B
    flat = bits(probe.v_host).reshape(-1, probe.D)
    lines = []
    for b, h in bad[:6]:
        b, h = int(b), int(h)
        row = got[b, h]
        hits = np.flatnonzero(np.all(flat == bits(row)[None, :], axis=1))
        where_from = [f"slot (block {c // hb}, head {c // probe.B % probe.H}, offset {c % probe.B})"
                      for c in hits[:3]]
        if new_rows is not None:
            nr = bits(new_rows).reshape(-1, probe.D)
            where_from += [f"new row of (b={i // probe.H}, h={i % probe.H})"
                           for i in np.flatnonzero(np.all(nr == bits(row)[None, :], axis=1))[:3]]
        c = tag_code(want[b, h])
        lines.append(
            f"(b={b}, h={h}) ctx {int(probe.ctx[b])} target t={int(t[b, h])} expected code {c} "
            f"values {want[b, h, :4].tolist()}; got values {row[:4].tolist()} found at "
            f"{where_from or 'no pool row'}")
    raise AssertionError(f"{where}: round {rnd}: {len(bad)} (sequence, head) rows differ:\n  "
                         + "\n  ".join(lines))


def run_decode(pa, probe, form, part):
    out = torch.empty_like(probe.q)
    maxctx = int(probe.ctx.max())
    host = probe.wl.context_lens if form == "listed" else None
    ws = pa.new_workspace(probe.N, probe.H, probe.D, maxctx, part or 256, device=probe.device)
    pa.pa_decode(out, probe.q, probe.k, probe.v, probe.t_tables, probe.t_ctx,
                 float(probe.scale), maxctx, partition_size=part, workspace=ws,
                 host_context_lens=host)
    return out


def check_forms(probe, forms, outs, want, t, rnd):
    """Every launch form's output equals the expected rows; otherwise fail
    with the report of each form that differs."""
    errors = []
    for (f, p), o in zip(forms, outs):
        got = o.cpu().numpy()
        if not np.array_equal(bits(got), bits(want)):
            try:
                describe_mismatch(probe, got, want, t, rnd, f"{f} partition {p}")
            except AssertionError as e:
                errors.append(str(e))
    if errors:
        raise AssertionError("\n".join(errors))


SHORT_CTX = [1, 2, 3, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 129, 200, 255, 257, 300]


@pytest.mark.parametrize("dtype,D,B", [(W.F32, 64, 8), (W.F32, 64, 16), (W.F32, 64, 32),
                                       (W.F32, 64, 64), (W.F32, 128, 8), (W.F32, 128, 16),
                                       (W.F32, 128, 32), (W.F32, 128, 64), (W.F16, 128, 16),
                                       (W.F16, 64, 8)])
def test_every_address_bit_exact(pa, oracle_lib, device, dtype, D, B):
    """Every logical position of 19 sequences (1 to 300 tokens) through the
    grid launch and the host-planned list (4-wave at these lengths), with one
    partition and with 64-token partitions merged by the second pass."""
    H = 8
    probe = Probe(f"probe-{dtype}-D{D}-B{B}", 300 + D + B, dtype, H, D, B, SHORT_CTX, device)
    forms = [("grid", 0), ("listed", 0), ("grid", 64), ("listed", 64)]
    announce(f"address probe {dtype} D{D} B{B}: {probe.rounds} rounds x {len(forms)} launch forms")
    for rnd in range(probe.rounds):
        t = probe.targets(rnd)
        phys, off = probe.set_targets(t)
        want = probe.expected(phys, off)
        outs = [run_decode(pa, probe, f, p) for f, p in forms]
        torch.cuda.synchronize()
        check_forms(probe, forms, outs, want, t, rnd)
        if rnd in (0, probe.rounds - 1):
            k, v = probe.host_pools(phys, off)
            ref = oracle_lib.decode(probe.q_host, k, v, probe.tables, probe.wl.context_lens,
                                    probe.scale)
            assert np.array_equal(bits(ref.astype(probe.npd)), bits(want)), \
                "the oracle's translation disagrees with the table lookup"


def test_long_row_every_address(pa, oracle_lib, device):
    """A row of 8300 tokens (above the 8192 that switches the default
    partition to 4096 tokens, so the grid launch merges three partitions)
    beside short rows, 64 heads x head_dim 64, fp32, B 16: every position of
    every row, grid and host-planned launches."""
    ctx = [8300, 1, 17, 700, 4096, 4097]
    H, D, B = 64, 64, 16
    probe = Probe("probe-long", 77, W.F32, H, D, B, ctx, device)
    forms = [("grid", 0), ("listed", 0)]
    announce(f"address probe long row: {probe.rounds} rounds")
    for rnd in range(probe.rounds):
        t = probe.targets(rnd)
        phys, off = probe.set_targets(t)
        want = probe.expected(phys, off)
        outs = [run_decode(pa, probe, f, p) for f, p in forms]
        torch.cuda.synchronize()
        check_forms(probe, forms, outs, want, t, rnd)
        if rnd % 40 == 0:
            announce(f"long row: round {rnd} of {probe.rounds}")
        if rnd in (0, probe.rounds - 1):
            k, v = probe.host_pools(phys, off)
            ref = oracle_lib.decode(probe.q_host, k, v, probe.tables, probe.wl.context_lens,
                                    probe.scale)
            assert np.array_equal(bits(ref.astype(np.float32)), bits(want))


@pytest.mark.parametrize("dtype,D,B", [(W.F32, 128, 16), (W.F32, 64, 8), (W.F16, 128, 64)])
@pytest.mark.parametrize("form,part", [("grid", 0), ("listed", 0), ("grid", 64),
                                       ("listed", 64)])
def test_fused_append_every_address(pa, oracle_lib, device, dtype, D, B, form, part):
    """pa_decode_append: the last position of each row is read from the new
    rows (its pool slot holds NaN before every call, so a read of the slot
    shows), every other position from its slot; after each call the slot
    holds the new rows, bit for bit."""
    H = 8
    probe = Probe(f"probe-append-{dtype}-D{D}-B{B}", 500 + D + B, dtype, H, D, B, SHORT_CTX,
                  device)
    N = probe.N
    last = probe.ctx - 1
    lp, lo = probe.slots_of(np.broadcast_to(last[:, None], (N, H)))
    lp, lo = lp[:, 0], lo[:, 0]
    slot_map = dev((lp * B + lo).astype(np.int64), device)
    lp_t, lo_t = torch.as_tensor(lp, device=device), torch.as_tensor(lo, device=device)
    # new V rows: tags of b * H + h, negated (unlike any pool tag)
    new_v_host = (-tag_rows(np.arange(N)[:, None] * H + np.arange(H)[None, :], D,
                            np.float32)).astype(probe.npd)
    new_v = dev(new_v_host, device)
    announce(f"fused-append probe {dtype} D{D} B{B} {form} partition {part}: "
             f"{probe.rounds} rounds")
    maxctx = int(probe.ctx.max())
    host = probe.wl.context_lens if form == "listed" else None
    ws = pa.new_workspace(N, H, D, maxctx, part or 256, device=device)
    for rnd in range(probe.rounds):
        t = probe.targets(rnd)
        is_last = t == last[:, None]
        phys, off = probe.set_targets(t, skip=is_last)
        new_k_host = np.where(is_last[..., None],
                              (GAIN * probe.q_host.astype(np.float32)).astype(probe.npd),
                              np.zeros((), probe.npd)).astype(probe.npd)
        new_k = dev(new_k_host, device)
        probe.k[lp_t, :, lo_t] = float("nan")
        probe.v[lp_t, :, lo_t] = float("nan")
        out = torch.empty_like(probe.q)
        pa.pa_decode_append(out, probe.q, new_k, new_v, probe.k, probe.v, probe.t_tables,
                            probe.t_ctx, slot_map, float(probe.scale), maxctx,
                            partition_size=part, workspace=ws, host_context_lens=host)
        torch.cuda.synchronize()
        want = probe.expected(phys, off)
        want = np.where(is_last[..., None], new_v_host, want)
        got = out.cpu().numpy()
        if not np.array_equal(bits(got), bits(want)):
            describe_mismatch(probe, got, want, t, rnd, f"append {form} partition {part}",
                              new_rows=new_v_host)
        # the new rows are stored at their slots, every head
        assert np.array_equal(bits(probe.k[lp_t, :, lo_t].cpu().numpy()), bits(new_k_host))
        assert np.array_equal(bits(probe.v[lp_t, :, lo_t].cpu().numpy()), bits(new_v_host))
        if rnd in (0, probe.rounds - 1):
            k, v = probe.host_pools(phys, off, skip=is_last)
            slots = (lp * B + lo).astype(np.int64)
            oracle_lib.write_kv(new_k_host, new_v_host, k, v, slots)
            ref = oracle_lib.decode(probe.q_host, k, v, probe.tables, probe.wl.context_lens,
                                    probe.scale)
            assert np.array_equal(bits(ref.astype(probe.npd)), bits(want))
