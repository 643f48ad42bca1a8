"""Benchmark: paged decode attention at the OPT-13B layer shape on one MI355X.

One step is the whole hot path over one batch: the copy-on-write block
copies due this step (none in this workload: no sequence shares blocks),
the write of every sequence's new token K/V into its slot (pa_write_kv),
and paged decode attention over every sequence's context (pa_decode).  The
workload is 64 sequences x 40 heads x head_dim 128, fp16, block size 16,
context lengths lognormal (median 300, sigma 0.9) clipped to [1, 2048], in a
pool 1.5x the blocks in use, randomly scattered.  Steps rotate over L layer
pools (separate K/V pools per layer, the same block tables, as every layer
of a model shares them) so that repeats are not served from the 256 MiB
Infinity Cache.

Prints one JSON line.  Timing: HIP events on the stream the kernels run on
(torch's current stream) around the timed region of exactly K steps, after
W untimed warm-up steps; then a second pass of K steps with events around
every decode launch (its average duration is the roofline's), and the same
steps replayed from a captured HIP graph (reported beside, not as value).

Also times the CPU oracle on the host (the full batch of layer 0, all host
threads) as a reported baseline, and checks sampled GPU rows against it.

``--workload generation`` instead times the multi-step decoding loop that
the host block manager drives (parallel sampling with beam-like pruning at
the same layer shape, every step over all L layers) and prints its own line;
``--workload beam`` does the same for beam search with fork and prune at
every step.
``--workload swap`` times block swapping between the device pool and a
pinned host pool against the block size and prints its own line.
``--workload prefill`` times paged prefill attention (MFMA) on a full
prompt mix and on shared-prefix requests and prints its own line.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: HBM GB/s (% of peak), decode steps/s at OPT-13B shape"
PEAK_HBM_GBS = 8000.0
# decoder layers of the model whose layer shape each decode workload takes (OPT-13B, OPT-175B)
MODEL_LAYERS = {"opt13b": 40, "short": 40, "long": 96}
COUNTER_FILE = os.path.join(ROOT, "profiles", "pa_decode_opt13b_hbm_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_05_amd", "csrc", f)
                  for f in ("pa_decode.hip", "pa_kernels.h")]
PREFILL_COUNTER_FILE = os.path.join(ROOT, "profiles", "pa_prefill_opt13b_hbm_counters.txt")
PREFILL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_05_amd", "csrc", f)
                   for f in ("pa_prefill.hip", "pa_prefill.h", "pa_kernels.h")]


def kernel_digest(sources=None):
    """Digest of the kernel sources' code: comments and whitespace are
    dropped first, so an edit of a comment keeps stored counters valid and
    any change to the code invalidates them."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES if sources is None else sources:
        with open(f, encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(counter_file=COUNTER_FILE, sources=None):
    """HBM bytes per call from the committed rocprofv3 counter runs
    (``key: value`` lines), if they were taken on the kernel source as it is
    now; otherwise None."""
    try:
        with open(counter_file) as f:
            c = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    c = {k.strip(): v.strip() for k, v in c.items()}
    if c.get("kernel_digest") != kernel_digest(sources):
        return None
    try:
        return int(c["hbm_bytes_per_call"])
    except (KeyError, ValueError):
        return None


def calibrate_copy():
    """One plain device copy of known size (1 GiB read, 1 GiB written), for
    scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 28  # fp32 elements: 1 GiB
    a = torch.empty(n, dtype=torch.float32, device="cuda:0")
    a.fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "torch.mul fp32 copy", "read_bytes": 4 * n,
                      "write_bytes": 4 * n}), flush=True)
    return 0


PEAK_FP16_TFLOPS = 2500.0   # dense fp16 MFMA, MI355X


def bench_prefill(args):
    """Paged prefill at the OPT-13B layer shape (40 heads x head_dim 128,
    fp16, B = 16): (a) full prefill of 16 prompts, lengths lognormal
    (median 300, sigma 0.9, clipped [1, 2048]); (b) 4 groups x 8 requests
    sharing a cached prefix of 256..1024 tokens, each with its own 16..256
    query tokens.  Throughput = causal attention FLOPs (4 D per query, key
    and head) / time per call, from K calls back to back between two events
    (each call between its own events is reported beside).  Every call gets a 64-slot workspace (the
    planner splits nothing in (a) or (b)); single requests (one 2048-token
    prompt; 256 query tokens over a 4096-token cached prefix) are reported
    beside, whole and split."""
    import torch

    import paged_kv_cache_05_amd as pa
    import workloads as W

    device = torch.device("cuda:0")
    K = max(1, min(args.steps, 50))
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    stream = torch.cuda.current_stream()
    ws = pa.new_prefill_workspace(40, 128, slots=64, device=device)

    def timed(wl, workspace):
        q, kp, vp = dev(wl.q), dev(wl.k_pool), dev(wl.v_pool)
        tables, ctx, qs = dev(wl.block_tables), dev(wl.context_lens), dev(wl.query_start)
        out = torch.empty_like(q)
        call = lambda: pa.pa_prefill(out, q, kp, vp, tables, ctx, qs, float(wl.scale),
                                     wl.max_context_len, wl.max_query_len,
                                     host_query_start=wl.query_start,
                                     host_context_lens=wl.context_lens, workspace=workspace)
        for _ in range(max(args.warmup, 1)):
            call()
        torch.cuda.synchronize()
        # K calls back to back between two events (the rate of a loop that
        # keeps the stream fed), then K calls each between its own events
        # (that span also holds the host's planning and launch of the call)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(K):
            call()
        t1.record(stream)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        for a, b in evs:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        per_call = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        got = out.cpu().numpy()
        if not np.isfinite(got).all():
            raise SystemExit(f"bench: non-finite prefill output ({wl.name})")
        return t0.elapsed_time(t1) / K, got, per_call

    res = {}
    for name, wl in (("mix", W.prefill_mix()), ("shared", W.prefill_shared())):
        ms, got, per_call = timed(wl, ws)
        res[name] = {"wl": wl, "ms": ms, "flops": wl.algorithmic_flops(),
                     "bytes": wl.algorithmic_bytes(), "out": got, "per_call": per_call}
    # Single requests on an otherwise idle GPU, whole and with the key range
    # of their heaviest query tiles split over the workspace.
    single = {}
    for name, groups in (("one_prompt_2048", ((0, [2048]),)),
                         ("suffix_256_over_4096", ((4096, [256]),))):
        wl = W.prefill_small(seed=51, num_heads=40, head_dim=128, block_size=16, groups=groups)
        ms_whole, _, _ = timed(wl, None)
        ms_split, _, _ = timed(wl, ws)
        f = wl.algorithmic_flops() / 1e12
        single[name] = {"ms_whole": round(ms_whole, 5), "ms_split": round(ms_split, 5),
                        "TFLOPs_whole": round(f / (ms_whole * 1e-3), 2),
                        "TFLOPs_split": round(f / (ms_split * 1e-3), 2)}
    mix = res["mix"]
    tflops = mix["flops"] / (mix["ms"] * 1e-3) / 1e12
    launch_tflops = mix["flops"] / (mix["per_call"] * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        if not os.path.exists(oracle.LIBRARY):
            oracle.build()
        wl = mix["wl"]
        threads = oracle.threads_available()
        # sample: the last 64 query rows of the longest prompt (the most keys each)
        b = int(np.argmax(wl.context_lens))
        n, m, q0 = int(wl.context_lens[b]), int(wl.query_lens[b]), int(wl.query_start[b])
        k = min(64, m)
        t = time.perf_counter()
        ref = oracle.prefill(wl.q[q0 + m - k:q0 + m], wl.k_pool, wl.v_pool,
                             wl.block_tables[b:b + 1], np.array([n], np.int32),
                             np.array([0, k], np.int32), wl.scale, threads=threads)
        secs = time.perf_counter() - t
        sample_flops = 4 * wl.head_dim * wl.num_heads * sum(n - k + i + 1 for i in range(k))
        cpu = {"value": round(sample_flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
               "kind": "oracle",
               "sample": f"last {k} query rows of the {n}-token prompt, fp64, {secs:.2f} s"}
        got = mix["out"][q0 + m - k:q0 + m].astype(np.float64)
        cpu["parity"] = bool(np.all(np.abs(got - ref) <= 2e-3 + 1e-2 * np.abs(ref)))

    sh = res["shared"]
    rec = {
        "metric": "paged prefill attention TFLOP/s (causal, MFMA fp16), OPT-13B layer shape",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(mix["ms"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded; lognormal prompt lengths, N(0,1) q/K/V, scattered blocks)",
        "config": {"workload": "full prefill of 16 prompts, lognormal lengths median 300 "
                               "clipped [1,2048], 40 heads x 128, block 16",
                   "sum_prompt": int(mix["wl"].context_lens.sum()),
                   "max_prompt": mix["wl"].max_context_len,
                   "algorithmic_gflop": round(mix["flops"] / 1e9, 3)},
        "roofline": {"bound": "mfma", "achieved": round(launch_tflops, 2),
                     "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(launch_tflops / PEAK_FP16_TFLOPS, 4),
                     "traffic": measured_traffic(PREFILL_COUNTER_FILE, PREFILL_SOURCES),
                     "kernel": "prefill_listed_kernel<128,16>",
                     "from": "algorithmic FLOPs / mean event span of one call"},
        "hbm_GBps_algorithmic": round(mix["bytes"] / (mix["ms"] * 1e-3) / 1e9, 1),
        "ms_per_call_events": round(mix["per_call"], 5),
        "shared_prefix": {"ms": round(sh["ms"], 5),
                          "TFLOPs": round(sh["flops"] / (sh["ms"] * 1e-3) / 1e12, 2),
                          "query_tokens": int(sh["wl"].query_start[-1]),
                          "context_tokens": int(sh["wl"].context_lens.sum()),
                          "groups": sh["wl"].extra["groups"].__len__()},
        "single_request": single,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction, before protocol overhead


def bench_swap(args):
    """Swap of one OPT-13B-shaped layer's KV for 32768 tokens (40 heads x
    head_dim 128, fp16, K and V: 671 MB each way) between the device pool and
    a pinned host pool, blocks mapped at random, for block sizes 1..256:
    pa_swap_blocks (one launch; the kernel moves the bytes over PCIe) against
    one hipMemcpyAsync per block and pool (torch copy_ of pinned views: the
    DMA path whose per-transfer cost grows with the number of blocks), with
    one contiguous copy of the same bytes as the ceiling."""
    import torch

    import paged_kv_cache_05_amd as pa

    device = torch.device("cuda:0")
    H, D, T = 40, 128, 32768
    es = 2
    total = 2 * T * H * D * es                    # K and V bytes moved per direction
    stream = torch.cuda.current_stream()
    reps = max(1, min(args.steps, 5))

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e-3

    # ceiling: one contiguous copy each way
    flat_d = torch.empty(total // 2, dtype=torch.float16, device=device)
    flat_h = torch.empty(total // 2, dtype=torch.float16).pin_memory()
    ceil_out = total / timed(lambda: flat_h.copy_(flat_d, non_blocking=True), reps) / 1e9
    ceil_in = total / timed(lambda: flat_d.copy_(flat_h, non_blocking=True), reps) / 1e9
    del flat_d, flat_h

    rng = np.random.default_rng(31)
    curve = {}
    for B in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        NB = T // B
        shape = (NB, H, B, D)
        dk = torch.randn(shape, dtype=torch.float16, device=device)
        dv = torch.randn(shape, dtype=torch.float16, device=device)
        hk = torch.empty(shape, dtype=torch.float16).pin_memory()
        hv = torch.empty(shape, dtype=torch.float16).pin_memory()
        perm_d, perm_h = rng.permutation(NB), rng.permutation(NB)
        out_pairs = torch.from_numpy(np.stack([perm_d, perm_h], 1).astype(np.int64)).to(device)
        in_pairs = torch.from_numpy(np.stack([perm_h, perm_d], 1).astype(np.int64)).to(device)
        k_out = timed(lambda: pa.pa_swap_blocks(hk, hv, dk, dv, out_pairs), reps)
        k_in = timed(lambda: pa.pa_swap_blocks(dk, dv, hk, hv, in_pairs), reps)
        # the round trip must give back the same bits
        ref = dk[int(perm_d[0])].clone()
        pa.pa_swap_blocks(hk, hv, dk, dv, out_pairs)
        dk.zero_()
        pa.pa_swap_blocks(dk, dv, hk, hv, in_pairs)
        torch.cuda.synchronize()
        if not torch.equal(dk[int(perm_d[0])], ref):
            raise SystemExit(f"bench: swap round trip changed block bits at B={B}")
        pd, ph = perm_d.tolist(), perm_h.tolist()

        def dma_out():
            for d_, h_ in zip(pd, ph):
                hk[h_].copy_(dk[d_], non_blocking=True)
                hv[h_].copy_(dv[d_], non_blocking=True)

        def dma_in():
            for d_, h_ in zip(pd, ph):
                dk[d_].copy_(hk[h_], non_blocking=True)
                dv[d_].copy_(hv[h_], non_blocking=True)

        w0 = time.perf_counter()
        d_out = timed(dma_out, 1)
        d_in = timed(dma_in, 1)
        curve[B] = {"blocks": NB, "block_bytes": H * B * D * es,
                    "kernel_out_GBps": round(total / k_out / 1e9, 2),
                    "kernel_in_GBps": round(total / k_in / 1e9, 2),
                    "dma_per_block_out_GBps": round(total / d_out / 1e9, 2),
                    "dma_per_block_in_GBps": round(total / d_in / 1e9, 2)}
        print(f"# B={B}: {curve[B]} ({time.perf_counter() - w0:.1f} s of per-block copies)",
              file=sys.stderr, flush=True)
        del dk, dv, hk, hv
        torch.cuda.empty_cache()
    c16 = curve[16]
    value = 2 * total / (total / (c16["kernel_out_GBps"] * 1e9) + total / (c16["kernel_in_GBps"] * 1e9)) / 1e9
    rec = {
        "metric": "KV block swap GB/s (device <-> pinned host, out and in), block size 16",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": round(2 * total / (value * 1e9) * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (N(0,1) K/V, random block mapping)",
        "config": {"workload": "swap one OPT-13B-shaped layer's KV of 32768 tokens out and in",
                   "num_heads": H, "head_dim": D, "tokens": T, "bytes_each_way": total},
        "roofline": {"bound": "pcie", "achieved": round(value, 2), "peak": PCIE_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / PCIE_PEAK_GBS, 4), "traffic": None,
                     "kernel": "move_blocks_kernel"},
        "contiguous_copy_GBps": {"out": round(ceil_out, 2), "in": round(ceil_in, 2)},
        "curve_by_block_size": curve,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_generation(args):
    """Decoding loop driven by the host block manager: 16 prompts (lengths
    lognormal, median 300, clipped [1, 2048]) x 4 parallel samples sharing
    each prompt's blocks, 40 heads x head_dim 128, fp16, B = 16; before a
    step, with probability 1/4, one sample is pruned and another sample of
    its prompt forked in its place.  With --workload beam: 16 prompts x
    beam width 4, every beam drawn again from its parents each step (pruned
    beams freed, repeated parents forked).  A step = the manager's decisions and
    their upload (once), then for each of L layers: copy-on-write copies,
    KV write, paged decode.  Model GEMMs are not part of this path."""
    import torch

    import paged_kv_cache_05_amd as pa
    from paged_kv_cache_05_amd import manager as M
    import workloads as W

    device = torch.device("cuda:0")
    L, K, Wm = args.layers, args.steps, args.warmup
    rng = np.random.default_rng(21)
    plens = W.lognormal_lengths(rng, 16)
    beam = args.workload == "beam"
    if beam:
        g = W.beam_search(seed=21, dtype=W.F16, num_heads=40, head_dim=128, block_size=16,
                          prompt_lens=tuple(int(x) for x in plens), width=4, steps=Wm + K)
        label = "beam search 16 prompts x width 4"
    else:
        g = W.generation(seed=21, dtype=W.F16, num_heads=40, head_dim=128, block_size=16,
                         prompt_lens=tuple(int(x) for x in plens), samples=4, steps=Wm + K,
                         churn=0.25)
        label = "parallel sampling 16 prompts x 4 samples"
    H, D, B = g.num_heads, g.head_dim, g.block_size
    shape = (g.num_blocks, H, B, D)
    pools = [tuple(torch.full(shape, float("nan"), dtype=torch.float16, device=device)
                   for _ in range(2)) for _ in range(L)]
    m = M.BlockManager(g.num_blocks, B)
    stepper = M.DecodeStepper(m, pools, g.max_blocks, args.partition)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    for p, (pk, pv) in enumerate(zip(g.prompt_keys, g.prompt_values)):
        m.add(p)
        slots, _ = m.append([p] * len(pk))
        dk, dv, ds = to(pk), to(pv), to(slots)
        for k, v in pools:
            pa.pa_write_kv(dk, dv, k, v, ds)
    inputs = [(to(st.key), to(st.value), to(st.q)) for st in g.steps]
    outs = [torch.empty_like(x[2]) for x in inputs]
    scale = float(g.scale)
    stream = torch.cuda.current_stream()
    host_s, mgr_s, copies, tokens, dec_bytes, blocks_used, private_need = [], [], 0, 0, 0, [], []
    evs = []

    def one(i, timed):
        nonlocal copies, tokens, dec_bytes
        st = g.steps[i]
        t = time.perf_counter()
        for s_ in st.frees:
            m.free(s_)
        for parent, child in st.forks:
            m.fork(parent, child)
        plan = stepper.plan(st.seqs)
        if timed:
            host_s.append(time.perf_counter() - t)
            mgr_s.append(plan.host_seconds)
            copies += len(plan.pairs)
            tokens += len(st.seqs)
            dec_bytes += L * W.algorithmic_bytes(plan.context_lens, H, D, B, 2)
            blocks_used.append(g.num_blocks - m.num_free)
            private_need.append(int(sum(-(-int(c) // B) for c in plan.context_lens)))
        key, value, q = inputs[i]
        for layer in range(L):
            if timed:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            stepper.layer(plan, layer, key, value, q, scale, outs[i])
            if timed:
                b.record(stream)
                evs.append((a, b))

    for i in range(Wm):
        one(i, False)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t0.record(stream)
    for i in range(Wm, Wm + K):
        one(i, True)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = t0.elapsed_time(t1)
    layer_ms = np.array([a.elapsed_time(b) for a, b in evs])
    for o in outs[Wm:]:
        if not torch.isfinite(o).all():
            raise SystemExit("bench: non-finite output in the generation loop")
    ms_per_step = total_ms / K
    rec = {
        "metric": "decode-loop attention tokens/s (block manager + COW + KV write + paged "
                  "decode, all layers)",
        "value": round(tokens / (total_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded; lognormal prompt lengths, N(0,1) q/K/V)",
        "config": {"workload": f"{label}, OPT-13B-shaped "
                               f"attention, {L} layers per step",
                   "num_heads": H, "head_dim": D, "block_size": B, "layers": L,
                   "prompt_lens_sum": int(sum(plens)), "num_blocks": g.num_blocks},
        "host_manager_us_mean": round(1e6 * float(np.mean(mgr_s)), 2),
        "host_manager_us_p90": round(1e6 * float(np.percentile(mgr_s, 90)), 2),
        "host_plan_incl_staging_wait_us_mean": round(1e6 * float(np.mean(host_s)), 2),
        "wall_ms_per_step": round(1e3 * wall / K, 5),
        "layer_ms_mean": round(float(layer_ms.mean()), 5),
        "layer_attention_GBps": round(dec_bytes / (L * K) / (float(layer_ms.mean()) * 1e-3) / 1e9, 1),
        "cow_copies_per_step": round(copies / K, 3),
        "forks_per_step": round(sum(len(g.steps[i].forks) for i in range(Wm, Wm + K)) / K, 3),
        "prunes_per_step": round(sum(len(g.steps[i].frees) for i in range(Wm, Wm + K)) / K, 3),
        "blocks_in_use_final": blocks_used[-1],
        "blocks_if_private_final": private_need[-1],
    }
    print(json.dumps(rec), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="layer pools to rotate over")
    ap.add_argument("--partition", type=int, default=0, help="pa_decode partition_size (0: default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra HIP-graph replay measurement")
    ap.add_argument("--split-step", action="store_true",
                    help="pa_write_kv then pa_decode (two launches) instead of the fused "
                         "pa_decode_append")
    ap.add_argument("--no-host-lengths", action="store_true",
                    help="do not pass host-side context lengths to pa_decode")
    ap.add_argument("--config", choices=["opt13b", "short", "long", "cow"], default="opt13b",
                    help="decode workload: opt13b (the default line: 64 seqs x 40 heads, "
                         "lognormal contexts), short (256 seqs of 20-200 tokens), long (32 seqs "
                         "x 96 heads of 4096-16384 tokens), cow (32 prompts x 6 samples sharing "
                         "prompt blocks: copy, write and decode timed apart and together); the "
                         "CPU baseline and the stored HBM counters cover opt13b only")
    ap.add_argument("--no-reference", action="store_true",
                    help="skip the reference stream and gather reads")
    ap.add_argument("--block-size", type=int, default=16, choices=[8, 16, 32, 64],
                    help="block size of the short workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run one 1 GiB device copy (counter calibration) and exit")
    ap.add_argument("--workload", choices=["decode", "generation", "beam", "swap", "prefill"],
                    default="decode",
                    help="decode: one layer's decode step (the default line); generation: the "
                         "block-manager decoding loop over all layers (beam: the same with "
                         "beam search forking and pruning every step); swap: block swap "
                         "device <-> pinned host against the block size; prefill: paged "
                         "prefill attention")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU mode); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        return 2

    if args.calibrate_copy:
        return calibrate_copy()
    if args.workload in ("generation", "beam"):
        return bench_generation(args)
    if args.workload == "swap":
        return bench_swap(args)
    if args.workload == "prefill":
        return bench_prefill(args)

    if args.config == "cow":
        return bench_cow(args)
    return bench_decode(args)


def bench_lib():
    """libpa_bench.so (the reference read kernels, include/pa_bench.h), loaded
    after torch and libpa.so so that it binds to torch's HIP runtime."""
    import ctypes

    import paged_kv_cache_05_amd as pa
    pa.library()
    path = os.path.join(ROOT, "paged_kv_cache_05_amd", "libpa_bench.so")
    if not os.path.exists(path):
        raise SystemExit(f"bench: {path} is not built (python -m paged_kv_cache_05_amd._build)")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.pa_bench_stream_read.argtypes = [vp, sz, i32, i32, vp, vp]
    lib.pa_bench_stream_read.restype = i32
    lib.pa_bench_gather_read.argtypes = [vp, vp, sz, vp, i32, i32, vp, vp]
    lib.pa_bench_gather_read.restype = i32
    return lib


def tile_offsets(wl):
    """Byte offsets of every (block, head) tile a decode of `wl` reads, once
    per distinct block: (phys * H + h) * B * D * element bytes."""
    import workloads as W
    ids, _ = W.live_rows(wl)
    H, B, D, s = wl.num_heads, wl.block_size, wl.head_dim, wl.elem_bytes
    off = (ids[:, None] * H + np.arange(H)[None, :]) * (B * D * s)
    return off.reshape(-1).astype(np.int64)


def reference_reads(wl, pools, reps):
    """The bandwidth ceilings the decode is read against, measured live:
    (a) a stream over a 4 GiB buffer, non-temporal 16-byte loads, the best
    of six launch shapes (1024 / 2048 / 4096 workgroups of 256 threads, one
    or four loads per thread in flight); (b) a gather of exactly the workload's
    (block, head) tiles of K and V at their places in the rotated layer
    pools, one wave per tile, the same loads.  Events around every launch."""
    import torch
    lib = bench_lib()
    device = pools[0][0].device
    stream = torch.cuda.current_stream()
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=device)

    def timed(fn, n):
        fn(0)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            fn(i)
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3

    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    buf.fill_(1)

    def stream_with(grid, unroll):
        def once(_):
            rc = lib.pa_bench_stream_read(buf.data_ptr(), nbytes, grid, unroll, sink.data_ptr(),
                                          stream.cuda_stream)
            if rc != 0:
                raise SystemExit(f"bench: pa_bench_stream_read returned {rc}")
        return once

    # a few launch shapes; the ceiling is the best of them
    shapes = {f"{g}x256 threads, {u} KiB/wave in flight": (g, u)
              for g in (1024, 2048, 4096) for u in (1, 4)}
    stream_rates = {name: nbytes / timed(stream_with(*gu), max(3, reps // 20)) / 1e9
                    for name, gu in shapes.items()}
    best = max(stream_rates, key=stream_rates.get)
    del buf
    torch.cuda.empty_cache()
    offs = torch.from_numpy(tile_offsets(wl)).to(device)
    piece = wl.block_size * wl.head_dim * wl.elem_bytes
    pool_bytes = pools[0][0].numel() * pools[0][0].element_size()

    def gather_once(i):
        k, v = pools[i % len(pools)]
        rc = lib.pa_bench_gather_read(k.data_ptr(), v.data_ptr(), pool_bytes, offs.data_ptr(),
                                      offs.numel(), piece, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise SystemExit(f"bench: pa_bench_gather_read returned {rc}")

    t_gather = timed(gather_once, reps)
    gather_bytes = 2 * offs.numel() * piece
    return {"stream_GBps": round(stream_rates[best], 1), "stream_bytes": nbytes,
            "stream_best_shape": best,
            "stream_GBps_by_shape": {k: round(v, 1) for k, v in stream_rates.items()},
            "gather_GBps": round(gather_bytes / t_gather / 1e9, 1),
            "gather_bytes": gather_bytes, "gather_pieces": int(offs.numel()),
            "gather_ms": round(t_gather * 1e3, 5),
            "what": "stream: 4 GiB read once, best of six launch shapes; gather: this "
                    "workload's (block, head) K and V tiles (whole blocks) at their places in "
                    "the rotated layer pools, one wave per tile"}


def single_thread_oracle(pools0, wl_default):
    """The oracle on one thread for the first three configurations (the
    tiny fp32 batch, the OPT-13B layer of this run, the short-request batch
    at B = 16): seconds per full decode call."""
    import oracle
    import workloads as W
    import torch
    res = {}
    tiny = W.tiny_fp32()
    t = time.perf_counter()
    oracle.decode(tiny.q, tiny.k_pool, tiny.v_pool, tiny.block_tables, tiny.context_lens,
                  tiny.scale, threads=1)
    res["tiny_fp32_s"] = round(time.perf_counter() - t, 5)
    kh, vh = pools0[0].cpu().numpy(), pools0[1].cpu().numpy()
    t = time.perf_counter()
    oracle.decode(wl_default.q, kh, vh, wl_default.block_tables, wl_default.context_lens,
                  wl_default.scale, threads=1)
    res["opt13b_layer_s"] = round(time.perf_counter() - t, 3)
    short = W.short_rows(block_size=16, host=False)
    sk, sv = W.device_pools(short, pools0[0].device)
    skh, svh = sk.cpu().numpy(), sv.cpu().numpy()
    del sk, sv
    torch.cuda.empty_cache()
    t = time.perf_counter()
    oracle.decode(short.q, skh, svh, short.block_tables, short.context_lens, short.scale,
                  threads=1)
    res["short_rows_s"] = round(time.perf_counter() - t, 3)
    res["opt13b_layer_GBps"] = round(wl_default.algorithmic_bytes() / res["opt13b_layer_s"] / 1e9, 3)
    res["short_rows_GBps"] = round(short.algorithmic_bytes() / res["short_rows_s"] / 1e9, 3)
    return res


def bench_decode(args):
    import torch

    import paged_kv_cache_05_amd as pa
    import workloads as W

    device = torch.device("cuda:0")
    # The default line is the OPT-13B-shaped layer; the other decode
    # workloads are the short-request batch (any block size) and the
    # long-context OPT-175B-shaped layer, whose pools (24 GB each) already
    # dwarf the caches, so two of them rotate.
    wl = {"opt13b": lambda: W.opt13b_layer(host=False),
          "short": lambda: W.short_rows(block_size=args.block_size, host=False),
          "long": lambda: W.long_context(host=False)}[args.config]()
    N, H, D, B = wl.num_seqs, wl.num_heads, wl.head_dim, wl.block_size
    L = min(args.layers, 2) if args.config == "long" else args.layers
    default_config = args.config == "opt13b"
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    pools = [W.device_pools(wl, device, seed_offset=layer) for layer in range(L)]
    tables, ctx = dev(wl.block_tables), dev(wl.context_lens)
    q = dev(wl.q)
    out = torch.empty_like(q)
    new_k, new_v, slots = dev(wl.new_key), dev(wl.new_value), dev(wl.slot_mapping)
    copies = dev(wl.block_mapping)
    maxctx = wl.max_context_len
    ws = pa.new_workspace(N, H, D, maxctx, args.partition or 256, device=device)
    scale = float(wl.scale)
    # The step's scheduler knows every context length on the host; passing
    # them lets pa_decode launch only non-empty work items, largest first.
    host_ctx = None if args.no_host_lengths else wl.context_lens
    part = pa.pa_decode_partition_size(N, H, D, maxctx, args.partition, host_ctx,
                                       ws.numel() if ws is not None else 0)
    merges = -(-maxctx // part) > 1
    # Waves per workgroup: 8 for the default workload; the planner may pick
    # fewer for batches of short rows, shown as W.
    waves = "8" if default_config or host_ctx is None else "W"
    kernel = ("decode_listed_kernel" if host_ctx is not None else "decode_kernel") + \
        f"<{'f16' if wl.dtype == W.F16 else 'f32'},{D},{B},{waves}>" + \
        (" + merge_kernel" if merges else "") + \
        ("" if args.split_step else " (fused append: pa_decode_append)")
    stream = torch.cuda.current_stream()

    def step(i, ev=None, plain=False):
        k, v = pools[i % L]
        pa.pa_copy_blocks(k, v, copies)              # no pairs in this workload: no launch
        if ev is not None:
            ev[0].record(stream)
        if plain:
            pa.pa_decode(out, q, k, v, tables, ctx, scale, maxctx, args.partition, ws,
                         host_context_lens=host_ctx)
        elif args.split_step:
            pa.pa_write_kv(new_k, new_v, k, v, slots)
            pa.pa_decode(out, q, k, v, tables, ctx, scale, maxctx, args.partition, ws,
                         host_context_lens=host_ctx)
        else:
            pa.pa_decode_append(out, q, new_k, new_v, k, v, tables, ctx, slots, scale, maxctx,
                                args.partition, ws, host_context_lens=host_ctx)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    # The timed region: exactly K steps, events only at its two ends.
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / K

    # A second pass of K steps with HIP events around every decode launch,
    # for the kernel's average launch duration (the roofline); its events
    # are kept out of the timed region above.
    def event_pass(plain):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        for i in range(K):
            step(i, evs[i], plain=plain)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    dec_ms = event_pass(False)
    # A third pass: pa_decode alone (no new-row store), the call the
    # bandwidth target names.
    plain_ms = event_pass(True)

    # The same steps replayed from a HIP graph (one captured step per layer
    # pool), as a serving loop that captures its launches would run them.
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(L):
                step(i)
        g.replay()
        torch.cuda.synchronize()
        reps = max(1, K // L)
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ga.record(stream)
        for _ in range(reps):
            g.replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph_ms = ga.elapsed_time(gb) / (reps * L)
        del g

    # The headline byte count: every context token's K and V row for every
    # head, plus one 4-byte table entry per block in use.  The step also
    # stores each sequence's new K/V rows once (reported, not credited).
    decode_bytes = wl.algorithmic_bytes()
    new_rows_bytes = 2 * N * H * D * wl.elem_bytes
    value = decode_bytes / (ms_per_step * 1e-3) / 1e9
    dec_mean = float(dec_ms.mean())
    plain_mean = float(plain_ms.mean())
    # The roofline's launch duration: when a step is exactly one launch of
    # the decode kernel (no copy pairs, one partition, fused append), the
    # timed region's events give it directly (K launches back to back);
    # otherwise the second pass's events around each call (decode, merge and
    # any write), whose spans also hold each call's dispatch.
    single_launch = len(wl.block_mapping) == 0 and not merges and not args.split_step
    launch_ms = ms_per_step if single_launch else dec_mean
    achieved = decode_bytes / (launch_ms * 1e-3) / 1e9
    # the stored counters cover the default workload's fused call only
    traffic = None if args.split_step or not default_config else measured_traffic()

    refs = reference_reads(wl, pools, max(20, min(K, 100))) if not args.no_reference else None

    # Output of layer 0 for the parity sample and the CPU baseline.
    k0, v0 = pools[0]
    step(0)                                      # the timed call, on layer 0's pools
    torch.cuda.synchronize()
    gpu_out = out.cpu().numpy().astype(np.float64)
    if not np.isfinite(gpu_out).all():
        raise SystemExit("bench: non-finite decode output")

    cpu = None
    parity = None
    if not args.no_cpu_baseline and default_config:
        import oracle
        if not os.path.exists(oracle.LIBRARY):
            oracle.build()
        kh, vh = k0.cpu().numpy(), v0.cpu().numpy()
        threads = oracle.threads_available()
        t = time.perf_counter()
        ref = oracle.decode(wl.q, kh, vh, wl.block_tables, wl.context_lens, wl.scale,
                            threads=threads)
        secs = time.perf_counter() - t
        cpu = {"value": round(decode_bytes / secs / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"one full decode call of layer 0 ({N} seqs x {H} heads, "
                         f"sum ctx {int(wl.context_lens.sum())}), fp64, {secs:.2f} s; "
                         f"{1.0 / secs:.3f} decode steps/s",
               "single_thread": single_thread_oracle((k0, v0), wl)}
        err = np.abs(gpu_out - ref)
        parity = bool(np.all(err <= 2e-3 + 1e-2 * np.abs(ref)))

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if wl.dtype == W.F16 else "f32",
        "data": "synthetic (seeded context lengths, N(0,1) q/K/V, scattered blocks)",
        "config": {
            "workload": {"opt13b": "OPT-13B-shaped single-layer decode step",
                         "short": "short-request high-batch decode step",
                         "long": "long-context OPT-175B-shaped single-layer decode step"}[
                             args.config] + " (new-token store + paged decode)",
            "num_seqs": N, "num_heads": H, "head_dim": D, "block_size": B,
            "context_lens": {"opt13b": "lognormal median 300 sigma 0.9 clipped [1,2048]",
                             "short": "uniform [20,200]",
                             "long": "uniform [4096,16384]"}[args.config],
            "sum_context": int(wl.context_lens.sum()), "max_context": maxctx,
            "num_blocks": wl.num_blocks, "layer_pools_rotated": L,
            "partition_size": part,
            "host_planned_launch": host_ctx is not None,
        },
        "value_bytes": "sum ctx x H x D x 2 x 2 B + 4 B per block in use",
        "decode_steps_per_s": round(1000.0 / ms_per_step, 1),
        "tokens_per_s": round(N * 1000.0 / ms_per_step, 1),
        "model_equivalent_steps_per_s": {
            "value": round(1000.0 / ms_per_step / MODEL_LAYERS[args.config], 1),
            "layers": MODEL_LAYERS[args.config],
            "what": "context only: this one layer's step rate divided by the model's layer count "
                    "(attention alone, every layer the same shape)"},
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "decode_bytes_per_call": decode_bytes,
        "new_rows_bytes_per_step": new_rows_bytes,
        "fused_ms_mean": round(dec_mean, 5),
        "fused_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(dec_ms, [10, 50, 90])],
        "pa_decode_only": {
            "ms_mean": round(plain_mean, 5),
            "ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(plain_ms, [10, 50, 90])],
            "GBps": round(decode_bytes / (plain_mean * 1e-3) / 1e9, 2),
            "frac": round(decode_bytes / (plain_mean * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "what": "pa_decode alone (no new-row store), HIP events around each call"},
        "graph_replay_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "graph_replay_GBps": None if graph_ms is None else round(decode_bytes / (graph_ms * 1e-3) / 1e9, 1),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "from": ("formula bytes / the timed region's mean launch duration (HIP events "
                     "around exactly K back-to-back launches of this one kernel)")
                    if single_launch else
                    ("formula bytes / mean HIP-event span of each step's calls (second pass; "
                     "the spans hold the decode and merge launches and their dispatch)"),
            "launch_ms": round(launch_ms, 5),
        },
        "reference_reads": refs,
        "decode_vs_gather": None if refs is None else round(achieved / refs["gather_GBps"], 4),
        "cpu_baseline": cpu,
        "parity_layer0_vs_oracle": parity,
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_cow(args):
    """The shared-prefix / copy-on-write step: 32 prompts of U[64, 512]
    tokens x 6 samples sharing the prompt's blocks, private tails of
    U[1, 256] tokens; the step copies the partial last prompt block for 5
    samples of each prompt (pa_copy_blocks), stores every sample's newest
    token (pa_write_kv) and decodes every sample (pa_decode), 40 heads x 128,
    fp16, B = 16, 8 layer pools rotated.  Reports each call's time, the
    combined step (and the fused form: copies, then pa_decode_append), and
    the decode's rate over logical bytes (every sample's context, shared
    blocks counted per sample, as in the headline byte count) and over unique bytes
    (each physical block once)."""
    import torch

    import paged_kv_cache_05_amd as pa
    import workloads as W

    device = torch.device("cuda:0")
    wl = W.shared_prompts(host=False)
    N, H, D, B = wl.num_seqs, wl.num_heads, wl.head_dim, wl.block_size
    L, K = args.layers, args.steps
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    pools = [W.device_pools(wl, device, seed_offset=layer) for layer in range(L)]
    # Every step re-copies the shared partial prompt blocks over the samples'
    # private copies, which also hold tail tokens: fill the source blocks in
    # every row (finite values) so that the copies stay finite.
    src = torch.as_tensor(np.unique(wl.block_mapping[:, 0]), device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(44)
    for k, v in pools:
        for pool in (k, v):
            pool[src] = torch.randn((len(src),) + tuple(pool.shape[1:]), generator=gen,
                                    device=device).to(pool.dtype)
    tables, ctx, q = dev(wl.block_tables), dev(wl.context_lens), dev(wl.q)
    out = torch.empty_like(q)
    # each sample's newest token: position ctx - 1
    last = wl.context_lens.astype(np.int64) - 1
    slots_np = (wl.block_tables[np.arange(N), last // B].astype(np.int64) * B + last % B)
    slots = dev(slots_np)
    rng = np.random.default_rng(4)
    new_k = dev(rng.standard_normal((N, H, D), dtype=np.float32).astype(np.float16))
    new_v = dev(rng.standard_normal((N, H, D), dtype=np.float32).astype(np.float16))
    pairs = dev(wl.block_mapping)
    maxctx = wl.max_context_len
    ws = pa.new_workspace(N, H, D, maxctx, 256, device=device)
    scale = float(wl.scale)
    host_ctx = wl.context_lens
    stream = torch.cuda.current_stream()

    calls = {
        "copy": lambda k, v: pa.pa_copy_blocks(k, v, pairs),
        "write": lambda k, v: pa.pa_write_kv(new_k, new_v, k, v, slots),
        "decode": lambda k, v: pa.pa_decode(out, q, k, v, tables, ctx, scale, maxctx, 0, ws,
                                            host_context_lens=host_ctx),
        "append": lambda k, v: pa.pa_decode_append(out, q, new_k, new_v, k, v, tables, ctx,
                                                   slots, scale, maxctx, 0, ws,
                                                   host_context_lens=host_ctx),
    }

    def timed(names, n):
        """Mean ms of the listed calls run back to back per step (events
        around the group), over n steps rotating the layer pools."""
        for i in range(max(args.warmup, 1)):
            for nm in names:
                calls[nm](*pools[i % L])
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            for nm in names:
                calls[nm](*pools[i % L])
            b.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    ms = {nm: timed([nm], K) for nm in ("copy", "write", "decode")}
    ms["step_split"] = timed(["copy", "write", "decode"], K)
    ms["step_fused"] = timed(["copy", "append"], K)
    # the timed region of the line: exactly K fused steps, events at its ends
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        calls["copy"](*pools[i % L])
        calls["append"](*pools[i % L])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / K
    got = out.cpu().numpy()
    if not np.isfinite(got.astype(np.float32)).all():
        raise SystemExit("bench: non-finite decode output (shared prefix)")

    logical = wl.algorithmic_bytes()
    ids, filled = W.live_rows(wl)
    blocks_used = int(np.sum(-(-wl.context_lens.astype(np.int64) // B)))
    unique = int(filled.sum()) * H * D * 2 * 2 + 4 * blocks_used
    npairs = int(wl.block_mapping.shape[0])
    copy_bytes = npairs * 4 * H * B * D * 2          # read and write, K and V
    write_bytes = N * H * D * 2 * 4                  # read key/value, write both pools
    rate = lambda nbytes, m: round(nbytes / (m * 1e-3) / 1e9, 1)
    rec = {
        "metric": "shared-prefix decode step: HBM GB/s over logical bytes (every sample's context)",
        "value": rate(logical, ms_per_step), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded prompt and tail lengths, N(0,1) q/K/V, scattered blocks)",
        "config": {"workload": "shared-prefix / copy-on-write decode step (32 prompts x 6 "
                               "samples, 40 heads x 128, B 16)",
                   "num_seqs": N, "cow_pairs": npairs, "layer_pools_rotated": L,
                   "sum_context_logical": int(wl.context_lens.sum()),
                   "unique_tokens": int(filled.sum()), "unique_blocks": int(len(ids))},
        "logical_bytes": logical, "unique_bytes": unique,
        "step": "copies (pa_copy_blocks) then pa_decode_append, one layer",
        "pa_copy_blocks": {"us": round(ms["copy"] * 1e3, 2), "pairs": npairs,
                           "bytes": copy_bytes, "GBps": rate(copy_bytes, ms["copy"])},
        "pa_write_kv": {"us": round(ms["write"] * 1e3, 2), "tokens": N,
                        "bytes": write_bytes, "GBps": rate(write_bytes, ms["write"])},
        "pa_decode": {"us": round(ms["decode"] * 1e3, 2),
                      "logical_GBps": rate(logical, ms["decode"]),
                      "unique_GBps": rate(unique, ms["decode"])},
        "step_split_us": round(ms["step_split"] * 1e3, 2),
        "step_fused_us": round(ms["step_fused"] * 1e3, 2),
        "step_fused_unique_GBps": rate(unique, ms["step_fused"]),
        "timing": "HIP events around each call (or group), mean over steps",
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
