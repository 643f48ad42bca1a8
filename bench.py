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
(torch's current stream), around the whole timed region and around every
pa_decode call (one kernel launch each), after W untimed warm-up steps.

Also times the CPU oracle on the host (the full batch of layer 0, all host
threads) as a reported baseline, and checks sampled GPU rows against it.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: HBM GB/s (% of peak), decode steps/s at OPT-13B shape"
PEAK_HBM_GBS = 8000.0
COUNTER_FILE = os.path.join(ROOT, "profiles", "pa_decode_opt13b_hbm_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_05_amd", "csrc", f)
                  for f in ("pa_decode.hip", "pa_kernels.h")]


def kernel_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode call from the committed rocprofv3 counter runs
    (``key: value`` lines), if they were taken on the kernel source as it is
    now; otherwise None."""
    try:
        with open(COUNTER_FILE) as f:
            c = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    c = {k.strip(): v.strip() for k, v in c.items()}
    if c.get("kernel_digest") != kernel_digest():
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=8, help="layer pools to rotate over")
    ap.add_argument("--partition", type=int, default=0, help="pa_decode partition_size (0: default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-host-lengths", action="store_true",
                    help="do not pass host-side context lengths to pa_decode")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run one 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path has no multi-GPU mode); got --gpus "
              f"{args.gpus}", file=sys.stderr)
        return 2

    if args.calibrate_copy:
        return calibrate_copy()

    import torch

    import paged_kv_cache_05_amd as pa
    import workloads as W

    device = torch.device("cuda:0")
    wl = W.config2(host=False)
    N, H, D, B = wl.num_seqs, wl.num_heads, wl.head_dim, wl.block_size
    L = args.layers
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    pools = [W.device_pools(wl, device, seed_offset=layer) for layer in range(L)]
    tables, ctx = dev(wl.block_tables), dev(wl.context_lens)
    q = dev(wl.q)
    out = torch.empty_like(q)
    new_k, new_v, slots = dev(wl.new_key), dev(wl.new_value), dev(wl.slot_mapping)
    copies = dev(wl.block_mapping)
    maxctx = wl.max_context_len
    ws = pa.new_workspace(N, H, D, maxctx, args.partition, device=device)
    scale = float(wl.scale)
    # The step's scheduler knows every context length on the host; passing
    # them lets pa_decode launch only non-empty work items, largest first.
    host_ctx = None if args.no_host_lengths else wl.context_lens
    part = pa.pa_decode_partition_size(N, H, D, maxctx, args.partition, host_ctx,
                                       ws.numel() if ws is not None else 0)
    merges = -(-maxctx // part) > 1
    kernel = ("decode_listed_kernel" if host_ctx is not None else "decode_kernel") + \
        f"<{'f16' if wl.dtype == W.F16 else 'f32'},{D},{B},8>" + \
        (" + merge_kernel" if merges else "")
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        k, v = pools[i % L]
        pa.pa_copy_blocks(k, v, copies)              # no pairs in this workload: no launch
        pa.pa_write_kv(new_k, new_v, k, v, slots)
        if ev is not None:
            ev[0].record(stream)
        pa.pa_decode(out, q, k, v, tables, ctx, scale, maxctx, args.partition, ws,
                     host_context_lens=host_ctx)
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        step(i, evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_per_step = total_ms / K

    decode_bytes = wl.algorithmic_bytes()
    write_bytes = 4 * N * H * D * wl.elem_bytes     # read key + value, write both pools
    step_bytes = decode_bytes + write_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_mean = float(dec_ms.mean())
    achieved = decode_bytes / (dec_mean * 1e-3) / 1e9
    traffic = measured_traffic()

    # Output of layer 0 for the parity sample and the CPU baseline.
    k0, v0 = pools[0]
    pa.pa_write_kv(new_k, new_v, k0, v0, slots)
    pa.pa_decode(out, q, k0, v0, tables, ctx, scale, maxctx, args.partition, ws,
                 host_context_lens=host_ctx)
    torch.cuda.synchronize()
    gpu_out = out.cpu().numpy().astype(np.float64)
    if not np.isfinite(gpu_out).all():
        raise SystemExit("bench: non-finite decode output")

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
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
                         f"{1.0 / secs:.3f} decode steps/s"}
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
        "dtype": "f16",
        "data": "synthetic (seeded; lognormal context lengths, N(0,1) q/K/V, scattered blocks)",
        "config": {
            "workload": "OPT-13B-shaped single-layer decode step (write_kv + paged decode)",
            "num_seqs": N, "num_heads": H, "head_dim": D, "block_size": B,
            "context_lens": "lognormal median 300 sigma 0.9 clipped [1,2048]",
            "sum_context": int(wl.context_lens.sum()), "max_context": maxctx,
            "num_blocks": wl.num_blocks, "layer_pools_rotated": L,
            "partition_size": part,
            "host_planned_launch": host_ctx is not None,
        },
        "decode_steps_per_s": round(1000.0 / ms_per_step, 1),
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "decode_bytes_per_call": decode_bytes,
        "decode_ms_mean": round(dec_mean, 5),
        "decode_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(dec_ms, [10, 50, 90])],
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": kernel,
        },
        "cpu_baseline": cpu,
        "parity_layer0_vs_oracle": parity,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
