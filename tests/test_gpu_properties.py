"""Property and integration tests of the HIP path on the GPU: random shapes
against the oracle (hypothesis, derandomized), and a decoding step captured
once in a HIP graph and replayed."""
import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import workloads as W
from test_gpu_parity import announce, assert_close, bits, dev, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu


@st.composite
def shapes(draw):
    dtype = draw(st.sampled_from([W.F16, W.F32]))
    D = draw(st.sampled_from([64, 128]))
    B = draw(st.sampled_from([8, 16, 32, 64]))
    H = draw(st.integers(1, 4))
    ctx = draw(st.lists(st.integers(0, 300), min_size=1, max_size=12))
    part = draw(st.sampled_from([0, 16, 64, 256]))
    planned = draw(st.booleans())
    seed = draw(st.integers(0, 2**31 - 1))
    return dtype, D, B, H, ctx, part, planned, seed


@settings(max_examples=40, deadline=None, derandomize=True,
          suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])
@given(shapes())
def test_random_shapes_match_oracle(pa, oracle_lib, device, case):
    dtype, D, B, H, ctx, part, planned, seed = case
    wl = W._simple("prop", seed, dtype, H, D, B, [max(c, 1) for c in ctx])
    ctx_dev = np.array(ctx, np.int32)       # zero-length rows kept on the device side
    announce(f"property: dtype={dtype} D={D} B={B} H={H} N={len(ctx)} part={part} "
             f"planned={planned} seed={seed}")
    got = gpu_decode(pa, wl, dev(wl.k_pool, device), dev(wl.v_pool, device), device,
                     partition_size=part, ctx=ctx_dev,
                     host_ctx=ctx_dev if planned else None)
    ref = oracle_lib.decode(wl.q, wl.k_pool, wl.v_pool, wl.block_tables, ctx_dev, wl.scale)
    assert_close(got, ref, dtype, "property")
    assert np.all(got[ctx_dev == 0] == 0)


@pytest.mark.parametrize("fused", [False, True], ids=["write-then-decode", "decode-append"])
def test_step_replayed_from_a_hip_graph(pa, oracle_lib, device, fused):
    """copy_blocks + write_kv + decode (or the fused decode_append, whose
    listed launch has writer workgroups) captured once and replayed three
    times, with eager work and synchronisation between replays; every replay
    reproduces the eager result bit for bit."""
    wl = W.tiny_fp32()
    k0, v0 = dev(wl.k_pool_pre, device), dev(wl.v_pool_pre, device)
    k, v = k0.clone(), v0.clone()
    pairs, key, val, slots = (dev(wl.block_mapping, device), dev(wl.new_key, device),
                              dev(wl.new_value, device), dev(wl.slot_mapping, device))
    q, tables, ctx = dev(wl.q, device), dev(wl.block_tables, device), dev(wl.context_lens, device)
    ws = pa.new_workspace(wl.num_seqs, wl.num_heads, wl.head_dim, wl.max_context_len, 16,
                          device=device)
    out = torch.empty_like(q)

    def step():
        pa.pa_copy_blocks(k, v, pairs)
        if fused:
            pa.pa_decode_append(out, q, key, val, k, v, tables, ctx, slots, float(wl.scale),
                                wl.max_context_len, partition_size=16, workspace=ws,
                                host_context_lens=wl.context_lens)
            return
        pa.pa_write_kv(key, val, k, v, slots)
        pa.pa_decode(out, q, k, v, tables, ctx, float(wl.scale), wl.max_context_len,
                     partition_size=16, workspace=ws, host_context_lens=wl.context_lens)

    announce("eager step")
    step()
    torch.cuda.synchronize()
    eager_out, eager_k = out.clone(), k.clone()
    ref = oracle_decode(oracle_lib, wl)
    assert_close(eager_out.cpu().numpy(), ref, wl.dtype, "eager")

    g = torch.cuda.CUDAGraph()
    k.copy_(k0)
    v.copy_(v0)
    torch.cuda.synchronize()
    announce("capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        k.copy_(k0)                      # eager work between replays
        v.copy_(v0)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        announce(f"replay {r}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(k.view(torch.int32), eager_k.view(torch.int32)), f"replay {r}: pools differ"
        assert np.array_equal(bits(out.cpu().numpy()), bits(eager_out.cpu().numpy())), \
            f"replay {r}: decode output differs"
