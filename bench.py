"""Throughput of the Gated DeltaNet mixer on one MI355X.

Headline (the JSON line's `value`): prefill tokens/s of one Qwen3.8-27B-like
Gated DeltaNet layer -- batch 1, T = 4096, 16 key heads / 48 value heads of
width 128, bf16 q/k/v, fp32 gates and state, chunks of 64 (the layer of the
page "L'attention hybride").  A step is one gdn_prefill call over inputs
already resident in HBM.  Extra fields of the same line report the decode
step (64 sequences x 48 heads of resident fp32 state, HBM GB/s), the full
block front end at batch 4, T = 32768, 16 key / 128 value heads (conv+SiLU,
prefill with the L2 flag, gated RMSNorm), the 262144-token prefill, the
roofline of the dominant kernel, and the fp64 oracle timed on the host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extras] [--no-cpu]
       python bench.py --calib-copy   (a plain device copy of 256 MiB, five times: the
                                       reference that HBM counters are scaled by)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 2.4 GHz x 4096 flop/clk)
C = 64                          # chunk length


def prefill_flops(B, T, Hk, Hv, D):
    """Algorithmic flops of one prefill call: per token and value head
    6 D^2 (state products) + (C+1)(D + 2D) (intra-chunk products) + C^2/3
    (triangular solve), plus 2 C D per token and key head (the two Gram
    matrices)."""
    per_tok = Hv * (6 * D * D + (C + 1) * (D + 2 * D) + C * C / 3.0) + Hk * 2 * C * D
    return per_tok * B * T


def prefill_bytes(B, T, Hk, Hv, D, io_bytes=2, state_in=False):
    """Algorithmic HBM bytes of one prefill call: q, k, v, o once at the I/O
    dtype, fp32 log_alpha and beta, the fp32 final state (and initial state)."""
    per_tok = 2 * Hk * D * io_bytes + 2 * Hv * D * io_bytes + 2 * Hv * 4
    st = B * Hv * D * D * 4
    return B * T * per_tok + st * (2 if state_in else 1)


def decode_bytes(B, Hk, Hv, D, io_bytes=2):
    """One decode step: state read + write (fp32), q, k, v, o and the gates."""
    return B * (2 * Hv * D * D * 4 + 2 * Hk * D * io_bytes + 2 * Hv * D * io_bytes + 2 * Hv * 4)


def bf16_dev(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def back_to_back(fn, steps, stream):
    """`steps` calls of fn() back to back between one event pair on `stream`, synchronised on
    both sides; returns ms per call."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def timed_launches(fn, steps, warmup, stream, p90=False):
    """Runs fn() warmup times, then `steps` times with a HIP event pair around
    each launch on `stream`.  Returns (total ms of the timed region from the
    first start event to the last end event, mean ms per launch, median ms),
    and the 90th percentile when p90 is set."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    with torch.cuda.stream(stream):
        for i in range(steps):
            starts[i].record(stream)
            fn()
            ends[i].record(stream)
    torch.cuda.synchronize()
    per = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    total = starts[0].elapsed_time(ends[-1])
    if p90:
        return total, float(per.mean()), float(np.median(per)), float(np.percentile(per, 90))
    return total, float(per.mean()), float(np.median(per))


def bench_prefill4k(steps, warmup, dev):
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    from gated_deltanet_recurrence_rule_amd import workloads as W
    p = W.cfg_prefill4k()
    B, T, Hk, Hv, D = p["B"], p["T"], p["Hk"], p["Hv"], p["D"]
    q, k, v = bf16_dev(p["q"], dev), bf16_dev(p["k"], dev), bf16_dev(p["v"], dev)
    la = torch.from_numpy(p["log_alpha"]).to(dev)
    be = torch.from_numpy(p["beta"]).to(dev)
    o = torch.empty((B, T, Hv * D), dtype=torch.bfloat16, device=dev)
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(G.gdn_prefill_workspace_size(G.make_dims(B, T, Hk, Hv, D, G.GDN_BF16)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        G.gdn_prefill(q, k, v, la, be, None, so, o, Hk=Hk, Hv=Hv, workspace=ws, stream=stream)

    # The timed region: `steps` calls back to back between one event pair on the call's
    # stream, synchronised on both sides.  (An event pair around every call adds ~7 us of
    # stream bubbles per call at this size, so per-call pairs are taken in a separate pass
    # after the timed region, for the per-call spread only.)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    total = e0.elapsed_time(e1)
    _, pair_mean, pair_med = timed_launches(step, steps, 0, stream)
    return dict(B=B, T=T, Hk=Hk, Hv=Hv, D=D, total_ms=total, mean_ms=total / steps,
                pair_mean_ms=pair_mean, pair_median_ms=pair_med,
                flops=prefill_flops(B, T, Hk, Hv, D), bytes=prefill_bytes(B, T, Hk, Hv, D))


def bench_prefill_cold(dev, steps=20):
    """The headline prefill with the 256 MB last-level cache emptied before each call: a
    512 MB buffer is written between calls, outside the timed events."""
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    from gated_deltanet_recurrence_rule_amd import workloads as W
    p = W.cfg_prefill4k()
    B, T, Hk, Hv, D = p["B"], p["T"], p["Hk"], p["Hv"], p["D"]
    q, k, v = bf16_dev(p["q"], dev), bf16_dev(p["k"], dev), bf16_dev(p["v"], dev)
    la = torch.from_numpy(p["log_alpha"]).to(dev)
    be = torch.from_numpy(p["beta"]).to(dev)
    o = torch.empty((B, T, Hv * D), dtype=torch.bfloat16, device=dev)
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(G.gdn_prefill_workspace_size(G.make_dims(B, T, Hk, Hv, D, G.GDN_BF16)),
                     dtype=torch.uint8, device=dev)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    call = lambda: G.gdn_prefill(q, k, v, la, be, None, so, o, Hk=Hk, Hv=Hv, workspace=ws, stream=stream)
    for _ in range(20):
        call()
    times = []
    for i in range(steps):
        scrub.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    med = float(np.median(times))
    return dict(median_us=med * 1e3, tokens_per_s=B * T / (med * 1e-3))


def attainable_peaks(dev):
    """What this machine reaches on plain work: a 1 GiB device copy (bytes read plus written per
    second) and a large bf16 GEMM through torch (hipBLASLt), then the library's probes: its
    own copy kernel over the same 1 GiB and bf16 MFMAs on register operands (gdn_probe.h)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    reps = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1))
    copy_gbs = 2 * n / (min(reps) * 1e-3) / 1e9
    del src, dst
    m = 8192
    a = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    b = torch.randn((m, m), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b)
    torch.cuda.synchronize()
    reps = []
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        reps.append(e0.elapsed_time(e1))
    gemm = 2 * m ** 3 / (min(reps) * 1e-3) / 1e12
    del a, b
    # the library's probes: a plain copy kernel over the same 1 GiB, and MFMAs on registers
    from gated_deltanet_recurrence_rule_amd import binding as G
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    _, _, med = timed_launches(lambda: G.gdn_probe_copy(src, dst, stream=stream), 5, 3, stream)
    probe_copy = 2 * n / (med * 1e-3) / 1e9
    del src, dst
    nwg, iters = 2048, 4096
    sink = torch.empty(nwg * 256, dtype=torch.float32, device=dev)
    fl = nwg * 4 * iters * 4 * 32768
    _, _, med = timed_launches(lambda: G.gdn_probe_mfma(nwg, iters, sink, stream=stream), 5, 2, stream)
    probe_mfma = fl / (med * 1e-3) / 1e12
    return dict(copy_1GiB_GBs=copy_gbs, copy_frac=copy_gbs / HBM_PEAK_GBS,
                bf16_gemm_8192_TFLOPs=gemm, bf16_gemm_frac=gemm / BF16_PEAK_TFLOPS,
                probe_copy_1GiB_GBs=probe_copy, probe_copy_frac=probe_copy / HBM_PEAK_GBS,
                probe_mfma_bf16_TFLOPs=probe_mfma, probe_mfma_frac=probe_mfma / BF16_PEAK_TFLOPS)


def bench_decode(dev, n_steps=256, pools=1, graph=False):
    """256 successive decode steps on a resident [64, 48, 128, 128] fp32 pool
    (`pools` independent pools rotated step by step to defeat the 256 MB
    last-level cache); per-step inputs are staged in HBM beforehand."""
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    from gated_deltanet_recurrence_rule_amd import workloads as W
    B, Hk, Hv, D = 64, 16, 48, 128
    pool_list = [torch.from_numpy(W.decode_pool(B, Hv, D, seed=3 + i)).to(dev) for i in range(pools)]
    steps_in = []
    for s in range(n_steps):
        d = W.decode_step_inputs(s, B=B, Hk=Hk, Hv=Hv, D=D)
        steps_in.append(tuple([bf16_dev(d[n][:, 0], dev) for n in ("q", "k", "v")] +
                              [torch.from_numpy(np.ascontiguousarray(d[n][:, 0])).to(dev)
                               for n in ("log_alpha", "beta")]))
    o = torch.empty((B, Hv * D), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    i = [0]

    def step():
        s = i[0] % n_steps
        q, k, v, la, be = steps_in[s]
        G.gdn_decode_step(q, k, v, la, be, pool_list[i[0] % pools], o, Hk=Hk, Hv=Hv, stream=stream)
        i[0] += 1

    # the steps back to back between one event pair (the rate), then each step between its own
    # pair (median and 90th percentile; the pairs add stream bubbles of their own)
    for _ in range(8):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    b2b_ms = e0.elapsed_time(e1) / n_steps
    total, mean_ms, med_ms, p90_ms = timed_launches(step, n_steps, 0, stream, p90=True)
    per = decode_bytes(B, Hk, Hv, D)
    out = dict(steps=n_steps, pools=pools, total_ms=total, mean_ms=mean_ms, median_ms=med_ms, p90_ms=p90_ms,
               b2b_ms=b2b_ms, bytes_per_step=per, GBs=per / (b2b_ms * 1e-3) / 1e9,
               median_GBs=per / (med_ms * 1e-3) / 1e9)
    if graph:
        # the same 256 steps captured once in a HIP graph and replayed: launch cost out of the way
        i[0] = 0
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()          # one eager step on the capture stream before capturing
            i[0] = 0
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            for _ in range(n_steps):
                q, k, v, la, be = steps_in[i[0] % n_steps]
                G.gdn_decode_step(q, k, v, la, be, pool_list[i[0] % pools], o, Hk=Hk, Hv=Hv, stream=side)
                i[0] += 1
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) / n_steps)
        gm = float(np.median(reps))
        out.update(graph_us_per_step=gm * 1e3, graph_GBs=per / (gm * 1e-3) / 1e9)
    return out


def bench_decode_front(dev, n_steps=256, n_inputs=32):
    """One layer's decode token for 64 sequences, front to back: single-token conv+SiLU over the
    q|k|v channels with the window handed on, gdn_decode_token (L2 flag, gates formed from raw
    in_proj_ba outputs, states in a 64-entry pool through a shuffled slot table), gated RMSNorm.
    n_inputs distinct per-step inputs are staged in HBM and cycled."""
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    B, Hk, Hv, D = 64, 16, 48, 128
    C = (2 * Hk + Hv) * D
    g = torch.Generator(device=dev)
    g.manual_seed(6)
    bf = torch.bfloat16
    xs = [torch.randn((B, 1, C), generator=g, device=dev).to(bf) for _ in range(n_inputs)]
    bas = [torch.randn((B, 2 * Hv), generator=g, device=dev).to(bf) for _ in range(n_inputs)]
    zs = [torch.randn((B, Hv * D), generator=g, device=dev).to(bf) for _ in range(n_inputs)]
    w = (0.5 * torch.randn((C, 4), generator=g, device=dev)).to(bf)
    nw = (1.0 + 0.1 * torch.randn((D,), generator=g, device=dev)).to(bf)
    A_log = torch.rand((Hv,), generator=g, device=dev) * float(np.log(16.0))
    dt_bias = 0.5 * torch.randn((Hv,), generator=g, device=dev)
    cs = [torch.zeros((B, C, 3), dtype=bf, device=dev) for _ in range(2)]
    pool = 0.02 * torch.randn((B, Hv, D, D), generator=g, device=dev)
    slots = torch.randperm(B, generator=g, device=dev).to(torch.int32)
    y = torch.empty((B, 1, C), dtype=bf, device=dev)
    o = torch.empty((B, Hv * D), dtype=bf, device=dev)
    out = torch.empty((B, Hv * D), dtype=bf, device=dev)
    stream = torch.cuda.current_stream()
    i = [0]

    def step():
        s = i[0] % n_inputs
        G.gdn_conv1d_silu(xs[s], w, cs[i[0] % 2], cs[(i[0] + 1) % 2], y, stream=stream)
        y2 = y[:, 0]
        G.gdn_decode_token(y2[:, :Hk * D], y2[:, Hk * D:2 * Hk * D], y2[:, 2 * Hk * D:], bas[s], A_log, dt_bias,
                           pool, slots, o, Hk=Hk, Hv=Hv, l2norm=True, stream=stream)
        G.gdn_gated_rmsnorm(o, zs[s], nw, 1e-6, out, H=Hv, stream=stream)
        i[0] += 1

    def token_only():
        s = i[0] % n_inputs
        y2 = y[:, 0]
        G.gdn_decode_token(y2[:, :Hk * D], y2[:, Hk * D:2 * Hk * D], y2[:, 2 * Hk * D:], bas[s], A_log, dt_bias,
                           pool, slots, o, Hk=Hk, Hv=Hv, l2norm=True, stream=stream)
        i[0] += 1

    # the same token through the fused kernel: window pools [S, C, 3] swapped each step
    xs2 = [x[:, 0] for x in xs]
    pools_cs = [torch.zeros((B, C, 3), dtype=bf, device=dev) for _ in range(2)]
    out2 = torch.empty((B, Hv * D), dtype=bf, device=dev)

    def fused():
        s = i[0] % n_inputs
        G.gdn_decode_layer(xs2[s], w, pools_cs[i[0] % 2], pools_cs[(i[0] + 1) % 2], bas[s], A_log, dt_bias, pool,
                           zs[s], nw, slots, out2, Hk=Hk, Hv=Hv, l2norm=True, stream=stream)
        i[0] += 1

    torch.cuda.synchronize()
    # each variant back to back between one event pair (the rates), then with an event pair
    # around each step (the medians)
    _, mean_ms, med_ms = timed_launches(step, n_steps, 300, stream)
    b2b = back_to_back(step, n_steps, stream)
    _, _, tok_med = timed_launches(token_only, n_steps, 8, stream)
    tok_b2b = back_to_back(token_only, n_steps, stream)
    _, _, fused_med = timed_launches(fused, n_steps, 8, stream)
    fused_b2b = back_to_back(fused, n_steps, stream)
    conv_b = B * (2 * C * 2 + 2 * 3 * C * 2) + C * 4 * 2
    tok_b = B * (2 * Hv * D * D * 4 + 2 * Hk * D * 2 + 2 * Hv * D * 2 + 2 * Hv * 2) + 4 * B
    norm_b = B * 3 * Hv * D * 2 + D * 2
    fused_b = B * (C * 2 + 2 * 3 * C * 2 + 2 * Hv * 2 + 2 * Hv * D * D * 4 + 2 * Hv * D * 2) + C * 4 * 2 + 4 * B
    return dict(us_per_step=b2b * 1e3, median_us=med_ms * 1e3, mean_us=mean_ms * 1e3,
                bytes_per_step=conv_b + tok_b + norm_b, GBs=(conv_b + tok_b + norm_b) / (b2b * 1e-3) / 1e9,
                token_us_per_step=tok_b2b * 1e3, token_median_us=tok_med * 1e3,
                token_GBs=tok_b / (tok_b2b * 1e-3) / 1e9,
                fused_us_per_step=fused_b2b * 1e3, fused_median_us=fused_med * 1e3,
                fused_bytes_per_step=fused_b, fused_GBs=fused_b / (fused_b2b * 1e-3) / 1e9)


def bench_block(dev, steps=5, warmup=2):
    """Block front end at batch 4, T = 32768, 16 key / 128 value heads: conv+SiLU over
    [q|k|v] (20480 channels), prefill on strided views with the L2 flag, gated
    RMSNorm x swish(z).  The block runs conv then gdn_prefill_gated, which applies
    the norm inside the chain kernel here (the 512 heads fill the GPU); the separate
    launches (prefill, then norm) are timed beside it.  Inputs are drawn on the GPU
    (seeded torch generator) with the recipe's distributions; timing does not depend
    on the values."""
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    B, T, Hk, Hv, D = 4, 32768, 16, 128, 128
    Cc = (2 * Hk + Hv) * D
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    x = torch.randn((B, T, Cc), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = (0.5 * torch.randn((Cc, 4), generator=g, device=dev)).to(torch.bfloat16)
    z = torch.randn((B * T, Hv * D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    nw = (1.0 + 0.1 * torch.randn((D,), generator=g, device=dev)).to(torch.bfloat16)
    A = torch.rand((Hv,), generator=g, device=dev) * float(np.log(16.0))
    dt = 0.5 * torch.randn((Hv,), generator=g, device=dev)
    la = (-torch.exp(A) * torch.nn.functional.softplus(torch.randn((B, T, Hv), generator=g, device=dev) + dt)).contiguous()
    be = torch.sigmoid(torch.randn((B, T, Hv), generator=g, device=dev)).contiguous()
    y = torch.empty_like(x)
    o = torch.empty((B, T, Hv * D), dtype=torch.bfloat16, device=dev)
    out = torch.empty((B * T, Hv * D), dtype=torch.bfloat16, device=dev)
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(G.gdn_prefill_workspace_size(G.make_dims(B, T, Hk, Hv, D, G.GDN_BF16)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    qv, kv, vv = y[:, :, :Hk * D], y[:, :, Hk * D:2 * Hk * D], y[:, :, 2 * Hk * D:]
    conv = lambda: G.gdn_conv1d_silu(x, w, None, None, y, stream=stream)
    pre = lambda: G.gdn_prefill(qv, kv, vv, la, be, None, so, o, Hk=Hk, Hv=Hv, l2norm=True, workspace=ws,
                                stream=stream)
    norm = lambda: G.gdn_gated_rmsnorm(o.view(B * T, Hv * D), z, nw, 1e-5, out, H=Hv, stream=stream)
    zv = z.view(B, T, Hv * D)
    gated = lambda: G.gdn_prefill_gated(qv, kv, vv, la, be, zv, nw, 1e-5, None, so, out.view(B, T, Hv * D), Hk=Hk,
                                        Hv=Hv, l2norm=True, workspace=ws, stream=stream)
    # the L2 norm of q and k in the conv's epilogue instead of in the prefill's loads
    conv_l2 = lambda: G.gdn_conv1d_silu(x, w, None, None, y, l2_channels=2 * Hk * D, l2_eps=1e-6, stream=stream)
    gated_nol2 = lambda: G.gdn_prefill_gated(qv, kv, vv, la, be, zv, nw, 1e-5, None, so, out.view(B, T, Hv * D), Hk=Hk,
                                             Hv=Hv, l2norm=False, workspace=ws, stream=stream)
    res = {}
    for name, fn in (("conv", conv), ("prefill", pre), ("norm", norm), ("prefill_gated", gated), ("conv_l2", conv_l2)):
        _, mean_ms, med_ms = timed_launches(fn, steps, warmup, stream)
        res[name + "_ms"] = med_ms

    def block():
        conv()
        gated()

    def block_unfused():
        conv()
        pre()
        norm()

    def block_l2():
        conv_l2()
        gated_nol2()

    total, _, med = timed_launches(block, steps, 1, stream)
    _, _, med_unfused = timed_launches(block_unfused, steps, 1, stream)
    _, _, med_l2 = timed_launches(block_l2, steps, 1, stream)
    res["block_unfused_ms"] = med_unfused
    res["block_conv_l2_ms"] = med_l2
    conv_bytes = B * T * Cc * 2 * 2 + Cc * 4 * 2
    norm_bytes = B * T * Hv * D * 2 * 3 + D * 2
    res.update(block_ms=med, tokens_per_s=B * T / (med * 1e-3),
               conv_GBs=conv_bytes / (res["conv_ms"] * 1e-3) / 1e9,
               norm_GBs=norm_bytes / (res["norm_ms"] * 1e-3) / 1e9,
               prefill_tokens_per_s=B * T / (res["prefill_ms"] * 1e-3),
               prefill_flops=prefill_flops(B, T, Hk, Hv, D),
               prefill_bytes=prefill_bytes(B, T, Hk, Hv, D))
    res["prefill_mfma_frac"] = res["prefill_flops"] / (res["prefill_ms"] * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)
    del x, y, z, o, out
    torch.cuda.empty_cache()
    return res


def bench_long(dev, steps=3, warmup=4):
    """Prefill at T = 262144 (batch 1, 16/48 heads), inputs drawn on the GPU.  Four
    untimed calls (~45 ms) let the clocks settle first."""
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    B, T, Hk, Hv, D = 1, 262144, 16, 48, 128
    g = torch.Generator(device=dev)
    g.manual_seed(4)

    def unit(n, h):
        a = torch.randn((B, T, h, D), generator=g, device=dev)
        return (a / a.norm(dim=-1, keepdim=True)).reshape(B, T, h * D).to(torch.bfloat16)

    q, k = unit(T, Hk), unit(T, Hk)
    v = torch.randn((B, T, Hv * D), generator=g, device=dev).to(torch.bfloat16)
    A = torch.rand((Hv,), generator=g, device=dev) * float(np.log(16.0))
    dt = 0.5 * torch.randn((Hv,), generator=g, device=dev)
    la = (-torch.exp(A) * torch.nn.functional.softplus(torch.randn((B, T, Hv), generator=g, device=dev) + dt)).contiguous()
    be = torch.sigmoid(torch.randn((B, T, Hv), generator=g, device=dev)).contiguous()
    o = torch.empty_like(v)
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(G.gdn_prefill_workspace_size(G.make_dims(B, T, Hk, Hv, D, G.GDN_BF16)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    fn = lambda: G.gdn_prefill(q, k, v, la, be, None, so, o, Hk=Hk, Hv=Hv, workspace=ws, stream=stream)
    _, _, med = timed_launches(fn, steps, warmup, stream)
    fl = prefill_flops(B, T, Hk, Hv, D)
    by = prefill_bytes(B, T, Hk, Hv, D)
    del q, k, v, o
    torch.cuda.empty_cache()
    return dict(T=T, ms=med, tokens_per_s=T / (med * 1e-3),
                mfma_frac=fl / (med * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                hbm_frac=by / (med * 1e-3) / (HBM_PEAK_GBS * 1e9))


def attn_prefill_flops(B, T, Hq, D):
    """Causal attention: query row t meets t + 1 keys, two products of 2 D flops each."""
    return 4.0 * D * Hq * B * T * (T + 1) / 2


def bench_attention(dev, steps=20, warmup=20):
    """The hybrid's full-attention layer (24 query / 4 key-value heads of 256, RoPE on 64
    dimensions, output gate).  Prefill: batch 1, T = 4096, one gdn_attn_prefill call (norm,
    RoPE, cache writes, attention).  Decode: 64 sequences with 4095 cached positions each,
    one gdn_attn_decode call (the new token's prep, split attention, combine).  Inputs drawn
    on the GPU; the decode caches hold random rotated keys and values."""
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    Hq, Hkv, D = 24, 4, 256
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    bf = lambda *shape: torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
    qw = (1 + 0.1 * torch.randn((D,), generator=g, device=dev)).to(torch.bfloat16)
    kw = (1 + 0.1 * torch.randn((D,), generator=g, device=dev)).to(torch.bfloat16)
    T = 4096
    qg, k, v = bf(1, T, Hq, 2, D), bf(1, T, Hkv, D), bf(1, T, Hkv, D)
    kc, vc = G.attn_cache(1, Hkv, T, D, device=dev)
    o = torch.empty((1, T, Hq, D), dtype=torch.bfloat16, device=dev)
    dims = G.make_attn_dims(1, T, Hq, Hkv, D, T)
    ws = torch.empty(G.lib().gdn_attn_prefill_workspace_size(ctypes.byref(dims)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    fn = lambda: G.gdn_attn_prefill(qg, k, v, qw, kw, kc, vc, o, workspace=ws, stream=stream)
    _, _, med_p_pair = timed_launches(fn, steps, warmup, stream)
    med_p = back_to_back(fn, steps, stream)
    fl = attn_prefill_flops(1, T, Hq, D)
    del qg, k, v, kc, vc, o, ws
    B, S = 64, 4096
    kc = torch.randn((B, Hkv, S, D), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, S // 64, D, 64), generator=g, device=dev).to(torch.bfloat16)
    lens = torch.full((B,), S - 1, dtype=torch.int32, device=dev)
    qg, k, v = bf(B, Hq, 2, D), bf(B, Hkv, D), bf(B, Hkv, D)
    o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    dims = G.make_attn_dims(B, 1, Hq, Hkv, D, S)
    ws = torch.empty(G.lib().gdn_attn_decode_workspace_size(ctypes.byref(dims)), dtype=torch.uint8, device=dev)
    fn = lambda: G.gdn_attn_decode(qg, k, v, qw, kw, lens, kc, vc, o, workspace=ws, stream=stream)
    _, _, med_d_pair = timed_launches(fn, steps * 5, warmup, stream)
    med_d = back_to_back(fn, steps * 5, stream)
    by = B * Hkv * S * D * 2 * 2 + B * (Hq * 2 * D + 2 * Hkv * D + Hq * D) * 2
    del kc, vc
    torch.cuda.empty_cache()
    # prefill_us / decode_us: calls back to back; *_pair_median_us: an event pair around each call
    return dict(prefill_T=T, prefill_us=med_p * 1e3, prefill_pair_median_us=med_p_pair * 1e3,
                decode_pair_median_us=med_d_pair * 1e3, prefill_tflops=fl / (med_p * 1e-3) / 1e12,
                prefill_mfma_frac=fl / (med_p * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                decode_B=B, decode_cached=S, decode_us=med_d * 1e3, decode_bytes=by,
                decode_GBs=by / (med_d * 1e-3) / 1e9, decode_hbm_frac=by / (med_d * 1e-3) / (HBM_PEAK_GBS * 1e9))


def bench_varlen(dev, steps=20, warmup=20):
    """Packed prefill of 32 requests of log-uniform lengths (16 to 8192 tokens,
    seeded), 16/48 heads, one gdn_prefill_varlen call per step, final states into a
    [32, 48, 128, 128] pool; beside it, the same requests as one gdn_prefill call
    each.  Inputs drawn on the GPU."""
    import torch
    from gated_deltanet_recurrence_rule_amd import binding as G
    from gated_deltanet_recurrence_rule_amd import workloads as W
    lens = W.varlen_lengths()
    Hk, Hv, D = 16, 48, 128
    T = int(lens.sum())
    cu_h = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(cu_h).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(6)

    def unit(h):
        a = torch.randn((T, h, D), generator=g, device=dev)
        return (a / a.norm(dim=-1, keepdim=True)).reshape(T, h * D).to(torch.bfloat16)

    q, k = unit(Hk), unit(Hk)
    v = torch.randn((T, Hv * D), generator=g, device=dev).to(torch.bfloat16)
    A = torch.rand((Hv,), generator=g, device=dev) * float(np.log(16.0))
    dt = 0.5 * torch.randn((Hv,), generator=g, device=dev)
    la = (-torch.exp(A) * torch.nn.functional.softplus(torch.randn((T, Hv), generator=g, device=dev) + dt)).contiguous()
    be = torch.sigmoid(torch.randn((T, Hv), generator=g, device=dev)).contiguous()
    o = torch.empty_like(v)
    n = len(lens)
    so = torch.empty((n, Hv, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(G.gdn_prefill_varlen_workspace_size(G.make_dims(n, T, Hk, Hv, D, G.GDN_BF16)),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    fn = lambda: G.gdn_prefill_varlen(q, k, v, la, be, cu, None, so, o, Hk=Hk, Hv=Hv, workspace=ws, stream=stream)
    _, _, med = timed_launches(fn, steps, warmup, stream)
    # the same requests, one call each (views into the packed tensors; one workspace that
    # holds the largest request's, whose windows may be longer than the packed call's)
    wszs = [G.gdn_prefill_workspace_size(G.make_dims(1, int(cu_h[s + 1] - cu_h[s]), Hk, Hv, D, G.GDN_BF16))
            for s in range(n)]
    ws1 = torch.empty(max(wszs), dtype=torch.uint8, device=dev)
    views = []
    for s in range(n):
        a, b = int(cu_h[s]), int(cu_h[s + 1])
        views.append((q[a:b].unsqueeze(0), k[a:b].unsqueeze(0), v[a:b].unsqueeze(0), la[a:b].unsqueeze(0),
                      be[a:b].unsqueeze(0), so[s:s + 1], o[a:b].unsqueeze(0), ws1[:wszs[s]]))

    def each():
        for qq, kk, vv, ll, bb, ss, oo, ww in views:
            G.gdn_prefill(qq, kk, vv, ll, bb, None, ss, oo, Hk=Hk, Hv=Hv, workspace=ww, stream=stream)

    _, _, med_each = timed_launches(each, max(steps // 4, 3), 3, stream)
    fl = prefill_flops(1, T, Hk, Hv, D)
    by = prefill_bytes(1, T, Hk, Hv, D) + (n - 1) * Hv * D * D * 4
    del q, k, v, o, ws, ws1, views
    torch.cuda.empty_cache()
    return dict(n_seq=n, tokens=T, min_len=int(lens.min()), max_len=int(lens.max()), ms=med,
                tokens_per_s=T / (med * 1e-3), hbm_frac=by / (med * 1e-3) / (HBM_PEAK_GBS * 1e9),
                mfma_frac=fl / (med * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                one_call_per_seq_ms=med_each, one_call_per_seq_tokens_per_s=T / (med_each * 1e-3))


def cpu_baseline(reps=2):
    """The fp64 oracle (gdn_oracle.c, OpenMP) on the headline workload: all 48 value
    heads over all 4096 tokens, timed on this host's cores."""
    import oracle
    from gated_deltanet_recurrence_rule_amd import workloads as W
    p = W.cfg_prefill4k()
    oracle.lib()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], p["Hk"], p["Hv"], None,
                          n_threads=threads)
        times.append(time.perf_counter() - t0)
    t = min(times)
    # one thread on a sample of 8 of the 48 value heads (its rate scaled to the whole layer)
    sel = list(range(0, p["Hv"], p["Hv"] // 8))
    t0 = time.perf_counter()
    oracle.recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], p["Hk"], p["Hv"], None,
                      sel=sel, n_threads=1)
    t1 = (time.perf_counter() - t0) * p["Hv"] / len(sel)
    model, phys, logical = cpu_info()
    return {"value": p["B"] * p["T"] / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole headline workload (B=1, T=4096, 48 value heads, fp64), best of {reps}: {t:.3f} s",
            "cpu_model": model, "physical_cores": phys, "logical_cpus": logical,
            "one_thread": {"value": p["B"] * p["T"] / t1, "unit": "tokens/s",
                           "sample": f"{len(sel)} of 48 value heads on 1 thread, scaled to 48: {t1:.3f} s"}}


def cpu_info():
    """CPU model name, physical cores and logical CPUs of this host, from /proc/cpuinfo."""
    model, cores, logical = "unknown", set(), 0
    try:
        phys = core = None
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k, v = k.strip(), v.strip()
            if k == "processor":
                logical += 1
            elif k == "model name":
                model = v
            elif k == "physical id":
                phys = v
            elif k == "core id":
                core = v
                cores.add((phys, core))
    except OSError:
        pass
    return model, (len(cores) or None), (logical or os.cpu_count())


def traffic_from_profile(kernel_src_hash):
    """HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
    scaled by a copy-kernel calibration; None when no matching measurement exists."""
    path = os.path.join(ROOT, "profiles", "prefill4k_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_src_sha256") != kernel_src_hash:
        return None
    return d.get("bytes_per_launch")


def kernel_src_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ("gdn_chunk.hip", "gdn_device.h"):
        h.update(open(os.path.join(ROOT, "gated_deltanet_recurrence_rule_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 40 ms of untimed calls: the GPU's clocks are still rising over the first
    # few hundred calls (at T=4096 the mean call time falls from ~143 to ~131 us)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-extras", action="store_true", help="headline only (no decode/block/long)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu baseline")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run only a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--decode-only", type=int, choices=(1, 2, 4), default=0,
                    help="run only the 256 decode steps on 1, 2 or 4 state pools (for counter runs)")
    ap.add_argument("--block-only", action="store_true",
                    help="run only the block leg (batch 4, T=32768, 16/128 heads; for trace runs)")
    args = ap.parse_args()
    if args.block_only:
        import torch
        r = bench_block(torch.device("cuda:0"))
        print(json.dumps(r))
        return
    if args.decode_only:
        import torch
        r = bench_decode(torch.device("cuda:0"), pools=args.decode_only)
        print(json.dumps({k: r[k] for k in ("pools", "b2b_ms", "median_ms", "GBs", "median_GBs", "bytes_per_step")}))
        return
    if args.calib_copy:
        import torch
        n = 256 << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "repeats": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: libgdn runs on a single GPU and has no multi-GPU path "
              f"(asked for {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    h = bench_prefill4k(args.steps, args.warmup, dev)
    ms = h["total_ms"] / args.steps
    tokens_per_s = h["B"] * h["T"] / (ms * 1e-3)
    kern_ms = h["mean_ms"]
    achieved = h["bytes"] / (kern_ms * 1e-3) / 1e9
    print(f"[bench] prefill4k: {ms * 1e3:.1f} us/step, kernel {kern_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
    line = {
        "metric": "GDN prefill tokens/s @T=4096, 16K/48V heads; decode-step HBM GB/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3.8-27B-like Gated DeltaNet layer prefill: batch 1, T=4096, "
                               "16 key / 48 value heads, d_k=d_v=128, bf16 q/k/v, fp32 gates and state, "
                               "chunk 64, S_0=0",
                   "B": h["B"], "T": h["T"], "Hk": h["Hk"], "Hv": h["Hv"], "D": h["D"], "chunk": C},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic_from_profile(kernel_src_hash()),
            "kernel": "gdn_prefill (chunk_prep_kernel + chunk_chain_kernel)",
            "kernel_mean_us": kern_ms * 1e3,
            "kernel_mean_note": "timed region / steps: back-to-back calls between one event pair",
            "per_call_event_pair_mean_us": h["pair_mean_ms"] * 1e3,
            "per_call_event_pair_median_us": h["pair_median_ms"] * 1e3,
            "algorithmic_bytes": h["bytes"],
            "algorithmic_flops": h["flops"],
            "mfma_frac": h["flops"] / (kern_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        },
    }
    if not args.no_extras:
        # decode's figure is the cold one: four pools (804 MB) rotate step by step, so that no
        # step finds its 201 MB pool in the 256 MB last-level cache; with two pools part of each
        # pool survives there (81 against 85 us a step)
        dec2 = bench_decode(dev, pools=4, graph=True)
        dec = bench_decode(dev)
        print(f"[bench] decode: {dec2['b2b_ms'] * 1e3:.1f} us/step back to back, {dec2['GBs']:.0f} GB/s cold "
              f"(median {dec2['median_ms'] * 1e3:.1f} us with a pair per step; one pool {dec['GBs']:.0f} GB/s; "
              f"graph of 256 steps {dec2['graph_us_per_step']:.1f} us/step)", file=sys.stderr, flush=True)
        line["decode"] = {"config": "64 sequences x 48 value heads x 128x128 fp32 state, 16 key heads, bf16 q/k/v, "
                                    "256 steps, four state pools rotated (cold)",
                          "us_per_step": dec2["b2b_ms"] * 1e3,
                          "us_per_step_note": "256 steps back to back between one event pair; GBs and hbm_frac "
                                              "from it; median/mean/p90 with an event pair around each step",
                          "median_us": dec2["median_ms"] * 1e3, "mean_us": dec2["mean_ms"] * 1e3,
                          "p90_us": dec2["p90_ms"] * 1e3, "median_GBs": dec2["median_GBs"],
                          "GBs": dec2["GBs"], "hbm_frac": dec2["GBs"] / HBM_PEAK_GBS,
                          "bytes_per_step": dec2["bytes_per_step"],
                          "graph_us_per_step": dec2["graph_us_per_step"], "graph_GBs": dec2["graph_GBs"],
                          "one_pool_us_per_step": dec["b2b_ms"] * 1e3,
                          "one_pool_median_us": dec["median_ms"] * 1e3, "one_pool_p90_us": dec["p90_ms"] * 1e3,
                          "one_pool_GBs": dec["GBs"]}
        cold = bench_prefill_cold(dev)
        print(f"[bench] prefill4k cold (cache emptied before each call): {cold['median_us']:.1f} us",
              file=sys.stderr, flush=True)
        line["prefill_cold"] = {"config": "headline prefill, 512 MB written between calls", **cold}
        pk = attainable_peaks(dev)
        print(f"[bench] attainable: copy {pk['copy_1GiB_GBs']:.0f} GB/s (probe {pk['probe_copy_1GiB_GBs']:.0f}), "
              f"bf16 GEMM {pk['bf16_gemm_8192_TFLOPs']:.0f} TFLOP/s (MFMA probe {pk['probe_mfma_bf16_TFLOPs']:.0f})",
              file=sys.stderr, flush=True)
        line["attainable"] = pk
        fr = bench_decode_front(dev)
        print(f"[bench] decode front end: {fr['us_per_step']:.1f} us/step back to back (token "
              f"{fr['token_us_per_step']:.1f} us, fused layer {fr['fused_us_per_step']:.1f} us)",
              file=sys.stderr, flush=True)
        line["decode_front_end"] = {
            "config": "64 sequences, one layer token: conv+SiLU over 10240 q|k|v channels (window rolled), "
                      "gdn_decode_token (L2 flag, gates from raw in_proj_ba, 64-entry state pool via a shuffled "
                      "slot table), gated RMSNorm over 48 x 128",
            **fr, "hbm_frac": fr["GBs"] / HBM_PEAK_GBS, "token_hbm_frac": fr["token_GBs"] / HBM_PEAK_GBS,
            "fused_hbm_frac": fr["fused_GBs"] / HBM_PEAK_GBS}
        blk = bench_block(dev)
        print(f"[bench] block: {blk['block_ms']:.2f} ms", file=sys.stderr, flush=True)
        line["block"] = {"config": "batch 4, T=32768, 16 key / 128 value heads: conv+SiLU, prefill (L2 flag) with "
                                   "the gated RMSNorm in the chain (gdn_prefill_gated); block_unfused_ms: conv, "
                                   "prefill, norm as three launches; block_conv_l2_ms: the L2 norm of q and k in the "
                                   "conv (gdn_conv1d_silu_l2), then gdn_prefill_gated without the L2 flag", **blk}
        lg = bench_long(dev)
        print(f"[bench] long: {lg['ms']:.2f} ms", file=sys.stderr, flush=True)
        line["long"] = {"config": "batch 1, T=262144, 16 key / 48 value heads", **lg}
        at = bench_attention(dev)
        print(f"[bench] attention: prefill {at['prefill_us']:.1f} us ({at['prefill_tflops']:.0f} TFLOP/s), "
              f"decode {at['decode_us']:.1f} us ({at['decode_GBs']:.0f} GB/s)", file=sys.stderr, flush=True)
        line["attention"] = {"config": "full-attention layer, 24 query / 4 key-value heads of 256, RoPE on 64 "
                                       "dims, output gate: prefill batch 1 T=4096; decode 64 sequences x 4095 "
                                       "cached positions", **at}
        vl = bench_varlen(dev)
        print(f"[bench] varlen: {vl['ms']:.3f} ms for {vl['tokens']} tokens in {vl['n_seq']} sequences "
              f"({vl['one_call_per_seq_ms']:.3f} ms as one call each)", file=sys.stderr, flush=True)
        line["varlen"] = {"config": "32 packed requests, log-uniform lengths 16..8192 (seed 6), 16 key / 48 value "
                                    "heads, final states into a 32-entry pool", **vl}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
