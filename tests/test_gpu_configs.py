"""The five workload configurations at their full sizes, in the launch
configuration bench.py times, checked against the fp64 oracle.

Large configs are checked on sampled (sequence, value head) pairs that the
oracle recomputes over every token (heads are independent, so a sampled head
is exact, not an approximation).  Inputs come from the seeded generators in
gated_deltanet_recurrence_rule_amd.workloads.

  tiny      batch 1, T=64, 1/1 heads, D=16, fp32 -- every output and the state
  prefill4k batch 1, T=4096, 16/48 heads, D=128, bf16 -- 8 sampled heads
  decode    64 sequences, 48 heads of 128x128 fp32 state, 256 steps --
            8 sampled (sequence, head) pairs, outputs at every step, state
            after steps 1, 16 and 256; both gate recipes
  long      batch 1, T=262144 -- 2 sampled heads; also two halves of 131072
            tokens chained through the state equal one pass
  block     batch 4, T=32768, 16/128 heads: conv+SiLU -> prefill with the L2
            flag -> gated RMSNorm x swish(z); sampled heads end to end, with
            the oracle rounding to bf16 exactly where the API hands a bf16
            tensor on (the conv output, the prefill output)
"""
import os

import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_rule_amd import binding as G
from gated_deltanet_recurrence_rule_amd import workloads as W
from helpers import assert_out, assert_state, conv_abs_sum, conv_tol, to_dev, to_host

pytestmark = pytest.mark.gpu
NTHR = min(16, os.cpu_count() or 1)


def _torch():
    import torch
    return torch


def _free():
    import gc
    torch = _torch()
    gc.collect()
    torch.cuda.empty_cache()


def test_cfg_tiny_full():
    torch = _torch()
    p = W.cfg_tiny()
    so = torch.empty((1, 1, 16, 16), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill(to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"]), to_dev(p["log_alpha"]),
                      to_dev(p["beta"]), None, so, Hk=1, Hv=1)
    torch.cuda.synchronize()
    orf, srf = oracle.recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], 1, 1)
    m = assert_out(to_host(o).reshape(64, 16), orf[0], bf16=False)
    e = assert_state(to_host(so).reshape(16, 16), srf[0])
    print(f"tiny: max err/RMS {m['max_err_rms']:.2e}, state {e:.2e}")


def _sampled_prefill_check(p, sel, o_dev, so_dev, tag):
    Hv, D, T = p["Hv"], p["D"], p["T"]
    orf, srf = oracle.recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], p["Hk"], Hv, None,
                                 sel=sel, n_threads=NTHR)
    og = o_dev.view(p["B"], T, Hv, D)
    for i, bh in enumerate(sel):
        b, h = divmod(int(bh), Hv)
        m = assert_out(to_host(og[b, :, h, :]), orf[i], bf16=True, what=f"{tag} o head {bh}")
        e = assert_state(to_host(so_dev[b, h]), srf[i], what=f"{tag} state head {bh}")
        print(f"{tag} head {bh}: excess/RMS {m['excess_rms']:.2e} (literal {m['max_err_rms']:.2e}, "
              f"bf16 floor {m['floor_rms']:.2e}), state {e:.2e}")


def test_cfg_prefill4k_full():
    torch = _torch()
    p = W.cfg_prefill4k()
    B, T, Hk, Hv, D = p["B"], p["T"], p["Hk"], p["Hv"], p["D"]
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill(to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"]), to_dev(p["log_alpha"]),
                      to_dev(p["beta"]), None, so, Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()
    _sampled_prefill_check(p, [0, 7, 13, 20, 26, 33, 41, 47], o, so, "prefill4k")


@pytest.mark.parametrize("recipe", ["qwen", "tiny"])
def test_cfg_decode_full(recipe):
    torch = _torch()
    B, Hk, Hv, D, steps = 64, 16, 48, 128, 256
    pool = W.decode_pool(B, Hv, D)
    sel = np.array([0, 101, 777, 1500, 2047, 2300, 2999, 3071], np.int64)   # b*Hv + h
    state = to_dev(pool)
    ref = pool.reshape(B * Hv, D, D)[sel].copy()
    sb, sh = sel // Hv, sel % Hv
    o = torch.empty((B, Hv * D), dtype=torch.bfloat16, device="cuda")
    for s in range(steps):
        d = W.decode_step_inputs(s, B=B, Hk=Hk, Hv=Hv, D=D, recipe=recipe)
        G.gdn_decode_step(to_dev(d["q"][:, 0]), to_dev(d["k"][:, 0]), to_dev(d["v"][:, 0]),
                          to_dev(np.ascontiguousarray(d["log_alpha"][:, 0])),
                          to_dev(np.ascontiguousarray(d["beta"][:, 0])), state, o, Hk=Hk, Hv=Hv)
        # oracle replay of the sampled heads: one sequence-head at a time, from its own state
        og = to_host(o).reshape(B, Hv, D)
        for i, (b, h) in enumerate(zip(sb, sh)):
            hk = h // (Hv // Hk)
            orf, srf = oracle.recurrence(
                np.ascontiguousarray(d["q"][b:b + 1, :, hk * D:(hk + 1) * D]),
                np.ascontiguousarray(d["k"][b:b + 1, :, hk * D:(hk + 1) * D]),
                np.ascontiguousarray(d["v"][b:b + 1, :, h * D:(h + 1) * D]),
                np.ascontiguousarray(d["log_alpha"][b:b + 1, :, h:h + 1]),
                np.ascontiguousarray(d["beta"][b:b + 1, :, h:h + 1]), 1, 1, ref[i][None, None])
            ref[i] = srf[0]
            assert_out(og[b, h], orf[0, 0], bf16=True, what=f"decode step {s} head {b},{h}")
        if s + 1 in (1, 16, 256):
            st = to_host(state.view(B * Hv, D, D)[torch.from_numpy(sel).cuda()])
            for i in range(len(sel)):
                e = assert_state(st[i], ref[i], what=f"decode state after step {s + 1}")
            print(f"decode {recipe}: state after step {s + 1}: last rel err {e:.2e}")
    del state
    _free()


def test_cfg_long_full_and_two_halves():
    torch = _torch()
    p = W.cfg_long()
    B, T, Hk, Hv, D = p["B"], p["T"], p["Hk"], p["Hv"], p["D"]
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill(q, k, v, la, be, None, so, Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()
    sel = [5, 38]
    _sampled_prefill_check(p, sel, o, so, "long")
    # two halves chained through the state equal one pass (and the oracle)
    h = T // 2
    so1 = torch.empty_like(so)
    so2 = torch.empty_like(so)
    o1 = G.gdn_prefill(q[:, :h], k[:, :h], v[:, :h], la[:, :h].contiguous(), be[:, :h].contiguous(), None, so1,
                       Hk=Hk, Hv=Hv)
    o2 = G.gdn_prefill(q[:, h:], k[:, h:], v[:, h:], la[:, h:].contiguous(), be[:, h:].contiguous(), so1, so2,
                       Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()
    for bh in sel:
        assert_state(to_host(so2[0, bh]), to_host(so[0, bh]), what="two halves vs one pass")
    o12 = torch.cat([o1, o2], dim=1)
    _sampled_prefill_check(p, sel, o12, so2, "long-halves")
    del q, k, v, o, o1, o2, o12
    _free()


def test_cfg_block_full():
    """conv+SiLU -> prefill (L2 flag) -> gated RMSNorm at batch 4, T=32768, 16/128 heads."""
    torch = _torch()
    blk = W.block_inputs()
    B, T, Hk, Hv, D, C = blk["B"], blk["T"], blk["Hk"], blk["Hv"], blk["D"], blk["C"]
    x = to_dev(blk["x"])
    y = G.gdn_conv1d_silu(x, to_dev(blk["conv_w"]))
    qv, kv, vv = y[:, :, :Hk * D], y[:, :, Hk * D:2 * Hk * D], y[:, :, 2 * Hk * D:]
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill(qv, kv, vv, to_dev(blk["log_alpha"]), to_dev(blk["beta"]), None, so, Hk=Hk, Hv=Hv,
                      l2norm=True, l2_eps=1e-6)
    z = to_dev(blk["z"])
    out = G.gdn_gated_rmsnorm(o.view(B * T, Hv * D), z.view(B * T, Hv * D), to_dev(blk["norm_w"]), 1e-5, H=Hv)
    torch.cuda.synchronize()
    del x
    for (b, h) in [(0, 0), (1, 37), (2, 71), (3, 127)]:
        hk = h // (Hv // Hk)
        chans = [(hk * D, "q"), (Hk * D + hk * D, "k"), (2 * Hk * D + h * D, "v")]
        ybf = {}
        for c0, name in chans:
            yr, _ = oracle.conv1d_silu(blk["x"], blk["conv_w"], b=b, c0=c0, c1=c0 + D, n_threads=NTHR)
            yg = to_host(y[b, :, c0:c0 + D])
            err = np.abs(yg - yr)
            tol = conv_tol(yr, conv_abs_sum(blk["x"], blk["conv_w"], None, b, c0, c0 + D))
            assert np.all(err <= tol), f"conv {name} head {h}: {(err - tol).max()}"
            ybf[name] = oracle.round_bf16(yr)   # the API fixes y as bf16
        orf, srf = oracle.recurrence(ybf["q"][None], ybf["k"][None], ybf["v"][None],
                                     np.ascontiguousarray(blk["log_alpha"][b:b + 1, :, h:h + 1]),
                                     np.ascontiguousarray(blk["beta"][b:b + 1, :, h:h + 1]), 1, 1, None,
                                     l2norm=True, l2_eps=1e-6, n_threads=NTHR)
        # q, k, v crossed a bf16 API boundary (the conv output): where a token's decay wipes
        # the state, o_t is beta (k^.q^) v_t, so one ulp of v_t, q_t, k_t moves it by up to
        # 2^-7 + 2^-8 + 2^-8 of |o_t|
        m = assert_out(to_host(o[b, :, h * D:(h + 1) * D]), orf[0], bf16=True, what=f"block prefill {b},{h}",
                       upstream_rel=2.0 ** -6)
        e = assert_state(to_host(so[b, h]), srf[0], what=f"block state {b},{h}")
        obf = oracle.round_bf16(orf[0])          # the API fixes o as bf16
        zr = np.ascontiguousarray(blk["z"][b, :, h * D:(h + 1) * D])
        yn = oracle.gated_rmsnorm(obf, zr, blk["norm_w"], 1e-5, n_threads=NTHR)
        # the norm's input o crossed a bf16 API boundary (2^-7) on top of the conv's (2^-6)
        mn = assert_out(to_host(out.view(B, T, Hv * D)[b, :, h * D:(h + 1) * D]), yn, bf16=True,
                        what=f"block out {b},{h}", upstream_rel=2.0 ** -7 + 2.0 ** -6)
        print(f"block head {b},{h}: prefill excess {m['excess_rms']:.2e}, state {e:.2e}, "
              f"out excess {mn['excess_rms']:.2e} (literal {mn['max_err_rms']:.2e})")
    del y, o, z, out
    _free()
