"""GPU parity of gdn_prefill_gated (the prefill, then the gated RMSNorm of every
output row) against the fp64 oracle: the oracle's recurrence gives the unrounded
outputs, the oracle's norm runs on those, and the GPU's bf16 y is held to the
output bound.  Both paths are covered: the norm inside the chain kernel (one
workgroup per value head, forced with GDN_FLAG_NORM_IN_CHAIN at these small
batches) and the prefill followed by the norm over y in place.  All calls go
through the C ABI."""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_rule_amd import binding as G
from gated_deltanet_recurrence_rule_amd import workloads as W
from helpers import WS_KEY_HEAD, WS_VALUE_HEAD, assert_out, assert_state, to_dev, to_host

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _torch():
    import torch
    return torch


def _gate_inputs(seed, B, T, Hv, D):
    """z as a strided view (rows of Hv*D + 64 channels) and norm weights about 1."""
    z = W.normal_tokens(seed, "z", B * T, Hv * D + 64).reshape(B, T, Hv * D + 64)
    w = W.normal_tokens(seed, "norm_w", 1, D, loc=1.0, scale=0.1)[0]
    return W.f32_to_bf16(z), W.f32_to_bf16(w)


def _oracle_gated(p, zb, wb, *, l2, q_scale=1.0):
    B, T, Hv, D = p["B"], p["T"], p["Hv"], p["D"]
    si = None if p["state_in"] is None else p["state_in"].astype(np.float32)
    o, st = oracle.recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], p["Hk"], Hv, si,
                              l2norm=l2, l2_eps=1e-6, q_scale=q_scale)
    o = o.reshape(B, Hv, T, D).transpose(0, 2, 1, 3)                     # [B, T, Hv, D], fp64
    z = W.bf16_to_f32(zb[:, :, 32:32 + Hv * D]).astype(np.float64).reshape(B * T * Hv, D)
    y = oracle.gated_rmsnorm(np.ascontiguousarray(o.reshape(B * T * Hv, D)), z,
                             W.bf16_to_f32(wb).astype(np.float64), EPS)
    return y.reshape(B, T, Hv, D), st.reshape(B, Hv, D, D)


def _run_gated(p, zb, wb, *, l2, in_chain, q_scale=1.0, ws_chunks=None, in_place=False):
    torch = _torch()
    B, T, Hk, Hv, D = p["B"], p["T"], p["Hk"], p["Hv"], p["D"]
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    z = to_dev(zb)[:, :, 32:32 + Hv * D]
    w = to_dev(wb)
    si = None if p["state_in"] is None else to_dev(p["state_in"].astype(np.float32))
    so = si if in_place else torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda")
    ws = None
    if ws_chunks is not None:
        per = B * Hv * WS_VALUE_HEAD + B * Hk * WS_KEY_HEAD
        ws = torch.empty(per * ws_chunks, dtype=torch.uint8, device="cuda")
    y = G.gdn_prefill_gated(q, k, v, la, be, z, w, EPS, si, so, Hk=Hk, Hv=Hv, l2norm=l2, q_scale=q_scale,
                            in_chain=in_chain, workspace=ws)
    torch.cuda.synchronize()
    return to_host(y).reshape(B, T, Hv, D), to_host(so)


GATED_CASES = [
    # B, T, Hk, Hv, recipe, state, l2, in_chain, one-chunk windows
    (1, 1, 1, 3, "qwen", False, True, True, False),
    (1, 63, 1, 3, "tiny", True, True, True, False),
    (2, 65, 2, 6, "qwen", False, True, True, False),
    (1, 200, 2, 16, "qwen", True, False, True, False),
    (2, 130, 1, 8, "tiny", True, True, True, False),
    (1, 300, 2, 6, "qwen", True, True, True, True),
    (1, 257, 1, 3, "qwen", True, True, False, False),
    (2, 100, 2, 6, "tiny", False, True, False, True),
]


@pytest.mark.parametrize("B,T,Hk,Hv,recipe,state,l2,in_chain,windows", GATED_CASES)
def test_prefill_gated_parity(B, T, Hk, Hv, recipe, state, l2, in_chain, windows):
    D = 128
    p = W.problem(7100 + 10 * B + T + Hv, B, T, Hk, Hv, D, recipe=recipe,
                  state="normal" if state else None, normalise=not l2)
    zb, wb = _gate_inputs(7200 + T, B, T, Hv, D)
    yg, sg = _run_gated(p, zb, wb, l2=l2, in_chain=in_chain, ws_chunks=1 if windows else None)
    yr, sr = _oracle_gated(p, zb, wb, l2=l2)
    m = assert_out(yg, yr, bf16=True, what="y")
    e = assert_state(sg, sr)
    print(f"gated B={B} T={T} {Hk}/{Hv} {recipe} in_chain={in_chain} windows={windows}: "
          f"y excess {m['metric']:.2e} state {e:.2e}")


def test_prefill_gated_state_matches_prefill_and_paths_agree():
    """The two-launch path's state is gdn_prefill's to the bit; the fused path (whole heads,
    the key rows stored once per key head and scaled in the chain) rounds its fp16 operands
    differently and is held to the oracle's bound.  The two y differ through o's bf16 rounding
    before the norm and through those operand roundings."""
    torch = _torch()
    B, T, Hk, Hv, D = 2, 200, 2, 6, 128
    p = W.problem(7301, B, T, Hk, Hv, D, recipe="qwen", state="normal")
    zb, wb = _gate_inputs(7302, B, T, Hv, D)
    y_chain, s_chain = _run_gated(p, zb, wb, l2=True, in_chain=True)
    y_two, s_two = _run_gated(p, zb, wb, l2=True, in_chain=False)
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda")
    G.gdn_prefill(q, k, v, to_dev(p["log_alpha"]), to_dev(p["beta"]), to_dev(p["state_in"].astype(np.float32)),
                  so, Hk=Hk, Hv=Hv, l2norm=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s_two, to_host(so))
    yr, sr = _oracle_gated(p, zb, wb, l2=True)
    assert_state(s_chain, sr, what="state (norm in the chain)")
    assert_out(y_two, yr, bf16=True, what="y (two launches)")
    assert_out(y_chain, yr, bf16=True, what="y (norm in the chain)")


def test_prefill_gated_windows_in_place_bit_identical():
    """One-chunk windows with the state updated in place give the same bits as one window."""
    B, T, Hk, Hv, D = 1, 300, 1, 3, 128
    p = W.problem(7401, B, T, Hk, Hv, D, recipe="qwen", state="normal")
    zb, wb = _gate_inputs(7402, B, T, Hv, D)
    y1, s1 = _run_gated(p, zb, wb, l2=True, in_chain=True)
    y2, s2 = _run_gated(p, zb, wb, l2=True, in_chain=True, ws_chunks=1, in_place=True)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(s1, s2)


def test_prefill_gated_value_range():
    """The chunked path's range scaling under the gated norm: v and S0 at 2^12."""
    B, T, Hk, Hv, D = 1, 200, 1, 3, 128
    p = W.problem(7501, B, T, Hk, Hv, D, recipe="qwen", state="normal")
    big = 2.0 ** 12
    p["v"] = W.f32_to_bf16(W.bf16_to_f32(p["v"]) * np.float32(big))
    p["state_in"] = (p["state_in"] * big).astype(p["state_in"].dtype)
    zb, wb = _gate_inputs(7502, B, T, Hv, D)
    yg, sg = _run_gated(p, zb, wb, l2=True, in_chain=True)
    yr, sr = _oracle_gated(p, zb, wb, l2=True)
    assert_out(yg, yr, bf16=True, what="y")
    assert_state(sg, sr)
