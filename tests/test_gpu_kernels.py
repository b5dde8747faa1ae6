"""GPU parity of every libgdn entry point against the fp64 oracle, at sizes
the oracle finishes in seconds: several chunks and ragged tails, both gate
recipes, with and without an initial state, the L2 flag, q scaling, the
token-serial and chunked prefill paths, decode steps, conv + SiLU and the
gated RMSNorm, plus edge cases (empty inputs, degenerate gates, state
chaining, determinism).  All calls go through the C ABI."""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_rule_amd import binding as G
from gated_deltanet_recurrence_rule_amd import workloads as W
from helpers import WS_KEY_HEAD, WS_VALUE_HEAD, assert_out, assert_state, to_dev, to_host

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def run_prefill(p, *, l2=False, q_scale=1.0, state_in=None, token_serial=False):
    torch = _torch()
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    B, Hv, D = p["B"], p["Hv"], p["D"]
    si = None if state_in is None else to_dev(state_in.astype(np.float32))
    so = torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill(q, k, v, la, be, si, so, Hk=p["Hk"], Hv=Hv, l2norm=l2, q_scale=q_scale,
                      token_serial=token_serial)
    torch.cuda.synchronize()
    return to_host(o).reshape(B, p["T"], Hv, D), to_host(so)


def oracle_prefill(p, *, l2=False, q_scale=1.0, state_in=None):
    B, T, Hv, D = p["B"], p["T"], p["Hv"], p["D"]
    si = None if state_in is None else state_in.astype(np.float32)
    o, st = oracle.recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], p["Hk"], Hv, si,
                              l2norm=l2, l2_eps=1e-6, q_scale=q_scale)
    # oracle o is [B*Hv, T, D] -> [B, T, Hv, D]
    return o.reshape(B, Hv, T, D).transpose(0, 2, 1, 3), st.reshape(B, Hv, D, D)


CHUNK_CASES = [
    # B, T, Hk, Hv, recipe, state, l2, q_scale
    (1, 1, 1, 1, "qwen", False, False, 1.0),
    (1, 63, 1, 3, "tiny", True, False, 1.0),
    (2, 64, 2, 6, "qwen", False, False, 1.0),
    (1, 65, 1, 8, "qwen", True, True, 1.0),
    (2, 130, 2, 6, "tiny", True, False, 0.5),
    (1, 200, 1, 1, "qwen", False, True, 1.0),
    (1, 257, 2, 6, "qwen", True, False, 1.0),
    # one short of two chunks, and one short of the 64 chunks of the headline length
    (1, 127, 1, 3, "qwen", True, False, 1.0),
    (1, 4095, 2, 6, "qwen", True, False, 1.0),
    # value heads per key head across the prep's groups of three: 4 (3 + 1), 5 (3 + 2), and 64,
    # the most the chunked path takes (21 groups of 3 + 1)
    (1, 100, 1, 4, "qwen", True, False, 1.0),
    (2, 90, 1, 5, "qwen", False, False, 1.0),
    (1, 70, 1, 64, "tiny", True, True, 1.0),
]


@pytest.mark.parametrize("B,T,Hk,Hv,recipe,state,l2,qs", CHUNK_CASES)
def test_prefill_chunk_kernel_parity(B, T, Hk, Hv, recipe, state, l2, qs):
    p = W.problem(1000 + T, B, T, Hk, Hv, 128, io="bf16", recipe=recipe,
                  state="normal" if state else None, normalise=not l2)
    og, sg = run_prefill(p, l2=l2, q_scale=qs, state_in=p["state_in"])
    orf, srf = oracle_prefill(p, l2=l2, q_scale=qs, state_in=p["state_in"])
    m = assert_out(og, orf, bf16=True)
    e = assert_state(sg, srf)
    print(f"chunk B={B} T={T} Hk={Hk} Hv={Hv} {recipe}: out {m} state {e:.2e}")


TOKEN_CASES = [
    # B, T, Hk, Hv, D, io, state, l2
    (1, 64, 1, 1, 16, "f32", False, False),
    (2, 37, 2, 4, 32, "f32", True, False),
    (1, 50, 1, 3, 64, "bf16", True, True),
    (1, 20, 1, 2, 128, "f32", False, False),
    (3, 9, 1, 2, 16, "bf16", True, False),
]


@pytest.mark.parametrize("B,T,Hk,Hv,D,io,state,l2", TOKEN_CASES)
def test_prefill_token_serial_parity(B, T, Hk, Hv, D, io, state, l2):
    p = W.problem(2000 + T + D, B, T, Hk, Hv, D, io=io, recipe="tiny",
                  state="normal" if state else None, normalise=not l2)
    og, sg = run_prefill(p, l2=l2, state_in=p["state_in"])
    orf, srf = oracle_prefill(p, l2=l2, state_in=p["state_in"])
    assert_out(og, orf, bf16=(io == "bf16"))
    assert_state(sg, srf)
    if io == "f32":   # fp32 arithmetic end to end: far inside the bound
        assert np.abs(og - orf).max() <= 1e-4 * np.sqrt(np.mean(orf ** 2))


@pytest.mark.parametrize("v_scale", [1.0, 4096.0])
def test_prefill_token_serial_flag(v_scale):
    """GDN_FLAG_TOKEN_SERIAL runs the fp32 token-serial kernel on a shape the chunked
    kernel would take (bf16, D = 128), including values far beyond fp16's range for
    the state (v scaled by 2^12, slowly decaying gates)."""
    p = W.problem(77, 1, 150, 1, 3, 128, io="bf16", recipe="tiny", state="normal")
    if v_scale != 1.0:
        p["v"] = W.f32_to_bf16(W.bf16_to_f32(p["v"]) * np.float32(v_scale))
        p["state_in"] = (p["state_in"] * v_scale).astype(np.float32)
    og, sg = run_prefill(p, state_in=p["state_in"], token_serial=True)
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    assert_out(og, orf, bf16=True)
    e = max(assert_state(sg[0, h], srf[0, h]) for h in range(3))
    assert e < 1e-5, e   # fp32 arithmetic throughout


# v and S0 far from unit scale on the chunked path (no token-serial flag): exponents of the
# power of two that scales v and that scales S0.  fp16 alone would overflow at 2^12 (values and
# the state past 65504) and drop bits at 2^-12 (most values below its normal range).
RANGE_CASES = [(12, 12), (-12, -12), (12, 0), (0, 12), (-12, 0), (0, -12), (12, -12), (-12, 12)]


def _scale_range(p, ev, es):
    p["v"] = W.f32_to_bf16(W.bf16_to_f32(p["v"]) * np.float32(2.0 ** ev))
    p["state_in"] = (p["state_in"] * np.float32(2.0 ** es)).astype(np.float32)
    return p


@pytest.mark.parametrize("recipe", ["tiny", "qwen"])
@pytest.mark.parametrize("ev,es", RANGE_CASES)
def test_prefill_chunk_value_range(ev, es, recipe):
    """The chunked kernels take V, U and the state into fp16 products scaled per chunk and
    value tile by powers of two, so results hold the stated bounds at any scale of v and
    S0.  The oracle runs on the same scaled inputs in fp64."""
    p = _scale_range(W.problem(4100 + 7 * ev + es, 1, 150, 1, 3, 128, io="bf16", recipe=recipe,
                               state="normal"), ev, es)
    og, sg = run_prefill(p, state_in=p["state_in"])
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    m = assert_out(og, orf, bf16=True)
    e = assert_state(sg, srf)
    print(f"range v 2^{ev} S0 2^{es} {recipe}: out {m} state {e:.2e}")


@pytest.mark.parametrize("ev,es", [(12, 12), (-12, -12)])
def test_prefill_chunk_value_range_windows(ev, es):
    """The same with a workspace of one chunk, so that the scaled state is handed from
    window to window through state_out (in place)."""
    torch = _torch()
    B, T, Hk, Hv, D = 2, 200, 1, 3, 128
    p = _scale_range(W.problem(4200 + ev, B, T, Hk, Hv, D, io="bf16", recipe="tiny", state="normal"), ev, es)
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    st = to_dev(p["state_in"].astype(np.float32))
    ws = torch.empty(B * (Hv * WS_VALUE_HEAD + Hk * WS_KEY_HEAD), dtype=torch.uint8, device="cuda")
    o = G.gdn_prefill(q, k, v, la, be, st, st, Hk=Hk, Hv=Hv, workspace=ws)
    torch.cuda.synchronize()
    assert_out(to_host(o).reshape(B, T, Hv, D), orf, bf16=True)
    assert_state(to_host(st), srf)


@pytest.mark.parametrize("D,io,l2", [(128, "bf16", False), (128, "bf16", True), (16, "f32", False), (64, "bf16", False)])
def test_decode_steps_parity(D, io, l2):
    torch = _torch()
    B, Hk, Hv, steps = 3, 2, 6, 5
    p = W.problem(3000 + D, B, steps, Hk, Hv, D, io=io, recipe="qwen", state="normal", normalise=not l2)
    state = to_dev(p["state_in"].astype(np.float32))
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    ref_state = p["state_in"].astype(np.float32)
    for s in range(steps):
        o = G.gdn_decode_step(q[:, s].contiguous(), k[:, s].contiguous(), v[:, s].contiguous(),
                              la[:, s].contiguous(), be[:, s].contiguous(), state, Hk=Hk, Hv=Hv, l2norm=l2)
        torch.cuda.synchronize()
        sl = slice(s, s + 1)
        c = np.ascontiguousarray
        orf, srf = oracle.recurrence(c(p["q"][:, sl]), c(p["k"][:, sl]), c(p["v"][:, sl]),
                                     c(p["log_alpha"][:, sl]), c(p["beta"][:, sl]), Hk, Hv, ref_state,
                                     l2norm=l2, l2_eps=1e-6)
        ref_state = srf.reshape(B, Hv, D, D)
        assert_out(to_host(o).reshape(B, Hv, D), orf.reshape(B, Hv, D), bf16=(io == "bf16"))
        assert_state(to_host(state), ref_state)


def test_two_halves_equal_one_pass_and_oracle():
    torch = _torch()
    p = W.problem(4001, 1, 200, 2, 6, 128, io="bf16", recipe="qwen", state="normal")
    o_full, s_full = run_prefill(p, state_in=p["state_in"])
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    for cut in (64, 100):
        a = {k_: (v_[:, :cut].copy() if isinstance(v_, np.ndarray) and v_.ndim == 3 else v_) for k_, v_ in p.items()}
        b = {k_: (v_[:, cut:].copy() if isinstance(v_, np.ndarray) and v_.ndim == 3 else v_) for k_, v_ in p.items()}
        a["T"], b["T"] = cut, 200 - cut
        o1, s1 = run_prefill(a, state_in=p["state_in"])
        o2, s2 = run_prefill(b, state_in=s1)
        o12 = np.concatenate([o1, o2], axis=1)
        assert_out(o12, orf, bf16=True)
        assert_state(s2, srf)
        assert_state(s2, s_full)


@pytest.mark.parametrize("with_state_out", [True, False])
def test_prefill_small_workspace_windows(with_state_out):
    # A workspace of one or two chunks forces several prep/chain windows; the state is
    # carried through state_out, or through the workspace's carry area without it.
    torch = _torch()
    B, T, Hk, Hv, D = 2, 300, 1, 3, 128
    p = W.problem(4005, B, T, Hk, Hv, D, io="bf16", recipe="qwen", state="normal")
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    si = to_dev(p["state_in"].astype(np.float32))
    dims = G.make_dims(B, T, Hk, Hv, D, G.GDN_BF16)
    full = G.gdn_prefill_workspace_size(dims)
    per_chunk = B * (Hv * WS_VALUE_HEAD + Hk * WS_KEY_HEAD)
    assert full == 5 * per_chunk
    for nwin in (1, 2):
        extra = 0 if with_state_out else B * Hv * D * D * 4
        ws = torch.empty(nwin * per_chunk + extra, dtype=torch.uint8, device="cuda")
        so = torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda") if with_state_out else None
        o = G.gdn_prefill(q, k, v, la, be, si, so, Hk=Hk, Hv=Hv, workspace=ws)
        torch.cuda.synchronize()
        assert_out(to_host(o).reshape(B, T, Hv, D), orf, bf16=True)
        if with_state_out:
            assert_state(to_host(so), srf)


@pytest.mark.parametrize("nwin", [1, 2, None])
def test_prefill_state_in_place(nwin):
    """state_out may be the same pointer as state_in (gdn.h): the chunked path reads the entry
    state before it writes the final one, also when the sequence runs over several windows (a
    workspace of one or two chunks) and each window hands the state on through state_out."""
    torch = _torch()
    B, T, Hk, Hv, D = 2, 300, 1, 3, 128
    p = W.problem(4007, B, T, Hk, Hv, D, io="bf16", recipe="qwen", state="normal")
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    st = to_dev(p["state_in"].astype(np.float32))
    ws = None
    if nwin is not None:
        ws = torch.empty(nwin * B * (Hv * WS_VALUE_HEAD + Hk * WS_KEY_HEAD), dtype=torch.uint8, device="cuda")
    o = G.gdn_prefill(q, k, v, la, be, st, st, Hk=Hk, Hv=Hv, workspace=ws)
    torch.cuda.synchronize()
    assert_out(to_host(o).reshape(B, T, Hv, D), orf, bf16=True)
    assert_state(to_host(st), srf)


@pytest.mark.parametrize("T,nwin,G_", [(200, None, 8), (130, 1, 8), (65, 2, 3)])
def test_prefill_whole_heads(T, nwin, G_):
    """B * Hv at least the CU count (2 x 128 value heads, or 3 x 96): one chain workgroup per
    value head, with diag(rk) K stored once per key head and the row factors applied in the
    chain.  All heads against the oracle, with an initial state, the L2 flag and ragged tails;
    also over one- or two-chunk windows with the state updated in place."""
    torch = _torch()
    B, Hk, D = (2, 16, 128) if G_ == 8 else (3, 32, 128)
    Hv = Hk * G_
    p = W.problem(4010 + T, B, T, Hk, Hv, D, io="bf16", recipe="qwen", state="normal", normalise=False)
    orf, srf = oracle_prefill(p, l2=True, state_in=p["state_in"])
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    st = to_dev(p["state_in"].astype(np.float32))
    ws = None
    if nwin is not None:
        ws = torch.empty(nwin * B * (Hv * WS_VALUE_HEAD + Hk * WS_KEY_HEAD), dtype=torch.uint8, device="cuda")
    o = G.gdn_prefill(q, k, v, la, be, st, st, Hk=Hk, Hv=Hv, l2norm=True, workspace=ws)
    torch.cuda.synchronize()
    m = assert_out(to_host(o).reshape(B, T, Hv, D), orf, bf16=True)
    e = assert_state(to_host(st), srf)
    print(f"whole heads B={B} T={T} {Hk}/{Hv} windows={nwin}: out excess {m['metric']:.2e} state {e:.2e}")


def test_prefill_one_slot_chain():
    # 3 x 24 value heads x 4 strips = 288 chain workgroups, more than the 256 CUs: the chain runs
    # with one input slot per workgroup and a second barrier per chunk.  Checked with the whole
    # workspace (one window) and with one chunk of workspace and no state_out (the state crosses
    # the four windows through the carry area).
    torch = _torch()
    B, T, Hk, Hv, D = 3, 200, 8, 24, 128
    p = W.problem(4006, B, T, Hk, Hv, D, io="bf16", recipe="qwen", state="normal")
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    o, so = run_prefill(p, state_in=p["state_in"])
    assert_out(o, orf, bf16=True)
    assert_state(so, srf)
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    si = to_dev(p["state_in"].astype(np.float32))
    per_chunk = B * (Hv * WS_VALUE_HEAD + Hk * WS_KEY_HEAD)
    ws = torch.empty(per_chunk + B * Hv * D * D * 4, dtype=torch.uint8, device="cuda")
    o2 = G.gdn_prefill(q, k, v, la, be, si, None, Hk=Hk, Hv=Hv, workspace=ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(o2).reshape(B, T, Hv, D), o)   # windows do not change the arithmetic


def test_decode_steps_equal_prefill():
    torch = _torch()
    B, T, Hk, Hv, D = 2, 40, 1, 3, 128
    p = W.problem(4002, B, T, Hk, Hv, D, io="bf16", recipe="tiny", state="normal")
    o_pre, s_pre = run_prefill(p, state_in=p["state_in"])
    state = to_dev(p["state_in"].astype(np.float32))
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    outs = []
    for t in range(T):
        outs.append(G.gdn_decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                      la[:, t].contiguous(), be[:, t].contiguous(), state, Hk=Hk, Hv=Hv))
    torch.cuda.synchronize()
    o_dec = np.stack([to_host(o).reshape(B, Hv, D) for o in outs], axis=1)
    orf, srf = oracle_prefill(p, state_in=p["state_in"])
    assert_out(o_dec, orf, bf16=True)
    assert_out(o_pre, orf, bf16=True)
    assert_state(to_host(state), srf)
    assert_state(to_host(state), s_pre)


def test_degenerate_gates():
    torch = _torch()
    B, T, Hk, Hv, D = 1, 100, 1, 2, 128
    p = W.problem(4003, B, T, Hk, Hv, D, io="bf16", recipe="qwen", state="normal")
    # alpha = 1, beta = 0: the state is left exactly as it was; o_t = S_0 q_t.
    p0 = dict(p, log_alpha=np.zeros_like(p["log_alpha"]), beta=np.zeros_like(p["beta"]))
    og, sg = run_prefill(p0, state_in=p["state_in"])
    np.testing.assert_array_equal(sg, p["state_in"].astype(np.float32).astype(np.float64))
    orf, _ = oracle_prefill(p0, state_in=p["state_in"])
    assert_out(og, orf, bf16=True)
    # very strong decay (alpha underflows to 0 in one chunk) must stay finite and match
    p1 = dict(p, log_alpha=np.full_like(p["log_alpha"], -1000.0))
    og, sg = run_prefill(p1, state_in=p["state_in"])
    orf, srf = oracle_prefill(p1, state_in=p["state_in"])
    assert_out(og, orf, bf16=True)
    assert_state(sg, srf)
    # beta = 1, alpha = 1 (pure overwrite writes)
    p2 = dict(p, log_alpha=np.zeros_like(p["log_alpha"]), beta=np.ones_like(p["beta"]))
    og, sg = run_prefill(p2)
    orf, srf = oracle_prefill(p2)
    assert_out(og, orf, bf16=True)
    assert_state(sg, srf)


def test_empty_inputs():
    torch = _torch()
    D, Hv = 128, 3
    st = to_dev(W.normal_tokens(7, "state", Hv * D, D).reshape(1, Hv, D, D))
    so = torch.full_like(st, 7.0)
    z = torch.empty((1, 0, 128), dtype=torch.bfloat16, device="cuda")
    zv = torch.empty((1, 0, Hv * 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((1, 0, Hv), dtype=torch.float32, device="cuda")
    G.gdn_prefill(z, z, zv, g, g, st, so, Hk=1, Hv=Hv)
    torch.cuda.synchronize()
    assert torch.equal(so, st)               # T = 0 hands the state through unchanged
    G.gdn_prefill(z, z, zv, g, g, None, so, Hk=1, Hv=Hv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(so).item() == 0   # ... or the zero state when none is given


def test_chunk_kernel_is_deterministic():
    torch = _torch()
    p = W.problem(4004, 1, 300, 2, 6, 128, io="bf16", recipe="qwen", state="normal")
    o1, s1 = run_prefill(p, state_in=p["state_in"])
    o2, s2 = run_prefill(p, state_in=p["state_in"])
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("T", [0, 1, 2, 5, 130])
def test_conv1d_silu_parity(io, T):
    torch = _torch()
    B, C = 2, 2048 + 64
    rng_x = W.normal_tokens(5000 + T, "x", B * max(T, 1), C + 16)[: B * T]
    x_full = rng_x.reshape(B, T, C + 16)
    w = W.normal_tokens(5000, "conv_w", C, 4, scale=0.5)
    cs = W.normal_tokens(5000, "conv_state", B * C, 3).reshape(B, C, 3)
    cv = W.f32_to_bf16 if io == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    xh, wh, csh = cv(x_full), cv(w), cv(cs)
    x_dev = to_dev(xh)[:, :, :C]          # strided view: token stride C + 16
    y = torch.zeros((B, T, C), dtype=x_dev.dtype, device="cuda")
    cso = torch.zeros((B, C, 3), dtype=x_dev.dtype, device="cuda")
    G.gdn_conv1d_silu(x_dev, to_dev(wh), to_dev(csh), cso, y)
    torch.cuda.synchronize()
    yg = to_host(y)
    xv = xh[:, :, :C]                      # the same strided view on the host
    for b in range(B):
        if T > 0:
            yr, _ = oracle.conv1d_silu(xv, wh, csh, b=b)
            err = np.abs(yg[b] - yr)
            if io == "bf16":
                from helpers import conv_abs_sum, conv_tol
                assert np.all(err <= conv_tol(yr, conv_abs_sum(xh, wh, csh, b, 0, C))), err.max()
            else:
                assert err.max() <= 1e-5 * np.abs(yr).max()
    _, csr = oracle.conv1d_silu(xv, wh, csh, want_state=True) if T > 0 else (None, None)
    if T > 0:
        np.testing.assert_array_equal(to_host(cso), csr)
    else:
        np.testing.assert_array_equal(to_host(cso), to_host(to_dev(csh)))


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 5, 130])
def test_conv1d_silu_l2_parity(io, T):
    """gdn_conv1d_silu_l2: conv + SiLU, then the q and k channels [0, 2 Hk D) L2-normalised per
    128-channel head, against the oracle's conv followed by the oracle's per-head normalisation.
    The v channels and the conv window handed on are gdn_conv1d_silu's, bit for bit."""
    from helpers import conv_abs_sum, ulp_bf16
    torch = _torch()
    B, Hk, Hv, D = 2, 2, 6, 128
    C, L = (2 * Hk + Hv) * D, 2 * Hk * D
    eps = 1e-6
    x_full = W.normal_tokens(5100 + T, "x", B * T, C + 16).reshape(B, T, C + 16)
    w = W.normal_tokens(5100, "conv_w", C, 4, scale=0.5)
    cs = W.normal_tokens(5100, "conv_state", B * C, 3).reshape(B, C, 3)
    cv = W.f32_to_bf16 if io == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    xh, wh, csh = cv(x_full), cv(w), cv(cs)
    x_dev = to_dev(xh)[:, :, :C]
    cso = torch.zeros((B, C, 3), dtype=x_dev.dtype, device="cuda")
    y = G.gdn_conv1d_silu(x_dev, to_dev(wh), to_dev(csh), cso, l2_channels=L, l2_eps=eps)
    cso_p = torch.zeros_like(cso)
    y_plain = G.gdn_conv1d_silu(x_dev, to_dev(wh), to_dev(csh), cso_p)
    torch.cuda.synchronize()
    yg, yp = to_host(y), to_host(y_plain)
    np.testing.assert_array_equal(yg[:, :, L:], yp[:, :, L:])
    np.testing.assert_array_equal(to_host(cso), to_host(cso_p))
    xv = xh[:, :, :C]
    for b in range(B):
        yr, _ = oracle.conv1d_silu(xv, wh, csh, b=b)
        yn = oracle.l2norm_heads(yr[:, :L], D, eps)
        norm = np.repeat(np.sqrt((yr[:, :L].reshape(T, -1, D) ** 2).sum(-1) + eps), D, axis=1)
        # the conv's fp32 accumulation error (2^-21 of the sum of |terms|) carried through the
        # normalisation, the normalisation's own fp32 rounding, and the final rounding to io
        tol = 2.0 ** -21 * conv_abs_sum(xh, wh, csh, b, 0, L) / norm + 2.0 ** -20
        if io == "bf16":
            tol = tol + ulp_bf16(yn)
        err = np.abs(yg[b, :, :L] - yn)
        assert np.all(err <= tol), float((err - tol).max())


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("H,D", [(1, 128), (3, 128), (4, 64)])
def test_gated_rmsnorm_parity(io, H, D):
    torch = _torch()
    n = 37
    x = W.normal_tokens(6000 + H, "x", n, H * D)
    z = W.normal_tokens(6000 + H, "z", n, H * D + 32)
    w = W.normal_tokens(6000, "norm_w", 1, D, loc=1.0, scale=0.1)[0]
    cv = W.f32_to_bf16 if io == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
    xh, zh, wh = cv(x), cv(z), cv(w)
    zd = to_dev(zh)[:, 16:16 + H * D]      # a view with row stride H*D + 32
    y = G.gdn_gated_rmsnorm(to_dev(xh), zd, to_dev(wh), 1e-5, H=H)
    torch.cuda.synchronize()
    zc = np.ascontiguousarray(zh[:, 16:16 + H * D])
    yr = oracle.gated_rmsnorm(xh.reshape(n * H, D), zc.reshape(n * H, D), wh, 1e-5)
    yg = to_host(y).reshape(n * H, D)
    if io == "bf16":
        assert_out(yg, yr, bf16=True, tol=1e-3)
    else:
        assert np.abs(yg - yr).max() <= 1e-5 * np.sqrt(np.mean(yr ** 2))
    # in place (y aliases x)
    xd = to_dev(xh)
    G.gdn_gated_rmsnorm(xd, zd, to_dev(wh), 1e-5, y=xd, H=H)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(xd).reshape(n * H, D), yg)


def _raw_ba(seed, n, Hv):
    """Raw in_proj_ba outputs: N(0, 2^2) draws plus fixed extreme values on the first rows."""
    rng = np.random.default_rng(seed)
    ba = (rng.standard_normal((n, 2 * Hv)) * 2.0).astype(np.float32)
    ext = np.array([0.0, 40.0, -40.0, 100.0, -100.0, 7.5, -7.5, 1e-3], np.float32)
    for i, x in enumerate(ext[: min(n, ext.size)]):
        ba[i, :] = x
    return ba


@pytest.mark.gpu
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_gates_parity(io):
    """gdn_gates against the oracle's fp64 activation.  fp32 arithmetic: the fast exponential
    scales its argument by log2(e) in fp32, so e^x carries a relative error up to about
    |x| * 2^-24; with |x| <= 100 here every output is within 1e-5 relative."""
    torch = _torch()
    n, Hv = 1003, 48
    rng = np.random.default_rng(51)
    A = np.log(rng.uniform(1.0, 16.0, Hv)).astype(np.float32)
    dt = (rng.standard_normal(Hv) * 0.5).astype(np.float32)
    ba = _raw_ba(52, n, Hv)
    if io == "bf16":
        ba = W.f32_to_bf16(ba)
    # a strided view: rows of 2*Hv + 8 elements
    pad = np.zeros((n, 2 * Hv + 8), ba.dtype)
    pad[:, : 2 * Hv] = ba
    dev = to_dev(pad)[:, : 2 * Hv]
    la, be = G.gdn_gates(dev, to_dev(A), to_dev(dt), Hv=Hv)
    torch.cuda.synchronize()
    la_ref, be_ref = oracle.gates(ba, Hv, A, dt)
    np.testing.assert_allclose(to_host(la), la_ref, rtol=1e-5, atol=1e-37)
    np.testing.assert_allclose(to_host(be), be_ref, rtol=1e-5, atol=1e-37)
    assert np.all(to_host(la) <= 0) and np.all((to_host(be) >= 0) & (to_host(be) <= 1))


@pytest.mark.gpu
@pytest.mark.parametrize("l2", [False, True])
@pytest.mark.parametrize("ba_io", ["bf16", "f32"])
def test_decode_token_gates_and_slots(l2, ba_io):
    """gdn_decode_token: gates formed in the kernel from raw in_proj_ba outputs, states in a
    pool addressed by a slot table (a permutation with a negative slot and one past the pool's
    end, both skipped), against the oracle's activation followed by its recurrence on the gathered
    states; untouched pool entries and the skipped output rows must stay bit-identical."""
    torch = _torch()
    B, Hk, Hv, D, S, steps = 6, 2, 6, 128, 8, 3
    slots = np.array([6, -1, 2, 0, 7, 8], np.int32)
    rng = np.random.default_rng(53)
    A = np.log(rng.uniform(1.0, 16.0, Hv)).astype(np.float32)
    dt = (rng.standard_normal(Hv) * 0.5).astype(np.float32)
    p = W.problem(5100, B, steps, Hk, Hv, D, io="bf16", recipe="qwen", state="normal", normalise=not l2)
    pool = (rng.standard_normal((S, Hv, D, D)) * 0.02).astype(np.float32)
    pool_dev = to_dev(pool)
    ref_pool = pool.astype(np.float64)
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    for s in range(steps):
        ba = _raw_ba(5200 + s, B, Hv)
        ba_in = W.f32_to_bf16(ba) if ba_io == "bf16" else ba
        o = torch.full((B, Hv * D), 7.0, dtype=torch.bfloat16, device="cuda")
        G.gdn_decode_token(q[:, s].contiguous(), k[:, s].contiguous(), v[:, s].contiguous(), to_dev(ba_in),
                           to_dev(A), to_dev(dt), pool_dev, to_dev(slots), o, Hk=Hk, Hv=Hv, l2norm=l2)
        torch.cuda.synchronize()
        la, be = oracle.gates(ba_in, Hv, A, dt)
        live = (slots >= 0) & (slots < S)
        c = np.ascontiguousarray
        sl = slice(s, s + 1)
        orf, srf = oracle.recurrence(c(p["q"][live][:, sl]), c(p["k"][live][:, sl]), c(p["v"][live][:, sl]),
                                     c(la[live][:, None]), c(be[live][:, None]), Hk, Hv,
                                     c(ref_pool[slots[live]]), l2norm=l2, l2_eps=1e-6)
        ref_pool[slots[live]] = srf.reshape(-1, Hv, D, D)
        oh = to_host(o).reshape(B, Hv, D)
        assert_out(oh[live], orf.reshape(-1, Hv, D), bf16=True)
        assert np.all(oh[~live] == 7.0)
        ph = to_host(pool_dev)
        for sidx in range(S):
            if sidx in slots[live]:
                assert_state(ph[sidx], ref_pool[sidx])
            else:
                np.testing.assert_array_equal(ph[sidx], pool[sidx])


@pytest.mark.gpu
def test_conv_single_token_steps_roll_the_window():
    """Decode front end: T single-token conv calls, each handing its 3-input window to the next,
    equal one conv over the T tokens (and the oracle)."""
    torch = _torch()
    B, T, C = 3, 9, 10240
    rng = np.random.default_rng(54)
    x = W.f32_to_bf16(rng.standard_normal((B, T, C)).astype(np.float32))
    w = W.f32_to_bf16((rng.standard_normal((C, 4)) * 0.5).astype(np.float32))
    cs0 = W.f32_to_bf16(rng.standard_normal((B, C, 3)).astype(np.float32))
    xd, wd = to_dev(x), to_dev(w)
    full = G.gdn_conv1d_silu(xd, wd, to_dev(cs0))
    cs = to_dev(cs0)
    steps = []
    for t in range(T):
        nxt = torch.empty_like(cs)
        steps.append(G.gdn_conv1d_silu(xd[:, t:t + 1], wd, cs, nxt))
        cs = nxt
    torch.cuda.synchronize()
    y_steps = np.concatenate([to_host(y) for y in steps], axis=1)
    np.testing.assert_array_equal(y_steps, to_host(full))
    ref = np.stack([oracle.conv1d_silu(x, w, cs0, b=b)[0] for b in range(B)])
    assert_out(y_steps, ref, bf16=True)
    # the window handed on after the last step holds the last three inputs, oldest first
    np.testing.assert_array_equal(to_host(cs), W.bf16_to_f32(np.ascontiguousarray(x[:, T - 3:].transpose(0, 2, 1))))


@pytest.mark.gpu
@pytest.mark.parametrize("l2", [True, False])
def test_decode_layer_fused_parity(l2):
    """gdn_decode_layer (conv window, L2 norm, gates from raw in_proj_ba, recurrence on a pooled
    state, gated RMSNorm) against the oracle's conv, gate activation, recurrence and norm applied
    in turn in fp64, over three tokens with the window pools swapped each step and a slot table
    with one skipped sequence.  Moved window entries are bf16 copies and must match exactly."""
    torch = _torch()
    B, Hk, Hv, D, S, steps = 5, 2, 6, 128, 8, 3
    C = (2 * Hk + Hv) * D
    slots = np.array([3, 7, -1, 0, 9], np.int32)   # -1 and 9 (past the 8-entry pools) are skipped
    live = (slots >= 0) & (slots < S)
    rng = np.random.default_rng(61)
    bf = lambda a: W.f32_to_bf16(np.asarray(a, np.float32))
    A = np.log(rng.uniform(1.0, 16.0, Hv)).astype(np.float32)
    dt = (rng.standard_normal(Hv) * 0.5).astype(np.float32)
    cw = bf(rng.standard_normal((C, 4)) * 0.5)
    nw = bf(1.0 + 0.1 * rng.standard_normal(D))
    cs = [bf(rng.standard_normal((S, C, 3))), bf(np.full((S, C, 3), 3.0))]
    pool = (rng.standard_normal((S, Hv, D, D)) * 0.02).astype(np.float32)
    ref_pool = pool.astype(np.float64)
    ref_cs = cs[0].copy()
    d_cs = [to_dev(cs[0]), to_dev(cs[1])]
    d_pool, d_cw, d_nw, d_A, d_dt, d_slots = to_dev(pool), to_dev(cw), to_dev(nw), to_dev(A), to_dev(dt), to_dev(slots)
    eps = 1e-6
    for s in range(steps):
        x = bf(rng.standard_normal((B, C)))
        ba = bf(rng.standard_normal((B, 2 * Hv)) * 2.0)
        z = bf(rng.standard_normal((B, Hv * D)))
        out = torch.full((B, Hv * D), 5.0, dtype=torch.bfloat16, device="cuda")
        o = torch.full((B, Hv * D), 5.0, dtype=torch.bfloat16, device="cuda")
        G.gdn_decode_layer(to_dev(x), d_cw, d_cs[s % 2], d_cs[(s + 1) % 2], to_dev(ba), d_A, d_dt, d_pool, to_dev(z),
                           d_nw, d_slots, out, o, Hk=Hk, Hv=Hv, l2norm=l2, norm_eps=eps)
        torch.cuda.synchronize()
        # oracle, sequence by sequence: conv with the pooled window, gates, recurrence, norm
        la, be = oracle.gates(ba, Hv, A, dt)
        outs, pres = [], []
        for b in np.nonzero(live)[0]:
            sl = slots[b]
            y, win = oracle.conv1d_silu(x[b][None, None], cw, ref_cs[sl][None], want_state=True)
            y = y[0]
            q, k, v = y[:Hk * D], y[Hk * D:2 * Hk * D], y[2 * Hk * D:]
            orf, srf = oracle.recurrence(q[None, None], k[None, None], v[None, None], la[b][None, None],
                                         be[b][None, None], Hk, Hv, ref_pool[sl][None], l2norm=l2, l2_eps=1e-6)
            ref_pool[sl] = srf.reshape(Hv, D, D)
            ref_cs[sl] = W.f32_to_bf16(win[0].astype(np.float32))
            pre = orf.reshape(Hv, D)
            pres.append(pre)
            outs.append(oracle.gated_rmsnorm(pre, W.bf16_to_f32(z[b]).reshape(Hv, D).astype(np.float64),
                                             W.bf16_to_f32(nw).astype(np.float64), eps))
        oh, ph = to_host(out).reshape(B, Hv, D), to_host(o).reshape(B, Hv, D)
        assert_out(ph[live], np.stack(pres), bf16=True, what="o")
        assert_out(oh[live], np.stack(outs), bf16=True, what="out")
        assert np.all(oh[~live] == 5.0) and np.all(ph[~live] == 5.0)
        hp = to_host(d_pool)
        for sl in range(S):
            if sl in slots[live]:
                assert_state(hp[sl], ref_pool[sl])
            else:
                np.testing.assert_array_equal(hp[sl], pool[sl])
        # window pools: entries of live slots moved on exactly; the others untouched
        written = d_cs[(s + 1) % 2].view(torch.int16).cpu().numpy().view(np.uint16)
        before = cs[(s + 1) % 2]
        for sl in range(S):
            if sl in slots[live]:
                np.testing.assert_array_equal(written[sl], ref_cs[sl])
            else:
                np.testing.assert_array_equal(written[sl], before[sl])
        cs[(s + 1) % 2] = written.copy()


# A seeded property grid over small shapes: batch <= 3, T <= 300, 1 or 2 key
# heads, 1, 3 or 8 value heads per key head, head width 16 or 128, fp32 or bf16 I/O.  Each case draws
# its own lengths, gate recipe, initial state, L2 flag and q scale.  bf16 with width 128 runs the
# chunked kernels; the other cases run the token-serial kernel.
PROPERTY_GRID = [(Hk, G_, D, io) for Hk in (1, 2) for G_ in (1, 3, 8) for D in (16, 128) for io in ("f32", "bf16")]


@pytest.mark.parametrize("Hk,G_,D,io", PROPERTY_GRID)
def test_property_grid(Hk, G_, D, io):
    rng = np.random.default_rng(9000 + 100 * Hk + 10 * G_ + D + (io == "bf16"))
    B = int(rng.integers(1, 4))
    T = int(rng.integers(1, 301))
    recipe = "qwen" if rng.random() < 0.5 else "tiny"
    state = bool(rng.random() < 0.5)
    l2 = bool(rng.random() < 0.5)
    qs = float(rng.choice([1.0, 0.5, D ** -0.5]))
    p = W.problem(int(rng.integers(1, 1 << 30)), B, T, Hk, Hk * G_, D, io=io, recipe=recipe,
                  state="normal" if state else None, normalise=not l2)
    og, sg = run_prefill(p, l2=l2, q_scale=qs, state_in=p["state_in"])
    orf, srf = oracle_prefill(p, l2=l2, q_scale=qs, state_in=p["state_in"])
    m = assert_out(og, orf, bf16=(io == "bf16"))
    e = assert_state(sg, srf)
    print(f"grid B={B} T={T} Hk={Hk} G={G_} D={D} {io} {recipe} state={state} l2={l2} qs={qs:.3f}: "
          f"out {m['metric']:.2e} state {e:.2e}")
