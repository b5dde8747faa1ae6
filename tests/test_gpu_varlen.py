"""GPU parity of the packed variable-length prefill (gdn_prefill_varlen) against the
fp64 oracle run sequence by sequence, and against one gdn_prefill call per sequence:
empty, one-token, chunk-sized and ragged sequences in one packed stream, with and
without initial and final states, workspaces small enough that windows split
sequences, and the token-serial path.  All calls go through the C ABI."""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_rule_amd import binding as G
from gated_deltanet_recurrence_rule_amd import workloads as W
from helpers import WS_KEY_HEAD, WS_VALUE_HEAD, assert_out, assert_state, to_dev, to_host

pytestmark = pytest.mark.gpu

LENS = [1, 63, 64, 65, 130, 0, 200, 7]


def _torch():
    import torch
    return torch


def packed_problem(seed, lens, Hk, Hv, D, io, recipe="qwen", state=True, normalise=True):
    p = W.problem(seed, 1, int(sum(lens)), Hk, Hv, D, io=io, recipe=recipe, normalise=normalise)
    st = None
    if state:
        st = W.problem(seed + 1, len(lens), 1, Hk, Hv, D, io=io, recipe=recipe, state="normal")["state_in"]
        st = st.astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return p, st, cu


def oracle_packed(p, st, cu, *, l2=False):
    """Per-sequence oracle runs on slices of the packed stream: o [T, Hv, D], states [n, Hv, D, D]."""
    Hk, Hv, D = p["Hk"], p["Hv"], p["D"]
    n = len(cu) - 1
    o = np.zeros((p["T"], Hv, D))
    states = np.zeros((n, Hv, D, D))
    for s in range(n):
        a, b = int(cu[s]), int(cu[s + 1])
        si = None if st is None else st[s:s + 1]
        if a == b:   # an empty sequence hands its state through
            states[s] = 0.0 if si is None else si[0]
            continue
        sl = lambda x: np.ascontiguousarray(x[:, a:b])
        os_, ss = oracle.recurrence(sl(p["q"]), sl(p["k"]), sl(p["v"]), sl(p["log_alpha"]), sl(p["beta"]),
                                    Hk, Hv, si, l2norm=l2, l2_eps=1e-6)
        o[a:b] = os_.reshape(Hv, b - a, D).transpose(1, 0, 2)
        states[s] = ss.reshape(Hv, D, D)
    return o, states


def run_packed(p, st, cu, *, l2=False, token_serial=False, with_state_out=True, workspace=None):
    torch = _torch()
    Hk, Hv, D = p["Hk"], p["Hv"], p["D"]
    n = len(cu) - 1
    q, k, v = (to_dev(p[x][0]) for x in ("q", "k", "v"))
    la, be = to_dev(p["log_alpha"][0]), to_dev(p["beta"][0])
    si = None if st is None else to_dev(st)
    so = torch.full((n, Hv, D, D), 3.0, dtype=torch.float32, device="cuda") if with_state_out else None
    o = G.gdn_prefill_varlen(q, k, v, la, be, to_dev(cu), si, so, Hk=Hk, Hv=Hv, l2norm=l2,
                             token_serial=token_serial, workspace=workspace)
    torch.cuda.synchronize()
    return to_host(o).reshape(p["T"], Hv, D), (to_host(so) if with_state_out else None)


def check_states(sg, srf, lens, tol=None):
    for s in range(len(lens)):
        if lens[s] == 0:
            np.testing.assert_array_equal(sg[s], srf[s])   # handed through exactly
        else:
            e = assert_state(sg[s], srf[s])
            if tol is not None:
                assert e < tol, (s, e)


@pytest.mark.parametrize("state,l2", [(True, False), (False, True)])
def test_varlen_chunked_parity(state, l2):
    Hk, Hv, D = 2, 6, 128
    p, st, cu = packed_problem(5100 + int(l2), LENS, Hk, Hv, D, "bf16", state=state, normalise=not l2)
    og, sg = run_packed(p, st, cu, l2=l2)
    orf, srf = oracle_packed(p, st, cu, l2=l2)
    m = assert_out(og, orf, bf16=True)
    check_states(sg, srf, LENS)
    print(f"varlen chunked lens={LENS} state={state} l2={l2}: out {m}")


def test_varlen_equals_one_call_per_sequence():
    """Chunks never span sequences, so the packed call computes exactly what separate
    per-sequence calls compute: outputs and states are bit-identical."""
    torch = _torch()
    Hk, Hv, D = 1, 3, 128
    lens = [70, 0, 129, 5]
    p, st, cu = packed_problem(5200, lens, Hk, Hv, D, "bf16")
    og, sg = run_packed(p, st, cu)
    for s, L in enumerate(lens):
        a = int(cu[s])
        if L == 0:
            continue
        q, k, v = (to_dev(np.ascontiguousarray(p[x][:, a:a + L])) for x in ("q", "k", "v"))
        la = to_dev(np.ascontiguousarray(p["log_alpha"][:, a:a + L]))
        be = to_dev(np.ascontiguousarray(p["beta"][:, a:a + L]))
        so = torch.empty((1, Hv, D, D), dtype=torch.float32, device="cuda")
        o = G.gdn_prefill(q, k, v, la, be, to_dev(st[s:s + 1]), so, Hk=Hk, Hv=Hv)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host(o).reshape(L, Hv, D), og[a:a + L])
        np.testing.assert_array_equal(to_host(so)[0], sg[s])


@pytest.mark.parametrize("with_state_out", [True, False])
def test_varlen_small_workspace_windows(with_state_out):
    """Windows of one to three chunks cut through sequences; the state crosses a window
    boundary through state_out, or through the workspace's carry area without it."""
    torch = _torch()
    Hk, Hv, D = 1, 3, 128
    p, st, cu = packed_problem(5300, LENS, Hk, Hv, D, "bf16")
    orf, srf = oracle_packed(p, st, cu)
    dims = G.make_dims(len(LENS), p["T"], Hk, Hv, D, G.GDN_BF16)
    per_chunk = Hv * WS_VALUE_HEAD + Hk * WS_KEY_HEAD
    nchunks = (p["T"] + 63) // 64 + len(LENS)
    maps = -(-(len(LENS) + 1 + nchunks) * 4 // 256) * 256   # chunk maps at the workspace start
    assert G.gdn_prefill_varlen_workspace_size(dims) == maps + nchunks * per_chunk
    for nwin in (1, 2, 3):
        extra = maps + (0 if with_state_out else len(LENS) * Hv * D * D * 4)
        ws = torch.empty(nwin * per_chunk + extra, dtype=torch.uint8, device="cuda")
        og, sg = run_packed(p, st, cu, with_state_out=with_state_out, workspace=ws)
        assert_out(og, orf, bf16=True)
        if with_state_out:
            check_states(sg, srf, LENS)


@pytest.mark.parametrize("D,io", [(16, "f32"), (128, "bf16")])
def test_varlen_token_serial_parity(D, io):
    Hk, Hv = 1, 2
    lens = [5, 0, 1, 33, 17]
    p, st, cu = packed_problem(5400 + D, lens, Hk, Hv, D, io, recipe="tiny")
    og, sg = run_packed(p, st, cu, token_serial=(io == "bf16"))
    orf, srf = oracle_packed(p, st, cu)
    assert_out(og, orf, bf16=(io == "bf16"))
    check_states(sg, srf, lens, tol=1e-5)   # fp32 arithmetic throughout


def test_varlen_all_empty_and_no_sequences():
    torch = _torch()
    Hk, Hv, D = 1, 3, 128
    st = W.problem(5500, 3, 1, Hk, Hv, D, state="normal")["state_in"].astype(np.float32)
    cu = to_dev(np.zeros(4, dtype=np.int32))
    z = torch.empty((0, D), dtype=torch.bfloat16, device="cuda")
    zv = torch.empty((0, Hv * D), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0, Hv), dtype=torch.float32, device="cuda")
    so = torch.full((3, Hv, D, D), 7.0, dtype=torch.float32, device="cuda")
    G.gdn_prefill_varlen(z, z, zv, g, g, cu, to_dev(st), so, Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(so), st)
    G.gdn_prefill_varlen(z, z, zv, g, g, cu, None, so, Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(so).item() == 0
    G.gdn_prefill_varlen(z, z, zv, g, g, to_dev(np.zeros(1, dtype=np.int32)), None, None, Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()


def test_varlen_many_sequences():
    """1100 sequences (more than the map kernel's 1024 threads scan at once), many of
    them empty or one chunk long, one of 300 tokens, with windows of four chunks."""
    torch = _torch()
    Hk, Hv, D = 1, 1, 128
    rng = np.random.default_rng(5600)
    lens = rng.integers(0, 20, 1100)
    lens[rng.choice(1100, 150, replace=False)] = 0
    lens[500] = 300
    lens = [int(x) for x in lens]
    p, st, cu = packed_problem(5600, lens, Hk, Hv, D, "bf16")
    orf, srf = oracle_packed(p, st, cu)
    og, sg = run_packed(p, st, cu)
    assert_out(og, orf, bf16=True)
    check_states(sg, srf, lens)
    dims = G.make_dims(len(lens), p["T"], Hk, Hv, D, G.GDN_BF16)
    full = G.gdn_prefill_varlen_workspace_size(dims)
    nchunks = (p["T"] + 63) // 64 + len(lens)
    maps = -(-(len(lens) + 1 + nchunks) * 4 // 256) * 256
    # windows of 1024 chunks (two rounds of 512 prep workgroups, 71 MiB) balanced over 1245: two of 623,
    # plus a state carry per sequence
    assert nchunks == 1245
    assert full == maps + 623 * (WS_VALUE_HEAD + WS_KEY_HEAD) + len(lens) * D * D * 4
    ws = torch.empty(maps + 4 * (WS_VALUE_HEAD + WS_KEY_HEAD), dtype=torch.uint8, device="cuda")
    og2, sg2 = run_packed(p, st, cu, workspace=ws)
    np.testing.assert_array_equal(og2, og)   # windows do not change the arithmetic
    np.testing.assert_array_equal(sg2, sg)


def test_varlen_bench_workload_sampled():
    """The packed workload the bench times (32 requests of log-uniform lengths, 38,693 tokens,
    16/48 heads, D = 128, final states into a 32-entry pool), checked on sampled (request,
    value head) pairs that the oracle recomputes over the whole request (heads are
    independent, so a sampled head is exact).  The longest and the shortest requests are
    among them."""
    torch = _torch()
    lens = [int(x) for x in W.varlen_lengths()]
    Hk, Hv, D = 16, 48, 128
    p, st, cu = packed_problem(5700, lens, Hk, Hv, D, "bf16", state=False)
    q, k, v = (to_dev(p[x][0]) for x in ("q", "k", "v"))
    la, be = to_dev(p["log_alpha"][0]), to_dev(p["beta"][0])
    so = torch.empty((len(lens), Hv, D, D), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill_varlen(q, k, v, la, be, to_dev(cu), None, so, Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()
    og, sg = to_host(o).reshape(p["T"], Hv, D), to_host(so)
    longest, shortest = int(np.argmax(lens)), int(np.argmin(lens))
    for s, h in [(longest, 0), (longest, 47), (shortest, 5), (3, 17), (20, 30), (31, 44)]:
        a, b = int(cu[s]), int(cu[s + 1])
        sl = lambda x: np.ascontiguousarray(x[:, a:b])
        orf, srf = oracle.recurrence(sl(p["q"]), sl(p["k"]), sl(p["v"]), sl(p["log_alpha"]), sl(p["beta"]),
                                     Hk, Hv, None, sel=[h])
        assert_out(og[a:b, h], orf[0], bf16=True)
        assert_state(sg[s, h], srf[0])
