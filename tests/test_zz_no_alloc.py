"""gdn_prefill_static, the prefill that allocates nothing (its workspace is the
library's fixed 64 MiB device array), against gdn_prefill with a workspace of
its own, through the C ABI: two calls in a row, the second smaller than the
first, so that it runs on whatever the first left in the array.  The static
call runs more windows than gdn_prefill with its full workspace (the first
call: 64 chunks of 2.97 MB each, 22 per window against 32), and the results
are the same bits for any window size, so the check is bit equality; the
first call is also checked against the fp64 oracle on two heads.  A third
call runs the whole-head chain (heads that fill the GPU) over two windows."""
import numpy as np
import pytest

import oracle
from gated_deltanet_recurrence_rule_amd import binding as G
from gated_deltanet_recurrence_rule_amd import workloads as W
from helpers import assert_out, assert_state, to_dev, to_host

pytestmark = pytest.mark.gpu


def _both(p, with_state_out):
    import torch
    B, T, Hk, Hv, D = p["B"], p["T"], p["Hk"], p["Hv"], p["D"]
    q, k, v = to_dev(p["q"]), to_dev(p["k"]), to_dev(p["v"])
    la, be = to_dev(p["log_alpha"]), to_dev(p["beta"])
    si = to_dev(p["state_in"].astype(np.float32)) if p["state_in"] is not None else None
    mk = lambda: torch.empty((B, Hv, D, D), dtype=torch.float32, device="cuda") if with_state_out else None
    so_ref, so = mk(), mk()
    o_ref = G.gdn_prefill(q, k, v, la, be, si, so_ref, Hk=Hk, Hv=Hv)
    o = torch.full_like(o_ref, 7)
    G.gdn_prefill_static(q, k, v, la, be, si, so, o, Hk=Hk, Hv=Hv)
    torch.cuda.synchronize()
    og, oref = to_host(o), to_host(o_ref)
    np.testing.assert_array_equal(og, oref)
    if with_state_out:
        np.testing.assert_array_equal(to_host(so), to_host(so_ref))
    return og.reshape(B, T, Hv, D), (to_host(so) if with_state_out else None)


def test_prefill_static_two_calls():
    # 1: the headline layer shape (B=1, T=4096, 16 key / 48 value heads) with an entry state
    p = W.problem(9100, 1, 4096, 16, 48, 128, io="bf16", recipe="qwen", state="normal")
    og, sg = _both(p, True)
    heads = [0, 47]
    orf, srf = oracle.recurrence(p["q"], p["k"], p["v"], p["log_alpha"], p["beta"], 16, 48,
                                 p["state_in"].astype(np.float32), sel=heads)
    assert_out(og[:, :, heads], orf[None].transpose(0, 2, 1, 3), bf16=True)
    assert_state(sg[0, heads], srf)
    # 2: smaller, no state_out (the state crosses windows through the carry inside the array)
    p2 = W.problem(9101, 2, 300, 1, 3, 128, io="bf16", recipe="tiny", state="normal")
    _both(p2, False)
    p2["state_in"] = None
    _both(p2, True)
    # 3: heads that fill the GPU (2 x 128): whole-head chains, K^ once per key head; 14.8 MB of
    # operands a chunk, so the array holds windows of 4 of the 5 chunks
    p3 = W.problem(9102, 2, 300, 16, 128, 128, io="bf16", recipe="qwen", state="normal")
    _both(p3, True)
