"""GPU parity of the full-attention entry points (include/gdn_attn.h) against the fp64
oracle (oracle/attention.py): prefill at sizes that span several 128-row query blocks and
64-key blocks with ragged tails, the caches it writes, decode against caches of different
lengths per sequence and several decode steps in a row, and sampled rows and sequences at
the layer's full size (24 query heads, 4 key/value heads, T = 4096; 64 sequences of 4096
cached positions).  All calls go through the C ABI.

Tolerance: outputs are bf16; per (token, query head) row, max |o - o_ref| <= 2e-2 RMS of the
reference row after a one-ulp bf16 allowance (helpers.assert_out_rows).  The reference keeps
the normalised, rotated q in fp64 and rounds k to bf16 (the cache holds two-byte keys).  The
kernel multiplies a bf16 q, so each element also gets the exact effect of rounding q once to
bf16 as an allowance: |o_ref(q rounded) - o_ref(q)|, both from the oracle.  Keys in the cache are compared to the oracle's rounded keys within one bf16 ulp
plus 2^-12 of the row's scale (both round once to bf16, the kernel from fp32 and the oracle
from fp64, so values near a rounding boundary may land one ulp apart); values are copied bit
for bit."""
import numpy as np
import pytest

from oracle import attention as A
from gated_deltanet_recurrence_rule_amd import binding as G
from gated_deltanet_recurrence_rule_amd import workloads as W
from helpers import assert_out_rows, to_dev, to_host, ulp_bf16

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def ref_prefill(*args, dense=False, **kw):
    """Oracle prefill with q in fp64 (the reference) and the allowance for one bf16 rounding of
    q: |o(q rounded) - o(q)|.  Returns (o, rotated keys, values, allowance); with ``dense`` the
    whole-matrix form, keys and values None."""
    if dense:
        o = A.prefill_dense(*args, **kw)
        return o, None, None, np.abs(A.prefill_dense(*args, q_bf16=True, **kw) - o)
    o, kr, vr = A.prefill(*args, **kw)
    oq, _, _ = A.prefill(*args, q_bf16=True, **kw)
    return o, kr, vr, np.abs(oq - o)


def ref_decode(*args, **kw):
    """Oracle decode with q in fp64 and the allowance for one bf16 rounding of q."""
    o, knew = A.decode(*args, **kw)
    oq, _ = A.decode(*args, q_bf16=True, **kw)
    return o, knew, np.abs(oq - o)


def dev_problem(p):
    return {k: to_dev(p[k]) for k in ("qg", "k", "v", "q_norm_w", "k_norm_w")}


def run_prefill(p, S_max):
    torch = _torch()
    d = dev_problem(p)
    kc, vc = G.attn_cache(p["B"], p["Hkv"], S_max)
    o = G.gdn_attn_prefill(d["qg"], d["k"], d["v"], d["q_norm_w"], d["k_norm_w"], kc, vc)
    torch.cuda.synchronize()
    return to_host(o), kc, vc


def cache_views(kc, vc, n):
    """Host copies of cached positions [0, n): keys [B, n, Hkv, D], values [B, n, Hkv, D]."""
    k = to_host(kc)[:, :, :n].transpose(0, 2, 1, 3)
    v = to_host(vc)                                    # [B, Hkv, S/64, D, 64]
    B, Hkv, nb, D, _ = v.shape
    v = v.transpose(0, 1, 2, 4, 3).reshape(B, Hkv, nb * 64, D)[:, :, :n].transpose(0, 2, 1, 3)
    return k, v


@pytest.mark.parametrize("B,T,Hq,Hkv", [(1, 1, 6, 1), (2, 64, 6, 1), (1, 129, 12, 2), (2, 200, 12, 2),
                                        (1, 300, 24, 4), (2, 300, 9, 3)])
def test_prefill_parity_and_caches(B, T, Hq, Hkv):
    p = W.attn_problem(700 + T, B, T, Hq, Hkv)
    S_max = ((T + 63) // 64) * 64 + 64
    og, kc, vc = run_prefill(p, S_max)
    orf, kr, vr, allow = ref_prefill(p["qg"], p["k"], p["v"], p["q_norm_w"], p["k_norm_w"])
    m = assert_out_rows(og.reshape(orf.shape), orf, allow=allow)
    kg, vg = cache_views(kc, vc, T)
    np.testing.assert_array_equal(vg, A.widen(p["v"]))                  # values copied exactly
    scale = np.abs(kr).max(axis=-1, keepdims=True)
    assert np.all(np.abs(kg - kr) <= ulp_bf16(kr) + 2.0 ** -12 * scale)
    print(f"attn prefill B={B} T={T} Hq={Hq} Hkv={Hkv}: {m}")


def test_prefill_full_size_every_row():
    """Every row of the full-size prefill (T = 4096, 24 query / 4 key-value heads) against the
    oracle's whole-matrix form of the same definition."""
    T = 4096
    p = W.attn_problem(710, 1, T, 24, 4)
    og, _, _ = run_prefill(p, T)
    orf, _, _, allow = ref_prefill(p["qg"], p["k"], p["v"], p["q_norm_w"], p["k_norm_w"], dense=True)
    m = assert_out_rows(og.reshape(orf.shape), orf, allow=allow)
    print(f"attn prefill T=4096, all rows: {m}")


def test_decode_against_caches_of_different_lengths():
    torch = _torch()
    B, T, Hq, Hkv = 3, 200, 12, 2
    S_max = 256
    p = W.attn_problem(720, B, T, Hq, Hkv)
    _, kc, vc = run_prefill(p, S_max)
    _, kr, vr = A.prefill(p["qg"], p["k"], p["v"], p["q_norm_w"], p["k_norm_w"])
    new = W.attn_problem(721, B, 1, Hq, Hkv)
    lens = np.array([5, 200, 130], dtype=np.int32)
    d = dev_problem(new)
    o = G.gdn_attn_decode(d["qg"][:, 0], d["k"][:, 0], d["v"][:, 0], d["q_norm_w"], d["k_norm_w"],
                          to_dev(lens), kc, vc)
    torch.cuda.synchronize()
    ow, kw, allow = ref_decode(new["qg"][:, 0], new["k"][:, 0], new["v"][:, 0], new["q_norm_w"],
                               new["k_norm_w"], kr, vr, lens)
    m = assert_out_rows(to_host(o), ow, allow=allow)
    kg, vg = cache_views(kc, vc, S_max)
    for b in range(B):
        n = lens[b]
        np.testing.assert_array_equal(vg[b, n], A.widen(new["v"][b, 0]))      # appended at cache_len
        assert np.all(np.abs(kg[b, n] - kw[b]) <= ulp_bf16(kw[b]) + 2.0 ** -12 * np.abs(kw[b]).max())
    print(f"attn decode lens={lens.tolist()}: {m}")


def test_decode_steps_continue_prefill():
    """Prefill 40 tokens, then decode tokens 40, 41, 42 one at a time (advancing cache_len):
    the outputs are the oracle's prefill rows 40..42 of the 43-token sequence."""
    torch = _torch()
    B, Hq, Hkv, T0, n = 2, 6, 1, 40, 3
    p = W.attn_problem(730, B, T0 + n, Hq, Hkv)
    head = {k: (v[:, :T0].copy() if k in ("qg", "k", "v") else v) for k, v in p.items()}
    head["T"] = T0
    _, kc, vc = run_prefill(head, 64)
    orf, _, _, allow = ref_prefill(p["qg"], p["k"], p["v"], p["q_norm_w"], p["k_norm_w"])
    d = dev_problem(p)
    lens = torch.full((B,), T0, dtype=torch.int32, device="cuda")
    for t in range(T0, T0 + n):
        o = G.gdn_attn_decode(d["qg"][:, t].contiguous(), d["k"][:, t].contiguous(), d["v"][:, t].contiguous(),
                              d["q_norm_w"], d["k_norm_w"], lens, kc, vc)
        lens += 1
        torch.cuda.synchronize()
        assert_out_rows(to_host(o), orf[:, t], allow=allow[:, t])


def test_decode_full_size_sampled_sequences():
    """64 sequences, caches of 4096 positions filled with the rotated keys and values of a
    random context (written straight into the documented cache layout), each sequence at its
    own length; 4 sequences are checked against the oracle."""
    torch = _torch()
    B, Hq, Hkv, D, S = 64, 24, 4, 256, 4096
    rng = np.random.default_rng(740)
    lens = rng.integers(1, S, B).astype(np.int32)
    lens[0], lens[1] = S - 1, 0
    kc = W.normal_tokens(740, "attn_cache", B * Hkv * S, D, post=W.f32_to_bf16, out_dtype=np.uint16)
    vc = W.normal_tokens(741, "attn_cache", B * Hkv * S, D, post=W.f32_to_bf16, out_dtype=np.uint16)
    kc = kc.reshape(B, Hkv, S, D)
    vc = vc.reshape(B, Hkv, S, D)
    vct = np.ascontiguousarray(vc.reshape(B, Hkv, S // 64, 64, D).transpose(0, 1, 2, 4, 3))
    kd, vd = to_dev(kc), to_dev(vct)
    new = W.attn_problem(742, B, 1, Hq, Hkv)
    d = dev_problem(new)
    o = G.gdn_attn_decode(d["qg"][:, 0], d["k"][:, 0], d["v"][:, 0], d["q_norm_w"], d["k_norm_w"],
                          to_dev(lens), kd, vd)
    torch.cuda.synchronize()
    og = to_host(o)
    assert np.isfinite(og).all()
    for b in (0, 1, 17, 63):
        ow, _, allow = ref_decode(new["qg"][b:b + 1, 0], new["k"][b:b + 1, 0], new["v"][b:b + 1, 0],
                                  new["q_norm_w"], new["k_norm_w"], kc[b:b + 1].transpose(0, 2, 1, 3),
                                  vc[b:b + 1].transpose(0, 2, 1, 3), lens[b:b + 1])
        assert_out_rows(og[b:b + 1], ow, allow=allow)


@pytest.mark.parametrize("B,T,Hq,Hkv,rot,S_max", [(2, 128, 4, 4, 64, 192), (1, 96, 8, 1, 0, 128),
                                                  (1, 70, 16, 2, 256, 128), (3, 256, 6, 3, 64, 320)])
def test_prefill_shapes_and_rotations(B, T, Hq, Hkv, rot, S_max):
    """One key/value head per query head, 8 query heads per group, no rotation, every
    dimension rotated, exact block multiples, and caches with spare room."""
    torch = _torch()
    p = W.attn_problem(760 + T + rot, B, T, Hq, Hkv)
    d = dev_problem(p)
    kc, vc = G.attn_cache(B, Hkv, S_max)
    o = G.gdn_attn_prefill(d["qg"], d["k"], d["v"], d["q_norm_w"], d["k_norm_w"], kc, vc, rot_dim=rot)
    torch.cuda.synchronize()
    orf, kr, _, allow = ref_prefill(p["qg"], p["k"], p["v"], p["q_norm_w"], p["k_norm_w"], rot_dim=rot)
    assert_out_rows(to_host(o), orf, allow=allow)
    kg, vg = cache_views(kc, vc, S_max)
    assert np.all(np.abs(kg[:, :T] - kr) <= ulp_bf16(kr) + 2.0 ** -12 * np.abs(kr).max(axis=-1, keepdims=True))
    np.testing.assert_array_equal(vg[:, :T], A.widen(p["v"]))
    tail = ((T + 63) // 64) * 64
    assert np.all(kg[:, T:tail] == 0) and np.all(vg[:, T:tail] == 0)   # the partial block's tail is zeroed


@pytest.mark.parametrize("G_,rot", [(16, 64), (8, 64), (1, 0)])
def test_decode_group_sizes(G_, rot):
    torch = _torch()
    B, Hkv, T0 = 2, 2, 100
    Hq = G_ * Hkv
    p = W.attn_problem(780 + G_, B, T0 + 1, Hq, Hkv)
    head = {k: (v[:, :T0].copy() if k in ("qg", "k", "v") else v) for k, v in p.items()}
    head["T"] = T0
    d0 = dev_problem(head)
    kc, vc = G.attn_cache(B, Hkv, 128)
    G.gdn_attn_prefill(d0["qg"], d0["k"], d0["v"], d0["q_norm_w"], d0["k_norm_w"], kc, vc, rot_dim=rot)
    d = dev_problem(p)
    lens = torch.full((B,), T0, dtype=torch.int32, device="cuda")
    o = G.gdn_attn_decode(d["qg"][:, T0].contiguous(), d["k"][:, T0].contiguous(), d["v"][:, T0].contiguous(),
                          d["q_norm_w"], d["k_norm_w"], lens, kc, vc, rot_dim=rot)
    torch.cuda.synchronize()
    orf, _, _, allow = ref_prefill(p["qg"], p["k"], p["v"], p["q_norm_w"], p["k_norm_w"], rot_dim=rot)
    assert_out_rows(to_host(o), orf[:, T0], allow=allow[:, T0])


def test_prefill_padded_strides():
    """qg, k, v and o as views with token strides 4 elements wider than their rows (8-byte but
    not 16-byte aligned rows, the weakest alignment the ABI accepts)."""
    torch = _torch()
    B, T, Hq, Hkv, D = 2, 100, 6, 1, 256
    p = W.attn_problem(790, B, T, Hq, Hkv)
    d = dev_problem(p)

    def padded(x, lead_shape, width):
        wide = torch.zeros(lead_shape + (width + 4,), dtype=torch.bfloat16, device="cuda")
        wide[..., :width] = x.reshape(lead_shape + (width,))
        return wide[..., :width]

    qg = padded(d["qg"], (B, T), 2 * Hq * D).view(B, T, Hq, 2, D)
    k = padded(d["k"], (B, T), Hkv * D).view(B, T, Hkv, D)
    v = padded(d["v"], (B, T), Hkv * D).view(B, T, Hkv, D)
    o = torch.zeros((B, T, Hq * D + 4), dtype=torch.bfloat16, device="cuda")[..., :Hq * D].view(B, T, Hq, D)
    kc, vc = G.attn_cache(B, Hkv, 128)
    G.gdn_attn_prefill(qg, k, v, d["q_norm_w"], d["k_norm_w"], kc, vc, o)
    torch.cuda.synchronize()
    orf, _, _, allow = ref_prefill(p["qg"], p["k"], p["v"], p["q_norm_w"], p["k_norm_w"])
    assert_out_rows(to_host(o), orf, allow=allow)
    _, vg = cache_views(kc, vc, T)
    np.testing.assert_array_equal(vg, A.widen(p["v"]))
