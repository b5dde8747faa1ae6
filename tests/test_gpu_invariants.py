"""Invariants of the gated delta rule driven through libgdn, checked against what the
mathematics fixes rather than against the oracle ("L'attention hybride", section "La
recurrence": with beta = 1 a write erases the line of its key and writes it anew).

With alpha = beta = 1, S_0 = 0 and orthonormal keys, the state after the writes recalls
each key's latest value exactly, S k_j = v_latest(j), and reading with q_t = k_t right
after the write returns v_t.  For bf16 inputs the keys are rows of a 16x16 Hadamard
matrix divided by 4, placed in the eight 16-dimension blocks of the 128-wide head: they
are exactly orthonormal as bf16 numbers.  The last 64 tokens write 64 of the 128 keys
again with new values.  Paths: the chunked prefill (bf16), the token-serial prefill
(fp32, random orthonormal keys), and 192 single-token decode steps (bf16)."""
import numpy as np
import pytest

from gated_deltanet_recurrence_rule_amd import binding as G
from gated_deltanet_recurrence_rule_amd import workloads as W
from helpers import STATE_TOL, assert_out, to_dev, to_host

pytestmark = pytest.mark.gpu

D, HV, T = 128, 3, 192


def hadamard_keys():
    h = np.array([[1.0]])
    while h.shape[0] < 16:
        h = np.block([[h, h], [h, -h]])
    keys = np.zeros((D, D))
    for blk in range(D // 16):
        keys[16 * blk:16 * blk + 16, 16 * blk:16 * blk + 16] = h / 4.0
    return keys                                    # rows: 128 orthonormal keys, entries 0 or +-1/4


def write_sequence(keys, seed):
    """Token order: all 128 keys once (shuffled), then 64 of them again; values per value head."""
    rng = np.random.default_rng(seed)
    order = np.concatenate([rng.permutation(D), rng.permutation(D)[:T - D]])
    k = keys[order]                                            # [T, D]
    v = rng.standard_normal((T, HV, D))
    return order, k, v


def expected(order, v):
    """The latest value written under each key, per value head: [HV, D keys, D]."""
    latest = np.zeros((HV, D, D))
    for t, j in enumerate(order):
        latest[:, j, :] = v[t]
    return latest


def check_state(M, keys, latest):
    # M = S^T per value head [HV, Dk, Dv]: S k_j = M^T k_j, i.e. rows of keys @ M
    for h in range(HV):
        rec = keys @ M[h]
        err = np.linalg.norm(rec - latest[h]) / np.linalg.norm(latest[h])
        assert err <= STATE_TOL, (h, err)


def gates():
    return (np.zeros((1, T, HV), np.float32), np.ones((1, T, HV), np.float32))


def test_orthonormal_recall_chunked_bf16():
    import torch
    keys = hadamard_keys()
    order, k, v = write_sequence(keys, 21)
    vb = W.f32_to_bf16(v.reshape(1, T, HV * D).astype(np.float32))
    kb = W.f32_to_bf16(k.reshape(1, T, D).astype(np.float32))
    assert np.array_equal(W.bf16_to_f32(kb).astype(np.float64).reshape(T, D), k)   # keys exact in bf16
    v = W.bf16_to_f32(vb).astype(np.float64).reshape(T, HV, D)
    la, be = gates()
    so = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill(to_dev(kb), to_dev(kb), to_dev(vb), to_dev(la), to_dev(be), None, so, Hk=1, Hv=HV)
    torch.cuda.synchronize()
    check_state(to_host(so)[0], keys, expected(order, v))
    assert_out(to_host(o).reshape(T, HV, D), v, bf16=True)          # o_t = S_t k_t = v_t


def test_orthonormal_recall_token_serial_f32():
    import torch
    rng = np.random.default_rng(22)
    keys, _ = np.linalg.qr(rng.standard_normal((D, D)))
    keys = keys.T.astype(np.float32).astype(np.float64)             # rows, as the kernel reads them
    order, k, v = write_sequence(keys, 23)
    v = v.astype(np.float32).astype(np.float64)
    la, be = gates()
    kd = to_dev(k.reshape(1, T, D).astype(np.float32))
    so = torch.empty((1, HV, D, D), dtype=torch.float32, device="cuda")
    o = G.gdn_prefill(kd, kd, to_dev(v.reshape(1, T, HV * D).astype(np.float32)), to_dev(la), to_dev(be),
                      None, so, Hk=1, Hv=HV)
    torch.cuda.synchronize()
    # fp32 keys are orthonormal to ~1e-7, so the recall holds to fp32 rounding
    M = to_host(so)[0]
    lat = expected(order, v)
    for h in range(HV):
        np.testing.assert_allclose(keys @ M[h], lat[h], atol=2e-5)
    np.testing.assert_allclose(to_host(o).reshape(T, HV, D), v, atol=2e-5)


def test_orthonormal_recall_decode_steps():
    import torch
    keys = hadamard_keys()
    order, k, v = write_sequence(keys, 24)
    vb = W.f32_to_bf16(v.reshape(T, HV * D).astype(np.float32))
    kb = W.f32_to_bf16(k.astype(np.float32))
    v = W.bf16_to_f32(vb).astype(np.float64).reshape(T, HV, D)
    st = torch.zeros((1, HV, D, D), dtype=torch.float32, device="cuda")
    la = torch.zeros((1, HV), dtype=torch.float32, device="cuda")
    be = torch.ones((1, HV), dtype=torch.float32, device="cuda")
    kd, vd = to_dev(kb), to_dev(vb)
    outs = []
    for t in range(T):
        o = G.gdn_decode_step(kd[t:t + 1], kd[t:t + 1], vd[t:t + 1], la, be, st, Hk=1, Hv=HV)
        outs.append(o)
    torch.cuda.synchronize()
    check_state(to_host(st)[0], keys, expected(order, v))
    og = np.stack([to_host(x)[0] for x in outs]).reshape(T, HV, D)
    assert_out(og, v, bf16=True)
