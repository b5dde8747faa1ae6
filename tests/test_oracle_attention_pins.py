"""Pins of the full-attention oracle (oracle/attention.py) to facts fixed by the
pages and by the mathematics, independent of the oracle's own code: a hand-worked
two-key case, RoPE's closed form on basis vectors and its relative-position
property, RMSNorm's invariants, causality, the GQA grouping, the gate's limits,
the decode/prefill agreement, and the cache size the pages print."""
import numpy as np
import pytest

from oracle import attention as A


def test_two_key_case_by_hand():
    # D = 4, no rotation, unit norm weights, eps = 0.  q = k0 = e0, k1 = e1: RMSNorm scales each by
    # 1/sqrt(1/4) = 2, so the scores are (2e0).(2e0) = 4 and 0, times 1/sqrt(4): (2, 0).  Gate 0 halves.
    D = 4
    e = np.eye(D)
    qg = np.zeros((1, 2, 1, 2, D))
    qg[0, 1, 0, 0] = e[0]
    qg[0, 0, 0, 0] = e[2]   # row 0 sees only key 0, whatever its query
    k = np.stack([e[0], e[1]])[None, :, None, :]
    v = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.5, 0.0, 2.0]])[None, :, None, :]
    o, _, _ = A.prefill(qg, k, v, np.ones(D), np.ones(D), rot_dim=0, eps=0.0)
    p0 = np.exp(2.0) / (np.exp(2.0) + 1.0)
    expect = 0.5 * (p0 * v[0, 0, 0] + (1 - p0) * v[0, 1, 0])
    np.testing.assert_allclose(o[0, 1, 0], expect, rtol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], 0.5 * v[0, 0, 0], rtol=1e-14)   # one visible key


@pytest.mark.parametrize("j", [0, 5, 31])
def test_rope_closed_form_on_basis_vectors(j):
    # dims j and j + 32 of the 64 rotated ones turn by pos * theta^(-2j/64); dims >= 64 stay put
    D, pos, theta = 256, 1234.0, 1e7
    ang = pos * theta ** (-2.0 * j / 64)
    x = np.zeros((1, 1, D))
    x[0, 0, j] = 1.0
    y = A.rope(x, np.array([pos]), 64, theta)[0, 0]
    expect = np.zeros(D)
    expect[j], expect[j + 32] = np.cos(ang), np.sin(ang)
    np.testing.assert_allclose(y, expect, atol=1e-15)
    x = np.zeros((1, 1, D))
    x[0, 0, j + 32] = 1.0
    y = A.rope(x, np.array([pos]), 64, theta)[0, 0]
    expect = np.zeros(D)
    expect[j], expect[j + 32] = -np.sin(ang), np.cos(ang)
    np.testing.assert_allclose(y, expect, atol=1e-15)
    x = np.random.default_rng(j).standard_normal((1, 1, D))
    y = A.rope(x, np.array([pos]), 64, theta)
    np.testing.assert_array_equal(y[..., 64:], x[..., 64:])
    np.testing.assert_array_equal(A.rope(x, np.array([0.0]), 64, theta), x)     # position 0: identity
    np.testing.assert_allclose(np.linalg.norm(y), np.linalg.norm(x), rtol=1e-14)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((1, 1, 256)), rng.standard_normal((1, 1, 256))
    s = lambda m, n: float(np.sum(A.rope(q, np.array([m]))[0, 0] * A.rope(k, np.array([n]))[0, 0]))
    for m, n, shift in [(10, 3, 1000), (0, 0, 77777), (5000, 4999, 123456)]:
        assert abs(s(m, n) - s(m + shift, n + shift)) < 1e-9 * abs(s(m, n)) + 1e-9
    assert abs(s(10, 3) - s(10, 4)) > 1e-6        # ... and do depend on it


def test_rms_norm_invariants():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((3, 256))
    y = A.rms_norm(x, np.ones(256), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)
    np.testing.assert_allclose(A.rms_norm(7.5 * x, np.ones(256), 0.0), y, rtol=1e-13)
    w = rng.standard_normal(256)
    np.testing.assert_allclose(A.rms_norm(x, w, 0.0), y * w, rtol=1e-13)


def problem(seed, B, T, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, T, Hq, 2, D)), rng.standard_normal((B, T, Hkv, D)),
            rng.standard_normal((B, T, Hkv, D)), 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D))


def test_causality_and_gate_limits():
    qg, k, v, wq, wk = problem(3, 1, 9, 6, 1, 32)
    o, _, _ = A.prefill(qg, k, v, wq, wk, rot_dim=8)
    qg2, k2, v2 = qg.copy(), k.copy(), v.copy()
    qg2[:, 5:] += 3.0
    k2[:, 5:] *= -2.0
    v2[:, 5:] += 1.0
    o2, _, _ = A.prefill(qg2, k2, v2, wq, wk, rot_dim=8)
    np.testing.assert_array_equal(o2[:, :5], o[:, :5])          # later tokens do not reach earlier rows
    assert np.abs(o2[:, 5:] - o[:, 5:]).max() > 1e-3
    # gate -> +inf passes the attention output, -inf closes it, and in between it scales each value
    open_ = qg.copy()
    open_[..., 1, :] = 60.0
    o3, _, _ = A.prefill(open_, k, v, wq, wk, rot_dim=8)
    shut = qg.copy()
    shut[..., 1, :] = -60.0
    o4, _, _ = A.prefill(shut, k, v, wq, wk, rot_dim=8)
    assert np.abs(o4).max() < 1e-20
    np.testing.assert_allclose(o, o3 / (1 + np.exp(-qg[..., 1, :])), rtol=1e-12)
    # identical keys, no rotation: every visible key weighs the same, so row t is the mean of v[0..t]
    k5 = np.repeat(k[:, :1], 9, axis=1)
    o5, _, _ = A.prefill(open_, k5, v, wq, wk, rot_dim=0)
    means = np.cumsum(v[0, :, 0], axis=0) / np.arange(1, 10)[:, None]
    for h in range(6):
        np.testing.assert_allclose(o5[0, :, h], means, rtol=1e-12, atol=1e-12)


def test_gqa_grouping():
    # 12 query heads on 2 key/value heads: heads 0-5 read group 0, heads 6-11 group 1.  Equal queries
    # give equal outputs inside a group and different ones across groups.
    qg, k, v, wq, wk = problem(4, 1, 6, 12, 2, 32)
    qg[:, :, :, :, :] = qg[:, :, :1, :, :]
    o, _, _ = A.prefill(qg, k, v, wq, wk, rot_dim=8)
    for h in range(1, 6):
        np.testing.assert_array_equal(o[0, :, h], o[0, :, 0])
        np.testing.assert_array_equal(o[0, :, 6 + h], o[0, :, 6])
    assert np.abs(o[0, 1:, 0] - o[0, 1:, 6]).max() > 1e-3


def test_peaked_attention_reads_one_value():
    # a query equal to the key at its own position, both with a large norm weight, puts nearly all
    # the weight on that key (the others are independent random directions)
    qg, k, v, _, _ = problem(5, 1, 8, 6, 1, 256)
    t = 6
    qg[0, t, :, 0] = k[0, t, 0]
    qg[0, t, :, 1] = 60.0
    w = np.full(256, 4.0)
    o, _, _ = A.prefill(qg, k, v, w, w, rot_dim=64)
    np.testing.assert_allclose(o[0, t, 0], v[0, t, 0], rtol=1e-8, atol=1e-8)


def test_decode_continues_prefill():
    qg, k, v, wq, wk = problem(6, 2, 7, 6, 1, 64)
    o, kr, vv = A.prefill(qg, k, v, wq, wk, rot_dim=16)
    for n in (0, 3, 6):
        od, knew = A.decode(qg[:, n], k[:, n], v[:, n], wq, wk, kr[:, :n], vv[:, :n], [n, n], rot_dim=16)
        np.testing.assert_allclose(od, o[:, n], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(knew, kr[:, n], rtol=1e-12, atol=1e-12)
    rows, _, _ = A.prefill(qg, k, v, wq, wk, rot_dim=16, rows=[(1, 4), (0, 0)])
    np.testing.assert_array_equal(rows[0], o[1, 4])
    np.testing.assert_array_equal(rows[1], o[0, 0])


def test_kv_cache_size_the_pages_print():
    # "GQA a 6:1": 4 key/value heads of 256 per token and layer; the page prints 24,576 bytes for the
    # 24-head (no GQA) case and says that is six times more
    assert A.kv_cache_bytes_per_token(24, 256) == 24576
    assert A.kv_cache_bytes_per_token(4, 256) * 6 == 24576


def test_bf16_operands():
    # with q_bf16 / k_bf16 the rotated q and k are bf16 values within half an ulp of the fp64 ones;
    # by default only k is rounded (the cache holds two-byte keys) and q stays fp64; the cache keys
    # returned are the rounded keys
    qg, k, v, wq, wk = problem(7, 1, 5, 6, 1, 256)
    q64, _, k64, _ = A.prepare(qg, k, v, wq, wk, np.arange(5), q_bf16=False, k_bf16=False)
    q16, _, k16, _ = A.prepare(qg, k, v, wq, wk, np.arange(5), q_bf16=True, k_bf16=True)
    for x64, x16 in ((q64, q16), (k64, k16)):
        f32 = x16.astype(np.float32)
        assert np.array_equal(f32.astype(np.float64), x16)
        assert np.all((f32.view(np.uint32) & 0xFFFF) == 0)               # bf16-representable
        m, e = np.frexp(np.abs(x64))
        assert np.all(np.abs(x16 - x64) <= np.ldexp(1.0, e - 9))          # half an ulp (8 significant bits)
    qd, _, kd, _ = A.prepare(qg, k, v, wq, wk, np.arange(5))
    np.testing.assert_array_equal(qd, q64)
    np.testing.assert_array_equal(kd, k16)
    _, kr, _ = A.prefill(qg, k, v, wq, wk)
    np.testing.assert_array_equal(kr, k16)


def test_dense_prefill_is_the_row_by_row_definition():
    # the whole-matrix form used for full-size checks equals the row-by-row softmax definition
    qg, k, v, wq, wk = problem(8, 2, 37, 12, 2, 256)
    o_rows, _, _ = A.prefill(qg, k, v, wq, wk, rot_dim=64)
    o_dense = A.prefill_dense(qg, k, v, wq, wk, rot_dim=64)
    np.testing.assert_allclose(o_dense, o_rows, rtol=1e-12, atol=1e-12)
