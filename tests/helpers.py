"""Shared test helpers: host <-> device conversion and the parity criteria.

Parity criteria (the oracle is fp64 and unrounded):
  * state: relative Frobenius error ||M_gpu - M_ref||_F / ||M_ref||_F <= 1e-3;
  * fp32 outputs: max |o_gpu - o_ref| <= 2e-2 * RMS(o_ref);
  * bf16 outputs: the same bound after a one-ulp allowance for the rounding
    that a bf16 output must undergo:
        max_i max(0, |o_gpu,i - o_ref,i| - ulp_bf16(o_ref,i)) <= 2e-2 * RMS(o_ref),
    with ulp_bf16(x) = 2^(floor(log2|x|) - 7).  Rounding the exact outputs to
    bf16 alone already costs up to ~8e-2 RMS on these heavy-tailed outputs,
    so the literal bound cannot hold for any bf16 result; the literal figure
    is reported next to that floor.
"""
from __future__ import annotations

import numpy as np

OUT_TOL = 2e-2
STATE_TOL = 1e-3

# Prefill workspace per chunk: per value head the -W, Kd and U0 fragments (16 KiB each), the P
# fragments (6 KiB) and 1 KiB of scalings; per key head the Q^ fragments (16 KiB).
WS_VALUE_HEAD = 56320
WS_KEY_HEAD = 16384


def to_dev(a: np.ndarray, device="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 values widened exactly)."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    m, e = np.frexp(np.abs(x))          # |x| = m 2^e, m in [0.5, 1): floor(log2|x|) = e - 1
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 8))


def round_bf16_f64(x: np.ndarray) -> np.ndarray:
    import oracle
    b = oracle.round_bf16(x)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def out_metrics(o_gpu: np.ndarray, o_ref: np.ndarray, bf16: bool) -> dict:
    rms = float(np.sqrt(np.mean(o_ref ** 2)))
    err = np.abs(o_gpu - o_ref)
    m = dict(rms=rms, max_err_rms=float(err.max() / rms), rms_err_rms=float(np.sqrt(np.mean(err ** 2)) / rms))
    if bf16:
        allow = ulp_bf16(o_ref)
        m["excess_rms"] = float(np.maximum(0.0, err - allow).max() / rms)
        m["floor_rms"] = float(np.abs(round_bf16_f64(o_ref) - o_ref).max() / rms)
        m["metric"] = m["excess_rms"]
    else:
        m["metric"] = m["max_err_rms"]
    return m


def assert_out(o_gpu, o_ref, bf16: bool, tol: float = OUT_TOL, what: str = "o"):
    m = out_metrics(np.asarray(o_gpu, np.float64), np.asarray(o_ref, np.float64), bf16)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite values"
    assert m["metric"] <= tol, f"{what}: {m}"
    return m


def assert_out_rows(o_gpu, o_ref, tol: float = OUT_TOL, what: str = "o", allow=None):
    """Attention outputs, bf16: per row r (the last axis, one query head of one token)
    max_i max(0, |o_gpu,ri - o_ref,ri| - ulp_bf16(o_ref,ri) - allow_ri) <= tol * RMS(o_ref,r),
    where ``allow`` (default 0) is an extra per-element allowance the caller derives.
    A row is a convex combination of the visible values, so its scale ranges from |v|
    (a row that sees one key) to about |v| / sqrt(n) (n keys of random direction); the
    kernel's own rounding (softmax weights to bf16 for the product, fp32 sums) errs in
    proportion to the row, so each row is held to its own RMS."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite values"
    rms = np.sqrt(np.mean(o_ref ** 2, axis=-1, keepdims=True))
    extra = 0.0 if allow is None else np.asarray(allow, np.float64)
    excess = np.maximum(0.0, np.abs(o_gpu - o_ref) - ulp_bf16(o_ref) - extra) / rms
    worst = np.unravel_index(np.argmax(excess), excess.shape)
    m = dict(max_excess_row_rms=float(excess.max()), worst=tuple(int(i) for i in worst),
             rms_err_row_rms=float(np.sqrt(np.mean((np.abs(o_gpu - o_ref) / rms) ** 2))))
    assert m["max_excess_row_rms"] <= tol, f"{what}: {m}"
    return m


def state_err(m_gpu, m_ref) -> float:
    m_gpu = np.asarray(m_gpu, np.float64)
    m_ref = np.asarray(m_ref, np.float64)
    return float(np.linalg.norm(m_gpu - m_ref) / np.linalg.norm(m_ref))


def assert_state(m_gpu, m_ref, tol: float = STATE_TOL, what: str = "state"):
    assert np.all(np.isfinite(m_gpu)), f"{what}: non-finite values"
    e = state_err(m_gpu, m_ref)
    assert e <= tol, f"{what}: relative Frobenius error {e:.3e} > {tol}"
    return e


def conv_abs_sum(x_bits_or_f32, w, cs, b, c0, c1):
    """S[t, c] = sum_j |w[c][j] x[b, t-3+j, c]| over the 4-tap causal window of
    channels [c0, c1): the scale of the fp32 accumulation error of one output
    (the error of a 4-term fp32 dot product is at most about 4 * 2^-24 * S)."""
    from gated_deltanet_recurrence_rule_amd.workloads import bf16_to_f32
    f = (lambda a: bf16_to_f32(a).astype(np.float64)) if x_bits_or_f32.dtype == np.uint16 else \
        (lambda a: np.asarray(a, np.float64))
    xs = f(x_bits_or_f32[b, :, c0:c1])
    T = xs.shape[0]
    pre = np.zeros((3, c1 - c0)) if cs is None else f(cs[b, c0:c1, :]).T
    xw = np.concatenate([pre, xs], axis=0)
    wf = np.abs(f(w[c0:c1]))
    return sum(np.abs(xw[j:j + T]) * wf[:, j] for j in range(4))


def conv_tol(yr, S):
    """One bf16 ulp of the exact value plus the fp32 accumulation bound 2^-21 * S."""
    return ulp_bf16(yr) + 2.0 ** -21 * S
