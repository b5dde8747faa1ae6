"""fp64 oracle for the hybrid's full-attention layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it; the HIP library never does, and this module imports
nothing from it.

What it computes follows "L'attention hybride" (the Qwen3.8-27B architecture
chapter), section "Les 16 couches d'attention complete": its configuration
block, its parameter table ("Le decompte"), "Le facteur 2 sur W_Q", "GQA a 6:1"
and "Le RoPE partiel"; RMSNorm as in "Les briques d'un reseau de neurones", 4:

* the query projection yields, per query head, the query and an output gate
  (the factor 2 on W_Q); the input ``qg`` is laid out [B, T, Hq, 2, D] with the
  query first (reading A1);
* q and k are RMS-normalised per head over their D = 256 values with a learned
  weight of D entries each (the "normalisations q, k" row of the parameter
  count, 2 x 256); y = x / sqrt(mean(x^2) + eps) * w (reading A2);
* RoPE turns only the first rot_dim = 64 of the 256 dimensions (partial factor
  0.25), base theta = 1e7; dimension pairs (j, j + rot_dim/2) with frequency
  theta^(-2j/rot_dim), the rotate-half convention (reading A3); text positions
  0, 1, 2, ... make the multimodal RoPE variant the plain one (reading A4);
* grouped-query attention: 24 query heads, 4 key/value heads, query head h
  reads key/value head h // 6; causal softmax(q k^T * scale) v with scale
  1/sqrt(D) (reading A5);
* the output of each query head is multiplied by sigmoid(gate) (reading A1);
* k enters the attention products as a bf16 value, rounded once to
  nearest-even after norm and RoPE, because the key cache holds it that way:
  the page's "GQA a 6:1" counts 4,096 bytes of cache per token and layer
  (4 key/value heads x 256 x 2 x 2 bytes), i.e. two-byte keys (reading A6).
  q is not cached and stays fp64 here (``q_bf16=True`` rounds it too, as a
  kernel that multiplies bf16 operands does); ``k_bf16=False`` keeps k fp64.

Inputs may be float64, float32, or uint16 holding bf16 bit patterns (widened
exactly).
"""
from __future__ import annotations

import numpy as np


def widen(x) -> np.ndarray:
    """float64 copy; uint16 arrays are bf16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def rms_norm(x, w, eps):
    """y = x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = widen(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * widen(w)


def rope(x, pos, rot_dim=64, theta=1e7):
    """Rotary embedding of the first rot_dim dimensions of x [..., T, H, D] at
    positions pos [T] (or [..., T]): pair (j, j + rot_dim/2) is turned by the angle
    pos * theta^(-2j/rot_dim); dimensions from rot_dim on are left as they are."""
    x = widen(x)
    half = rot_dim // 2
    inv = theta ** (-2.0 * np.arange(half) / rot_dim)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv          # [..., T, half]
    c, s = np.cos(ang)[..., None, :], np.sin(ang)[..., None, :]       # broadcast over heads
    y = x.copy()
    a, b = x[..., :half], x[..., half:rot_dim]
    y[..., :half] = a * c - b * s
    y[..., half:rot_dim] = b * c + a * s
    return y


def to_bf16(x):
    """x rounded once to the nearest bf16 value (ties to even), as float64."""
    from oracle import round_bf16
    return widen(round_bf16(x))


def prepare(qg, k, v, q_norm_w, k_norm_w, pos, *, rot_dim=64, theta=1e7, eps=1e-6, q_bf16=False, k_bf16=True):
    """Per-head norm and RoPE of q and k.  qg [B, T, Hq, 2, D]; k, v [B, T, Hkv, D];
    pos [B, T] or [T].  Returns (q, gate, k, v) as float64 with q and k rotated (each
    rounded to bf16 values when its flag is set)."""
    qg = widen(qg)
    q, gate = qg[..., 0, :], qg[..., 1, :]
    q = rope(rms_norm(q, q_norm_w, eps), pos, rot_dim, theta)
    kr = rope(rms_norm(k, k_norm_w, eps), pos, rot_dim, theta)
    if q_bf16:
        q = to_bf16(q)
    if k_bf16:
        kr = to_bf16(kr)
    return q, gate, kr, widen(v)


def attend(q, gate, k, v, n_keys, scale):
    """One query row per head against keys [0, n_keys): q, gate [Hq, D];
    k, v [S, Hkv, D].  Returns the gated output [Hq, D]."""
    Hq, Hkv = q.shape[0], k.shape[1]
    G = Hq // Hkv
    out = np.empty_like(q)
    for h in range(Hq):
        kk, vv = k[:n_keys, h // G], v[:n_keys, h // G]
        s = kk @ q[h] * scale
        p = np.exp(s - s.max())
        out[h] = (p @ vv) / p.sum()
    return out / (1.0 + np.exp(-gate))


def prefill(qg, k, v, q_norm_w, k_norm_w, *, rot_dim=64, theta=1e7, eps=1e-6, scale=None, rows=None,
            q_bf16=False, k_bf16=True):
    """Causal prefill of B sequences of T tokens from position 0.  Returns
    (o [B, T, Hq, D] (only ``rows``, a list of (b, t), when given: [n, Hq, D]),
    k_cache [B, T, Hkv, D] rotated keys, v [B, T, Hkv, D])."""
    qg = widen(qg)
    B, T, Hq, _, D = qg.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    q, gate, kr, vv = prepare(qg, k, v, q_norm_w, k_norm_w, np.arange(T), rot_dim=rot_dim, theta=theta, eps=eps,
                              q_bf16=q_bf16, k_bf16=k_bf16)
    if rows is not None:
        return np.stack([attend(q[b, t], gate[b, t], kr[b], vv[b], t + 1, scale) for b, t in rows]), kr, vv
    o = np.empty((B, T, Hq, D))
    for b in range(B):
        for t in range(T):
            o[b, t] = attend(q[b, t], gate[b, t], kr[b], vv[b], t + 1, scale)
    return o, kr, vv


def prefill_dense(qg, k, v, q_norm_w, k_norm_w, *, rot_dim=64, theta=1e7, eps=1e-6, scale=None, q_bf16=False,
                  k_bf16=True):
    """The causal prefill of ``prefill`` for every row at once: per sequence and query head,
    softmax(q k^T * scale) with the future masked, times v, times sigmoid(gate), written as
    whole matrices.  Returns o [B, T, Hq, D]."""
    qg = widen(qg)
    B, T, Hq, _, D = qg.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    q, gate, kr, vv = prepare(qg, k, v, q_norm_w, k_norm_w, np.arange(T), rot_dim=rot_dim, theta=theta, eps=eps,
                              q_bf16=q_bf16, k_bf16=k_bf16)
    Hkv = kr.shape[2]
    G = Hq // Hkv
    future = np.triu(np.ones((T, T), dtype=bool), 1)
    o = np.empty((B, T, Hq, D))
    for b in range(B):
        for h in range(Hq):
            s = (q[b, :, h] @ kr[b, :, h // G].T) * scale
            s[future] = -np.inf
            p = np.exp(s - s.max(axis=1, keepdims=True))
            o[b, :, h] = (p @ vv[b, :, h // G]) / p.sum(axis=1, keepdims=True)
    return o / (1.0 + np.exp(-gate))


def decode(qg, k, v, q_norm_w, k_norm_w, k_cache, v_cache, lens, *, rot_dim=64, theta=1e7, eps=1e-6, scale=None,
           q_bf16=False, k_bf16=True):
    """One new token per sequence at position lens[b]: qg [B, Hq, 2, D]; k, v
    [B, Hkv, D]; k_cache, v_cache [B, S, Hkv, D] (rotated keys, values) holding
    lens[b] tokens.  Returns (o [B, Hq, D], new rotated key [B, Hkv, D])."""
    qg = widen(qg)
    B, Hq, _, D = qg.shape
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    kc, vc = widen(k_cache), widen(v_cache)
    o = np.empty((B, Hq, D))
    knew = np.empty((B, widen(k).shape[1], D))
    for b in range(B):
        n = int(lens[b])
        q, gate, kr, vv = prepare(qg[b][None, None], widen(k)[b][None, None], widen(v)[b][None, None],
                                  q_norm_w, k_norm_w, np.array([n]), rot_dim=rot_dim, theta=theta, eps=eps,
                                  q_bf16=q_bf16, k_bf16=k_bf16)
        keys = np.concatenate([kc[b, :n], kr[0]], axis=0)
        vals = np.concatenate([vc[b, :n], vv[0]], axis=0)
        o[b] = attend(q[0, 0], gate[0, 0], keys, vals, n + 1, scale)
        knew[b] = kr[0, 0]
    return o, knew


def kv_cache_bytes_per_token(Hkv, D, elem_bytes=2):
    """Bytes one token adds to a layer's key/value cache."""
    return 2 * Hkv * D * elem_bytes
