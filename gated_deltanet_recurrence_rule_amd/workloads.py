"""Seeded synthetic inputs for the Gated DeltaNet mixer.

This module is the one place shared by the GPU side (tests, bench) and the
oracle side (tests, cpu baseline): it draws input tensors and holds none of
the method's arithmetic (no recurrence, conv, norm or gating of the mixer).
Everything it produces is input data: Gaussian draws, the per-head L2
normalisation that the input recipe applies before the bf16 cast, the gate
recipes, and the bf16 round-to-nearest-even used to store inputs.

Streams: every tensor is drawn from its own numpy PCG64 stream keyed by
(seed, tag, slab), in slabs of 4096 tokens, so any token range of any tensor
can be regenerated on its own and slabs can be drawn on several threads.
bf16 tensors are returned as uint16 bit patterns; their exact values are
``bf16_to_f32(bits)``.

Shapes follow the layer described on the page "L'attention hybride"
(Qwen3.8-27B architecture chapter), config block "Les 48 couches Gated
DeltaNet" and table "Le decompte": 16 key heads and 48 value heads of width
128, conv kernel 4 over the q|k|v channels, one 128-weight output norm; and
the larger variant of section "La dissymetrie 16 / 48" (16 key heads for
128 value heads).  The full-attention inputs follow section "Les 16 couches
d'attention complete" of the same page: 24 query heads (each with its gate)
and 4 key/value heads of width 256.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SLAB = 4096
_TAGS = {
    "q": 1, "k": 2, "v": 3, "beta": 4, "alpha": 5, "A": 6, "dt_bias": 7, "state": 8,
    "conv_w": 9, "norm_w": 10, "z": 11, "x": 12, "conv_state": 13, "step": 14,
    "attn_qg": 15, "attn_k": 16, "attn_v": 17, "attn_qw": 18, "attn_kw": 19, "attn_cache": 20,
}


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, tag: str, slab: int = 0, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TAGS[tag], slab, sub])))


def normal_tokens(seed: int, tag: str, n_tok: int, width: int, loc: float = 0.0,
                  scale: float = 1.0, sub: int = 0, tok0: int = 0, tok1: int | None = None,
                  post=None, out_dtype=np.float32) -> np.ndarray:
    """[tok1-tok0, width] slice of an N(loc, scale^2) float32 stream laid out
    as n_tok rows, drawn slab by slab (rows [tok0, tok1)).  ``post`` maps each
    float32 slab block to the stored values (e.g. normalise + round to bf16),
    stored as ``out_dtype``."""
    tok1 = n_tok if tok1 is None else tok1
    out = np.empty((tok1 - tok0, width), out_dtype)
    s_first, s_last = tok0 // SLAB, (max(tok1, 1) - 1) // SLAB

    def one(s):
        a0, a1 = s * SLAB, min((s + 1) * SLAB, n_tok)
        blk = _rng(seed, tag, s, sub).standard_normal((a1 - a0, width), dtype=np.float32)
        if scale != 1.0:
            blk *= np.float32(scale)
        if loc != 0.0:
            blk += np.float32(loc)
        lo, hi = max(a0, tok0), min(a1, tok1)
        part = blk[lo - a0:hi - a0]
        out[lo - tok0:hi - tok0] = part if post is None else post(part)

    if tok1 > tok0:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(s_first, s_last + 1)))
    return out


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def l2_rows(a: np.ndarray, heads: int) -> np.ndarray:
    """Input recipe step: divide each head's D-vector by its L2 norm (float32)."""
    sh = a.shape
    h = a.reshape(sh[:-1] + (heads, sh[-1] // heads))
    n = np.sqrt(np.einsum("...i,...i->...", h, h, dtype=np.float64))[..., None].astype(np.float32)
    return (h / n).reshape(sh)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def gates(seed: int, B: int, T: int, Hv: int, recipe: str, sub: int = 0):
    """(log_alpha, beta) float32 [B, T, Hv].

    recipe "tiny": beta = sigmoid(N(0,1)), log alpha = -0.1 softplus(N(0,1)).
    recipe "qwen": beta = sigmoid(N(0,1)), log alpha = -exp(A_h) softplus(N(0,1) + dt_bias_h),
                   A_h ~ U(0, ln 16), dt_bias_h ~ N(0, 0.5) per value head.
    """
    nb = normal_tokens(seed, "beta", B * T, Hv, sub=sub).astype(np.float64)
    na = normal_tokens(seed, "alpha", B * T, Hv, sub=sub).astype(np.float64)
    beta = _sigmoid(nb)
    if recipe == "tiny":
        la = -0.1 * _softplus(na)
    elif recipe == "qwen":
        hr = _rng(seed, "A")
        A = hr.uniform(0.0, np.log(16.0), size=Hv)
        dt = _rng(seed, "dt_bias").normal(0.0, 0.5, size=Hv)
        la = -np.exp(A)[None, :] * _softplus(na + dt[None, :])
    else:
        raise ValueError(recipe)
    return (la.astype(np.float32).reshape(B, T, Hv), beta.astype(np.float32).reshape(B, T, Hv))


def qkv(seed: int, B: int, T: int, Hk: int, Hv: int, D: int, io: str = "bf16", sub: int = 0,
        normalise: bool = True):
    """q, k [B, T, Hk*D] (L2-normalised per head when ``normalise``), v [B, T, Hv*D] ~ N(0,1).
    io "bf16" -> uint16 bits; "f32" -> float32."""
    cast = f32_to_bf16 if io == "bf16" else (lambda a: a)
    odt = np.uint16 if io == "bf16" else np.float32
    qk_post = (lambda a: cast(l2_rows(a, Hk))) if normalise else cast
    q = normal_tokens(seed, "q", B * T, Hk * D, sub=sub, post=qk_post, out_dtype=odt)
    k = normal_tokens(seed, "k", B * T, Hk * D, sub=sub, post=qk_post, out_dtype=odt)
    v = normal_tokens(seed, "v", B * T, Hv * D, sub=sub, post=cast, out_dtype=odt)
    return q.reshape(B, T, Hk * D), k.reshape(B, T, Hk * D), v.reshape(B, T, Hv * D)


def problem(seed: int, B: int, T: int, Hk: int, Hv: int, D: int, io: str = "bf16",
            recipe: str = "qwen", state: str | None = None, state_scale: float = 0.02,
            normalise: bool = True) -> dict:
    """One prefill problem: q, k, v, log_alpha, beta and an optional fp32 state_in."""
    q, k, v = qkv(seed, B, T, Hk, Hv, D, io, normalise=normalise)
    la, be = gates(seed, B, T, Hv, recipe)
    p = dict(B=B, T=T, Hk=Hk, Hv=Hv, D=D, io=io, q=q, k=k, v=v, log_alpha=la, beta=be,
             state_in=None)
    if state == "normal":
        p["state_in"] = normal_tokens(seed, "state", B * Hv * D, D, scale=state_scale).reshape(B, Hv, D, D)
    return p


# The five workload configurations -----------------------------------------

def cfg_tiny() -> dict:
    """Batch 1, T=64, 1 key / 1 value head, D=16, all fp32, tiny gate recipe, zero state."""
    return problem(1, 1, 64, 1, 1, 16, io="f32", recipe="tiny")


def cfg_prefill4k(T: int = 4096) -> dict:
    """Batch 1, T=4096, 16 key / 48 value heads, D=128, bf16 q/k/v, qwen gate recipe."""
    return problem(2, 1, T, 16, 48, 128, io="bf16", recipe="qwen")


def decode_pool(B: int = 64, Hv: int = 48, D: int = 128, seed: int = 3) -> np.ndarray:
    """fp32 state pool [B, Hv, D, D] ~ N(0, 0.02^2)."""
    return normal_tokens(seed, "state", B * Hv * D, D, scale=0.02).reshape(B, Hv, D, D)


def decode_step_inputs(step: int, B: int = 64, Hk: int = 16, Hv: int = 48, D: int = 128,
                       recipe: str = "qwen", seed: int = 3) -> dict:
    """Single-token inputs of decode step ``step`` (own streams per step)."""
    q, k, v = qkv(seed, B, 1, Hk, Hv, D, "bf16", sub=step + 1)
    la, be = gates(seed, B, 1, Hv, recipe, sub=step + 1)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=be)


def cfg_long(T: int = 262144, recipe: str = "qwen") -> dict:
    return problem(4, 1, T, 16, 48, 128, io="bf16", recipe=recipe)


def block_inputs(B: int = 4, T: int = 32768, Hk: int = 16, Hv: int = 128, D: int = 128,
                 seed: int = 5, recipe: str = "qwen", tok0: int = 0, tok1: int | None = None) -> dict:
    """Full-block front end inputs: pre-conv channels x = [q|k|v] [B, T, (2Hk+Hv)D] bf16 ~ N(0,1),
    conv weights [C, 4] ~ N(0, 0.5^2) bf16, gates (qwen recipe), norm weight [D] ~ N(1, 0.1^2)
    bf16, gate input z [B, T, Hv*D] bf16 ~ N(0,1).  ``tok0/tok1`` restrict x and z to a
    token range of the flattened B*T rows (for sampled checks)."""
    C = (2 * Hk + Hv) * D
    n = B * T
    t1 = n if tok1 is None else tok1
    x = normal_tokens(seed, "x", n, C, tok0=tok0, tok1=t1, post=f32_to_bf16, out_dtype=np.uint16)
    z = normal_tokens(seed, "z", n, Hv * D, tok0=tok0, tok1=t1, post=f32_to_bf16, out_dtype=np.uint16)
    cw = f32_to_bf16(_rng(seed, "conv_w").normal(0.0, 0.5, size=(C, 4)).astype(np.float32))
    nw = f32_to_bf16(_rng(seed, "norm_w").normal(1.0, 0.1, size=(D,)).astype(np.float32))
    la, be = gates(seed, B, T, Hv, recipe)
    if tok1 is None and tok0 == 0:
        x = x.reshape(B, T, C)
        z = z.reshape(B, T, Hv * D)
    return dict(B=B, T=T, Hk=Hk, Hv=Hv, D=D, C=C, x=x, conv_w=cw, norm_w=nw, z=z,
                log_alpha=la, beta=be)


def attn_problem(seed: int, B: int, T: int, Hq: int = 24, Hkv: int = 4, D: int = 256, sub: int = 0) -> dict:
    """Full-attention layer inputs, bf16 bits: qg [B, T, Hq, 2, D] (query then gate per head),
    k, v [B, T, Hkv, D], all N(0, 1) (projection outputs before the q/k norms); q_norm_w,
    k_norm_w [D] ~ N(1, 0.1^2)."""
    qg = normal_tokens(seed, "attn_qg", B * T, Hq * 2 * D, sub=sub, post=f32_to_bf16, out_dtype=np.uint16)
    k = normal_tokens(seed, "attn_k", B * T, Hkv * D, sub=sub, post=f32_to_bf16, out_dtype=np.uint16)
    v = normal_tokens(seed, "attn_v", B * T, Hkv * D, sub=sub, post=f32_to_bf16, out_dtype=np.uint16)
    qw = normal_tokens(seed, "attn_qw", 1, D, loc=1.0, scale=0.1, post=f32_to_bf16, out_dtype=np.uint16)[0]
    kw = normal_tokens(seed, "attn_kw", 1, D, loc=1.0, scale=0.1, post=f32_to_bf16, out_dtype=np.uint16)[0]
    return dict(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, qg=qg.reshape(B, T, Hq, 2, D), k=k.reshape(B, T, Hkv, D),
                v=v.reshape(B, T, Hkv, D), q_norm_w=qw, k_norm_w=kw)


def varlen_lengths(n: int = 32, lo: int = 16, hi: int = 8192, seed: int = 6) -> np.ndarray:
    """Request lengths of a continuous-batching prefill: n draws, log-uniform on [lo, hi]
    (numpy default_rng(seed)), truncated to integers."""
    rng = np.random.default_rng(seed)
    return np.exp(rng.uniform(np.log(lo), np.log(hi), n)).astype(np.int64)
