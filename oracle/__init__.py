"""fp64 CPU oracle for the Gated DeltaNet mixer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package never
imports the product package: the two share no code.  Where they meet is the
seeded input generator module, which holds no arithmetic of the method.

The numerics live in ``gdn_oracle.c`` (plain fp64 loops, OpenMP across
independent heads/columns); this module compiles it with gcc and marshals
numpy arrays to it.  ``chunked.py`` holds a second, independent fp64
implementation of the chunkwise (WY/UT) form, used only to pin that form to
the sequential definition on tiny inputs.

Input arrays may be float64, float32, or uint16 holding bf16 bit patterns;
the C code widens them exactly to double.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")

F64, F32, BF16 = 0, 1, 2


def build(verbose: bool = False) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so next to it (gcc, -O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o",
           _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Dims(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("T", ctypes.c_int64), ("Hk", ctypes.c_int64),
        ("Hv", ctypes.c_int64), ("Dk", ctypes.c_int64), ("Dv", ctypes.c_int64),
        ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64), ("stride_v", ctypes.c_int64),
        ("q_dtype", ctypes.c_int32), ("k_dtype", ctypes.c_int32), ("v_dtype", ctypes.c_int32),
        ("gate_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
        ("l2norm", ctypes.c_int32),
        ("q_scale", ctypes.c_double), ("l2_eps", ctypes.c_double),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = load_library(_LIB_PATH)
    return _lib


def load_library(path: str) -> ctypes.CDLL:
    """Loads a build of gdn_oracle.c from ``path`` and declares its entry points."""
    L = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    L.gdn_oracle_recurrence.argtypes = [ctypes.POINTER(_Dims), p, p, p, p, p, p, i64, p, p, p, i32]
    L.gdn_oracle_recurrence.restype = ctypes.c_int
    L.gdn_oracle_conv1d_silu.argtypes = [i64, i64, i64, i64, i64, i32, p, i32, p, i32, p,
                                         i64, i64, i64, i64, i64, p, p, i32]
    L.gdn_oracle_conv1d_silu.restype = ctypes.c_int
    L.gdn_oracle_gated_rmsnorm.argtypes = [i64, i64, i32, p, i32, p, i32, p, ctypes.c_double,
                                           i64, p, p, i32]
    L.gdn_oracle_gated_rmsnorm.restype = ctypes.c_int
    L.gdn_oracle_gates.argtypes = [i64, i64, i64, i32, p, i32, p, p, p, p]
    L.gdn_oracle_gates.restype = ctypes.c_int
    L.gdn_oracle_round_bf16.argtypes = [p, p, i64]
    L.gdn_oracle_round_bf16.restype = None
    return L


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float64, float32 or uint16 (bf16 bits), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _token_view(a: np.ndarray, B: int, T: int, width: int, name: str) -> int:
    """Checks a [B,T,>=width] view whose last dim is contiguous and whose
    batch stride is T*token_stride; returns the token stride in elements."""
    if a.ndim != 3 or a.shape[0] != B or a.shape[1] != T or a.shape[2] < width:
        raise ValueError(f"{name}: expected [B={B},T={T},{width}], got {a.shape}")
    it = a.itemsize
    s0, s1, s2 = a.strides
    if s2 != it or s1 % it or s0 % it or (T > 1 and B > 1 and s0 != T * s1):
        raise ValueError(f"{name}: unsupported strides {a.strides}")
    if T > 1:
        return s1 // it
    return s0 // it if B > 1 else max(width, s1 // it)


def recurrence(q, k, v, log_alpha, beta, Hk: int, Hv: int, state_in=None, *, l2norm=False,
               l2_eps=1e-6, q_scale=1.0, sel=None, want_o=True, want_state=True, n_threads=0):
    """Sequential fp64 gated delta rule.

    q, k: [B, T, Hk*Dk] views; v: [B, T, Hv*Dv] view; log_alpha, beta: [B, T, Hv];
    state_in: [B, Hv, Dk, Dv] or None (zero state).  ``sel`` lists flat
    b*Hv + h indices to compute (None = all).  Returns (o [n_sel, T, Dv],
    state [n_sel, Dk, Dv]) as float64 (None where not wanted).
    """
    B, T = q.shape[0], q.shape[1]
    Dk = q.shape[2] // Hk
    Dv = v.shape[2] // Hv
    sq = _token_view(q, B, T, Hk * Dk, "q")
    sk = _token_view(k, B, T, Hk * Dk, "k")
    sv = _token_view(v, B, T, Hv * Dv, "v")
    la = np.ascontiguousarray(log_alpha)
    bt = np.ascontiguousarray(beta)
    if la.shape != (B, T, Hv) or bt.shape != (B, T, Hv):
        raise ValueError("gates must be [B, T, Hv]")
    if la.dtype != bt.dtype:
        bt = bt.astype(la.dtype)
    if state_in is not None:
        state_in = np.ascontiguousarray(state_in)
        if state_in.shape != (B, Hv, Dk, Dv):
            raise ValueError("state_in must be [B, Hv, Dk, Dv]")
    d = _Dims(B, T, Hk, Hv, Dk, Dv, sq, sk, sv, _code(q), _code(k), _code(v), _code(la),
              _code(state_in) if state_in is not None else F64, int(bool(l2norm)),
              float(q_scale), float(l2_eps))
    if sel is None:
        n_sel = B * Hv
        sel_arr = None
    else:
        sel_arr = np.ascontiguousarray(np.asarray(sel, dtype=np.int64))
        n_sel = sel_arr.size
    o = np.empty((n_sel, T, Dv), np.float64) if want_o else None
    st = np.empty((n_sel, Dk, Dv), np.float64) if want_state else None
    rc = lib().gdn_oracle_recurrence(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(bt),
                                     _ptr(state_in), n_sel, _ptr(sel_arr), _ptr(o), _ptr(st),
                                     int(n_threads))
    if rc != 0:
        raise ValueError("gdn_oracle_recurrence rejected its arguments")
    return o, st


def conv1d_silu(x, w, conv_state_in=None, *, b=0, t0=0, t1=None, c0=0, c1=None,
                want_state=False, n_threads=0):
    """fp64 depthwise causal conv + SiLU.  x: [B, T, C] (last dim contiguous),
    w: [C, K], conv_state_in: [B, C, K-1] or None.  Returns
    (y[t1-t0, c1-c0] for batch b, conv_state_out [B, C, K-1] or None)."""
    B, T, C = x.shape
    K = w.shape[1]
    sx = _token_view(x, B, T, C, "x")
    w = np.ascontiguousarray(w)
    if w.shape != (C, K):
        raise ValueError("w must be [C, K]")
    if conv_state_in is not None:
        conv_state_in = np.ascontiguousarray(conv_state_in)
        if conv_state_in.shape != (B, C, K - 1):
            raise ValueError("conv_state_in must be [B, C, K-1]")
    t1 = T if t1 is None else t1
    c1 = C if c1 is None else c1
    y = np.empty((t1 - t0, c1 - c0), np.float64)
    cs = np.empty((B, C, K - 1), np.float64) if want_state else None
    rc = lib().gdn_oracle_conv1d_silu(B, T, C, K, sx, _code(x), _ptr(x), _code(w), _ptr(w),
                                      _code(conv_state_in) if conv_state_in is not None else F64,
                                      _ptr(conv_state_in), b, t0, t1, c0, c1, _ptr(y), _ptr(cs),
                                      int(n_threads))
    if rc != 0:
        raise ValueError("gdn_oracle_conv1d_silu rejected its arguments")
    return y, cs


def l2norm_heads(y, head_dim: int, eps: float):
    """fp64 per-head L2 normalisation along the last axis, in groups of head_dim channels:
    each group x becomes x / sqrt(sum x^2 + eps), what the recurrence's L2 flag does to q and
    k before they enter the rule (gdn_oracle.c, l2_normalise)."""
    y = np.asarray(y, np.float64)
    if y.shape[-1] % head_dim:
        raise ValueError("the last axis must be a whole number of heads")
    g = y.reshape(y.shape[:-1] + (y.shape[-1] // head_dim, head_dim))
    return (g / np.sqrt((g * g).sum(-1, keepdims=True) + eps)).reshape(y.shape)


def gated_rmsnorm(x, z, w, eps: float, *, rows=None, n_threads=0):
    """fp64 y = x / sqrt(mean(x^2)+eps) * w * z * sigmoid(z) over rows of D.
    x, z: [R, D] contiguous; w: [D]; rows: selected row indices (None = all)."""
    x = np.ascontiguousarray(x)
    z = np.ascontiguousarray(z)
    w = np.ascontiguousarray(w)
    R, D = x.shape
    if z.shape != (R, D) or w.shape != (D,):
        raise ValueError("shape mismatch")
    sel = None if rows is None else np.ascontiguousarray(np.asarray(rows, np.int64))
    n = R if sel is None else sel.size
    y = np.empty((n, D), np.float64)
    rc = lib().gdn_oracle_gated_rmsnorm(R, D, _code(x), _ptr(x), _code(z), _ptr(z), _code(w), _ptr(w),
                                        float(eps), n, _ptr(sel), _ptr(y), int(n_threads))
    if rc != 0:
        raise ValueError("gdn_oracle_gated_rmsnorm rejected its arguments")
    return y


def gates(ba, Hv: int, A_log, dt_bias):
    """fp64 gate activation from raw in_proj_ba outputs (gdn_oracle.c, gdn_oracle_gates).
    ba: [..., >= 2*Hv] (beta logits in [0, Hv), alpha inputs in [Hv, 2*Hv)); A_log, dt_bias:
    [Hv] (same dtype).  Returns (log_alpha, beta), float64 [..., Hv]."""
    ba = np.asarray(ba)
    lead = ba.shape[:-1]
    ba2 = ba.reshape(-1, ba.shape[-1])
    if ba2.strides[-1] != ba2.itemsize:
        ba2 = np.ascontiguousarray(ba2)
    A_log = np.ascontiguousarray(A_log)
    dt_bias = np.ascontiguousarray(dt_bias, dtype=A_log.dtype)
    if A_log.shape != (Hv,) or dt_bias.shape != (Hv,):
        raise ValueError("A_log and dt_bias must be [Hv]")
    n = ba2.shape[0]
    la = np.empty((n, Hv), np.float64)
    be = np.empty((n, Hv), np.float64)
    stride = ba2.strides[0] // ba2.itemsize if n > 1 else ba2.shape[1]
    rc = lib().gdn_oracle_gates(n, Hv, stride, _code(ba2), _ptr(ba2), _code(A_log), _ptr(A_log), _ptr(dt_bias),
                                _ptr(la), _ptr(be))
    if rc != 0:
        raise ValueError("gdn_oracle_gates rejected its arguments")
    return la.reshape(lead + (Hv,)), be.reshape(lead + (Hv,))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Rounds float64 values once to the nearest bf16 (ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().gdn_oracle_round_bf16(_ptr(a), _ptr(out), a.size)
    return out
