"""ctypes binding of libgdn (include/gdn.h, include/gdn_attn.h): argument marshalling only.

Each function takes torch tensors, checks their layout enough to build the C
arguments (pointers, element strides, the current HIP stream) and calls the
same-named C entry point.  Every step of the computation runs in the HIP
kernels of libgdn.so; there is no Python or CPU fallback.  If the library
has not been built, loading fails with an error that says so.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdn.so")

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_ALIGN, GDN_ERR_DEVICE = range(6)
GDN_F32, GDN_BF16 = 0, 1
GDN_FLAG_QK_L2NORM = 1
GDN_FLAG_TOKEN_SERIAL = 2
GDN_FLAG_NORM_IN_CHAIN = 4

# Every exported symbol, in the order include/gdn.h, then include/gdn_attn.h declare them.
EXPORTS = ("gdn_prefill", "gdn_prefill_gated", "gdn_prefill_static", "gdn_prefill_workspace_size", "gdn_prefill_varlen", "gdn_prefill_varlen_workspace_size",
           "gdn_decode_step", "gdn_conv1d_silu", "gdn_conv1d_silu_l2",
           "gdn_gated_rmsnorm", "gdn_gates", "gdn_decode_token", "gdn_decode_layer", "gdn_last_error",
           "gdn_version",
           "gdn_attn_prefill", "gdn_attn_prefill_workspace_size", "gdn_attn_decode", "gdn_attn_decode_workspace_size",
           "gdn_probe_mfma", "gdn_probe_copy")


class GdnDims(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hk", ctypes.c_int32),
        ("Hv", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("io", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64),
        ("stride_v", ctypes.c_int64), ("stride_o", ctypes.c_int64),
        ("q_scale", ctypes.c_float), ("l2_eps", ctypes.c_float),
    ]


class GdnDecodeLayerArgs(ctypes.Structure):
    p = ctypes.c_void_p
    _fields_ = [
        ("B", ctypes.c_int32), ("Hk", ctypes.c_int32), ("Hv", ctypes.c_int32), ("D", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("q_scale", ctypes.c_float), ("l2_eps", ctypes.c_float),
        ("norm_eps", ctypes.c_float), ("n_slots", ctypes.c_int32),
        ("x", p), ("stride_x", ctypes.c_int64), ("conv_w", p), ("conv_state_in", p), ("conv_state_out", p),
        ("ba", p), ("stride_ba", ctypes.c_int64), ("A_log", p), ("dt_bias", p), ("state_pool", p),
        ("slots", p), ("z", p), ("stride_z", ctypes.c_int64), ("norm_w", p), ("out", p),
        ("stride_out", ctypes.c_int64), ("o", p), ("stride_o", ctypes.c_int64),
    ]
    del p


class GdnAttnDims(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32), ("rot_dim", ctypes.c_int32), ("S_max", ctypes.c_int32),
        ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float), ("scale", ctypes.c_float),
        ("stride_qg", ctypes.c_int64), ("stride_k", ctypes.c_int64), ("stride_v", ctypes.c_int64),
        ("stride_o", ctypes.c_int64),
    ]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libgdn status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libgdn.so (built in-tree by build_lib.py); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                               "(or python gated_deltanet_recurrence_rule_amd/build_lib.py)")
        L = ctypes.CDLL(LIB_PATH)
        p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.gdn_prefill.argtypes = [ctypes.POINTER(GdnDims), p, p, p, p, p, p, p, p, p, ctypes.c_size_t, p]
        L.gdn_prefill.restype = ctypes.c_int
        L.gdn_prefill_gated.argtypes = [ctypes.POINTER(GdnDims), p, p, p, p, p, p, p, p, i64, p, ctypes.c_float, p, p,
                                        ctypes.c_size_t, p]
        L.gdn_prefill_gated.restype = ctypes.c_int
        L.gdn_prefill_static.argtypes = [ctypes.POINTER(GdnDims), p, p, p, p, p, p, p, p, p]
        L.gdn_prefill_static.restype = ctypes.c_int
        L.gdn_prefill_workspace_size.argtypes = [ctypes.POINTER(GdnDims)]
        L.gdn_prefill_workspace_size.restype = ctypes.c_size_t
        L.gdn_prefill_varlen.argtypes = [ctypes.POINTER(GdnDims), p, p, p, p, p, p, p, p, p, p, ctypes.c_size_t, p]
        L.gdn_prefill_varlen.restype = ctypes.c_int
        L.gdn_prefill_varlen_workspace_size.argtypes = [ctypes.POINTER(GdnDims)]
        L.gdn_prefill_varlen_workspace_size.restype = ctypes.c_size_t
        L.gdn_decode_step.argtypes = [ctypes.POINTER(GdnDims), p, p, p, p, p, p, p, p]
        L.gdn_decode_step.restype = ctypes.c_int
        L.gdn_conv1d_silu.argtypes = [i32, i32, i32, i32, i32, p, i64, p, p, p, p, i64, p]
        L.gdn_conv1d_silu_l2.argtypes = [i32, i32, i32, i32, i32, p, i64, p, p, p, p, i64, i32, ctypes.c_float, p]
        L.gdn_conv1d_silu_l2.restype = ctypes.c_int
        L.gdn_conv1d_silu.restype = ctypes.c_int
        L.gdn_gated_rmsnorm.argtypes = [i64, i32, i32, i32, p, i64, p, i64, p, ctypes.c_float, p, i64, p]
        L.gdn_gated_rmsnorm.restype = ctypes.c_int
        L.gdn_probe_mfma.argtypes = [i32, i32, p, p]
        L.gdn_probe_mfma.restype = ctypes.c_int
        L.gdn_probe_copy.argtypes = [p, p, ctypes.c_size_t, p]
        L.gdn_probe_copy.restype = ctypes.c_int
        L.gdn_gates.argtypes = [i64, i32, i32, p, i64, p, p, p, p, p]
        L.gdn_gates.restype = ctypes.c_int
        L.gdn_decode_token.argtypes = [ctypes.POINTER(GdnDims), p, p, p, i32, p, i64, p, p, p, i32, p, p, p]
        L.gdn_decode_token.restype = ctypes.c_int
        L.gdn_decode_layer.argtypes = [ctypes.POINTER(GdnDecodeLayerArgs), p]
        L.gdn_decode_layer.restype = ctypes.c_int
        AD = ctypes.POINTER(GdnAttnDims)
        L.gdn_attn_prefill.argtypes = [AD, p, p, p, p, p, p, p, p, p, ctypes.c_size_t, p]
        L.gdn_attn_prefill.restype = ctypes.c_int
        L.gdn_attn_prefill_workspace_size.argtypes = [AD]
        L.gdn_attn_prefill_workspace_size.restype = ctypes.c_size_t
        L.gdn_attn_decode.argtypes = [AD, p, p, p, p, p, p, p, p, p, p, ctypes.c_size_t, p]
        L.gdn_attn_decode.restype = ctypes.c_int
        L.gdn_attn_decode_workspace_size.argtypes = [AD]
        L.gdn_attn_decode_workspace_size.restype = ctypes.c_size_t
        L.gdn_last_error.argtypes = []
        L.gdn_last_error.restype = ctypes.c_char_p
        L.gdn_version.argtypes = []
        L.gdn_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, lib().gdn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(stream, *tensors):
    """Buffers this binding allocated come from the current stream's pool; when the
    kernels run on another stream, mark them used there so that the caching
    allocator does not hand their memory out before that stream's work is done."""
    import torch
    if stream is None:
        return
    if stream.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _io(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"io tensors must be bfloat16 or float32, got {t.dtype}")


def _token_stride(t, B: int, T: int, width: int, name: str) -> int:
    """[B, T, >= width] tensor (or view) with contiguous last dim and batch
    stride T * token stride; returns the token stride in elements."""
    if t.dim() != 3 or t.shape[0] != B or t.shape[1] != T or t.shape[2] < width:
        raise ValueError(f"{name}: expected [B={B}, T={T}, >={width}], got {tuple(t.shape)}")
    s0, s1, s2 = t.stride()
    if s2 != 1:
        raise ValueError(f"{name}: last dim must be contiguous")
    if T > 1:
        if B > 1 and s0 != T * s1:
            raise ValueError(f"{name}: batch stride must be T * token stride")
        return s1
    return s0 if B > 1 else max(width, s1)


def make_dims(B, T, Hk, Hv, D, io, flags=0, sq=None, sk=None, sv=None, so=None,
              q_scale=1.0, l2_eps=1e-6) -> GdnDims:
    return GdnDims(B, T, Hk, Hv, D, D, io, flags,
                   Hk * D if sq is None else sq, Hk * D if sk is None else sk,
                   Hv * D if sv is None else sv, Hv * D if so is None else so,
                   q_scale, l2_eps)


def gdn_prefill_workspace_size(dims: GdnDims) -> int:
    return int(lib().gdn_prefill_workspace_size(ctypes.byref(dims)))


def gdn_prefill(q, k, v, log_alpha, beta, state_in=None, state_out=None, o=None, *, Hk: int,
                Hv: int, l2norm: bool = False, l2_eps: float = 1e-6, q_scale: float = 1.0,
                token_serial: bool = False, workspace=None, stream=None):
    """q, k: [B, T, Hk*D] views; v: [B, T, Hv*D]; log_alpha, beta: [B, T, Hv] fp32;
    state_in / state_out: [B, Hv, D, D] fp32 or None; o: [B, T, >=Hv*D] or None
    (allocated); workspace: uint8 device tensor or None (allocated with the size
    gdn_prefill_workspace_size asks for); token_serial: GDN_FLAG_TOKEN_SERIAL.
    Returns o."""
    import torch
    B, T = int(q.shape[0]), int(q.shape[1])
    if q.shape[2] % Hk or v.shape[2] % Hv or q.shape[2] // Hk != v.shape[2] // Hv:
        raise ValueError("q must be [B, T, Hk*D] and v [B, T, Hv*D] (views of exactly that width)")
    D = int(q.shape[2]) // Hk
    io = _io(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or (o is not None and o.dtype != q.dtype):
        raise ValueError("q, k, v and o must share one dtype")
    own = []
    if o is None:
        o = torch.empty((B, T, Hv * D), dtype=q.dtype, device=q.device)
        own.append(o)
    flags = (GDN_FLAG_QK_L2NORM if l2norm else 0) | (GDN_FLAG_TOKEN_SERIAL if token_serial else 0)
    dims = make_dims(B, T, Hk, Hv, D, io, flags,
                     _token_stride(q, B, T, Hk * D, "q"), _token_stride(k, B, T, Hk * D, "k"),
                     _token_stride(v, B, T, Hv * D, "v"), _token_stride(o, B, T, Hv * D, "o"),
                     q_scale, l2_eps)
    for name, g in (("log_alpha", log_alpha), ("beta", beta)):
        if g.dtype != torch.float32 or not g.is_contiguous() or tuple(g.shape) != (B, T, Hv):
            raise ValueError(f"{name} must be contiguous fp32 [B, T, Hv]")
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()
                              or tuple(s.shape) != (B, Hv, D, D)):
            raise ValueError(f"{name} must be contiguous fp32 [B, Hv, D, D]")
    ws_bytes = gdn_prefill_workspace_size(dims)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_prefill(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                             _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(o), _ptr(workspace),
                             ws_len, _stream(stream)))
    _on_stream(stream, *own)
    return o


def gdn_prefill_gated(q, k, v, log_alpha, beta, z, norm_w, norm_eps: float = 1e-6, state_in=None, state_out=None,
                      y=None, *, Hk: int, Hv: int, l2norm: bool = False, l2_eps: float = 1e-6,
                      q_scale: float = 1.0, token_serial: bool = False, in_chain: bool = False,
                      workspace=None, stream=None):
    """gdn_prefill_gated: the prefill, then the gated RMSNorm of every output row.
    Shapes as gdn_prefill; z: [B, T, >=Hv*D] view; norm_w: [D]; y: [B, T, >=Hv*D]
    or None (allocated); in_chain: GDN_FLAG_NORM_IN_CHAIN.  Returns y."""
    import torch
    B, T = int(q.shape[0]), int(q.shape[1])
    if q.shape[2] % Hk or v.shape[2] % Hv or q.shape[2] // Hk != v.shape[2] // Hv:
        raise ValueError("q must be [B, T, Hk*D] and v [B, T, Hv*D] (views of exactly that width)")
    D = int(q.shape[2]) // Hk
    io = _io(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or z.dtype != q.dtype or norm_w.dtype != q.dtype or (
            y is not None and y.dtype != q.dtype):
        raise ValueError("q, k, v, z, norm_w and y must share one dtype")
    if tuple(norm_w.shape) != (D,) or not norm_w.is_contiguous():
        raise ValueError(f"norm_w must be contiguous [{D}]")
    own = []
    if y is None:
        y = torch.empty((B, T, Hv * D), dtype=q.dtype, device=q.device)
        own.append(y)
    flags = ((GDN_FLAG_QK_L2NORM if l2norm else 0) | (GDN_FLAG_TOKEN_SERIAL if token_serial else 0) |
             (GDN_FLAG_NORM_IN_CHAIN if in_chain else 0))
    dims = make_dims(B, T, Hk, Hv, D, io, flags,
                     _token_stride(q, B, T, Hk * D, "q"), _token_stride(k, B, T, Hk * D, "k"),
                     _token_stride(v, B, T, Hv * D, "v"), _token_stride(y, B, T, Hv * D, "y"),
                     q_scale, l2_eps)
    sz = _token_stride(z, B, T, Hv * D, "z")
    for name, g in (("log_alpha", log_alpha), ("beta", beta)):
        if g.dtype != torch.float32 or not g.is_contiguous() or tuple(g.shape) != (B, T, Hv):
            raise ValueError(f"{name} must be contiguous fp32 [B, T, Hv]")
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()
                              or tuple(s.shape) != (B, Hv, D, D)):
            raise ValueError(f"{name} must be contiguous fp32 [B, Hv, D, D]")
    ws_bytes = gdn_prefill_workspace_size(dims)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_prefill_gated(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                   _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(z), sz, _ptr(norm_w),
                                   float(norm_eps), _ptr(y), _ptr(workspace), ws_len, _stream(stream)))
    _on_stream(stream, *own)
    return y


def gdn_prefill_static(q, k, v, log_alpha, beta, state_in, state_out, o, *, Hk: int, Hv: int,
                       l2norm: bool = False, l2_eps: float = 1e-6, q_scale: float = 1.0,
                       token_serial: bool = False, stream=None):
    """gdn_prefill_static: gdn_prefill on the library's fixed device scratch.  The
    caller passes every buffer (o included); nothing is allocated here or below.
    Shapes as gdn_prefill.  Returns o."""
    import torch
    B, T = int(q.shape[0]), int(q.shape[1])
    if q.shape[2] % Hk or v.shape[2] % Hv or q.shape[2] // Hk != v.shape[2] // Hv:
        raise ValueError("q must be [B, T, Hk*D] and v [B, T, Hv*D] (views of exactly that width)")
    D = int(q.shape[2]) // Hk
    io = _io(q)
    if o is None or k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise ValueError("q, k, v and o (required) must share one dtype")
    flags = (GDN_FLAG_QK_L2NORM if l2norm else 0) | (GDN_FLAG_TOKEN_SERIAL if token_serial else 0)
    dims = make_dims(B, T, Hk, Hv, D, io, flags,
                     _token_stride(q, B, T, Hk * D, "q"), _token_stride(k, B, T, Hk * D, "k"),
                     _token_stride(v, B, T, Hv * D, "v"), _token_stride(o, B, T, Hv * D, "o"),
                     q_scale, l2_eps)
    for name, g in (("log_alpha", log_alpha), ("beta", beta)):
        if g.dtype != torch.float32 or not g.is_contiguous() or tuple(g.shape) != (B, T, Hv):
            raise ValueError(f"{name} must be contiguous fp32 [B, T, Hv]")
    for name, s in (("state_in", state_in), ("state_out", state_out)):
        if s is not None and (s.dtype != torch.float32 or not s.is_contiguous()
                              or tuple(s.shape) != (B, Hv, D, D)):
            raise ValueError(f"{name} must be contiguous fp32 [B, Hv, D, D]")
    _check(lib().gdn_prefill_static(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                    _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(o), _stream(stream)))
    return o


def gdn_prefill_varlen_workspace_size(dims: GdnDims) -> int:
    return int(lib().gdn_prefill_varlen_workspace_size(ctypes.byref(dims)))


def gdn_prefill_varlen(q, k, v, log_alpha, beta, cu_seqlens, state_in=None, state_out=None, o=None, *, Hk: int,
                       Hv: int, l2norm: bool = False, l2_eps: float = 1e-6, q_scale: float = 1.0,
                       token_serial: bool = False, workspace=None, stream=None):
    """Packed sequences: q, k [T, Hk*D]; v [T, Hv*D]; log_alpha, beta [T, Hv] fp32; cu_seqlens [B+1]
    int32 device tensor (sequence s = tokens cu[s]..cu[s+1]); states [B, Hv, D, D] or None;
    o [T, >=Hv*D] or None.  Returns o."""
    import torch
    T = int(q.shape[0])
    nseq = int(cu_seqlens.shape[0]) - 1
    if q.shape[1] % Hk or v.shape[1] % Hv or q.shape[1] // Hk != v.shape[1] // Hv:
        raise ValueError("q must be [T, Hk*D] and v [T, Hv*D]")
    D = int(q.shape[1]) // Hk
    io = _io(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or (o is not None and o.dtype != q.dtype):
        raise ValueError("q, k, v and o must share one dtype")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous() or cu_seqlens.dim() != 1 or nseq < 0:
        raise ValueError("cu_seqlens must be a contiguous int32 [B+1] tensor")
    if cu_seqlens.device != q.device:
        raise ValueError("cu_seqlens must be on the device of q")
    own = []
    if o is None:
        o = torch.empty((T, Hv * D), dtype=q.dtype, device=q.device)
        own.append(o)
    for name, t, w in (("q", q, Hk * D), ("k", k, Hk * D), ("v", v, Hv * D), ("o", o, Hv * D)):
        if t.dim() != 2 or t.shape[0] != T or t.shape[1] < w or (T > 0 and t.stride(1) != 1):
            raise ValueError(f"{name}: expected [T, >={w}] with contiguous rows")
    for name, g in (("log_alpha", log_alpha), ("beta", beta)):
        if g.dtype != torch.float32 or not g.is_contiguous() or tuple(g.shape) != (T, Hv):
            raise ValueError(f"{name} must be contiguous fp32 [T, Hv]")
    for name, s_ in (("state_in", state_in), ("state_out", state_out)):
        if s_ is not None and (s_.dtype != torch.float32 or not s_.is_contiguous()
                               or tuple(s_.shape) != (nseq, Hv, D, D)):
            raise ValueError(f"{name} must be contiguous fp32 [B, Hv, D, D]")
    flags = (GDN_FLAG_QK_L2NORM if l2norm else 0) | (GDN_FLAG_TOKEN_SERIAL if token_serial else 0)
    st = lambda t, w: t.stride(0) if T > 1 else w
    dims = make_dims(nseq, T, Hk, Hv, D, io, flags, st(q, Hk * D), st(k, Hk * D), st(v, Hv * D), st(o, Hv * D),
                     q_scale, l2_eps)
    ws_bytes = gdn_prefill_varlen_workspace_size(dims)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
        own.append(workspace)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().gdn_prefill_varlen(ctypes.byref(dims), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(log_alpha), _ptr(beta), _ptr(state_in), _ptr(state_out), _ptr(o),
                                    _ptr(workspace), ws_len, _stream(stream)))
    _on_stream(stream, *own)
    return o


def gdn_decode_step(q, k, v, log_alpha, beta, state, o=None, *, Hk: int, Hv: int,
                    l2norm: bool = False, l2_eps: float = 1e-6, q_scale: float = 1.0, stream=None):
    """q, k: [B, >=Hk*D]; v: [B, >=Hv*D]; log_alpha, beta: [B, Hv] fp32;
    state: [B, Hv, D, D] fp32 (updated in place); o: [B, >=Hv*D] or None.  Returns o."""
    import torch
    B = int(state.shape[0])
    D = int(state.shape[2])
    io = _io(q)
    own = None
    if o is None:
        o = own = torch.empty((B, Hv * D), dtype=q.dtype, device=q.device)
    for name, t, w in (("q", q, Hk * D), ("k", k, Hk * D), ("v", v, Hv * D), ("o", o, Hv * D)):
        if t.dim() != 2 or t.shape[0] != B or t.shape[1] < w or t.stride(1) != 1:
            raise ValueError(f"{name}: expected [B, >={w}] with contiguous rows")
    for name, g in (("log_alpha", log_alpha), ("beta", beta)):
        if g.dtype != torch.float32 or not g.is_contiguous() or tuple(g.shape) != (B, Hv):
            raise ValueError(f"{name} must be contiguous fp32 [B, Hv]")
    if state.dtype != torch.float32 or not state.is_contiguous() or tuple(state.shape) != (B, Hv, D, D):
        raise ValueError("state must be contiguous fp32 [B, Hv, D, D]")
    dims = make_dims(B, 1, Hk, Hv, D, io, GDN_FLAG_QK_L2NORM if l2norm else 0,
                     q.stride(0) if B > 1 else Hk * D, k.stride(0) if B > 1 else Hk * D,
                     v.stride(0) if B > 1 else Hv * D, o.stride(0) if B > 1 else Hv * D,
                     q_scale, l2_eps)
    _check(lib().gdn_decode_step(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                 _ptr(beta), _ptr(state), _ptr(o), _stream(stream)))
    _on_stream(stream, own)
    return o


def gdn_conv1d_silu(x, w, conv_state_in=None, conv_state_out=None, y=None, *, l2_channels: int = 0,
                    l2_eps: float = 1e-6, stream=None):
    """x: [B, T, >=C] view (contiguous channels); w: [C, 4]; conv states [B, C, 3] or None;
    y: [B, T, >=C] or None (allocated [B, T, C]); l2_channels > 0 calls gdn_conv1d_silu_l2
    (channels [0, l2_channels) L2-normalised per 128-channel head).  Returns y."""
    import torch
    B, T = int(x.shape[0]), int(x.shape[1])
    C, K = int(w.shape[0]), int(w.shape[1])
    io = _io(x)
    own = None
    if y is None:
        y = own = torch.empty((B, T, C), dtype=x.dtype, device=x.device)
    sx = _token_stride(x, B, T, C, "x") if T > 0 else C
    sy = _token_stride(y, B, T, C, "y") if T > 0 else C
    if w.dtype != x.dtype or not w.is_contiguous():
        raise ValueError("w must be contiguous with x's dtype")
    for name, s in (("conv_state_in", conv_state_in), ("conv_state_out", conv_state_out)):
        if s is not None and (s.dtype != x.dtype or not s.is_contiguous() or tuple(s.shape) != (B, C, K - 1)):
            raise ValueError(f"{name} must be contiguous [B, C, K-1] with x's dtype")
    if l2_channels:
        _check(lib().gdn_conv1d_silu_l2(B, T, C, K, io, _ptr(x), sx, _ptr(w), _ptr(conv_state_in),
                                        _ptr(conv_state_out), _ptr(y), sy, int(l2_channels), float(l2_eps),
                                        _stream(stream)))
    else:
        _check(lib().gdn_conv1d_silu(B, T, C, K, io, _ptr(x), sx, _ptr(w), _ptr(conv_state_in),
                                     _ptr(conv_state_out), _ptr(y), sy, _stream(stream)))
    _on_stream(stream, own)
    return y


def gdn_gated_rmsnorm(x, z, w, eps: float = 1e-5, y=None, *, H: int, stream=None):
    """x, z: [n_tok, >=H*D] (contiguous channels); w: [D]; y: [n_tok, >=H*D] or None.
    Rows are (token, head) D-vectors.  Returns y."""
    import torch
    D = int(w.shape[0])
    n = int(x.shape[0])
    io = _io(x)
    own = None
    if y is None:
        y = own = torch.empty((n, H * D), dtype=x.dtype, device=x.device)
    for name, t in (("x", x), ("z", z), ("y", y)):
        if t.dim() != 2 or t.shape[0] != n or t.shape[1] < H * D or t.stride(1) != 1 or t.dtype != x.dtype:
            raise ValueError(f"{name}: expected [n_tok, >={H * D}] with contiguous channels")
    if w.dtype != x.dtype or not w.is_contiguous():
        raise ValueError("w must be contiguous with x's dtype")
    _check(lib().gdn_gated_rmsnorm(n, H, D, io, _ptr(x), x.stride(0) if n > 1 else H * D, _ptr(z),
                                   z.stride(0) if n > 1 else H * D, _ptr(w), float(eps), _ptr(y),
                                   y.stride(0) if n > 1 else H * D, _stream(stream)))
    _on_stream(stream, own)
    return y


def gdn_probe_mfma(n_workgroups: int, iters: int, sink, stream=None):
    """Matrix-core probe: n_workgroups x 4 waves of `iters` rounds of four 32x32x16 bf16
    MFMAs; sink: fp32 [n_workgroups * 256], each entry 1024 * iters afterwards.  Returns
    the flop count."""
    import torch
    if sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() < n_workgroups * 256:
        raise ValueError("sink must be contiguous fp32 with n_workgroups * 256 entries")
    _check(lib().gdn_probe_mfma(int(n_workgroups), int(iters), _ptr(sink), _stream(stream)))
    return n_workgroups * 4 * iters * 4 * 32 * 32 * 16 * 2


def gdn_probe_copy(src, dst, stream=None):
    """Device-copy probe: dst <- src, both contiguous, the same byte size (a multiple of 32 KiB)."""
    n = src.numel() * src.element_size()
    if not src.is_contiguous() or not dst.is_contiguous() or dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must be contiguous and of the same byte size")
    _check(lib().gdn_probe_copy(_ptr(src), _ptr(dst), n, _stream(stream)))


def _params(A_log, dt_bias, Hv: int):
    import torch
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (Hv,):
            raise ValueError(f"{name} must be contiguous fp32 [Hv]")


def gdn_gates(ba, A_log, dt_bias, log_alpha=None, beta=None, *, Hv: int, stream=None):
    """ba: [n_tok, >=2*Hv] raw in_proj_ba outputs (bf16 or fp32, contiguous columns; beta
    logits first); A_log, dt_bias: [Hv] fp32.  Returns (log_alpha, beta), [n_tok, Hv] fp32."""
    import torch
    n = int(ba.shape[0])
    if ba.dim() != 2 or ba.shape[1] < 2 * Hv or (n > 0 and ba.stride(1) != 1):
        raise ValueError(f"ba: expected [n_tok, >={2 * Hv}] with contiguous columns")
    _params(A_log, dt_bias, Hv)
    own = []
    if log_alpha is None:
        log_alpha = torch.empty((n, Hv), dtype=torch.float32, device=ba.device)
        own.append(log_alpha)
    if beta is None:
        beta = torch.empty((n, Hv), dtype=torch.float32, device=ba.device)
        own.append(beta)
    for name, g in (("log_alpha", log_alpha), ("beta", beta)):
        if g.dtype != torch.float32 or not g.is_contiguous() or g.numel() != n * Hv:
            raise ValueError(f"{name} must be contiguous fp32 with n_tok * Hv elements")
    _check(lib().gdn_gates(n, Hv, _io(ba), _ptr(ba), ba.stride(0) if n > 1 else 2 * Hv, _ptr(A_log),
                           _ptr(dt_bias), _ptr(log_alpha), _ptr(beta), _stream(stream)))
    _on_stream(stream, *own)
    return log_alpha, beta


def gdn_decode_token(q, k, v, ba, A_log, dt_bias, state_pool, slots=None, o=None, *, Hk: int, Hv: int,
                     l2norm: bool = False, l2_eps: float = 1e-6, q_scale: float = 1.0, stream=None):
    """One decode token per sequence with gates formed from the raw in_proj_ba outputs
    ba [B, >=2*Hv] (bf16 or fp32) and A_log, dt_bias [Hv] fp32, and states in a pool
    state_pool [S, Hv, D, D] fp32 (updated in place): sequence b uses entry slots[b]
    (slots: [B] int32 device tensor; None = entry b; negative = skipped).
    q, k: [B, >=Hk*D]; v: [B, >=Hv*D]; o: [B, >=Hv*D] or None.  Returns o."""
    import torch
    B = int(q.shape[0])
    D = int(state_pool.shape[2])
    io = _io(q)
    own = None
    if o is None:
        o = own = torch.empty((B, Hv * D), dtype=q.dtype, device=q.device)
    for name, t, w in (("q", q, Hk * D), ("k", k, Hk * D), ("v", v, Hv * D), ("o", o, Hv * D),
                       ("ba", ba, 2 * Hv)):
        if t.dim() != 2 or t.shape[0] != B or t.shape[1] < w or t.stride(1) != 1:
            raise ValueError(f"{name}: expected [B, >={w}] with contiguous rows")
    _params(A_log, dt_bias, Hv)
    if (state_pool.dtype != torch.float32 or not state_pool.is_contiguous() or state_pool.dim() != 4
            or tuple(state_pool.shape[1:]) != (Hv, D, D)):
        raise ValueError("state_pool must be contiguous fp32 [S, Hv, D, D]")
    if slots is None and state_pool.shape[0] < B:
        raise ValueError("without slots the pool needs at least B entries")
    if slots is not None and (slots.dtype != torch.int32 or not slots.is_contiguous() or tuple(slots.shape) != (B,)):
        raise ValueError("slots must be a contiguous int32 [B] tensor")
    dims = make_dims(B, 1, Hk, Hv, D, io, GDN_FLAG_QK_L2NORM if l2norm else 0,
                     q.stride(0) if B > 1 else Hk * D, k.stride(0) if B > 1 else Hk * D,
                     v.stride(0) if B > 1 else Hv * D, o.stride(0) if B > 1 else Hv * D,
                     q_scale, l2_eps)
    _check(lib().gdn_decode_token(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _io(ba), _ptr(ba),
                                  ba.stride(0) if B > 1 else 2 * Hv, _ptr(A_log), _ptr(dt_bias),
                                  _ptr(state_pool), int(state_pool.shape[0]), _ptr(slots), _ptr(o),
                                  _stream(stream)))
    _on_stream(stream, own)
    return o


def gdn_decode_layer(x, conv_w, conv_state_in, conv_state_out, ba, A_log, dt_bias, state_pool, z, norm_w,
                     slots=None, out=None, o=None, *, Hk: int, Hv: int, l2norm: bool = True,
                     l2_eps: float = 1e-6, q_scale: float = 1.0, norm_eps: float = 1e-6, stream=None):
    """One fused decode token of the layer (bf16, D = 128).  x: [B, >=C] pre-conv q|k|v channels
    (C = (2*Hk + Hv)*128); conv_w: [C, 4]; conv_state_in / _out: [S, C, 3] window pools (distinct);
    ba: [B, >=2*Hv]; A_log, dt_bias: [Hv] fp32; state_pool: [S, Hv, 128, 128] fp32 (in place);
    z: [B, >=Hv*128]; norm_w: [128]; slots: [B] int32 or None; out: [B, >=Hv*128] or None;
    o: optional pre-norm output.  Returns out."""
    import torch
    D = 128
    B = int(x.shape[0])
    C = (2 * Hk + Hv) * D
    own = None
    if out is None:
        out = own = torch.empty((B, Hv * D), dtype=torch.bfloat16, device=x.device)
    for name, t, wdt in (("x", x, C), ("ba", ba, 2 * Hv), ("z", z, Hv * D), ("out", out, Hv * D)) + \
            ((("o", o, Hv * D),) if o is not None else ()):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.shape[0] != B or t.shape[1] < wdt or t.stride(1) != 1:
            raise ValueError(f"{name}: expected bf16 [B, >={wdt}] with contiguous rows")
    for name, t in (("conv_w", conv_w), ("norm_w", norm_w), ("conv_state_in", conv_state_in),
                    ("conv_state_out", conv_state_out)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous bf16")
    if tuple(conv_w.shape) != (C, 4) or tuple(norm_w.shape) != (D,):
        raise ValueError("conv_w must be [C, 4] and norm_w [128]")
    S = int(state_pool.shape[0])
    if tuple(conv_state_in.shape) != (S, C, 3) or tuple(conv_state_out.shape) != (S, C, 3):
        raise ValueError("conv states must be [S, C, 3] with the state pool's S")
    _params(A_log, dt_bias, Hv)
    if (state_pool.dtype != torch.float32 or not state_pool.is_contiguous()
            or tuple(state_pool.shape[1:]) != (Hv, D, D)):
        raise ValueError("state_pool must be contiguous fp32 [S, Hv, 128, 128]")
    if slots is None and S < B:
        raise ValueError("without slots the pools need at least B entries")
    if slots is not None and (slots.dtype != torch.int32 or not slots.is_contiguous() or tuple(slots.shape) != (B,)):
        raise ValueError("slots must be a contiguous int32 [B] tensor")
    st = lambda t, wdt: t.stride(0) if B > 1 else wdt
    a = GdnDecodeLayerArgs(B, Hk, Hv, D, GDN_FLAG_QK_L2NORM if l2norm else 0, q_scale, l2_eps, norm_eps, S,
                           _ptr(x), st(x, C), _ptr(conv_w), _ptr(conv_state_in), _ptr(conv_state_out),
                           _ptr(ba), st(ba, 2 * Hv), _ptr(A_log), _ptr(dt_bias), _ptr(state_pool), _ptr(slots),
                           _ptr(z), st(z, Hv * D), _ptr(norm_w), _ptr(out), st(out, Hv * D), _ptr(o),
                           st(o, Hv * D) if o is not None else 0)
    _check(lib().gdn_decode_layer(ctypes.byref(a), _stream(stream)))
    _on_stream(stream, own)
    return out


def gdn_version() -> int:
    return int(lib().gdn_version())


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


# -- full-attention layer (include/gdn_attn.h) ---------------------------------

def make_attn_dims(B: int, T: int, Hq: int, Hkv: int, D: int = 256, S_max: int = 64, rot_dim: int = 64,
                   rope_theta: float = 1e7, norm_eps: float = 1e-6, scale: float | None = None,
                   stride_qg: int | None = None, stride_k: int | None = None, stride_v: int | None = None,
                   stride_o: int | None = None) -> GdnAttnDims:
    return GdnAttnDims(B, T, Hq, Hkv, D, rot_dim, S_max, rope_theta, norm_eps,
                       D ** -0.5 if scale is None else scale,
                       2 * Hq * D if stride_qg is None else stride_qg, Hkv * D if stride_k is None else stride_k,
                       Hkv * D if stride_v is None else stride_v, Hq * D if stride_o is None else stride_o)


def attn_cache(B: int, Hkv: int, S_max: int, D: int = 256, device="cuda"):
    """Zeroed key and value caches in the layout gdn_attn.h describes:
    k [B, Hkv, S_max, D] and v [B, Hkv, S_max // 64, D, 64], bf16."""
    import torch
    k = torch.zeros((B, Hkv, S_max, D), dtype=torch.bfloat16, device=device)
    v = torch.zeros((B, Hkv, S_max // 64, D, 64), dtype=torch.bfloat16, device=device)
    return k, v


def _rows(t, lead: int, width: int, name: str) -> int:
    """Token stride of a bf16 tensor whose first `lead` dims index tokens (batch-major, the
    token rows evenly spaced) and whose remaining dims are `width` contiguous elements."""
    import torch
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")
    inner = 1
    for n in t.shape[lead:]:
        inner *= int(n)
    if inner != width or (width and not t[(0,) * lead].is_contiguous() if t.numel() else False):
        raise ValueError(f"{name}: each token row must be {width} contiguous elements")
    st = int(t.stride(lead - 1))
    if lead == 2 and t.shape[1] > 0 and int(t.stride(0)) != st * int(t.shape[1]):
        raise ValueError(f"{name}: the sequence stride must be T times the token stride")
    return st if t.numel() else width


def gdn_attn_prefill(qg, k, v, q_norm_w, k_norm_w, k_cache, v_cache, o=None, *, rot_dim: int = 64,
                     rope_theta: float = 1e7, norm_eps: float = 1e-6, scale: float | None = None,
                     workspace=None, stream=None):
    """qg [B, T, Hq, 2, D] (query then gate per head); k, v [B, T, Hkv, D]; q_norm_w, k_norm_w [D];
    k_cache, v_cache from attn_cache (positions [0, T) are written); o [B, T, Hq, D] or None.
    Returns o."""
    import torch
    B, T, Hq, two, D = (int(x) for x in qg.shape)
    Hkv = int(k.shape[2])
    if two != 2 or tuple(k.shape) != (B, T, Hkv, D) or tuple(v.shape) != (B, T, Hkv, D):
        raise ValueError("qg must be [B, T, Hq, 2, D] and k, v [B, T, Hkv, D]")
    S_max = int(k_cache.shape[2])
    own = []
    if o is None:
        o = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device=qg.device)
        own.append(o)
    dims = make_attn_dims(B, T, Hq, Hkv, D, S_max, rot_dim, rope_theta, norm_eps, scale,
                          _rows(qg, 2, 2 * Hq * D, "qg"), _rows(k, 2, Hkv * D, "k"), _rows(v, 2, Hkv * D, "v"),
                          _rows(o, 2, Hq * D, "o"))
    need = int(lib().gdn_attn_prefill_workspace_size(ctypes.byref(dims)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=qg.device)
        own.append(workspace)
    ws_len = 0 if workspace is None else workspace.numel()
    _check(lib().gdn_attn_prefill(ctypes.byref(dims), _ptr(qg), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(workspace), ws_len, _stream(stream)))
    _on_stream(stream, *own)
    return o


def gdn_attn_decode(qg, k, v, q_norm_w, k_norm_w, cache_len, k_cache, v_cache, o=None, *, rot_dim: int = 64,
                    rope_theta: float = 1e7, norm_eps: float = 1e-6, scale: float | None = None,
                    workspace=None, stream=None):
    """One token per sequence: qg [B, Hq, 2, D]; k, v [B, Hkv, D]; cache_len [B] int32 on the device
    (the new token's position); caches from attn_cache.  Returns o [B, Hq, D]."""
    import torch
    B, Hq, two, D = (int(x) for x in qg.shape)
    Hkv = int(k.shape[1])
    if two != 2 or tuple(k.shape) != (B, Hkv, D) or tuple(v.shape) != (B, Hkv, D):
        raise ValueError("qg must be [B, Hq, 2, D] and k, v [B, Hkv, D]")
    if cache_len.dtype != torch.int32 or tuple(cache_len.shape) != (B,) or cache_len.device != qg.device:
        raise ValueError("cache_len must be an int32 [B] tensor on the device of qg")
    S_max = int(k_cache.shape[2])
    own = []
    if o is None:
        o = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=qg.device)
        own.append(o)
    dims = make_attn_dims(B, 1, Hq, Hkv, D, S_max, rot_dim, rope_theta, norm_eps, scale,
                          _rows(qg, 1, 2 * Hq * D, "qg"), _rows(k, 1, Hkv * D, "k"), _rows(v, 1, Hkv * D, "v"),
                          _rows(o, 1, Hq * D, "o"))
    need = int(lib().gdn_attn_decode_workspace_size(ctypes.byref(dims)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=qg.device)
        own.append(workspace)
    ws_len = 0 if workspace is None else workspace.numel()
    _check(lib().gdn_attn_decode(ctypes.byref(dims), _ptr(qg), _ptr(k), _ptr(v), _ptr(q_norm_w), _ptr(k_norm_w),
                                 _ptr(cache_len), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(workspace), ws_len,
                                 _stream(stream)))
    _on_stream(stream, *own)
    return o
