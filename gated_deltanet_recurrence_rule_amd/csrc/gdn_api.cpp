// gdn_api.cpp -- the extern "C" entry points of libgdn (declared in
// include/gdn.h and include/gdn_attn.h): argument validation on the host, kernel dispatch, status
// codes and the thread-local error message.  Validation happens before any
// HIP call, so argument errors are reported even on a machine without a GPU.
#include "../../include/gdn.h"
#include "../../include/gdn_attn.h"
#include "../../include/gdn_probe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "gdn_internal.h"

namespace gdn {

int device_cu_count() {
  static std::atomic<int> count[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 256;
  if (dev < 64) count[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace gdn

namespace {

// gdn_prefill_static's workspace: a fixed device array that each GPU the library runs on holds
// until the process ends.  Host code reaches its device address only through
// hipGetSymbolAddress (the array's name on the host is not a device pointer), once per device
// with that device current.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** out) {
  static std::atomic<void*> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

thread_local char g_err[512] = "";

gdn_status fail(gdn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

gdn_status ok() {
  g_err[0] = '\0';
  return GDN_OK;
}

gdn_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GDN_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Checks shared by prefill and decode.  `T1` demands T == 1.
gdn_status check_dims(const gdn_dims* d, bool T1) {
  if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
  if (d->B < 0 || d->T < 0) return fail(GDN_ERR_SHAPE, "B=%d T=%d must be >= 0", d->B, d->T);
  if (T1 && d->T != 1) return fail(GDN_ERR_SHAPE, "decode step needs T == 1 (got %d)", d->T);
  if (d->Hk < 1 || d->Hv < 1) return fail(GDN_ERR_SHAPE, "Hk=%d Hv=%d must be >= 1", d->Hk, d->Hv);
  if (d->Hv % d->Hk != 0) return fail(GDN_ERR_SHAPE, "Hv=%d is not a multiple of Hk=%d", d->Hv, d->Hk);
  if (d->Dk < 1 || d->Dv < 1) return fail(GDN_ERR_SHAPE, "Dk=%d Dv=%d must be >= 1", d->Dk, d->Dv);
  if (d->io != GDN_F32 && d->io != GDN_BF16) return fail(GDN_ERR_SHAPE, "io dtype %d unknown", d->io);
  if (d->Dk != d->Dv || !supported_d(d->Dk))
    return fail(GDN_ERR_UNSUPPORTED, "head widths Dk=%d Dv=%d: kernels take Dk == Dv in {16,32,64,128}",
                d->Dk, d->Dv);
  if ((d->flags & ~(GDN_FLAG_QK_L2NORM | GDN_FLAG_TOKEN_SERIAL)) != 0)
    return fail(GDN_ERR_SHAPE, "unknown flag bits 0x%x", d->flags);
  const int64_t wq = static_cast<int64_t>(d->Hk) * d->Dk, wv = static_cast<int64_t>(d->Hv) * d->Dv;
  if (d->stride_q < wq || d->stride_k < wq)
    return fail(GDN_ERR_SHAPE, "stride_q=%lld / stride_k=%lld below Hk*Dk=%lld", (long long)d->stride_q,
                (long long)d->stride_k, (long long)wq);
  if (d->stride_v < wv || d->stride_o < wv)
    return fail(GDN_ERR_SHAPE, "stride_v=%lld / stride_o=%lld below Hv*Dv=%lld", (long long)d->stride_v,
                (long long)d->stride_o, (long long)wv);
  if (d->flags & GDN_FLAG_QK_L2NORM) {
    if (!(d->l2_eps >= 0.0f)) return fail(GDN_ERR_SHAPE, "l2_eps must be >= 0");
  }
  return GDN_OK;
}

// The chunked kernels keep the gate vectors of all value heads of a key head in
// LDS, which bounds the heads per key head at 64.
bool use_chunk_kernel(const gdn_dims* d) {
  return d->io == GDN_BF16 && d->Dk == 128 && d->T > 0 && d->Hv / d->Hk <= 64 &&
         !(d->flags & GDN_FLAG_TOKEN_SERIAL);
}

gdn::RecArgs rec_args(const gdn_dims* d, const void* q, const void* k, const void* v, const float* la,
                      const float* beta, const float* sin, float* sout, void* o) {
  gdn::RecArgs a;
  a.B = d->B;
  a.T = d->T;
  a.Hk = d->Hk;
  a.Hv = d->Hv;
  a.G = d->Hv / d->Hk;
  a.D = d->Dk;
  a.flags = d->flags;
  a.q_scale = d->q_scale;
  a.l2_eps = d->l2_eps;
  a.sq = d->stride_q;
  a.sk = d->stride_k;
  a.sv = d->stride_v;
  a.so = d->stride_o;
  a.q = q;
  a.k = k;
  a.v = v;
  a.la = la;
  a.beta = beta;
  a.state_in = sin;
  a.state_out = sout;
  a.o = o;
  return a;
}

// Marks a packed (variable-length) batch in the workspace-size query, where
// cu_seqlens is not known; only its being non-null is looked at on the host.
const int32_t kPackedMarker[1] = {0};

// Arguments of the chunked path.  A packed batch is one token stream (B = 1 for
// the workspace layout) of d->B sequences.
gdn::RecArgs chunk_args(const gdn_dims* d, const int32_t* cu, const void* q, const void* k, const void* v,
                        const float* la, const float* beta, const float* sin, float* sout, void* o) {
  gdn::RecArgs a = rec_args(d, q, k, v, la, beta, sin, sout, o);
  if (cu) {
    a.B = 1;
    a.cu_seqlens = cu;
    a.nseq = d->B;
  }
  return a;
}

size_t workspace_size(const gdn_dims* dims, const int32_t* cu) {
  if (!dims) return 0;
  gdn_dims dd = *dims;   // gdn_prefill_gated's dims ask for the same workspace
  dd.flags &= ~GDN_FLAG_NORM_IN_CHAIN;
  const gdn_dims* d = &dd;
  if (check_dims(d, false) != GDN_OK || d->B == 0 || !use_chunk_kernel(d)) return 0;
  const gdn::RecArgs a = chunk_args(d, cu, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  const size_t per_chunk = gdn::chunk_ws_bytes_per_chunk(a);
  const int64_t nchunks = gdn::chunk_count(a);
  const int64_t nwin = gdn::chunk_window_chunks(a);
  const size_t maps = gdn::chunk_map_bytes(a);
  if (nwin >= nchunks) return maps + static_cast<size_t>(nchunks) * per_chunk;
  return maps + static_cast<size_t>(nwin) * per_chunk + gdn::chunk_ws_carry_bytes(a);
}

// The gated RMSNorm the chain applies to each output row (gdn_prefill_gated).
struct NormIn {
  const void* z;
  int64_t stride_z;
  const void* w;
  float eps;
};

gdn_status prefill(const gdn_dims* d, const int32_t* cu, const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* beta, const float* state_in, float* state_out, void* o,
                   void* workspace, size_t workspace_bytes, void* stream, const NormIn* norm = nullptr) {
  gdn_status st = check_dims(d, false);
  if (st != GDN_OK) return st;
  if (d->B == 0) return ok();
  if (d->T > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
    return fail(GDN_ERR_NULL, "q, k, v, log_alpha, beta and o are required");
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16)))
    return fail(GDN_ERR_ALIGN, "state pointers must be 16-byte aligned");
  if (d->T == 0 && !state_out) return ok();
  if (use_chunk_kernel(d)) {
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
      return fail(GDN_ERR_ALIGN, "bf16 q, k, v, o must be 16-byte aligned");
    if ((d->stride_q % 8) || (d->stride_k % 8) || (d->stride_v % 8) || (d->stride_o % 8))
      return fail(GDN_ERR_ALIGN, "bf16 strides of q, k, v, o must be multiples of 8 elements");
    gdn::RecArgs a = chunk_args(d, cu, q, k, v, log_alpha, beta, state_in, state_out, o);
    if (norm) {
      a.gz = norm->z;
      a.sz = norm->stride_z;
      a.gw = norm->w;
      a.geps = norm->eps;
    }
    const size_t per_chunk = gdn::chunk_ws_bytes_per_chunk(a);
    const int64_t nchunks = gdn::chunk_count(a);
    const size_t maps = gdn::chunk_map_bytes(a);
    const size_t need_min =
        maps + per_chunk + ((nchunks > 1 && !state_out) ? gdn::chunk_ws_carry_bytes(a) : 0);
    if (!workspace) return fail(GDN_ERR_NULL, "the chunked prefill needs a workspace");
    if (!aligned(workspace, 256)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (workspace_bytes < need_min && workspace_bytes < maps + static_cast<size_t>(nchunks) * per_chunk)
      return fail(GDN_ERR_SHAPE, "workspace of %zu bytes is below the minimum %zu", workspace_bytes, need_min);
    return from_hip(gdn::launch_chunk_prefill(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
                    "gdn_prefill (chunk kernels)");
  }
  const size_t es = d->io == GDN_BF16 ? 2 : 4;
  if (d->T > 0 && (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(o, es)))
    return fail(GDN_ERR_ALIGN, "q, k, v, o must be aligned to their element size");
  gdn::RecArgs a = rec_args(d, q, k, v, log_alpha, beta, state_in, state_out, o);
  if (cu) {
    a.B = 1;
    a.cu_seqlens = cu;
    a.nseq = d->B;
  }
  return from_hip(gdn::launch_recurrent(a, d->io, static_cast<hipStream_t>(stream)),
                  "gdn_prefill (token-serial kernel)");
}

}  // namespace

namespace {

// Full-attention layer: checks shared by prefill and decode.
gdn_status check_attn(const gdn_attn_dims* d, bool decode) {
  if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
  if (d->B < 0 || d->T < 0) return fail(GDN_ERR_SHAPE, "B=%d T=%d must be >= 0", d->B, d->T);
  if (decode && d->T != 1) return fail(GDN_ERR_SHAPE, "decode needs T == 1 (got %d)", d->T);
  if (d->Hq < 1 || d->Hkv < 1 || d->Hq % d->Hkv)
    return fail(GDN_ERR_SHAPE, "Hq=%d must be a positive multiple of Hkv=%d", d->Hq, d->Hkv);
  if (decode && d->Hq / d->Hkv > 16)
    return fail(GDN_ERR_UNSUPPORTED, "decode takes at most 16 query heads per key/value head (got %d)",
                d->Hq / d->Hkv);
  if (d->D != 256) return fail(GDN_ERR_UNSUPPORTED, "head width D=%d: the kernels take 256", d->D);
  if (d->rot_dim < 0 || d->rot_dim > d->D || d->rot_dim % 8)
    return fail(GDN_ERR_SHAPE, "rot_dim=%d must be a multiple of 8 in [0, D]", d->rot_dim);
  if (d->S_max < 64 || d->S_max % 64) return fail(GDN_ERR_SHAPE, "S_max=%d must be a positive multiple of 64",
                                                  d->S_max);
  if (!decode && d->T > d->S_max) return fail(GDN_ERR_SHAPE, "T=%d exceeds S_max=%d", d->T, d->S_max);
  if (!(d->rope_theta > 0.0f) || !(d->norm_eps >= 0.0f) || !(d->scale > 0.0f) || std::isinf(d->scale))
    return fail(GDN_ERR_SHAPE, "rope_theta and scale must be > 0 (finite), norm_eps >= 0");
  const int64_t wq = 2LL * d->Hq * d->D, wkv = static_cast<int64_t>(d->Hkv) * d->D;
  if (d->stride_qg < wq || d->stride_k < wkv || d->stride_v < wkv || d->stride_o < wq / 2)
    return fail(GDN_ERR_SHAPE, "strides below the rows: qg %lld (>= %lld), k %lld, v %lld (>= %lld), o %lld (>= %lld)",
                (long long)d->stride_qg, (long long)wq, (long long)d->stride_k, (long long)d->stride_v,
                (long long)wkv, (long long)d->stride_o, (long long)(wq / 2));
  if ((d->stride_qg | d->stride_k | d->stride_v | d->stride_o) % 4)
    return fail(GDN_ERR_ALIGN, "strides must be multiples of 4 elements");
  return GDN_OK;
}

gdn::AttnArgs attn_args(const gdn_attn_dims* d, const void* qg, const void* k, const void* v, const void* qw,
                        const void* kw, void* kc, void* vc, void* o) {
  gdn::AttnArgs a{};
  a.B = d->B;
  a.T = d->T;
  a.Hq = d->Hq;
  a.Hkv = d->Hkv;
  a.rot_dim = d->rot_dim;
  a.S_max = d->S_max;
  a.theta = d->rope_theta;
  a.eps = d->norm_eps;
  a.scale = d->scale;
  a.sqg = d->stride_qg;
  a.sk = d->stride_k;
  a.sv = d->stride_v;
  a.so = d->stride_o;
  a.qg = static_cast<const uint16_t*>(qg);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.qw = static_cast<const uint16_t*>(qw);
  a.kw = static_cast<const uint16_t*>(kw);
  a.kc = static_cast<uint16_t*>(kc);
  a.vc = static_cast<uint16_t*>(vc);
  a.o = static_cast<uint16_t*>(o);
  return a;
}

gdn_status check_attn_pointers(const void* qg, const void* k, const void* v, const void* qw, const void* kw,
                               const void* kc, const void* vc, const void* o, const void* ws) {
  if (!qg || !k || !v || !qw || !kw || !kc || !vc || !o || !ws)
    return fail(GDN_ERR_NULL, "qg, k, v, the norm weights, both caches, o and the workspace are required");
  if (!aligned(qg, 8) || !aligned(k, 8) || !aligned(v, 8) || !aligned(qw, 8) || !aligned(kw, 8) || !aligned(o, 8))
    return fail(GDN_ERR_ALIGN, "qg, k, v, o and the norm weights must be 8-byte aligned");
  if (!aligned(kc, 16) || !aligned(vc, 16)) return fail(GDN_ERR_ALIGN, "the caches must be 16-byte aligned");
  if (!aligned(ws, 256)) return fail(GDN_ERR_ALIGN, "workspace must be 256-byte aligned");
  return GDN_OK;
}

size_t round256(size_t n) { return (n + 255) & ~size_t(255); }

size_t attn_qrot_bytes(const gdn_attn_dims* d) {
  return round256(static_cast<size_t>(d->B) * d->T * d->Hq * d->D * 2);
}

}  // namespace

extern "C" {

size_t gdn_prefill_workspace_size(const gdn_dims* d) { return workspace_size(d, nullptr); }

size_t gdn_prefill_varlen_workspace_size(const gdn_dims* d) { return workspace_size(d, kPackedMarker); }

gdn_status gdn_prefill(const gdn_dims* d, const void* q, const void* k, const void* v,
                       const float* log_alpha, const float* beta, const float* state_in,
                       float* state_out, void* o, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return prefill(d, nullptr, q, k, v, log_alpha, beta, state_in, state_out, o, workspace, workspace_bytes, stream);
}

gdn_status gdn_prefill_static(const gdn_dims* d, const void* q, const void* k, const void* v,
                              const float* log_alpha, const float* beta, const float* state_in, float* state_out,
                              void* o, void* stream) {
  gdn_status st = check_dims(d, false);
  if (st != GDN_OK) return st;
  if (d->B == 0) return ok();
  size_t need = 0;
  if (use_chunk_kernel(d)) {
    // the same smallest workspace gdn_prefill takes: one chunk per window (the whole call when it
    // has one chunk) and the state carry when there is no state_out
    const gdn::RecArgs a = chunk_args(d, nullptr, q, k, v, log_alpha, beta, state_in, state_out, o);
    const int64_t nchunks = gdn::chunk_count(a);
    need = gdn::chunk_ws_bytes_per_chunk(a) + ((nchunks > 1 && !state_out) ? gdn::chunk_ws_carry_bytes(a) : 0);
    if (need > kStaticScratchBytes)
      return fail(GDN_ERR_SHAPE, "gdn_prefill_static: these dims need at least %zu bytes of scratch, above its %zu",
                  need, kStaticScratchBytes);
  }
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) return from_hip(e, "gdn_prefill_static (scratch address)");
  }
  return prefill(d, nullptr, q, k, v, log_alpha, beta, state_in, state_out, o, ws, need > 0 ? kStaticScratchBytes : 0,
                 stream);
}

gdn_status gdn_prefill_gated(const gdn_dims* d, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, const float* state_in, float* state_out,
                             const void* z, int64_t stride_z, const void* norm_w, float norm_eps, void* y,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
  gdn_dims dd = *d;
  const bool force = (dd.flags & GDN_FLAG_NORM_IN_CHAIN) != 0;
  dd.flags &= ~GDN_FLAG_NORM_IN_CHAIN;
  gdn_status st = check_dims(&dd, false);
  if (st != GDN_OK) return st;
  if (dd.Dv != 64 && dd.Dv != 128) return fail(GDN_ERR_UNSUPPORTED, "the gated norm takes Dv in {64, 128}");
  const int64_t wv = static_cast<int64_t>(dd.Hv) * dd.Dv;
  if (stride_z < wv) return fail(GDN_ERR_SHAPE, "stride_z=%lld below Hv*Dv=%lld", (long long)stride_z, (long long)wv);
  if (!(norm_eps >= 0.0f)) return fail(GDN_ERR_SHAPE, "norm_eps must be >= 0");
  if (dd.B == 0) return ok();
  if (dd.T > 0) {
    if (!z || !norm_w || !y) return fail(GDN_ERR_NULL, "z, norm_w and y are required");
    if (!aligned(z, 16) || !aligned(norm_w, 16) || !aligned(y, 16))
      return fail(GDN_ERR_ALIGN, "z, norm_w and y must be 16-byte aligned");
    if ((stride_z % 8) || (dd.stride_o % 8)) return fail(GDN_ERR_ALIGN, "stride_z and stride_o must be multiples of 8");
  }
  // In the chain when the per-head grid fills the GPU (or when asked): otherwise the
  // prefill writes its outputs into y and the norm runs over y in place.
  const bool fused = use_chunk_kernel(&dd) && (force || static_cast<int64_t>(dd.B) * dd.Hv >= gdn::device_cu_count());
  if (fused) {
    const NormIn n{z, stride_z, norm_w, norm_eps};
    return prefill(&dd, nullptr, q, k, v, log_alpha, beta, state_in, state_out, y, workspace, workspace_bytes, stream,
                   &n);
  }
  st = prefill(&dd, nullptr, q, k, v, log_alpha, beta, state_in, state_out, y, workspace, workspace_bytes, stream);
  if (st != GDN_OK || dd.T == 0) return st;
  return gdn_gated_rmsnorm(static_cast<int64_t>(dd.B) * dd.T, dd.Hv, dd.Dv, dd.io, y, dd.stride_o, z, stride_z, norm_w,
                           norm_eps, y, dd.stride_o, stream);
}

gdn_status gdn_prefill_varlen(const gdn_dims* d, const int32_t* cu_seqlens, const void* q, const void* k,
                              const void* v, const float* log_alpha, const float* beta, const float* state_in,
                              float* state_out, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return fail(GDN_ERR_NULL, "cu_seqlens is required");
  if (!aligned(cu_seqlens, 4)) return fail(GDN_ERR_ALIGN, "cu_seqlens must be 4-byte aligned");
  return prefill(d, cu_seqlens, q, k, v, log_alpha, beta, state_in, state_out, o, workspace, workspace_bytes,
                 stream);
}

gdn_status gdn_decode_step(const gdn_dims* d, const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, float* state, void* o,
                           void* stream) {
  gdn_status st = check_dims(d, true);
  if (st != GDN_OK) return st;
  if (d->B == 0) return ok();
  if (!q || !k || !v || !log_alpha || !beta || !state || !o)
    return fail(GDN_ERR_NULL, "q, k, v, log_alpha, beta, state and o are required");
  if (!aligned(state, 16)) return fail(GDN_ERR_ALIGN, "state must be 16-byte aligned");
  const size_t es = d->io == GDN_BF16 ? 2 : 4;
  if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(o, es))
    return fail(GDN_ERR_ALIGN, "q, k, v, o must be aligned to their element size");
  return from_hip(gdn::launch_recurrent(rec_args(d, q, k, v, log_alpha, beta, state, state, o), d->io,
                                        static_cast<hipStream_t>(stream)),
                  "gdn_decode_step");
}

namespace {
gdn_status conv1d_silu(int32_t B, int32_t T, int32_t C, int32_t K, int32_t dtype, const void* x, int64_t stride_x,
                       const void* w, const void* conv_state_in, void* conv_state_out, void* y, int64_t stride_y,
                       int32_t l2_channels, float l2_eps, const char* what, void* stream) {
  if (B < 0 || T < 0 || C < 1) return fail(GDN_ERR_SHAPE, "B=%d T=%d C=%d", B, T, C);
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_SHAPE, "dtype %d unknown", dtype);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "conv kernel width K=%d: only K=4 is implemented", K);
  if (C % 8) return fail(GDN_ERR_UNSUPPORTED, "C=%d must be a multiple of 8", C);
  if (stride_x < C || stride_y < C) return fail(GDN_ERR_SHAPE, "strides must be >= C");
  if (B == 0 || (T == 0 && !conv_state_out)) return ok();
  if (!w || (T > 0 && (!x || !y))) return fail(GDN_ERR_NULL, "x, w and y are required");
  if (conv_state_in && conv_state_in == conv_state_out)
    return fail(GDN_ERR_SHAPE, "conv_state_out must not alias conv_state_in");
  const size_t vec = 16;
  if ((x && !aligned(x, vec)) || (y && !aligned(y, vec)))
    return fail(GDN_ERR_ALIGN, "x and y must be 16-byte aligned");
  if ((stride_x % 8) || (stride_y % 8)) return fail(GDN_ERR_ALIGN, "strides must be multiples of 8");
  gdn::ConvArgs a;
  a.B = B;
  a.T = T;
  a.C = C;
  a.K = K;
  a.sx = stride_x;
  a.sy = stride_y;
  a.x = x;
  a.w = w;
  a.cs_in = conv_state_in;
  a.cs_out = conv_state_out;
  a.y = y;
  a.l2c = l2_channels;
  a.l2_eps = l2_eps;
  return from_hip(gdn::launch_conv1d_silu(a, dtype, static_cast<hipStream_t>(stream)), what);
}
}  // namespace

gdn_status gdn_conv1d_silu(int32_t B, int32_t T, int32_t C, int32_t K, int32_t dtype, const void* x,
                           int64_t stride_x, const void* w, const void* conv_state_in,
                           void* conv_state_out, void* y, int64_t stride_y, void* stream) {
  return conv1d_silu(B, T, C, K, dtype, x, stride_x, w, conv_state_in, conv_state_out, y, stride_y, 0, 0.f,
                     "gdn_conv1d_silu", stream);
}

gdn_status gdn_conv1d_silu_l2(int32_t B, int32_t T, int32_t C, int32_t K, int32_t dtype, const void* x,
                              int64_t stride_x, const void* w, const void* conv_state_in, void* conv_state_out,
                              void* y, int64_t stride_y, int32_t l2_channels, float l2_eps, void* stream) {
  if (l2_channels < 0 || l2_channels % 128 || l2_channels > C)
    return fail(GDN_ERR_SHAPE, "l2_channels=%d must be a multiple of 128 in [0, C=%d]", l2_channels, C);
  if (l2_channels > 0 && C % 128)
    return fail(GDN_ERR_UNSUPPORTED, "C=%d must be a multiple of 128 with l2_channels", C);
  if (!(l2_eps >= 0.0f)) return fail(GDN_ERR_SHAPE, "l2_eps must be >= 0");
  return conv1d_silu(B, T, C, K, dtype, x, stride_x, w, conv_state_in, conv_state_out, y, stride_y, l2_channels,
                     l2_eps, "gdn_conv1d_silu_l2", stream);
}

gdn_status gdn_gated_rmsnorm(int64_t n_tok, int32_t H, int32_t D, int32_t dtype, const void* x,
                             int64_t stride_x, const void* z, int64_t stride_z, const void* w, float eps,
                             void* y, int64_t stride_y, void* stream) {
  if (n_tok < 0 || H < 1) return fail(GDN_ERR_SHAPE, "n_tok=%lld H=%d", (long long)n_tok, H);
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_SHAPE, "dtype %d unknown", dtype);
  if (D != 64 && D != 128) return fail(GDN_ERR_UNSUPPORTED, "D=%d: only 64 and 128 are implemented", D);
  const int64_t wd = static_cast<int64_t>(H) * D;
  if (stride_x < wd || stride_z < wd || stride_y < wd) return fail(GDN_ERR_SHAPE, "strides must be >= H*D");
  if (!(eps >= 0.0f)) return fail(GDN_ERR_SHAPE, "eps must be >= 0");
  if (n_tok == 0) return ok();
  if (!x || !z || !w || !y) return fail(GDN_ERR_NULL, "x, z, w and y are required");
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(w, 16) || !aligned(y, 16))
    return fail(GDN_ERR_ALIGN, "x, z, w, y must be 16-byte aligned");
  if ((stride_x % 8) || (stride_z % 8) || (stride_y % 8))
    return fail(GDN_ERR_ALIGN, "strides must be multiples of 8");
  gdn::NormArgs a;
  a.n_tok = n_tok;
  a.H = H;
  a.D = D;
  a.sx = stride_x;
  a.sz = stride_z;
  a.sy = stride_y;
  a.x = x;
  a.z = z;
  a.w = w;
  a.eps = eps;
  a.y = y;
  return from_hip(gdn::launch_gated_rmsnorm(a, dtype, static_cast<hipStream_t>(stream)), "gdn_gated_rmsnorm");
}

gdn_status gdn_gates(int64_t n_tok, int32_t Hv, int32_t dtype, const void* ba, int64_t stride_ba,
                     const float* A_log, const float* dt_bias, float* log_alpha, float* beta, void* stream) {
  if (n_tok < 0 || Hv < 1) return fail(GDN_ERR_SHAPE, "n_tok=%lld Hv=%d", (long long)n_tok, Hv);
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_SHAPE, "dtype %d unknown", dtype);
  if (stride_ba < 2 * static_cast<int64_t>(Hv))
    return fail(GDN_ERR_SHAPE, "stride_ba=%lld below 2*Hv=%d", (long long)stride_ba, 2 * Hv);
  if (n_tok == 0) return ok();
  if (!ba || !A_log || !dt_bias || !log_alpha || !beta)
    return fail(GDN_ERR_NULL, "ba, A_log, dt_bias, log_alpha and beta are required");
  if (!aligned(ba, dtype == GDN_BF16 ? 2 : 4) || !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
      !aligned(log_alpha, 4) || !aligned(beta, 4))
    return fail(GDN_ERR_ALIGN, "pointers must be aligned to their element size");
  gdn::GateArgs a;
  a.n_tok = n_tok;
  a.Hv = Hv;
  a.sba = stride_ba;
  a.ba = ba;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.la = log_alpha;
  a.beta = beta;
  return from_hip(gdn::launch_gates(a, dtype, static_cast<hipStream_t>(stream)), "gdn_gates");
}

gdn_status gdn_decode_token(const gdn_dims* d, const void* q, const void* k, const void* v, int32_t ba_dtype,
                            const void* ba, int64_t stride_ba, const float* A_log, const float* dt_bias,
                            float* state_pool, int32_t n_slots, const int32_t* slots, void* o, void* stream) {
  gdn_status st = check_dims(d, true);
  if (st != GDN_OK) return st;
  if (ba_dtype != GDN_F32 && ba_dtype != GDN_BF16) return fail(GDN_ERR_SHAPE, "ba dtype %d unknown", ba_dtype);
  if (stride_ba < 2 * static_cast<int64_t>(d->Hv))
    return fail(GDN_ERR_SHAPE, "stride_ba=%lld below 2*Hv=%d", (long long)stride_ba, 2 * d->Hv);
  if (n_slots < 0 || (!slots && n_slots < d->B))
    return fail(GDN_ERR_SHAPE, "n_slots=%d: the pool needs >= 0 entries, and >= B=%d without slots", n_slots, d->B);
  if (d->B == 0) return ok();
  if (!q || !k || !v || !ba || !A_log || !dt_bias || !state_pool || !o)
    return fail(GDN_ERR_NULL, "q, k, v, ba, A_log, dt_bias, state_pool and o are required");
  if (!aligned(state_pool, 16)) return fail(GDN_ERR_ALIGN, "state_pool must be 16-byte aligned");
  const size_t es = d->io == GDN_BF16 ? 2 : 4;
  if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(o, es) ||
      !aligned(ba, ba_dtype == GDN_BF16 ? 2 : 4) || !aligned(A_log, 4) || !aligned(dt_bias, 4) ||
      !aligned(slots, 4))
    return fail(GDN_ERR_ALIGN, "pointers must be aligned to their element size");
  gdn::RecArgs a = rec_args(d, q, k, v, nullptr, nullptr, state_pool, state_pool, o);
  a.ba = ba;
  a.sba = stride_ba;
  a.ba_io = ba_dtype;
  a.A_log = A_log;
  a.dt_bias = dt_bias;
  a.slots = slots;
  a.nslots = n_slots;
  return from_hip(gdn::launch_recurrent(a, d->io, static_cast<hipStream_t>(stream)), "gdn_decode_token");
}

gdn_status gdn_decode_layer(const gdn_decode_layer_args* p, void* stream) {
  if (!p) return fail(GDN_ERR_NULL, "args is NULL");
  if (p->B < 0 || p->Hk < 1 || p->Hv < 1 || p->Hv % p->Hk)
    return fail(GDN_ERR_SHAPE, "B=%d Hk=%d Hv=%d (Hv must be a multiple of Hk)", p->B, p->Hk, p->Hv);
  if (p->D != 128) return fail(GDN_ERR_UNSUPPORTED, "D=%d: the fused decode layer takes D=128", p->D);
  if (p->flags & ~static_cast<uint32_t>(GDN_FLAG_QK_L2NORM))
    return fail(GDN_ERR_SHAPE, "flags 0x%x: only GDN_FLAG_QK_L2NORM applies", p->flags);
  if (!(p->l2_eps >= 0.0f) || !(p->norm_eps >= 0.0f)) return fail(GDN_ERR_SHAPE, "eps values must be >= 0");
  if (p->n_slots < 0 || (!p->slots && p->n_slots < p->B))
    return fail(GDN_ERR_SHAPE, "n_slots=%d: the pools need >= 0 entries, and >= B=%d without slots", p->n_slots,
                p->B);
  const int64_t C = static_cast<int64_t>(2 * p->Hk + p->Hv) * p->D, W = static_cast<int64_t>(p->Hv) * p->D;
  if (p->stride_x < C || p->stride_ba < 2 * static_cast<int64_t>(p->Hv) || p->stride_z < W || p->stride_out < W ||
      (p->o && p->stride_o < W))
    return fail(GDN_ERR_SHAPE, "row strides below the row widths (x %lld, ba %d, z/out/o %lld)", (long long)C,
                2 * p->Hv, (long long)W);
  if (p->B == 0) return ok();
  if (!p->x || !p->conv_w || !p->conv_state_in || !p->conv_state_out || !p->ba || !p->A_log || !p->dt_bias ||
      !p->state_pool || !p->z || !p->norm_w || !p->out)
    return fail(GDN_ERR_NULL, "x, conv_w, conv states, ba, A_log, dt_bias, state_pool, z, norm_w, out are required");
  if (p->conv_state_in == p->conv_state_out) return fail(GDN_ERR_SHAPE, "conv_state_out must not alias conv_state_in");
  if (!aligned(p->x, 4) || (p->stride_x % 2) || !aligned(p->conv_w, 16) || !aligned(p->conv_state_in, 4) ||
      !aligned(p->conv_state_out, 4) || !aligned(p->ba, 2) || !aligned(p->A_log, 4) || !aligned(p->dt_bias, 4) ||
      !aligned(p->state_pool, 16) || !aligned(p->slots, 4) || !aligned(p->z, 2) || !aligned(p->norm_w, 2) ||
      !aligned(p->out, 2) || !aligned(p->o, 2))
    return fail(GDN_ERR_ALIGN, "alignment: state_pool and conv_w 16 bytes, x and the conv states 4 bytes "
                               "(stride_x even), the rest their element size");
  gdn::LayerArgs a;
  a.B = p->B;
  a.Hk = p->Hk;
  a.Hv = p->Hv;
  a.G = p->Hv / p->Hk;
  a.flags = p->flags;
  a.q_scale = p->q_scale;
  a.l2_eps = p->l2_eps;
  a.norm_eps = p->norm_eps;
  a.x = static_cast<const uint16_t*>(p->x);
  a.sx = p->stride_x;
  a.conv_w = static_cast<const uint16_t*>(p->conv_w);
  a.cs_in = static_cast<const uint16_t*>(p->conv_state_in);
  a.cs_out = static_cast<uint16_t*>(p->conv_state_out);
  a.ba = static_cast<const uint16_t*>(p->ba);
  a.sba = p->stride_ba;
  a.A_log = p->A_log;
  a.dt_bias = p->dt_bias;
  a.pool = p->state_pool;
  a.slots = p->slots;
  a.nslots = p->n_slots;
  a.z = static_cast<const uint16_t*>(p->z);
  a.sz = p->stride_z;
  a.norm_w = static_cast<const uint16_t*>(p->norm_w);
  a.out = static_cast<uint16_t*>(p->out);
  a.sout = p->stride_out;
  a.o = static_cast<uint16_t*>(p->o);
  a.so = p->stride_o;
  return from_hip(gdn::launch_decode_layer(a, static_cast<hipStream_t>(stream)), "gdn_decode_layer");
}

size_t gdn_attn_prefill_workspace_size(const gdn_attn_dims* d) {
  if (check_attn(d, false) != GDN_OK) return 0;
  return attn_qrot_bytes(d);
}

gdn_status gdn_attn_prefill(const gdn_attn_dims* d, const void* qg, const void* k, const void* v,
                            const void* q_norm_w, const void* k_norm_w, void* k_cache, void* v_cache, void* o,
                            void* workspace, size_t workspace_bytes, void* stream) {
  gdn_status st = check_attn(d, false);
  if (st != GDN_OK) return st;
  if (d->B == 0 || d->T == 0) return ok();
  st = check_attn_pointers(qg, k, v, q_norm_w, k_norm_w, k_cache, v_cache, o, workspace);
  if (st != GDN_OK) return st;
  if (workspace_bytes < attn_qrot_bytes(d))
    return fail(GDN_ERR_SHAPE, "workspace of %zu bytes is below %zu", workspace_bytes, attn_qrot_bytes(d));
  gdn::AttnArgs a = attn_args(d, qg, k, v, q_norm_w, k_norm_w, k_cache, v_cache, o);
  a.qrot = static_cast<uint16_t*>(workspace);
  return from_hip(gdn::launch_attn_prefill(a, static_cast<hipStream_t>(stream)), "gdn_attn_prefill");
}

size_t gdn_attn_decode_workspace_size(const gdn_attn_dims* d) {
  if (check_attn(d, true) != GDN_OK) return 0;
  return attn_qrot_bytes(d) + static_cast<size_t>(d->B) * d->Hq * gdn::attn_splits(d->S_max) *
                                  gdn::kAttnPartFloats * sizeof(float);
}

gdn_status gdn_attn_decode(const gdn_attn_dims* d, const void* qg, const void* k, const void* v,
                           const void* q_norm_w, const void* k_norm_w, const int32_t* cache_len, void* k_cache,
                           void* v_cache, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  gdn_status st = check_attn(d, true);
  if (st != GDN_OK) return st;
  if (d->B == 0) return ok();
  st = check_attn_pointers(qg, k, v, q_norm_w, k_norm_w, k_cache, v_cache, o, workspace);
  if (st != GDN_OK) return st;
  if (!cache_len) return fail(GDN_ERR_NULL, "cache_len is required");
  if (!aligned(cache_len, 4)) return fail(GDN_ERR_ALIGN, "cache_len must be 4-byte aligned");
  const size_t need = gdn_attn_decode_workspace_size(d);
  if (workspace_bytes < need) return fail(GDN_ERR_SHAPE, "workspace of %zu bytes is below %zu", workspace_bytes, need);
  gdn::AttnArgs a = attn_args(d, qg, k, v, q_norm_w, k_norm_w, k_cache, v_cache, o);
  a.cache_len = cache_len;
  a.qrot = static_cast<uint16_t*>(workspace);
  a.part = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + attn_qrot_bytes(d));
  return from_hip(gdn::launch_attn_decode(a, static_cast<hipStream_t>(stream)), "gdn_attn_decode");
}

gdn_status gdn_probe_mfma(int32_t n_workgroups, int32_t iters, float* sink, void* stream) {
  if (n_workgroups < 1 || n_workgroups > (1 << 20) || iters < 4 || iters > 65536 || iters % 4)
    return fail(GDN_ERR_SHAPE, "n_workgroups=%d must be in [1, 2^20] and iters=%d a multiple of 4 in [4, 65536]",
                n_workgroups, iters);
  if (!sink) return fail(GDN_ERR_NULL, "sink is required");
  if (!aligned(sink, 4)) return fail(GDN_ERR_ALIGN, "sink must be 4-byte aligned");
  return from_hip(gdn::launch_probe_mfma(n_workgroups, iters, sink, static_cast<hipStream_t>(stream)),
                  "gdn_probe_mfma");
}

gdn_status gdn_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % gdn::kProbeCopyBlockBytes || bytes >= (static_cast<size_t>(1) << 46))
    return fail(GDN_ERR_SHAPE, "bytes=%zu must be a multiple of %zu below 2^46", bytes, gdn::kProbeCopyBlockBytes);
  if (bytes == 0) return ok();
  if (!src || !dst) return fail(GDN_ERR_NULL, "src and dst are required");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(GDN_ERR_ALIGN, "src and dst must be 16-byte aligned");
  const unsigned char* s0 = static_cast<const unsigned char*>(src);
  const unsigned char* d0 = static_cast<const unsigned char*>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(GDN_ERR_SHAPE, "src and dst overlap");
  return from_hip(gdn::launch_probe_copy(src, dst, bytes, static_cast<hipStream_t>(stream)), "gdn_probe_copy");
}

const char* gdn_last_error(void) { return g_err; }

int32_t gdn_version(void) { return 200; /* 0.2.0 */ }

}  // extern "C"
