// gdn_conv_norm.hip -- the HBM-bound front and back ends of the mixer.
//
// conv1d_silu: depthwise causal conv, 4 taps per channel, no bias, then SiLU
// ("L'attention hybride", table "Le decompte": kernel 4 over the q|k|v
// channels, 4 weights per channel; "Les briques d'un reseau de neurones",
// section 2: SiLU(x) = x sigmoid(x)).  Each thread owns 8 adjacent channels
// and a run of TT tokens, slides a 4-token window in registers, and reads x
// and writes y once with 16-byte accesses (a wave covers 512 consecutive
// channels of one token).  Only the 3 halo tokens before a run are re-read.
// Optionally the q and k channels are L2-normalised per 128-channel head in the
// same pass (the per-head normalisation the prefill otherwise applies as it
// loads q and k), before the one rounding of y.
//
// gated_rmsnorm: y = x / sqrt(mean(x^2) + eps) * w * z * sigmoid(z) per
// D-row ("Les briques", section 4; "L'attention hybride", swish output gate
// and one 128-weight norm shared by the heads).  D/8 lanes own one row, 8
// elements each, and reduce the sum of squares with lane shuffles.
//
// gates: beta and log alpha of every (token, value head) from the raw
// in_proj_ba outputs ("L'attention hybride", table "Le decompte": one beta and
// one alpha per value head, beta first), one element per thread.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvTT = 64;  // tokens per thread

template <typename IO>
struct Vec8;

template <>
struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const void* p, int64_t i, float (&x)[8]) {
    const u16x8 v = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bf16_bits_to_f32(v[e]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, const float (&x)[8]) {
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16_bits(x[e]);
    *reinterpret_cast<u16x8*>(static_cast<uint16_t*>(p) + i) = v;
  }
};

template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const void* p, int64_t i, float (&x)[8]) {
    const floatx4* q = reinterpret_cast<const floatx4*>(static_cast<const float*>(p) + i);
    const floatx4 a = q[0], b = q[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[e + 4] = b[e];
    }
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, const float (&x)[8]) {
    floatx4* q = reinterpret_cast<floatx4*>(static_cast<float*>(p) + i);
    q[0] = floatx4{x[0], x[1], x[2], x[3]};
    q[1] = floatx4{x[4], x[5], x[6], x[7]};
  }
};

template <typename IO>
__global__ __launch_bounds__(kConvThreads) void conv1d_silu_kernel(ConvArgs a) {
  constexpr int K = 4;
  const int c8 = (blockIdx.x * kConvThreads + threadIdx.x) * 8;
  if (c8 >= a.C) return;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * kConvTT;
  const int t1 = min(t0 + kConvTT, a.T);

  float w[8][K];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < K; ++j) w[e][j] = IoTraits<IO>::load(a.w, static_cast<int64_t>(c8 + e) * K + j);

  const int64_t xb = static_cast<int64_t>(b) * a.T * a.sx;
  const int64_t yb = static_cast<int64_t>(b) * a.T * a.sy;
  // win[j] holds x at token t-(K-1)+j for the token about to be produced.
  float win[K - 1][8];
#pragma unroll
  for (int j = 0; j < K - 1; ++j) {
    const int ts = t0 - (K - 1) + j;
    if (ts >= 0) {
      Vec8<IO>::load(a.x, xb + static_cast<int64_t>(ts) * a.sx + c8, win[j]);
    } else if (a.cs_in) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        win[j][e] = IoTraits<IO>::load(a.cs_in, (static_cast<int64_t>(b) * a.C + c8 + e) * (K - 1) + (K - 1) + ts);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
    }
  }
  for (int t = t0; t < t1; ++t) {
    float xt[8], y[8];
    Vec8<IO>::load(a.x, xb + static_cast<int64_t>(t) * a.sx + c8, xt);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = w[e][0] * win[0][e];
#pragma unroll
      for (int j = 1; j < K - 1; ++j) acc = fmaf(w[e][j], win[j][e], acc);
      acc = fmaf(w[e][K - 1], xt[e], acc);
      y[e] = acc * sigmoidf_(acc);
    }
    if (c8 < a.l2c) {
      // the head's 128 channels are the 16 lanes of this lane's row (16-lane rows start at
      // multiples of 128 channels, and so do l2c and C), all of them here
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
      const float inv = rsqrtf(row16_sum(ss) + a.l2_eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= inv;
    }
    Vec8<IO>::store(a.y, yb + static_cast<int64_t>(t) * a.sy + c8, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int j = 0; j < K - 2; ++j) win[j][e] = win[j + 1][e];
      win[K - 2][e] = xt[e];
    }
  }
  // The run that ends the sequence hands its window on (the last K-1 inputs).
  if (a.cs_out && t1 == a.T) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int j = 0; j < K - 1; ++j)
        IoTraits<IO>::store(a.cs_out, (static_cast<int64_t>(b) * a.C + c8 + e) * (K - 1) + j, win[j][e]);
  }
}

template <typename IO, int D>
__global__ __launch_bounds__(256) void gated_rmsnorm_kernel(NormArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  constexpr int RPB = 256 / LPR;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int64_t rows = a.n_tok * a.H;
  const int sub = threadIdx.x % LPR;
  const bool live = row < rows;
  const int64_t t = live ? row / a.H : 0;
  const int h = live ? static_cast<int>(row - t * a.H) : 0;
  const int c = sub * 8;
  float x[8], z[8], w[8];
  if (live) {
    Vec8<IO>::load(a.x, t * a.sx + static_cast<int64_t>(h) * D + c, x);
    Vec8<IO>::load(a.z, t * a.sz + static_cast<int64_t>(h) * D + c, z);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = z[e] = 0.f;
  }
  Vec8<IO>::load(a.w, c, w);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
  const float inv = rsqrtf(ss * (1.0f / D) + a.eps);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = x[e] * inv * w[e] * z[e] * sigmoidf_(z[e]);
  if (live) Vec8<IO>::store(a.y, t * a.sy + static_cast<int64_t>(h) * D + c, y);
}

template <typename IO>
__global__ __launch_bounds__(256) void gates_kernel(GateArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= a.n_tok * a.Hv) return;
  const int64_t t = i / a.Hv;
  const int h = static_cast<int>(i - t * a.Hv);
  float la, be;
  gate_activation(IoTraits<IO>::load(a.ba, t * a.sba + h), IoTraits<IO>::load(a.ba, t * a.sba + a.Hv + h),
                  a.A_log[h], a.dt_bias[h], la, be);
  a.la[i] = la;
  a.beta[i] = be;
}

}  // namespace

hipError_t launch_gates(const GateArgs& a, int io, hipStream_t s) {
  const int64_t n = a.n_tok * a.Hv;
  if (n == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (io == 1)
    hipLaunchKernelGGL(gates_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gates_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_conv1d_silu(const ConvArgs& a, int io, hipStream_t s) {
  const int groups = (a.C + 7) / 8;
  // T == 0 still runs one (empty) token run per channel group to hand the window on.
  const dim3 grid((groups + kConvThreads - 1) / kConvThreads, max(1, (a.T + kConvTT - 1) / kConvTT), a.B);
  if (io == 1)
    hipLaunchKernelGGL(conv1d_silu_kernel<uint16_t>, grid, dim3(kConvThreads), 0, s, a);
  else
    hipLaunchKernelGGL(conv1d_silu_kernel<float>, grid, dim3(kConvThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gated_rmsnorm(const NormArgs& a, int io, hipStream_t s) {
  const int64_t rows = a.n_tok * a.H;
  const int rpb = 256 / (a.D / 8);
  const int64_t nb = (rows + rpb - 1) / rpb;
  if (nb == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nb));
  if (io == 1) {
    if (a.D == 128) hipLaunchKernelGGL((gated_rmsnorm_kernel<uint16_t, 128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gated_rmsnorm_kernel<uint16_t, 64>), grid, dim3(256), 0, s, a);
  } else {
    if (a.D == 128) hipLaunchKernelGGL((gated_rmsnorm_kernel<float, 128>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((gated_rmsnorm_kernel<float, 64>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
