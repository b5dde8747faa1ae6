// gdn_recurrent.hip -- token-serial gated delta rule on gfx950.
//
// One workgroup owns one (sequence b, value head h) state M = S^T ([D][D]
// fp32, row = key coordinate, column = value coordinate) for the whole call:
// it is read from HBM once, kept in VGPRs across all tokens, and written back
// once.  Per token ("L'attention hybride", section "La recurrence"; course
// page "Chapitre 16", 16.3 -- decode reads the fixed state, emits the output
// and updates the state):
//     u = M^T k,  w = M^T q                      (one pass over M)
//     d = beta (v - alpha u)
//     M <- alpha M + k d^T
//     o = alpha w + (k . q) d                    (= M'^T q, read after update)
// This is the decode-step kernel (T = 1: one HBM read and one HBM write of the
// 64 KiB state, 128-bit coalesced, both non-temporal since every byte is used
// once per call) and the prefill kernel for shapes the
// chunked MFMA kernel does not take (fp32 I/O, head widths 16..64).  It can
// form the gates from raw in_proj_ba outputs and address its state through a
// slot table into a pool (the serving decode token).  decode_layer_kernel
// below fuses a whole layer's decode token: conv window, L2 norm, gates, this
// update and the gated output norm.
//
// Thread layout: TPR = D/4 threads cover one row of M with a float4 each;
// RG = NT/TPR row groups take rows rg, rg+RG, ... so that one wave's loads
// cover whole consecutive rows.  Column partial sums over a thread's rows are
// reduced across the RG groups through LDS.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int D, int NTH = 256>
struct RecShape {
  static constexpr int NT = (D * D / 4 < NTH) ? D * D / 4 : NTH;
  static constexpr int TPR = D / 4;
  static constexpr int RG = NT / TPR;
  static constexpr int RPT = D / RG;
  static_assert(RG * RPT == D, "row split");
  static_assert(NT % 64 == 0, "whole waves");
};

template <int D, typename IO, int NTH>
__global__ __launch_bounds__((RecShape<D, NTH>::NT)) void recurrent_kernel(RecArgs a) {
  using S = RecShape<D, NTH>;
  constexpr int RG = S::RG, RPT = S::RPT, TPR = S::TPR;
  constexpr int QPL = (D + 63) / 64;  // q/k elements per lane in the staging wave

  __shared__ float s_q[D];
  __shared__ float s_k[D];
  __shared__ float s_red[2][RG][D];
  __shared__ float s_uw[2][D];
  __shared__ float s_scal[4];

  const int bh = blockIdx.x;
  const int b = bh / a.Hv, h = bh - b * a.Hv, hk = h / a.G;
  const int tid = threadIdx.x;
  const int cg = tid % TPR, rg = tid / TPR;
  const int c0 = cg * 4;
  // state entry of this (sequence, head): its own, or pool slot slots[b]
  int64_t sidx = bh;
  if (a.slots) {
    const int slot = a.slots[b];
    if (slot < 0 || slot >= a.nslots) return;  // the whole workgroup skips the row
    sidx = static_cast<int64_t>(slot) * a.Hv + h;
  }

  floatx4 M[RPT];
  if (a.state_in) {
    const float* sp = a.state_in + sidx * D * D;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      M[r] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(sp + (rg + RG * r) * D + c0));
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) M[r] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // tokens of this sequence: [b*T, b*T + T), or its packed range
  int64_t tbase = static_cast<int64_t>(b) * a.T;
  int ntok = a.T;
  if (a.cu_seqlens) packed_range(a.cu_seqlens, b, a.T, tbase, ntok);
  for (int t = 0; t < ntok; ++t) {
    const int64_t tok = tbase + t;
    if (tid < 64) {
      float qv[QPL], kv[QPL];
      float sqq = 0.f, skk = 0.f, sqk = 0.f;
#pragma unroll
      for (int e = 0; e < QPL; ++e) {
        const int i = tid + 64 * e;
        qv[e] = (i < D) ? IoTraits<IO>::load(a.q, tok * a.sq + hk * D + i) : 0.f;
        kv[e] = (i < D) ? IoTraits<IO>::load(a.k, tok * a.sk + hk * D + i) : 0.f;
        sqq += qv[e] * qv[e];
        skk += kv[e] * kv[e];
        sqk += qv[e] * kv[e];
      }
      sqq = wave_sum(sqq);
      skk = wave_sum(skk);
      sqk = wave_sum(sqk);
      float rq = 1.f, rk = 1.f;
      if (a.flags & 1u) {
        rq = rsqrtf(sqq + a.l2_eps);
        rk = rsqrtf(skk + a.l2_eps);
      }
      rq *= a.q_scale;
#pragma unroll
      for (int e = 0; e < QPL; ++e) {
        const int i = tid + 64 * e;
        if (i < D) {
          s_q[i] = qv[e] * rq;
          s_k[i] = kv[e] * rk;
        }
      }
      if (tid == 0) {
        s_scal[0] = sqk * rq * rk;  // (k^ . q^)
        if (a.ba) {
          float la, be;
          const int64_t r = tok * a.sba;
          if (a.ba_io == 1)
            gate_activation(IoTraits<uint16_t>::load(a.ba, r + h), IoTraits<uint16_t>::load(a.ba, r + a.Hv + h),
                            a.A_log[h], a.dt_bias[h], la, be);
          else
            gate_activation(IoTraits<float>::load(a.ba, r + h), IoTraits<float>::load(a.ba, r + a.Hv + h),
                            a.A_log[h], a.dt_bias[h], la, be);
          s_scal[1] = __expf(la);
          s_scal[2] = be;
        } else {
          s_scal[1] = __expf(a.la[tok * a.Hv + h]);
          s_scal[2] = a.beta[tok * a.Hv + h];
        }
      }
    }
    __syncthreads();

    floatx4 pu = {0.f, 0.f, 0.f, 0.f}, pw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int i = rg + RG * r;
      pu += M[r] * s_k[i];
      pw += M[r] * s_q[i];
    }
    *reinterpret_cast<floatx4*>(&s_red[0][rg][c0]) = pu;
    *reinterpret_cast<floatx4*>(&s_red[1][rg][c0]) = pw;
    __syncthreads();

    floatx4 u = {0.f, 0.f, 0.f, 0.f}, w = {0.f, 0.f, 0.f, 0.f};
    if constexpr (RG <= 8) {
      // few row groups: every thread sums all of them for its columns
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        u += *reinterpret_cast<const floatx4*>(&s_red[0][g][c0]);
        w += *reinterpret_cast<const floatx4*>(&s_red[1][g][c0]);
      }
    } else {
      // many row groups: groups 0 and 1 sum u and w once, the rest read them
      if (rg < 2) {
        floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < RG; ++g) t += *reinterpret_cast<const floatx4*>(&s_red[rg][g][c0]);
        *reinterpret_cast<floatx4*>(&s_uw[rg][c0]) = t;
      }
      __syncthreads();
      u = *reinterpret_cast<const floatx4*>(&s_uw[0][c0]);
      w = *reinterpret_cast<const floatx4*>(&s_uw[1][c0]);
    }
    const float kq = s_scal[0], alpha = s_scal[1], beta = s_scal[2];
    floatx4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = IoTraits<IO>::load(a.v, tok * a.sv + h * D + c0 + e);
    const floatx4 d = beta * (vv - alpha * u);
    if (rg == 0) {
      const floatx4 o = alpha * w + kq * d;
#pragma unroll
      for (int e = 0; e < 4; ++e) IoTraits<IO>::store(a.o, tok * a.so + h * D + c0 + e, o[e]);
    }
#pragma unroll
    for (int r = 0; r < RPT; ++r) M[r] = alpha * M[r] + s_k[rg + RG * r] * d;
    __syncthreads();  // s_q, s_k, s_red, s_scal are rewritten by the next token
  }

  if (a.state_out) {
    float* sp = a.state_out + sidx * D * D;
#pragma unroll
    for (int r = 0; r < RPT; ++r) __builtin_nontemporal_store(M[r], reinterpret_cast<floatx4*>(sp + (rg + RG * r) * D + c0));
  }
}

// ---------------------------------------------------------------------------
// One decode token of the layer, fused: the conv window, L2 norm, gates, the
// recurrence and the output norm of one (sequence, value head) in one
// workgroup.  The channels of a token are q (Hk*128) | k (Hk*128) | v (Hv*128)
// ("L'attention hybride", table "Le decompte": the conv runs over those
// channels).  Conv: y = silu(w0 s0 + w1 s1 + w2 s2 + w3 x) with s the window
// of the three previous inputs, and the window moves on to (s1, s2, x); the
// key head's q and k windows are written by the first of its value heads only.
// Output: y = o / sqrt(mean(o^2) + eps) * w * z * sigmoid(z) over the 128
// outputs of the head ("Les briques", section 4; swish output gate).
// Two adjacent channels c, c+1 (c even) of one token: their 4 weights each
// (16 bytes), the two inputs (4 bytes) and their windows (12 bytes, oldest
// first), loaded as whole words.  conv_finish forms silu(w . (s0, s1, s2, x))
// and, when `keep`, stores the moved windows (s1, s2, x).
struct ConvPair {
  u16x8 w;
  uint32_t x;
  uint32_t s[3];
};

__device__ __forceinline__ ConvPair conv_load(const LayerArgs& a, int64_t crow, int64_t xrow, int c) {
  ConvPair p;
  p.w = *reinterpret_cast<const u16x8*>(a.conv_w + static_cast<int64_t>(c) * 4);
  p.x = *reinterpret_cast<const uint32_t*>(a.x + xrow + c);
  const uint32_t* sp = reinterpret_cast<const uint32_t*>(a.cs_in + (crow + c) * 3);
  p.s[0] = sp[0];
  p.s[1] = sp[1];
  p.s[2] = sp[2];
  return p;
}

__device__ __forceinline__ void conv_finish(const LayerArgs& a, const ConvPair& p, int64_t crow, int c, bool keep,
                                            float& y0, float& y1) {
  // window halfwords: channel c = (h0, h1, h2), channel c+1 = (h3, h4, h5)
  const uint16_t h[6] = {static_cast<uint16_t>(p.s[0]), static_cast<uint16_t>(p.s[0] >> 16),
                         static_cast<uint16_t>(p.s[1]), static_cast<uint16_t>(p.s[1] >> 16),
                         static_cast<uint16_t>(p.s[2]), static_cast<uint16_t>(p.s[2] >> 16)};
  const uint16_t x0 = static_cast<uint16_t>(p.x), x1 = static_cast<uint16_t>(p.x >> 16);
  const float a0 = bf16_bits_to_f32(p.w[0]) * bf16_bits_to_f32(h[0]) + bf16_bits_to_f32(p.w[1]) * bf16_bits_to_f32(h[1]) +
                   bf16_bits_to_f32(p.w[2]) * bf16_bits_to_f32(h[2]) + bf16_bits_to_f32(p.w[3]) * bf16_bits_to_f32(x0);
  const float a1 = bf16_bits_to_f32(p.w[4]) * bf16_bits_to_f32(h[3]) + bf16_bits_to_f32(p.w[5]) * bf16_bits_to_f32(h[4]) +
                   bf16_bits_to_f32(p.w[6]) * bf16_bits_to_f32(h[5]) + bf16_bits_to_f32(p.w[7]) * bf16_bits_to_f32(x1);
  y0 = a0 * sigmoidf_(a0);
  y1 = a1 * sigmoidf_(a1);
  if (keep) {
    uint32_t* so = reinterpret_cast<uint32_t*>(a.cs_out + (crow + c) * 3);
    so[0] = static_cast<uint32_t>(h[1]) | (static_cast<uint32_t>(h[2]) << 16);
    so[1] = static_cast<uint32_t>(x0) | (static_cast<uint32_t>(h[4]) << 16);
    so[2] = static_cast<uint32_t>(h[5]) | (static_cast<uint32_t>(x1) << 16);
  }
}

constexpr int kLayerThreads = 1024;

__global__ __launch_bounds__(kLayerThreads) void decode_layer_kernel(LayerArgs a) {
  constexpr int D = 128;
  using S = RecShape<D, kLayerThreads>;
  constexpr int RG = S::RG, RPT = S::RPT, TPR = S::TPR;

  __shared__ float s_q[D];
  __shared__ float s_k[D];
  __shared__ float s_v[D];
  __shared__ float s_red[2][RG][D];
  __shared__ float s_uw[2][D];
  __shared__ float s_scal[4];

  const int bh = blockIdx.x;
  const int b = bh / a.Hv, h = bh - b * a.Hv, hk = h / a.G;
  const int tid = threadIdx.x;
  const int cg = tid % TPR, rg = tid / TPR;
  const int c0 = cg * 4;
  int slot = b;
  if (a.slots) {
    slot = a.slots[b];
    if (slot < 0 || slot >= a.nslots) return;  // the whole workgroup skips the sequence
  }
  const int64_t C = static_cast<int64_t>(2 * a.Hk + a.Hv) * D;
  const int64_t crow = static_cast<int64_t>(slot) * C;   // window pool row of this sequence
  const int64_t xrow = static_cast<int64_t>(b) * a.sx;
  const int64_t sidx = static_cast<int64_t>(slot) * a.Hv + h;

  // conv operands first (wave 0: q and k pairs of the key head, wave 1: v pairs),
  // so that their latency overlaps the state's loads
  ConvPair cp0, cp1;
  int ch0 = 0, ch1 = 0;
  if (tid < 64) {
    ch0 = hk * D + 2 * tid;
    ch1 = a.Hk * D + hk * D + 2 * tid;
  } else if (tid < 128) {
    ch0 = 2 * a.Hk * D + h * D + 2 * (tid - 64);
  }
  if (tid < 128) cp0 = conv_load(a, crow, xrow, ch0);
  if (tid < 64) cp1 = conv_load(a, crow, xrow, ch1);

  floatx4 M[RPT];
  {
    const float* sp = a.pool + sidx * D * D;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      M[r] = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(sp + (rg + RG * r) * D + c0));
  }

  if (tid < 64) {
    // q and k of the key head (2 channels each per lane), their norms, the gates
    const bool keep = (h % a.G) == 0;
    float qv[2], kv[2];
    conv_finish(a, cp0, crow, ch0, keep, qv[0], qv[1]);
    conv_finish(a, cp1, crow, ch1, keep, kv[0], kv[1]);
    float sqq = qv[0] * qv[0] + qv[1] * qv[1], skk = kv[0] * kv[0] + kv[1] * kv[1];
    float sqk = qv[0] * kv[0] + qv[1] * kv[1];
    sqq = wave_sum(sqq);
    skk = wave_sum(skk);
    sqk = wave_sum(sqk);
    float rq = 1.f, rk = 1.f;
    if (a.flags & 1u) {
      rq = rsqrtf(sqq + a.l2_eps);
      rk = rsqrtf(skk + a.l2_eps);
    }
    rq *= a.q_scale;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      s_q[2 * tid + e] = qv[e] * rq;
      s_k[2 * tid + e] = kv[e] * rk;
    }
    if (tid == 0) {
      s_scal[0] = sqk * rq * rk;
      float la, be;
      const int64_t r = static_cast<int64_t>(b) * a.sba;
      gate_activation(bf16_bits_to_f32(a.ba[r + h]), bf16_bits_to_f32(a.ba[r + a.Hv + h]), a.A_log[h],
                      a.dt_bias[h], la, be);
      s_scal[1] = __expf(la);
      s_scal[2] = be;
    }
  } else if (tid < 128) {
    // v of this value head (2 channels per lane)
    float v0, v1;
    conv_finish(a, cp0, crow, ch0, true, v0, v1);
    s_v[2 * (tid - 64)] = v0;
    s_v[2 * (tid - 64) + 1] = v1;
  }
  __syncthreads();

  floatx4 pu = {0.f, 0.f, 0.f, 0.f}, pw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int i = rg + RG * r;
    pu += M[r] * s_k[i];
    pw += M[r] * s_q[i];
  }
  *reinterpret_cast<floatx4*>(&s_red[0][rg][c0]) = pu;
  *reinterpret_cast<floatx4*>(&s_red[1][rg][c0]) = pw;
  __syncthreads();

  // row groups 0 and 1 sum u and w over all row groups once, the rest read them
  if (rg < 2) {
    floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < RG; ++g) t += *reinterpret_cast<const floatx4*>(&s_red[rg][g][c0]);
    *reinterpret_cast<floatx4*>(&s_uw[rg][c0]) = t;
  }
  __syncthreads();
  const floatx4 u = *reinterpret_cast<const floatx4*>(&s_uw[0][c0]);
  const floatx4 w = *reinterpret_cast<const floatx4*>(&s_uw[1][c0]);
  const float kq = s_scal[0], alpha = s_scal[1], beta = s_scal[2];
  const floatx4 vv = *reinterpret_cast<const floatx4*>(&s_v[c0]);
  const floatx4 d = beta * (vv - alpha * u);
  if (rg == 0) {
    // row group 0 is lanes 0..31 of wave 0: 4 outputs each, the head's 128 in all
    const floatx4 o = alpha * w + kq * d;
    float ss = o[0] * o[0] + o[1] * o[1] + o[2] * o[2] + o[3] * o[3];
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float inv = rsqrtf(ss * (1.0f / D) + a.norm_eps);
    const int64_t zr = static_cast<int64_t>(b) * a.sz + h * D + c0;
    const int64_t orow = static_cast<int64_t>(b) * a.sout + h * D + c0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float zv = bf16_bits_to_f32(a.z[zr + e]);
      a.out[orow + e] = f32_to_bf16_bits(o[e] * inv * bf16_bits_to_f32(a.norm_w[c0 + e]) * zv * sigmoidf_(zv));
      if (a.o) a.o[static_cast<int64_t>(b) * a.so + h * D + c0 + e] = f32_to_bf16_bits(o[e]);
    }
  }
  {
    float* sp = a.pool + sidx * D * D;
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      __builtin_nontemporal_store(alpha * M[r] + s_k[rg + RG * r] * d,
                                  reinterpret_cast<floatx4*>(sp + (rg + RG * r) * D + c0));
  }
}

template <int D, typename IO>
hipError_t launch_rec(const RecArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.cu_seqlens ? a.nseq : a.B) * a.Hv));
  if (grid.x == 0) return hipSuccess;
  // A single token (the decode step) is one pass over the state: 1024 threads per
  // state keep more of its 64 KiB in flight per CU than 256 (measured on a plain
  // non-temporal read-modify-write of the same layout, 3,072 states: 68.6 us with
  // 1024 threads, 69.6 with 512, 75.7 with 256).
  if (D == 128 && a.T == 1)
    hipLaunchKernelGGL((recurrent_kernel<D, IO, 1024>), grid, dim3(RecShape<D, 1024>::NT), 0, s, a);
  else
    hipLaunchKernelGGL((recurrent_kernel<D, IO, 256>), grid, dim3(RecShape<D, 256>::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_layer(const LayerArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_layer_kernel, dim3(static_cast<unsigned>(a.B * a.Hv)), dim3(kLayerThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_recurrent(const RecArgs& a, int io, hipStream_t s) {
  if (io == 1) {
    switch (a.D) {
      case 16: return launch_rec<16, uint16_t>(a, s);
      case 32: return launch_rec<32, uint16_t>(a, s);
      case 64: return launch_rec<64, uint16_t>(a, s);
      case 128: return launch_rec<128, uint16_t>(a, s);
    }
  } else {
    switch (a.D) {
      case 16: return launch_rec<16, float>(a, s);
      case 32: return launch_rec<32, float>(a, s);
      case 64: return launch_rec<64, float>(a, s);
      case 128: return launch_rec<128, float>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
