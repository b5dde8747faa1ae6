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
// 64 KiB state, 128-bit coalesced) and the prefill kernel for shapes the
// chunked MFMA kernel does not take (fp32 I/O, head widths 16..64).
//
// Thread layout: TPR = D/4 threads cover one row of M with a float4 each;
// RG = NT/TPR row groups take rows rg, rg+RG, ... so that one wave's loads
// cover whole consecutive rows.  Column partial sums over a thread's rows are
// reduced across the RG groups through LDS.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int D>
struct RecShape {
  static constexpr int NT = (D * D / 4 < 256) ? D * D / 4 : 256;
  static constexpr int TPR = D / 4;
  static constexpr int RG = NT / TPR;
  static constexpr int RPT = D / RG;
  static_assert(RG * RPT == D, "row split");
  static_assert(NT % 64 == 0, "whole waves");
};

template <int D, typename IO>
__global__ __launch_bounds__(RecShape<D>::NT) void recurrent_kernel(RecArgs a) {
  using S = RecShape<D>;
  constexpr int RG = S::RG, RPT = S::RPT, TPR = S::TPR;
  constexpr int QPL = (D + 63) / 64;  // q/k elements per lane in the staging wave

  __shared__ float s_q[D];
  __shared__ float s_k[D];
  __shared__ float s_red[2][RG][D];
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
    if (slot < 0) return;  // the whole workgroup skips the row
    sidx = static_cast<int64_t>(slot) * a.Hv + h;
  }

  floatx4 M[RPT];
  if (a.state_in) {
    const float* sp = a.state_in + sidx * D * D;
#pragma unroll
    for (int r = 0; r < RPT; ++r) M[r] = *reinterpret_cast<const floatx4*>(sp + (rg + RG * r) * D + c0);
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) M[r] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  for (int t = 0; t < a.T; ++t) {
    const int64_t tok = static_cast<int64_t>(b) * a.T + t;
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
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      u += *reinterpret_cast<const floatx4*>(&s_red[0][g][c0]);
      w += *reinterpret_cast<const floatx4*>(&s_red[1][g][c0]);
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
    for (int r = 0; r < RPT; ++r) *reinterpret_cast<floatx4*>(sp + (rg + RG * r) * D + c0) = M[r];
  }
}

template <int D, typename IO>
hipError_t launch_rec(const RecArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.B * a.Hv));
  hipLaunchKernelGGL((recurrent_kernel<D, IO>), grid, dim3(RecShape<D>::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace

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
