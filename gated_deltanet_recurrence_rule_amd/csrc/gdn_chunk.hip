// gdn_chunk.hip -- chunkwise gated delta rule prefill on gfx950 MFMA.
//
// The pages describe prefill of a recurrent layer as block-by-block work:
// large matrix products inside each block of 64 tokens, and the state handed
// from one block to the next (course page "Chapitre 16 - Assembler un systeme
// de type Kimi K3", section 16.2, with the 256-token / 4-block example); the
// state itself is a 128 x 128 fp32 matrix per value head that must stay fp32
// ("L'attention hybride", sections "La recurrence", "L'etat, en memoire",
// "Le float32 n'est pas un detail").  The per-block algebra is not on the
// pages; the one used here (state stored as M = S^T, [Dk][Dv]) is:
//
//   rows r = 0..63 of a chunk, g_r = sum_{i<=r} log alpha_i, gamma_r = e^{g_r}
//   k^_r = rk_r k_r, q^_r = rq_r q_r  (rk, rq: L2 factors or 1; rq has q_scale)
//   A_ri  = beta_r e^{g_r-g_i} (k^_r . k^_i)        i < r   (strictly lower)
//   T     = (I + A)^-1,   T' = T diag(beta)          (unit lower-triangular)
//   P_ri  = e^{g_r-g_i} (q^_r . k^_i)                i <= r
//   X     = V - diag(gamma rk) K M                   [64 x Dv]
//   U     = T' X                                     (WY / UT transform)
//   O     = diag(gamma rq) Q M + P U
//   M    <- gamma_63 M + K^T diag(rk e^{g_63 - g}) U
//
// which reproduces the token-by-token rule exactly (up to rounding).  Every
// exponent is <= 0.  K and Q stay raw bf16 MFMA operands: the L2 factors are
// folded into fp32 row scalings.  Columns of M (value coordinates) evolve
// independently, so a workgroup takes a slice of DVS = 16*NW value columns of
// one (sequence, value head) and each wave owns a 16-column strip of M in
// MFMA accumulator registers for the whole sequence: the fp32 state never
// leaves the chip between chunks.
//
// Precision.  MFMA operands are bf16 with fp32 accumulation.  Genuine bf16
// inputs (K, Q, V) enter as they are.  fp32 operands whose rounding would
// reach the state or output tolerance are split into hi + lo bf16 pairs:
// T' and X in T'X (3 products), P and U in P U (3), U' in K^T U' (2).  M
// enters K M and Q M as a single bf16 (its rounding error stays ~1e-6 of the
// state).
//
// MFMA layout (v_mfma_f32_16x16x32_bf16, wave64): the A operand row and the B
// operand column are lane & 15; the accumulator holds column lane & 15, rows
// 4*(lane>>4) + i.  The contraction index of A and B is permuted the same way
// on both sides: lane group kg = lane >> 4 carries, for a 32-wide k block,
// k = 4kg..4kg+3 and 16+4kg..16+4kg+3.  With that permutation two
// accumulator tiles stacked along k (rows 0-15 and 16-31) are directly a B
// operand, so K M, T'X, P U and K^T U' take M, X and U straight from
// registers; A operands come from LDS as two 8-byte reads.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int CH = 64;    // chunk length
constexpr int DK = 128;   // head width
constexpr int KP = 136;   // LDS row pitch (bf16 elements) of the 64 x 128 K and Q tiles
constexpr int RP = 72;    // LDS row pitch (bf16) of 64-wide bf16 matrices (K^T, T', P)
constexpr int FP = 65;    // LDS row pitch (floats) of fp32 64 x 64 matrices

template <int NW>
struct ChunkLds {
  static constexpr int DVS = 16 * NW;
  static constexpr int VP = DVS + 8;
  // byte offsets
  static constexpr int kK = 0;
  static constexpr int kQ = kK + CH * KP * 2;
  static constexpr int kKt = kQ + CH * KP * 2;
  static constexpr int kV = kKt + DK * RP * 2;
  static constexpr int kG = kV + CH * VP * 2;      // fp32 64x64: K K^T, then A
  static constexpr int kF = kG + CH * FP * 4;      // fp32 64x64: Q K^T, then T
  static constexpr int kTh = kF + CH * FP * 4;
  static constexpr int kTl = kTh + CH * RP * 2;
  static constexpr int kPh = kTl + CH * RP * 2;
  static constexpr int kPl = kPh + CH * RP * 2;
  static constexpr int kY = kPl + CH * RP * 2;      // 3 x 16x16 fp32 scratch for the inverse
  static constexpr int kVec = kY + 3 * 256 * 4;
  static constexpr int kNumVec = 8;                 // g, beta, rk, rq, grk, grq, drk, spare
  static constexpr int kBytes = kVec + kNumVec * CH * 4;
};

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* row_k0, int kg) {
  const u16x4 lo = *reinterpret_cast<const u16x4*>(row_k0 + 4 * kg);
  const u16x4 hi = *reinterpret_cast<const u16x4*>(row_k0 + 16 + 4 * kg);
  const u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 acc_frag(const floatx4& t0, const floatx4& t1) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = static_cast<__bf16>(t0[e]);
    r[e + 4] = static_cast<__bf16>(t1[e]);
  }
  return r;
}

__device__ __forceinline__ void acc_frag_split(const floatx4& t0, const floatx4& t1, bf16x8& hi,
                                               bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h0 = static_cast<__bf16>(t0[e]);
    const __bf16 h1 = static_cast<__bf16>(t1[e]);
    hi[e] = h0;
    hi[e + 4] = h1;
    lo[e] = static_cast<__bf16>(t0[e] - static_cast<float>(h0));
    lo[e + 4] = static_cast<__bf16>(t1[e] - static_cast<float>(h1));
  }
}

__device__ __forceinline__ floatx4 mfma(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split_store(uint16_t* hi, uint16_t* lo, int idx, float x) {
  const __bf16 h = static_cast<__bf16>(x);
  hi[idx] = __builtin_bit_cast(uint16_t, h);
  lo[idx] = f32_to_bf16_bits(x - static_cast<float>(h));
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void chunk_prefill_kernel(RecArgs a) {
  using L = ChunkLds<NW>;
  constexpr int NT = 64 * NW;
  constexpr int DVS = L::DVS;
  constexpr int VP = L::VP;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + L::kK);
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + L::kQ);
  uint16_t* sKt = reinterpret_cast<uint16_t*>(smem + L::kKt);
  uint16_t* sV = reinterpret_cast<uint16_t*>(smem + L::kV);
  float* sG = reinterpret_cast<float*>(smem + L::kG);
  float* sF = reinterpret_cast<float*>(smem + L::kF);
  uint16_t* sTh = reinterpret_cast<uint16_t*>(smem + L::kTh);
  uint16_t* sTl = reinterpret_cast<uint16_t*>(smem + L::kTl);
  uint16_t* sPh = reinterpret_cast<uint16_t*>(smem + L::kPh);
  uint16_t* sPl = reinterpret_cast<uint16_t*>(smem + L::kPl);
  float* sY = reinterpret_cast<float*>(smem + L::kY);
  float* vG = reinterpret_cast<float*>(smem + L::kVec);
  float* vBeta = vG + CH;
  float* vRk = vG + 2 * CH;
  float* vRq = vG + 3 * CH;
  float* vGrk = vG + 4 * CH;
  float* vGrq = vG + 5 * CH;
  float* vDrk = vG + 6 * CH;

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int kg = lane >> 4;

  const int slice = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / a.G;
  const int bh = b * a.Hv + h;
  const int col = slice * DVS + 16 * wv + lr;  // this lane's value column (global)

  const uint16_t* gq = static_cast<const uint16_t*>(a.q);
  const uint16_t* gk = static_cast<const uint16_t*>(a.k);
  const uint16_t* gv = static_cast<const uint16_t*>(a.v);
  uint16_t* go = static_cast<uint16_t*>(a.o);
  const bool l2 = (a.flags & 1u) != 0;

  // State strip: rows 16*dt + 4*kg + i, column `col`.
  floatx4 Ms[8];
  if (a.state_in) {
    const float* sp = a.state_in + static_cast<int64_t>(bh) * DK * DK;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ms[dt][i] = sp[(16 * dt + 4 * kg + i) * DK + col];
  } else {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) Ms[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int nchunks = (a.T + CH - 1) / CH;
  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * CH;
    const int nval = min(CH, a.T - t0);
    const int64_t tokbase = static_cast<int64_t>(b) * a.T + t0;

    // ---- P1: stage K, Q (and K^T), the V slice and the gates in LDS --------
#pragma unroll
    for (int j = 0; j < (CH * DK / 8) / NT; ++j) {
      const int vi = tid + NT * j;
      const int r = vi >> 4, c8 = (vi & 15) * 8;
      u16x8 kv = {0, 0, 0, 0, 0, 0, 0, 0}, qv = {0, 0, 0, 0, 0, 0, 0, 0};
      if (r < nval) {
        kv = *reinterpret_cast<const u16x8*>(gk + (tokbase + r) * a.sk + hk * DK + c8);
        qv = *reinterpret_cast<const u16x8*>(gq + (tokbase + r) * a.sq + hk * DK + c8);
      }
      *reinterpret_cast<u16x8*>(sK + r * KP + c8) = kv;
      *reinterpret_cast<u16x8*>(sQ + r * KP + c8) = qv;
      float ssk = 0.f, ssq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sKt[(c8 + e) * RP + r] = kv[e];
        const float kf = bf16_bits_to_f32(kv[e]), qf = bf16_bits_to_f32(qv[e]);
        ssk = fmaf(kf, kf, ssk);
        ssq = fmaf(qf, qf, ssq);
      }
      // the 16 lanes holding one row are consecutive: reduce over them
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1) {
        ssk += __shfl_xor(ssk, m, 64);
        ssq += __shfl_xor(ssq, m, 64);
      }
      if ((vi & 15) == 0) {
        vRk[r] = l2 ? rsqrtf(ssk + a.l2_eps) : 1.f;
        vRq[r] = (l2 ? rsqrtf(ssq + a.l2_eps) : 1.f) * a.q_scale;
      }
    }
#pragma unroll
    for (int j = 0; j < (CH * DVS / 8 + NT - 1) / NT; ++j) {
      const int vi = tid + NT * j;
      if (vi < CH * DVS / 8) {
        const int r = vi / (DVS / 8), c8 = (vi % (DVS / 8)) * 8;
        u16x8 vv = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < nval) vv = *reinterpret_cast<const u16x8*>(gv + (tokbase + r) * a.sv + h * DK + slice * DVS + c8);
        *reinterpret_cast<u16x8*>(sV + r * VP + c8) = vv;
      }
    }
    if (wv == 0) {
      float la = 0.f, be = 0.f;
      if (lane < nval) {
        la = a.la[(tokbase + lane) * a.Hv + h];
        be = a.beta[(tokbase + lane) * a.Hv + h];
      }
      float g = la;  // inclusive prefix sum over the chunk
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(g, off, 64);
        if (lane >= off) g += t;
      }
      vG[lane] = g;
      vBeta[lane] = be;
    }
    __syncthreads();

    // ---- P2: Gram tiles K K^T (strictly lower needed) and Q K^T (lower) ----
    // 20 jobs: 10 lower-triangle 16x16 tiles of each product.
    for (int job = wv; job < 20; job += NW) {
      const int m = job / 10, tI = job % 10;
      int rt = 0;
      while ((rt + 1) * (rt + 2) / 2 <= tI) ++rt;
      const int ct = tI - rt * (rt + 1) / 2;
      const uint16_t* As = (m == 0) ? sK : sQ;
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 A = lds_frag(As + (16 * rt + lr) * KP + 32 * kb, kg);
        const bf16x8 Bf = lds_frag(sK + (16 * ct + lr) * KP + 32 * kb, kg);
        acc = mfma(A, Bf, acc);
      }
      float* dst = (m == 0) ? sG : sF;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * rt + 4 * kg + i) * FP + 16 * ct + lr] = acc[i];
    }
    __syncthreads();

    // ---- P3: A (into sG), P = e^{g_r-g_i} rq_r rk_i (QK^T)_ri split into sPh/sPl,
    //          and the per-row scalings ----------------------------------------
    for (int e = tid; e < CH * CH; e += NT) {
      const int r = e >> 6, i = e & 63;
      const float gr = vG[r], gi = vG[i];
      float av = 0.f, pv = 0.f;
      if (i <= r) {
        const float dec = __expf(gr - gi);
        pv = dec * vRq[r] * vRk[i] * sF[r * FP + i];
        if (i < r) av = vBeta[r] * dec * vRk[r] * vRk[i] * sG[r * FP + i];
      }
      sG[r * FP + i] = av;
      split_store(sPh, sPl, r * RP + i, pv);
    }
    if (tid < CH) {
      const float gr = vG[tid], gl = vG[CH - 1];
      const float gam = __expf(gr);
      vGrk[tid] = gam * vRk[tid];
      vGrq[tid] = gam * vRq[tid];
      vDrk[tid] = __expf(gl - gr) * vRk[tid];
    }
    __syncthreads();

    // ---- P4: T = (I + A)^-1 in fp32 (into sF), 16x16 blocks ----------------
    if (wv == 0) {
      // diagonal blocks by forward substitution: lane = 16*blk + column j
      const int blk = lane >> 4, j = lane & 15;
      const float* Ab = sG + (16 * blk) * FP + 16 * blk;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s = fmaf(Ab[r * FP + i], x[i], s);
        x[r] = (r < j) ? 0.f : ((r == j) ? 1.f : -s);
      }
      float* Tb = sF + (16 * blk) * FP + 16 * blk;
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[r * FP + j] = x[r];
    }
    __syncthreads();
    // off-diagonal blocks, by distance d = I - J:
    //   Y = sum_{k=J}^{I-1} A_Ik T_kJ ;  T_IJ = -T_II Y
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      const int nb = 4 - d;  // blocks at this distance: (J + d, J), J = 0..nb-1
      const int yr = lane >> 2, yc = (lane & 3) * 4;
      if (wv < nb) {
        const int J = wv, I = J + d;
        floatx4 y = {0.f, 0.f, 0.f, 0.f};
        for (int kk = J; kk < I; ++kk) {
          const float* Arow = sG + (16 * I + yr) * FP + 16 * kk;
          const float* Tcol = sF + (16 * kk) * FP + 16 * J + yc;
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            const float av = Arow[m];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = fmaf(av, Tcol[m * FP + e], y[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sY[wv * 256 + yr * 16 + yc + e] = y[e];
      }
      __syncthreads();
      if (wv < nb) {
        const int J = wv, I = J + d;
        floatx4 t = {0.f, 0.f, 0.f, 0.f};
        const float* Trow = sF + (16 * I + yr) * FP + 16 * I;
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const float tv = Trow[m];
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = fmaf(tv, sY[wv * 256 + m * 16 + yc + e], t[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sF[(16 * I + yr) * FP + 16 * J + yc + e] = -t[e];
      }
      __syncthreads();
    }
    // T' = T diag(beta) (lower triangle; zero above), split into sTh/sTl
    for (int e = tid; e < CH * CH; e += NT) {
      const int r = e >> 6, i = e & 63;
      const float tv = (i <= r) ? sF[r * FP + i] * vBeta[i] : 0.f;
      split_store(sTh, sTl, r * RP + i, tv);
    }
    __syncthreads();

    // ---- P5: the state chain for this wave's 16 value columns --------------
    const int vcol = 16 * wv + lr;  // column inside the V slice
    floatx4 X[4];
    {
      floatx4 km[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) km[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 Bm = acc_frag(Ms[2 * kb], Ms[2 * kb + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          km[rt] = mfma(lds_frag(sK + (16 * rt + lr) * KP + 32 * kb, kg), Bm, km[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * kg + i;
          X[rt][i] = bf16_bits_to_f32(sV[r * VP + vcol]) - vGrk[r] * km[rt][i];
        }
    }
    // U = T' X  (T' lower-triangular: skip the all-zero upper 16x32 blocks)
    floatx4 U[4];
    {
      bf16x8 Xh[2], Xl[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) acc_frag_split(X[2 * kb], X[2 * kb + 1], Xh[kb], Xl[kb]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        U[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (32 * kb > 16 * rt + 15) continue;
          const bf16x8 Ah = lds_frag(sTh + (16 * rt + lr) * RP + 32 * kb, kg);
          const bf16x8 Al = lds_frag(sTl + (16 * rt + lr) * RP + 32 * kb, kg);
          U[rt] = mfma(Ah, Xh[kb], U[rt]);
          U[rt] = mfma(Ah, Xl[kb], U[rt]);
          U[rt] = mfma(Al, Xh[kb], U[rt]);
        }
      }
    }
    // O = diag(gamma rq) Q M + P U
    {
      floatx4 O[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) O[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 Bm = acc_frag(Ms[2 * kb], Ms[2 * kb + 1]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
          O[rt] = mfma(lds_frag(sQ + (16 * rt + lr) * KP + 32 * kb, kg), Bm, O[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[rt][i] *= vGrq[16 * rt + 4 * kg + i];
      bf16x8 Uh[2], Ul[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) acc_frag_split(U[2 * kb], U[2 * kb + 1], Uh[kb], Ul[kb]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (32 * kb > 16 * rt + 15) continue;
          const bf16x8 Ah = lds_frag(sPh + (16 * rt + lr) * RP + 32 * kb, kg);
          const bf16x8 Al = lds_frag(sPl + (16 * rt + lr) * RP + 32 * kb, kg);
          O[rt] = mfma(Ah, Uh[kb], O[rt]);
          O[rt] = mfma(Ah, Ul[kb], O[rt]);
          O[rt] = mfma(Al, Uh[kb], O[rt]);
        }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * kg + i;
          if (r < nval) go[(tokbase + r) * a.so + h * DK + col] = f32_to_bf16_bits(O[rt][i]);
        }
    }
    // M <- gamma_63 M + K^T diag(rk e^{g_63 - g}) U
    {
      bf16x8 Wh[2], Wl[2];
      floatx4 Us[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) Us[rt][i] = U[rt][i] * vDrk[16 * rt + 4 * kg + i];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) acc_frag_split(Us[2 * kb], Us[2 * kb + 1], Wh[kb], Wl[kb]);
      const float gC = __expf(vG[CH - 1]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        Ms[dt] *= gC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 A = lds_frag(sKt + (16 * dt + lr) * RP + 32 * kb, kg);
          Ms[dt] = mfma(A, Wh[kb], Ms[dt]);
          Ms[dt] = mfma(A, Wl[kb], Ms[dt]);
        }
      }
    }
    __syncthreads();  // LDS is restaged by the next chunk
  }

  if (a.state_out) {
    float* sp = a.state_out + static_cast<int64_t>(bh) * DK * DK;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sp[(16 * dt + 4 * kg + i) * DK + col] = Ms[dt][i];
  }
}

template <int NW>
hipError_t launch_nw(const RecArgs& a, hipStream_t s) {
  using L = ChunkLds<NW>;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_prefill_kernel<NW>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, L::kBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(DK / L::DVS, a.Hv, a.B);
  hipLaunchKernelGGL(chunk_prefill_kernel<NW>, grid, dim3(64 * NW), L::kBytes, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_prefill(const RecArgs& a, hipStream_t s) { return launch_nw<4>(a, s); }

}  // namespace gdn
