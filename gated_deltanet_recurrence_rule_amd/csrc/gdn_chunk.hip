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
//   T'    = (I + A)^-1 diag(beta)                   (lower-triangular)
//   P_ri  = e^{g_r-g_i} (q^_r . k^_i)                i <= r
//   X     = V - diag(gamma rk) K M                   [64 x Dv]
//   U     = T' X                                     (WY / UT transform)
//   O     = diag(gamma rq) Q M + P U
//   M    <- gamma_63 M + K^T diag(rk e^{g_63 - g}) U
//
// which reproduces the token-by-token rule exactly (up to rounding).  Every
// exponent is <= 0.  K and Q stay raw bf16 MFMA operands; the L2 factors are
// folded into fp32 row scalings.
//
// Two kernels per window of chunks:
//  * prep (one workgroup per chunk and key head, fully parallel): everything
//    that does not depend on the state -- row norms, the Gram products
//    K K^T and Q K^T (MFMA), the gate prefix sums, A, the triangular inverse
//    (fp32, blocked 16/32), T' and P -- written to the workspace as ready
//    MFMA A-operand fragments (fp16) plus three row-scaling
//    vectors per (chunk, value head).
//    The prep kernel also writes K, Q and K^T as fragments, so the chain
//    kernel stages its inputs with plain 16-byte copies and reads every MFMA
//    A operand with one conflict-free 16-byte LDS read per lane.
//  * chain (one workgroup per sequence, value head and 64 value columns,
//    looping over the chunks): only the state-dependent products.  Columns of
//    M evolve independently; waves 0-1 ("state") each own a 32-column strip
//    of M in MFMA accumulators for the whole window and run the serial path
//    K M, X, U = T'X and the update, with nothing else to do; waves 2-3
//    ("output") compute Q M and P U for the same strips from fragments the
//    state waves publish in LDS, and move the next chunk's inputs from HBM
//    into LDS: loads are issued at the start of a chunk; inputs the update
//    phase reads go to one of two alternating buffers at the chunk's end,
//    the rest is restaged while the update runs.
//
// Precision.  MFMA accumulation is fp32 throughout.  K M and Q M run on bf16
// operands (K and Q are bf16 inputs; M is rounded once to bf16 for them).
// T'X, P U and K^T U' run on fp16 operands: T', P and the update's K^T are
// written as fp16 by the prep kernel (bf16 K converts exactly), X and U are
// rounded once to fp16.  fp16 keeps 11 significant bits, which holds the
// state within a few 1e-4 of the exact result and the outputs well inside
// their bound; its range (|x| < 65504) bounds the values of v, the state and
// the intra-chunk matrices this path accepts.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16 and _f16, wave64): A row = B column =
// lane & 31; the accumulator holds column lane & 31, rows 8j + 4h + i
// (h = lane >> 5, value index 4j + i).  The contraction index is permuted the
// same way on A and B: inside each 16-wide k step, lane half h carries
// k = 4h..4h+3 and 8+4h..8+4h+3.  With that permutation accumulator values
// [8s, 8s+8) of a tile are directly the B operand for k step s of that tile,
// so M, X and U feed the next product from registers.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));

constexpr int CH = 64;    // chunk length
constexpr int DK = 128;   // head width
constexpr int KP = 136;   // LDS row pitch (bf16) of 64 x 128 K / Q tiles
constexpr int RP = 72;    // LDS row pitch (bf16) of K^T and of the V slice
constexpr int FP = 68;    // LDS row pitch (floats) of fp32 64 x 64 matrices (16-byte rows)
constexpr int DVS = 64;   // value columns per chain workgroup
constexpr int FT = 6;     // 32x16 fragment tiles covering a 64x64 lower triangle
constexpr int WS_TP = 2 * FT * 1024;      // T' and P fragments (fp16)
constexpr int WS_CHUNK = WS_TP + 2048;    // + grk[64], grq[64], drk[64], gamma_63 (2 KiB slot)
constexpr int WS_KQ = 3 * 16 * 1024;      // per (b, key head, chunk): K, Q and K^T fragments

// fragment tile f covers rows 32*kFtRt[f].., k step kFtKs[f] (16 columns)
__device__ __forceinline__ int ft_rt(int f) { return f < 2 ? 0 : 1; }
__device__ __forceinline__ int ft_ks(int f) { return f < 2 ? f : f - 2; }
// k offset (inside a 16-wide step) of element e for lane half h
__device__ __forceinline__ int kperm(int h, int e) { return (e < 4) ? 4 * h + e : 8 + 4 * h + (e - 4); }

__device__ __forceinline__ bf16x8 lds_frag32(const uint16_t* row_k0, int h) {
  const u16x4 lo = *reinterpret_cast<const u16x4*>(row_k0 + 4 * h);
  const u16x4 hi = *reinterpret_cast<const u16x4*>(row_k0 + 8 + 4 * h);
  const u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma32h(const halfx8& a, const halfx8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ halfx8 acc_frag_h(const floatx16& t, int s) {
  halfx8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<_Float16>(t[8 * s + e]);
  return r;
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

__device__ __forceinline__ bf16x8 acc_frag(const floatx16& t, int s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(t[8 * s + e]);
  return r;
}

__device__ __forceinline__ floatx16 zero16() {
  floatx16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// accumulator value index v of a 32x32 tile -> row inside the tile
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// =========================================================================
// prep kernel: one workgroup (4 waves) per (chunk in window, key head, batch)
// =========================================================================
struct PrepLds {
  static constexpr int kKQ = 0;                       // sK, sQ bf16 [64][KP]; later sA, sT fp32
  static constexpr int kA = 0;
  static constexpr int kT = CH * FP * 4;
  static constexpr int kKK = 2 * CH * KP * 2;         // fp32 [64][FP]
  static constexpr int kQK = kKK + CH * FP * 4;
  static constexpr int kY = kQK + CH * FP * 4;        // fp32 32 x 36 (or 2 x 16 x 20)
  static constexpr int kVec = kY + 32 * 36 * 4;       // rk, rq, g, beta
  static constexpr int kBytes = kVec + 4 * CH * 4;
};

__global__ __launch_bounds__(256, 2) void chunk_prep_kernel(RecArgs a, int c0, unsigned char* ws, int nwin) {
  // workspace: region H = [B][Hv][nwin] x WS_CHUNK, then region K = [B][Hk][nwin] x WS_KQ
  using L = PrepLds;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + L::kKQ);
  uint16_t* sQ = sK + CH * KP;
  float* sA = reinterpret_cast<float*>(smem + L::kA);
  float* sT = reinterpret_cast<float*>(smem + L::kT);
  float* sKK = reinterpret_cast<float*>(smem + L::kKK);
  float* sQK = reinterpret_cast<float*>(smem + L::kQK);
  float* sY = reinterpret_cast<float*>(smem + L::kY);
  float* vRk = reinterpret_cast<float*>(smem + L::kVec);
  float* vRq = vRk + CH;
  float* vG = vRk + 2 * CH;
  float* vBe = vRk + 3 * CH;

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int cl = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int c = c0 + cl;
  const int t0 = c * CH;
  const int nval = min(CH, a.T - t0);
  const int64_t tokbase = static_cast<int64_t>(b) * a.T + t0;
  const bool l2 = (a.flags & 1u) != 0;
  const uint16_t* gq = static_cast<const uint16_t*>(a.q);
  const uint16_t* gk = static_cast<const uint16_t*>(a.k);

  // ---- K, Q rows and their norms ------------------------------------------
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int vi = tid + 256 * j;
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
      const float kf = bf16_bits_to_f32(kv[e]), qf = bf16_bits_to_f32(qv[e]);
      ssk = fmaf(kf, kf, ssk);
      ssq = fmaf(qf, qf, ssq);
    }
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
  __syncthreads();

  // ---- K, Q and K^T as the chain kernel's MFMA A fragments ------------------
  // K, Q (A of K M / Q M): tile (rt, ks) holds rows 32rt + (lane&31), k = 16ks + kperm;
  // K^T (A of K^T U): tile (dt, ks) holds key rows 32dt + (lane&31), k = chunk rows 16ks + kperm.
  {
    unsigned char* wsk = ws + static_cast<int64_t>(a.B) * a.Hv * nwin * WS_CHUNK +
                         (static_cast<int64_t>(b * a.Hk + hk) * nwin + cl) * WS_KQ;
    for (int slot = tid; slot < 3 * 16 * 64; slot += 256) {
      const int mat = slot >> 10, tile = (slot >> 6) & 15, ln = slot & 63;
      const int r32 = ln & 31, hh = ln >> 5;
      u16x8 f;
      if (mat < 2) {
        const uint16_t* src = (mat == 0 ? sK : sQ) + (32 * (tile >> 3) + r32) * KP + 16 * (tile & 7);
        const u16x4 lo = *reinterpret_cast<const u16x4*>(src + 4 * hh);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(src + 8 + 4 * hh);
        f = u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const int d = 32 * (tile >> 2) + r32, k0 = 16 * (tile & 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = f32_to_f16_bits(bf16_bits_to_f32(sK[(k0 + kperm(hh, e)) * KP + d]));
      }
      *reinterpret_cast<u16x8*>(wsk + mat * 16384 + tile * 1024 + ln * 16) = f;
    }
  }

  // ---- Gram tiles (32x32): K K^T and Q K^T, lower blocks (0,0) (1,0) (1,1) --
  for (int job = wv; job < 6; job += 4) {
    const int m = job / 3, tI = job % 3;
    const int rt = tI == 0 ? 0 : 1, ct = tI == 2 ? 1 : 0;
    const uint16_t* As = m == 0 ? sK : sQ;
    floatx16 acc = zero16();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 A = lds_frag32(As + (32 * rt + l32) * KP + 16 * ks, h);
      const bf16x8 B = lds_frag32(sK + (32 * ct + l32) * KP + 16 * ks, h);
      acc = mfma32(A, B, acc);
    }
    float* dst = m == 0 ? sKK : sQK;
#pragma unroll
    for (int v = 0; v < 16; ++v) dst[(32 * rt + acc_row(v, h)) * FP + 32 * ct + l32] = acc[v];
  }
  __syncthreads();  // sK / sQ are dead from here on: their bytes become sA / sT

  for (int j = 0; j < a.G; ++j) {
    const int hv = hk * a.G + j;
    unsigned char* wsc = ws + (static_cast<int64_t>(b * a.Hv + hv) * nwin + cl) * WS_CHUNK;
    // ---- gates: prefix sums and the chain's row scalings ------------------
    if (wv == 0) {
      float la = 0.f, be = 0.f;
      if (lane < nval) {
        la = a.la[(tokbase + lane) * a.Hv + hv];
        be = a.beta[(tokbase + lane) * a.Hv + hv];
      }
      float g = la;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(g, off, 64);
        if (lane >= off) g += t;
      }
      const float gl = __shfl(g, 63, 64);
      vG[lane] = g;
      vBe[lane] = be;
      float* sc = reinterpret_cast<float*>(wsc + WS_TP);
      const float eg = __expf(g);
      sc[lane] = eg * vRk[lane];
      sc[64 + lane] = eg * vRq[lane];
      sc[128 + lane] = __expf(gl - g) * vRk[lane];
      if (lane == 0) sc[192] = __expf(gl);
    }
    __syncthreads();
    // ---- A (fp32, strictly lower), the P fragments, and zeros in the two ----
    //      upper blocks of T that the block inverse reads
    {
      // A: thread -> row r, 16 consecutive columns; every load issued before use
      const int r = tid >> 2, i0 = (tid & 3) * 16;
      const float gr = vG[r], cr = vBe[r] * vRk[r];
      floatx4 kk[4], gi[4], rki[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kk[q] = *reinterpret_cast<const floatx4*>(sKK + r * FP + i0 + 4 * q);
        gi[q] = *reinterpret_cast<const floatx4*>(vG + i0 + 4 * q);
        rki[q] = *reinterpret_cast<const floatx4*>(vRk + i0 + 4 * q);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        floatx4 av;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i0 + 4 * q + e;
          const float x = cr * __expf(fminf(gr - gi[q][e], 0.f)) * rki[q][e] * kk[q][e];
          av[e] = i < r ? x : 0.f;
        }
        *reinterpret_cast<floatx4*>(sA + r * FP + i0 + 4 * q) = av;
      }
      // T blocks (0,1) and (2,3) (above the diagonal, inside S0 and S1) are read as zeros
      {
        const int blk = tid >> 7, e2 = (tid & 127) * 2;
        const int rr = 32 * blk + (e2 >> 4), cc = 32 * blk + 16 + (e2 & 15);
        sT[rr * FP + cc] = 0.f;
        sT[rr * FP + cc + 1] = 0.f;
      }
    }
    for (int slot = tid; slot < FT * 64; slot += 256) {
      const int f = slot >> 6, ln = slot & 63;
      const int r = 32 * ft_rt(f) + (ln & 31), hh = ln >> 5;
      const int ca = 16 * ft_ks(f) + 4 * hh, cb = ca + 8;   // the lane's two 4-column runs
      const float gr = vG[r], rq = vRq[r];
      const floatx4 qa = *reinterpret_cast<const floatx4*>(sQK + r * FP + ca);
      const floatx4 qb = *reinterpret_cast<const floatx4*>(sQK + r * FP + cb);
      const floatx4 ga = *reinterpret_cast<const floatx4*>(vG + ca), gb = *reinterpret_cast<const floatx4*>(vG + cb);
      const floatx4 ka = *reinterpret_cast<const floatx4*>(vRk + ca), kb = *reinterpret_cast<const floatx4*>(vRk + cb);
      u16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = e < 4 ? ca + e : cb + e - 4;
        const float qk = e < 4 ? qa[e] : qb[e - 4], g = e < 4 ? ga[e] : gb[e - 4], rk = e < 4 ? ka[e] : kb[e - 4];
        const float x = __expf(fminf(gr - g, 0.f)) * rq * rk * qk;
        pf[e] = f32_to_f16_bits(i <= r ? x : 0.f);
      }
      *reinterpret_cast<u16x8*>(wsc + (6 + f) * 1024 + ln * 16) = pf;
    }
    __syncthreads();
    // ---- T = (I + A)^-1: diagonal 16x16 blocks by forward substitution ------
    if (wv == 0) {
      const int blk = lane >> 4, jc = lane & 15;
      const float* Ab = sA + (16 * blk) * FP + 16 * blk;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) s = fmaf(Ab[r * FP + i], x[i], s);
        x[r] = (r < jc) ? 0.f : ((r == jc) ? 1.f : -s);
      }
      float* Tb = sT + (16 * blk) * FP + 16 * blk;
#pragma unroll
      for (int r = 0; r < 16; ++r) Tb[r * FP + jc] = x[r];
    }
    __syncthreads();
    // level 1: T_10 = -T_11 A_10 T_00 and T_32 = -T_33 A_32 T_22 (128 threads each)
    {
      const int half = tid >> 7, idx = (tid & 127) * 2;
      const int yr = idx >> 4, yc = idx & 15;
      const int I = 2 * half + 1, J = 2 * half;
      float arow[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 av = *reinterpret_cast<const floatx4*>(sA + (16 * I + yr) * FP + 16 * J + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) arow[4 * q + e] = av[e];
      }
      floatx2 y = {0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const floatx2 tv = *reinterpret_cast<const floatx2*>(sT + (16 * J + m) * FP + 16 * J + yc);
        y[0] = fmaf(arow[m], tv[0], y[0]);
        y[1] = fmaf(arow[m], tv[1], y[1]);
      }
      *reinterpret_cast<floatx2*>(sY + half * 16 * 20 + yr * 20 + yc) = y;
      __syncthreads();
      float trow[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 tv = *reinterpret_cast<const floatx4*>(sT + (16 * I + yr) * FP + 16 * I + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) trow[4 * q + e] = tv[e];
      }
      floatx2 t = {0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const floatx2 yv = *reinterpret_cast<const floatx2*>(sY + half * 16 * 20 + m * 20 + yc);
        t[0] = fmaf(trow[m], yv[0], t[0]);
        t[1] = fmaf(trow[m], yv[1], t[1]);
      }
      *reinterpret_cast<floatx2*>(sT + (16 * I + yr) * FP + 16 * J + yc) = floatx2{-t[0], -t[1]};
    }
    __syncthreads();
    // level 2: T[32:64, 0:32] = -S1 (A[32:64, 0:32] S0), S0/S1 the 32x32 diagonal inverses
    {
      const int idx = tid * 4;
      const int yr = idx >> 5, yc = idx & 31;
      floatx4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const floatx4 av = *reinterpret_cast<const floatx4*>(sA + (32 + yr) * FP + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const floatx4 tv = *reinterpret_cast<const floatx4*>(sT + (4 * q + e) * FP + yc);
          y += av[e] * tv;
        }
      }
      *reinterpret_cast<floatx4*>(sY + yr * 36 + yc) = y;
      __syncthreads();
      floatx4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const floatx4 tv = *reinterpret_cast<const floatx4*>(sT + (32 + yr) * FP + 32 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) t += tv[e] * *reinterpret_cast<const floatx4*>(sY + (4 * q + e) * 36 + yc);
      }
      *reinterpret_cast<floatx4*>(sT + (32 + yr) * FP + yc) = -t;
    }
    __syncthreads();
    // ---- T' = T diag(beta) fragments ----------------------------------------
    for (int slot = tid; slot < FT * 64; slot += 256) {
      const int f = slot >> 6, ln = slot & 63;
      const int r = 32 * ft_rt(f) + (ln & 31), hh = ln >> 5;
      const int ca = 16 * ft_ks(f) + 4 * hh, cb = ca + 8;
      const floatx4 ta = *reinterpret_cast<const floatx4*>(sT + r * FP + ca);
      const floatx4 tb = *reinterpret_cast<const floatx4*>(sT + r * FP + cb);
      const floatx4 ba = *reinterpret_cast<const floatx4*>(vBe + ca), bb = *reinterpret_cast<const floatx4*>(vBe + cb);
      u16x8 tf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = e < 4 ? ca + e : cb + e - 4;
        const float x = e < 4 ? ta[e] * ba[e] : tb[e - 4] * bb[e - 4];
        tf[e] = f32_to_f16_bits(i <= r ? x : 0.f);
      }
      *reinterpret_cast<u16x8*>(wsc + f * 1024 + ln * 16) = tf;
    }
    __syncthreads();  // vG, vBe, sA, sT are rewritten for the next value head
  }
}

// =========================================================================
// chain kernel: one workgroup (4 waves) per (64-column slice, value head, batch)
// =========================================================================
// LDS: a primary buffer (K, Q, T' fragments and the V slice) restaged once per
// chunk after the state waves' first phase, and two alternating buffers
// (K^T and P fragments, row scalings) staged a chunk ahead.
struct ChainLds {
  static constexpr int kK = 0;                     // 16 fragment tiles
  static constexpr int kQ = kK + 16 * 1024;        // 16 fragment tiles
  static constexpr int kTp = kQ + 16 * 1024;       // T' 6 fp16 tiles
  static constexpr int kV = kTp + 6 * 1024;        // bf16 [64][RP]
  static constexpr int kAlt = kV + CH * RP * 2;    // 2 x {K^T 16 fp16 tiles | P 6 fp16 tiles | scalings}
  static constexpr int kAltKt = 0, kAltP = 16 * 1024, kAltSc = 22 * 1024;
  static constexpr int kAltBytes = 24 * 1024;
  static constexpr int kMf = kAlt + 2 * kAltBytes;  // M B-fragments (bf16) [2 strips][8 k steps][64 lanes] x 16 B
  static constexpr int kUf = kMf + 2 * 8 * 1024;    // U B-fragments (fp16) [2 strips][4 k steps][64] x 16 B
  static constexpr int kO = kUf + 2 * 4 * 1024;     // O staging: [2 strips][64 rows][OP] bf16
  static constexpr int OP = 40;
  static constexpr int kBytes = kO + 2 * CH * OP * 2;
};

// Loader waves (2 and 3) move a chunk's chain inputs global -> registers -> LDS in two parts:
// part A (K^T fragments, P fragments, row scalings; 24 KiB) into the alternating buffer, and
// part B (K, Q, T' fragments; 38 KiB; plus the 8 KiB V slice) into the primary buffer.  Both
// parts are whole multiples of 128 16-byte vectors and every source is a compile-time function of
// the unrolled index, so the loads carry no per-lane branches and the compiler can wait for each
// part on its own in issue order.
constexpr int kRegA = 12;   // 8 x 128 K^T vectors, 3 x 128 P vectors, 1 x 128 scaling vectors
constexpr int kRegB = 23;   // 16 x 128 K|Q vectors, 3 x 128 T' vectors, 4 x 128 V vectors

struct ChainSrc {
  const unsigned char* wsh;   // region H block of (b, hv, chunk)
  const unsigned char* wsk;   // region K block of (b, hk, chunk)
  const uint16_t* v;          // first V row of the chunk for this head and slice
  int64_t sv;
  int nval;
};

__device__ __forceinline__ void load_part_a(u32x4 (&r)[kRegA], const ChainSrc& src, int lt) {
#pragma unroll
  for (int m = 0; m < kRegA; ++m) {
    const unsigned char* p = m < 8 ? src.wsk + 32768 + 16 * (lt + 128 * m)              // K^T fragments
                                   : src.wsh + 6144 + 16 * (lt + 128 * (m - 8));        // P | scalings
    r[m] = *reinterpret_cast<const u32x4*>(p);
  }
}

__device__ __forceinline__ void store_part_a(const u32x4 (&r)[kRegA], unsigned char* alt, int lt) {
#pragma unroll
  for (int m = 0; m < kRegA; ++m) reinterpret_cast<u32x4*>(alt)[lt + 128 * m] = r[m];
}

__device__ __forceinline__ void load_part_b(u32x4 (&r)[kRegB], const ChainSrc& src, int lt) {
#pragma unroll
  for (int m = 0; m < kRegB; ++m) {
    if (m < 16) {
      r[m] = *reinterpret_cast<const u32x4*>(src.wsk + 16 * (lt + 128 * m));          // K, Q fragments
    } else if (m < 19) {
      r[m] = *reinterpret_cast<const u32x4*>(src.wsh + 16 * (lt + 128 * (m - 16)));   // T' fragments
    } else {
      const int vi = lt + 128 * (m - 19), row = vi >> 3, c8 = (vi & 7) * 8;
      const int rr = row < src.nval ? row : src.nval - 1;                             // stays in bounds
      const u32x4 x = *reinterpret_cast<const u32x4*>(src.v + rr * src.sv + c8);
      r[m] = row < src.nval ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
}

__device__ __forceinline__ void store_part_b(const u32x4 (&r)[kRegB], unsigned char* smem, int lt) {
  using L = ChainLds;
#pragma unroll
  for (int m = 0; m < kRegB; ++m) {
    if (m < 19) {
      reinterpret_cast<u32x4*>(smem + L::kK)[lt + 128 * m] = r[m];   // K | Q | T' are contiguous
    } else {
      const int vi = lt + 128 * (m - 19);
      *reinterpret_cast<u32x4*>(smem + L::kV + ((vi >> 3) * RP + (vi & 7) * 8) * 2) = r[m];
    }
  }
}

__global__ __launch_bounds__(256) void chunk_chain_kernel(RecArgs a, int c0, const unsigned char* ws, int nwin,
                                                          const float* state_in, float* state_out) {
  using L = ChainLds;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const unsigned char* sK = smem + L::kK;
  const unsigned char* sQ = smem + L::kQ;
  const unsigned char* sTp = smem + L::kTp;
  const uint16_t* sV = reinterpret_cast<const uint16_t*>(smem + L::kV);
  unsigned char* sMf = smem + L::kMf;
  unsigned char* sUf = smem + L::kUf;

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int slice = blockIdx.x, hv = blockIdx.y, b = blockIdx.z;
  const int hk = hv / a.G;
  const int bh = b * a.Hv + hv;
  const int strip = wv & 1;                        // 32-column strip inside the slice
  const bool state_wave = wv < 2;
  const int lt = tid - 128;                        // loader thread index (waves 2, 3)
  const int col = slice * DVS + 32 * strip + l32;  // this lane's value column (global)
  const int vcol = 32 * strip + l32;               // ... inside the V slice
  uint16_t* go = static_cast<uint16_t*>(a.o);

  const int nchunk = min(nwin, (a.T + CH - 1) / CH - c0);
  const unsigned char* regK = ws + static_cast<int64_t>(a.B) * a.Hv * nwin * WS_CHUNK;
  auto src_of = [&](int cl) {
    ChainSrc s;
    s.wsh = ws + (static_cast<int64_t>(bh) * nwin + cl) * WS_CHUNK;
    s.wsk = regK + (static_cast<int64_t>(b * a.Hk + hk) * nwin + cl) * WS_KQ;
    const int t0 = (c0 + cl) * CH;
    s.nval = min(CH, a.T - t0);
    s.sv = a.sv;
    s.v = static_cast<const uint16_t*>(a.v) + (static_cast<int64_t>(b) * a.T + t0) * a.sv + hv * DK + slice * DVS;
    return s;
  };

  floatx16 Ms[4];
  u32x4 regA[kRegA], regB[kRegB];
  if (state_wave) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      if (state_in) {
        const float* sp = state_in + static_cast<int64_t>(bh) * DK * DK;
#pragma unroll
        for (int v = 0; v < 16; ++v) Ms[dt][v] = sp[(32 * dt + acc_row(v, h)) * DK + col];
      } else {
        Ms[dt] = zero16();
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      *reinterpret_cast<bf16x8*>(sMf + (strip * 8 + ks) * 1024 + lane * 16) = acc_frag(Ms[ks >> 1], ks & 1);
  } else {
    const ChainSrc s0 = src_of(0);
    load_part_b(regB, s0, lt);
    load_part_a(regA, s0, lt);
    store_part_b(regB, smem, lt);
    store_part_a(regA, smem + L::kAlt, lt);
  }
  __syncthreads();

  for (int cl = 0; cl < nchunk; ++cl) {
    const int t0 = (c0 + cl) * CH;
    const int nval = min(CH, a.T - t0);
    const int64_t tokbase = static_cast<int64_t>(b) * a.T + t0;
    const unsigned char* alt = smem + L::kAlt + (cl & 1) * L::kAltBytes;
    const float* sSc = reinterpret_cast<const float*>(alt + L::kAltSc);
    if (state_wave) {
      // ---- phase 1: X = V - diag(gamma rk) K M ; U = T' X ; publish U ----
      floatx16 X[2];
      {
        // four independent accumulation chains (row tile x even/odd k step) keep the
        // MFMA pipe busy instead of waiting on one dependent chain
        floatx16 Xe[2] = {zero16(), zero16()}, Xo[2] = {zero16(), zero16()};
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
          const bf16x8 B0 = acc_frag(Ms[kp], 0), B1 = acc_frag(Ms[kp], 1);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(sK + (rt * 8 + 2 * kp) * 1024 + lane * 16);
            const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(sK + (rt * 8 + 2 * kp + 1) * 1024 + lane * 16);
            Xe[rt] = mfma32(A0, B0, Xe[rt]);
            Xo[rt] = mfma32(A1, B1, Xo[rt]);
          }
        }
        X[0] = Xe[0] + Xo[0];
        X[1] = Xe[1] + Xo[1];
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * rt + acc_row(v, h);
          X[rt][v] = fmaf(-sSc[r], X[rt][v], bf16_bits_to_f32(sV[r * RP + vcol]));
        }
      floatx16 U[2];
      {
        halfx8 Xf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Xf[ks] = acc_frag_h(X[ks >> 1], ks & 1);
        // T' X in fp16 with four independent accumulators (row tile x k-step parity)
        floatx16 Ue[2] = {zero16(), zero16()}, Uo[2] = {zero16(), zero16()};
#pragma unroll
        for (int f = 0; f < FT; ++f) {
          const int rt = f < 2 ? 0 : 1, ks = f < 2 ? f : f - 2;
          const halfx8 At = *reinterpret_cast<const halfx8*>(sTp + f * 1024 + lane * 16);
          if (ks & 1) Uo[rt] = mfma32h(At, Xf[ks], Uo[rt]);
          else Ue[rt] = mfma32h(At, Xf[ks], Ue[rt]);
        }
        U[0] = Ue[0] + Uo[0];
        U[1] = Ue[1] + Uo[1];
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        *reinterpret_cast<halfx8*>(sUf + (strip * 4 + ks) * 1024 + lane * 16) = acc_frag_h(U[ks >> 1], ks & 1);
      __syncthreads();  // B1: U published; Q M has read M
      // ---- phase 2: M <- gamma_63 M + K^T diag(rk e^{g_63-g}) U ; publish M ----
      {
        const unsigned char* sKt = alt + L::kAltKt;
        halfx8 Wf[4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int v = 0; v < 16; ++v) U[rt][v] *= sSc[128 + 32 * rt + acc_row(v, h)];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Wf[ks] = acc_frag_h(U[ks >> 1], ks & 1);
        const float gC = sSc[192];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) Ms[dt] *= gC;
        // four state tiles interleaved: four independent accumulation chains
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const halfx8 A = *reinterpret_cast<const halfx8*>(sKt + (dt * 4 + ks) * 1024 + lane * 16);
            Ms[dt] = mfma32h(A, Wf[ks], Ms[dt]);
          }
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        *reinterpret_cast<bf16x8*>(sMf + (strip * 8 + ks) * 1024 + lane * 16) = acc_frag(Ms[ks >> 1], ks & 1);
      __syncthreads();  // B2
    } else {
      // ---- phase 1: issue the next chunk's loads (part B first: it is consumed
      //      first); O = diag(gamma rq) Q M ----
      const bool more = cl + 1 < nchunk;
      if (more) {
        const ChainSrc sn = src_of(cl + 1);
        load_part_b(regB, sn, lt);
        load_part_a(regA, sn, lt);
      }
      floatx16 O[2];
      {
        floatx16 Oe[2] = {zero16(), zero16()}, Oo[2] = {zero16(), zero16()};
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
          const bf16x8 B0 = *reinterpret_cast<const bf16x8*>(sMf + (strip * 8 + 2 * kp) * 1024 + lane * 16);
          const bf16x8 B1 = *reinterpret_cast<const bf16x8*>(sMf + (strip * 8 + 2 * kp + 1) * 1024 + lane * 16);
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) {
            const bf16x8 A0 = *reinterpret_cast<const bf16x8*>(sQ + (rt * 8 + 2 * kp) * 1024 + lane * 16);
            const bf16x8 A1 = *reinterpret_cast<const bf16x8*>(sQ + (rt * 8 + 2 * kp + 1) * 1024 + lane * 16);
            Oe[rt] = mfma32(A0, B0, Oe[rt]);
            Oo[rt] = mfma32(A1, B1, Oo[rt]);
          }
        }
        O[0] = Oe[0] + Oo[0];
        O[1] = Oe[1] + Oo[1];
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[rt][v] *= sSc[64 + 32 * rt + acc_row(v, h)];
      __syncthreads();  // B1: wait for U; the primary buffer is free
      // ---- phase 2: stage part B of chunk cl+1 ; O += P U ; store O ; stage part A ----
      if (more) store_part_b(regB, smem, lt);
      {
        const unsigned char* sP = alt + L::kAltP;
        floatx16 Op[2] = {zero16(), zero16()};
#pragma unroll
        for (int f = 0; f < FT; ++f) {
          const int rt = f < 2 ? 0 : 1, ks = f < 2 ? f : f - 2;
          const halfx8 Pf = *reinterpret_cast<const halfx8*>(sP + f * 1024 + lane * 16);
          const halfx8 Uf = *reinterpret_cast<const halfx8*>(sUf + (strip * 4 + ks) * 1024 + lane * 16);
          if (ks & 1) Op[rt] = mfma32h(Pf, Uf, Op[rt]);
          else O[rt] = mfma32h(Pf, Uf, O[rt]);
        }
        O[0] += Op[0];
        O[1] += Op[1];
      }
      // O through LDS so that HBM sees 16-byte row segments
      uint16_t* sO = reinterpret_cast<uint16_t*>(smem + L::kO) + strip * CH * L::OP;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v) sO[(32 * rt + acc_row(v, h)) * L::OP + l32] = f32_to_bf16_bits(O[rt][v]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int vi = lane + 64 * m, r = vi >> 2, c8 = (vi & 3) * 8;
        if (r < nval)
          *reinterpret_cast<u16x8*>(go + (tokbase + r) * a.so + hv * DK + slice * DVS + 32 * strip + c8) =
              *reinterpret_cast<const u16x8*>(sO + r * L::OP + c8);
      }
      if (more) store_part_a(regA, smem + L::kAlt + ((cl + 1) & 1) * L::kAltBytes, lt);
      __syncthreads();  // B2
    }
  }

  if (state_wave && state_out) {
    float* sp = state_out + static_cast<int64_t>(bh) * DK * DK;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) sp[(32 * dt + acc_row(v, h)) * DK + col] = Ms[dt][v];
  }
}

}  // namespace

size_t chunk_ws_bytes_per_chunk(const RecArgs& a) {
  return static_cast<size_t>(a.B) * (static_cast<size_t>(a.Hv) * WS_CHUNK + static_cast<size_t>(a.Hk) * WS_KQ);
}

size_t chunk_ws_carry_bytes(const RecArgs& a) { return static_cast<size_t>(a.B) * a.Hv * DK * DK * 4; }

hipError_t launch_chunk_prefill(const RecArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_prep_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, PrepLds::kBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds::kBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int nchunks = (a.T + CH - 1) / CH;
  const size_t per_chunk = chunk_ws_bytes_per_chunk(a);
  // One window when the whole sequence fits; otherwise the state is carried
  // between windows through state_out (or a carry area at the workspace end).
  int nwin = static_cast<int>(ws_bytes / per_chunk);
  bool need_carry = false;
  if (nwin < nchunks) {
    need_carry = a.state_out == nullptr;
    const size_t carry_b = need_carry ? chunk_ws_carry_bytes(a) : 0;
    const size_t avail = ws_bytes > carry_b ? ws_bytes - carry_b : 0;
    nwin = static_cast<int>(avail / per_chunk);
  }
  if (nwin < 1) return hipErrorInvalidValue;
  if (nwin > nchunks) nwin = nchunks;
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  float* carry = need_carry ? reinterpret_cast<float*>(wsb + static_cast<size_t>(nwin) * per_chunk) : a.state_out;
  const float* sin = a.state_in;
  for (int c0 = 0; c0 < nchunks; c0 += nwin) {
    const int nw = min(nwin, nchunks - c0);
    const bool last = c0 + nw >= nchunks;
    float* sout = last ? a.state_out : carry;
    hipLaunchKernelGGL(chunk_prep_kernel, dim3(nw, a.Hk, a.B), dim3(256), PrepLds::kBytes, s, a, c0, wsb, nwin);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(chunk_chain_kernel, dim3(DK / DVS, a.Hv, a.B), dim3(256), ChainLds::kBytes, s, a, c0,
                       static_cast<const unsigned char*>(wsb), nwin, sin, sout);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    sin = sout;
  }
  return hipSuccess;
}

}  // namespace gdn
