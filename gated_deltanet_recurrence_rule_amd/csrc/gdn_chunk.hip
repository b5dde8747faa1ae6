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
//    MFMA A-operand fragments (bf16 hi + lo pairs) plus three row-scaling
//    vectors per (chunk, value head).
//  * chain (one workgroup per sequence, value head and 64 value columns,
//    looping over the chunks): only the state-dependent products.  Columns of
//    M evolve independently; waves 0-1 ("state") each own a 32-column strip
//    of M in MFMA accumulators for the whole window and compute
//    K M, X, U = T'X and the update; waves 2-3 ("output") compute
//    Q M and P U for the same strips from fragments the state waves publish
//    in LDS, so the output work runs beside the critical path.  The next
//    chunk's inputs are prefetched into registers while a chunk computes.
//
// Precision.  MFMA operands are bf16 with fp32 accumulation.  Genuine bf16
// inputs (K, Q, V) enter as they are.  fp32 operands whose rounding would
// reach the state or output tolerance are split into hi + lo bf16 pairs:
// T' and X in T'X (3 products), P and U in P U (3), U' in K^T U' (2).  M
// enters K M and Q M as a single bf16.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, wave64): A row = B column =
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

constexpr int CH = 64;    // chunk length
constexpr int DK = 128;   // head width
constexpr int KP = 136;   // LDS row pitch (bf16) of 64 x 128 K / Q tiles
constexpr int RP = 72;    // LDS row pitch (bf16) of K^T and of the V slice
constexpr int FP = 65;    // LDS row pitch (floats) of fp32 64 x 64 matrices
constexpr int DVS = 64;   // value columns per chain workgroup
constexpr int FT = 6;     // 32x16 fragment tiles covering a 64x64 lower triangle
constexpr int WS_TP = 2 * FT * 2 * 1024;  // T' and P fragments, hi and lo
constexpr int WS_CHUNK = WS_TP + 1024;    // + grk[64], grq[64], drk[64], gamma_63

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

__device__ __forceinline__ bf16x8 acc_frag(const floatx16& t, int s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(t[8 * s + e]);
  return r;
}

__device__ __forceinline__ void acc_frag_split(const floatx16& t, int s, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = t[8 * s + e];
    const __bf16 hb = static_cast<__bf16>(x);
    hi[e] = hb;
    lo[e] = static_cast<__bf16>(x - static_cast<float>(hb));
  }
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
  static constexpr int kY = kQK + CH * FP * 4;        // fp32 32 x 33 (or 2 x 16 x 17)
  static constexpr int kVec = kY + 32 * 33 * 4;       // rk, rq, g, beta
  static constexpr int kBytes = kVec + 4 * CH * 4;
};

__global__ __launch_bounds__(256, 2) void chunk_prep_kernel(RecArgs a, int c0, unsigned char* ws, int nwin) {
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
    // ---- A (fp32, strictly lower) and the P fragments ----------------------
    for (int e = tid; e < CH * CH; e += 256) {
      const int r = e >> 6, i = e & 63;
      float av = 0.f;
      if (i < r) av = vBe[r] * __expf(vG[r] - vG[i]) * vRk[r] * vRk[i] * sKK[r * FP + i];
      sA[r * FP + i] = av;
    }
    for (int slot = tid; slot < FT * 64; slot += 256) {
      const int f = slot >> 6, ln = slot & 63;
      const int r = 32 * ft_rt(f) + (ln & 31), hh = ln >> 5;
      u16x8 hi, lo;
      const float gr = vG[r], rq = vRq[r];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 16 * ft_ks(f) + kperm(hh, e);
        const float pv = (i <= r) ? __expf(gr - vG[i]) * rq * vRk[i] * sQK[r * FP + i] : 0.f;
        const __bf16 hb = static_cast<__bf16>(pv);
        hi[e] = __builtin_bit_cast(uint16_t, hb);
        lo[e] = f32_to_bf16_bits(pv - static_cast<float>(hb));
      }
      *reinterpret_cast<u16x8*>(wsc + ((6 + f) * 2 + 0) * 1024 + ln * 16) = hi;
      *reinterpret_cast<u16x8*>(wsc + ((6 + f) * 2 + 1) * 1024 + ln * 16) = lo;
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
      float y0 = 0.f, y1 = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float av = sA[(16 * I + yr) * FP + 16 * J + m];
        y0 = fmaf(av, sT[(16 * J + m) * FP + 16 * J + yc], y0);
        y1 = fmaf(av, sT[(16 * J + m) * FP + 16 * J + yc + 1], y1);
      }
      sY[half * 16 * 17 + yr * 17 + yc] = y0;
      sY[half * 16 * 17 + yr * 17 + yc + 1] = y1;
      __syncthreads();
      float t0v = 0.f, t1v = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float tv = sT[(16 * I + yr) * FP + 16 * I + m];
        t0v = fmaf(tv, sY[half * 16 * 17 + m * 17 + yc], t0v);
        t1v = fmaf(tv, sY[half * 16 * 17 + m * 17 + yc + 1], t1v);
      }
      sT[(16 * I + yr) * FP + 16 * J + yc] = -t0v;
      sT[(16 * I + yr) * FP + 16 * J + yc + 1] = -t1v;
    }
    __syncthreads();
    // level 2: T[32:64, 0:32] = -S1 (A[32:64, 0:32] S0), S0/S1 the 32x32 diagonal inverses
    {
      const int idx = tid * 4;
      const int yr = idx >> 5, yc = idx & 31;
      floatx4 y = {0.f, 0.f, 0.f, 0.f};
      for (int m = yc; m < 32; ++m) {  // S0 is lower-triangular: rows m >= yc only
        const float av = sA[(32 + yr) * FP + m];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fmaf(av, sT[m * FP + yc + e], y[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sY[yr * 33 + yc + e] = y[e];
      __syncthreads();
      floatx4 t = {0.f, 0.f, 0.f, 0.f};
      for (int m = 0; m <= yr; ++m) {  // S1 is lower-triangular: columns m <= yr only
        const float tv = sT[(32 + yr) * FP + 32 + m];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = fmaf(tv, sY[m * 33 + yc + e], t[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sT[(32 + yr) * FP + yc + e] = -t[e];
    }
    __syncthreads();
    // ---- T' = T diag(beta) fragments ----------------------------------------
    for (int slot = tid; slot < FT * 64; slot += 256) {
      const int f = slot >> 6, ln = slot & 63;
      const int r = 32 * ft_rt(f) + (ln & 31), hh = ln >> 5;
      u16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 16 * ft_ks(f) + kperm(hh, e);
        const float tv = (i <= r) ? sT[r * FP + i] * vBe[i] : 0.f;
        const __bf16 hb = static_cast<__bf16>(tv);
        hi[e] = __builtin_bit_cast(uint16_t, hb);
        lo[e] = f32_to_bf16_bits(tv - static_cast<float>(hb));
      }
      *reinterpret_cast<u16x8*>(wsc + (f * 2 + 0) * 1024 + ln * 16) = hi;
      *reinterpret_cast<u16x8*>(wsc + (f * 2 + 1) * 1024 + ln * 16) = lo;
    }
    __syncthreads();  // vG, vBe, sA, sT are rewritten for the next value head
  }
}

// =========================================================================
// chain kernel: one workgroup (4 waves) per (64-column slice, value head, batch)
// =========================================================================
struct ChainLds {
  static constexpr int kK = 0;                        // bf16 [64][KP]
  static constexpr int kQ = kK + CH * KP * 2;         // bf16 [64][KP]
  static constexpr int kKt = kQ + CH * KP * 2;        // bf16 [128][RP]
  static constexpr int kV = kKt + DK * RP * 2;        // bf16 [64][RP]
  static constexpr int kTP = kV + CH * RP * 2;        // fragments, WS_TP bytes
  static constexpr int kSc = kTP + WS_TP;             // 256 floats
  static constexpr int kMf = kSc + 1024;              // M B-fragments: [2 strips][8 k steps][64 lanes] x 16 B
  static constexpr int kUf = kMf + 2 * 8 * 1024;      // U B-fragments: [2 strips][4 k steps][hi/lo][64] x 16 B
  static constexpr int kBytes = kUf + 2 * 4 * 2 * 1024;
};

// Per-thread prefetch of one chunk's chain inputs (global -> registers).
struct ChainPrefetch {
  u16x8 kq[8];   // an 8x8 block of K (threads 0-127) or Q (threads 128-255)
  u16x8 v[2];
  u32x4 tp[6];
  floatx4 sc;
};

__device__ __forceinline__ void chain_prefetch(ChainPrefetch& pf, const RecArgs& a, const unsigned char* wsc,
                                               int64_t tokbase, int nval, int hk, int h, int slice, int tid) {
  const int which = tid >> 7, blk = tid & 127;
  const int br = blk >> 4, bc = blk & 15;
  const uint16_t* src = static_cast<const uint16_t*>(which == 0 ? a.k : a.q);
  const int64_t st = which == 0 ? a.sk : a.sq;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 8 * br + j;
    pf.kq[j] = (r < nval) ? *reinterpret_cast<const u16x8*>(src + (tokbase + r) * st + hk * DK + 8 * bc)
                          : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  const uint16_t* gv = static_cast<const uint16_t*>(a.v);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int vi = tid + 256 * j;
    const int r = vi >> 3, c8 = (vi & 7) * 8;
    pf.v[j] = (r < nval) ? *reinterpret_cast<const u16x8*>(gv + (tokbase + r) * a.sv + h * DK + slice * DVS + c8)
                         : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < 6; ++j) pf.tp[j] = reinterpret_cast<const u32x4*>(wsc)[tid + 256 * j];
  if (tid < 64) pf.sc = reinterpret_cast<const floatx4*>(wsc + WS_TP)[tid];
}

__device__ __forceinline__ void chain_stage(const ChainPrefetch& pf, unsigned char* smem, int tid) {
  using L = ChainLds;
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + L::kK);
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + L::kQ);
  uint16_t* sKt = reinterpret_cast<uint16_t*>(smem + L::kKt);
  uint16_t* sV = reinterpret_cast<uint16_t*>(smem + L::kV);
  const int which = tid >> 7, blk = tid & 127;
  const int br = blk >> 4, bc = blk & 15;
  uint16_t* dst = which == 0 ? sK : sQ;
#pragma unroll
  for (int j = 0; j < 8; ++j) *reinterpret_cast<u16x8*>(dst + (8 * br + j) * KP + 8 * bc) = pf.kq[j];
  if (which == 0) {  // K^T: transpose the 8x8 block in registers
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      u16x8 col;
#pragma unroll
      for (int j = 0; j < 8; ++j) col[j] = pf.kq[j][cc];
      *reinterpret_cast<u16x8*>(sKt + (8 * bc + cc) * RP + 8 * br) = col;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int vi = tid + 256 * j;
    *reinterpret_cast<u16x8*>(sV + (vi >> 3) * RP + (vi & 7) * 8) = pf.v[j];
  }
#pragma unroll
  for (int j = 0; j < 6; ++j) reinterpret_cast<u32x4*>(smem + L::kTP)[tid + 256 * j] = pf.tp[j];
  if (tid < 64) reinterpret_cast<floatx4*>(smem + L::kSc)[tid] = pf.sc;
}

__global__ __launch_bounds__(256) void chunk_chain_kernel(RecArgs a, int c0, const unsigned char* ws, int nwin,
                                                          const float* state_in, float* state_out) {
  using L = ChainLds;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const uint16_t* sK = reinterpret_cast<const uint16_t*>(smem + L::kK);
  const uint16_t* sQ = reinterpret_cast<const uint16_t*>(smem + L::kQ);
  const uint16_t* sKt = reinterpret_cast<const uint16_t*>(smem + L::kKt);
  const uint16_t* sV = reinterpret_cast<const uint16_t*>(smem + L::kV);
  const unsigned char* sTP = smem + L::kTP;
  const float* sSc = reinterpret_cast<const float*>(smem + L::kSc);
  unsigned char* sMf = smem + L::kMf;
  unsigned char* sUf = smem + L::kUf;

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int slice = blockIdx.x, hv = blockIdx.y, b = blockIdx.z;
  const int hk = hv / a.G;
  const int bh = b * a.Hv + hv;
  const int strip = wv & 1;                    // 32-column strip inside the slice
  const bool state_wave = wv < 2;
  const int col = slice * DVS + 32 * strip + l32;  // this lane's value column (global)
  const int vcol = 32 * strip + l32;               // ... inside the V slice
  uint16_t* go = static_cast<uint16_t*>(a.o);

  const int nchunk = min(nwin, (a.T + CH - 1) / CH - c0);
  auto wsc_of = [&](int cl) { return ws + (static_cast<int64_t>(bh) * nwin + cl) * WS_CHUNK; };

  // State strip (state waves): 4 tiles of 32 key rows x 32 value columns.
  floatx16 Ms[4];
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
    // publish M as B fragments for the output waves' Q M
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      *reinterpret_cast<bf16x8*>(sMf + (strip * 8 + ks) * 1024 + lane * 16) = acc_frag(Ms[ks >> 1], ks & 1);
  }

  ChainPrefetch pf;
  {
    const int t0 = c0 * CH;
    chain_prefetch(pf, a, wsc_of(0), static_cast<int64_t>(b) * a.T + t0, min(CH, a.T - t0), hk, hv, slice, tid);
    chain_stage(pf, smem, tid);
  }
  __syncthreads();

  for (int cl = 0; cl < nchunk; ++cl) {
    const int t0 = (c0 + cl) * CH;
    const int nval = min(CH, a.T - t0);
    const int64_t tokbase = static_cast<int64_t>(b) * a.T + t0;
    if (cl + 1 < nchunk) {
      const int t1 = t0 + CH;
      chain_prefetch(pf, a, wsc_of(cl + 1), tokbase + CH, min(CH, a.T - t1), hk, hv, slice, tid);
    }
    if (state_wave) {
      // X = V - diag(gamma rk) K M
      floatx16 X[2] = {zero16(), zero16()};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 Bm = acc_frag(Ms[ks >> 1], ks & 1);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          X[rt] = mfma32(lds_frag32(sK + (32 * rt + l32) * KP + 16 * ks, h), Bm, X[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * rt + acc_row(v, h);
          X[rt][v] = bf16_bits_to_f32(sV[r * RP + vcol]) - sSc[r] * X[rt][v];
        }
      // U = T' X
      floatx16 U[2] = {zero16(), zero16()};
      {
        bf16x8 Xh[4], Xl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc_frag_split(X[ks >> 1], ks & 1, Xh[ks], Xl[ks]);
#pragma unroll
        for (int f = 0; f < FT; ++f) {
          const int rt = f < 2 ? 0 : 1, ks = f < 2 ? f : f - 2;
          const bf16x8 Ah = *reinterpret_cast<const bf16x8*>(sTP + (f * 2 + 0) * 1024 + lane * 16);
          const bf16x8 Al = *reinterpret_cast<const bf16x8*>(sTP + (f * 2 + 1) * 1024 + lane * 16);
          U[rt] = mfma32(Ah, Xh[ks], U[rt]);
          U[rt] = mfma32(Ah, Xl[ks], U[rt]);
          U[rt] = mfma32(Al, Xh[ks], U[rt]);
        }
      }
      // publish U (hi/lo B fragments) for P U
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 hi, lo;
        acc_frag_split(U[ks >> 1], ks & 1, hi, lo);
        *reinterpret_cast<bf16x8*>(sUf + ((strip * 4 + ks) * 2 + 0) * 1024 + lane * 16) = hi;
        *reinterpret_cast<bf16x8*>(sUf + ((strip * 4 + ks) * 2 + 1) * 1024 + lane * 16) = lo;
      }
      __syncthreads();  // (1) U published; the output waves' Q M has read sMf
      // M <- gamma_63 M + K^T diag(rk e^{g_63-g}) U
      {
        bf16x8 Wh[4], Wl[4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int v = 0; v < 16; ++v) U[rt][v] *= sSc[128 + 32 * rt + acc_row(v, h)];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc_frag_split(U[ks >> 1], ks & 1, Wh[ks], Wl[ks]);
        const float gC = sSc[192];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          Ms[dt] *= gC;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 A = lds_frag32(sKt + (32 * dt + l32) * RP + 16 * ks, h);
            Ms[dt] = mfma32(A, Wh[ks], Ms[dt]);
            Ms[dt] = mfma32(A, Wl[ks], Ms[dt]);
          }
        }
      }
      // M for the next chunk's Q M
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        *reinterpret_cast<bf16x8*>(sMf + (strip * 8 + ks) * 1024 + lane * 16) = acc_frag(Ms[ks >> 1], ks & 1);
    } else {
      // output waves: O = diag(gamma rq) Q M + P U
      floatx16 O[2] = {zero16(), zero16()};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 Bm = *reinterpret_cast<const bf16x8*>(sMf + (strip * 8 + ks) * 1024 + lane * 16);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          O[rt] = mfma32(lds_frag32(sQ + (32 * rt + l32) * KP + 16 * ks, h), Bm, O[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[rt][v] *= sSc[64 + 32 * rt + acc_row(v, h)];
      __syncthreads();  // (1) wait for U
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        const int rt = f < 2 ? 0 : 1, ks = f < 2 ? f : f - 2;
        const bf16x8 Ph = *reinterpret_cast<const bf16x8*>(sTP + ((6 + f) * 2 + 0) * 1024 + lane * 16);
        const bf16x8 Pl = *reinterpret_cast<const bf16x8*>(sTP + ((6 + f) * 2 + 1) * 1024 + lane * 16);
        const bf16x8 Uh = *reinterpret_cast<const bf16x8*>(sUf + ((strip * 4 + ks) * 2 + 0) * 1024 + lane * 16);
        const bf16x8 Ul = *reinterpret_cast<const bf16x8*>(sUf + ((strip * 4 + ks) * 2 + 1) * 1024 + lane * 16);
        O[rt] = mfma32(Ph, Uh, O[rt]);
        O[rt] = mfma32(Ph, Ul, O[rt]);
        O[rt] = mfma32(Pl, Uh, O[rt]);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * rt + acc_row(v, h);
          if (r < nval) go[(tokbase + r) * a.so + hv * DK + col] = f32_to_bf16_bits(O[rt][v]);
        }
    }
    __syncthreads();  // (2) every wave is done with this chunk's LDS inputs
    if (cl + 1 < nchunk) chain_stage(pf, smem, tid);
    __syncthreads();  // (3) next chunk staged
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

size_t chunk_ws_bytes_per_chunk(const RecArgs& a) { return static_cast<size_t>(a.B) * a.Hv * WS_CHUNK; }

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
