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
// exponent is <= 0.  Everything that does not depend on the state is folded
// before the serial loop:
//
//   W  = T' diag(gamma rk) K,   U0 = T' V,   Kd = K^T diag(rk e^{g_63 - g}),
//   Q^ = diag(rq) Q,            so that per chunk
//   U  = U0 - W M,   M <- gamma_63 M + Kd U,   O = diag(gamma) Q^ M + P U.
//
// Two kernels per window of chunks:
//  * prep (one workgroup per chunk and key head, fully parallel over chunks):
//    row norms, the Gram products K K^T and K Q^T (bf16 MFMA, kept in
//    registers), and per value head the gate prefix sums, A, the inverse
//    (16x16 forward substitution, a 16-block merge on fp32 MFMA, and the
//    32x32 merge on MFMA with split-fp16 operands), T', and the products -W
//    and U0 (fp16 MFMA).  The value heads of a key head are inverted up to
//    three at a time, each on its own wave and in place.  All of it is
//    written to the workspace as MFMA-ready fp16 fragments; U0 in the
//    accumulator layout of the chain's U.
//  * chain (one workgroup per sequence, value head and 32-column strip of M,
//    looping over the window's chunks; columns of M evolve independently).
//    One wave carries the fp32 strip of M in registers and runs the serial
//    path: 16 MFMAs for U = U0 - W M, 16 for the update.  A second wave forms
//    the outputs from the M and U fragments the first publishes in LDS; a
//    third copies the next operands from the workspace into LDS two chunks
//    ahead with direct global-to-LDS loads.
//
// Precision.  MFMA accumulation is fp32 throughout and the state stays fp32.
// The Gram products take the bf16 inputs as they are; every other product
// runs on fp16 operands, each rounded once (in prep: -W, Kd, U0, P, Q^; in
// the chain: M and U).  fp16 keeps 11 significant bits, which holds the state
// within a few 1e-4 of the exact result and the outputs well inside their
// bound; its range (|x| < 65504) bounds the values of v, the state and the
// intra-chunk matrices this path accepts.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16 and _f16, wave64): A row = B column =
// lane & 31; the accumulator holds column lane & 31, rows 8j + 4h + i
// (h = lane >> 5, value index 4j + i).  The contraction index is permuted the
// same way on A and B: inside each 16-wide k step, lane half h carries
// k = 4h..4h+3 and 8+4h..8+4h+3.  With that permutation accumulator values
// [8s, 8s+8) of a tile are directly the B operand for k step s of that tile,
// so M and U feed the next product from registers, and a product computed in
// transposed form (C^T = B^T A^T) leaves its result as an A fragment.
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
constexpr int KP = 136;   // LDS row pitch (bf16) of 64 x 128 row tiles
constexpr int FP = 68;    // LDS row pitch (floats) of fp32 64 x 64 matrices (16-byte rows)
constexpr int FT = 6;     // 32x16 fragment tiles covering a 64x64 lower triangle
// workspace block per (batch, value head, chunk): fp16 MFMA fragments and fp32 scalings
constexpr int WH_W = 0;        // -W = -T' diag(gamma rk) K: tile rt*8+ks (rows 32rt.., key step ks)
constexpr int WH_KD = 16384;   // Kd = K^T diag(rk e^{g_63-g}): tile dt*4+ks (keys 32dt.., chunk step ks)
constexpr int WH_U0 = 32768;   // U0 = T' V in accumulator layout: [value tile 4][row tile 2][lane 64][16]
constexpr int WH_P = 49152;    // P: 6 tiles of the lower triangle
constexpr int WH_SC = 55296;   // gamma_r (64 floats), gamma_63
constexpr int WH_BYTES = 56320;
// workspace block per (batch, key head, chunk): Q^ = diag(rq) Q fragments, tile rt*8+ks
constexpr int WK_BYTES = 16384;

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
// LDS: the chunk's K and Q rows (bf16, padded rows) while the norms, the Q^
// fragments and the Gram products are formed; then, over the same bytes, one
// fp32 64 x 64 matrix per value head of the current group of up to three,
// stored as its three lower 32 x 32 tiles (0,0), (1,0), (1,1): A, which the
// wave owning the head turns into T = (I + A)^-1 in place.  After them each
// wave's tile of a value head's V (64 rows x its 32 columns), then the row
// scalings rk, rq and per value head the gate vectors.
struct PrepLds {
  static constexpr int kNH = 3;                   // value heads per group (waves 0-2 invert one each)
  static constexpr int kTP = 36;                  // tile row pitch in floats (16-byte rows)
  static constexpr int kTile = 32 * kTP;          // floats per tile
  static constexpr int kMat = 3 * kTile * 4;      // bytes per head
  static constexpr int kK = 0;                    // bf16 [64][KP]
  static constexpr int kQ = CH * KP * 2;          // bf16 [64][KP]
  static constexpr int kVP = 40;                  // V tile row pitch (bf16): 80-byte rows
  static constexpr int kV = kNH * kMat > 2 * CH * KP * 2 ? kNH * kMat : 2 * CH * KP * 2;
  static constexpr int kVec = kV + 4 * CH * kVP * 2;
  static constexpr int bytes(int G) { return kVec + (2 + 4 * G) * CH * 4; }
};

// Orders one wave's LDS accesses across its lanes: the wave's LDS instructions
// execute in program order, so only the compiler has to keep them there.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ floatx4 mfma16f32(float a, float b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// T = (I + A)^-1 of one 64 x 64 strictly lower A (tiles of pitch kTP), in place,
// by one wave.  Unit lower-triangular blocks: the four diagonal 16 x 16 blocks by
// forward substitution, then T_IJ = -T_II A_IJ T_JJ for the 16-blocks (1,0) and
// (3,2), then the same for the 32-blocks, T_10 = -T_11 A_10 T_00.
__device__ __forceinline__ void invert_unit_lower(float* M, int lane) {
  using L = PrepLds;
  const int l32 = lane & 31, h = lane >> 5;
  {
    // lane = (block, column jc): x = column jc of the block's inverse,
    // x_s = [s == jc] - sum_{r<s} A_sr x_r, taking the columns of A four at a time
    const int blk = lane >> 4, jc = lane & 15;
    float* D = M + (blk >> 1) * 2 * L::kTile + (blk & 1) * 16 * (L::kTP + 1);
    float x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = s == jc ? 1.f : 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      floatx4 ap[16];
#pragma unroll
      for (int s = 4 * p + 1; s < 16; ++s) ap[s] = *reinterpret_cast<const floatx4*>(D + s * L::kTP + 4 * p);
#pragma unroll
      for (int s = 4 * p + 1; s < 16; ++s)
#pragma unroll
        for (int r = 4 * p; r < (s < 4 * p + 4 ? s : 4 * p + 4); ++r) x[s] = fmaf(-ap[s][r - 4 * p], x[r], x[s]);
    }
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < 16; ++s) D[s * L::kTP + jc] = x[s];
  }
  wave_lds_sync();
  {
    // 16-blocks (1,0) in tile (0,0) and (3,2) in tile (1,1), each at rows 16.., columns
    // 0.. of its tile, on fp32 MFMA (16x16x4: A row = B column = lane & 15, k = lane >> 4;
    // the result holds column lane & 15, rows 4 (lane >> 4) + v).  Y = A_IJ T_JJ; in the
    // second product the k index runs over 4 (lane >> 4) + s so that Y's values are
    // its B operand as they stand.
    const int q = lane >> 4, n = lane & 15;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      float* Tt = M + 2 * m * L::kTile;
      floatx4 Y = {0.f, 0.f, 0.f, 0.f}, Z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) Y = mfma16f32(Tt[(16 + n) * L::kTP + 4 * s + q], Tt[(4 * s + q) * L::kTP + n], Y);
#pragma unroll
      for (int s = 0; s < 4; ++s) Z = mfma16f32(Tt[(16 + n) * L::kTP + 16 + 4 * q + s], Y[s], Z);
      wave_lds_sync();
#pragma unroll
      for (int v = 0; v < 4; ++v) Tt[(16 + 4 * q + v) * L::kTP + n] = -Z[v];
    }
  }
  wave_lds_sync();
  {
    // 32-blocks: tile (1,0) <- -T_11 (A_10 T_00) on MFMA, each fp32 operand split into
    // fp16 hi + lo and three products kept (hi hi, hi lo, lo hi): about 22 bits
    const float* T0 = M;
    float* T1 = M + L::kTile;
    const float* T2 = M + 2 * L::kTile;
    floatx16 Y = zero16(), Y2 = zero16();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float* ar = T1 + l32 * L::kTP + 16 * ks + 4 * h;
      const floatx4 a0 = *reinterpret_cast<const floatx4*>(ar), a1 = *reinterpret_cast<const floatx4*>(ar + 8);
      halfx8 ahi, alo, bhi, blo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float av = e < 4 ? a0[e] : a1[e - 4];
        const float bv = T0[(16 * ks + kperm(h, e)) * L::kTP + l32];
        ahi[e] = static_cast<_Float16>(av);
        alo[e] = static_cast<_Float16>(av - static_cast<float>(ahi[e]));
        bhi[e] = static_cast<_Float16>(bv);
        blo[e] = static_cast<_Float16>(bv - static_cast<float>(bhi[e]));
      }
      Y = mfma32h(ahi, bhi, Y);
      Y2 = mfma32h(ahi, blo, Y2);
      Y2 = mfma32h(alo, bhi, Y2);
    }
    Y += Y2;
    floatx16 Z = zero16(), Z2 = zero16();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const float* sr = T2 + l32 * L::kTP + 16 * ks + 4 * h;
      const floatx4 a0 = *reinterpret_cast<const floatx4*>(sr), a1 = *reinterpret_cast<const floatx4*>(sr + 8);
      halfx8 ahi, alo, bhi, blo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float av = e < 4 ? a0[e] : a1[e - 4];
        const float bv = Y[8 * ks + e];   // accumulator values [8ks, 8ks+8) are the B fragment
        ahi[e] = static_cast<_Float16>(av);
        alo[e] = static_cast<_Float16>(av - static_cast<float>(ahi[e]));
        bhi[e] = static_cast<_Float16>(bv);
        blo[e] = static_cast<_Float16>(bv - static_cast<float>(bhi[e]));
      }
      Z = mfma32h(ahi, bhi, Z);
      Z2 = mfma32h(ahi, blo, Z2);
      Z2 = mfma32h(alo, bhi, Z2);
    }
    Z += Z2;
    wave_lds_sync();
#pragma unroll
    for (int v = 0; v < 16; ++v) T1[acc_row(v, h) * L::kTP + l32] = -Z[v];
  }
}

// kOneGroup: at most kNH value heads per key head, so that the Gram tiles die
// after the first group's A and P.
template <bool kOneGroup>
__global__ __launch_bounds__(256, 2) void chunk_prep_kernel(RecArgs a, int c0, unsigned char* ws, int nwin) {
  // workspace: region H = [B][Hv][nwin] x WH_BYTES, then region K = [B][Hk][nwin] x WK_BYTES
  using L = PrepLds;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + L::kK);
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + L::kQ);
  float* vRk = reinterpret_cast<float*>(smem + L::kVec);
  float* vRq = vRk + CH;
  // gate vectors of value head j of this key head
  auto vgate = [&](int j) { return vRk + (2 + 4 * j) * CH; };
  // matrix of head jj of the current group
  auto mat = [&](int jj) { return reinterpret_cast<float*>(smem + jj * L::kMat); };

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int cl = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int c = c0 + cl;
  int nval;
  int64_t tokbase;
  if (a.cu_seqlens) {
    // packed sequences: global chunk c is chunk c - chunk_start[s] of sequence s
    const int s = a.chunk_seq[c];
    if (s >= a.nseq) return;  // past the last chunk: the whole workgroup leaves
    int len;
    int64_t start;
    packed_range(a.cu_seqlens, s, a.T, start, len);
    const int t0 = (c - a.chunk_start[s]) * CH;
    tokbase = start + t0;
    nval = min(CH, len - t0);
  } else {
    const int t0 = c * CH;
    nval = min(CH, a.T - t0);
    tokbase = static_cast<int64_t>(b) * a.T + t0;
  }
  const bool l2 = (a.flags & 1u) != 0;
  const uint16_t* gq = static_cast<const uint16_t*>(a.q);
  const uint16_t* gk = static_cast<const uint16_t*>(a.k);
  const uint16_t* gv = static_cast<const uint16_t*>(a.v);

  // The V values this wave needs for a value head's U0 product are its value
  // tile, columns 32 wv.. of the 64 rows: loaded into registers one head ahead,
  // 16 bytes a lane, rows 16 m + (lane >> 2) (rows past the sequence end read the
  // last valid row and are replaced by zeros), and staged through the wave's own
  // LDS tile, from which the k-ordered B operand is read.  The first head's loads
  // are issued before the K and Q rows are waited for, and wave w loads the gates
  // of value head w as well.
  u32x4 vr[4];
  auto load_v = [&](int hv) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = 16 * m + (lane >> 2), rr = r < nval ? r : nval - 1;
      vr[m] = *reinterpret_cast<const u32x4*>(gv + (tokbase + rr) * a.sv + hv * DK + 32 * wv + 8 * (lane & 3));
    }
  };
  uint16_t* sVw = reinterpret_cast<uint16_t*>(smem + L::kV) + wv * CH * L::kVP;
  load_v(hk * a.G);
  const int tr = lane < nval ? lane : nval - 1;
  float la = 0.f, be = 0.f;
  if (wv < a.G) {
    la = a.la[(tokbase + tr) * a.Hv + hk * a.G + wv];
    be = a.beta[(tokbase + tr) * a.Hv + hk * a.G + wv];
  }

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

  // ---- gates of every value head: prefix sums and the row scalings ----------
  for (int j = wv; j < a.G; j += 4) {
    if (j != wv) {
      la = a.la[(tokbase + tr) * a.Hv + hk * a.G + j];
      be = a.beta[(tokbase + tr) * a.Hv + hk * a.G + j];
    }
    if (lane >= nval) la = be = 0.f;
    float g = la;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float t = __shfl_up(g, off, 64);
      if (lane >= off) g += t;
    }
    const float gl = __shfl(g, 63, 64);
    const float eg = __expf(g);
    float* vg = vgate(j);
    vg[lane] = g;
    vg[CH + lane] = be;
    vg[2 * CH + lane] = eg * vRk[lane];
    vg[3 * CH + lane] = __expf(gl - g) * vRk[lane];
    float* sc = reinterpret_cast<float*>(ws + (static_cast<int64_t>(b * a.Hv + hk * a.G + j) * nwin + cl) * WH_BYTES + WH_SC);
    sc[lane] = eg;
    if (lane == 0) sc[64] = __expf(gl);
  }

  // ---- Q^ = diag(rq) Q as the output product's A fragments (fp16) -----------
  //      tile rt*8+ks holds rows 32rt + (lane&31), k = 16ks + kperm
  {
    unsigned char* wsk = ws + static_cast<int64_t>(a.B) * a.Hv * nwin * WH_BYTES +
                         (static_cast<int64_t>(b * a.Hk + hk) * nwin + cl) * WK_BYTES;
    for (int slot = tid; slot < 16 * 64; slot += 256) {
      const int tile = slot >> 6, ln = slot & 63;
      const int r = 32 * (tile >> 3) + (ln & 31), hh = ln >> 5;
      const uint16_t* src = sQ + r * KP + 16 * (tile & 7);
      const u16x4 lo = *reinterpret_cast<const u16x4*>(src + 4 * hh);
      const u16x4 hi = *reinterpret_cast<const u16x4*>(src + 8 + 4 * hh);
      const float rq = vRq[r];
      u16x8 f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = f32_to_f16_bits(bf16_bits_to_f32(lo[e]) * rq);
        f[4 + e] = f32_to_f16_bits(bf16_bits_to_f32(hi[e]) * rq);
      }
      *reinterpret_cast<u16x8*>(wsk + tile * 1024 + ln * 16) = f;
    }
  }
  // ---- this wave's columns of K^T (key rows 32 wv + (lane&31)) at the chunk rows
  //      of each 16-row k step, in fragment order; scaled per value head below
  u16x8 kt[4];
  {
    const int d = 32 * wv + l32;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) kt[ks][e] = sK[(16 * ks + kperm(h, e)) * KP + d];
  }
  // ---- Gram tiles (32x32), kept in registers of waves 0-2 -------------------
  //  K K^T tile (rtK, ctK) in {(0,0), (1,0), (1,1)} -- tile wv of the lower
  //  triangle: element (row r, column i) = k_r . k_i
  //  K Q^T tile (itP, rtP) in {(0,0), (0,1), (1,1)}: element (row i, column r) = k_i . q_r
  const int rtK = wv == 0 ? 0 : 1, ctK = wv == 2 ? 1 : 0;
  const int itP = wv == 2 ? 1 : 0, rtP = wv == 0 ? 0 : 1;
  floatx16 gKK = zero16(), gKQ = zero16();
  if (wv < 3) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      gKK = mfma32(lds_frag32(sK + (32 * rtK + l32) * KP + 16 * ks, h),
                   lds_frag32(sK + (32 * ctK + l32) * KP + 16 * ks, h), gKK);
      gKQ = mfma32(lds_frag32(sK + (32 * itP + l32) * KP + 16 * ks, h),
                   lds_frag32(sQ + (32 * rtP + l32) * KP + 16 * ks, h), gKQ);
    }
  }
  __syncthreads();  // the K and Q rows are dead from here on: their bytes hold the matrices

  // Value heads in groups of up to kNH: A and P of the group from the Gram tiles,
  // then each head's inverse on its own wave, then the products of each head.
  for (int j0 = 0; j0 < (kOneGroup ? 1 : a.G); j0 += L::kNH) {
    const int ng = kOneGroup ? a.G : min(L::kNH, a.G - j0);
    // ---- A (fp32, strictly lower; tile wv) and the P fragments --------------
    if (wv < 3) {
      for (int jj = 0; jj < ng; ++jj) {
        const int j = j0 + jj;
        const float* vG = vgate(j);
        const float* vBe = vG + CH;
        {
          float* At = mat(jj) + wv * L::kTile;
          const int i = 32 * ctK + l32;
          const float gi = vG[i], rki = vRk[i];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r0 = 32 * rtK + 8 * q + 4 * h;
            const floatx4 g4 = *reinterpret_cast<const floatx4*>(vG + r0);
            const floatx4 b4 = *reinterpret_cast<const floatx4*>(vBe + r0);
            const floatx4 k4 = *reinterpret_cast<const floatx4*>(vRk + r0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = r0 + e;
              const float x = b4[e] * k4[e] * rki * __expf(fminf(g4[e] - gi, 0.f)) * gKK[4 * q + e];
              At[(8 * q + 4 * h + e) * L::kTP + l32] = i < r ? x : 0.f;
            }
          }
        }
        {
          unsigned char* wsc = ws + (static_cast<int64_t>(b * a.Hv + hk * a.G + j) * nwin + cl) * WH_BYTES;
          const int r = 32 * rtP + l32;
          const float gr = vG[r], rq = vRq[r];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const int f = rtP == 0 ? s2 : 2 + 2 * itP + s2;
            const int ia = 32 * itP + 16 * s2 + 4 * h, ib = ia + 8;
            const floatx4 ga = *reinterpret_cast<const floatx4*>(vG + ia), gb = *reinterpret_cast<const floatx4*>(vG + ib);
            const floatx4 ka = *reinterpret_cast<const floatx4*>(vRk + ia), kb = *reinterpret_cast<const floatx4*>(vRk + ib);
            u16x8 pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int i = e < 4 ? ia + e : ib + e - 4;
              const float gi = e < 4 ? ga[e] : gb[e - 4], rki = e < 4 ? ka[e] : kb[e - 4];
              const float x = __expf(fminf(gr - gi, 0.f)) * rq * rki * gKQ[8 * s2 + e];
              pf[e] = f32_to_f16_bits(i <= r ? x : 0.f);
            }
            *reinterpret_cast<u16x8*>(wsc + WH_P + f * 1024 + lane * 16) = pf;
          }
        }
      }
    }
    __syncthreads();
    // ---- T = (I + A)^-1, head j0 + wv on wave wv ----------------------------
    if (wv < ng) invert_unit_lower(mat(wv), lane);
    __syncthreads();
    // ---- per head, all waves: T' = T diag(beta) fragments (all six), the K^T
    //      columns of key tile wv scaled two ways, and the V columns of value tile wv
    for (int jj = 0; jj < ng; ++jj) {
      const int j = j0 + jj, hv = hk * a.G + j;
      unsigned char* wsc = ws + (static_cast<int64_t>(b * a.Hv + hv) * nwin + cl) * WH_BYTES;
      const float* vBe = vgate(j) + CH;
      const float* vKs = vgate(j) + 2 * CH;
      const float* vKd = vgate(j) + 3 * CH;
      // this head's V tile through the wave's LDS tile, then the next head's loads
      wave_lds_sync();   // the previous head's reads of the tile are done
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 16 * m + (lane >> 2);
        *reinterpret_cast<u32x4*>(sVw + r * L::kVP + 8 * (lane & 3)) = r < nval ? vr[m] : u32x4{0u, 0u, 0u, 0u};
      }
      if (j + 1 < a.G) load_v(hv + 1);
      wave_lds_sync();
      halfx8 vf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          vf[ks][e] = static_cast<_Float16>(bf16_bits_to_f32(sVw[(16 * ks + kperm(h, e)) * L::kVP + l32]));
      const float* M = mat(jj);
      halfx8 tf[FT];
#pragma unroll
      for (int f = 0; f < FT; ++f) {
        // tile (0,0) for the row tile 0 fragments, (1,0) and (1,1) for row tile 1
        const int r = 32 * ft_rt(f) + l32;
        const float* tr4 = M + (f < 2 ? 0 : (f < 4 ? 1 : 2)) * L::kTile + l32 * L::kTP + 16 * (ft_ks(f) & 1) + 4 * h;
        const int ca = 16 * ft_ks(f) + 4 * h, cb = ca + 8;
        const floatx4 ta = *reinterpret_cast<const floatx4*>(tr4);
        const floatx4 tb = *reinterpret_cast<const floatx4*>(tr4 + 8);
        const floatx4 ba = *reinterpret_cast<const floatx4*>(vBe + ca), bb = *reinterpret_cast<const floatx4*>(vBe + cb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = e < 4 ? ca + e : cb + e - 4;
          const float x = e < 4 ? ta[e] * ba[e] : tb[e - 4] * bb[e - 4];
          tf[f][e] = static_cast<_Float16>(i <= r ? x : 0.f);
        }
      }
      {
        // W^T tiles (key tile wv, row tile 0 / 1) = Ks^T T'^T with Ks = diag(gamma rk) K;
        // Kd = K^T diag(rk e^{g_63 - g}) fragments go out as they are
        floatx16 w0 = zero16(), w1 = zero16();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const floatx4 sa = *reinterpret_cast<const floatx4*>(vKs + 16 * ks + 4 * h);
          const floatx4 sb = *reinterpret_cast<const floatx4*>(vKs + 16 * ks + 8 + 4 * h);
          const floatx4 da = *reinterpret_cast<const floatx4*>(vKd + 16 * ks + 4 * h);
          const floatx4 db = *reinterpret_cast<const floatx4*>(vKd + 16 * ks + 8 + 4 * h);
          halfx8 kf, df;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kv = bf16_bits_to_f32(kt[ks][e]);
            kf[e] = static_cast<_Float16>(kv * (e < 4 ? sa[e] : sb[e - 4]));
            df[e] = static_cast<_Float16>(kv * (e < 4 ? da[e] : db[e - 4]));
          }
          *reinterpret_cast<halfx8*>(wsc + WH_KD + (wv * 4 + ks) * 1024 + lane * 16) = df;
          if (ks < 2) w0 = mfma32h(kf, tf[ks], w0);
          w1 = mfma32h(kf, tf[2 + ks], w1);
        }
        // accumulator values [8s, 8s+8) of W^T tile (wv, rt) are the -W fragment (rt, 2 wv + s)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          halfx8 n0, n1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            n0[e] = static_cast<_Float16>(-w0[8 * s2 + e]);
            n1[e] = static_cast<_Float16>(-w1[8 * s2 + e]);
          }
          *reinterpret_cast<halfx8*>(wsc + WH_W + (2 * wv + s2) * 1024 + lane * 16) = n0;
          *reinterpret_cast<halfx8*>(wsc + WH_W + (8 + 2 * wv + s2) * 1024 + lane * 16) = n1;
        }
      }
      {
        // U0 tiles (row tile 0 / 1, value tile wv) = T' V, stored in accumulator layout
        floatx16 u0 = zero16(), u1 = zero16();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (ks < 2) u0 = mfma32h(tf[ks], vf[ks], u0);
          u1 = mfma32h(tf[2 + ks], vf[ks], u1);
        }
        unsigned char* du = wsc + WH_U0 + (wv * 2) * 2048 + lane * 32;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          halfx8 x0, x1;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x0[e] = static_cast<_Float16>(u0[8 * s2 + e]);
            x1[e] = static_cast<_Float16>(u1[8 * s2 + e]);
          }
          *reinterpret_cast<halfx8*>(du + 16 * s2) = x0;
          *reinterpret_cast<halfx8*>(du + 2048 + 16 * s2) = x1;
        }
      }
    }
    if (!kOneGroup && j0 + L::kNH < a.G) __syncthreads();  // the next group rewrites the matrices
  }
}


// =========================================================================
// chain kernel: one workgroup (3 waves) per (32-column strip, value head, batch)
// =========================================================================
// LDS: NS input slots (a chunk's -W, Kd, U0 strip and scalings, copied from the
// workspace by the copy wave, NS - 1 chunks ahead, or with one slot once the
// chunk's operands have been read), two buffers each of the M and U fragments
// that the state wave publishes for the output wave, and the output wave's
// staging tile.  The output wave reads its own operands (Q^ and P fragments)
// from the workspace straight into registers.  Two slots take 98 KiB, so one
// workgroup per CU; one slot 61 KiB, so two share a CU and cover each other's
// copies when the grid holds more workgroups than there are CUs.
template <int NS>
struct ChainLds {
  static constexpr int kW = 0, kKd = 16384, kU0 = 32768, kSc = 36864;
  static constexpr int kSlot = 37888;               // 37 blocks of 1 KiB
  static constexpr int kNSlot = NS;
  static constexpr int kMf = kNSlot * kSlot;        // 2 x M fragments (fp16) [k step 8][lane 64] x 16 B
  static constexpr int kUf = kMf + 2 * 8192;        // 2 x U fragments (fp16) [k step 4][lane 64] x 16 B;
                                                    // once read, a U buffer stages the output tile
  static constexpr int kBytes = kUf + 2 * 4096;
};
constexpr int kSlotBlocks = 37;

// source of 1 KiB block m of a chunk's input slot (blocks follow the slot layout)
__device__ __forceinline__ const unsigned char* slot_src(int m, const unsigned char* wsh, int strip) {
  return m < 32 ? wsh + 1024 * m                                         // -W, Kd
       : m < 36 ? wsh + WH_U0 + strip * 4096 + 1024 * (m - 32)           // U0 columns of this strip
                : wsh + WH_SC;                                           // scalings
}

// s_waitcnt immediate that waits until at most n vector memory operations are outstanding
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

// Workgroup barrier that orders LDS only: global stores and the LDS copies in
// flight are not waited for (the copy wave waits for its own copies explicitly).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float floatx2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

// One barrier per chunk.  Between barrier c-1 and barrier c:
//  * the state wave turns M_c into U_c and M_{c+1}, publishing U_c into U buffer
//    c & 1 and M_{c+1} into M buffer (c+1) & 1;
//  * the output wave forms diag(gamma) Q^ M_c from M buffer c & 1 and completes the
//    previous chunk, O_{c-1} += P U_{c-1} from U buffer (c-1) & 1, and stores it;
//  * the copy wave starts chunk c+2's copy into the slot chunk c-1 used and waits
//    until chunk c+1's copy has landed.
// Each buffer is rewritten two chunks after it was filled, by which time its
// reader has passed the barrier in between.
// Chunks [cs, ce) of sequence b in the window numbering, the token index of its
// first token and its length.  Fixed-length batches: every sequence has chunks
// [0, ceil(T/64)) and starts at token b*T.
__device__ __forceinline__ void seq_chunks(const RecArgs& a, int b, int& cs, int& ce, int64_t& tok0, int& len) {
  if (!a.cu_seqlens) {
    cs = 0;
    ce = (a.T + CH - 1) / CH;
    tok0 = static_cast<int64_t>(b) * a.T;
    len = a.T;
    return;
  }
  cs = a.chunk_start[b];
  packed_range(a.cu_seqlens, b, a.T, tok0, len);
  ce = cs + (len + CH - 1) / CH;
}

// The window holds chunks [c0, c0 + nw) (workspace stride nwin).  A sequence's
// state comes from state_in at its first chunk and from `carry` otherwise, and
// goes to state_out after its last chunk and to `carry` otherwise.
// With one slot the copy of chunk c+1 waits for a second barrier per chunk, which
// each wave reaches once it has read chunk c's slot.
__device__ __forceinline__ void slot_read_done() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS reads have returned
  __builtin_amdgcn_s_barrier();
}

template <int NS>
__global__ __launch_bounds__(192, 2) void chunk_chain_kernel(RecArgs a, int c0, const unsigned char* ws, int nwin,
                                                             int nw, float* carry) {
  using L = ChainLds<NS>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  // Workgroups are handed to the 8 XCDs round-robin by linear index; when the
  // (slot, head) count is a multiple of 8, the 4 strips of a head get indices
  // that are equal modulo 8, so they share one XCD's L2 for the head's inputs.
  const int L0 = blockIdx.x;
  const int nheads = static_cast<int>(gridDim.x) >> 2;
  int jh, strip;
  if ((nheads & 7) == 0) {
    jh = (L0 >> 5) * 8 + (L0 & 7);
    strip = (L0 >> 3) & 3;
  } else {
    jh = L0 >> 2;
    strip = L0 & 3;
  }
  const int j = jh / a.Hv, hv = jh - j * a.Hv;   // slot, value head
  int b = j;                                      // sequence
  if (a.cu_seqlens) {
    // packed batch: slot j stands for chunk c0 + j of the window and runs the
    // sequence of that chunk when the sequence's part of the window starts there
    const int c = c0 + j;
    b = a.chunk_seq[c];
    if (b >= a.nseq || (j > 0 && a.chunk_seq[c - 1] == b)) return;
  }
  const int bhv = b * a.Hv + hv;
  const int hk = hv / a.G;
  const int bw = a.cu_seqlens ? 0 : b;               // batch index inside the workspace
  const int bh = bw * a.Hv + hv;
  int cs, ce, len;
  int64_t tok0;
  seq_chunks(a, b, cs, ce, tok0, len);
  const int lo = max(cs, c0), hi = min(ce, c0 + nw);
  if (lo >= hi) return;
  const int lofs = lo - c0;
  const float* state_in = lo == cs ? a.state_in : carry;
  float* state_out = hi == ce ? a.state_out : carry;
  // roles (one wave per SIMD): wave 1 carries the state of the strip, wave 0 produces
  // its outputs, wave 2 copies the next chunks' inputs into LDS
  const int role = wv == 2 ? 2 : (wv == 1 ? 0 : 1);
  const int col = 32 * strip + l32;  // this lane's value column
  uint16_t* go = static_cast<uint16_t*>(a.o);

  const int nchunk = hi - lo;
  const unsigned char* regK = ws + static_cast<int64_t>(a.B) * a.Hv * nwin * WH_BYTES;
  auto wsh_of = [&](int cl) { return ws + (static_cast<int64_t>(bh) * nwin + lofs + cl) * WH_BYTES; };
  auto wsk_of = [&](int cl) { return regK + (static_cast<int64_t>(bw * a.Hk + hk) * nwin + lofs + cl) * WK_BYTES; };
  auto copy_chunk = [&](int cl) {
    unsigned char* slot = smem + (cl % L::kNSlot) * L::kSlot;
    const unsigned char* wsh = wsh_of(cl);
#pragma unroll
    for (int m = 0; m < kSlotBlocks; ++m)
      __builtin_amdgcn_global_load_lds(slot_src(m, wsh, strip) + 16 * lane, slot + 1024 * m, 16, 0, 0);
  };

  // Each role runs its own chunk loop (same trip count, one barrier per chunk),
  // so that the registers one role carries across chunks are free in the others.
  if (role == 0) {
    floatx16 Ms[4];
    halfx8 Mfr[8];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      if (state_in) {
        const float* sp = state_in + static_cast<int64_t>(bhv) * DK * DK;
#pragma unroll
        for (int v = 0; v < 16; ++v) Ms[dt][v] = sp[(32 * dt + acc_row(v, h)) * DK + col];
      } else {
        Ms[dt] = zero16();
      }
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      Mfr[ks] = acc_frag_h(Ms[ks >> 1], ks & 1);
      *reinterpret_cast<halfx8*>(smem + L::kMf + ks * 1024 + lane * 16) = Mfr[ks];
    }
    __syncthreads();
    for (int cl = 0; cl < nchunk; ++cl) {
      unsigned char* slot = smem + (cl % L::kNSlot) * L::kSlot;
      const float* sSc = reinterpret_cast<const float*>(slot + L::kSc);
      unsigned char* sUf = smem + L::kUf + (cl & 1) * 4096;
      unsigned char* sMf = smem + L::kMf + ((cl + 1) & 1) * 8192;
      // ---- U = U0 - W M (U0 enters as the accumulator) ; publish U ----------
      // all reads are issued before the first use: the gate, U0, then the -W
      // fragments in the order the products take them
      const float gC = sSc[64];
      __builtin_amdgcn_sched_barrier(0);
      halfx8 x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const halfx8*>(slot + L::kU0 + (i >> 1) * 2048 + lane * 32 + (i & 1) * 16);
      halfx8 Af[16];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          Af[rt * 8 + ks] = *reinterpret_cast<const halfx8*>(slot + L::kW + (rt * 8 + ks) * 1024 + lane * 16);
      __builtin_amdgcn_sched_barrier(0);
      floatx16 U[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          U[rt][e] = static_cast<float>(x[2 * rt][e]);
          U[rt][8 + e] = static_cast<float>(x[2 * rt + 1][e]);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) U[rt] = mfma32h(Af[rt * 8 + ks], Mfr[ks], U[rt]);
      // the state's decay runs on the vector unit while the products occupy the
      // matrix unit
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) Ms[dt] *= gC;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Kd fragments for the update, read while the last products drain
#pragma unroll
      for (int i = 0; i < 16; ++i) Af[i] = *reinterpret_cast<const halfx8*>(slot + L::kKd + i * 1024 + lane * 16);
      if constexpr (NS == 1) slot_read_done();
      halfx8 Uf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        Uf[ks] = acc_frag_h(U[ks >> 1], ks & 1);
        *reinterpret_cast<halfx8*>(sUf + ks * 1024 + lane * 16) = Uf[ks];
      }
      // ---- M <- gamma_63 M + Kd U, two state tiles at a time so that the first
      //      pair's fragments are formed while the second pair runs ; publish M ----
#pragma unroll
      for (int dp = 0; dp < 4; dp += 2) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int dt = dp; dt < dp + 2; ++dt) Ms[dt] = mfma32h(Af[dt * 4 + ks], Uf[ks], Ms[dt]);
#pragma unroll
        for (int ks = 2 * dp; ks < 2 * dp + 4; ++ks) {
          Mfr[ks] = acc_frag_h(Ms[ks >> 1], ks & 1);
          *reinterpret_cast<halfx8*>(sMf + ks * 1024 + lane * 16) = Mfr[ks];
        }
      }
      lds_sync();
    }
    if (state_out) {
      float* sp = state_out + static_cast<int64_t>(bhv) * DK * DK;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) sp[(32 * dt + acc_row(v, h)) * DK + col] = Ms[dt][v];
    }
  } else if (role == 1) {
    halfx8 Bq[16], Bp[FT];  // Q^ fragments of the current chunk, P fragments of the previous one
#pragma unroll
    for (int i = 0; i < 16; ++i) Bq[i] = *reinterpret_cast<const halfx8*>(wsk_of(0) + i * 1024 + lane * 16);
#pragma unroll
    for (int f = 0; f < FT; ++f) Bp[f] = *reinterpret_cast<const halfx8*>(wsh_of(0) + WH_P + f * 1024 + lane * 16);

    // O_c += U_c^T P_c^T, then the 64 x 32 bf16 tile is staged in LDS over the U
    // fragments just read (64-byte rows, 16-byte units swizzled by the row so that the
    // 4-column writes spread over the banks) and stored as 16-byte runs of 8 columns.
    // The state wave refills that U buffer only after the next barrier.
    auto finish = [&](floatx16 (&O)[2], int cp) {
      unsigned char* sO = smem + L::kUf + (cp & 1) * 4096;
      {
        const unsigned char* sUf = sO;
        halfx8 Au[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Au[ks] = *reinterpret_cast<const halfx8*>(sUf + ks * 1024 + lane * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < FT; ++f) O[ft_rt(f)] = mfma32h(Au[ft_ks(f)], Bp[f], O[ft_rt(f)]);
      }
      if (cp + 1 < nchunk) {
        const unsigned char* wp = wsh_of(cp + 1) + WH_P;
#pragma unroll
        for (int f = 0; f < FT; ++f) Bp[f] = *reinterpret_cast<const halfx8*>(wp + f * 1024 + lane * 16);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int r = 32 * rt + l32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 w = {pack_bf16x2(O[rt][4 * j], O[rt][4 * j + 1]), pack_bf16x2(O[rt][4 * j + 2], O[rt][4 * j + 3])};
          *reinterpret_cast<uint2*>(sO + r * 64 + ((j ^ (r & 3)) * 16) + 8 * h) = w;
        }
      }
      const int ci = lo - cs + cp;   // chunk index inside the sequence
      const int nval = min(CH, len - ci * CH);
      uint16_t* obase = go + (tok0 + static_cast<int64_t>(ci) * CH) * a.so + hv * DK + 32 * strip;
      u16x8 x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int vi = lane + 64 * m, r = vi >> 2, u = vi & 3;
        x[m] = *reinterpret_cast<const u16x8*>(sO + r * 64 + ((u ^ (r & 3)) * 16));
      }
      if (nval == CH) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int vi = lane + 64 * m, r = vi >> 2, u = vi & 3;
          *reinterpret_cast<u16x8*>(obase + static_cast<int64_t>(r) * a.so + 8 * u) = x[m];
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int vi = lane + 64 * m, r = vi >> 2, u = vi & 3;
          if (r < nval) *reinterpret_cast<u16x8*>(obase + static_cast<int64_t>(r) * a.so + 8 * u) = x[m];
        }
      }
    };

    floatx16 Op[2];  // the previous chunk's outputs, waiting for P U
    __syncthreads();
    for (int cl = 0; cl < nchunk; ++cl) {
      unsigned char* slot = smem + (cl % L::kNSlot) * L::kSlot;
      const float* sSc = reinterpret_cast<const float*>(slot + L::kSc);
      const unsigned char* sMf = smem + L::kMf + (cl & 1) * 8192;
      const float g0 = sSc[l32], g1 = sSc[32 + l32];
      if constexpr (NS == 1) slot_read_done();
      // ---- O^T = M^T Q^^T diag(gamma) + U^T P^T: the M and U fragments serve as A
      //      operands and Q^, P as B operands, so each lane holds one token and
      //      runs of four value columns ------------------------------------------
      floatx16 O[2] = {zero16(), zero16()};
      {
        halfx8 Am[8];   // M fragments, all read before the first product
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) Am[ks] = *reinterpret_cast<const halfx8*>(sMf + ks * 1024 + lane * 16);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
          for (int rt = 0; rt < 2; ++rt) O[rt] = mfma32h(Am[ks], Bq[rt * 8 + ks], O[rt]);
      }
      // the next chunk's Q^ fragments: a chunk ahead of their use (the last chunk
      // reloads its own)
      {
        const unsigned char* wq = wsk_of(min(cl + 1, nchunk - 1));
#pragma unroll
        for (int i = 0; i < 16; ++i) Bq[i] = *reinterpret_cast<const halfx8*>(wq + i * 1024 + lane * 16);
      }
      if (cl > 0) finish(Op, cl - 1);
      Op[0] = O[0] * g0;
      Op[1] = O[1] * g1;
      // the first chunk issues no stores; draining its loads here keeps the counts
      // the compiler waits for at the loop head those of the later chunks, whose
      // stores need not complete before the next chunk's products
      if (cl == 0) wait_vm_all();
      lds_sync();
    }
    if (nchunk > 0) finish(Op, nchunk - 1);
  } else if constexpr (NS == 1) {
    // one slot: chunk cl+1 is copied once every wave has read chunk cl's
    copy_chunk(0);
    wait_vm_all();
    __syncthreads();
    for (int cl = 0; cl < nchunk; ++cl) {
      __builtin_amdgcn_s_barrier();
      if (cl + 1 < nchunk) {
        copy_chunk(cl + 1);
        wait_vm_all();
      }
      __builtin_amdgcn_s_barrier();
    }
  } else {
    // copies run kAhead = slots - 1 chunks ahead
    constexpr int kAhead = L::kNSlot - 1;
    static_assert(kAhead == 1 || kAhead == 2, "one or two chunks ahead");
    copy_chunk(0);
    if (kAhead == 2 && nchunk > 1) {
      copy_chunk(1);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kSlotBlocks));
    } else {
      wait_vm_all();
    }
    __syncthreads();
    for (int cl = 0; cl < nchunk; ++cl) {
      // slot (cl + kAhead) % slots was last read during chunk cl-1
      if (cl + kAhead < nchunk) {
        copy_chunk(cl + kAhead);
        // chunk cl+1 has landed
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kAhead - 1) * kSlotBlocks));
      } else {
        wait_vm_all();
      }
      // barrier without a fence: this wave writes LDS only through its copies, and
      // the vector memory count above already covers the ones the others read next
      __builtin_amdgcn_s_barrier();
    }
  }
}

// Packed batches: an empty sequence hands its state on unchanged (the zero state
// without state_in).  One workgroup per (sequence, value head); the others leave.
__global__ __launch_bounds__(256) void empty_state_kernel(RecArgs a) {
  const int bhv = blockIdx.x, b = bhv / a.Hv;
  int64_t st;
  int len;
  packed_range(a.cu_seqlens, b, a.T, st, len);
  if (len) return;
  const int64_t base = static_cast<int64_t>(bhv) * DK * DK;
  const floatx4* src = reinterpret_cast<const floatx4*>(a.state_in + base);
  floatx4* dst = reinterpret_cast<floatx4*>(a.state_out + base);
  for (int i = threadIdx.x; i < DK * DK / 4; i += 256)
    dst[i] = a.state_in ? src[i] : floatx4{0.f, 0.f, 0.f, 0.f};
}

// Chunk maps of a packed batch, for the prep and chain kernels: one workgroup
// scans the per-sequence chunk counts ceil(len/64) into chunk_start, then finds
// each chunk's sequence by binary search (the last s with chunk_start[s] <= c, so
// that empty sequences, which share their successor's start, are passed over).
__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* cu, int nseq, int T, int ncap,
                                                         int32_t* chunk_start, int32_t* chunk_seq) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < nseq; base += 1024) {
    const int s = base + tid;
    int n = 0;
    if (s < nseq) {
      int64_t st;
      int len;
      packed_range(cu, s, T, st, len);
      n = (len + CH - 1) / CH;
    }
    int x = n;  // inclusive scan inside the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      before += i < wv ? wsum[i] : 0;
      total += wsum[i];
    }
    if (s < nseq) chunk_start[s] = carry + before + x - n;
    carry += total;
    __syncthreads();  // wsum is rewritten by the next block of sequences
  }
  if (tid == 0) chunk_start[nseq] = carry;
  __syncthreads();  // chunk_start is complete and visible to the workgroup
  for (int c = tid; c < ncap; c += 1024) {
    int sq = nseq;
    if (c < carry) {
      int lo = 0, hi = nseq - 1;  // chunk_start[0] = 0 <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_start[mid] <= c) lo = mid;
        else hi = mid - 1;
      }
      sq = lo;
    }
    chunk_seq[c] = sq;
  }
}

}  // namespace

size_t chunk_ws_bytes_per_chunk(const RecArgs& a) {
  return static_cast<size_t>(a.B) * (static_cast<size_t>(a.Hv) * WH_BYTES + static_cast<size_t>(a.Hk) * WK_BYTES);
}

size_t chunk_map_bytes(const RecArgs& a) {
  if (!a.cu_seqlens) return 0;
  const size_t b = (static_cast<size_t>(a.nseq) + 1 + chunk_count(a)) * 4;
  return (b + 255) & ~size_t(255);
}

size_t chunk_ws_carry_bytes(const RecArgs& a) {
  return static_cast<size_t>(a.cu_seqlens ? a.nseq : a.B) * a.Hv * DK * DK * 4;
}

// Chunks the windows run over: ceil(T/64) per sequence, or for packed sequences at
// most ceil(T/64) + nseq (each sequence ends in at most one partial chunk).
int chunk_count(const RecArgs& a) { return (a.T + CH - 1) / CH + (a.cu_seqlens ? a.nseq : 0); }

// Prep workgroups resident at once on the 256 CUs: their LDS lets two share a CU
// up to 19 value heads per key head, one beyond.
int prep_slots(int G) { return 256 * max(1, min(2, (160 * 1024) / PrepLds::bytes(G))); }

// Chunks per window.  The chain kernel reads a window's operands back from the
// memory-side last-level cache (256 MB) when they are still there: with the whole
// T=4096, 16/48-head workspace (190 MB) in one window, the prep's input reads and
// the outputs push part of it out, and the chain runs 20 % slower than with two
// windows of 95 MB.  The prep kernel costs about one workgroup's latency per round
// of resident workgroups, so a window is a whole number of rounds (at least one):
// as many as keep it within about 96 MiB of workspace.  When one round alone
// exceeds that, the cache cannot hold a window anyway and each window only adds
// launches (batch 4, T=32768, 16/128 heads: 13.7 ms with windows of 8 chunks,
// 10.7 ms with 64), so windows then take as many rounds as fit in 2 GiB.
// Windows are then balanced, which never adds a round.
int chunk_window_chunks(const RecArgs& a) {
  const int nchunks = chunk_count(a);
  const size_t per = chunk_ws_bytes_per_chunk(a);
  const int round = max(1, prep_slots(a.G) / (a.Hk * a.B));   // chunks one round of prep covers
  const size_t cache = size_t(96) << 20;
  const size_t budget = static_cast<size_t>(round) * per <= cache ? cache : size_t(2) << 30;
  const int fit = static_cast<int>(min(budget / per, static_cast<size_t>(1) << 30));
  int w = max(1, fit / round) * round;
  w = max(1, min(w, fit));
  if (w >= nchunks) return nchunks;
  const int nwins = (nchunks + w - 1) / w;
  return (nchunks + nwins - 1) / nwins;
}

hipError_t launch_chunk_prefill(const RecArgs& a, void* ws, size_t ws_bytes, hipStream_t s) {
  static PerDeviceOnce attrs;
  hipError_t ea = attrs.run([] {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_prep_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_prep_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel<2>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds<2>::kBytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel<1>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds<1>::kBytes);
  });
  if (ea != hipSuccess) return ea;
  const int nchunks = chunk_count(a);
  if (nchunks == 0) return hipSuccess;
  RecArgs r = a;
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  if (a.cu_seqlens) {
    // packed batch: chunk maps first, at the workspace start
    const size_t mb = chunk_map_bytes(a);
    if (ws_bytes < mb) return hipErrorInvalidValue;
    int32_t* cstart = reinterpret_cast<int32_t*>(wsb);
    int32_t* cseq = cstart + a.nseq + 1;
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, s, a.cu_seqlens, a.nseq, a.T, nchunks, cstart, cseq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.state_out) {
      hipLaunchKernelGGL(empty_state_kernel, dim3(a.nseq * a.Hv), dim3(256), 0, s, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    r.chunk_start = cstart;
    r.chunk_seq = cseq;
    wsb += mb;
    ws_bytes -= mb;
  }
  const size_t per_chunk = chunk_ws_bytes_per_chunk(a);
  // One window when the whole sequence fits; otherwise the state is carried
  // between windows through state_out (or a carry area at the workspace end).
  // the preferred window, or what the workspace holds when it is smaller
  int nwin = static_cast<int>(min(ws_bytes / per_chunk, static_cast<size_t>(chunk_window_chunks(a))));
  bool need_carry = false;
  if (nwin < nchunks) {
    need_carry = a.state_out == nullptr;
    const size_t carry_b = need_carry ? chunk_ws_carry_bytes(a) : 0;
    const size_t avail = ws_bytes > carry_b ? ws_bytes - carry_b : 0;
    nwin = min(nwin, static_cast<int>(avail / per_chunk));
  }
  if (nwin < 1) return hipErrorInvalidValue;
  if (nwin > nchunks) nwin = nchunks;
  float* carry = need_carry ? reinterpret_cast<float*>(wsb + static_cast<size_t>(nwin) * per_chunk) : a.state_out;
  for (int c0 = 0; c0 < nchunks; c0 += nwin) {
    const int nw = min(nwin, nchunks - c0);
    if (a.G <= PrepLds::kNH)
      hipLaunchKernelGGL(chunk_prep_kernel<true>, dim3(nw, a.Hk, a.B), dim3(256), PrepLds::bytes(a.G), s, r, c0, wsb,
                         nwin);
    else
      hipLaunchKernelGGL(chunk_prep_kernel<false>, dim3(nw, a.Hk, a.B), dim3(256), PrepLds::bytes(a.G), s, r, c0, wsb,
                         nwin);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // chain workgroups per (sequence, value head, strip); for a packed batch per
    // (chunk slot of the window, value head, strip), since at most nw sequences
    // have chunks in the window
    const int slots = a.cu_seqlens ? nw : a.B;
    // With more workgroups than CUs the one-slot kernel lets two share a CU (batch
    // 4, 128 value heads: 9.9 ms of prefill against 10.7 ms).  A packed batch
    // runs one slot per sequence with chunks in the window, which the host does
    // not know; the few it has per window run better with two slots.
    const dim3 grid(slots * a.Hv * (DK / 32));
    if (!a.cu_seqlens && a.B * a.Hv * (DK / 32) > 256)
      hipLaunchKernelGGL(chunk_chain_kernel<1>, grid, dim3(192), ChainLds<1>::kBytes, s, r, c0,
                         static_cast<const unsigned char*>(wsb), nwin, nw, carry);
    else
      hipLaunchKernelGGL(chunk_chain_kernel<2>, grid, dim3(192), ChainLds<2>::kBytes, s, r, c0,
                         static_cast<const unsigned char*>(wsb), nwin, nw, carry);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
