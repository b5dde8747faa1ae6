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
//   W  = T' diag(gamma rk) K,   U0 = T' V,   K^ = diag(rk) K,   Q^ = diag(rq) Q,
//   f_r = e^{g_63 - g_r},       so that per chunk
//   U  = U0 - W M,   M <- gamma_63 M + K^T diag(f) U,   O = diag(gamma) Q^ M + P U.
//
// K^ and Q^ depend on the key head only and are stored once per key head; W,
// U0, P and f once per value head.
//
// Two kernels per window of chunks:
//  * prep (one workgroup per chunk and key head, fully parallel over chunks):
//    row norms, the Gram products K K^T and K Q^T (bf16 MFMA, kept in
//    registers), and per value head the gate prefix sums, A, the inverse
//    (16x16 forward substitution, a 16-block merge on fp32 MFMA, and the
//    32x32 merge on MFMA with split-fp16 operands), T', and the products -W
//    and U0 (fp16 MFMA), and once per key head K^ and Q^.  The value heads of a key head are inverted up to
//    three at a time, each on its own wave and in place.  All of it is
//    written to the workspace as MFMA-ready fp16 fragments; U0 in the
//    accumulator layout of the chain's U.
//  * chain (one workgroup per sequence, value head and 32-column strip of M,
//    looping over the window's chunks; columns of M evolve independently).
//    Two waves each carry 16 columns of the fp32 strip in registers and run,
//    per chunk, U = U0 - W M interleaved with O^T = M^T Q^T (32 MFMAs), the
//    update M <- gamma_63 M + K^T (diag(f) U) (16) and O^T += U^T P^T (6), then
//    store their outputs; a third copies the next chunk's operands from the
//    workspace into LDS with direct global-to-LDS loads while they work.
//    When the heads alone fill the GPU, one workgroup takes a whole value
//    head (eight such waves and one copy wave); with the gated norm, that
//    workgroup also normalises and gates its output rows.
//
// Precision.  MFMA accumulation is fp32 throughout and the state stays fp32.
// The Gram products take the bf16 inputs as they are; every other product
// runs on fp16 operands, each rounded once (in prep: -W, K^, U0, P, Q^; in
// the chain: M, U and diag(f) U).  fp16 keeps 11 significant bits, which holds the state
// within a few 1e-4 of the exact result and the outputs well inside their
// bound.  Its range does not bound the inputs: the value-side operands (V,
// U0, U, M) enter fp16 scaled by powers of two chosen per chunk and 16-column
// value tile (see kRangeTop), and the key-side ones (-W, K^, P, Q^) are
// bounded by the L2-normalised keys and queries and the gates (every decay
// factor is at most 1).

// MFMA layouts (wave64).  The chunk operands that leave the prep kernel are
// fragments of v_mfma_f32_16x16x32_f16: A row = B column = lane & 15, and the
// lane group g = lane >> 4 carries 8 of a k step's 32 contraction indices; the
// accumulator holds column lane & 15, rows 4g + v (v < 4).  The contraction
// index is permuted the same way on A and B: slot e of group g is
// kperm(g, e) = 4g + e for e < 4 and 16 + 4g + (e - 4) otherwise.  With that
// permutation the values of two accumulator tiles stacked in rows (rows 0-15
// and 16-31 of a 32-row block) are, lane by lane, the B operand of the k step
// over that block, so M and U feed the next product straight from registers,
// and a product computed in transposed form (C^T = B^T A^T) leaves its result
// as an A fragment.  The key Gram K K^T that feeds the inverse is taken on
// 32x32x16 tiles (A row = B column = lane & 31), whose layout stays inside the
// prep kernel.
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
// Workspace block per (batch, value head, chunk): 16x16x32 fp16 fragments (1 KiB each:
// 64 lanes x 8 halves) and fp32 scalings.
constexpr int WH_W = 0;        // -W = -T' diag(gamma rk) K, A operand: fragment rt*4+ks (rows 16rt.., keys 32ks..)
constexpr int WH_KD = 16384;   // K^T = (diag(rk) K)^T, A operand: fragment dt*2+ks (keys 16dt.., rows 32ks..);
                               // written in the block of the key head's first value head only
constexpr int WH_U0 = 32768;   // U0 = T' V as accumulators of U: [value tile 8][lane 64][row tile 4][4 halves]
constexpr int WH_P = 49152;    // P^T, B operand: 6 fragments (token tile ct, rows 32ks..), see pfrag()
constexpr int WH_SC = 55296;   // gamma_r (64 floats), gamma_63; int32: V scale exponents of the 8 value
                               // tiles at [65, 73), gamma_63's exponent at 73, the next chunk's V scale
                               // exponents at [80, 88); [96, 112): the chain's scale hand-over between windows;
                               // f_r = e^{g_63 - g_r} (64 floats) at [128, 192)
constexpr int WH_BYTES = 56320;
// workspace block per (batch, key head, chunk): Q^T = (diag(rq) Q)^T, B operand: fragment ks*4+ct
// (keys 32ks.., tokens 16ct..)
constexpr int WK_BYTES = 16384;

// contraction index of slot e for lane group g, inside a 32-wide k step (16x16x32)
__device__ __forceinline__ int kperm(int g, int e) { return (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4); }
// the same for a 16-wide k step of 32x32x16 and lane half h (the inverse's 32-block merge)
__device__ __forceinline__ int kperm32(int h, int e) { return (e < 4) ? 4 * h + e : 8 + 4 * h + (e - 4); }
// Range of the fp16 operands on the value side.  V, U0, U and the state M enter the
// fp16 products scaled by powers of two: each 16-column V tile of a chunk by 2^r, r
// chosen so that its largest magnitude lands in [2^(kRangeTop-3), 2^(kRangeTop+1)) and
// stored with the chunk's scalings; the chain's M and U by 2^s, s <= r, chosen from
// the state's measured range (see the chain kernel).  Exponents are multiples of 4, so
// that values of about unit size keep r = s = 0 and no rescaling at all.  Scaling by a
// power of two is exact, so the fp32 results are those of unscaled operands; only
// values smaller than a tile's largest by more than fp16's normal range lose bits.
constexpr int kRangeTop = 2;
constexpr int kCheck = 6;   // chunks between two measurements of the chain state's range
constexpr int kExpLo = -120, kExpHi = 124;   // exponents whose powers of two are normal fp32
// the multiple of 4 at or below x
__device__ __forceinline__ int floor4(int x) { return (x >> 2) * 4; }

// Largest x over the wave, in every lane, for x >= 0 as fp32 bits (they compare as
// integers): the maximum over each row of 16 lanes by DPP, then over the four rows.
__device__ __forceinline__ uint32_t wave_max_bits(uint32_t x) {
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0xB1, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x4E, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x141, 0xF, 0xF, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x140, 0xF, 0xF, false)));
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return max(max(r0, r1), max(r2, r3));
}

// max(|a|, |b|, |c|) in one instruction (fmaxf would add a NaN-quieting step per operand)
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// 2^st in all eight halves, -14 <= st <= 15 (normal fp16 powers of two)
__device__ __forceinline__ halfx8 scale_h(int st) {
  const _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>((st + 15) << 10));
  return halfx8{h, h, h, h, h, h, h, h};
}

// largest |x| of a lane's 32 state values, as four chains of three-way maxima
__device__ __forceinline__ float lane_max_abs32(const floatx4 (&m)[8]) {
  float m4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const floatx4 x = m[2 * i], y = m[2 * i + 1];
    m4[i] = max3_abs(x[0], x[1], x[2]);
    m4[i] = max3_abs(m4[i], x[3], y[0]);
    m4[i] = max3_abs(m4[i], y[1], y[2]);
    m4[i] = max3_abs(m4[i], y[3], y[3]);
  }
  return max3_abs(max3_abs(m4[0], m4[1], m4[2]), m4[3], m4[3]);
}

// exponent e with 2^e <= m < 2^(e+1) for the fp32 bits of m > 0 (subnormals count as 2^-127)
__device__ __forceinline__ int exp_of_bits(uint32_t m) { return static_cast<int>((m >> 23) & 0xFFu) - 127; }

// the scale exponent (a multiple of 4) that brings a largest magnitude with fp32 bits m to
// [2^(kRangeTop-3), 2^(kRangeTop+1))
__device__ __forceinline__ int range_exp(uint32_t m) {
  return m == 0u ? 0 : min(kExpHi, max(kExpLo, floor4(kRangeTop - exp_of_bits(m))));
}

// P^T fragments: (token tile ct, chunk-row step ks) pairs with ks == 0 or ct >= 2 (the others are zero)
__device__ __forceinline__ int pfrag(int ct, int ks) { return ks == 0 ? ct : 2 + ct; }
// (row tile rt, k step ki) pairs of the lower-triangular T' that are not all zero: ki == 0 or rt >= 2
constexpr int kTriRt[6] = {0, 1, 2, 3, 2, 3};
constexpr int kTriKi[6] = {0, 0, 0, 0, 1, 1};

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

__device__ __forceinline__ floatx4 mfma16h(const halfx8& a, const halfx8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx4 mfma16b(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// two stacked 16x16 accumulator tiles (rows 0-15, 16-31) as the fp16 B operand of a 32-wide k step
__device__ __forceinline__ halfx8 stack_h(const floatx4& lo, const floatx4& hi) {
  halfx8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = static_cast<_Float16>(lo[e]);
    r[4 + e] = static_cast<_Float16>(hi[e]);
  }
  return r;
}

// a bf16 row segment of 32 contraction indices as a 16x16x32 operand slot set: lane group g
// takes [4g, 4g+4) and [16+4g, 20+4g) of the segment
__device__ __forceinline__ bf16x8 lds_frag16(const uint16_t* row_k0, int g) {
  const u16x4 lo = *reinterpret_cast<const u16x4*>(row_k0 + 4 * g);
  const u16x4 hi = *reinterpret_cast<const u16x4*>(row_k0 + 16 + 4 * g);
  const u16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
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
  static constexpr int bytes(int G) { return kVec + (2 + 3 * G) * CH * 4; }
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
        const float bv = T0[(16 * ks + kperm32(h, e)) * L::kTP + l32];
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
  // gate vectors of value head j of this key head: g, beta, gamma rk
  auto vgate = [&](int j) { return vRk + (2 + 3 * j) * CH; };
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
  // All eight 16-byte loads go out before any is used (rows past the sequence end
  // read the last valid row and are replaced by zeros), so the rows cost one memory
  // round trip; each row's sums of squares over its 16 lanes by DPP.
  u16x8 kq[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int vi = tid + 256 * j;
    const int r = vi >> 4, c8 = (vi & 15) * 8, rr = r < nval ? r : nval - 1;
    kq[2 * j] = *reinterpret_cast<const u16x8*>(gk + (tokbase + rr) * a.sk + hk * DK + c8);
    kq[2 * j + 1] = *reinterpret_cast<const u16x8*>(gq + (tokbase + rr) * a.sq + hk * DK + c8);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int vi = tid + 256 * j;
    const int r = vi >> 4, c8 = (vi & 15) * 8;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    const u16x8 kv = r < nval ? kq[2 * j] : z8, qv = r < nval ? kq[2 * j + 1] : z8;
    *reinterpret_cast<u16x8*>(sK + r * KP + c8) = kv;
    *reinterpret_cast<u16x8*>(sQ + r * KP + c8) = qv;
    float ssk = 0.f, ssq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float kf = bf16_bits_to_f32(kv[e]), qf = bf16_bits_to_f32(qv[e]);
      ssk = fmaf(kf, kf, ssk);
      ssq = fmaf(qf, qf, ssq);
    }
    ssk = row16_sum(ssk);
    ssq = row16_sum(ssq);
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
    float* sc = reinterpret_cast<float*>(ws + (static_cast<int64_t>(b * a.Hv + hk * a.G + j) * nwin + cl) * WH_BYTES + WH_SC);
    sc[lane] = eg;
    sc[128 + lane] = __expf(gl - g);
    if (lane == 0) {
      const float g63 = __expf(gl);
      sc[64] = g63;
      reinterpret_cast<int32_t*>(sc)[73] = exp_of_bits(__float_as_uint(g63));   // gamma_63 < 2^(this + 1)
    }
  }

  // ---- Q^T = (diag(rq) Q)^T as the output product's B fragments (fp16) ------
  //      fragment ks*4+ct: token 16ct + (lane & 15), keys 32ks + kperm(g, e)
  {
    unsigned char* wsk = ws + static_cast<int64_t>(a.B) * a.Hv * nwin * WH_BYTES +
                         (static_cast<int64_t>(b * a.Hk + hk) * nwin + cl) * WK_BYTES;
    for (int slot = tid; slot < 16 * 64; slot += 256) {
      const int f = slot >> 6, ln = slot & 63;
      const int r = 16 * (f & 3) + (ln & 15), gg = ln >> 4;
      const uint16_t* src = sQ + r * KP + 32 * (f >> 2);
      const u16x4 lo = *reinterpret_cast<const u16x4*>(src + 4 * gg);
      const u16x4 hi = *reinterpret_cast<const u16x4*>(src + 16 + 4 * gg);
      const float rq = vRq[r];
      u16x8 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = f32_to_f16_bits(bf16_bits_to_f32(lo[e]) * rq);
        x[4 + e] = f32_to_f16_bits(bf16_bits_to_f32(hi[e]) * rq);
      }
      *reinterpret_cast<u16x8*>(wsk + f * 1024 + ln * 16) = x;
    }
  }
  // ---- this wave's K^T values in A-fragment order: key tiles dt = 2wv, 2wv+1 (keys
  //      16dt + (lane & 15)) at chunk rows 32ks + kperm(g, e); scaled per value head below
  const int g4 = lane >> 4, l16 = lane & 15;
  u16x8 kt[4];   // [dt - 2wv][ks]
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int d = 16 * (2 * wv + t) + l16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) kt[2 * t + ks][e] = sK[(32 * ks + kperm(g4, e)) * KP + d];
  }
  // K^T = (diag(rk) K)^T fragments of the same key tiles: they do not depend on the value
  // head, so they go once into the block of the key head's first value head
  {
    unsigned char* wkd = ws + (static_cast<int64_t>(b * a.Hv + hk * a.G) * nwin + cl) * WH_BYTES + WH_KD;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        halfx8 df;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          df[e] = static_cast<_Float16>(bf16_bits_to_f32(kt[2 * t + ks][e]) * vRk[32 * ks + kperm(g4, e)]);
        *reinterpret_cast<halfx8*>(wkd + ((2 * wv + t) * 2 + ks) * 1024 + lane * 16) = df;
      }
  }
  // ---- Gram tiles, kept in registers ---------------------------------------
  //  K K^T (waves 0-2, 32x32 tile wv of the lower triangle): element (row r, column i) = k_r . k_i
  //  K Q^T (all waves, 16x16 tiles): element (row i, column r) = k_i . q_r, for the P^T fragments
  //  this wave writes: wave 0 (ct 0, 1 at ks 0), wave 1 (ct 2, 3 at ks 0), wave 2 (ct 2 at ks 1),
  //  wave 3 (ct 3 at ks 1); a fragment (ct, ks) needs the tiles of rows 32ks.. and 32ks+16..
  const int rtK = wv == 0 ? 0 : 1, ctK = wv == 2 ? 1 : 0;
  floatx16 gKK = zero16();
  if (wv < 3) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      gKK = mfma32(lds_frag32(sK + (32 * rtK + l32) * KP + 16 * ks, h),
                   lds_frag32(sK + (32 * ctK + l32) * KP + 16 * ks, h), gKK);
  }
  const int npf = wv < 2 ? 2 : 1;                         // P^T fragments of this wave
  const int pct0 = wv < 2 ? 2 * wv : wv, pks = wv < 2 ? 0 : 1;
  floatx4 gKQ[4];                                         // [fragment][row half]
#pragma unroll
  for (int t = 0; t < 4; ++t) gKQ[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if ((t >> 1) < npf) {
        const int ct = pct0 + (t >> 1), it = 2 * pks + (t & 1);
        gKQ[t] = mfma16b(lds_frag16(sK + (16 * it + l16) * KP + 32 * kk, g4),
                         lds_frag16(sQ + (16 * ct + l16) * KP + 32 * kk, g4), gKQ[t]);
      }
    }
  }
  __syncthreads();  // the K and Q rows are dead from here on: their bytes hold the matrices

  // ---- P^T fragments of value head j: P_ri = e^{g_r - g_i} rq_r rk_i (q_r . k_i), i <= r
  auto write_p = [&](int j) {
    const float* vG = vgate(j);
    unsigned char* wsc = ws + (static_cast<int64_t>(b * a.Hv + hk * a.G + j) * nwin + cl) * WH_BYTES;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u < npf) {
        const int ct = pct0 + u, r = 16 * ct + l16;
        const float gr = vG[r], rq = vRq[r];
        halfx8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 32 * pks + kperm(g4, e);
          const float x = __expf(fminf(gr - vG[i], 0.f)) * rq * vRk[i] * gKQ[2 * u + (e >> 2)][e & 3];
          pf[e] = static_cast<_Float16>(i <= r ? x : 0.f);
        }
        *reinterpret_cast<halfx8*>(wsc + WH_P + pfrag(ct, pks) * 1024 + lane * 16) = pf;
      }
    }
  };
  // With more value heads than one group, every head's P goes out first, so that the
  // K Q^T tiles do not stay live across the groups.
  if (!kOneGroup)
    for (int j = 0; j < a.G; ++j) write_p(j);

  // Value heads in groups of up to kNH: A (and with one group P) from the Gram tiles,
  // then each head's inverse on its own wave, then the products of each head.
  for (int j0 = 0; j0 < (kOneGroup ? 1 : a.G); j0 += L::kNH) {
    const int ng = kOneGroup ? a.G : min(L::kNH, a.G - j0);
    for (int jj = 0; jj < ng; ++jj) {
      const int j = j0 + jj;
      const float* vG = vgate(j);
      const float* vBe = vG + CH;
      // ---- A (fp32, strictly lower; tile wv) -----------------------------------
      if (wv < 3) {
        float* At = mat(jj) + wv * L::kTile;
        const int i = 32 * ctK + l32;
        const float gi = vG[i], rki = vRk[i];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r0 = 32 * rtK + 8 * q + 4 * h;
          const floatx4 g4v = *reinterpret_cast<const floatx4*>(vG + r0);
          const floatx4 b4 = *reinterpret_cast<const floatx4*>(vBe + r0);
          const floatx4 k4 = *reinterpret_cast<const floatx4*>(vRk + r0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = r0 + e;
            const float x = b4[e] * k4[e] * rki * __expf(fminf(g4v[e] - gi, 0.f)) * gKK[4 * q + e];
            At[(8 * q + 4 * h + e) * L::kTP + l32] = i < r ? x : 0.f;
          }
        }
      }
      if (kOneGroup) write_p(j);
    }
    __syncthreads();
    // ---- T = (I + A)^-1, head j0 + wv on wave wv ----------------------------
    if (wv < ng) invert_unit_lower(mat(wv), lane);
    __syncthreads();
    // ---- per head, all waves: the six nonzero T' = T diag(beta) fragments (A operand of
    //      T' V; the same registers are the B operand of Ks^T T'^T), then
    //      -W (key tiles 2wv, 2wv+1) and U0 (value tiles 2wv, 2wv+1)
    for (int jj = 0; jj < ng; ++jj) {
      const int j = j0 + jj, hv = hk * a.G + j;
      unsigned char* wsc = ws + (static_cast<int64_t>(b * a.Hv + hv) * nwin + cl) * WH_BYTES;
      const float* vBe = vgate(j) + CH;
      const float* vKs = vgate(j) + 2 * CH;
      // this head's V tile (value columns 32wv..) through the wave's LDS tile, then the next head's loads
      wave_lds_sync();   // the previous head's reads of the tile are done
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 16 * m + (lane >> 2);
        *reinterpret_cast<u32x4*>(sVw + r * L::kVP + 8 * (lane & 3)) = r < nval ? vr[m] : u32x4{0u, 0u, 0u, 0u};
      }
      if (j + 1 < a.G) load_v(hv + 1);
      wave_lds_sync();
      // value tile 2wv + hh goes into fp16 scaled by 2^r, r from its largest |v| in the chunk
      // (bf16 bits without the sign, shifted, are the fp32 bits of |v|)
      halfx8 vf[4];   // [ki][value tile half]: value column 16 hh + (lane & 15), rows 32ki + kperm
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t mb = 0u;
#pragma unroll
        for (int ki = 0; ki < 2; ++ki)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            mb = max(mb, static_cast<uint32_t>(sVw[(32 * ki + kperm(g4, e)) * L::kVP + 16 * hh + l16] & 0x7FFFu));
        const int rexp = range_exp(wave_max_bits(mb << 16));
#pragma unroll
        for (int ki = 0; ki < 2; ++ki)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            vf[2 * ki + hh][e] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(
                bf16_bits_to_f32(sVw[(32 * ki + kperm(g4, e)) * L::kVP + 16 * hh + l16]), rexp));
        if (lane == 0) {
          // this chunk's exponent, and the same as the previous chunk's "next" one, so that the chain
          // can choose a chunk's scale before the chunk's operands are in LDS
          reinterpret_cast<int32_t*>(wsc + WH_SC)[65 + 2 * wv + hh] = rexp;
          if (cl > 0) reinterpret_cast<int32_t*>(wsc - WH_BYTES + WH_SC)[80 + 2 * wv + hh] = rexp;
        }
      }
      const float* M = mat(jj);
      halfx8 tf[6];
#pragma unroll
      for (int f = 0; f < 6; ++f) {
        const int rt = kTriRt[f], ki = kTriKi[f];
        const int r = 16 * rt + l16;
        const int tile = rt < 2 ? 0 : (ki == 0 ? 1 : 2);
        const float* tr4 = M + tile * L::kTile + (r & 31) * L::kTP + 4 * g4;
        const floatx4 ta = *reinterpret_cast<const floatx4*>(tr4);
        const floatx4 tb = *reinterpret_cast<const floatx4*>(tr4 + 16);
        const floatx4 ba = *reinterpret_cast<const floatx4*>(vBe + 32 * ki + 4 * g4);
        const floatx4 bb = *reinterpret_cast<const floatx4*>(vBe + 32 * ki + 16 + 4 * g4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tf[f][e] = static_cast<_Float16>(ta[e] * ba[e]);
          tf[f][4 + e] = static_cast<_Float16>(tb[e] * bb[e]);
        }
      }
      {
        // W^T tiles (key tile 2wv + t, row tile rt) = Ks^T T'^T with Ks = diag(gamma rk) K; the two
        // key tiles of a row tile stack into the -W fragment (rt, wv).
        floatx4 w[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) w[t][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int ki = 0; ki < 2; ++ki) {
            const floatx4 sa = *reinterpret_cast<const floatx4*>(vKs + 32 * ki + 4 * g4);
            const floatx4 sb = *reinterpret_cast<const floatx4*>(vKs + 32 * ki + 16 + 4 * g4);
            halfx8 kf;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              kf[e] = static_cast<_Float16>(bf16_bits_to_f32(kt[2 * t + ki][e]) * (e < 4 ? sa[e] : sb[e - 4]));
#pragma unroll
            for (int f = 0; f < 6; ++f)
              if (kTriKi[f] == ki) w[t][kTriRt[f]] = mfma16h(kf, tf[f], w[t][kTriRt[f]]);
          }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          halfx8 n;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            n[e] = static_cast<_Float16>(-w[0][rt][e]);
            n[4 + e] = static_cast<_Float16>(-w[1][rt][e]);
          }
          *reinterpret_cast<halfx8*>(wsc + WH_W + (rt * 4 + wv) * 1024 + lane * 16) = n;
        }
      }
      {
        // U0 tiles (row tile rt, value tile 2wv + hh) = T' V, stored as U's accumulators
        floatx4 u[2][4];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) u[hh][rt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < 6; ++f)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            u[hh][kTriRt[f]] = mfma16h(tf[f], vf[2 * kTriKi[f] + hh], u[hh][kTriRt[f]]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          unsigned char* du = wsc + WH_U0 + (2 * wv + hh) * 2048 + lane * 32;
          *reinterpret_cast<halfx8*>(du) = stack_h(u[hh][0], u[hh][1]);
          *reinterpret_cast<halfx8*>(du + 16) = stack_h(u[hh][2], u[hh][3]);
        }
      }
    }
    if (!kOneGroup && j0 + L::kNH < a.G) __syncthreads();  // the next group rewrites the matrices
  }
}


// =========================================================================
// chain kernel: one workgroup per (value head, batch) and column range of M
// =========================================================================
// A workgroup covers SPW 32-column strips of a value head's M (SPW = 1: a strip,
// three waves; SPW = 4: the whole head, nine waves): two state waves per strip,
// each carrying 16 columns, and one copy wave.  LDS: NS input slots, each a
// chunk's -W, K^, the U0 of the workgroup's columns, the scalings, Q^T and P^T,
// copied from the workspace by the copy wave NS - 1 chunks ahead (or, with one
// slot, once the chunk's slot has been read).  A strip's two slots take 118 KiB,
// so one workgroup per CU; one slot 59 KiB, so two share a CU and cover each
// other's copies when the grid holds more workgroups than there are CUs.  A
// whole head takes 142 KiB with two slots, and with GATED 4 KiB more for the
// per-token sums of squares of the gated norm (see the kernel).
template <int NS, int SPW, bool GATED>
struct ChainLds {
  static constexpr int kW = 0, kKd = 16384, kU0 = 32768;
  static constexpr int kSc = kU0 + 4096 * SPW, kQ = kSc + 1024, kP = kQ + 16384;
  static constexpr int kSlot = kP + 6144;           // 59 (a strip) or 71 (a head) blocks of 1 KiB
  static constexpr int kBlocks = kSlot / 1024;
  static constexpr int kNSlot = NS;
  static constexpr int kNorm = NS * kSlot;          // GATED: [2 chunks][8 waves][64 tokens] fp32
  static constexpr int kBytes = kNorm + (GATED ? 2 * 8 * CH * 4 : 0);
};
constexpr int kAhead = 6;    // operand fragments a state wave reads ahead of its products
// A state wave's 54 operand fragments per chunk, as slot offsets of a one-strip slot,
// in the order its products take them: [0, 32) pairs of -W (even: row tile (j/2) & 3,
// key step j/8) and Q^T (odd: key step j/8, token tile (j/2) & 3); [32, 48) K^T (key
// tile (j-32) & 7, chunk step (j-32) / 8); [48, 54) the P^T fragments.
constexpr int kNFrag = 54;
constexpr int kFragOff[kNFrag] = {0, 37888, 4096, 38912, 8192, 39936, 12288, 40960, 1024, 41984, 5120, 43008, 9216, 44032, 13312, 45056, 2048, 46080, 6144, 47104, 10240, 48128, 14336, 49152, 3072, 50176, 7168, 51200, 11264, 52224, 15360, 53248, 16384, 18432, 20480, 22528, 24576, 26624, 28672, 30720, 17408, 19456, 21504, 23552, 25600, 27648, 29696, 31744, 54272, 55296, 56320, 57344, 58368, 59392};
// the same offsets in a slot of spw strips (Q^T and P^T follow the longer U0).  spw
// and the slot helpers below take the strip count as an argument, not a template
// parameter: the kernel calls them from lambdas, where a call of a function template
// keeps the host side from instantiating the kernel template's launch stub.
__device__ __forceinline__ constexpr int frag_off(int jf, int spw) {
  return (jf < 32 && (jf & 1)) || jf >= 48 ? kFragOff[jf] + 4096 * (spw - 1) : kFragOff[jf];
}

// source of 1 KiB block m of a chunk's input slot of spw strips (blocks follow the
// slot layout); strip: the first of the workgroup's strips
__device__ __forceinline__ const unsigned char* slot_src(int m, const unsigned char* wsh, const unsigned char* wkd,
                                                         const unsigned char* wsk, int strip, int spw) {
  const int kU = 32 + 4 * spw;
  return m < 16 ? wsh + 1024 * m                                           // -W
       : m < 32 ? wkd + 1024 * m                                           // K^T of the key head
       : m < kU ? wsh + WH_U0 + strip * 4096 + 1024 * (m - 32)             // U0 of the strips' value tiles
       : m < kU + 1 ? wsh + WH_SC                                          // scalings
       : m < kU + 17 ? wsk + 1024 * (m - kU - 1)                           // Q^T of the key head
                     : wsh + WH_P + 1024 * (m - kU - 17);                  // P^T
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float floatx2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const floatx2v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}
// four outputs of a row as bf16
__device__ __forceinline__ uint64_t pack_bf16x4(const floatx4& o) {
  return static_cast<uint64_t>(pack_bf16x2(o[0], o[1])) | (static_cast<uint64_t>(pack_bf16x2(o[2], o[3])) << 32);
}

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

// Each state wave runs one chunk step per barrier; the copy wave fills the slot
// of chunk c+1 (two slots) while the state waves read chunk c's, and waits for
// its copies before the barrier.  With one slot the copy waits for a second
// barrier per chunk, which each state wave reaches once it has read the slot.
// The window holds chunks [c0, c0 + nw) (workspace stride nwin).  A sequence's
// state comes from state_in at its first chunk and from `carry` otherwise, and
// goes to state_out after its last chunk and to `carry` otherwise.
// GATED (whole heads only): the gated RMSNorm of each output row needs the sum of
// squares over the head's 128 columns, which eight waves hold.  Each state wave
// leaves its 16 columns' sums of chunk c in LDS before the chunk's barrier and
// finishes chunk c's rows (norm, gate, store) during chunk c+1, after the barrier;
// the last chunk's rows after one more barrier.
template <int NS, int SPW, bool GATED, bool NTO = false>
__global__ __launch_bounds__(64 * (2 * SPW + 1), SPW == 1 ? 2 : 1) void chunk_chain_kernel(
    RecArgs a, int c0, unsigned char* ws, int nwin, int nw, float* carry) {
  static_assert(SPW == 1 || SPW == 4, "a strip or a whole head");
  static_assert(!GATED || SPW == 4, "the gated norm needs whole rows");
  using L = ChainLds<NS, SPW, GATED>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int L0 = blockIdx.x;
  int jh, strip;
  if constexpr (SPW == 4) {
    jh = L0;
    strip = wv < 8 ? wv >> 1 : 0;   // a state wave's strip; the copy wave copies all four
  } else {
    // Workgroups are handed to the 8 XCDs round-robin by linear index; when the
    // (slot, head) count is a multiple of 8, the 4 strips of a head get indices
    // that are equal modulo 8, so they share one XCD's L2 for the head's inputs.
    const int nheads = static_cast<int>(gridDim.x) >> 2;
    if ((nheads & 7) == 0) {
      jh = (L0 >> 5) * 8 + (L0 & 7);
      strip = (L0 >> 3) & 3;
    } else {
      jh = L0 >> 2;
      strip = L0 & 3;
    }
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

  const int nchunk = hi - lo;
  const unsigned char* regK = ws + static_cast<int64_t>(a.B) * a.Hv * nwin * WH_BYTES;
  auto wsh_of = [&](int cl) { return ws + (static_cast<int64_t>(bh) * nwin + lofs + cl) * WH_BYTES; };
  auto wsk_of = [&](int cl) { return regK + (static_cast<int64_t>(bw * a.Hk + hk) * nwin + lofs + cl) * WK_BYTES; };
  // K^ sits in the block of the key head's first value head
  auto wkd_of = [&](int cl) { return ws + (static_cast<int64_t>(bw * a.Hv + hk * a.G) * nwin + lofs + cl) * WH_BYTES; };
  auto copy_chunk = [&](int cl) {
    unsigned char* slot = smem + (cl % L::kNSlot) * L::kSlot;
    const unsigned char* wsh = wsh_of(cl);
    const unsigned char* wkd = wkd_of(cl);
    const unsigned char* wsk = wsk_of(cl);
#pragma unroll
    for (int m = 0; m < L::kBlocks; ++m)
      __builtin_amdgcn_global_load_lds(slot_src(m, wsh, wkd, wsk, SPW == 1 ? strip : 0, SPW) + 16 * lane,
                                       slot + 1024 * m, 16, 0, 0);
  };

  // Waves 2s and 2s+1 each carry 16 value columns of strip s (32 strip + 16 wave ..)
  // and form their outputs; the last wave copies.  With one strip the three waves
  // sit on three SIMDs.
  if (wv < 2 * SPW) {
    const int sh = wv & 1;
    const int col = 32 * strip + 16 * sh + l16;   // this lane's value column
    const int vtile = 2 * strip + sh;             // value tile of the head (16 columns)
    floatx4 Ms[8];     // 2^s_cur M, rows 16dt + 4g + v, column col
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (state_in) {
        const float* sp = state_in + static_cast<int64_t>(bhv) * DK * DK;
#pragma unroll
        for (int v = 0; v < 4; ++v) Ms[dt][v] = sp[(16 * dt + 4 * g4 + v) * DK + col];
      } else {
        Ms[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // Range of the fp16 products.  The state is held scaled by 2^s_cur (a multiple of 4)
    // and s_cur never exceeds the chunk's V exponent, so the chunk's V, scaled, stays below
    // 2^(kRangeTop+1) = 8.  Every kCheck chunks of the sequence the largest |M| over the
    // wave is measured; outside [2^(kRangeTop-4), 2^(kRangeTop+4)) s_cur moves by a
    // multiple of 4 that brings it into [2^(kRangeTop-3), 2^(kRangeTop+1)).  So at a check
    // |M| < 64 and its spectral norm is below 128 * 64; each token changes the state by at
    // most |v|_2 < 8 sqrt(128) (for beta <= 1, log alpha <= 0 and key norms <= 1), so six
    // chunks later it is below 8192 + 6 * 64 * 90.6 < 43000, and the rows of U (at most
    // |v|_2 + |S|) stay below fp16's 65504 as well.  A large state that decays under small
    // values is measured as soon as its decayed bound (est) leaves the window.  A sequence
    // that runs on from the previous window starts from the scale and bound that window left
    // in the scalings block of its last chunk (words 96 + value tile, 104 + value tile), so
    // the scales, and so the results, do not depend on the window size.
    const int hand = 96 + vtile;
    const int ci0 = lo - cs;   // chunk index inside the sequence of the window's first chunk
    uint16_t* go = static_cast<uint16_t*>(a.o) + tok0 * a.so + hv * DK + 32 * strip + 16 * sh + 4 * g4;
    int64_t roff[4];   // element offsets of this lane's output rows inside a chunk
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) roff[ct] = static_cast<int64_t>(16 * ct + l16) * a.so;
    // GATED: the rows of the previous chunk (unscaled outputs, z) until they are normed
    float* nrm = reinterpret_cast<float*>(smem + L::kNorm);
    const uint16_t* gz = static_cast<const uint16_t*>(a.gz) + tok0 * a.sz + hv * DK + 32 * strip + 16 * sh + 4 * g4;
    // the gated norm's registers leave fewer for fragments in flight: with three the
    // kernel fits the 168 registers that three waves per SIMD allow, without spills
    constexpr int kAh = GATED ? 3 : kAhead;
    uint2 nwb;        // norm weights of this lane's four columns (bf16)
    floatx4 Op[4];    // the previous chunk's outputs
    uint2 zp[4];      // its gate inputs, four bf16 per token tile
    if constexpr (GATED) {
      nwb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.gw) + 16 * vtile + 4 * g4);
    }
    // z of chunk ci (rows past the sequence's end are not read)
    auto load_z = [&](int ci, int nval) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int r = 16 * ct + l16;
        zp[ct] = r < nval ? *reinterpret_cast<const uint2*>(gz + (static_cast<int64_t>(ci) * CH + r) * a.sz)
                          : uint2{0u, 0u};
      }
    };
    // the gated norm of chunk ci's rows (window chunk pcl), once every wave's sums are in LDS
    auto finish_rows = [&](int pcl, int ci, int nval) {
      const float* nb = nrm + (pcl & 1) * 8 * CH;
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) tot += nb[w * CH + lane];   // token `lane`
      const float inv = rsqrtf(tot * (1.0f / DK) + a.geps);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int r = 16 * ct + l16;
        const float iv = __shfl(inv, r, 64);
        const uint32_t zw[2] = {zp[ct].x, zp[ct].y};
        float y[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float z = bf16_bits_to_f32(static_cast<uint16_t>(zw[v >> 1] >> (16 * (v & 1))));
          const float nw = bf16_bits_to_f32(static_cast<uint16_t>((v < 2 ? nwb.x : nwb.y) >> (16 * (v & 1))));
          y[v] = Op[ct][v] * iv * nw * z * sigmoidf_(z);
        }
        const uint2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        if (r < nval) *reinterpret_cast<uint2*>(go + (static_cast<int64_t>(ci) * CH + r) * a.so) = w;
      }
    };
    int pnval = 0;    // GATED: rows of the previous chunk
    __syncthreads();
    int s_cur, est;   // est: 2^(est+1) bounds the decayed part of the state measured last (scaled)
    halfx8 Mfr[4];
    // The scale of chunk ci (V exponent rn), decided once the previous chunk is done: the
    // state is measured every kCheck chunks and when its decayed bound has faded below the
    // window while V leaves room to raise the scale; s_cur never exceeds rn.  A change by 2^d
    // reaches the fp32 state through the next decay factor and M's fp16 fragments through
    // exact multiplies by powers of two.
    auto decide = [&](int ci, int rn) {
      const bool faded = est < kRangeTop - 4 && s_cur < rn - 3;
      int d = 0;
      if (s_cur > rn || ci % kCheck == 0 || faded) {
        int s_new = s_cur;
        if (ci % kCheck == 0 || faded) {
          const uint32_t mb = wave_max_bits(__float_as_uint(lane_max_abs32(Ms)));
          const int e = exp_of_bits(mb);
          est = mb == 0u ? kExpLo : e;
          if (mb == 0u) s_new = rn;
          else if (e < kRangeTop - 4 || e >= kRangeTop + 4) s_new = floor4(kRangeTop - e) + s_cur;
        }
        s_new = __builtin_amdgcn_readfirstlane(min(kExpHi, max(kExpLo, min(s_new, rn))));
        d = s_new - s_cur;
        s_cur = s_new;
        est = __builtin_amdgcn_readfirstlane(max(kExpLo, est + d));
      }
      return d;
    };
    auto scale_frags = [&](int d) {
      while (d != 0) {
        const int st = max(-14, min(15, d));
        const halfx8 f = scale_h(st);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Mfr[ks] *= f;
        d -= st;
      }
    };
    int dpend = 0;   // a change of scale that the next decay factor still has to apply to Ms
    if (ci0 > 0) {
      const int32_t* hw = reinterpret_cast<const int32_t*>(ws + (static_cast<int64_t>(bh) * nwin + nwin - 1) * WH_BYTES + WH_SC);
      s_cur = __builtin_amdgcn_readfirstlane(hw[hand]);
      est = __builtin_amdgcn_readfirstlane(hw[hand + 8]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) Ms[dt][v] = __builtin_amdgcn_ldexpf(Ms[dt][v], s_cur);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Mfr[ks] = stack_h(Ms[2 * ks], Ms[2 * ks + 1]);
      // the decision an unbroken run takes at the end of the previous chunk
      dpend = decide(ci0, __builtin_amdgcn_readfirstlane(reinterpret_cast<const int32_t*>(smem + L::kSc)[65 + vtile]));
      scale_frags(dpend);
    } else {
      // the sequence's first chunk: from the entry state's range and the chunk's V exponent
      const int r0 = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int32_t*>(smem + L::kSc)[65 + vtile]);
      const uint32_t mb = wave_max_bits(__float_as_uint(lane_max_abs32(Ms)));
      s_cur = mb == 0u ? r0 : min(r0, range_exp(mb));
      est = mb == 0u ? kExpLo : exp_of_bits(mb) + s_cur;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) Ms[dt][v] = __builtin_amdgcn_ldexpf(Ms[dt][v], s_cur);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Mfr[ks] = stack_h(Ms[2 * ks], Ms[2 * ks + 1]);
    }
    if constexpr (GATED) load_z(ci0, min(CH, len - ci0 * CH));
#pragma clang loop unroll(disable)
    for (int cl = 0; cl < nchunk; ++cl) {
      unsigned char* slot = smem + (cl % L::kNSlot) * L::kSlot;
      const float* sSc = reinterpret_cast<const float*>(slot + L::kSc);
      // The step's operand fragments are read kAh ahead of their products
      // (kFragOff), across the three phases below.
      auto rd = [&](int jf) { return *reinterpret_cast<const halfx8*>(slot + frag_off(jf, SPW) + lane * 16); };
      const float gC = sSc[64];
      const int u0t = SPW == 1 ? sh : vtile;   // the value tile's place in the slot's U0
      const halfx8 u0a = *reinterpret_cast<const halfx8*>(slot + L::kU0 + u0t * 2048 + lane * 32);
      const halfx8 u0b = *reinterpret_cast<const halfx8*>(slot + L::kU0 + u0t * 2048 + lane * 32 + 16);
      float gam[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) gam[ct] = sSc[16 * ct + l16];
      // U0 holds 2^rexp U0; gamma_63 < 2^(gexp+1); rnext: the next chunk's V exponent (the same
      // words in every lane)
      const int rexp = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int32_t*>(sSc)[65 + vtile]);
      const int gexp = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int32_t*>(sSc)[73]);
      const int rnext = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int32_t*>(sSc)[80 + vtile]);
      const int ci = ci0 + cl;   // chunk index inside the sequence
      halfx8 F[kNFrag];
#pragma unroll
      for (int jf = 0; jf < kAh; ++jf) F[jf] = rd(jf);
      const float gCs = dpend == 0 ? gC : __builtin_amdgcn_ldexpf(gC, dpend);
      __builtin_amdgcn_sched_barrier(0);
      // U = -W M first and U0 after: the first products wait for nothing but their fragments
      floatx4 U[4], O[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) U[rt] = O[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
      // ---- U = U0 - W M and O^T = M^T Q^T, interleaved ---------------------------
#pragma unroll
      for (int jf = 0; jf < 32; ++jf) {
        F[jf + kAh] = rd(jf + kAh);
        __builtin_amdgcn_sched_barrier(0);
        const int x = (jf >> 1) & 3, ks = jf >> 3;
        if (jf & 1) O[x] = mfma16h(Mfr[ks], F[jf], O[x]);
        else U[x] = mfma16h(F[jf], Mfr[ks], U[x]);
        if (jf == 16) {
          // the state's decay, on the vector unit while the products run
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) Ms[dt] *= gCs;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        const float u0s = __builtin_amdgcn_ldexpf(1.f, s_cur - rexp);   // 1, or a power of two < 1 (0 far below)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            U[rt][v] = fmaf(static_cast<float>(rt < 2 ? u0a[4 * rt + v] : u0b[4 * (rt - 2) + v]), u0s, U[rt][v]);
      }
      halfx8 Uf[2], Ug[2];   // U for the output products; Ug = diag(f) U for the update
      Uf[0] = stack_h(U[0], U[1]);
      Uf[1] = stack_h(U[2], U[3]);
      {
        floatx4 Us[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Us[rt] = U[rt] * *reinterpret_cast<const floatx4*>(sSc + 128 + 16 * rt + 4 * g4);
        Ug[0] = stack_h(Us[0], Us[1]);
        Ug[1] = stack_h(Us[2], Us[3]);
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) O[ct] *= gam[ct];
      // ---- M <- gamma_63 M + K^T diag(f) U -----------------------------------------
#pragma unroll
      for (int jf = 32; jf < 48; ++jf) {
        if (jf + kAh < kNFrag) F[jf + kAh] = rd(jf + kAh);
        if constexpr (NS == 1) {
          if (jf + kAh == kNFrag - 1) {
            // the slot's last fragment is in flight: once it is back and every wave is here,
            // the slot is refilled with chunk cl+1
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        Ms[(jf - 32) & 7] = mfma16h(F[jf], Ug[(jf - 32) >> 3], Ms[(jf - 32) & 7]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (GATED) {
        if (cl > 0) {
          finish_rows(cl - 1, ci - 1, pnval);
          load_z(ci, min(CH, len - ci * CH));
        }
      }
      // the last fragments, when fewer than six are read ahead
#pragma unroll
      for (int jf = 48 + kAh; jf < kNFrag; ++jf) F[jf] = rd(jf);
      // ---- O^T += U^T P^T: P^T fragment f covers token tile f (chunk step 0) or f - 2 (step 1)
#pragma unroll
      for (int f = 0; f < 6; ++f) {
        const int ct = f < 4 ? f : f - 2;
        O[ct] = mfma16h(Uf[f < 4 ? 0 : 1], F[48 + f], O[ct]);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) Mfr[ks] = stack_h(Ms[2 * ks], Ms[2 * ks + 1]);
      // outputs, unscaled: lane holds token 16ct + (lane & 15), value columns 4g..4g+3 of the wave's 16
      const int nval = min(CH, len - ci * CH);
      const int s_out = s_cur;
      est = __builtin_amdgcn_readfirstlane(max(kExpLo, est + gexp + 1));   // this chunk's decay
      dpend = 0;
      if (cl + 1 < nchunk) {
        dpend = decide(ci + 1, rnext);
        scale_frags(dpend);
      }
      if (s_out != 0) {
        const float os = __builtin_amdgcn_ldexpf(1.f, -s_out);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) O[ct] *= os;
      }
      if constexpr (GATED) {
        // this chunk's sums of squares over the wave's 16 columns: token tile ct's in every
        // lane of the row, token `lane`'s to LDS
        float p[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          p[ct] = O[ct][0] * O[ct][0];
#pragma unroll
          for (int v = 1; v < 4; ++v) p[ct] = fmaf(O[ct][v], O[ct][v], p[ct]);
          p[ct] += __shfl_xor(p[ct], 16, 64);
          p[ct] += __shfl_xor(p[ct], 32, 64);
          Op[ct] = O[ct];
        }
        nrm[((cl & 1) * 8 + wv) * CH + lane] = g4 == 0 ? p[0] : g4 == 1 ? p[1] : g4 == 2 ? p[2] : p[3];
        pnval = nval;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      } else {
        uint16_t* gc = go + static_cast<int64_t>(ci) * CH * a.so;
        if (nval == CH) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) {
            // NTO: without allocating in the caches (chosen at compile time: the compiler
            // merges the two stores of a run-time choice into a plain one)
            if constexpr (NTO) __builtin_nontemporal_store(pack_bf16x4(O[ct]), reinterpret_cast<uint64_t*>(gc + roff[ct]));
            else *reinterpret_cast<uint64_t*>(gc + roff[ct]) = pack_bf16x4(O[ct]);
          }
        } else {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct)
            if (16 * ct + l16 < nval) {
              if constexpr (NTO) __builtin_nontemporal_store(pack_bf16x4(O[ct]), reinterpret_cast<uint64_t*>(gc + roff[ct]));
              else *reinterpret_cast<uint64_t*>(gc + roff[ct]) = pack_bf16x4(O[ct]);
            }
        }
      }
      // slot cl may be refilled once both state waves have passed this barrier
      __builtin_amdgcn_s_barrier();
      if constexpr (GATED) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    if constexpr (GATED) {
      // the last chunk's rows, once every wave's sums are in LDS
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      finish_rows(nchunk - 1, ci0 + nchunk - 1, pnval);
    }
    if (hi < ce && lane == 0) {
      // the scale handed to the next window (the block of this window's last chunk, nwin - 1)
      int32_t* hw = reinterpret_cast<int32_t*>(ws + (static_cast<int64_t>(bh) * nwin + nwin - 1) * WH_BYTES + WH_SC);
      hw[hand] = s_cur;
      hw[hand + 8] = est;
    }
    if (state_out) {
      float* sp = state_out + static_cast<int64_t>(bhv) * DK * DK;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int v = 0; v < 4; ++v) sp[(16 * dt + 4 * g4 + v) * DK + col] = __builtin_amdgcn_ldexpf(Ms[dt][v], -s_cur);
    }
  } else {
    // copy wave: chunk cl+1 into the other slot (two slots; slot (cl + 1) % 2 was last
    // read during chunk cl-1) or, with one slot, once both state waves have read
    // chunk cl's
    copy_chunk(0);
    wait_vm_all();
    __syncthreads();
    for (int cl = 0; cl < nchunk; ++cl) {
      if constexpr (NS == 1) __builtin_amdgcn_s_barrier();
      if (cl + 1 < nchunk) copy_chunk(cl + 1);
      wait_vm_all();
      // this wave writes LDS only through its copies, and the vector memory count
      // above covers the ones the others read next
      __builtin_amdgcn_s_barrier();
    }
    if constexpr (GATED) __builtin_amdgcn_s_barrier();   // the state waves' last rows
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

// Prep workgroups resident at once: their LDS lets two share a CU up to 19 value
// heads per key head, one beyond.
int prep_slots(int G) { return device_cu_count() * max(1, min(2, (160 * 1024) / PrepLds::bytes(G))); }

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
//
// A long sequence on the two-slot strip chain (more than two such windows) runs
// windows of about 200 MiB instead, with the chain's outputs stored without allocating
// in the caches, so that they do not push the window's operands out: batch 1, 16/48
// heads, 64-chunk windows against 32, T=8192 250 against 267 us, T=65536 2.00 against
// 2.14 ms, T=262144 8.01 against 8.55 ms (8.58 ms with 64 and plain stores); 32 packed
// requests of 16 to 7,574 tokens (38,693 in all) 1.27 against 1.38 ms.  At T=4096
// one such window is slower than two of 32 (127.0 against 125.1 us), and whole-head
// chains write their outputs in pieces that the caches should merge (batch 4, T=32768:
// 8.69 against 7.30 ms), so neither takes it.
namespace {
int window_for(const RecArgs& a, size_t cache) {
  const int nchunks = chunk_count(a);
  const size_t per = chunk_ws_bytes_per_chunk(a);
  const int round = max(1, prep_slots(a.G) / (a.Hk * a.B));   // chunks one round of prep covers
  const size_t budget = static_cast<size_t>(round) * per <= cache ? cache : size_t(2) << 30;
  const int fit = static_cast<int>(min(budget / per, static_cast<size_t>(1) << 30));
  int w = max(1, fit / round) * round;
  w = max(1, min(w, fit));
  if (w >= nchunks) return nchunks;
  const int nwins = (nchunks + w - 1) / w;
  return (nchunks + nwins - 1) / nwins;
}
// the chain runs one workgroup per value head (and the prep stores for it)
bool whole_heads(const RecArgs& a) { return a.gz || (!a.cu_seqlens && a.B * a.Hv >= device_cu_count()); }
// the two-slot strip chain runs the sequences (a workgroup per CU at most for a fixed batch;
// a packed batch always runs it)
bool long_strip_run(const RecArgs& a) {
  if (whole_heads(a) || a.B * a.Hv * (DK / 32) > device_cu_count()) return false;
  return chunk_count(a) > 2 * window_for(a, size_t(96) << 20);
}
}  // namespace

int chunk_window_chunks(const RecArgs& a) {
  return window_for(a, long_strip_run(a) ? size_t(200) << 20 : size_t(96) << 20);
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
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel<2, 1, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds<2, 1, false>::kBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel<2, 1, false, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds<2, 1, false>::kBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel<1, 1, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds<1, 1, false>::kBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel<2, 4, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds<2, 4, false>::kBytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_chain_kernel<2, 4, true>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, ChainLds<2, 4, true>::kBytes);
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
  // When the heads alone fill the GPU, one chain workgroup per head copies each chunk's
  // operands into LDS once instead of once per strip (batch 4, T=32768, 128 value heads:
  // 7.31 ms of prefill against 10.34 ms with the one-slot strips); the gated norm needs
  // whole rows and always runs so.
  const bool heads = whole_heads(a), ntout = long_strip_run(a);
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
    if (a.gz)
      hipLaunchKernelGGL((chunk_chain_kernel<2, 4, true>), dim3(slots * a.Hv), dim3(576),
                         (ChainLds<2, 4, true>::kBytes), s, r, c0, wsb, nwin, nw, carry);
    else if (heads)
      hipLaunchKernelGGL((chunk_chain_kernel<2, 4, false>), dim3(slots * a.Hv), dim3(576),
                         (ChainLds<2, 4, false>::kBytes), s, r, c0, wsb, nwin, nw, carry);
    else if (ntout)
      hipLaunchKernelGGL((chunk_chain_kernel<2, 1, false, true>), grid, dim3(192), (ChainLds<2, 1, false>::kBytes), s,
                         r, c0, wsb, nwin, nw, carry);
    else if (!a.cu_seqlens && a.B * a.Hv * (DK / 32) > device_cu_count())
      hipLaunchKernelGGL((chunk_chain_kernel<1, 1, false>), grid, dim3(192), (ChainLds<1, 1, false>::kBytes), s, r,
                         c0, wsb, nwin, nw, carry);
    else
      hipLaunchKernelGGL((chunk_chain_kernel<2, 1, false>), grid, dim3(192), (ChainLds<2, 1, false>::kBytes), s, r,
                         c0, wsb, nwin, nw, carry);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
