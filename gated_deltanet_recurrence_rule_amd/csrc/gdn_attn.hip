// gdn_attn.hip -- the full-attention layer of the hybrid stack ("L'attention
// hybride", section "Les 16 couches d'attention complete"): per-head RMSNorm
// and partial RoPE of q and k, causal grouped-query attention with head width
// 256, and the sigmoid output gate that the doubled query projection carries
// ("Le facteur 2 sur W_Q", "GQA a 6:1", "Le RoPE partiel").
//
// Kernels:
//  * attn_prep_kernel: one workgroup per token, a wave per 256-wide row.  Query
//    rows are normalised and rotated into the qrot scratch, key rows likewise
//    into the key cache at the token's position; a decode token's value row is
//    copied into the value cache, whose 64-position blocks are stored transposed
//    ([256][64]) so that the products read them as MFMA operands with positions
//    along k.  attn_vblock_kernel writes a prefill's values a block at a time.
//  * attn_fwd_kernel (prefill): 4 waves x 32 query rows of one query head.
//    Per block of 64 keys: S^T = K Q^T on 32x32x16 bf16 MFMA (keys on the MFMA
//    rows, queries on its columns, so each lane holds one query's scores and
//    the softmax statistics are per lane plus one exchange across the two lane
//    halves), the weights 2^(s - m) against a fixed per-row reference m, then
//    O^T += V^T P^T, whose B operand is the score accumulator itself rounded to
//    bf16 (the key order of the accumulator rows is the k order of the operand).
//    Key and value blocks are copied into LDS, double-buffered, with the next
//    block's copies in flight during the products.
//  * attn_decode_kernel: one wave per (256 cached positions, key/value head,
//    sequence) runs the same products on 16x16x32 tiles with the group's query
//    heads as the MFMA columns, streaming keys and values through its own LDS
//    (keys a 32-position block at a time, values two blocks at a time);
//    attn_combine_kernel merges the partial maxima, sums and outputs of a head
//    and applies the gate.
#include <cmath>

#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int AD = 256;      // head width
constexpr int QB = 128;      // query rows per prefill workgroup (4 waves x 32)
constexpr int KB = 64;       // keys per block
constexpr int KBUF = KB * AD * 2;   // LDS key block: 64 rows of 512 bytes
constexpr int VBUF = AD * KB * 2;   // LDS transposed value block: 256 rows of 128 bytes
constexpr int kFwdLds = 2 * (KBUF + VBUF);
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// row of value v of a 32x32 accumulator in lane half h
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }
// Key held by row r of a 32-key S^T tile: rows 16a + 8b + 4h + c hold key
// 16a + 8h + 4b + c (bits 2 and 3 swapped).  The accumulator values 8s..8s+7
// of lane half h, which become the k slots of the P^T operand, then hold the 8
// consecutive keys 16s + 8h.., so a value operand is one 16-byte read.
__device__ __forceinline__ int key_of_row(int r) { return (r & ~12) | ((r & 8) >> 1) | ((r & 4) << 1); }

__device__ __forceinline__ int64_t kc_index(const AttnArgs& a, int b, int j, int pos) {
  return ((static_cast<int64_t>(b) * a.Hkv + j) * a.S_max + pos) * AD;
}
// first element of the transposed value block holding position pos
__device__ __forceinline__ int64_t vc_block(const AttnArgs& a, int b, int j, int pos) {
  return ((static_cast<int64_t>(b) * a.Hkv + j) * (a.S_max / KB) + pos / KB) * KB * AD;
}

// ---------------------------------------------------------------------------
// prep: rows are, per token, Hq query rows and Hkv key rows, then (decode only)
// Hkv value rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_prep_kernel(AttnArgs a, RopeTable rt) {
  // one workgroup per token; wave w takes the token's rows w, w + 4, ...
  const int64_t tok = blockIdx.x;
  const int b = static_cast<int>(tok / a.T), t = static_cast<int>(tok - static_cast<int64_t>(b) * a.T);
  const int pos = a.cache_len ? min(max(a.cache_len[b], 0), a.S_max - 1) : t;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int d0 = 4 * lane;
  const int R = a.Hq + (a.cache_len ? 2 : 1) * a.Hkv;   // prefill values go through attn_vblock_kernel
  // RoPE: dimension i < half pairs with i + half; half is a multiple of 4, so a
  // lane's partner lane is half/4 away.  The angle and its reduction to
  // [-pi, pi] are fp64 (positions reach 10^5 and more, where an fp32 angle would
  // be off by ~1e-2 rad); sin and cos are fp32, once per lane and token.
  const int half = a.rot_dim / 2, lo = half / 4;
  const int pl = lane < lo ? lane + lo : lane - lo;
  const bool rot = d0 < a.rot_dim, first = d0 < half;
  float cs[4], sn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cs[i] = 1.f;
    sn[i] = 0.f;
    if (rot) {
      const double ang = static_cast<double>(pos) * rt.inv_freq[(first ? d0 : d0 - half) + i];
      const double turns = rint(ang * 0.15915494309189535);
      sincosf(static_cast<float>(fma(-turns, 6.283185307179586, ang)), &sn[i], &cs[i]);
    }
  }
  auto src_of = [&](int r) -> const uint16_t* {
    if (r < a.Hq) return a.qg + tok * a.sqg + static_cast<int64_t>(r) * 2 * AD;
    if (r < a.Hq + a.Hkv) return a.k + tok * a.sk + static_cast<int64_t>(r - a.Hq) * AD;
    return a.v + tok * a.sv + static_cast<int64_t>(r - a.Hq - a.Hkv) * AD;
  };
  const u16x4 wq = *reinterpret_cast<const u16x4*>(a.qw + d0);
  const u16x4 wk = *reinterpret_cast<const u16x4*>(a.kw + d0);
  u16x4 nxt = w < R ? *reinterpret_cast<const u16x4*>(src_of(w) + d0) : u16x4{0, 0, 0, 0};
  for (int r = w; r < R; r += 4) {
    const u16x4 x4 = nxt;
    if (r + 4 < R) nxt = *reinterpret_cast<const u16x4*>(src_of(r + 4) + d0);   // next row in flight
    if (r >= a.Hq + a.Hkv) {   // decode only: the token's value, into its transposed block
      const int j = r - a.Hq - a.Hkv;
      uint16_t* dst = a.vc + vc_block(a, b, j, pos) + pos % KB;
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(d0 + i) * KB] = x4[i];
      continue;
    }
    const bool isq = r < a.Hq;
    const u16x4 w4 = isq ? wq : wk;
    float y[4];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = bf16_bits_to_f32(x4[i]);
      ss += y[i] * y[i];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / AD + a.eps);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = y[i] * inv * bf16_bits_to_f32(w4[i]);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __shfl(y[i], pl, 64);
    if (rot) {
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = first ? y[i] * cs[i] - p[i] * sn[i] : y[i] * cs[i] + p[i] * sn[i];
    }
    u16x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = f32_to_bf16_bits(y[i]);
    uint16_t* dst = isq ? a.qrot + (tok * a.Hq + r) * AD : a.kc + kc_index(a, b, r - a.Hq, pos);
    *reinterpret_cast<u16x4*>(dst + d0) = out;
  }
}

// ---------------------------------------------------------------------------
// prefill attention
// ---------------------------------------------------------------------------
// LDS layout of a block.  Row m of key tile u (rows 32u..32u+31) holds key
// 32u + key_of_row(m), so the A operand's lane m reads LDS row 32u + m.  The
// 16-byte chunk c (keys: dims 8c..; values: positions 8c..) of key row r sits
// at chunk position c ^ (r & 15), of value row r at c ^ ((r >> 1) & 7): sixteen
// consecutive rows, read by sixteen consecutive lanes, then fall on distinct
// 16-byte bank groups of a 256-byte bank line (5 % faster than swizzling with
// r & 7).  A block is 32 + 32 pieces of 1 KiB copied straight from the caches
// into LDS (lane i of a piece fills bytes 16i..16i+15 of it), 16 per wave.
__device__ __forceinline__ void copy_pieces(const AttnArgs& a, int b, int j, int kb, int w, int lane,
                                            unsigned char* kbuf, unsigned char* vbuf, int i0, int n) {
  const unsigned char* ks = reinterpret_cast<const unsigned char*>(a.kc + kc_index(a, b, j, kb * KB));
  const unsigned char* vs = reinterpret_cast<const unsigned char*>(a.vc + vc_block(a, b, j, kb * KB));
#pragma unroll
  for (int i = i0; i < i0 + n; ++i) {
    if (i < 8) {
      const int pc = 8 * w + i;
      const int r = 2 * pc + (lane >> 5), c = (lane & 31) ^ (r & 15);
      const int key = 32 * (r >> 5) + key_of_row(r & 31);
      __builtin_amdgcn_global_load_lds(ks + key * (AD * 2) + 16 * c, kbuf + 1024 * pc, 16, 0, 0);
    } else {
      const int pc = 8 * w + i - 8;
      const int r = 8 * pc + (lane >> 3), c = (lane & 7) ^ ((r >> 1) & 7);
      __builtin_amdgcn_global_load_lds(vs + r * (KB * 2) + 16 * c, vbuf + 1024 * pc, 16, 0, 0);
    }
  }
}

__device__ __forceinline__ void copy_block(const AttnArgs& a, int b, int j, int kb, int w, int lane,
                                           unsigned char* kbuf, unsigned char* vbuf) {
  copy_pieces(a, b, j, kb, w, lane, kbuf, vbuf, 0, 16);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)

__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // Workgroup -> (sequence, query head, query block).  Workgroups start in
  // index order, so the longest work goes first: index L is rank L / NG of
  // key/value group L % NG, and a rank is a query block counted from the last
  // (the most keys) with the group's query heads inside it.  The 8 XCDs take
  // indices round-robin; with NG dividing 8, or a multiple of it, each XCD then
  // sees one group only (its keys and values stay in that XCD's L2), and the
  // XCDs sharing a group take alternate ranks, i.e. equal causal work.  Inside
  // an XCD, a CU that finishes takes the longest item left, which balances
  // the CUs far better than any fixed long/short interleave.
  const int nqb = (a.T + QB - 1) / QB;
  const int G = a.Hq / a.Hkv;
  const int NG = a.B * a.Hkv;
  const int L = static_cast<int>(blockIdx.x);
  const int grp = L % NG, rank = L / NG;
  const int qb = nqb - 1 - rank / G;
  const int b = grp / a.Hkv, j = grp - b * a.Hkv;
  const int h = j * G + rank % G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int q0 = qb * QB + 32 * w;  // the wave's first query
  const int qi = q0 + l32;          // the lane's query
  const int64_t tok = static_cast<int64_t>(b) * a.T + min(qi, a.T - 1);

  // queries as the B operand of S^T = K Q^T: k step s = dims 16s.., lane half hh
  // holds 8 consecutive dims (the key fragments use the same assignment)
  bf16x8 Qf[16];
  {
    const uint16_t* qr = a.qrot + (tok * a.Hq + h) * AD + 8 * hh;
#pragma unroll
    for (int s = 0; s < 16; ++s) Qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(qr + 16 * s));
  }
  floatx16 O[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) O[t][v] = 0.f;
  float m = 0.f, l = 0.f;
  bool over = false;
  const float sl2 = a.scale * kLog2e;

  // blocks: keys past T are zero in the caches (the value block kernel writes
  // whole blocks), and masked as later than every query
  const int last_key = min(qb * QB + QB, a.T) - 1;   // the largest key any row here sees
  const int nkb = last_key / KB + 1;
  const int xk = l32 & 15, xv = (l32 >> 1) & 7;   // this lane's chunk swizzles (key rows, value rows)
  copy_block(a, b, j, 0, w, lane, smem, smem + 2 * KBUF);
  wait_vm_all();
  __syncthreads();
  // The softmax reference of a row is the maximum of its scores in the first
  // block (which holds key 0, seen by every row), and it stays fixed: the
  // output then only ever accumulates in the matrix cores, with no rescaling.
  // Weights 2^(s - m) are fp32 and bf16 numbers, whose range is the same, and
  // stay far inside it unless a later score exceeds the reference by more than
  // 96 (base 2); a wave that sees one redoes its rows exactly after the loop.
  // Blocks that end before the wave's first query need no causal mask: they run
  // through a copy of the body without it.  Every wave runs nkb bodies, one
  // barrier each.
  auto body = [&](int kb, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const int cur = kb & 1;
    const unsigned char* sk = smem + cur * KBUF;
    const unsigned char* sv = smem + 2 * KBUF + cur * VBUF;
    // the next block's copy goes out two pieces per group of products, so that
    // the memory path works under the matrix cores instead of stalling the
    // wave; after the last block the current one is copied again (harmless,
    // nothing reads that buffer any more)
    const int kn = min(kb + 1, nkb - 1);
    auto cp = [&](int i0) {
      copy_pieces(a, b, j, kn, w, lane, smem + (cur ^ 1) * KBUF, smem + 2 * KBUF + (cur ^ 1) * VBUF, i0, 2);
    };

    // S^T tiles u = keys 32u.. of the block; key fragments are read from LDS eight
    // at a time, one group ahead of the products
    floatx16 S[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) S[u][v] = 0.f;
    {
      const unsigned char* kr = sk + l32 * (AD * 2);
      u16x8 kf[2][8];
      auto kload = [&](int g, u16x8* dst) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int st = 4 * g + (i >> 1), u = i & 1;
          dst[i] = *reinterpret_cast<const u16x8*>(kr + 32 * u * (AD * 2) + 16 * ((2 * st + hh) ^ xk));
        }
      };
      kload(0, kf[0]);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g < 3) kload(g + 1, kf[(g + 1) & 1]);
        cp(2 * g);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int st = 4 * g + (i >> 1), u = i & 1;
          S[u] = mfma32(__builtin_bit_cast(bf16x8, kf[g & 1][i]), Qf[st], S[u]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // mask keys after the query (blocks that reach past the wave's first query
    // only), block maximum of the raw scores; the weights are 2^(s sl2 - m)
    const int kbase = kb * KB;
    float sc[2][16];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sc[u][v] = kMasked && kbase + 32 * u + key_of_row(acc_row(v, hh)) > qi ? -INFINITY : S[u][v];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[u][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;
    if (kb == 0) m = mx;            // finite: key 0 precedes every query
    over |= mx > m + 96.0f;
    // P^T fragments: accumulator values 8s2..8s2+7 of tile u are keys
    // 32u + 16 s2 + 8hh + 0..7
    bf16x8 P[4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[u][8 * s2 + e], sl2, -m));
          l += p;
          P[2 * u + s2][e] = static_cast<__bf16>(p);
        }
    // O^T += V^T P^T: A operand rows = dims 32t + l32, k = the same key order;
    // value fragments eight at a time (one k step), one group ahead
    {
      const unsigned char* vr = sv + l32 * (KB * 2);
      u16x8 vf[2][8];
      auto vload = [&](int ks, u16x8* dst) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          dst[t] = *reinterpret_cast<const u16x8*>(vr + 32 * t * (KB * 2) + 16 * ((2 * ks + hh) ^ xv));
      };
      vload(0, vf[0]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (ks < 3) vload(ks + 1, vf[(ks + 1) & 1]);
        cp(8 + 2 * ks);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 8; ++t) O[t] = mfma32(__builtin_bit_cast(bf16x8, vf[ks & 1][t]), P[ks], O[t]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vm_all();   // this wave's pieces of the next block are in LDS
    __syncthreads();
  };
  // blocks whose keys all precede the wave's first query (uniform over the wave)
  const int nfree = __builtin_amdgcn_readfirstlane(min(nkb, (q0 + 1) / KB));
  for (int kb = 0; kb < nfree; ++kb) body(kb, std::false_type{});
  for (int kb = nfree; kb < nkb; ++kb) body(kb, std::true_type{});
  if (__builtin_amdgcn_ballot_w64(over)) {
    // Exact redo of this wave's rows, straight from the caches: the row maxima
    // over all visible keys first, then the weights and values against them.
    const unsigned char* kcb = reinterpret_cast<const unsigned char*>(a.kc + kc_index(a, b, j, 0));
    auto scores = [&](int kb, floatx16* Sx) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int v = 0; v < 16; ++v) Sx[u][v] = 0.f;
        const unsigned char* kr = kcb + static_cast<int64_t>(kb * KB + 32 * u + key_of_row(l32)) * (AD * 2) + 16 * hh;
#pragma unroll
        for (int st = 0; st < 16; ++st)
          Sx[u] = mfma32(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr + 32 * st)), Qf[st], Sx[u]);
#pragma unroll
        for (int v = 0; v < 16; ++v)
          Sx[u][v] = kb * KB + 32 * u + key_of_row(acc_row(v, hh)) > qi ? -INFINITY : Sx[u][v] * sl2;
      }
    };
    float m2 = -INFINITY;
    for (int kb = 0; kb < nkb; ++kb) {
      floatx16 Sx[2];
      scores(kb, Sx);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 16; ++v) m2 = fmaxf(m2, Sx[u][v]);
    }
    m = fmaxf(m2, __shfl_xor(m2, 32, 64));
    l = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[t][v] = 0.f;
    for (int kb = 0; kb < nkb; ++kb) {
      floatx16 Sx[2];
      scores(kb, Sx);
      bf16x8 P[4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(Sx[u][8 * s2 + e] - m);
            l += p;
            P[2 * u + s2][e] = static_cast<__bf16>(p);
          }
      const uint16_t* vb = a.vc + vc_block(a, b, j, kb * KB) + l32 * KB + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          O[t] = mfma32(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(vb + 32 * t * KB + 16 * ks)),
                        P[ks], O[t]);
    }
  }
  // epilogue: normalise, gate, store (rows past T are not stored)
  l += __shfl_xor(l, 32, 64);
  if (qi >= a.T) return;
  const float inv = 1.0f / l;
  const uint16_t* gate = a.qg + tok * a.sqg + static_cast<int64_t>(h) * 2 * AD + AD;
  uint16_t* orow = a.o + tok * a.so + static_cast<int64_t>(h) * AD;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * t + 8 * q4 + 4 * hh;
      const u16x4 g = *reinterpret_cast<const u16x4*>(gate + d);
      u16x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = f32_to_bf16_bits(O[t][4 * q4 + i] * inv * sigmoidf_(bf16_bits_to_f32(g[i])));
      *reinterpret_cast<u16x4*>(orow + d) = out;
    }
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------
// One wave per (256 cached positions, key/value head, sequence), on 16x16x32
// bf16 MFMA: the group's query heads are the 16 columns of the B operand (the
// columns past the group are zero).  Keys and values stream through the wave's
// own 32 KiB of LDS, 32 positions at a time, copied with whole-row 16-byte
// direct loads (1 KiB per instruction); five such waves share a CU, so one
// wave's copies overlap the others' products.  A 16x16 accumulator gives lane l
// column l % 16 and rows 4 (l / 16) .. + 3; the key rows of the two score tiles
// are ordered so that these eight values of a lane are eight consecutive
// positions, which are then the k slots of the weight operand and one 16-byte
// read of the transposed values.  Online softmax over the blocks; the partial
// maximum, sum and unnormalised output of each query head go to the workspace.
__device__ __forceinline__ floatx4 mfma16(const bf16x8& a, const bf16x8& b, const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int DB = 32;                       // positions per decode block
constexpr int kDecLds = DB * AD * 2 * 3;     // keys 16 KiB + transposed values of two blocks 32 KiB

__global__ __launch_bounds__(64, 2) void attn_decode_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* sk = smem;                  // 32 rows of 512 B: row 16 kt + r holds score tile kt's row r
  unsigned char* sv = smem + DB * AD * 2;    // 256 rows (dims) of 64 B (32 positions)
  const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int n = min(max(a.cache_len[b], 0), a.S_max - 1) + 1;   // positions [0, n)
  const int k0 = sp * a.split;
  if (k0 >= n) return;   // the combine reads ceil(n / 256) splits only
  const int lane = threadIdx.x, c16 = lane & 15, g4 = lane >> 4;
  // queries: k step s = dims 32s.., lane group g4 holds 8 consecutive dims
  bf16x8 Qf[8];
  {
    const uint16_t* qr = a.qrot + (static_cast<int64_t>(b) * a.Hq + j * G + min(c16, G - 1)) * AD + 8 * g4;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u16x8 x = *reinterpret_cast<const u16x8*>(qr + 32 * s);
      if (c16 >= G) x = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      Qf[s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  floatx4 O[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) O[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * kLog2e;
  const unsigned char* kcb = reinterpret_cast<const unsigned char*>(a.kc + kc_index(a, b, j, 0));
  const int nblk = min(a.split / DB, (n - k0 + DB - 1) / DB);
  for (int blk = 0; blk < nblk; ++blk) {
    const int kb0 = k0 + DB * blk;           // kb0 + 31 < S_max: S_max is a multiple of 64
    const int valid = min(DB, n - kb0);
    // Copy.  Key row r = 16 kt + m of LDS holds position 8 (m / 4) + 4 kt + m % 4, its
    // 16-byte chunk c at chunk position c ^ (r & 15); value row d (64 B) holds
    // positions kb0.. kb0+31 of dim d, chunk c at c ^ ((d / 4) & 3).  The values of a
    // block and the next are copied together at the even block, both halves of each
    // 128-byte cache row back to back: copied a block at a time, the second half was
    // gone from L2 when the next block asked for it, and the values crossed from memory
    // nearly twice (1,542 MB fetched per call against 1,074 MB of cache).  (Copying the
    // next block's keys and values while this one is worked on timed the same.)
    __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): the previous block's LDS reads are done
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = 2 * q + (lane >> 5), cp = lane & 31;
      const int kt = r >> 4, mm = r & 15;
      const int pos = kb0 + 8 * (mm >> 2) + 4 * kt + (mm & 3);
      __builtin_amdgcn_global_load_lds(kcb + static_cast<int64_t>(pos) * (AD * 2) + 16 * (cp ^ (r & 15)),
                                       sk + 1024 * q, 16, 0, 0);
    }
    if ((blk & 1) == 0) {
      // values of this block and the next together: whole 128-byte rows of the value block
      const unsigned char* vsrc = reinterpret_cast<const unsigned char*>(a.vc + vc_block(a, b, j, kb0));
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int d = 16 * q + (lane >> 2), cp = lane & 3;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          __builtin_amdgcn_global_load_lds(vsrc + 64 * hh + d * (KB * 2) + 16 * (cp ^ ((d >> 2) & 3)),
                                           sv + 16384 * hh + 1024 * q, 16, 0, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);      // vmcnt(0): the block is in LDS
    floatx4 S[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const unsigned char* kr = sk + (16 * kt + c16) * (AD * 2);
      S[kt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s)
        S[kt] = mfma16(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr + 16 * ((4 * s + g4) ^ c16))),
                       Qf[s], S[kt]);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = 8 * g4 + 4 * kt + i < valid ? S[kt][i] * sl2 : -INFINITY;   // row 4 g4 + i of tile kt
        S[kt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);           // finite: position kb0 is valid
    const float c = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    l *= c;
#pragma unroll
    for (int t = 0; t < 16; ++t) O[t] *= c;
    // weights: lane group g4 holds positions 8 g4 + 0..7 (tile 0 rows, then tile 1 rows)
    bf16x8 P;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __builtin_amdgcn_exp2f(S[e >> 2][e & 3] - mn);
      l += p;
      P[e] = static_cast<__bf16>(p);
    }
    // values: rows = dims 16 dt + c16; positions past n may hold arbitrary bits
    // (a NaN would survive a zero weight), so they are zeroed
#pragma unroll
    for (int dt = 0; dt < 16; ++dt) {
      const int d = 16 * dt + c16;
      u16x8 vv = *reinterpret_cast<const u16x8*>(sv + 16384 * (blk & 1) + d * (DB * 2) + 16 * (g4 ^ ((d >> 2) & 3)));
      if (valid < DB) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (8 * g4 + e >= valid) vv[e] = 0;
      }
      O[dt] = mfma16(__builtin_bit_cast(bf16x8, vv), P, O[dt]);
    }
  }
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (c16 >= G) return;
  float* part = a.part + ((static_cast<int64_t>(b) * a.Hq + j * G + c16) * attn_splits(a.S_max) + sp) *
                             kAttnPartFloats;
  if (g4 == 0) {
    part[0] = m;
    part[1] = l;
  }
#pragma unroll
  for (int dt = 0; dt < 16; ++dt) *reinterpret_cast<floatx4*>(part + 4 + 16 * dt + 4 * g4) = O[dt];
}

// Merges the partial results of a query head: M = max m_s, L = sum 2^(m_s - M) l_s,
// o = sum 2^(m_s - M) o_s / L, then the gate.  One thread per dimension.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  __shared__ float wsp[256];
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int n = min(max(a.cache_len[b], 0), a.S_max - 1) + 1;
  const int nsp = (n + a.split - 1) / a.split;
  const float* part = a.part + (static_cast<int64_t>(b) * a.Hq + h) * attn_splits(a.S_max) * kAttnPartFloats;
  float mloc = -INFINITY;
  for (int sp = d; sp < nsp; sp += 256) mloc = fmaxf(mloc, part[sp * kAttnPartFloats]);
#pragma unroll
  for (int mm = 32; mm >= 1; mm >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, mm, 64));
  if ((d & 63) == 0) red[d >> 6] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float Lloc = 0.f, o = 0.f;
  for (int base = 0; base < nsp; base += 256) {
    __syncthreads();   // red and wsp are rewritten
    const int sp = base + d;
    if (sp < nsp) {
      const float wgt = exp2f(part[sp * kAttnPartFloats] - M);
      wsp[d] = wgt;
      Lloc += wgt * part[sp * kAttnPartFloats + 1];
    }
    __syncthreads();
    const int cnt = min(256, nsp - base);
    const float* pp = part + static_cast<int64_t>(base) * kAttnPartFloats + 4 + d;
#pragma unroll 8
    for (int i = 0; i < cnt; ++i) o += wsp[i] * pp[i * kAttnPartFloats];
  }
  Lloc = wave_sum(Lloc);
  __syncthreads();
  if ((d & 63) == 0) red[d >> 6] = Lloc;
  __syncthreads();
  const float L = red[0] + red[1] + red[2] + red[3];
  const int64_t tok = b;   // T == 1
  const float g = bf16_bits_to_f32(a.qg[tok * a.sqg + static_cast<int64_t>(h) * 2 * AD + AD + d]);
  a.o[tok * a.so + static_cast<int64_t>(h) * AD + d] = f32_to_bf16_bits(o / L * sigmoidf_(g));
}

// Prefill: the values of 64 positions of one key/value head go into their
// transposed cache block through LDS.  Positions past T are written as zeros,
// values and keys, so that the attention kernel can read whole blocks.
__global__ __launch_bounds__(256) void attn_vblock_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sv[KB][AD + 8];
  const int blk = blockIdx.x, j = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int p0 = blk * KB;
  const u16x8 zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;   // position c / 32, dims 8 (c % 32)..
    const int p = c / 32, d = 8 * (c % 32);
    u16x8 x = zero;
    if (p0 + p < a.T) {
      // two 8-byte loads: v rows are 8-byte aligned (strides are multiples of 4)
      const uint16_t* src = a.v + (static_cast<int64_t>(b) * a.T + p0 + p) * a.sv + static_cast<int64_t>(j) * AD + d;
      const u16x4 lo = *reinterpret_cast<const u16x4*>(src), hi = *reinterpret_cast<const u16x4*>(src + 4);
      x = u16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else
      *reinterpret_cast<u16x8*>(a.kc + kc_index(a, b, j, p0 + p) + d) = zero;
    *reinterpret_cast<u16x8*>(&sv[p][d]) = x;
  }
  __syncthreads();
  uint16_t* dst = a.vc + vc_block(a, b, j, p0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;   // dim c / 8, positions 8 (c % 8)..
    const int d = c / 8, p = 8 * (c % 8);
    u16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = sv[p + e][d];
    *reinterpret_cast<u16x8*>(dst + d * KB + p) = y;
  }
}

hipError_t launch_prep(const AttnArgs& a, hipStream_t s) {
  const int64_t ntok = static_cast<int64_t>(a.B) * a.T;
  if (ntok == 0) return hipSuccess;
  RopeTable rt{};
  for (int f = 0; f < a.rot_dim / 2; ++f) rt.inv_freq[f] = std::pow(static_cast<double>(a.theta), -2.0 * f / a.rot_dim);
  hipLaunchKernelGGL(attn_prep_kernel, dim3(static_cast<unsigned>(ntok)), dim3(256), 0, s, a, rt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s) {
  static PerDeviceOnce attrs;
  hipError_t ea = attrs.run([] {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, kFwdLds);
  });
  if (ea != hipSuccess) return ea;
  if (a.B == 0 || a.T == 0) return hipSuccess;
  hipError_t e = launch_prep(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_vblock_kernel, dim3((a.T + KB - 1) / KB, a.Hkv, a.B), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((a.T + QB - 1) / QB * a.Hq * a.B), dim3(256), kFwdLds, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipError_t e = launch_prep(a, s);
  if (e != hipSuccess) return e;
  // 512 positions per wave when 256 would give more than four rounds of the three waves a CU
  // holds (64 sequences x 4 heads x 4096 positions: 215 against 225 us per call); 256 otherwise,
  // so that small batches keep their parallelism
  AttnArgs r = a;
  const int64_t waves = static_cast<int64_t>(attn_splits(a.S_max)) * a.Hkv * a.B;
  r.split = waves > 4 * 3 * static_cast<int64_t>(device_cu_count()) ? 2 * kAttnSplit : kAttnSplit;
  hipLaunchKernelGGL(attn_decode_kernel, dim3((a.S_max + r.split - 1) / r.split, a.Hkv, a.B), dim3(64), kDecLds, s,
                     r);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.Hq, a.B), dim3(256), 0, s, r);
  return hipGetLastError();
}

}  // namespace gdn
