// gdn_attn.hip -- the full-attention layer of the hybrid stack ("L'attention
// hybride", section "Les 16 couches d'attention complete"): per-head RMSNorm
// and partial RoPE of q and k, causal grouped-query attention with head width
// 256, and the sigmoid output gate that the doubled query projection carries
// ("Le facteur 2 sur W_Q", "GQA a 6:1", "Le RoPE partiel").
//
// Kernels:
//  * attn_prep_kernel: one wave per 256-wide row of a token.  Query rows are
//    normalised and rotated into the qrot scratch; key rows likewise into the
//    key cache at the token's position; value rows are copied into the value
//    cache, whose 64-position blocks are stored transposed ([256][64]) so that
//    the products read them as MFMA operands with keys along k.
//  * attn_fwd_kernel (prefill): 4 waves x 32 query rows of one query head.
//    Per block of 64 keys: S^T = K Q^T on 32x32x16 bf16 MFMA (keys on the MFMA
//    rows, queries on its columns, so each lane holds one query's scores and
//    the softmax statistics are per lane plus one exchange across the two lane
//    halves), the online softmax in base 2, then O^T += V^T P^T, whose
//    B operand is the score accumulator itself rounded to bf16 (the key order
//    of the accumulator rows is the k order of the operand).  Key and value
//    blocks are staged through LDS, double-buffered, with the next block's
//    loads in flight during the products.
//  * attn_decode_kernel: one workgroup per (256 cached positions, key/value
//    head, sequence) scores the group's query heads (one position per thread,
//    fp32), and accumulates the softmax-weighted values (one dimension per
//    thread); attn_combine_kernel merges the partial maxima, sums and outputs
//    of a head and applies the gate.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int AD = 256;      // head width
constexpr int QB = 128;      // query rows per prefill workgroup (4 waves x 32)
constexpr int KB = 64;       // keys per block
constexpr int KPITCH = 264;  // LDS row pitch (bf16) of a key block [64][256]
constexpr int VPITCH = 72;   // LDS row pitch (bf16) of a transposed value block [256][64]
constexpr int KBUF = KB * KPITCH * 2;
constexpr int VBUF = AD * VPITCH * 2;
constexpr int kFwdLds = 2 * (KBUF + VBUF);
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ floatx16 mfma32(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// row of value v of a 32x32 accumulator in lane half h
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

__device__ __forceinline__ int64_t kc_index(const AttnArgs& a, int b, int j, int pos) {
  return ((static_cast<int64_t>(b) * a.Hkv + j) * a.S_max + pos) * AD;
}
// first element of the transposed value block holding position pos
__device__ __forceinline__ int64_t vc_block(const AttnArgs& a, int b, int j, int pos) {
  return ((static_cast<int64_t>(b) * a.Hkv + j) * (a.S_max / KB) + pos / KB) * KB * AD;
}

// ---------------------------------------------------------------------------
// prep: rows are, per token, Hq query rows, Hkv key rows, Hkv value rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_prep_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int R = a.Hq + 2 * a.Hkv;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<int64_t>(a.B) * a.T * R) return;
  const int64_t tok = row / R;
  const int r = static_cast<int>(row - tok * R);
  const int b = static_cast<int>(tok / a.T), t = static_cast<int>(tok - static_cast<int64_t>(b) * a.T);
  const int pos = a.cache_len ? min(max(a.cache_len[b], 0), a.S_max - 1) : t;
  const int d0 = 4 * lane;
  if (r >= a.Hq + a.Hkv) {
    const int j = r - a.Hq - a.Hkv;
    const u16x4 x = *reinterpret_cast<const u16x4*>(a.v + tok * a.sv + static_cast<int64_t>(j) * AD + d0);
    uint16_t* dst = a.vc + vc_block(a, b, j, pos) + pos % KB;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(d0 + i) * KB] = x[i];
    return;
  }
  const bool isq = r < a.Hq;
  const uint16_t* src = isq ? a.qg + tok * a.sqg + static_cast<int64_t>(r) * 2 * AD
                            : a.k + tok * a.sk + static_cast<int64_t>(r - a.Hq) * AD;
  const uint16_t* w = isq ? a.qw : a.kw;
  const u16x4 x4 = *reinterpret_cast<const u16x4*>(src + d0);
  const u16x4 w4 = *reinterpret_cast<const u16x4*>(w + d0);
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
  // RoPE: dimension i < half pairs with i + half; half is a multiple of 4, so a
  // lane's partner lane is half/4 away
  const int half = a.rot_dim / 2, lo = half / 4;
  const int pl = lane < lo ? lane + lo : lane - lo;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __shfl(y[i], pl, 64);
  if (d0 < a.rot_dim) {
    const bool first = d0 < half;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int f = (first ? d0 : d0 - half) + i;
      // the angle in fp64: positions reach 10^5 and more, where fp32 would lose ~1e-2 rad
      const double ang = static_cast<double>(pos) * pow(static_cast<double>(a.theta), -2.0 * f / a.rot_dim);
      double sn, cs;
      sincos(ang, &sn, &cs);
      const float c = static_cast<float>(cs), s = static_cast<float>(sn);
      y[i] = first ? y[i] * c - p[i] * s : y[i] * c + p[i] * s;
    }
  }
  u16x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = f32_to_bf16_bits(y[i]);
  uint16_t* dst = isq ? a.qrot + (tok * a.Hq + r) * AD : a.kc + kc_index(a, b, r - a.Hq, pos);
  *reinterpret_cast<u16x4*>(dst + d0) = out;
}

// ---------------------------------------------------------------------------
// prefill attention
// ---------------------------------------------------------------------------
// 16-byte chunk i (of 2048) of key block kb and of value block kb, into registers
struct BlockRegs {
  u16x8 k[8], v[8];
};

__device__ __forceinline__ void load_block(const AttnArgs& a, int b, int j, int kb, int tid, BlockRegs& r) {
  const uint16_t* ks = a.kc + kc_index(a, b, j, kb * KB);
  const uint16_t* vs = a.vc + vc_block(a, b, j, kb * KB);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    r.k[i] = *reinterpret_cast<const u16x8*>(ks + 8 * c);   // key row c/32, dims 8 (c%32)..
    r.v[i] = *reinterpret_cast<const u16x8*>(vs + 8 * c);   // dim row c/8, keys 8 (c%8)..
  }
}

// Keys at or beyond `valid` in the block are zeroed: cache positions past the
// written ones hold arbitrary bits, and a NaN there would survive a zero weight.
__device__ __forceinline__ void store_block(unsigned char* kbuf, unsigned char* vbuf, int tid, BlockRegs& r,
                                            int valid) {
  uint16_t* sk = reinterpret_cast<uint16_t*>(kbuf);
  uint16_t* sv = reinterpret_cast<uint16_t*>(vbuf);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + 256 * i;
    u16x8 kk = r.k[i], vv = r.v[i];
    if (valid < KB) {
      if (c / 32 >= valid) kk = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (8 * (c % 8) + e >= valid) vv[e] = 0;
    }
    *reinterpret_cast<u16x8*>(sk + (c / 32) * KPITCH + 8 * (c % 32)) = kk;
    *reinterpret_cast<u16x8*>(sv + (c / 8) * VPITCH + 8 * (c % 8)) = vv;
  }
}

__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int nqb = (a.T + QB - 1) / QB;
  const int qb = nqb - 1 - static_cast<int>(blockIdx.x);  // the longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int j = h / (a.Hq / a.Hkv);
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
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * kLog2e;

  const int last_key = min(qb * QB + QB, a.T) - 1;   // the largest key any row here sees
  const int nkb = last_key / KB + 1;
  BlockRegs br;
  load_block(a, b, j, 0, tid, br);
  store_block(smem, smem + 2 * KBUF, tid, br, min(KB, a.T));
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const uint16_t* sk = reinterpret_cast<const uint16_t*>(smem + cur * KBUF);
    const uint16_t* sv = reinterpret_cast<const uint16_t*>(smem + 2 * KBUF + cur * VBUF);
    if (kb + 1 < nkb) load_block(a, b, j, kb + 1, tid, br);

    // S^T tiles u = keys 32u.. of the block
    floatx16 S[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int v = 0; v < 16; ++v) S[u][v] = 0.f;
      const uint16_t* kr = sk + (32 * u + l32) * KPITCH + 8 * hh;
#pragma unroll
      for (int s = 0; s < 16; ++s)
        S[u] = mfma32(__builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(kr + 16 * s)), Qf[s], S[u]);
    }
    // scale to base 2, mask keys after the query, block maximum
    const int kbase = kb * KB;
    const bool diag = kbase + KB - 1 > q0;
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = S[u][v] * sl2;
        if (diag && kbase + 32 * u + acc_row(v, hh) > qi) x = -INFINITY;
        S[u][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);        // finite: key 0 precedes every query
    const float c = exp2f(m - mn);
    m = mn;
    l *= c;
    if (__builtin_amdgcn_ballot_w64(c != 1.0f)) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) O[t][v] *= c;
    }
    // P^T fragments: accumulator values 8s2..8s2+7 of tile u are keys
    // 32u + 16 s2 + {4hh..4hh+3, 8+4hh..8+4hh+3}
    bf16x8 P[4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = exp2f(S[u][8 * s2 + e] - mn);
          l += p;
          P[2 * u + s2][e] = static_cast<__bf16>(p);
        }
    // O^T += V^T P^T: A operand rows = dims 32t + l32, k = the same key order
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint16_t* vr = sv + l32 * VPITCH + 16 * ks + 4 * hh;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const uint16_t* vt = vr + 32 * t * VPITCH;
        const u16x4 lo = *reinterpret_cast<const u16x4*>(vt);
        const u16x4 hi = *reinterpret_cast<const u16x4*>(vt + 8);
        const u16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        O[t] = mfma32(__builtin_bit_cast(bf16x8, vv), P[ks], O[t]);
      }
    }
    if (kb + 1 < nkb) {
      const int nxt = cur ^ 1;
      store_block(smem + nxt * KBUF, smem + 2 * KBUF + nxt * VBUF, tid, br, min(KB, a.T - (kb + 1) * KB));
    }
    __syncthreads();
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
constexpr int kMaxGroup = 8;

__device__ __forceinline__ float block_max(float x, float* red) {
#pragma unroll
  for (int mm = 32; mm >= 1; mm >>= 1) x = fmaxf(x, __shfl_xor(x, mm, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return x;
}
__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return x;
}

__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a) {
  __shared__ float qs[kMaxGroup][AD];
  __shared__ float ps[kMaxGroup][kAttnSplit];
  __shared__ float red[4];
  const int sp = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int n = min(max(a.cache_len[b], 0), a.S_max - 1) + 1;   // positions [0, n)
  const int k0 = sp * kAttnSplit;
  if (k0 >= n) return;   // the combine reads ceil(n / 256) splits only
  const int tid = threadIdx.x;
  for (int i = tid; i < G * AD; i += 256)
    qs[i / AD][i % AD] = bf16_bits_to_f32(a.qrot[(static_cast<int64_t>(b) * a.Hq + j * G + i / AD) * AD + i % AD]);
  __syncthreads();
  // scores: one position per thread
  const int key = k0 + tid;
  float s[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) s[g] = 0.f;
  if (key < n) {
    const uint16_t* kr = a.kc + kc_index(a, b, j, key);
    for (int c = 0; c < AD / 8; ++c) {
      const u16x8 kv = *reinterpret_cast<const u16x8*>(kr + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kf = bf16_bits_to_f32(kv[e]);
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g)
          if (g < G) s[g] += kf * qs[g][8 * c + e];
      }
    }
  }
  const float sl2 = a.scale * kLog2e;
  float* part = a.part + ((static_cast<int64_t>(b) * a.Hq + j * G) * attn_splits(a.S_max) + sp) * kAttnPartFloats;
  const int64_t gstride = static_cast<int64_t>(attn_splits(a.S_max)) * kAttnPartFloats;
  for (int g = 0; g < G; ++g) {
    const float x = key < n ? s[g] * sl2 : -INFINITY;
    const float mg = block_max(x, red);
    const float p = key < n ? exp2f(x - mg) : 0.f;
    ps[g][tid] = p;
    const float lg = block_sum(p, red);
    if (tid == 0) {
      part[g * gstride + 0] = mg;
      part[g * gstride + 1] = lg;
    }
  }
  __syncthreads();
  // weighted values: one dimension per thread; positions past n are skipped
  float o[kMaxGroup];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) o[g] = 0.f;
  const int d = tid;
  for (int blk = 0; blk < kAttnSplit / KB && k0 + KB * blk < n; ++blk) {
    const uint16_t* vr = a.vc + vc_block(a, b, j, k0 + KB * blk) + d * KB;
    const int valid = min(KB, n - k0 - KB * blk);
    for (int c = 0; c < KB / 8; ++c) {
      const u16x8 vv = *reinterpret_cast<const u16x8*>(vr + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = 8 * c + e;
        const float vf = kk < valid ? bf16_bits_to_f32(vv[e]) : 0.f;
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g)
          if (g < G) o[g] += ps[g][KB * blk + kk] * vf;
      }
    }
  }
  for (int g = 0; g < G; ++g) part[g * gstride + 4 + d] = o[g];
}

__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int n = min(max(a.cache_len[b], 0), a.S_max - 1) + 1;
  const int nsp = (n + kAttnSplit - 1) / kAttnSplit;
  const float* part = a.part + (static_cast<int64_t>(b) * a.Hq + h) * attn_splits(a.S_max) * kAttnPartFloats;
  float M = -INFINITY;
  for (int sp = 0; sp < nsp; ++sp) M = fmaxf(M, part[sp * kAttnPartFloats]);
  float L = 0.f, o = 0.f;
  for (int sp = 0; sp < nsp; ++sp) {
    const float* pp = part + sp * kAttnPartFloats;
    const float c = exp2f(pp[0] - M);
    L += c * pp[1];
    o += c * pp[4 + d];
  }
  const int64_t tok = b;   // T == 1
  const float g = bf16_bits_to_f32(a.qg[tok * a.sqg + static_cast<int64_t>(h) * 2 * AD + AD + d]);
  a.o[tok * a.so + static_cast<int64_t>(h) * AD + d] = f32_to_bf16_bits(o / L * sigmoidf_(g));
}

hipError_t launch_prep(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.B) * a.T * (a.Hq + 2 * a.Hkv);
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_prep_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kFwdLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (a.B == 0 || a.T == 0) return hipSuccess;
  hipError_t e = launch_prep(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((a.T + QB - 1) / QB, a.Hq, a.B), dim3(256), kFwdLds, s, a);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipError_t e = launch_prep(a, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_decode_kernel, dim3(attn_splits(a.S_max), a.Hkv, a.B), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(a.Hq, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gdn
