// gdn_device.h -- small device helpers for the gfx950 kernels: bf16 <-> fp32,
// typed loads, wave reductions and the MFMA operand vector types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}

template <typename IO>
struct IoTraits;

template <>
struct IoTraits<float> {
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
    static_cast<float*>(p)[i] = x;
  }
};

template <>
struct IoTraits<uint16_t> {  // bf16 bit patterns
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, int64_t i, float x) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(x);
  }
};

// Sum over the 64 lanes of a wave (result in every lane).
// Token range of sequence s of a packed batch: [cu[s], cu[s+1]), clamped into
// [0, T] and to a non-negative length, so that a malformed offset table can
// give wrong results but never send a kernel outside the token arrays.
__device__ __forceinline__ void packed_range(const int32_t* cu, int s, int T, int64_t& start, int& len) {
  const int lo = min(max(cu[s], 0), T);
  const int hi = min(max(cu[s + 1], lo), T);
  start = lo;
  len = hi - lo;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// Sum of x over each row of 16 lanes, in every lane of the row: pairs within quads,
// then quads (lane i with 7 - i of each half row), then half rows (i with 15 - i).
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// Gate activation of one value head from its raw in_proj_ba outputs b (beta
// logit) and a (alpha input): beta = sigmoid(b), log alpha = -exp(A_log) *
// softplus(a + dt_bias) ("Les briques d'un reseau de neurones", section 2
// table: sigmoid and softplus(x) = log(1 + e^x); the alpha recipe of the layer
// inputs).  softplus is evaluated as max(x, 0) + log1p(e^-|x|) and sigmoid
// from e^-|x|, so neither overflows.
__device__ __forceinline__ void gate_activation(float b, float a, float A_log, float dt_bias, float& log_alpha,
                                                float& beta) {
  const float eb = __expf(-fabsf(b));
  beta = b >= 0.f ? 1.0f / (1.0f + eb) : eb / (1.0f + eb);
  const float x = a + dt_bias;
  log_alpha = -__expf(A_log) * (fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))));
}

}  // namespace gdn
