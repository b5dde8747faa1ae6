// gdn_probe.hip -- measurement probes (gfx950): what this GPU attains on plain
// matrix-core work and on a plain device-memory stream, so that the library's
// kernels can be set beside an attainable figure as well as the datasheet's.
// Neither takes part in the Gated DeltaNet computation.
//
// mfma_probe_kernel: each wave runs `iters` rounds of four independent
// 32x32x16 bf16 MFMAs on register operands (every operand element 1.0, so each
// accumulator element gains 16 per product and the result is known exactly);
// four chains keep the matrix core of the wave's SIMD issuing back to back.
// (The 32x32 form reached 2.48 PFLOP/s with 2048 workgroups where eight chains
// of 16x16x32 MFMAs stayed near 2.1-2.2.)
// copy_probe_kernel: 16-byte loads, eight per thread issued before the first
// store, 32 KiB per workgroup of 256 threads.
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  // bf16 1.0 is 0x3F80; built from the thread index so that the operands are not constants
  const uint16_t one = static_cast<uint16_t>(0x3F80u | (threadIdx.x >> 16));
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = __builtin_bit_cast(__bf16, one);
  floatx16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  // four rounds per trip (iters is a multiple of 4): 16 MFMAs in the loop body
  for (int i = 0; i < iters; i += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 2048 + threadIdx.x;
  u32x4 v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = src[i + 256 * j];
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[i + 256 * j] = v[j];
}

}  // namespace

hipError_t launch_probe_mfma(int n_workgroups, int iters, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(static_cast<unsigned>(n_workgroups)), dim3(256), 0, s, iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t blocks = bytes / kProbeCopyBlockBytes;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_probe_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst));
  return hipGetLastError();
}

}  // namespace gdn
