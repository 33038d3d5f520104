// Measured ceilings for the roofline denominators: a dense bf16 MFMA loop
// (which also reports the shader clock it ran at) and a streaming HBM read.
// They are diagnostics beside the three attention calls: the benchmark runs
// them in the same job as the kernels, so each kernel's fraction of the
// published MI355X peaks (2.5 PFLOP/s dense bf16, 8 TB/s) also has a
// fraction of what this GPU sustains in that run.
#include "inkattn.h"

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace {

using inkattn::bf16;
using inkattn::f32x16;
using inkattn::Frag8;
using inkattn::mfma32;
using inkattn::u32x4;

constexpr int kMfmaWaves = INKATTN_PROBE_MFMA_WAVES;
constexpr int kMfmaChains = INKATTN_PROBE_MFMA_CHAINS;
constexpr int kReadGroups = INKATTN_PROBE_READ_GROUPS;
constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
  return x;
}

// bf16 pairs in +-[1, 2) with random mantissas: operands that toggle like
// real data (all-zero operands draw less power and overstate the ceiling).
__device__ __forceinline__ uint32_t operand_bits(uint32_t seed) {
  const uint32_t r = mix(seed);
  return (r & 0x807F807FU) | 0x3F803F80U;
}

// 8 waves (two per SIMD) of kMfmaChains independent 32x32x16 bf16 MFMA
// accumulator chains.  Wave 0 stamps the shader clock and the 100 MHz
// real-time counter around its loop.
__global__ __launch_bounds__(64 * kMfmaWaves) void probe_mfma_kernel(int iters, float* out) {
  const uint32_t t = blockIdx.x * (64 * kMfmaWaves) + threadIdx.x;
  Frag8<bf16> a, b;
  a.v = u32x4{operand_bits(4 * t), operand_bits(4 * t + 1), operand_bits(4 * t + 2),
              operand_bits(4 * t + 3)};
  b.v = u32x4{operand_bits(4 * t + 7), operand_bits(4 * t + 11), operand_bits(4 * t + 13),
              operand_bits(4 * t + 17)};
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  __builtin_amdgcn_sched_barrier(0);
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  __builtin_amdgcn_sched_barrier(0);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if (threadIdx.x == 0) {
    out[3 * blockIdx.x + 0] = s;
    out[3 * blockIdx.x + 1] = (float)(c1 - c0);
    out[3 * blockIdx.x + 2] = (float)(r1 - r0);
  }
}

// Grid-stride read of n16 16-byte words, kReadUnroll loads in flight per
// thread, one work-group per CU (the fastest of the grid shapes measured on
// MI355X).  The XOR of everything read is written only if it matches a
// constant, which the compiler cannot rule out, so no load is dropped.
__global__ __launch_bounds__(kReadThreads) void probe_read_kernel(const u32x4* p, size_t n16,
                                                                  float* out) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = p[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (x == 0x9E3779B9U) out[blockIdx.x] = (float)x;
}

}  // namespace

extern "C" {

inkattn_status_t inkattn_probe_mfma_bf16(int32_t num_groups, int32_t iters, float* out,
                                         void* stream) {
  if (num_groups < 1 || iters < 1 || !out) return INKATTN_EINVAL;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3((unsigned)num_groups), dim3(64 * kMfmaWaves), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return hipGetLastError() == hipSuccess ? INKATTN_OK : INKATTN_EHIP;
}

inkattn_status_t inkattn_probe_stream_read(const void* buf, size_t bytes, float* out,
                                           void* stream) {
  if (!buf || !out || bytes == 0) return INKATTN_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || bytes % 16 != 0) return INKATTN_EINVAL;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kReadGroups), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     bytes / 16, out);
  return hipGetLastError() == hipSuccess ? INKATTN_OK : INKATTN_EHIP;
}

}  // extern "C"
