// Peak probes: a dense bf16 MFMA loop and a streaming device-memory read
// (declared in ssa_probes.h).  Neither depends on the method's kernels.
#include "ssa_common.hpp"
#include "ssa_probes.h"

using ssa::bf16x8;
using ssa::floatx16;

namespace {

constexpr int kChains = 4;    // independent accumulators per wave
constexpr int kPerIter = 16;  // MFMAs per loop iteration

__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x % 64;
  // operands that depend on the lane (never all zero), fixed over the loop
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * float((lane + e) % 7 + 1));
    b[e] = static_cast<__bf16>(0.002f * float((lane * 3 + e) % 5 + 1));
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < kPerIter; ++j) acc[j % kChains] = ssa::mma16(a, b, acc[j % kChains]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ buf, size_t n16,
                                                         uint32_t* __restrict__ out) {
  const size_t stride = size_t(gridDim.x) * 256;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = buf[i], v1 = buf[i + stride], v2 = buf[i + 2 * stride], v3 = buf[i + 3 * stride];
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = buf[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[size_t(blockIdx.x) * 256 + threadIdx.x] = acc;
}

ssa_status launch_status(hipError_t e) { return e == hipSuccess ? SSA_OK : SSA_ERR_HIP; }

}  // namespace

extern "C" ssa_status ssa_probe_mfma_bf16(float* out, int32_t workgroups, int32_t iters,
                                          double* flops, void* stream) {
  if (out == nullptr || flops == nullptr || workgroups <= 0 || iters <= 0)
    return SSA_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(unsigned(workgroups)), dim3(256), 0,
                     (hipStream_t)stream, out, int(iters));
  *flops = double(workgroups) * 4.0 * double(iters) * kPerIter * (2.0 * 32 * 32 * 16);
  return launch_status(hipGetLastError());
}

extern "C" ssa_status ssa_probe_hbm_read(const void* buf, size_t bytes, uint32_t* out,
                                         int32_t workgroups, void* stream) {
  if (buf == nullptr || out == nullptr || workgroups <= 0 || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return SSA_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(probe_read_kernel, dim3(unsigned(workgroups)), dim3(256), 0,
                     (hipStream_t)stream, static_cast<const uint4*>(buf), bytes / 16, out);
  return launch_status(hipGetLastError());
}
