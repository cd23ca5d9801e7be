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

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Grid-stride streaming read, eight 16-byte nontemporal loads in flight per
// thread (of the layouts tried on MI355X -- four or eight loads, cached or
// nontemporal, grid-stride or one contiguous span per workgroup -- this one
// read fastest).
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4v* __restrict__ buf, size_t n16,
                                                         uint32_t* __restrict__ out) {
  constexpr int U = 8;
  const size_t stride = size_t(gridDim.x) * 256;
  size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4v v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4v v = buf[i];
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
                     (hipStream_t)stream, static_cast<const u32x4v*>(buf), bytes / 16, out);
  return launch_status(hipGetLastError());
}
