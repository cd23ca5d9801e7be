// Per-block key statistics: mean mu_c and population covariance Sigma_c.
//
// Write-up "Subquadratic Sparse Attention (SSA)", section "The idea in one
// screen": the router reads only per-block summaries, the block mean and the
// covariance whose quadratic form q^T Sigma_c q is the variance of the logit
// q.k across the block.  Computed as a centred two-pass in float32: pass 1
// sums the block's keys per column; pass 2 accumulates (k - mu)(k - mu)^T
// over 64-key chunks staged in LDS, each thread owning a (d/16) x (d/16) tile
// of Sigma.  The kernel reads B*d input elements twice (the second time from
// L2) and writes d + d*d floats: it is bound by HBM/L2, well under 1% of a
// prefill's time, so it stays on the vector ALUs.
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 64;

template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void block_stats_kernel(
    const TIn* __restrict__ K, float* __restrict__ mu, float* __restrict__ sigma, int64_t n,
    int B, int64_t n_slots, int hkv, const int32_t* __restrict__ cache_len) {
  constexpr int G = kThreads / D;        // key groups in pass 1
  constexpr int TS = D / 16;             // Sigma tile per thread: TS x TS
  __shared__ float red[kThreads];
  __shared__ float smu[D];
  __shared__ float X[kChunk][D + 4];

  const int tid = threadIdx.x;
  const int64_t bkv = blockIdx.y;
  int64_t c;
  if (cache_len != nullptr) {
    const int64_t L = cache_len[bkv / hkv];   // the new key sits at position L
    if (L < 0 || (L + 1) % B != 0) return;
    c = (L + 1) / B - 1;
    if (c >= n_slots) return;                 // cache_len beyond capacity: write nothing
  } else {
    c = blockIdx.x;
  }
  const TIn* Kb = K + (bkv * n + c * B) * D;

  // pass 1: mean
  {
    const int col = tid % D, grp = tid / D;
    float s = 0.f;
    for (int j = grp; j < B; j += G) s += load_f32(Kb, int64_t(j) * D + col);
    red[tid] = s;
  }
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) s += red[gi * D + tid];
    const float m = s / float(B);
    smu[tid] = m;
    mu[(bkv * n_slots + c) * D + tid] = m;
  }
  __syncthreads();

  // pass 2: covariance of the centred keys
  const int ti = tid / 16, tj = tid % 16;
  float acc[TS][TS];
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) acc[i][j] = 0.f;

  for (int j0 = 0; j0 < B; j0 += kChunk) {
    for (int e = tid; e < kChunk * D; e += kThreads) {
      const int r = e / D, col = e % D;
      X[r][col] = load_f32(Kb, int64_t(j0 + r) * D + col) - smu[col];
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < kChunk; ++r) {
      float a[TS], bb[TS];
#pragma unroll
      for (int i = 0; i < TS; ++i) {
        a[i] = X[r][ti * TS + i];
        bb[i] = X[r][tj * TS + i];
      }
#pragma unroll
      for (int i = 0; i < TS; ++i)
#pragma unroll
        for (int j = 0; j < TS; ++j) acc[i][j] = fmaf(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* S = sigma + (bkv * n_slots + c) * int64_t(D) * D;
#pragma unroll
  for (int i = 0; i < TS; ++i)
#pragma unroll
    for (int j = 0; j < TS; ++j) {
      S[(ti * TS + i) * D + tj * TS + j] = acc[i][j] / float(B);
    }
}

template <typename TIn, int D>
hipError_t launch(const Shape& s, const void* K, float* mu, float* sigma, const int32_t* cl,
                  hipStream_t st) {
  const int64_t bkv = int64_t(s.b) * s.hkv;
  dim3 grid(cl ? 1 : unsigned(s.nb), unsigned(bkv));
  if (grid.x == 0) return hipSuccess;
  hipLaunchKernelGGL((block_stats_kernel<TIn, D>), grid, dim3(kThreads), 0, st,
                     static_cast<const TIn*>(K), mu, sigma, s.n, s.B, s.nb, s.hkv, cl);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_stats(const Shape& s, const void* K, float* mu, float* sigma,
                              const int32_t* cache_len, hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch<bf16_t, 64>(s, K, mu, sigma, cache_len, st)
                     : launch<bf16_t, 128>(s, K, mu, sigma, cache_len, st);
  return s.d == 64 ? launch<float, 64>(s, K, mu, sigma, cache_len, st)
                   : launch<float, 128>(s, K, mu, sigma, cache_len, st);
}

}  // namespace ssa
