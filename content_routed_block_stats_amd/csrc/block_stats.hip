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
  constexpr int TS = D / 16;             // Sigma tile per thread: TS x TS
  __shared__ float smu[D];
  __shared__ __attribute__((aligned(16))) float X[kChunk][D + 4];

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

  // 16-byte pieces of a key row: EP elements each, PPR per row
  constexpr int EP = 16 / int(sizeof(TIn));
  constexpr int PPR = D / EP;
  constexpr int RSTEP = kThreads / PPR;  // rows per step of pass 1
  static_assert(RSTEP * D <= kChunk * (D + 4), "pass-1 partial sums fit the chunk buffer");
  auto piece = [&](int64_t j, int pc, float (&v)[EP]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(Kb + j * D + pc * EP);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (EP == 8) {
        v[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
        v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
      } else {
        // copy the element out first: bit-casting a vector element lvalue
        // directly reads element 0 with this compiler
        const uint32_t u = w[i];
        v[i] = __builtin_bit_cast(float, u);
      }
    }
  };

  // pass 1: mean (each thread sums one piece column over every RSTEP-th row)
  {
    const int pc = tid % PPR, rg = tid / PPR;
    float sv[EP];
#pragma unroll
    for (int i = 0; i < EP; ++i) sv[i] = 0.f;
    for (int j = rg; j < B; j += RSTEP) {
      float v[EP];
      piece(j, pc, v);
#pragma unroll
      for (int i = 0; i < EP; ++i) sv[i] += v[i];
    }
    float* part = &X[0][0];   // [rg][D]
#pragma unroll
    for (int i = 0; i < EP; ++i) part[rg * D + pc * EP + i] = sv[i];
  }
  __syncthreads();
  if (tid < D) {
    const float* part = &X[0][0];
    float s = 0.f;
#pragma unroll
    for (int gi = 0; gi < RSTEP; ++gi) s += part[gi * D + tid];
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
    for (int e = tid; e < kChunk * PPR; e += kThreads) {
      const int r = e / PPR, pc = e % PPR;
      float v[EP];
      piece(j0 + r, pc, v);
#pragma unroll
      for (int i = 0; i < EP; i += 4)
        *reinterpret_cast<floatx4*>(&X[r][pc * EP + i]) =
            floatx4{v[i] - smu[pc * EP + i], v[i + 1] - smu[pc * EP + i + 1],
                    v[i + 2] - smu[pc * EP + i + 2], v[i + 3] - smu[pc * EP + i + 3]};
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
