// Exact hierarchical routing: the flat top-k by branch and bound over groups
// of blocks (decode queries).
//
// Write-up "Subquadratic Sparse Attention (SSA)": its module list pairs the
// flat router with branch-and-bound exact selection under an admissible bound
// and a tree router with a recursive radius, and its "Selected results"
// report lossless branch-and-bound selection costs as a fraction of keys.
// Groups of m consecutive blocks carry a summary -- the mean mu_G of their
// mu_c, the radius R_G = max ||mu_c - mu_G||, the mean S_G of their Sigma_c
// and lam_G = max (tr (Sigma_c - S_G)^4)^(1/4) >= ||Sigma_c - S_G||_2 -- so that
// for beta >= 0 every member's score is at most
//   UB_G(q) = q.mu_G + ||q|| R_G + (beta/2) (q^T S_G q + lam_G ||q||^2).
// Groups are visited in decreasing order of their bound (largest over the
// q-heads of a KV head) and a group is skipped when, for every row, its bound
// is strictly below the row's running k-th score; skipped blocks cannot enter
// any row's top-k (their scores are below it, ties included), so the
// selection is the flat one.  The bound carries a relative margin of 1e-4
// over its float32 rounding and the float32 scores, so the pruning stays
// conservative.  Levels compose (a group of groups has radius
// max(||mu_G - mu_GG|| + R_G) and slack max(||S_G - S_GG|| + lam_G)); one
// level is built.
//
//  * group_stats: one workgroup per (sequence, KV head, group): mu_G, S_G, R_G
//    and lam_G, the last from A = Sigma_c - S_G staged in LDS, A^T A formed in
//    register tiles, then (sum of squares of A^T A)^(1/4).
//  * bound: one workgroup per (sequence, KV head, group): UB_G for the KV
//    head's q-heads (one decode query row each), symmetric upper-tile reads.
//  * bb: one 1024-thread workgroup per (sequence, KV head) runs the visit.
//    The order is a bitonic sort in LDS; a visited group's blocks are scored
//    four at a time (one 256-thread subgroup per block, every load of the
//    block's upper 32 x 32 tiles issued at once, so the stream is bandwidth-
//    rather than latency-bound) and merged into the rows' top-k lists.
#include <algorithm>
#include <cmath>

#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kHierThreads = 256;
constexpr int kHierMaxRows = 16;        // q-heads per KV head
constexpr int kHierMaxBounds = 8192;    // q-heads x groups per (sequence, KV head)
constexpr int kHierMaxGroup = 64;       // blocks per group
constexpr int kBBThreads = 1024;        // branch-and-bound workgroup
constexpr int kBBSubs = kBBThreads / kHierThreads;   // blocks scored at once
constexpr float kHierMargin = 1e-4f;

__device__ __forceinline__ float hier_block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += wave_shfl_xor(v, o);
  const int wave = threadIdx.x / 64;
  __syncthreads();
  if (threadIdx.x % 64 == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < int(blockDim.x) / 64; ++w) s += red[w];
  return s;
}

template <int D>
__global__ __launch_bounds__(kHierThreads) void group_stats_kernel(
    const float* __restrict__ mu, const float* __restrict__ sigma, float* __restrict__ gmu,
    float* __restrict__ gS, float* __restrict__ grl, int64_t nb, int m, int64_t G) {
  constexpr int PER = D * D / kHierThreads;      // covariance entries per thread (tid + 256 i)
  __shared__ float A[D * D];
  __shared__ float mg[D];
  __shared__ float red[kHierThreads / 64];
  const int tid = threadIdx.x;
  const int64_t gi = blockIdx.x, bkv = blockIdx.y;
  const int64_t c0 = gi * m, c1 = min(nb, c0 + m);
  const float inv = 1.f / float(c1 - c0);
  const float* mu_b = mu + bkv * nb * D;
  const float* sg_b = sigma + bkv * nb * D * D;
  // mean centroid and mean covariance (the latter kept in registers)
  for (int i = tid; i < D; i += kHierThreads) {
    float s = 0.f;
    for (int64_t c = c0; c < c1; ++c) s += mu_b[c * D + i];
    mg[i] = s * inv;
    gmu[(bkv * G + gi) * D + i] = s * inv;
  }
  float sg[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) sg[i] = 0.f;
  for (int64_t c = c0; c < c1; ++c) {
    const float* S = sg_b + c * D * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) sg[i] += S[tid + kHierThreads * i];
  }
  float* Sg = gS + (bkv * G + gi) * D * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    sg[i] *= inv;
    Sg[tid + kHierThreads * i] = sg[i];
  }
  __syncthreads();
  float R = 0.f, lam = 0.f;
  // TS x TS tile of A^T A (= A^2, A symmetric) per thread; both operands are
  // read along row kk of A, so a wave's reads are broadcasts or one full row
  const int ti = tid / 16, tj = tid % 16;
  constexpr int TS = D / 16;
  for (int64_t c = c0; c < c1; ++c) {
    float dv = 0.f;
    for (int i = tid; i < D; i += kHierThreads) {
      const float x = mu_b[c * D + i] - mg[i];
      dv += x * x;
    }
    const float r2 = hier_block_sum(dv, red);
    R = fmaxf(R, sqrtf(r2));
    const float* S = sg_b + c * D * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) A[tid + kHierThreads * i] = S[tid + kHierThreads * i] - sg[i];
    __syncthreads();
    float acc[TS][TS];
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
      for (int bb = 0; bb < TS; ++bb) acc[a][bb] = 0.f;
    for (int kk = 0; kk < D; ++kk) {
      float ra[TS], rb[TS];
#pragma unroll
      for (int a = 0; a < TS; ++a) ra[a] = A[kk * D + TS * ti + a];
#pragma unroll
      for (int bb = 0; bb < TS; ++bb) rb[bb] = A[kk * D + TS * tj + bb];
#pragma unroll
      for (int a = 0; a < TS; ++a)
#pragma unroll
        for (int bb = 0; bb < TS; ++bb) acc[a][bb] = fmaf(ra[a], rb[bb], acc[a][bb]);
    }
    float sq = 0.f;
#pragma unroll
    for (int a = 0; a < TS; ++a)
#pragma unroll
      for (int bb = 0; bb < TS; ++bb) sq += acc[a][bb] * acc[a][bb];
    // sum of squares of A^T A: the sum of sigma_i^4 over A's singular values
    // (tr A^4 for symmetric A), at least ||A||_2^4 for any A
    const float t4 = hier_block_sum(sq, red);
    lam = fmaxf(lam, sqrtf(sqrtf(t4)));
    __syncthreads();
  }
  if (tid == 0) {
    // relative margins over the float32 rounding of these sums
    grl[(bkv * G + gi) * 2] = R * (1.f + 1e-5f);
    grl[(bkv * G + gi) * 2 + 1] = lam * (1.f + 1e-4f);
  }
}

// q^T M q, q . v (and, with NORM, ||q||^2) for the g rows in LDS
// (qs[r * D + i]) over one 256-thread workgroup, M symmetric: thread
// (ri = tid / 8, cq = tid % 8) reads 4 floats of every upper 32 x 32 tile
// (row 32 ti + ri, columns 32 tj + 4 cq); off-diagonal tiles count twice.
// The per-row totals land in out[3 * r + {0: quad, 1: lin, 2: norm^2}].
template <int D, bool NORM>
__device__ __forceinline__ void wg_forms(const float* __restrict__ M, const float* __restrict__ v,
                                         const float* qs, int g, float* red, float* out) {
  constexpr int MT = D / 32;
  const int tid = threadIdx.x, ri = tid / 8, cq = tid % 8, wave = tid / 64, lane = tid % 64;
  floatx4 sv[MT * (MT + 1) / 2];
#pragma unroll
  for (int ti = 0, t = 0; ti < MT; ++ti)
#pragma unroll
    for (int tj = ti; tj < MT; ++tj, ++t)
      sv[t] = *reinterpret_cast<const floatx4*>(M + (32 * ti + ri) * D + 32 * tj + 4 * cq);
  const float vi = tid < D ? v[tid] : 0.f;
  constexpr int NW = kHierThreads / 64;
#pragma unroll
  for (int r = 0; r < kHierMaxRows; ++r) {
    if (r < g) {
      const float* qr = qs + r * D;
      float quad = 0.f;
#pragma unroll
      for (int ti = 0, t = 0; ti < MT; ++ti) {
        float inner = 0.f;
#pragma unroll
        for (int tj = ti; tj < MT; ++tj, ++t) {
          const floatx4 qv = *reinterpret_cast<const floatx4*>(qr + 32 * tj + 4 * cq);
          const float w = tj == ti ? 1.f : 2.f;
          inner += w * (sv[t][0] * qv[0] + sv[t][1] * qv[1] + sv[t][2] * qv[2] + sv[t][3] * qv[3]);
        }
        quad = fmaf(qr[32 * ti + ri], inner, quad);
      }
      const float x = tid < D ? qr[tid] : 0.f;
      float lin = vi * x, nrm = x * x;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        quad += wave_shfl_xor(quad, o);
        lin += wave_shfl_xor(lin, o);
        if (NORM) nrm += wave_shfl_xor(nrm, o);
      }
      if (lane == 0) {
        red[(3 * r) * NW + wave] = quad;
        red[(3 * r + 1) * NW + wave] = lin;
        red[(3 * r + 2) * NW + wave] = NORM ? nrm : 0.f;
      }
    }
  }
  __syncthreads();
  if (tid < 3 * g) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) x += red[tid * NW + w];
    out[tid] = x;
  }
  __syncthreads();
}

template <typename TIn, int D>
__device__ __forceinline__ void stage_rows(const TIn* q, int64_t row0, int g, float* qs) {
  for (int e = threadIdx.x; e < g * D; e += kHierThreads) qs[e] = load_f32(q, row0 * D + e);
  __syncthreads();
}

__device__ __forceinline__ int64_t routable_blocks(const int32_t* pos, int64_t b, int B,
                                                  int64_t nb) {
  const int64_t t = pos[b];
  return t < 0 ? 0 : min(nb, (t + 1) / B);
}

// UB_G for every routable group and row: ub[(bkv * g + r) * G + gi], with a
// relative margin over the float32 rounding of the terms.
template <typename TIn, int D>
__global__ __launch_bounds__(kHierThreads) void hier_bound_kernel(
    const TIn* __restrict__ q, const float* __restrict__ gmu, const float* __restrict__ gS,
    const float* __restrict__ grl, const int32_t* __restrict__ pos, float* __restrict__ ub, int g,
    int hq, int hkv, int B, int64_t nb, int m, int64_t G, float beta) {
  __shared__ __align__(16) float qs[kHierMaxRows * D];
  __shared__ float red[3 * kHierMaxRows * (kHierThreads / 64)];
  __shared__ float tot[3 * kHierMaxRows];
  const int64_t gi = blockIdx.x, bkv = blockIdx.y, b = bkv / hkv, kv = bkv % hkv;
  const int64_t C = routable_blocks(pos, b, B, nb);
  if (gi >= (C + m - 1) / m) return;
  stage_rows<TIn, D>(q, b * hq + kv * g, g, qs);
  wg_forms<D, true>(gS + (bkv * G + gi) * D * D, gmu + (bkv * G + gi) * D, qs, g, red, tot);
  if (threadIdx.x < g) {
    const int r = threadIdx.x;
    const float R = grl[(bkv * G + gi) * 2], lam = grl[(bkv * G + gi) * 2 + 1];
    const float quad = tot[3 * r], lin = tot[3 * r + 1], n2 = tot[3 * r + 2], qn = sqrtf(n2);
    const float u = lin + qn * R + 0.5f * beta * (quad + lam * n2);
    const float mag = fabsf(lin) + qn * R + 0.5f * beta * (fabsf(quad) + lam * n2);
    ub[(bkv * g + r) * G + gi] = u + kHierMargin * mag;
  }
}

// Partial q^T M q and q . v of one 256-thread subgroup of a larger
// workgroup (wg_forms without the final sum): lane 0 of each of the
// subgroup's waves leaves its sums in red_sub[(2 r + {0: quad, 1: lin}) * 4 + wave].
template <int D>
__device__ __forceinline__ void sub_forms(const float* __restrict__ M, const float* __restrict__ v,
                                          const float* qs, int g, float* red_sub) {
  constexpr int MT = D / 32;
  const int t = threadIdx.x % kHierThreads, ri = t / 8, cq = t % 8, ws = t / 64, lane = t % 64;
  floatx4 sv[MT * (MT + 1) / 2];
#pragma unroll
  for (int ti = 0, k = 0; ti < MT; ++ti)
#pragma unroll
    for (int tj = ti; tj < MT; ++tj, ++k)
      sv[k] = *reinterpret_cast<const floatx4*>(M + (32 * ti + ri) * D + 32 * tj + 4 * cq);
  const float vi = t < D ? v[t] : 0.f;
#pragma unroll
  for (int r = 0; r < kHierMaxRows; ++r) {
    if (r < g) {
      const float* qr = qs + r * D;
      float quad = 0.f;
#pragma unroll
      for (int ti = 0, k = 0; ti < MT; ++ti) {
        float inner = 0.f;
#pragma unroll
        for (int tj = ti; tj < MT; ++tj, ++k) {
          const floatx4 qv = *reinterpret_cast<const floatx4*>(qr + 32 * tj + 4 * cq);
          const float w = tj == ti ? 1.f : 2.f;
          inner += w * (sv[k][0] * qv[0] + sv[k][1] * qv[1] + sv[k][2] * qv[2] + sv[k][3] * qv[3]);
        }
        quad = fmaf(qr[32 * ti + ri], inner, quad);
      }
      float lin = t < D ? vi * qr[t] : 0.f;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        quad += wave_shfl_xor(quad, o);
        lin += wave_shfl_xor(lin, o);
      }
      if (lane == 0) {
        red_sub[(2 * r) * 4 + ws] = quad;
        red_sub[(2 * r + 1) * 4 + ws] = lin;
      }
    }
  }
}

// Ascending sort key of a group: decreasing largest bound (a NaN bound counts
// as +inf), then increasing group index.
__device__ __forceinline__ uint64_t visit_key(float u, int64_t gi) {
  if (u != u) u = __builtin_inff();
  const uint32_t bits = __builtin_bit_cast(uint32_t, u);
  const uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);   // ascending in u
  return (uint64_t(~ord) << 32) | uint64_t(gi);
}

// Branch and bound for one (sequence, KV head): the group's q-heads (one
// decode query row each) share the visit.  Groups are taken in decreasing
// order of their largest bound; a group is skipped when, for every row, its
// bound is strictly below the row's current k-th score; otherwise its blocks
// are scored (four at a time, one 256-thread subgroup each) and merged into
// every row's top-k list (one wave per row, rank by (score desc, block asc)).
template <typename TIn, int D, int KMAX>
__global__ __launch_bounds__(kBBThreads) void hier_bb_kernel(
    const TIn* __restrict__ q, const float* __restrict__ mu, const float* __restrict__ sigma,
    const float* __restrict__ ub, const int32_t* __restrict__ pos, int32_t* __restrict__ idx,
    int32_t* __restrict__ evaluated, int g, int hq, int hkv, int B, int64_t nb, int m, int64_t G,
    int k, float beta) {
  __shared__ uint64_t keys[kHierMaxBounds];
  __shared__ float ubl[kHierMaxBounds];                    // [row][group]
  __shared__ __align__(16) float qs[kHierMaxRows * D];
  __shared__ float sc[kHierMaxRows * kHierMaxGroup];
  __shared__ float red[kBBSubs * 2 * kHierMaxRows * 4];
  __shared__ float ls[2][kHierMaxRows * KMAX];
  __shared__ int32_t li[2][kHierMaxRows * KMAX];
  __shared__ float tau[kHierMaxRows];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int sub = tid / kHierThreads, t = tid % kHierThreads;
  const int64_t bkv = blockIdx.x, b = bkv / hkv, kv = bkv % hkv;
  const int64_t C = routable_blocks(pos, b, B, nb);
  const int64_t Gc = (C + m - 1) / m;
  int64_t P = 1;
  while (P < Gc) P <<= 1;
  for (int e = tid; e < g * D; e += kBBThreads) qs[e] = load_f32(q, (b * hq + kv * g) * D + e);
  for (int64_t e = tid; e < int64_t(g) * Gc; e += kBBThreads)
    ubl[e] = ub[(bkv * g + e / Gc) * G + e % Gc];
  for (int e = tid; e < g * KMAX; e += kBBThreads) {
    ls[0][e] = -__builtin_inff();
    li[0][e] = 0x7FFFFFFF;
  }
  if (tid < g) tau[tid] = -__builtin_inff();
  __syncthreads();
  for (int64_t gi = tid; gi < P; gi += kBBThreads) {
    if (gi < Gc) {
      float u = -__builtin_inff();
      for (int r = 0; r < g; ++r) {
        const float x = ubl[r * Gc + gi];
        u = fmaxf(u, x != x ? __builtin_inff() : x);
      }
      keys[gi] = visit_key(u, gi);
    } else {
      keys[gi] = ~uint64_t(0);
    }
  }
  __syncthreads();
  // bitonic sort of the P keys
  for (int64_t k2 = 2; k2 <= P; k2 <<= 1) {
    for (int64_t j = k2 >> 1; j > 0; j >>= 1) {
      for (int64_t i = tid; i < P; i += kBBThreads) {
        const int64_t ij = i ^ j;
        if (ij > i) {
          const uint64_t a = keys[i], c = keys[ij];
          const bool up = (i & k2) == 0;
          if ((a > c) == up) {
            keys[i] = c;
            keys[ij] = a;
          }
        }
      }
      __syncthreads();
    }
  }

  int buf = 0;
  int32_t n_eval = 0;
  const int iters = (m + kBBSubs - 1) / kBBSubs;
  for (int64_t oi = 0; oi < Gc; ++oi) {
    const int64_t gi = int64_t(keys[oi] & 0xFFFFFFFFu);
    const bool need = tid < g && !(ubl[tid * Gc + gi] < tau[tid]);
    if (!__syncthreads_or(need)) continue;
    const int64_t c0 = gi * m, c1 = min(C, c0 + m);
    const int nnew = int(c1 - c0);
    for (int it = 0; it < iters; ++it) {
      const int jb = it * kBBSubs + sub;
      const int64_t c = c0 + jb;
      float* rs = red + sub * 2 * kHierMaxRows * 4;
      if (c < c1) sub_forms<D>(sigma + (bkv * nb + c) * D * D, mu + (bkv * nb + c) * D, qs, g, rs);
      __syncthreads();
      if (t < g && c < c1) {
        const float quad = rs[(2 * t) * 4] + rs[(2 * t) * 4 + 1] + rs[(2 * t) * 4 + 2] + rs[(2 * t) * 4 + 3];
        const float lin = rs[(2 * t + 1) * 4] + rs[(2 * t + 1) * 4 + 1] + rs[(2 * t + 1) * 4 + 2] +
                          rs[(2 * t + 1) * 4 + 3];
        sc[t * kHierMaxGroup + jb] = lin + 0.5f * beta * quad;
      }
      __syncthreads();
    }
    n_eval += nnew;
    // merge: candidate e < k is the row's list entry e, e >= k the block
    // c0 + e - k; rank by (score desc, block asc, candidate asc)
    if (wave < g) {
      const int r = wave, nc = k + nnew;
      const float* cs = ls[buf] + r * KMAX;
      const int32_t* ci = li[buf] + r * KMAX;
      for (int e = lane; e < nc; e += 64) {
        const float se = e < k ? cs[e] : sc[r * kHierMaxGroup + e - k];
        const int32_t ie = e < k ? ci[e] : int32_t(c0 + e - k);
        int rank = 0;
        for (int f = 0; f < nc; ++f) {
          const float sf = f < k ? cs[f] : sc[r * kHierMaxGroup + f - k];
          const int32_t jf = f < k ? ci[f] : int32_t(c0 + f - k);
          rank += (sf > se || (sf == se && (jf < ie || (jf == ie && f < e)))) ? 1 : 0;
        }
        if (rank < k) {
          ls[buf ^ 1][r * KMAX + rank] = se;
          li[buf ^ 1][r * KMAX + rank] = ie;
        }
      }
    }
    __syncthreads();
    buf ^= 1;
    if (tid < g) tau[tid] = ls[buf][tid * KMAX + k - 1];   // -inf until k blocks are held
  }

  // ascending block order, -1 padded
  if (wave < g && lane < k) {
    const int r = wave;
    const int32_t v = li[buf][r * KMAX + lane];
    int rank = 0;
    for (int f = 0; f < k; ++f) {
      const int32_t w = li[buf][r * KMAX + f];
      rank += (w < v || (w == v && f < lane)) ? 1 : 0;
    }
    idx[(b * hq + kv * g + r) * k + rank] = v == 0x7FFFFFFF ? -1 : v;
  }
  if (evaluated != nullptr && tid == 0) evaluated[bkv] = n_eval;
}

__global__ void hier_fill_i32_kernel(int32_t* p, int64_t count, int32_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

size_t hier_ws_bytes(const Shape& s) {
  // bounds [b, hkv, g, G], G <= nb
  return align_up(size_t(int64_t(s.b) * s.hq * s.nb) * 4);
}

template <int D>
hipError_t launch_group_stats_d(const Shape& s, const float* mu, const float* sigma, int m,
                                float* gmu, float* gS, float* grl, hipStream_t st) {
  const int64_t G = (s.nb + m - 1) / m;
  hipLaunchKernelGGL((group_stats_kernel<D>), dim3(unsigned(G), unsigned(s.b * s.hkv)),
                     dim3(kHierThreads), 0, st, mu, sigma, gmu, gS, grl, s.nb, m, G);
  return hipGetLastError();
}

template <typename TIn, int D, int KMAX>
hipError_t launch_hier_t(const Shape& s, const TIn* q, const float* mu, const float* sigma,
                         const float* ub, int m, const int32_t* pos, int32_t* idx,
                         int32_t* evaluated, hipStream_t st) {
  const int64_t G = (s.nb + m - 1) / m;
  hipLaunchKernelGGL((hier_bb_kernel<TIn, D, KMAX>), dim3(unsigned(int64_t(s.b) * s.hkv)),
                     dim3(kBBThreads), 0, st, q, mu, sigma, ub, pos, idx, evaluated, s.g, s.hq,
                     s.hkv, s.B, s.nb, m, G, s.k, s.beta);
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_hier_d(const Shape& s, const void* q_, const float* mu, const float* sigma,
                         const float* gmu, const float* gS, const float* grl, int m,
                         const int32_t* pos, int32_t* idx, int32_t* evaluated, void* ws,
                         hipStream_t st) {
  const TIn* q = static_cast<const TIn*>(q_);
  const int64_t G = (s.nb + m - 1) / m, bkv = int64_t(s.b) * s.hkv;
  float* ub = static_cast<float*>(ws);
  hipLaunchKernelGGL((hier_bound_kernel<TIn, D>), dim3(unsigned(G), unsigned(bkv)),
                     dim3(kHierThreads), 0, st, q, gmu, gS, grl, pos, ub, s.g, s.hq, s.hkv, s.B,
                     s.nb, m, G, s.beta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (s.k <= 8) return launch_hier_t<TIn, D, 8>(s, q, mu, sigma, ub, m, pos, idx, evaluated, st);
  if (s.k <= 16) return launch_hier_t<TIn, D, 16>(s, q, mu, sigma, ub, m, pos, idx, evaluated, st);
  return launch_hier_t<TIn, D, 32>(s, q, mu, sigma, ub, m, pos, idx, evaluated, st);
}

}  // namespace

int hier_max_rows() { return kHierMaxRows; }
int hier_max_bounds() { return kHierMaxBounds; }
int hier_max_group() { return kHierMaxGroup; }
size_t route_hier_workspace_bytes(const Shape& s) { return hier_ws_bytes(s); }

hipError_t launch_group_stats(const Shape& s, const float* mu, const float* sigma, int m, float* gmu,
                              float* gS, float* grl, hipStream_t st) {
  return s.d == 64 ? launch_group_stats_d<64>(s, mu, sigma, m, gmu, gS, grl, st)
                   : launch_group_stats_d<128>(s, mu, sigma, m, gmu, gS, grl, st);
}

hipError_t launch_route_hier(const Shape& s, const void* q, const float* mu, const float* sigma,
                             const float* gmu, const float* gS, const float* grl, int m,
                             const int32_t* pos, int32_t* idx, int32_t* evaluated, void* ws,
                             hipStream_t st) {
  if (s.k == 0 || s.nb == 0) {
    // nothing to select, or no block slots: no block is scored
    const int64_t rows = int64_t(s.b) * s.hq;
    if (s.k > 0)
      hipLaunchKernelGGL(hier_fill_i32_kernel,
                         dim3(unsigned(std::min<int64_t>((rows * s.k + 255) / 256, 1024))),
                         dim3(256), 0, st, idx, rows * s.k, -1);
    if (evaluated != nullptr)
      hipLaunchKernelGGL(hier_fill_i32_kernel, dim3(1), dim3(256), 0, st, evaluated,
                         int64_t(s.b) * s.hkv, 0);
    return hipGetLastError();
  }
  if (s.in_bf16)
    return s.d == 64 ? launch_hier_d<bf16_t, 64>(s, q, mu, sigma, gmu, gS, grl, m, pos, idx, evaluated, ws, st)
                     : launch_hier_d<bf16_t, 128>(s, q, mu, sigma, gmu, gS, grl, m, pos, idx, evaluated, ws, st);
  return s.d == 64 ? launch_hier_d<float, 64>(s, q, mu, sigma, gmu, gS, grl, m, pos, idx, evaluated, ws, st)
                   : launch_hier_d<float, 128>(s, q, mu, sigma, gmu, gS, grl, m, pos, idx, evaluated, ws, st);
}

}  // namespace ssa
