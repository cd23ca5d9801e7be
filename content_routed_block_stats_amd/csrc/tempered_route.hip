// Exact tempered block score and top-k (prefill).
//
// Write-up "Subquadratic Sparse Attention (SSA)", "The idea in one screen",
// the temperature family of its module list (centroid score <-> second-cumulant
// score <-> exact block maximum), read as the block's exact log-mean-exp of
// the raw logits:
//
//   T_c(q) = (1/beta) ln( (1/B) sum_{j in block c} exp(beta q.k_j) ),  beta > 0,
//
// whose second-order expansion in beta is the routing score
// r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q; beta -> 0 gives the block mean
// of the logits, beta -> infinity the block maximum.  Every complete causal
// block (c+1)B-1 <= t is scored and the top k are kept by the cumulant
// router's rule (ties to the lower block).  The score reads every key of
// every routable block, so the pass costs what dense causal Q K^T costs: it is
// the exact end of the family, the yardstick for the summary-based scores.
//
// One workgroup (4 waves) takes 256 consecutive query rows of one (sequence,
// KV head), rows ordered rho = t * g + j over the group's q-heads as in the
// cumulant router; each wave holds 64 rows as two 32-row MFMA column tiles.
// Keys move in chunks of 64, global -> LDS directly (no register pass), in
// the K fragment layout of the attention kernels (kv_chunks.hpp), double
// buffered.  Per chunk: S^T = K Q^T on MFMA (bf16 32x32x16, or f32 32x32x2
// for float32 inputs) with float32 accumulation, then per row a base-2
// running log-sum-exp: u = beta log2(e) s against a reference m (the block's
// first-chunk maximum, raised only when a later chunk exceeds it by more than
// 2^8, so every term stays below 2^8 and the sum holds at least one term of 1).
// At a block's last chunk the two lane halves combine and
// T = ((m + log2 l) ln 2 - ln B) / beta enters the running top-(k+1).
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "kv_chunks.hpp"
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kTempThreads = 512;   // 8 waves, two per SIMD in two groups
constexpr int kTempRows = 512;      // 64 query rows per wave
constexpr float kTempLazy = 8.f;    // largest term of a running sum, log2

// Keys [key0, key0 + 64) of one head -> LDS, K fragment (mt, s) at
// (mt * NS + s) * FRAG, lane (m, h) holding K[key0 + 32mt + m][16s + 8h + e]
// for e < 8.  One 1 KB direct global->LDS load per bfloat16 fragment (lane l
// is fragment lane l) and two per float32 fragment (load r of the fragment:
// lane l writes the half l % 2 of fragment lane 32r + l / 2).
template <bool F32, int D, typename In>
__device__ __forceinline__ void stage_keys(uint8_t* lds, const In* Kh, int64_t key0, int wave,
                                           int lane) {
  using A = AT<F32, D>;
  constexpr int PER = F32 ? 2 : 1;
  constexpr int LOADS = 2 * A::NS * PER;
#pragma unroll
  for (int i = 0; i < (LOADS + kTempThreads / 64 - 1) / (kTempThreads / 64); ++i) {
    const int r = wave + i * (kTempThreads / 64);
    if (r < LOADS) {
      const int f = r / PER, mt = f / A::NS, s = f % A::NS;
      const int m = F32 ? lane / 2 : lane % 32;
      const int h = F32 ? r % 2 : lane / 32;
      const int sel = F32 ? lane % 2 : 0;
      const uint8_t* src = reinterpret_cast<const uint8_t*>(
          Kh + (key0 + 32 * mt + m) * D + 16 * s + 8 * h + 4 * sel);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + r * 1024),
                                       16, 0, 0);
    }
  }
}

template <bool F32, int D, int KMAX>
__global__ __launch_bounds__(kTempThreads) void tempered_route_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const typename AT<F32, D>::In* __restrict__ K,
    int32_t* __restrict__ idx, float* __restrict__ kth, int64_t n, int g, int hq, int hkv, int B,
    int64_t nb, int k, float c2, float inv_beta, float log_b, int64_t n_tiles, int64_t n_bkv) {
  using A = AT<F32, D>;
  using Frag = typename A::Frag;
  constexpr int NS = A::NS;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * A::KBYTES];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int grp = wave / (kTempThreads / 128);      // waves w and w + 4 share a SIMD
  const int64_t wid = blockIdx.x;
  const int64_t bkv = wid % n_bkv;
  const int64_t tile = n_tiles - 1 - wid / n_bkv;   // longest rows first
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rows_total = n * g;
  const int64_t rho0 = tile * kTempRows;

  // query fragments of the wave's two 32-row tiles (B operand of S^T = K Q^T)
  Frag bq[2][NS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t rho = rho0 + 64 * wave + 32 * nt + ln;
    const bool valid = rho < rows_total;
    const int64_t t = valid ? rho / g : 0, jg = valid ? rho % g : 0;
    const auto* row = Q + (((b * hq + kv * g + jg) * n) + t) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) bq[nt][s] = load_row_frag<F32, D>(row, s, h, valid);
  }
  // the row this lane ranks: tile nt = h
  const int64_t my_rho = rho0 + 64 * wave + 32 * h + ln;
  const bool my_valid = my_rho < rows_total;
  const int64_t my_t = my_valid ? my_rho / g : 0;
  const int64_t my_C = my_valid ? min(nb, (my_t + 1) / B) : 0;
  const int64_t t_max = min(n - 1, (rho0 + kTempRows - 1) / g);
  const int64_t C_wg = min(nb, (t_max + 1) / B);
  const int cpb = B / kKeyChunk;
  const int64_t n_chunks = C_wg * cpb;
  const auto* Kh = K + bkv * n * D;

  float ls[KMAX + 1];
  int li[KMAX + 1];
#pragma unroll
  for (int i = 0; i <= KMAX; ++i) {
    ls[i] = -__builtin_inff();
    li[i] = -1;
  }

  floatx16 sacc[2][2];
  // S^T = K Q^T for the chunk in LDS buffer L.  K fragments move in pairs of
  // 16-wide chunks (4 fragments); the next pair's LDS reads are issued after
  // the second MFMA of the current pair, so the wait before a pair covers
  // that pair alone (while a direct-to-LDS copy is in flight only a full wait
  // on LDS reads is possible).
  auto scores = [&](const uint8_t* L) {
    auto kfrag = [&](int mt, int s) {
      return *reinterpret_cast<const Frag*>(L + (mt * NS + s) * A::FRAG + lane * 8 * A::ES);
    };
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[nt][mt][j] = 0.f;
    Frag ka[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) ka[0][q] = kfrag(q % 2, q / 2);
#pragma unroll
    for (int sp = 0; sp < NS / 2; ++sp) {
      const int slot = sp & 1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int s2 = i / 4, mt = (i / 2) % 2, nt = i % 2;
        sacc[nt][mt] = mma16(ka[slot][2 * s2 + mt], bq[nt][2 * sp + s2], sacc[nt][mt]);
        if (i == 1 && sp + 1 < NS / 2) {
#pragma unroll
          for (int q = 0; q < 4; ++q) ka[slot ^ 1][q] = kfrag(q % 2, 2 * (sp + 1) + q / 2);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Running base-2 log-sum-exp per row over the chunk's logits (lane (ln, h)
  // holds keys 32mt + 8a + 4h + b of the chunk for rows 32nt + ln); at a
  // block's last chunk, its score enters the running top-(k+1).
  float m2[2] = {0.f, 0.f}, l[2] = {0.f, 0.f};
  int jb = 0;          // chunk within the current block
  int64_t cb = 0;      // current block
  auto accumulate = [&]() {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[nt][mt][j]);
      mx = fmaxf(mx, wave_shfl_xor(mx, 32)) * c2;
      if (jb == 0) {
        m2[nt] = mx;
        l[nt] = 0.f;
      } else if (__builtin_amdgcn_ballot_w64(mx > m2[nt] + kTempLazy) != 0) {
        const float mn = fmaxf(m2[nt], mx);
        l[nt] *= __builtin_amdgcn_exp2f(m2[nt] - mn);
        m2[nt] = mn;
      }
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          ps[j % 4] += __builtin_amdgcn_exp2f(fmaf(sacc[nt][mt][j], c2, -m2[nt]));
      l[nt] += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
    if (jb == cpb - 1) {
      float T[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float lt = l[nt] + wave_shfl_xor(l[nt], 32);
        T[nt] = ((m2[nt] + __builtin_amdgcn_logf(lt)) * kLn2 - log_b) * inv_beta;
      }
      const float sn = (cb < my_C) ? (h ? T[1] : T[0]) : -__builtin_inff();
      float sc = sn;
      int ci = int(cb);
      // one pass of the running top-(k+1), sorted by (score descending, block
      // ascending) with blocks arriving in ascending order: the NEW score is
      // tested against each slot, so the entries it displaces move down one
      // and never slip past an equal later entry (strict >: the new block
      // goes after equal scores)
#pragma unroll
      for (int i = 0; i <= KMAX; ++i) {
        const bool gt = sn > ls[i];
        const float ts = ls[i];
        const int ti = li[i];
        ls[i] = gt ? sc : ts;
        li[i] = gt ? ci : ti;
        sc = gt ? ts : sc;
        ci = gt ? ti : ci;
      }
      jb = 0;
      ++cb;
    } else {
      ++jb;
    }
  };

  // Half-step schedule.  Every wave alternates scores(c) and accumulate(c);
  // the second group of waves runs half a step behind the first, so on each
  // SIMD one wave issues MFMAs while the other runs the exponentials.  Chunk
  // c + 1 is staged during half-step 2c + 1 into the buffer that chunk c - 1
  // used (read by both groups before half-step 2c); the barrier that ends a
  // half-step also waits for the copies issued in it.
  if (n_chunks > 0) stage_keys<F32, D>(lds, Kh, 0, wave, lane);
  __syncthreads();
  for (int64_t hs = 0; hs <= 2 * n_chunks; ++hs) {
    const int64_t c = hs >> 1;
    if ((hs & 1) && c + 1 < n_chunks)
      stage_keys<F32, D>(lds + ((c + 1) & 1) * A::KBYTES, Kh, (c + 1) * kKeyChunk, wave, lane);
    const int64_t j = hs - grp;
    if (j >= 0 && j < 2 * n_chunks) {
      if ((j & 1) == 0)
        scores(lds + ((j >> 1) & 1) * A::KBYTES);
      else
        accumulate();
    }
    __syncthreads();
  }

  if (!my_valid) return;
  const int64_t jg = my_rho % g;
  const int64_t orow = (b * hq + kv * g + jg) * n + my_t;
  if (k > 0) {
    int32_t* out = idx + orow * k;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < k) {
        // ascending block index, -1 (absent) last; equal keys (only -1) keep slot order
        const unsigned key_i = unsigned(li[i]);
        int rank = 0;
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k) {
            const unsigned key_j = unsigned(li[j]);
            rank += (key_j < key_i || (key_j == key_i && j < i)) ? 1 : 0;
          }
        out[rank] = li[i];
      }
    }
  }
  if (kth != nullptr) {
    float r_k = -__builtin_inff(), r_k1 = -__builtin_inff();
#pragma unroll
    for (int i = 0; i <= KMAX; ++i) {
      if (i == k - 1) r_k = ls[i];
      if (i == k) r_k1 = ls[i];
    }
    kth[orow * 2] = r_k;
    kth[orow * 2 + 1] = r_k1;
  }
}

template <bool F32, int D, int KMAX>
hipError_t launch_t(const Shape& s, const void* Q, const void* K, int32_t* idx, float* kth,
                    hipStream_t st) {
  using In = typename AT<F32, D>::In;
  const int64_t n_bkv = int64_t(s.b) * s.hkv;
  const int64_t n_tiles = tempered_route_tiles(s) / n_bkv;
  const float c2 = float(double(s.beta) * 1.4426950408889634);
  const float inv_beta = float(1.0 / double(s.beta));
  const float log_b = float(std::log(double(s.B)));
  hipLaunchKernelGGL((tempered_route_kernel<F32, D, KMAX>), dim3(unsigned(n_tiles * n_bkv)),
                     dim3(kTempThreads), 0, st, static_cast<const In*>(Q), static_cast<const In*>(K),
                     idx, kth, s.n, s.g, s.hq, s.hkv, s.B, s.nb, s.k, c2, inv_beta, log_b, n_tiles,
                     n_bkv);
  return hipGetLastError();
}

template <bool F32, int D>
hipError_t launch_d(const Shape& s, const void* Q, const void* K, int32_t* idx, float* kth,
                    hipStream_t st) {
  if (s.k <= 8) return launch_t<F32, D, 8>(s, Q, K, idx, kth, st);
  if (s.k <= 16) return launch_t<F32, D, 16>(s, Q, K, idx, kth, st);
  return launch_t<F32, D, 32>(s, Q, K, idx, kth, st);
}

}  // namespace

int64_t tempered_route_tiles(const Shape& s) {
  return (s.n * s.g + kTempRows - 1) / kTempRows * int64_t(s.b) * s.hkv;
}

hipError_t launch_route_tempered(const Shape& s, const void* Q, const void* K, int32_t* idx,
                                 float* kth, hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch_d<false, 64>(s, Q, K, idx, kth, st)
                     : launch_d<false, 128>(s, Q, K, idx, kth, st);
  return s.d == 64 ? launch_d<true, 64>(s, Q, K, idx, kth, st)
                   : launch_d<true, 128>(s, Q, K, idx, kth, st);
}

}  // namespace ssa
