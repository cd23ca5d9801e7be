// Query-tile-shared routing (prefill): one block selection per tile of B
// consecutive query positions of one (sequence, q-head).
//
// Write-up "Subquadratic Sparse Attention (SSA)": its fused kernel routes per
// query block; the notes on the compute floor ("Selected results") name an
// (n/b)^2 block-score GEMM and an argsort block-mask build.  Reading: tile j
// holds positions [jB, (j+1)B) and selects, for all its queries, the top k of
// the blocks complete before it (c < j) by the summed routing score
//
//   R_c(j) = sum_{t in tile} r_c(q_t) = s_j . mu_c + (beta/2) <Sigma_c, M_j>,
//   s_j = sum_t q_t,   M_j = sum_t q_t q_t^T,
//
// (ties to the lower block).  The second form turns the whole routing step
// into one GEMM per KV head over the tile moments:
//
//  1. tile_moments: s_j and M_j per tile on MFMA (bf16 products exact, float32
//     accumulation; Q^T staged through LDS), packed per tile as the 32x32
//     tiles (mt <= nt) of M -- off-diagonal tiles doubled, so the Frobenius
//     product with the symmetric Sigma_c counts both halves -- followed by s_j;
//  2. tile_score: R = [packed M | s] . [(beta/2) packed Sigma_c | mu_c]^T on
//     float32 MFMA, reading Sigma and mu as ssa_block_stats wrote them; rows
//     are the group's (tile, q-head) pairs, columns the blocks; output tiles
//     with no block before any of their tiles are skipped (the causal half);
//  3. tile_topk: per tile, k rounds of a wave arg-max over c < min(j, nb),
//     the selection written in ascending order, padded with -1.
#include <algorithm>
#include <type_traits>

#include "kv_chunks.hpp"
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kMomRows = 64;         // query rows per LDS chunk of the moments kernel
constexpr int kScoreRows = 128;      // GEMM rows (tile, q-head pairs) per workgroup
constexpr int kScoreCols = 64;       // GEMM columns (blocks) per workgroup
constexpr int kScoreStages = 4;      // register stages of the GEMM's operand prefetch

// Packed moment coordinates for head dimension D: the NUP upper 32x32 tiles
// of the d x d matrix in (mt, nt >= mt) order, 1024 coordinates each
// (row-major inside the tile), then the D coordinates of the first moment --
// P in all, contracted 16 at a time (STEPS steps).  Stored step-major per KV
// head, [step][row][16] with row = j g + jg, so that the GEMM's operand loads
// for 32 consecutive rows are one contiguous 2 KB run.
template <int D>
struct Moments {
  static constexpr int MT = D / 32;
  static constexpr int NUP = MT * (MT + 1) / 2;
  static constexpr int P = NUP * 1024 + D;      // floats per tile
  static constexpr int SIG_STEPS = NUP * 64;    // 16-coordinate steps of the M part
  static constexpr int STEPS = P / 16;          // ... and of M then s
};

__host__ __device__ constexpr void up_tile(int u, int mt_count, int& mt, int& nt) {
  int m = 0;
  while (u >= mt_count - m) {
    u -= mt_count - m;
    ++m;
  }
  mt = m;
  nt = m + u;
}

// ------------------------------------------------------------ tile moments --
//
// One workgroup (4 waves) per (sequence, q-head, tile).  A chunk of 64 query
// rows is staged transposed (Q^T: one LDS row of 64 query values per
// dimension, 8-row groups XOR-swizzled by the dimension against bank
// conflicts), so that both MFMA operands of M = Q^T Q are 16-byte reads: the
// fragment F(x, s) of lane (m, h) holds q_{16s+8h+e}[32x + m].  The jobs --
// the NUP tiles of M and the MT tiles of Q^T 1 (the first moment, every
// column equal) -- are spread over the waves.
template <bool F32, int D>
__global__ __launch_bounds__(256) void tile_moments_kernel(const typename AT<F32, D>::In* __restrict__ Q,
                                                           float* __restrict__ Am, int64_t n, int g,
                                                           int hq, int hkv, int B, int64_t n_tiles) {
  using A = AT<F32, D>;
  using In = typename A::In;
  using Frag = typename A::Frag;
  using Mo = Moments<D>;
  constexpr int ES = A::ES;
  constexpr int JOBS = Mo::NUP + Mo::MT;
  constexpr int JPW = (JOBS + 3) / 4;            // jobs per wave
  __shared__ __attribute__((aligned(16))) uint8_t qt[D * kMomRows * ES];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t j = blockIdx.x, bh = blockIdx.y;
  const int64_t b = bh / hq, hh = bh % hq, kv = hh / g, jg = hh % g;
  const int64_t t0 = j * B, t1 = min(n, t0 + B);
  const In* Qh = Q + bh * n * D;
  const int64_t rows_total = n_tiles * g;
  // coordinate p of this tile's row -> [step p / 16][row][p % 16]
  float* out = Am + ((b * hkv + kv) * Mo::STEPS * rows_total + j * g + jg) * 16;
  auto put = [&](int p, float v) { out[(int64_t(p / 16) * rows_total) * 16 + p % 16] = v; };

  // byte offset of (dimension c, row r) in the transposed chunk
  auto qt_off = [](int c, int r) { return (c * kMomRows + 8 * ((r / 8) ^ (c % 8)) + r % 8) * ES; };
  auto frag = [&](int x, int s) {
    return *reinterpret_cast<const Frag*>(qt + qt_off(32 * x + ln, 16 * s + 8 * h));
  };
  Frag ones;
  if constexpr (F32) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = 1.f;
  } else {
    ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  }

  floatx16 acc[JPW];
#pragma unroll
  for (int q = 0; q < JPW; ++q)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[q][i] = 0.f;

  for (int64_t r0 = t0; r0 < t1; r0 += kMomRows) {
    // rows across lanes, 8 consecutive dimensions per lane: each LDS store
    // instruction fills one dimension's 64-row line
    for (int w = tid; w < kMomRows * (D / 8); w += 256) {
      const int r = w % kMomRows, cp = w / kMomRows;
      const bool valid = r0 + r < t1;
      In v[8];
      if constexpr (F32) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f}, c = a;
        if (valid) {
          a = *reinterpret_cast<const floatx4*>(Qh + (r0 + r) * D + 8 * cp);
          c = *reinterpret_cast<const floatx4*>(Qh + (r0 + r) * D + 8 * cp + 4);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = a[e];
          v[e + 4] = c[e];
        }
      } else {
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (valid) wv = *reinterpret_cast<const u32x4*>(Qh + (r0 + r) * D + 8 * cp);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf16_t{u16((wv[e / 2] >> (16 * (e & 1))) & 0xFFFFu)};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) *reinterpret_cast<In*>(qt + qt_off(8 * cp + e, r)) = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < JPW; ++q) {
      const int job = wave + 4 * q;
      if (job < JOBS) {
        int mt, nt;
        if (job < Mo::NUP) up_tile(job, Mo::MT, mt, nt); else mt = nt = job - Mo::NUP;
#pragma unroll
        for (int s = 0; s < kMomRows / 16; ++s)
          acc[q] = mma16(frag(mt, s), job < Mo::NUP ? frag(nt, s) : ones, acc[q]);
      }
    }
    __syncthreads();
  }

  // acc lane (ln, h): entries (8a + 4h + b, ln) of the job's 32x32 tile
#pragma unroll
  for (int q = 0; q < JPW; ++q) {
    const int job = wave + 4 * q;
    if (job >= JOBS) continue;
    if (job < Mo::NUP) {
      int mt, nt;
      up_tile(job, Mo::MT, mt, nt);
      const float w = mt == nt ? 1.f : 2.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * (i / 4) + 4 * h + i % 4;
        put(job * 1024 + row * 32 + ln, w * acc[q][i]);
      }
    } else if (ln == 0) {
      const int x = job - Mo::NUP;
#pragma unroll
      for (int i = 0; i < 16; ++i) put(Mo::NUP * 1024 + 32 * x + 8 * (i / 4) + 4 * h + i % 4, acc[q][i]);
    }
  }
}

// -------------------------------------------------------------- tile score --
//
// Per KV head, rows rho = j g + jg (tile j, q-head jg of the group), columns
// the blocks.  Workgroup tile kScoreRows x kScoreCols, four waves in 2 x 2,
// each 64 rows (two accumulator chains) x 32 blocks.  Operands come straight
// from global memory (both are read by two waves of the workgroup, mostly
// from cache), kScoreStages contraction steps ahead of their MFMAs.  One step
// contracts 16 coordinates: lane (m, h) supplies coordinates 8h..8h+7 of its
// row (A) or block (B), 32 contiguous bytes on both sides.
template <int D>
__global__ __launch_bounds__(256) void tile_score_kernel(const float* __restrict__ Am,
                                                         const float* __restrict__ sigma,
                                                         const float* __restrict__ mu,
                                                         float* __restrict__ R, int g, int hq,
                                                         int hkv, int64_t nb, int64_t n_tiles,
                                                         float half_beta, int64_t n_ct,
                                                         int64_t n_rt, int64_t n_work) {
  using Mo = Moments<D>;
  constexpr int SIG_STEPS = Mo::SIG_STEPS;
  constexpr int MU_STEPS = D / 16;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int wr = wave / 2, wc = wave % 2;
  // Work items run column tile fastest, then row tile, then KV head, and
  // consecutive items go to one XCD (workgroup i runs on XCD i % 8): the
  // column tiles of a row tile read the same moment rows at about the same
  // time, from that XCD's L2.
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t wi = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (wi >= n_work) return;
  const int64_t ct = wi % n_ct, rt = (wi / n_ct) % n_rt, bkv = wi / (n_ct * n_rt);
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rows_total = n_tiles * g;
  const int64_t rt0 = rt * kScoreRows, c0 = ct * kScoreCols;
  const int64_t j_hi = min(n_tiles - 1, (rt0 + kScoreRows - 1) / g);
  if (c0 >= min(nb, j_hi)) return;               // no block before any tile of this row tile

  const int64_t r_base = rt0 + 64 * wr;
  const int64_t c = c0 + 32 * wc + ln;
  const bool c_ok = c < nb;
  // operand rows past the end read row 0 / block 0 (their results are never
  // stored), so every load is unconditional and stays in flight
  const float* arow[2];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs) {
    const int64_t r = r_base + 32 * rs + ln;
    arow[rs] = Am + (bkv * Mo::STEPS * rows_total + (r < rows_total ? r : 0)) * 16 + 8 * h;
  }
  const int64_t step_stride = rows_total * 16;
  const float* sig_c = sigma + (bkv * nb + (c_ok ? c : 0)) * int64_t(D) * D + 8 * h;
  const float* mu_c = mu + (bkv * nb + (c_ok ? c : 0)) * int64_t(D) + 8 * h;

  auto ld8 = [](const float* p) {
    const floatx4 a = *reinterpret_cast<const floatx4*>(p);
    const floatx4 b2 = *reinterpret_cast<const floatx4*>(p + 4);
    floatx8 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[e + 4] = b2[e];
    }
    return v;
  };
  // Contraction step st of the Sigma part covers packed tile u = st / 64,
  // its row i = (st / 2) % 32 and half j0 = 16 (st % 2): 16 st + 8h on the
  // packed-moment side; on the Sigma side row 32 mt + i, columns 32 nt + j0
  // + 8h, with (mt, nt) the u-th upper tile (scalar arithmetic: u >= T_m,
  // T_m = m MT - m (m - 1) / 2, for each m counts one more mt).
  auto sig_off = [](int st) {
    const int u = st >> 6, i = (st >> 1) & 31, j0 = (st & 1) << 4;
    int mt = 0;
#pragma unroll
    for (int m = 1; m < Mo::MT; ++m) mt += u >= m * Mo::MT - m * (m - 1) / 2 ? 1 : 0;
    const int nt = u - (mt * Mo::MT - mt * (mt - 1) / 2) + mt;
    return (32 * mt + i) * D + 32 * nt + j0;
  };

  floatx16 acc[2];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rs][i] = 0.f;

  floatx8 fa[kScoreStages][2], fb[kScoreStages];
  auto load_step = [&](int st, int slot) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) fa[slot][rs] = ld8(arow[rs] + st * step_stride);
    fb[slot] = ld8(sig_c + sig_off(st));
  };
#pragma unroll
  for (int q = 0; q < kScoreStages; ++q) load_step(q, q);
  for (int st0 = 0; st0 < SIG_STEPS; st0 += kScoreStages) {
#pragma unroll
    for (int q = 0; q < kScoreStages; ++q) {
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) acc[rs] = mma16(fa[q][rs], fb[q], acc[rs]);
      // the last stages re-read step 0 instead of running past the end
      const int nx = st0 + q + kScoreStages;
      load_step(nx < SIG_STEPS ? nx : 0, q);
    }
  }
  // (beta/2) <Sigma_c, M_j>, then + s_j . mu_c
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rs][i] *= half_beta;
#pragma unroll
  for (int s2 = 0; s2 < MU_STEPS; ++s2) {
    const floatx8 mb = ld8(mu_c + 16 * s2);
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
      acc[rs] = mma16(ld8(arow[rs] + (SIG_STEPS + s2) * step_stride), mb, acc[rs]);
  }

  // acc lane (ln, h): rows 8a + 4h + b of the 32-row group, block c
  if (!c_ok) return;
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t r = r_base + 32 * rs + 8 * (i / 4) + 4 * h + i % 4;
      if (r >= rows_total) continue;
      const int64_t jt = r / g, jg = r % g;
      if (c >= min(nb, jt)) continue;
      R[((b * hq + kv * g + jg) * n_tiles + jt) * nb + c] = acc[rs][i];
    }
}

// --------------------------------------------------------------- tile top-k --
//
// One wave per tile: k rounds, each the largest score strictly after the
// previous pick in the order (score descending, block ascending), so ties go
// to the lower block; then the picks in ascending block order.
template <int KMAX>
__global__ __launch_bounds__(256) void tile_topk_kernel(const float* __restrict__ R,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ kth, int64_t rows,
                                                        int64_t n_tiles, int64_t nb, int k) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t ro = int64_t(blockIdx.x) * 4 + wave;
  if (ro >= rows) return;
  const int64_t j = ro % n_tiles;
  const int64_t C = min(nb, j);
  const float* r = R + ro * nb;
  constexpr int kNone = 0x7FFFFFFF;
  float pv = __builtin_inff();
  int pi = -1;
  int sel[KMAX];
  float r_k = -__builtin_inff(), r_k1 = -__builtin_inff();
  const int rounds = k + (kth != nullptr ? 1 : 0);
  for (int rd = 0; rd < rounds; ++rd) {
    float bv = -__builtin_inff();
    int bi = kNone;
    for (int64_t cc = lane; cc < C; cc += 64) {
      const float v = r[cc];
      const int ci = int(cc);
      const bool after = v < pv || (v == pv && ci > pi);
      const bool better = v > bv || (v == bv && ci < bi);
      if (after && better) {
        bv = v;
        bi = ci;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = wave_shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (rd < k) {
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i == rd) sel[i] = bi == kNone ? -1 : bi;
      if (rd == k - 1 && bi != kNone) r_k = bv;
    } else if (bi != kNone) {
      r_k1 = bv;
    }
    if (bi == kNone) {
      for (int rr = rd + 1; rr < k; ++rr) {
#pragma unroll
        for (int i = 0; i < KMAX; ++i)
          if (i == rr) sel[i] = -1;
      }
      break;
    }
    pv = bv;
    pi = bi;
  }
  if (k > 0) {
    // the picks are distinct blocks then -1s: rank = #picks with a smaller
    // (unsigned) value, so -1 goes last
    int mine = -1;
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i == lane) mine = sel[i];
    if (lane < k) {
      int rank = 0;
#pragma unroll
      for (int i = 0; i < KMAX; ++i)
        if (i < k) {
          const unsigned a = unsigned(sel[i]), m = unsigned(mine);
          rank += (a < m || (a == m && i < lane)) ? 1 : 0;
        }
      idx[ro * k + rank] = mine;
    }
  }
  if (kth != nullptr && lane == 0) {
    kth[ro * 2] = r_k;
    kth[ro * 2 + 1] = r_k1;
  }
}

template <bool F32, int D>
hipError_t launch_moments(const Shape& s, const void* Q, float* Am, int64_t n_tiles, hipStream_t st) {
  using In = typename AT<F32, D>::In;
  hipLaunchKernelGGL((tile_moments_kernel<F32, D>), dim3(unsigned(n_tiles), unsigned(s.b * s.hq)),
                     dim3(256), 0, st, static_cast<const In*>(Q), Am, s.n, s.g, s.hq, s.hkv, s.B,
                     n_tiles);
  return hipGetLastError();
}

template <int KMAX>
hipError_t launch_tile_topk(const Shape& s, const float* R, int32_t* idx, float* kth,
                            int64_t n_tiles, hipStream_t st) {
  const int64_t rows = int64_t(s.b) * s.hq * n_tiles;
  hipLaunchKernelGGL((tile_topk_kernel<KMAX>), dim3(unsigned((rows + 3) / 4)), dim3(256), 0, st, R,
                     idx, kth, rows, n_tiles, s.nb, s.k);
  return hipGetLastError();
}

size_t moments_bytes(const Shape& s) {
  const int64_t per = s.d == 64 ? Moments<64>::P : Moments<128>::P;
  return align_up(size_t(s.b) * s.hq * size_t(tile_count(s)) * size_t(per) * 4);
}

}  // namespace

int64_t tile_count(const Shape& s) { return (s.n + s.B - 1) / s.B; }

size_t route_tiles_workspace_bytes(const Shape& s) {
  return moments_bytes(s) +
         align_up(size_t(s.b) * s.hq * size_t(tile_count(s)) * size_t(std::max<int64_t>(s.nb, 1)) * 4);
}

hipError_t launch_route_tiles(const Shape& s, const void* Q, const float* mu, const float* sigma,
                              int32_t* idx, float* kth, void* ws, hipStream_t st) {
  const int64_t n_tiles = tile_count(s);
  float* Am = static_cast<float*>(ws);
  float* R = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + moments_bytes(s));
  hipError_t e = hipSuccess;
  if (s.nb > 0) {
    e = s.in_bf16 ? (s.d == 64 ? launch_moments<false, 64>(s, Q, Am, n_tiles, st)
                               : launch_moments<false, 128>(s, Q, Am, n_tiles, st))
                  : (s.d == 64 ? launch_moments<true, 64>(s, Q, Am, n_tiles, st)
                               : launch_moments<true, 128>(s, Q, Am, n_tiles, st));
    if (e != hipSuccess) return e;
    const int64_t n_ct = (s.nb + kScoreCols - 1) / kScoreCols;
    const int64_t n_rt = (n_tiles * s.g + kScoreRows - 1) / kScoreRows;
    const int64_t n_work = n_ct * n_rt * s.b * s.hkv;
    const dim3 grid(unsigned((n_work + 7) / 8 * 8));   // a multiple of the 8 XCDs
    const float hb = 0.5f * s.beta;
    if (s.d == 64)
      hipLaunchKernelGGL((tile_score_kernel<64>), grid, dim3(256), 0, st, Am, sigma, mu, R, s.g,
                         s.hq, s.hkv, s.nb, n_tiles, hb, n_ct, n_rt, n_work);
    else
      hipLaunchKernelGGL((tile_score_kernel<128>), grid, dim3(256), 0, st, Am, sigma, mu, R, s.g,
                         s.hq, s.hkv, s.nb, n_tiles, hb, n_ct, n_rt, n_work);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (s.k <= 8) return launch_tile_topk<8>(s, R, idx, kth, n_tiles, st);
  if (s.k <= 16) return launch_tile_topk<16>(s, R, idx, kth, n_tiles, st);
  return launch_tile_topk<32>(s, R, idx, kth, n_tiles, st);
}

}  // namespace ssa
