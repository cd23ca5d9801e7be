// Routing scores and top-k block selection (prefill).
//
// Write-up "Subquadratic Sparse Attention (SSA)", section "The idea in one
// screen" (second-cumulant score r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q)
// and introduction step (i) (keep a small content-dependent set of blocks).
//
// Formulation.  With T_c the upper triangle of (beta/2) Sigma_c with doubled
// off-diagonal (T_ij = beta Sigma_ij for i < j, (beta/2) Sigma_ii on the
// diagonal, 0 below), q^T T_c q = (beta/2) q^T Sigma_c q for symmetric Sigma_c,
// so   r_c(q) = sum_j q_j (P_j + mu_cj)   with   P = q T_c.
// For a tile of query rows that share a KV head, P = Q_tile T_c is a dense
// contraction on MFMA; its triangular shape lets 32-column tile mt skip
// every 16-row chunk below the diagonal (20 of 32 chunks computed at d=128).
// The row-dot with q and the running top-k run on the vector ALUs in the
// MFMA's own register layout (see frag_k in ssa_common.hpp), so Q is read
// once per tile and stays in registers for the whole sweep over blocks.
//
// Precision.  Q is bfloat16, which float16 holds exactly in its normal
// range, so Q enters the float16 MFMA after an exact power-of-two scaling per
// (sequence, KV head) that brings its largest |q| into [2^14, 2^15).  T_c (float32) is scaled per block by a power
// of two that brings its largest entry to [2^14, 2^15) and split into a high
// and a low float16 part; both are contracted with float32 accumulation, so
// scores carry ~2^-22 relative error instead of the 2^-11 of a single float16
// rounding -- enough to reproduce the exact top-k except where two scores are
// nearly tied.  The row-dot reads q from the same float16 registers (mixed
// float16 x float32 fused multiply-adds, no conversions).  float32 inputs use
// the float32 MFMA.
//
// Work split.  A workgroup of 8 waves owns 512 consecutive query rows of one
// (sequence, KV head), ordered (token, group member), so one Sigma_c tile in
// LDS serves 512 rows: 64 rows per wave, two 32-row MFMA tiles.  Blocks are
// streamed in order c = 0, 1, ... through a double-buffered LDS copy of a
// prepared fragment image; ties in the top-k therefore keep the lower block.
// Workgroups are issued longest (most routable blocks) first.
#include <algorithm>

#include "kv_chunks.hpp"
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kRouteThreads = 512;   // 8 waves, two per SIMD
constexpr int kRouteRows = 512;      // 64 query rows per wave
constexpr int kFragBytes = 2048;   // one 32x16 operand fragment: 64 lanes x 32 bytes

template <int D>
struct RouteLayout {
  static constexpr int MT = D / 32;                 // 32-wide output tiles
  static constexpr int NS = D / 16;                 // 16-wide contraction chunks
  static constexpr int NF = MT * (MT + 1);          // chunks on or above the diagonal
  static constexpr int MU_OFF = NF * kFragBytes;
  static constexpr int MU_BYTES = 2 * MT * 16 * 4;  // mu in accumulator order, both lane halves
  static constexpr int SCALE_OFF = MU_OFF + MU_BYTES;  // float: 2^e, T_c and mu are stored times 2^-e
  static constexpr int BLOCK_BYTES = (SCALE_OFF + 16 + 255) / 256 * 256;
  // LDS copy of one image, whole 1 KB DMA rows (the last row reads past the image)
  static constexpr int DMA_ROWS = (BLOCK_BYTES + 1023) / 1024;
  static constexpr int LDS_BYTES = DMA_ROWS * 1024;
  __host__ __device__ static constexpr int frag(int mt, int s) { return mt * (mt + 1) + s; }
};

// Exponent eq with max|q| * 2^-eq in [2^14, 2^15) for the largest |q| given as
// bfloat16 bits (0 for zero, infinite or NaN maxima): the float16 scale of Q.
__device__ __forceinline__ int query_exponent(uint32_t qmax_bits) {
  const float v = bf16_bits_to_f32(qmax_bits & 0x7FFFu);
  if (!(v > 0.f) || !(v < __builtin_inff())) return 0;
  int E = 0;
  (void)frexpf(v, &E);   // v < 2^E
  return E - 15;
}

// Prepared image of one block (workspace): for every output tile mt and
// chunk s <= 2mt+1, lane (m, h) of the fragment holds T_c[frag_k(s,h,e)][32mt+m]
// for e = 0..7 -- times 2^-e as float16 hi (bytes 0..1023) and lo
// (1024..2047), or float32 (e = 0); then mu_c times 2^-(e + eq) in accumulator
// order: [h][mt][4a+b] = mu_c[32mt + 8a + 4h + b], where 2^-eq is the float16
// scale of the KV head's query rows; then the float 2^e.
template <bool F32, int D>
__global__ __launch_bounds__(256) void route_prep_kernel(const float* __restrict__ mu,
                                                          const float* __restrict__ sigma,
                                                          const uint32_t* __restrict__ qmax,
                                                          uint8_t* __restrict__ prep, int64_t nb,
                                                          float beta) {
  using Lay = RouteLayout<D>;
  const int64_t blk = int64_t(blockIdx.y) * nb + blockIdx.x;
  const float* S = sigma + blk * int64_t(D) * D;
  const float* M = mu + blk * D;
  uint8_t* out = prep + blk * Lay::BLOCK_BYTES;
  const float half_beta = 0.5f * beta;
  // float16 parts: scale by 2^-e so that the largest |T_ij| lies in [2^14, 2^15)
  float scale = 1.f, unscale = 1.f;
  if constexpr (!F32) {
    __shared__ float red[4];
    float mx = 0.f;
    for (int w = threadIdx.x; w < D * D; w += blockDim.x) {
      const int i = w / D, j = w % D;
      if (i <= j) mx = fmaxf(mx, fabsf((i < j ? beta : half_beta) * S[w]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, wave_shfl_xor(mx, o));
    if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (mx > 0.f && mx == mx && mx < __builtin_inff()) {
      const int e = ilogbf(mx) - 14;
      scale = ldexpf(1.f, -e);
      unscale = ldexpf(1.f, e);
    }
  }
  for (int w = threadIdx.x; w < Lay::NF * 64; w += blockDim.x) {
    const int f = w / 64, lane = w % 64, m = lane % 32, h = lane / 32;
    int mt = 0;
    while ((mt + 1) * (mt + 2) <= f) ++mt;
    const int s = f - mt * (mt + 1);
    const int j = 32 * mt + m;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = frag_k(s, h, e);
      const float sij = S[i * D + j];
      x[e] = i < j ? beta * sij : (i == j ? half_beta * sij : 0.f);
    }
    if constexpr (F32) {
      floatx8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = x[e];
      *reinterpret_cast<floatx8*>(out + f * kFragBytes + lane * 32) = v;
    } else {
      f16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = x[e] * scale;
        const _Float16 hv = static_cast<_Float16>(v);
        hi[e] = hv;
        lo[e] = static_cast<_Float16>(v - static_cast<float>(hv));
      }
      *reinterpret_cast<f16x8*>(out + f * kFragBytes + lane * 16) = hi;
      *reinterpret_cast<f16x8*>(out + f * kFragBytes + 1024 + lane * 16) = lo;
    }
  }
  const float mscale = F32 ? scale : scale * ldexpf(1.f, -query_exponent(qmax[blockIdx.y]));
  for (int w = threadIdx.x; w < 2 * Lay::MT * 16; w += blockDim.x) {
    const int h = w / (Lay::MT * 16), mt = (w / 16) % Lay::MT, i = w % 16;
    reinterpret_cast<float*>(out + Lay::MU_OFF)[w] = M[32 * mt + 8 * (i / 4) + 4 * h + (i % 4)] * mscale;
  }
  if (threadIdx.x == 0) *reinterpret_cast<float*>(out + Lay::SCALE_OFF) = unscale;
}

template <bool F32>
struct QFrag;
template <>
struct QFrag<false> {
  using T = f16x8;      // bfloat16 rows held as float16 (exact in the normal range)
  using In = bf16_t;
  __device__ static float elem(const T& v, int e) { return static_cast<float>(v[e]); }
};
template <>
struct QFrag<true> {
  using T = floatx8;
  using In = float;
  __device__ static float elem(const T& v, int e) { return v[e]; }
};

// Load the B-operand fragment of chunk s for one query row (lane half h).
template <bool F32>
__device__ __forceinline__ typename QFrag<F32>::T load_q_frag(const typename QFrag<F32>::In* row,
                                                              int s, int h, bool valid) {
  typename QFrag<F32>::T v;
  if constexpr (F32) {
    floatx4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
    if (valid) {
      a = *reinterpret_cast<const floatx4*>(row + 16 * s + 4 * h);
      b = *reinterpret_cast<const floatx4*>(row + 16 * s + 8 + 4 * h);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[e + 4] = b[e];
    }
  }
  return v;
}

// The bfloat16 bits of the same fragment (converted to float16 by the caller).
__device__ __forceinline__ u32x4 load_q_bits(const bf16_t* row, int s, int h, bool valid) {
  u32x2 a = {0u, 0u}, b = a;
  if (valid) {
    a = *reinterpret_cast<const u32x2*>(row + 16 * s + 4 * h);
    b = *reinterpret_cast<const u32x2*>(row + 16 * s + 8 + 4 * h);
  }
  return u32x4{a[0], a[1], b[0], b[1]};
}

template <bool F32, int D, int KMAX>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const typename QFrag<F32>::In* __restrict__ Q, const uint8_t* __restrict__ prep,
    const uint32_t* __restrict__ qmax, int32_t* __restrict__ idx, float* __restrict__ kth,
    int64_t n, int g, int hq, int hkv, int B, int64_t nb, int k, int64_t n_tiles,
    int64_t n_bkv) {
  using Lay = RouteLayout<D>;
  using QT = typename QFrag<F32>::T;
  constexpr int MT = Lay::MT, NS = Lay::NS, BYTES = Lay::BLOCK_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * Lay::LDS_BYTES];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t wid = blockIdx.x;
  const int64_t bkv = wid % n_bkv;
  const int64_t tile = n_tiles - 1 - wid / n_bkv;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rows_total = n * g;
  const int64_t rho0 = tile * kRouteRows;

  // query fragments of this lane's two 32-row tiles.  bfloat16 rows become
  // float16 (exact in the normal range) after scaling by 2^-eq, which brings
  // the KV head's largest |q| into [2^14, 2^15); the images' mu carry the same
  // factor.
  QT bq[2][NS];
  float qsc = 1.f, qsq = 1.f;   // 2^-eq and 2^(2 eq)
  if constexpr (!F32) {
    const int eq = query_exponent(qmax[bkv]);
    qsc = ldexpf(1.f, -eq);
    qsq = ldexpf(1.f, 2 * eq);
  }
  {
    const int64_t rows_of[2] = {rho0 + 64 * wave + ln, rho0 + 64 * wave + 32 + ln};
    if constexpr (F32) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t rho = rows_of[nt];
        const bool valid = rho < rows_total;
        const int64_t t = valid ? rho / g : 0, jg = valid ? rho % g : 0;
        const auto* row = Q + (((b * hq + kv * g + jg) * n) + t) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) bq[nt][s] = load_q_frag<F32>(row, s, h, valid);
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t rho = rows_of[nt];
        const bool valid = rho < rows_total;
        const int64_t t = valid ? rho / g : 0, jg = valid ? rho % g : 0;
        const auto* row = Q + (((b * hq + kv * g + jg) * n) + t) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const u32x4 raw = load_q_bits(row, s, h, valid);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t u = raw[w];
            bq[nt][s][2 * w] = static_cast<_Float16>(bf16_bits_to_f32(u & 0xFFFFu) * qsc);
            bq[nt][s][2 * w + 1] = static_cast<_Float16>(bf16_bits_to_f32(u >> 16) * qsc);
          }
        }
      }
    }
  }
  // the row this lane scores and ranks
  const int64_t my_rho = rho0 + 64 * wave + 32 * h + ln;
  const bool my_valid = my_rho < rows_total;
  const int64_t my_t = my_valid ? my_rho / g : 0;
  const int64_t my_C = my_valid ? min(nb, (my_t + 1) / B) : 0;
  const int64_t t_max = min(n - 1, (rho0 + kRouteRows - 1) / g);
  const int64_t C_wg = min(nb, (t_max + 1) / B);

  float ls[KMAX + 1];
  int li[KMAX + 1];
#pragma unroll
  for (int i = 0; i <= KMAX; ++i) {
    ls[i] = -__builtin_inff();
    li[i] = -1;
  }

  // block c's image -> an LDS buffer by direct global->LDS loads (1 KB per
  // wave instruction); the barrier that ends a block's iteration waits for them
  const uint8_t* src_base = prep + bkv * nb * int64_t(BYTES);
  auto stage = [&](int64_t c, uint8_t* dst) {
    const uint8_t* src = src_base + c * BYTES;
    for (int r = wave; r < Lay::DMA_ROWS; r += kRouteThreads / 64)
      __builtin_amdgcn_global_load_lds(src + r * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void*)(dst + r * 1024),
                                       16, 0, 0);
  };
  if (C_wg > 0) stage(0, lds);
  __syncthreads();

  // Hand-scheduled sweep.  Output tiles run from the widest (mt = MT-1, all
  // 2MT chunks) down to mt = 0, two accumulator sets alternating, and every
  // MFMA call is followed by a fixed share of vector work that depends only on
  // earlier tiles: the row-dot of the previous tile (lane (ln, h) holds
  // P_j + mu_j for j = 32mt + 8a + 4h + b, P's column = this lane's query
  // row), and, during the widest tile, the finish of the previous block --
  // the dot of its last tile, the lane-half reduction and the running top-k
  // insert.  sched_barrier pins that interleave, so the matrix cores stay fed
  // while the vector units work, whatever the other wave on the SIMD does.
  // Operand fragments are read from LDS two steps ahead; each tile's first
  // MFMA takes mu as its accumulator input.
  constexpr int PARTS = F32 ? 1 : 2;               // float16: high and low part of T
  constexpr int NFR = Lay::NF * PARTS;             // fragment reads per block
  constexpr int NDOT = 32;                         // row-dot FMAs per tile (2 tiles x 16)
  floatx16 acc[2][2];                              // [set][nt]; tile mt uses set (MT-1-mt)&1
#pragma unroll
  for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[st2][nt][j] = 0.f;
  float pt[2] = {0.f, 0.f};
  float sc_new = -__builtin_inff();   // the score being inserted
  float sc_ins = -__builtin_inff();   // the entry carried down the list
  int ci_ins = -1;

  // fragment k (= chunk-in-pair * PARTS + part) of chunk pair gp of tile mt
  auto read_frag = [&](const uint8_t* L, int mt, int gp, int k) {
    const int sidx = 2 * gp + k / PARTS, part = k % PARTS;
    const uint8_t* F = L + Lay::frag(mt, sidx) * kFragBytes;
    if constexpr (F32)
      return *reinterpret_cast<const QT*>(F + lane * 32);
    else
      return *reinterpret_cast<const QT*>(F + part * 1024 + lane * 16);
  };
  auto read_mu = [&](const uint8_t* L, int mt) {
    floatx16 m;
    const floatx4* p = reinterpret_cast<const floatx4*>(L + Lay::MU_OFF + mt * 64) + h * (MT * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const floatx4 v = p[q];
#pragma unroll
      for (int e = 0; e < 4; ++e) m[4 * q + e] = v[e];
    }
    return m;
  };
  auto dot_item = [&](int set, int mt, int i) {
    const int nt = i / 16, j = i % 16, a = j / 4, bb = j % 4;
    pt[nt] = fmaf(acc[set][nt][j], QFrag<F32>::elem(bq[nt][2 * mt + (a >> 1)], 4 * (a & 1) + bb),
                  pt[nt]);
  };
  // both lane halves combined: the score of this lane's row for block cb,
  // times cb's image scale (blk_scale; the wave's common 2^(2 eq) stays out)
  float blk_scale = 1.f;
  auto reduce = [&](int64_t cb) {
    const float p0 = pt[0] + wave_shfl_xor(pt[0], 32);
    const float p1 = pt[1] + wave_shfl_xor(pt[1], 32);
    pt[0] = pt[1] = 0.f;
    sc_new = (cb >= 0 && cb < my_C) ? (h ? p1 : p0) * blk_scale : -__builtin_inff();
    sc_ins = sc_new;
    ci_ins = int(cb);
  };
  // one step of the running top-(k+1) insertion.  The list is sorted by
  // (score descending, block ascending) and blocks arrive in ascending order,
  // so the new block goes after every entry with a score >= its own, and
  // every entry from that slot on moves down one: the test is the NEW score
  // against the slot (true from the insertion slot on, the list being
  // sorted), never the carried entry's -- a displaced entry compared with an
  // equal later one would otherwise slip past it.  NaN is never inserted.
  auto insert_step = [&](int i) {
    const bool gt = sc_new > ls[i];
    const float ts = ls[i];
    const int ti = li[i];
    ls[i] = gt ? sc_ins : ts;
    li[i] = gt ? ci_ins : ti;
    sc_ins = gt ? ts : sc_ins;
    ci_ins = gt ? ti : ci_ins;
  };

  auto sweep = [&](int64_t c, const uint8_t* L) {
    const float scale_c = *reinterpret_cast<const float*>(L + Lay::SCALE_OFF);
    // the query fragments are loop-invariant; an empty register constraint
    // keeps the compiler from hoisting float32 copies of them (for the
    // row-dot) out of the loop, which would need 128 more registers -- the
    // row-dot reads the float16 fragments with mixed-precision FMAs instead
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) asm volatile("" : "+v"(bq[nt][s2]));
    // Operands move in chunk pairs (2 PARTS fragments): the reads of pair
    // p+1 are issued after the first MFMA of pair p, so that MFMA's
    // wait covers pair p alone (while a direct-to-LDS copy is in flight the
    // compiler can only wait for all outstanding LDS reads) and pair p+1 has
    // the rest of pair p to arrive.  Tile mt has mt+1 pairs.
    constexpr int PK = 2 * PARTS;                  // fragments per pair
    QT fr[2][PK];
#pragma unroll
    for (int k2 = 0; k2 < PK; ++k2) fr[0][k2] = read_frag(L, MT - 1, 0, k2);
    floatx16 mu_next = read_mu(L, MT - 1);
    int pslot = 0;                                 // slot of the current pair
#pragma unroll
    for (int mt = MT - 1; mt >= 0; --mt) {
      const int set = (MT - 1 - mt) & 1, pset = set ^ 1;
      const floatx16 mu_t = mu_next;
      constexpr int kCallsPerPair = PK * 2;
      const int calls = (mt + 1) * kCallsPerPair;
      // vector work of this tile: the previous tile's dot (for the widest
      // tile: the previous block's last tile), then, for the widest tile,
      // the reduction and the KMAX+1 insert steps
      const int nwork = NDOT + (mt == MT - 1 ? 1 + KMAX + 1 : 0);
#pragma unroll
      for (int i = 0; i < calls; ++i) {
        const int gp = i / kCallsPerPair, k2 = (i / 2) % PK, nt = i % 2;
        const int sidx = 2 * gp + k2 / PARTS;
        const int slot = (pslot + gp) & 1;
        const floatx16 cin = (i < 2) ? mu_t : acc[set][nt];
        acc[set][nt] = mma16(fr[slot][k2], bq[nt][sidx], cin);
        if (i % kCallsPerPair == 1) {
          // next pair: later in this tile, else the first of the next tile
          // (issued in the second call's slot: the scheduler may lift a read
          // above its own call's MFMA, but not above the previous call's)
          if (gp < mt) {
#pragma unroll
            for (int q2 = 0; q2 < PK; ++q2) fr[slot ^ 1][q2] = read_frag(L, mt, gp + 1, q2);
          } else if (mt > 0) {
#pragma unroll
            for (int q2 = 0; q2 < PK; ++q2) fr[slot ^ 1][q2] = read_frag(L, mt - 1, 0, q2);
            mu_next = read_mu(L, mt - 1);
          }
        }
#pragma unroll
        for (int w = i * nwork / calls; w < (i + 1) * nwork / calls; ++w) {
          if (w < NDOT) {
            dot_item(pset, mt == MT - 1 ? 0 : mt + 1, w);
          } else if (w == NDOT) {
            reduce(c - 1);
          } else {
            insert_step(w - NDOT - 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      pslot = (pslot + mt + 1) & 1;
    }
    blk_scale = scale_c;   // the next reduction is this block's
  };
  for (int64_t c = 0; c < C_wg; ++c) {
    if (c + 1 < C_wg) stage(c + 1, lds + ((c + 1) & 1) * Lay::LDS_BYTES);
    sweep(c, lds + (c & 1) * Lay::LDS_BYTES);
    __syncthreads();
  }
  // the last block's final tile, reduction and insert
  if (C_wg > 0) {
#pragma unroll
    for (int w = 0; w < NDOT; ++w) dot_item((MT - 1) & 1, 0, w);
    reduce(C_wg - 1);
#pragma unroll
    for (int i = 0; i <= KMAX; ++i) insert_step(i);
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
      if (i == k - 1) r_k = ls[i] * qsq;
      if (i == k) r_k1 = ls[i] * qsq;
    }
    kth[orow * 2] = r_k;
    kth[orow * 2 + 1] = r_k1;
  }
}

template <bool F32, int D, int KMAX>
hipError_t launch_route_t(const Shape& s, const void* Q, const float* mu, const float* sigma,
                          int32_t* idx, float* kth, void* ws, hipStream_t st) {
  using Lay = RouteLayout<D>;
  const int64_t n_bkv = int64_t(s.b) * s.hkv;
  uint8_t* prep = static_cast<uint8_t*>(ws);
  // per (sequence, KV head): the largest |q| of its query rows (bfloat16
  // bits), which sets the float16 scale of Q (the group's rows are contiguous)
  uint32_t* qmax =
      reinterpret_cast<uint32_t*>(prep + align_up(size_t(n_bkv * s.nb) * Lay::BLOCK_BYTES + 1024));
  if constexpr (!F32) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<int32_t*>(qmax),
                       n_bkv, 0);
    const int64_t per_group = int64_t(s.g) * s.n * D;
    const unsigned gx = unsigned(std::min<int64_t>((per_group / 8 + 255) / 256, 64));
    hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bkv)), dim3(256), 0, st,
                       static_cast<const bf16_t*>(Q), qmax, per_group);
  }
  if (s.nb > 0) {
    hipLaunchKernelGGL((route_prep_kernel<F32, D>), dim3(unsigned(s.nb), unsigned(n_bkv)),
                       dim3(256), 0, st, mu, sigma, qmax, prep, s.nb, s.beta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n_tiles = (s.n * s.g + kRouteRows - 1) / kRouteRows;
  auto kern = route_topk_kernel<F32, D, KMAX>;
  constexpr size_t shmem = 0;   // the kernel's LDS buffers are static
  using In = typename QFrag<F32>::In;
  hipLaunchKernelGGL(kern, dim3(unsigned(n_tiles * n_bkv)), dim3(kRouteThreads), shmem, st,
                     static_cast<const In*>(Q), prep, qmax, idx, kth, s.n, s.g, s.hq, s.hkv, s.B,
                     s.nb, s.k, n_tiles, n_bkv);
  return hipGetLastError();
}

template <bool F32, int D>
hipError_t launch_route_d(const Shape& s, const void* Q, const float* mu, const float* sigma,
                          int32_t* idx, float* kth, void* ws, hipStream_t st) {
  if (s.k <= 8) return launch_route_t<F32, D, 8>(s, Q, mu, sigma, idx, kth, ws, st);
  if (s.k <= 16) return launch_route_t<F32, D, 16>(s, Q, mu, sigma, idx, kth, ws, st);
  return launch_route_t<F32, D, 32>(s, Q, mu, sigma, idx, kth, ws, st);
}

}  // namespace

size_t route_workspace_bytes(const Shape& s) {
  const size_t per = s.d == 64 ? RouteLayout<64>::BLOCK_BYTES : RouteLayout<128>::BLOCK_BYTES;
  // + 1 KB: the DMA of the last image reads up to one row past its end; then
  // the largest |q| of every (sequence, KV head)
  return align_up(size_t(s.b) * s.hkv * size_t(s.nb) * per + 1024) +
         align_up(size_t(s.b) * s.hkv * 4);
}

hipError_t launch_route_topk(const Shape& s, const void* Q, const float* mu, const float* sigma,
                             int32_t* idx, float* kth, void* ws, hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch_route_d<false, 64>(s, Q, mu, sigma, idx, kth, ws, st)
                     : launch_route_d<false, 128>(s, Q, mu, sigma, idx, kth, ws, st);
  return s.d == 64 ? launch_route_d<true, 64>(s, Q, mu, sigma, idx, kth, ws, st)
                   : launch_route_d<true, 128>(s, Q, mu, sigma, idx, kth, ws, st);
}

}  // namespace ssa
