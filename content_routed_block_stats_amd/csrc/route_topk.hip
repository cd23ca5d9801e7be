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
// Diagonal shift (bfloat16 inputs).  A vector D, common to all blocks of a
// (sequence, KV head), is subtracted from every T_c's diagonal: the scores of
// one query all move by q^T diag(D) q, so the ranking is unchanged, and
// T'_c = T_c - diag(D) has smaller entries than T_c (the blocks' variances
// are alike), which is what the float16 rounding below is relative to.  D is
// the mean of the first blocks' (beta/2) diagonals; k-th scores reported on
// request add q^T diag(D) q back.
//
// Precision and the passes (bfloat16 inputs).  Q is bfloat16, exact in
// float16's normal range after one power-of-two scaling per (sequence, KV
// head); T'_c is scaled per block by a power of two that brings its largest
// entry into [2^14, 2^15) and split into float16 hi + lo.
//  * Single pass: every row is scored against every routable block with the
//    hi part only (half the MFMA work of hi + lo) and keeps a running list of
//    its best KMAX+5 (KMAX: k rounded up to 8, 16 or 32) as packed 32-bit
//    keys.  Dropping the rest of T'_c moves a
//    score by q^T sym(L_c) q, L_c = T'_c - hi_c, at most lam ||q||^2 with lam
//    a bound on every ||sym(L_c)||_2 (the prep kernel derives it from tr A^4
//    on the float16 MFMA, with margins for its own rounding); float32
//    accumulation adds at most about 2^-17 (G ||q||^2 + nu ||q||) (G bounds
//    |q|^T |T'_c| |q| / ||q||^2, nu = max ||mu_c||); a packed key stands for
//    the range of scores that share its top bits.  With e the sum of these
//    bounds (the accumulated part taken 1.25 times), a listed block whose
//    range lies more than 2e above the (k+1)-th key's is certainly in the
//    exact top-k, one more than 2e below the k-th key's certainly out.  A row
//    whose k best keys are all certainly in is done (about 83% of rows at
//    the 128K GQA workload).
//  * Block-major rescoring: for the other rows only the blocks in between
//    (typically 2-3 per row) need exact scores.  They are grouped by block,
//    and one workgroup per block stages its hi + lo image once and rescores
//    every (row, block) pair of it with the exact pass's arithmetic; a final
//    kernel merges the certain blocks with the best rescored ones.  Rows
//    whose undecided range may reach past the list (a few per KV head) are
//    rescored on every block the same way, then take a wave top-k.
//  * Exact pass: rows with a non-finite key, or beyond the capacity of the
//    structures above, are rescored against every routable block with
//    hi + lo (~2^-22 relative error), one row per lane.
// All three reproduce the exact pass's selection, except where two scores
// are within about 1e-6 relative.
// Requests for the k-th scores run the exact pass on every row.  float32
// inputs use the float32 MFMA in the exact pass on every row.
//
// Work split.  A workgroup of 8 waves owns 512 query rows of one (sequence,
// KV head), ordered (token, group member), so one block image in LDS serves
// 512 rows: 64 rows per wave, two 32-row MFMA tiles.  Blocks are streamed in
// order c = 0, 1, ... through a double- (exact pass) or triple-buffered
// (single pass) LDS copy of a prepared fragment image; the top-k lists are sorted by (score descending, block
// ascending).  Workgroups are issued longest (most routable blocks) first.
#include <algorithm>

#include "kv_chunks.hpp"
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kRouteThreads = 512;   // 8 waves, two per SIMD
constexpr int kRouteRows = 512;      // 64 query rows per wave
constexpr int kFragBytes = 2048;     // one 32x16 operand fragment: 64 lanes x 32 bytes
constexpr int kShiftBlocks = 8;      // blocks whose diagonals average into D
constexpr int kMaxKeyBits = 16;      // single pass: packed keys hold a block index of <= 16 bits
constexpr int kExtra = 4;            // single pass: list slots kept beyond the (k+1)-th
constexpr int kRecCap = 128;         // single pass: rescore records per 512-row tile
constexpr int kFullCap = 256;        // single pass: rows rescored on every block, per KV head

// KMAX of the kernels built for top_k = k, and the single pass's list length
__host__ __device__ constexpr int route_kmax(int k) { return k <= 8 ? 8 : (k <= 16 ? 16 : 32); }
__host__ __device__ constexpr int route_list_len(int k) { return route_kmax(k) + 1 + kExtra; }

template <int D>
struct RouteLayout {
  static constexpr int MT = D / 32;                 // 32-wide output tiles
  static constexpr int NS = D / 16;                 // 16-wide contraction chunks
  static constexpr int NF = MT * (MT + 1);          // chunks on or above the diagonal
  static constexpr int MU_OFF = NF * kFragBytes;
  static constexpr int MU_BYTES = 2 * MT * 16 * 4;  // mu in accumulator order, both lane halves
  static constexpr int SCALE_OFF = MU_OFF + MU_BYTES;  // float: 2^e, T'_c and mu are stored times 2^-e
  static constexpr int BLOCK_BYTES = (SCALE_OFF + 16 + 255) / 256 * 256;
  // LDS copy of one image, whole 1 KB DMA rows (the last row reads past the image)
  static constexpr int DMA_ROWS = (BLOCK_BYTES + 1023) / 1024;
  static constexpr int LDS_BYTES = DMA_ROWS * 1024;
  __host__ __device__ static constexpr int frag(int mt, int s) { return mt * (mt + 1) + s; }
};

// LDS copy of an image's hi parts for the single pass: fragment f's hi half
// (bytes [2048 f, 2048 f + 1024) of the image) at 1024 f, then one 1 KB row
// copied from the image's mu offset (mu, then the scale).
template <int D>
struct HiLayout {
  using Lay = RouteLayout<D>;
  static constexpr int MU_OFF = Lay::NF * 1024;
  static constexpr int SCALE_OFF = MU_OFF + Lay::MU_BYTES;
  static constexpr int DMA_ROWS = Lay::NF + 1;
  static constexpr int LDS_BYTES = DMA_ROWS * 1024;
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += wave_shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, wave_shfl_xor(v, o));
  return v;
}

// Workspace of one call.  bounds[4] per (sequence, KV head) = float bits of
// (lam, G, nu, max|D|), zeroed with qmax before the prep kernel raises them.
struct RouteWs {
  uint8_t* img;       // [b*hkv][nb] images
  uint32_t* qmax;     // [b*hkv]
  uint32_t* bounds;   // [b*hkv][4], right after qmax (one fill clears both)
  float* dbar;        // [b*hkv][d]
  int32_t* tcnt;      // [b*hkv][n_tiles] uncertain rows of each single-pass tile
  int32_t* toff;      // [b*hkv][n_tiles] exclusive prefix of tcnt
  int32_t* dcnt;      // [b*hkv] uncertain rows in all
  int32_t* trows;     // [b*hkv][n_tiles][512] their row ids, per tile
  int32_t* drows;     // [b*hkv][n_tiles * 512] the same, dense, in row order
  // block-major rescoring of the uncertain rows' in-band blocks: record
  // (tile, slot) holds (row, p0, p1) and the row's first p1 list blocks;
  // blocks [p0, p1) each have a rank in their block's pair list and get an
  // exact score
  int32_t* rcnt;      // [b*hkv][n_tiles] records of each tile
  int4* rmeta;        // [b*hkv][n_tiles][kRecCap]
  int32_t* rblk;      // [b*hkv][n_tiles][kRecCap][L]
  int32_t* rrank;     // same shape
  float* rscore;      // same shape
  int32_t* pcnt;      // [b*hkv][nb] pairs per block
  int32_t* poff;      // [b*hkv][nb] exclusive prefix of pcnt
  int32_t* pscratch;  // [b*hkv] (pair totals, unused)
  uint32_t* pent;     // [b*hkv][n_tiles * kRecCap * L] pairs, block-major: rec << 6 | slot
  // rows rescored on every routable block (their bands may reach past the
  // list): row id, position t (-1: unused slot), scores, selections
  int32_t* fcnt;      // [b*hkv] (may pass kFullCap: slots past it are not taken)
  int32_t* frow;      // [b*hkv][kFullCap]
  int32_t* fpos;      // [b*hkv][kFullCap]
  float* fscore;      // [b*hkv][kFullCap][nb]
  int32_t* fidx;      // [b*hkv][kFullCap][k]
  size_t bytes;
};

int64_t route_tiles(const Shape& s) { return (s.n * s.g + kRouteRows - 1) / kRouteRows; }

RouteWs route_ws_layout(const Shape& s, void* base) {
  RouteWs w{};
  const size_t per = s.d == 64 ? RouteLayout<64>::BLOCK_BYTES : RouteLayout<128>::BLOCK_BYTES;
  const size_t n_bkv = size_t(s.b) * s.hkv, nt = size_t(route_tiles(s));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  // + 1 KB: a DMA row of the last image reads up to one row past its end
  const size_t o_img = take(n_bkv * size_t(s.nb) * per + 1024);
  const size_t o_q = take(n_bkv * 4 * 5);
  const size_t o_db = take(n_bkv * size_t(s.d) * 4);
  const size_t o_tc = take(n_bkv * nt * 4);
  const size_t o_to = take(n_bkv * nt * 4);
  const size_t o_dc = take(n_bkv * 4);
  const size_t o_tr = take(n_bkv * nt * kRouteRows * 4);
  const size_t o_dr = take(n_bkv * nt * kRouteRows * 4);
  const size_t L = size_t(route_list_len(s.k)), recs = n_bkv * nt * kRecCap;
  const size_t o_rc = take(n_bkv * nt * 4);
  const size_t o_rm = take(recs * 16);
  const size_t o_rb = take(recs * L * 4);
  const size_t o_rr = take(recs * L * 4);
  const size_t o_rs = take(recs * L * 4);
  const size_t o_pc = take(n_bkv * size_t(s.nb) * 4);
  const size_t o_po = take(n_bkv * size_t(s.nb) * 4);
  const size_t o_ps = take(n_bkv * 4);
  const size_t o_pe = take(recs * L * 4);
  const size_t o_fc = take(n_bkv * 4);
  const size_t o_fr = take(n_bkv * kFullCap * 4);
  const size_t o_fp = take(n_bkv * kFullCap * 4);
  const size_t o_fs = take(n_bkv * kFullCap * size_t(s.nb) * 4);
  const size_t o_fi = take(n_bkv * kFullCap * size_t(s.k) * 4);
  w.bytes = off;
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.img = p + o_img;
    w.qmax = reinterpret_cast<uint32_t*>(p + o_q);
    w.bounds = w.qmax + n_bkv;
    w.dbar = reinterpret_cast<float*>(p + o_db);
    w.tcnt = reinterpret_cast<int32_t*>(p + o_tc);
    w.toff = reinterpret_cast<int32_t*>(p + o_to);
    w.dcnt = reinterpret_cast<int32_t*>(p + o_dc);
    w.trows = reinterpret_cast<int32_t*>(p + o_tr);
    w.drows = reinterpret_cast<int32_t*>(p + o_dr);
    w.rcnt = reinterpret_cast<int32_t*>(p + o_rc);
    w.rmeta = reinterpret_cast<int4*>(p + o_rm);
    w.rblk = reinterpret_cast<int32_t*>(p + o_rb);
    w.rrank = reinterpret_cast<int32_t*>(p + o_rr);
    w.rscore = reinterpret_cast<float*>(p + o_rs);
    w.pcnt = reinterpret_cast<int32_t*>(p + o_pc);
    w.poff = reinterpret_cast<int32_t*>(p + o_po);
    w.pscratch = reinterpret_cast<int32_t*>(p + o_ps);
    w.pent = reinterpret_cast<uint32_t*>(p + o_pe);
    w.fcnt = reinterpret_cast<int32_t*>(p + o_fc);
    w.frow = reinterpret_cast<int32_t*>(p + o_fr);
    w.fpos = reinterpret_cast<int32_t*>(p + o_fp);
    w.fscore = reinterpret_cast<float*>(p + o_fs);
    w.fidx = reinterpret_cast<int32_t*>(p + o_fi);
  }
  return w;
}

// Prepared image of one block (workspace): for every output tile mt and
// chunk s <= 2mt+1, lane (m, h) of the fragment holds T'_c[frag_k(s,h,e)][32mt+m]
// for e = 0..7 -- times 2^-e as float16 hi (bytes 0..1023) and lo
// (1024..2047), or float32 (e = 0); then mu_c times 2^-(e + eq) in accumulator
// order: [h][mt][4a+b] = mu_c[32mt + 8a + 4h + b], where 2^-eq is the float16
// scale of the KV head's query rows; then the float 2^e.  T'_c = T_c for
// float32 inputs, T_c - diag(D) for bfloat16 inputs.
//
// bfloat16 inputs also raise the KV head's bounds: lam >= ||sym(T'_c - hi_c)||_2,
// G = the largest absolute row sum of sym(T'_c), nu = ||mu_c||.  With
// A = lo + lo^T (lo the float16 low part, its diagonal counted twice),
// ||sym(lo)||_2 = ||A||_2 / 2 <= sqrt(||A^2||_F) / 2; A^2 runs on the float16
// MFMA (products exact, float32 sums: ||A^2 - computed||_F <= d 2^-24 ||A||_F^2);
// the low part's own rounding E = (T'_c - hi_c) - lo adds at most ||E||_F.
//
// D comes from shift_sigma (shift_nb blocks per KV head): the blocks' own
// Sigma for block images, the blocks' Sigma too for images of group summaries,
// so that group bounds and block scores leave out the same q^T diag(D) q.
template <bool F32, int D>
__global__ __launch_bounds__(256) void route_prep_kernel(const float* __restrict__ mu,
                                                          const float* __restrict__ sigma,
                                                          const uint32_t* __restrict__ qmax,
                                                          uint32_t* __restrict__ bounds,
                                                          float* __restrict__ dbar,
                                                          uint8_t* __restrict__ prep, int64_t nb,
                                                          float beta,
                                                          const float* __restrict__ shift_sigma,
                                                          int64_t shift_nb) {
  using Lay = RouteLayout<D>;
  constexpr int AS = D + 8;   // row stride of A (halves), against LDS bank conflicts
  __shared__ float red[4][4];
  __shared__ float nred[4];
  __shared__ float sdb[D];
  __shared__ __attribute__((aligned(16))) _Float16 A16[F32 ? 8 : D * AS];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const int64_t bkv = blockIdx.y;
  const int64_t blk = bkv * nb + blockIdx.x;
  const float* S = sigma + blk * int64_t(D) * D;
  const float* M = mu + blk * D;
  uint8_t* out = prep + blk * Lay::BLOCK_BYTES;
  const float half_beta = 0.5f * beta;
  if constexpr (!F32) {
    // D: mean of the first blocks' (beta/2) diagonals (any vector common to
    // the KV head's blocks leaves the ranking unchanged; this one keeps T' small)
    const int64_t m = shift_nb < kShiftBlocks ? shift_nb : kShiftBlocks;
    const float* S0 = shift_sigma + bkv * shift_nb * int64_t(D) * D;
    for (int j = tid; j < D; j += blockDim.x) {
      // the (at most kShiftBlocks) loads go out together, summed in block order
      float dv[kShiftBlocks];
#pragma unroll
      for (int c = 0; c < kShiftBlocks; ++c) dv[c] = c < m ? S0[(c * D + j) * D + j] : 0.f;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < kShiftBlocks; ++c)
        if (c < m) acc += half_beta * dv[c];
      sdb[j] = acc / float(m);
      if (blockIdx.x == 0) dbar[bkv * D + j] = sdb[j];
    }
    __syncthreads();
  }
  // float16 parts: scale by 2^-e so that the largest |T'_ij| lies in [2^14, 2^15).
  // One pass over Sigma gives that maximum and, for the bound G below, the
  // absolute column sums of sym(T'_c) (Sigma is symmetric, so column sums
  // equal row sums and read coalesced): thread (column j, quarter r) covers
  // rows [r D/QR, (r+1) D/QR) of column j, sixteen loads in flight.
  float scale = 1.f, unscale = 1.f;
  static_assert(D * 4 <= 512 && 256 % D == 0, "column split");
  constexpr int QR = 256 / D;   // row groups per column
  __shared__ float colsum[256];
  if constexpr (!F32) {
    float mx = 0.f;
    {
      const int j = tid % D, r = tid / D;
      const float dj = sdb[j];
      float cs = 0.f;
      // sixteen loads go out before any is used, and the sums take selects,
      // not branches (a branch per element would make every load wait alone)
      for (int i0 = r * (D / QR); i0 < (r + 1) * (D / QR); i0 += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = S[(i0 + u) * D + j];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int i = i0 + u;
          const float diag = fabsf(half_beta * v[u] - dj);
          cs += i == j ? diag : fabsf(half_beta * v[u]);
          const float t = i < j ? fabsf(beta * v[u]) : diag;
          mx = i <= j ? fmaxf(mx, t) : mx;
        }
      }
      colsum[tid] = cs;
    }
    mx = wave_max(mx);
    if (lane == 0) red[0][wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    if (mx > 0.f && mx == mx && mx < __builtin_inff()) {
      const int e = ilogbf(mx) - 14;
      scale = ldexpf(1.f, -e);
      unscale = ldexpf(1.f, e);
    }
  }
  float e2 = 0.f, a2 = 0.f;   // this thread's shares of ||E||_F^2 and ||A||_F^2
  for (int w = tid; w < Lay::NF * 64; w += blockDim.x) {
    const int f = w / 64, ln = w % 64, m = ln % 32, h = ln / 32;
    int mt = 0;
    while ((mt + 1) * (mt + 2) <= f) ++mt;
    const int s = f - mt * (mt + 1);
    const int j = 32 * mt + m;
    // the eight loads go out together; tval's cases are then selects
    float raw[8], x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) raw[e] = S[frag_k(s, h, e) * D + j];
    const float dj = F32 ? 0.f : sdb[j];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = frag_k(s, h, e);
      const float diag = half_beta * raw[e] - dj;
      x[e] = i < j ? beta * raw[e] : (i == j ? diag : 0.f);
    }
    if constexpr (F32) {
      floatx8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = x[e];
      *reinterpret_cast<floatx8*>(out + f * kFragBytes + ln * 32) = v;
    } else {
      f16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = frag_k(s, h, e);
        const float v = x[e] * scale;
        const _Float16 hv = static_cast<_Float16>(v);
        const float l = v - static_cast<float>(hv);       // exact
        const _Float16 lv = static_cast<_Float16>(l);
        hi[e] = hv;
        lo[e] = lv;
        if (i <= j) {   // each upper-triangle entry once (the rest of the tile is 0)
          const float er = l - static_cast<float>(lv);   // exact
          e2 = fmaf(er, er, e2);
          const float lf = static_cast<float>(lv);
          if (i == j) {
            A16[i * AS + i] = static_cast<_Float16>(2.f * lf);
            a2 = fmaf(4.f * lf, lf, a2);
          } else {
            A16[i * AS + j] = lv;
            A16[j * AS + i] = lv;
            a2 = fmaf(2.f * lf, lf, a2);
          }
        }
      }
      *reinterpret_cast<f16x8*>(out + f * kFragBytes + ln * 16) = hi;
      *reinterpret_cast<f16x8*>(out + f * kFragBytes + 1024 + ln * 16) = lo;
    }
  }
  // (a null qmax leaves mu at 2^-e: route_mu_scale_kernel applies 2^-eq)
  const float mscale =
      F32 || qmax == nullptr ? scale : scale * ldexpf(1.f, -query_exponent(qmax[blockIdx.y]));
  for (int w = tid; w < 2 * Lay::MT * 16; w += blockDim.x) {
    const int h = w / (Lay::MT * 16), mt = (w / 16) % Lay::MT, i = w % 16;
    reinterpret_cast<float*>(out + Lay::MU_OFF)[w] = M[32 * mt + 8 * (i / 4) + 4 * h + (i % 4)] * mscale;
  }
  if (tid == 0) *reinterpret_cast<float*>(out + Lay::SCALE_OFF) = unscale;
  if constexpr (!F32) {
    // G: largest absolute row sum of sym(T'_c) (real units), from the
    // column sums above; nu = ||mu_c||
    float nu2 = 0.f;
    for (int i = tid; i < D; i += blockDim.x) nu2 = fmaf(M[i], M[i], nu2);
    __syncthreads();   // A and the column sums complete
    float g = 0.f;
    if (tid < D) {
      float cs = 0.f;
#pragma unroll
      for (int r = 0; r < QR; ++r) cs += colsum[r * D + tid];
      g = cs;
    }
    // ||A^2||_F^2 on the float16 MFMA: the 32x32 output tiles dealt to the waves
    constexpr int MT = Lay::MT;
    float b2 = 0.f;
    const int ln = lane % 32, kh = lane / 32;
    for (int tile = wave; tile < MT * MT; tile += 4) {
      const int tm = tile / MT, tn = tile % MT;
      floatx16 acc;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        // row 32tm+ln of A and row 32tn+ln (= column, A symmetric), same k slots
        const f16x8 a = *reinterpret_cast<const f16x8*>(&A16[(32 * tm + ln) * AS + 16 * ks + 8 * kh]);
        const f16x8 b = *reinterpret_cast<const f16x8*>(&A16[(32 * tn + ln) * AS + 16 * ks + 8 * kh]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) b2 = fmaf(acc[q], acc[q], b2);
    }
    e2 = wave_sum(e2);
    a2 = wave_sum(a2);
    b2 = wave_sum(b2);
    g = wave_max(g);
    nu2 = wave_sum(nu2);
    __syncthreads();
    if (lane == 0) {
      red[0][wave] = e2;
      red[1][wave] = a2;
      red[2][wave] = b2;
      red[3][wave] = g;
      nred[wave] = nu2;
    }
    __syncthreads();
    if (tid == 0) {
      const float E2 = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
      const float A2 = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
      const float B2 = (red[2][0] + red[2][1]) + (red[2][2] + red[2][3]);
      const float G = fmaxf(fmaxf(red[3][0], red[3][1]), fmaxf(red[3][2], red[3][3]));
      const float NU2 = (nred[0] + nred[1]) + (nred[2] + nred[3]);
      // float32 sums of squares of these sizes stay within 2^-9 relative
      const float normB = (sqrtf(B2) + float(D) * 0x1p-24f * A2) * (1.f + 0x1p-9f);
      const float lam_scaled = 0.5f * sqrtf(normB) + sqrtf(E2 * (1.f + 0x1p-9f));
      float lam = lam_scaled * unscale * (1.f + 0x1p-10f);
      if (!(lam == lam)) lam = __builtin_inff();
      atomicMax(&bounds[bkv * 4 + 0], __float_as_uint(lam));
      atomicMax(&bounds[bkv * 4 + 1], __float_as_uint(G * (1.f + 0x1p-10f)));
      atomicMax(&bounds[bkv * 4 + 2], __float_as_uint(sqrtf(NU2) * (1.f + 0x1p-10f)));
      float dm = 0.f;
      for (int j = 0; j < D; ++j) dm = fmaxf(dm, fabsf(sdb[j]));
      atomicMax(&bounds[bkv * 4 + 3], __float_as_uint(dm));
    }
  }
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

// Query fragments of a lane's two 32-row tiles (KV-head rows rho_of[nt] =
// t g + jg where valid[nt]): bfloat16 rows become float16 after scaling by
// qsc = 2^-eq.
template <bool F32, int D>
__device__ __forceinline__ void load_q_tiles(typename QFrag<F32>::T (&bq)[2][D / 16],
                                             const typename QFrag<F32>::In* Q,
                                             const int64_t (&rho_of)[2], const bool (&valid)[2],
                                             int64_t b, int64_t kv, int g, int hq, int64_t n, int h,
                                             float qsc) {
  constexpr int NS = D / 16;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const RowTJ q = split_rho(valid[nt] ? rho_of[nt] : 0, g);
    const auto* row = Q + (((b * hq + kv * g + q.jg) * n) + q.t) * D;
    if constexpr (F32) {
#pragma unroll
      for (int s = 0; s < NS; ++s) bq[nt][s] = load_q_frag<F32>(row, s, h, valid[nt]);
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 raw = load_q_bits(row, s, h, valid[nt]);
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

// ------------------------------------------------------------- exact pass --
//
// hi + lo (float16) or float32 contraction against every routable block of
// each row.  Dense mode: the workgroup owns 512 consecutive rows of its
// (sequence, KV head).  List mode (rows != nullptr): it owns positions
// [512 j, 512 j + 512) of the KV head's row list (j its tile), in any row
// order; workgroups past the end of the list exit.
template <bool F32, int D, int KMAX>
__global__ __launch_bounds__(kRouteThreads) void route_topk_kernel(
    const typename QFrag<F32>::In* __restrict__ Q, const uint8_t* __restrict__ prep,
    const uint32_t* __restrict__ qmax, const float* __restrict__ dbar,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ row_count,
    int32_t* __restrict__ idx, float* __restrict__ kth, int64_t n, int g, int hq, int hkv, int B,
    int64_t nb, int k, int64_t n_tiles, int64_t n_bkv) {
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
  const bool listed = rows != nullptr;
  const int64_t list_len = listed ? int64_t(row_count[bkv]) : rows_total;
  if (rho0 >= list_len) return;   // list mode: past the end of the list (uniform)
  const int32_t* list = listed ? rows + bkv * n_tiles * kRouteRows : nullptr;
  // the KV head's row (t g + jg) at position p
  auto row_at = [&](int64_t p) -> int64_t { return listed ? int64_t(list[p]) : p; };

  QT bq[2][NS];
  float qsc = 1.f, qsq = 1.f;   // 2^-eq and 2^(2 eq)
  if constexpr (!F32) {
    const int eq = query_exponent(qmax[bkv]);
    qsc = ldexpf(1.f, -eq);
    qsq = ldexpf(1.f, 2 * eq);
  }
  {
    const int64_t p0 = rho0 + 64 * wave + ln, p1 = p0 + 32;
    const bool valid[2] = {p0 < list_len, p1 < list_len};
    const int64_t rho_of[2] = {valid[0] ? row_at(p0) : 0, valid[1] ? row_at(p1) : 0};
    load_q_tiles<F32, D>(bq, Q, rho_of, valid, b, kv, g, hq, n, h, qsc);
  }
  // the row this lane scores and ranks
  const int64_t my_p = rho0 + 64 * wave + 32 * h + ln;
  const bool my_valid = my_p < list_len;
  const int64_t my_rho = my_valid ? row_at(my_p) : 0;
  const int64_t my_t = my_valid ? split_rho(my_rho, g).t : 0;
  const int64_t my_C = my_valid ? min(nb, (my_t + 1) / B) : 0;
  // the workgroup's routable range: in dense mode its last row's; a list
  // need not be in row order (the hierarchical visit's is not), so there the
  // largest over its rows
  int64_t C_wg;
  if (!listed) {
    const int64_t t_max = min(n - 1, (rho0 + kRouteRows - 1) / g);
    C_wg = min(nb, (t_max + 1) / B);
  } else {
    __shared__ int32_t cw[kRouteThreads / 64];
    int c = int(my_C);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c = max(c, __shfl_xor(c, o, 64));
    if (lane == 0) cw[wave] = c;
    __syncthreads();
    C_wg = 0;
#pragma unroll
    for (int w = 0; w < kRouteThreads / 64; ++w) C_wg = max(C_wg, int64_t(cw[w]));
  }

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

  // q^T diag(D) q of this lane's row (bfloat16: the scores above leave it out)
  float qdq = 0.f;
  if (kth != nullptr && !F32) {
    const float* dv = dbar + bkv * D;
    float part[2] = {0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = QFrag<F32>::elem(bq[nt][s2], e);
          part[nt] = fmaf(dv[frag_k(s2, h, e)] * x, x, part[nt]);
        }
    const float q0 = part[0] + wave_shfl_xor(part[0], 32);
    const float q1 = part[1] + wave_shfl_xor(part[1], 32);
    qdq = (h ? q1 : q0) * qsq;
  }
  if (!my_valid) return;
  const RowTJ rt = split_rho(my_rho, g);
  const int64_t orow = (b * hq + kv * g + rt.jg) * n + rt.t;
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
      if (i == k - 1) r_k = ls[i] * qsq + qdq;
      if (i == k) r_k1 = ls[i] * qsq + qdq;
    }
    kth[orow * 2] = r_k;
    kth[orow * 2 + 1] = r_k1;
  }
}

// ------------------------------------------------------------ single pass --

// A packed key's score: the key's top bits are the float's bits mapped to an
// unsigned integer of the same order (sign bit flipped for x >= 0, all bits
// for x < 0); the low bits hold (mask - block), so among equal top bits the
// lower block is the larger key.  Key 0 means "no entry".
__device__ __forceinline__ float key_score(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key ^ 0x80000000u) : ~key;
  return __uint_as_float(u);
}

// The single pass's way out for one lane's row, from its running top-NL
// packed keys (shared by the flat single pass and the hierarchical visit):
// certification against the rigorous error bound e of the hi-part scores,
// then either the row's selection (certified), a rescore record of its band
// (block-major exact scores, then the final top-k), a full row (exact scores
// on every routable block) or, past the caps, the exact pass.  nq2 is the
// row's ||q||^2 in scaled units (float16 values, float32 sum, times
// 1 + 2^-16); every wave of the workgroup calls it (ballots and barriers).
template <int KMAX>
__device__ __forceinline__ void certify_emit(
    const uint32_t (&lk)[KMAX + 1 + kExtra], float nq2, float qsc, uint32_t mask,
    const uint32_t* __restrict__ bounds, int64_t bkv, int64_t tile, int64_t n_tiles,
    bool my_valid, int64_t my_rho, int64_t my_t, int64_t my_C, int* wave_rec, int* wave_unc,
    int tid, int wave, int lane, int32_t* __restrict__ idx, int32_t* __restrict__ tcnt,
    int32_t* __restrict__ trows, int32_t* __restrict__ rcnt, int4* __restrict__ rmeta,
    int32_t* __restrict__ rblk, int32_t* __restrict__ rrank, int32_t* __restrict__ pcnt,
    int32_t* __restrict__ fcnt, int32_t* __restrict__ frow, int32_t* __restrict__ fpos, int64_t n,
    int g, int hq, int hkv, int64_t nb, int k) {
  constexpr int NL = KMAX + 1 + kExtra;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  // Rows with at most k routable blocks keep them all.  Otherwise: a packed
  // key stands for every score with the same top bits (its bucket), whose
  // ends are the key with its low bits cleared and set; e bounds |approximate
  // - exact| for every block.  A listed block whose bucket floor minus e
  // exceeds the ceiling plus e of the (k+1)-th key's bucket is in the exact
  // top-k (only blocks of the approximate top-k can beat it); a block whose
  // ceiling plus e is below the floor minus e of the k-th key's bucket is out
  // (k blocks beat it).  Keys are sorted, so the in-blocks are list positions
  // [0, p0), the out-blocks [p1, NL) and every unlisted block when p1 < NL.
  // p0 == k certifies the row.  Otherwise the blocks at [p0, p1) get exact
  // scores, block-major (a record of the row); when p1 == NL and blocks past
  // the list may be in, or the tile's records are full, every block of the
  // row does (a full row); rows with a non-finite key, and full rows past
  // the cap, go to the exact pass.
  bool cert = true, ok = true, wide = false;
  int p0 = 0, p1 = 0;
  if (my_C > k) {
    uint32_t kk = 0u, kk1 = 0u;
#pragma unroll
    for (int i = 0; i <= KMAX; ++i) {
      if (i == k - 1) kk = lk[i];
      if (i == k) kk1 = lk[i];
    }
    const float lam = __uint_as_float(bounds[bkv * 4 + 0]);
    const float G = __uint_as_float(bounds[bkv * 4 + 1]);
    const float nu = __uint_as_float(bounds[bkv * 4 + 2]);
    const float dm = __uint_as_float(bounds[bkv * 4 + 3]);
    // the hi part's rounding; float32 accumulation (and the diagonal shift's
    // own float32 rounding, at most 2^-23 (|D| + |T'_ii|) per diagonal entry),
    // the latter taken 1.25 times
    const float e_hi = lam * nq2;
    const float e_acc = 0x1p-17f * (G * nq2 + nu * qsc * sqrtf(nq2)) + 0x1p-22f * (dm + G) * nq2;
    const float e = 1.25f * (e_hi + e_acc);
    const float lo_k = key_score(kk & ~mask), hi_k1 = key_score(kk1 | mask);
    ok = kk != 0u && kk1 != 0u && fabsf(lo_k) >= 0x1p-100f && fabsf(hi_k1) >= 0x1p-100f &&
         e < __builtin_inff();
    const float in_edge = hi_k1 + 2.f * e, out_edge = lo_k - 2.f * e;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const float lo_i = key_score(lk[i] & ~mask), hi_i = key_score(lk[i] | mask);
      const bool listed = lk[i] != 0u;
      ok = ok && (!listed || (fabsf(lo_i) < __builtin_inff() && fabsf(hi_i) < __builtin_inff()));
      p0 += (listed && lo_i > in_edge) ? 1 : 0;
      p1 += (listed && hi_i >= out_edge) ? 1 : 0;
    }
    cert = ok && p0 == k;
    wide = p1 == NL && my_C > NL;
  }
  // records first: rows with a band inside the list, in row order, up to
  // kRecCap per tile (wave ballots; lane = row offset within the wave)
  const bool want_rec = my_valid && !cert && ok && !wide;
  const uint64_t bal_r = __ballot(want_rec);
  if (lane == 0) wave_rec[wave] = __popcll(bal_r);
  __syncthreads();
  int rbase = 0, rtotal = 0;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) {
    rbase += w < wave ? wave_rec[w] : 0;
    rtotal += wave_rec[w];
  }
  const int rslot = rbase + __popcll(bal_r & ((uint64_t(1) << lane) - 1u));
  const bool rec = want_rec && rslot < kRecCap;
  // then full rows, up to kFullCap per KV head
  int fslot = kFullCap;
  if (my_valid && !cert && ok && !rec) fslot = atomicAdd(&fcnt[bkv], 1);
  const bool full = fslot < kFullCap;
  if (full) {
    frow[bkv * kFullCap + fslot] = int32_t(my_rho);
    fpos[bkv * kFullCap + fslot] = int32_t(my_t);
  }
  // everything else uncertain -> this tile's list for the exact pass
  const bool unc = my_valid && !cert && !rec && !full;
  const uint64_t bal = __ballot(unc);
  if (lane == 0) wave_unc[wave] = __popcll(bal);
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) {
    base += w < wave ? wave_unc[w] : 0;
    total += wave_unc[w];
  }
  const int64_t tix = bkv * n_tiles + tile;
  if (unc) {
    const int rank = __popcll(bal & ((uint64_t(1) << lane) - 1u));
    trows[tix * kRouteRows + base + rank] = int32_t(my_rho);
  }
  if (tid == 0) {
    tcnt[tix] = total;
    rcnt[tix] = min(rtotal, kRecCap);
  }
  if (rec) {
    // the record: (row, p0, p1), the first p1 blocks, and each in-band block's
    // rank in its block's pair list
    const int64_t r = tix * kRecCap + rslot;
    rmeta[r] = int4{int32_t(my_rho), p0, p1, 0};
    int32_t* rb = rblk + r * NL;
    int32_t* rr = rrank + r * NL;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (i < p1) {
        const int32_t c = int32_t(mask - (lk[i] & mask));
        rb[i] = c;
        if (i >= p0) rr[i] = atomicAdd(&pcnt[bkv * nb + c], 1);
      }
    }
  }
  if (!my_valid || !cert || k == 0) return;
  // certified: the blocks of the first min(k, C) keys, ascending, -1 padded
  const int64_t orow = (b * hq + kv * g + split_rho(my_rho, g).jg) * n + my_t;
  int32_t* out = idx + orow * k;
  int cidx[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
    cidx[i] = (i < my_C && lk[i] != 0u) ? int(mask - (lk[i] & mask)) : -1;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < k) {
      const unsigned key_i = unsigned(cidx[i]);
      int rank = 0;
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k) {
          const unsigned key_j = unsigned(cidx[j]);
          rank += (key_j < key_i || (key_j == key_i && j < i)) ? 1 : 0;
        }
      out[rank] = cidx[i];
    }
  }}

template <int D, int KMAX>
__global__ __launch_bounds__(kRouteThreads) void route_fast_kernel(
    const bf16_t* __restrict__ Q, const uint8_t* __restrict__ prep,
    const uint32_t* __restrict__ qmax, const uint32_t* __restrict__ bounds,
    int32_t* __restrict__ idx, int32_t* __restrict__ tcnt, int32_t* __restrict__ trows,
    int32_t* __restrict__ rcnt, int4* __restrict__ rmeta, int32_t* __restrict__ rblk,
    int32_t* __restrict__ rrank, int32_t* __restrict__ pcnt, int32_t* __restrict__ fcnt,
    int32_t* __restrict__ frow, int32_t* __restrict__ fpos, int64_t n, int g, int hq, int hkv,
    int B, int64_t nb, int k, int key_bits, int64_t n_tiles, int64_t n_bkv) {
  using Lay = RouteLayout<D>;
  using HL = HiLayout<D>;
  using QT = f16x8;
  constexpr int MT = Lay::MT, NS = Lay::NS, BYTES = Lay::BLOCK_BYTES;
  constexpr int NL = KMAX + 1 + kExtra;                // list length (route_list_len)
  constexpr int NBUF = 3;                              // block images in flight
  constexpr int NW = kRouteThreads / 64;
  constexpr int R = (HL::DMA_ROWS + NW - 1) / NW;      // copy instructions per wave per block
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * HL::LDS_BYTES];
  __shared__ int wave_unc[kRouteThreads / 64];
  __shared__ int wave_rec[kRouteThreads / 64];

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t wid = blockIdx.x;
  const int64_t bkv = wid % n_bkv;
  const int64_t tile = n_tiles - 1 - wid / n_bkv;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rows_total = n * g;
  const int64_t rho0 = tile * kRouteRows;
  const uint32_t mask = (1u << key_bits) - 1u;

  QT bq[2][NS];
  const int eq = query_exponent(qmax[bkv]);
  const float qsc = ldexpf(1.f, -eq);
  {
    const int64_t p0 = rho0 + 64 * wave + ln, p1 = p0 + 32;
    const bool valid[2] = {p0 < rows_total, p1 < rows_total};
    const int64_t rho_of[2] = {p0, p1};
    load_q_tiles<false, D>(bq, Q, rho_of, valid, b, kv, g, hq, n, h, qsc);
  }
  const int64_t my_rho = rho0 + 64 * wave + 32 * h + ln;
  const bool my_valid = my_rho < rows_total;
  const int64_t my_t = my_valid ? split_rho(my_rho, g).t : 0;
  const int64_t my_C = my_valid ? min(nb, (my_t + 1) / B) : 0;
  const int64_t t_max = min(n - 1, (rho0 + kRouteRows - 1) / g);
  const int64_t C_wg = min(nb, (t_max + 1) / B);

  uint32_t lk[NL];   // running top-NL packed keys, descending
#pragma unroll
  for (int i = 0; i < NL; ++i) lk[i] = 0u;

  // Block c's hi fragments, mu and scale -> LDS buffer c % 3 by direct
  // global->LDS copies (1 KB per wave instruction), issued two blocks ahead.
  // Every wave issues exactly R copies per block (rows past the last repeat
  // it), so at the top of iteration c "this wave's copies of block c are
  // done" is vmcnt <= R (block c+1's may still be in flight); a barrier then
  // makes every wave's copies visible, and also tells that block c-1's buffer
  // -- the next copy's target -- is no longer read.  The copies are written
  // in asm, with m0 saved and restored around them: the compiler would
  // otherwise make every LDS read wait for all copies in flight (it cannot
  // tell the buffers apart), which leaves each copy's latency exposed.
  const uint8_t* src_base = prep + bkv * nb * int64_t(BYTES);
  const uint32_t lds_base =
      uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(lds)));
  // the wave index as a uniform (scalar) value: the copies' LDS rows are then
  // scalar arithmetic, with no lane-to-scalar move per copy
  const int swave = __builtin_amdgcn_readfirstlane(wave);
  auto stage = [&](int c, int buf) {
    const uint8_t* src = src_base + uint64_t(uint32_t(c)) * BYTES;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int r = min(swave + NW * i, HL::DMA_ROWS - 1);
      const int off = r < Lay::NF ? r * kFragBytes : Lay::MU_OFF;
      const uint8_t* g = src + off + lane * 16;
      const uint32_t l =
          __builtin_amdgcn_readfirstlane(lds_base + uint32_t(buf * HL::LDS_BYTES + r * 1024));
      uint32_t keep;
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %2\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %1, off\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(keep)
          : "v"(g), "s"(l)
          : "memory");
    }
  };
  // (C_wg <= nb < 2^16: block indices fit 32 bits)
  const int C_w = int(C_wg);
  if (C_w > 0) {
    stage(0, 0);
    stage(min(1, C_w - 1), 1);
  }

  // The exact pass's hand-scheduled sweep with the hi part only: chunk pairs
  // (two fragments), each MFMA call followed by its share of the previous
  // tile's row-dot and, during the widest tile, the previous block's
  // reduction, key and insert (two instructions a slot: the max and the min
  // of two distinct keys).
  constexpr int PK = 2;
  constexpr int NDOT = 32;
  floatx16 acc[2][2];
#pragma unroll
  for (int st2 = 0; st2 < 2; ++st2)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[st2][nt][j] = 0.f;
  // the row-dot of each row tile in two partial sums (alternate terms): two
  // dependent chains per tile instead of one, which the vector unit overlaps
  // better with the matrix core; any order stays within the bound's float32
  // accumulation term
  float pt[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
  uint32_t key_ins = 0u;
  auto read_frag = [&](const uint8_t* L, int mt, int gp, int k2) {
    return *reinterpret_cast<const QT*>(L + Lay::frag(mt, 2 * gp + k2) * 1024 + lane * 16);
  };
  auto read_mu = [&](const uint8_t* L, int mt) {
    floatx16 m;
    const floatx4* p = reinterpret_cast<const floatx4*>(L + HL::MU_OFF + mt * 64) + h * (MT * 4);
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
    pt[nt][j & 1] = fmaf(acc[set][nt][j],
                         static_cast<float>(bq[nt][2 * mt + (a >> 1)][4 * (a & 1) + bb]),
                         pt[nt][j & 1]);
  };
  float blk_scale = 1.f;
  auto reduce = [&](int64_t cb) {
    const float s0 = pt[0][0] + pt[0][1], s1 = pt[1][0] + pt[1][1];
    const float p0 = s0 + wave_shfl_xor(s0, 32);
    const float p1 = s1 + wave_shfl_xor(s1, 32);
    pt[0][0] = pt[0][1] = pt[1][0] = pt[1][1] = 0.f;
    const float a = (h ? p1 : p0) * blk_scale;
    const uint32_t u = __float_as_uint(a);
    const uint32_t o = u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
    const uint32_t key = (o & ~mask) | (mask - uint32_t(cb));
    key_ins = (cb >= 0 && cb < my_C && a == a) ? key : 0u;
  };
  // the smaller key first, so the larger can take the old slot's register
  // (no copies of the list at the loop's back edge)
  auto insert_step = [&](int i) {
    const uint32_t v = lk[i];
    const uint32_t lower = min(v, key_ins);
    lk[i] = max(v, key_ins);
    key_ins = lower;
  };

  auto sweep = [&](int c, const uint8_t* L) {
    const float scale_c = *reinterpret_cast<const float*>(L + HL::SCALE_OFF);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) asm volatile("" : "+v"(bq[nt][s2]));
    QT fr[2][PK];
#pragma unroll
    for (int k2 = 0; k2 < PK; ++k2) fr[0][k2] = read_frag(L, MT - 1, 0, k2);
    floatx16 mu_next = read_mu(L, MT - 1);
    int pslot = 0;
#pragma unroll
    for (int mt = MT - 1; mt >= 0; --mt) {
      const int set = (MT - 1 - mt) & 1, pset = set ^ 1;
      const floatx16 mu_t = mu_next;
      constexpr int kCallsPerPair = PK * 2;
      const int calls = (mt + 1) * kCallsPerPair;
      const int nwork = NDOT + (mt == MT - 1 ? 1 + NL : 0);
#pragma unroll
      for (int i = 0; i < calls; ++i) {
        const int gp = i / kCallsPerPair, k2 = (i / 2) % PK, nt = i % 2;
        const int sidx = 2 * gp + k2;
        const int slot = (pslot + gp) & 1;
        const floatx16 cin = (i < 2) ? mu_t : acc[set][nt];
        acc[set][nt] = mma16(fr[slot][k2], bq[nt][sidx], cin);
        if (i % kCallsPerPair == 1) {
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
    blk_scale = scale_c;
  };
  // ring positions of block c (read) and block c + 2 (staged), kept as counters
  int rbuf = 0, sbuf = 2 % NBUF;
  for (int c = 0; c < C_w; ++c) {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(R) : "memory");
    stage(min(c + 2, C_w - 1), sbuf);   // past the end: a repeat, never read
    sweep(c, lds + rbuf * HL::LDS_BYTES);
    rbuf = rbuf == NBUF - 1 ? 0 : rbuf + 1;
    sbuf = sbuf == NBUF - 1 ? 0 : sbuf + 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy outlives the loop
  if (C_w > 0) {
#pragma unroll
    for (int w = 0; w < NDOT; ++w) dot_item((MT - 1) & 1, 0, w);
    reduce(C_w - 1);
#pragma unroll
    for (int i = 0; i < NL; ++i) insert_step(i);
  }

  // ---- certification.  ||q||^2 of this lane's row (scaled units, exact
  // float16 values, float32 sum)
  float nq[2] = {0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = static_cast<float>(bq[nt][s2][e]);
        nq[nt] = fmaf(x, x, nq[nt]);
      }
  const float nq0 = nq[0] + wave_shfl_xor(nq[0], 32);
  const float nq1 = nq[1] + wave_shfl_xor(nq[1], 32);
  const float nq2 = (h ? nq1 : nq0) * (1.f + 0x1p-16f);

  certify_emit<KMAX>(lk, nq2, qsc, mask, bounds, bkv, tile, n_tiles, my_valid, my_rho, my_t, my_C,
                     wave_rec, wave_unc, tid, wave, lane, idx, tcnt, trows, rcnt, rmeta, rblk, rrank,
                     pcnt, fcnt, frow, fpos, n, g, hq, hkv, nb, k);

}

// Exclusive prefix of the per-tile uncertain counts of one (sequence, KV
// head), and their total.
__global__ __launch_bounds__(1024) void route_scan_kernel(const int32_t* __restrict__ tcnt,
                                                          int32_t* __restrict__ toff,
                                                          int32_t* __restrict__ dcnt,
                                                          int64_t n_tiles) {
  __shared__ int32_t part[1024];
  const int64_t bkv = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t per = (n_tiles + 1023) / 1024;
  const int64_t j0 = min(n_tiles, tid * per), j1 = min(n_tiles, j0 + per);
  int32_t s = 0;
  for (int64_t j = j0; j < j1; ++j) s += tcnt[bkv * n_tiles + j];
  part[tid] = s;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive Hillis-Steele scan
    const int32_t v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t run = part[tid] - s;
  for (int64_t j = j0; j < j1; ++j) {
    toff[bkv * n_tiles + j] = run;
    run += tcnt[bkv * n_tiles + j];
  }
  if (tid == 1023) dcnt[bkv] = part[1023];
}

// One wave per single-pass tile: its uncertain rows -> the dense list.
__global__ __launch_bounds__(64) void route_gather_kernel(const int32_t* __restrict__ tcnt,
                                                          const int32_t* __restrict__ toff,
                                                          const int32_t* __restrict__ trows,
                                                          int32_t* __restrict__ drows,
                                                          int64_t n_tiles) {
  const int64_t t = blockIdx.x, bkv = t / n_tiles;
  const int32_t cnt = tcnt[t], off = toff[t];
  for (int i = threadIdx.x; i < cnt; i += 64)
    drows[bkv * n_tiles * kRouteRows + off + i] = trows[t * kRouteRows + i];
}

// ------------------------------------------------- block-major rescoring --
//
// The single pass's records name, for each row left uncertain, the list
// blocks whose exact scores decide its top-k.  Those (record, block) pairs
// are counted per block (ranks taken by the single pass), laid out
// block-major by an exclusive scan, and rescored one block at a time: a
// workgroup stages block c's full hi + lo image once and scores every pair
// of c, so each image is read once however many rows need it.

// One thread per record slot of a tile: its in-band pairs -> their blocks'
// lists, entry = (record within the KV head) << 6 | list position.
__global__ __launch_bounds__(kRecCap) void route_scatter_kernel(
    const int32_t* __restrict__ rcnt, const int4* __restrict__ rmeta,
    const int32_t* __restrict__ rblk, const int32_t* __restrict__ rrank,
    const int32_t* __restrict__ poff, uint32_t* __restrict__ pent, int64_t nb, int64_t n_tiles,
    int L) {
  const int64_t tix = blockIdx.x, bkv = tix / n_tiles;
  const int slot = threadIdx.x;
  if (slot >= rcnt[tix]) return;
  const int64_t r = tix * kRecCap + slot;
  const uint32_t local = uint32_t(r - bkv * n_tiles * kRecCap);
  const int4 m = rmeta[r];
  uint32_t* out = pent + bkv * n_tiles * kRecCap * L;
  for (int u = m.y; u < m.z; ++u) {
    const int32_t c = rblk[r * L + u];
    out[poff[bkv * nb + c] + rrank[r * L + u]] = local << 6 | uint32_t(u);
  }
}

constexpr int kRescoreThreads = 256;

// The exact (hi + lo) score of a lane's row against the block image at L (in
// LDS), with the exact pass's arithmetic operation for operation: per output
// tile from the widest down, an MFMA chain from mu over the chunks in order
// (hi then lo of each), then the row-dot of the tile; the lane halves summed;
// times the image's scale.  Lane (ln, h) returns row ln of query tile h.
//
// With lin != nullptr it also returns, in the same units, the mean term
// <q, mu> alone (the row-dot of q with the image's mu).  LO = false: the hi
// part alone (the single pass's arithmetic), within the single pass's error
// bound e of the hi + lo score.
template <int D, bool LO = true>
__device__ __forceinline__ float hilo_score(const uint8_t* L, const f16x8 (&bq)[2][D / 16],
                                            int lane, float* lin = nullptr) {
  using Lay = RouteLayout<D>;
  constexpr int MT = Lay::MT;
  const int h = lane / 32;
  // fragment (mt, chunk s2, part) of the image
  auto frag = [&](int mt, int s2, int part) {
    return *reinterpret_cast<const f16x8*>(L + Lay::frag(mt, s2) * kFragBytes + part * 1024 +
                                           lane * 16);
  };
  float pt[2] = {0.f, 0.f}, pl[2] = {0.f, 0.f};
  // chunks move one ahead of their MFMAs (hi and lo of the next chunk are
  // read before this chunk's four MFMAs); the scheduling barriers keep the
  // compiler from reading the whole image ahead, which needs more registers
  // than a wave has
  constexpr int PARTS = LO ? 2 : 1;
  f16x8 cur[2] = {frag(MT - 1, 0, 0), LO ? frag(MT - 1, 0, 1) : f16x8{}};
#pragma unroll
  for (int mt = MT - 1; mt >= 0; --mt) {
    floatx16 acc[2];
    {
      const floatx4* p = reinterpret_cast<const floatx4*>(L + Lay::MU_OFF + mt * 64) + h * (MT * 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 v = p[q];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[0][4 * q + e] = v[e];
      }
      acc[1] = acc[0];
    }
    if (lin != nullptr) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int a = j / 4, bb = j % 4;
          pl[nt] = fmaf(acc[nt][j], static_cast<float>(bq[nt][2 * mt + (a >> 1)][4 * (a & 1) + bb]), pl[nt]);
        }
    }
#pragma unroll
    for (int s2 = 0; s2 <= 2 * mt + 1; ++s2) {
      f16x8 nxt[2] = {cur[0], cur[1]};
      if (s2 < 2 * mt + 1) {
        nxt[0] = frag(mt, s2 + 1, 0);
        if constexpr (LO) nxt[1] = frag(mt, s2 + 1, 1);
      } else if (mt > 0) {
        nxt[0] = frag(mt - 1, 0, 0);
        if constexpr (LO) nxt[1] = frag(mt - 1, 0, 1);
      }
#pragma unroll
      for (int part = 0; part < PARTS; ++part)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[nt] = mma16(cur[part], bq[nt][s2], acc[nt]);
      cur[0] = nxt[0];
      cur[1] = nxt[1];
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int a = j / 4, bb = j % 4;
        pt[nt] = fmaf(acc[nt][j], static_cast<float>(bq[nt][2 * mt + (a >> 1)][4 * (a & 1) + bb]), pt[nt]);
      }
  }
  const float scale = *reinterpret_cast<const float*>(L + Lay::SCALE_OFF);
  if (lin != nullptr) {
    const float l0 = pl[0] + wave_shfl_xor(pl[0], 32);
    const float l1 = pl[1] + wave_shfl_xor(pl[1], 32);
    *lin = (h ? l1 : l0) * scale;
  }
  const float s0 = pt[0] + wave_shfl_xor(pt[0], 32);
  const float s1 = pt[1] + wave_shfl_xor(pt[1], 32);
  return (h ? s1 : s0) * scale;
}

// Workgroup (c, KV head): the exact (hi + lo) score of block c for every pair
// in c's list, then for every full row that can route to c, 64 rows per wave
// at a time (two 32-row MFMA tiles).  The arithmetic is the exact pass's,
// operation for operation (MFMA chains from mu over the chunks in order, the
// row-dot over the tiles from the widest down), so the scores are the ones
// the exact pass would compute; like them they leave out the KV head's
// common factor 2^(2 eq).
template <int D>
__global__ __launch_bounds__(kRescoreThreads) void route_rescore_kernel(
    const bf16_t* __restrict__ Q, const uint8_t* __restrict__ prep,
    const uint32_t* __restrict__ qmax, const int32_t* __restrict__ pcnt,
    const int32_t* __restrict__ poff, const uint32_t* __restrict__ pent,
    const int4* __restrict__ rmeta, float* __restrict__ rscore, const int32_t* __restrict__ fcnt,
    const int32_t* __restrict__ frow, const int32_t* __restrict__ fpos,
    float* __restrict__ fscore, int64_t n, int g, int hq, int hkv, int B, int64_t nb,
    int64_t n_tiles, int L) {
  using Lay = RouteLayout<D>;
  using QT = f16x8;
  constexpr int NS = Lay::NS, BYTES = Lay::BLOCK_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[Lay::LDS_BYTES];
  const int64_t c = blockIdx.x, bkv = blockIdx.y;
  const int32_t cnt = pcnt[bkv * nb + c];
  const int32_t fc = min(fcnt[bkv], kFullCap);
  if (cnt == 0 && fc == 0) return;   // uniform
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  {
    const uint8_t* src = prep + (bkv * nb + c) * int64_t(BYTES);
    for (int r = wave; r < Lay::DMA_ROWS; r += kRescoreThreads / 64)
      __builtin_amdgcn_global_load_lds(src + r * 1024 + lane * 16,
                                       (__attribute__((address_space(3))) void*)(lds + r * 1024),
                                       16, 0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  const float qsc = ldexpf(1.f, -query_exponent(qmax[bkv]));
  // the score of the lane's row (tile h, row ln) for block c
  auto score = [&](const int64_t (&rho_of)[2], const bool (&valid)[2]) {
    QT bq[2][NS];
    load_q_tiles<false, D>(bq, Q, rho_of, valid, b, kv, g, hq, n, h, qsc);
    return hilo_score<D>(lds, bq, lane);
  };
  const int64_t rec0 = bkv * n_tiles * kRecCap;
  const uint32_t* ent = pent + rec0 * L + poff[bkv * nb + c];
  const int4* meta = rmeta + rec0;
  float* rs = rscore + rec0 * L;
  for (int j0 = 64 * wave; j0 < cnt; j0 += kRescoreThreads) {
    bool valid[2];
    int64_t rho_of[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int j = j0 + 32 * nt + ln;
      valid[nt] = j < cnt;
      rho_of[nt] = valid[nt] ? int64_t(meta[ent[j] >> 6].x) : 0;
    }
    const float sc = score(rho_of, valid);
    const int my_j = j0 + 32 * h + ln;
    if (my_j < cnt) {
      const uint32_t e = ent[my_j];
      rs[int64_t(e >> 6) * L + (e & 63u)] = sc;
    }
  }
  const int32_t* fr = frow + bkv * kFullCap;
  const int32_t* fp = fpos + bkv * kFullCap;
  float* fs = fscore + bkv * kFullCap * nb;
  // full rows start at the last wave, so that with few pairs and few full
  // rows (the common case) both run side by side instead of one after the other
  for (int j0 = 64 * (kRescoreThreads / 64 - 1 - wave); j0 < fc; j0 += kRescoreThreads) {
    bool valid[2];
    int64_t rho_of[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int j = j0 + 32 * nt + ln;
      valid[nt] = j < fc && c < min(nb, (int64_t(fp[j]) + 1) / B);
      rho_of[nt] = valid[nt] ? int64_t(fr[j]) : 0;
    }
    if (__ballot(valid[0] || valid[1]) == 0) continue;   // uniform
    const float sc = score(rho_of, valid);
    const int my_j = j0 + 32 * h + ln;
    if (my_j < fc && c < min(nb, (int64_t(fp[my_j]) + 1) / B)) fs[int64_t(my_j) * nb + c] = sc;
  }
}

// One wave per (KV head, full-row slot) group: the full rows' selections
// (computed in slot order) -> their rows of idx.
__global__ __launch_bounds__(256) void route_full_out_kernel(
    const int32_t* __restrict__ fcnt, const int32_t* __restrict__ frow,
    const int32_t* __restrict__ fidx, int32_t* __restrict__ idx, int64_t n, int g, int hq, int hkv,
    int k) {
  const int64_t bkv = blockIdx.x;
  const int fc = min(fcnt[bkv], kFullCap);
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  for (int e = threadIdx.x; e < fc * k; e += 256) {
    const int j = e / k, i = e % k;
    const RowTJ q = split_rho(frow[bkv * kFullCap + j], g);
    idx[((b * hq + kv * g + q.jg) * n + q.t) * k + i] = fidx[(bkv * kFullCap + j) * k + i];
  }
}

// One thread per record: the blocks certainly in, plus the best (k - p0) of
// the rescored band by (score descending, block ascending) -- blocks with a
// score of -inf or NaN are never taken, as in the exact pass -- ascending,
// -1 padded.
template <int KMAX>
__global__ __launch_bounds__(kRecCap) void route_finalize_kernel(
    const int32_t* __restrict__ rcnt, const int4* __restrict__ rmeta,
    const int32_t* __restrict__ rblk, const float* __restrict__ rscore, int32_t* __restrict__ idx,
    int64_t n, int g, int hq, int hkv, int k, int64_t n_tiles) {
  constexpr int L = KMAX + 1 + kExtra;
  const int64_t tix = blockIdx.x, bkv = tix / n_tiles;
  const int slot = threadIdx.x;
  if (slot >= rcnt[tix]) return;
  const int64_t r = tix * kRecCap + slot;
  const int4 m = rmeta[r];
  const int p0 = m.y, p1 = m.z;
  int blk[L];
  float sc[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    blk[i] = i < p1 ? rblk[r * L + i] : -1;
    sc[i] = (i >= p0 && i < p1) ? rscore[r * L + i] : -__builtin_inff();
  }
  bool take[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    int rank = 0;
#pragma unroll
    for (int j = 0; j < L; ++j)
      rank += (j >= p0 && j < p1 && (sc[j] > sc[i] || (sc[j] == sc[i] && blk[j] < blk[i]))) ? 1 : 0;
    take[i] = i < p0 || (i < p1 && sc[i] > -__builtin_inff() && rank < k - p0);
  }
  const RowTJ q = split_rho(m.x, g);
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  int32_t* out = idx + ((b * hq + kv * g + q.jg) * n + q.t) * k;
  int count = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    int pos = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) pos += (take[j] && blk[j] < blk[i]) ? 1 : 0;
    if (take[i]) out[pos] = blk[i];
    count += take[i] ? 1 : 0;
  }
  for (int i = count; i < k; ++i) out[i] = -1;
}

// Before the single pass (or the hierarchical visit): the counts its rows
// add to start at zero, and every full-row slot at position -1 (no blocks).
// Up to four (pointer, count, value) int32 ranges filled by one launch
// (unused ranges have count 0).
struct FillSpec {
  int32_t* p[4];
  int64_t count[4];
  int32_t v[4];
};

__global__ __launch_bounds__(256) void fill_ranges_kernel(FillSpec f) {
  const int64_t stride = int64_t(gridDim.x) * 256;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < f.count[r]; i += stride)
      f.p[r][i] = f.v[r];
}

void launch_fill_ranges(const FillSpec& f, hipStream_t st) {
  int64_t mx = 0;
  for (int r = 0; r < 4; ++r) mx = std::max(mx, f.count[r]);
  if (mx == 0) return;
  hipLaunchKernelGGL(fill_ranges_kernel, dim3(unsigned(std::min<int64_t>((mx + 255) / 256, 1024))),
                     dim3(256), 0, st, f);
}

void route_resolve_clear(const Shape& s, const RouteWs& w, int64_t n_bkv, hipStream_t st) {
  const int64_t pairs = n_bkv * s.nb;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned(std::min<int64_t>((pairs + 255) / 256, 1024))),
                     dim3(256), 0, st, w.pcnt, pairs, 0);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, w.fcnt, n_bkv, 0);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned(std::min<int64_t>((n_bkv * kFullCap + 255) / 256, 1024))),
                     dim3(256), 0, st, w.fpos, n_bkv * kFullCap, -1);
}

// After the single pass (or the hierarchical visit), which certified what it
// could and left records, full rows and uncertain rows in the workspace: the
// exact selection of every row that is left.
template <int D, int KMAX>
hipError_t route_resolve(const Shape& s, const void* Q, const RouteWs& w, int32_t* idx,
                         int64_t n_tiles, int64_t n_bkv, hipStream_t st) {
  const unsigned grid = unsigned(n_tiles * n_bkv);
  const int L = route_list_len(s.k);
  // rows the records could not take: the exact pass over the compacted list
  hipLaunchKernelGGL(route_scan_kernel, dim3(unsigned(n_bkv)), dim3(1024), 0, st, w.tcnt, w.toff,
                     w.dcnt, n_tiles);
  hipLaunchKernelGGL(route_gather_kernel, dim3(grid), dim3(64), 0, st, w.tcnt, w.toff, w.trows,
                     w.drows, n_tiles);
  hipLaunchKernelGGL((route_topk_kernel<false, D, KMAX>), dim3(grid), dim3(kRouteThreads), 0,
                     st, static_cast<const bf16_t*>(Q), w.img, w.qmax, w.dbar, w.drows, w.dcnt,
                     idx, nullptr, s.n, s.g, s.hq, s.hkv, s.B, s.nb, s.k, n_tiles, n_bkv);
  // the records: block-major pair lists, exact band scores, final top-k
  hipLaunchKernelGGL(route_scan_kernel, dim3(unsigned(n_bkv)), dim3(1024), 0, st, w.pcnt, w.poff,
                     w.pscratch, s.nb);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(grid), dim3(kRecCap), 0, st, w.rcnt, w.rmeta,
                     w.rblk, w.rrank, w.poff, w.pent, s.nb, n_tiles, L);
  hipLaunchKernelGGL((route_rescore_kernel<D>), dim3(unsigned(s.nb), unsigned(n_bkv)),
                     dim3(kRescoreThreads), 0, st, static_cast<const bf16_t*>(Q), w.img, w.qmax,
                     w.pcnt, w.poff, w.pent, w.rmeta, w.rscore, w.fcnt, w.frow, w.fpos, w.fscore,
                     s.n, s.g, s.hq, s.hkv, s.B, s.nb, n_tiles, L);
  hipLaunchKernelGGL((route_finalize_kernel<KMAX>), dim3(grid), dim3(kRecCap), 0, st, w.rcnt,
                     w.rmeta, w.rblk, w.rscore, idx, s.n, s.g, s.hq, s.hkv, s.k, n_tiles);
  // the full rows: the wave top-k over each one's scores (unused slots have
  // position -1, hence no blocks), then out to idx
  hipError_t e = launch_decode_topk(w.fscore, w.fpos, w.fidx, s.k, s.nb, 1, s.B,
                                    n_bkv * kFullCap, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_full_out_kernel, dim3(unsigned(n_bkv)), dim3(256), 0, st, w.fcnt,
                     w.frow, w.fidx, idx, s.n, s.g, s.hq, s.hkv, s.k);
  return hipGetLastError();
}

// Multiplies the mu section of every block image of (sequence, KV head)
// blockIdx.y by 2^-eq, the float16 scale of that KV head's query rows, for
// images that route_prep_kernel wrote with a null qmax (so that it could run
// beside the max|q| pass).  Both factors are powers of two, so the result is
// the one a single multiplication by 2^-(e + eq) gives.
template <int D>
__global__ __launch_bounds__(256) void route_mu_scale_kernel(const uint32_t* __restrict__ qmax,
                                                             uint8_t* __restrict__ prep,
                                                             int64_t nb) {
  using Lay = RouteLayout<D>;
  constexpr int NMU = Lay::MU_BYTES / 4;
  const int64_t bkv = blockIdx.y;
  const float f = ldexpf(1.f, -query_exponent(qmax[bkv]));
  for (int64_t w = int64_t(blockIdx.x) * 256 + threadIdx.x; w < nb * NMU;
       w += int64_t(gridDim.x) * 256) {
    float* m = reinterpret_cast<float*>(prep + (bkv * nb + w / NMU) * Lay::BLOCK_BYTES + Lay::MU_OFF);
    m[w % NMU] *= f;
  }
}

template <bool F32, int D, int KMAX>
hipError_t launch_route_t(const Shape& s, const void* Q, const float* mu, const float* sigma,
                          int32_t* idx, float* kth, void* ws, hipStream_t st) {
  const int64_t n_bkv = int64_t(s.b) * s.hkv;
  const RouteWs w = route_ws_layout(s, ws);
  const int64_t n_tiles = route_tiles(s);
  using In = typename QFrag<F32>::In;
  // per (sequence, KV head): the largest |q| of its query rows (bfloat16
  // bits), which sets the float16 scale of Q (the group's rows are
  // contiguous); the bounds start at zero, and so do the single pass's pair
  // and full-row counts (full-row positions at -1), in the same launch
  {
    FillSpec f{};
    f.p[0] = reinterpret_cast<int32_t*>(w.qmax);
    f.count[0] = 5 * n_bkv;
    f.p[1] = w.pcnt;
    f.count[1] = n_bkv * s.nb;
    f.p[2] = w.fcnt;
    f.count[2] = n_bkv;
    f.p[3] = w.fpos;
    f.count[3] = n_bkv * kFullCap;
    f.v[3] = -1;
    launch_fill_ranges(f, st);
  }
  // the max|q| pass (bfloat16 inputs) runs on the device's second stream
  // beside the image preparation, which then leaves mu unscaled by the
  // query scale until both are done
  {
    SideLease side(st);
    if constexpr (!F32) {
      const int64_t per_group = int64_t(s.g) * s.n * D;
      const unsigned gx = value_max_groups(per_group);
      hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bkv)), dim3(256), 0, side.stream(),
                         static_cast<const bf16_t*>(Q), w.qmax, per_group);
    }
    if (s.nb > 0)
      hipLaunchKernelGGL((route_prep_kernel<F32, D>), dim3(unsigned(s.nb), unsigned(n_bkv)),
                         dim3(256), 0, st, mu, sigma, nullptr, w.bounds, w.dbar, w.img, s.nb,
                         s.beta, sigma, s.nb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = side.join()) != hipSuccess) return e;
    if (!F32 && s.nb > 0) {
      const int64_t elems = s.nb * (RouteLayout<D>::MU_BYTES / 4);
      const unsigned gx = unsigned(std::min<int64_t>((elems + 255) / 256, 64));
      hipLaunchKernelGGL((route_mu_scale_kernel<D>), dim3(gx, unsigned(n_bkv)), dim3(256), 0, st,
                         w.qmax, w.img, s.nb);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  int key_bits = 1;
  while ((int64_t(1) << key_bits) < s.nb) ++key_bits;
  const unsigned grid = unsigned(n_tiles * n_bkv);
  // (record entries hold a record index below 2^26)
  if (F32 || kth != nullptr || key_bits > kMaxKeyBits || s.nb == 0 || s.k == 0 ||
      n_tiles * kRecCap > (int64_t(1) << 26)) {
    hipLaunchKernelGGL((route_topk_kernel<F32, D, KMAX>), dim3(grid), dim3(kRouteThreads), 0, st,
                       static_cast<const In*>(Q), w.img, w.qmax, w.dbar, nullptr, nullptr, idx, kth,
                       s.n, s.g, s.hq, s.hkv, s.B, s.nb, s.k, n_tiles, n_bkv);
    return hipGetLastError();
  }
  if constexpr (!F32) {
    hipLaunchKernelGGL((route_fast_kernel<D, KMAX>), dim3(grid), dim3(kRouteThreads), 0, st,
                       static_cast<const bf16_t*>(Q), w.img, w.qmax, w.bounds, idx, w.tcnt, w.trows,
                       w.rcnt, w.rmeta, w.rblk, w.rrank, w.pcnt, w.fcnt, w.frow, w.fpos, s.n, s.g,
                       s.hq, s.hkv, s.B, s.nb, s.k, key_bits, n_tiles, n_bkv);
    if (hipError_t e = route_resolve<D, KMAX>(s, Q, w, idx, n_tiles, n_bkv, st); e != hipSuccess)
      return e;
  }
  return hipGetLastError();
}

template <bool F32, int D>
hipError_t launch_route_d(const Shape& s, const void* Q, const float* mu, const float* sigma,
                          int32_t* idx, float* kth, void* ws, hipStream_t st) {
  if (s.k <= 8) return launch_route_t<F32, D, 8>(s, Q, mu, sigma, idx, kth, ws, st);
  if (s.k <= 16) return launch_route_t<F32, D, 16>(s, Q, mu, sigma, idx, kth, ws, st);
  return launch_route_t<F32, D, 32>(s, Q, mu, sigma, idx, kth, ws, st);
}

// ------------------------------------------ hierarchical routing (prefill) --
//
// The flat top-k by branch and bound over groups of m consecutive blocks,
// for prefill query rows.  A group's summary (ssa_group_stats: mean centroid
// mu_G, radius R_G, mean covariance S_G, slack lam_G) bounds every member's
// score for beta >= 0:
//   UB_G(q) = r_G(q) + ||q|| R_G + (beta/2) lam_G ||q||^2,
// r_G the routing score of (mu_G, S_G).  r_G is computed like a block score:
// the summaries are prepared into the same images (with the blocks' diagonal
// shift, so bounds and scores leave out the same q^T diag(D) q) and scored
// with the hi part alone, as in the single pass, plus that pass's rigorous
// bound e on |hi - (hi + lo)| (the group images' own constants), so it never
// falls below the exact pass's r_G; the bound carries a relative margin
// (kHierPrefillMargin of its terms' magnitudes) over float32 rounding.
//
// Blocks are scored for a tile of rows at a time (one image in LDS serves
// 512 rows), so a tile pays for the union of what its rows need.  Rows are
// therefore regrouped first: within each chunk of kHierChunk consecutive
// 512-row tiles (nearby positions, so similar routable ranges), by the group
// of their largest bound, so that a tile's rows tend to need the same few
// groups.
//
//  * bound: per 512-row tile of a KV head's rows (in row order), UB_G of
//    every row for every group with a routable block in the tile (row-major
//    in the workspace), each row's best group, and per group the number of
//    the tile's rows it is best for.
//  * scan + order: rows listed chunk by chunk, by best group within a chunk
//    (ties keep row order); tiles of 512 consecutive list entries.
//  * visit: per listed tile, the groups in decreasing order of the tile's
//    largest bound; a group is scored -- each of its blocks against all the
//    tile's rows with the single pass's arithmetic, into each row's running
//    packed keys -- unless, for every row, its bound is strictly below what
//    the row's k listed blocks are known to score exactly.  The rows then
//    leave through the single pass's certification and resolution, so every
//    row gets exactly the flat selection.  (k = 0, or keys or records beyond
//    the single pass's range: a visit that scores every needed block with
//    the exact pass's arithmetic and prunes against the exact k-th score.)

constexpr float kHierPrefillMargin = 1e-4f;
constexpr int kHierSortMax = 4096;   // groups per (sequence, KV head) the visit orders
constexpr int kHierChunk = 16;       // row tiles whose rows are regrouped together

__host__ __device__ inline int64_t hier_chunks(int64_t n_tiles) {
  return (n_tiles + kHierChunk - 1) / kHierChunk;
}

int64_t hier_groups(const Shape& s, int m) { return (s.nb + m - 1) / m; }

struct HierWs {
  RouteWs rw;        // the flat router's workspace: block images, max|q|, the
                     // blocks' error-bound constants, records and full rows
  uint8_t* img;      // = rw.img: block images [b*hkv][nb]
  uint8_t* gimg;     // group images [b*hkv][G]
  uint32_t* qmax;    // = rw.qmax: [b*hkv], then the blocks' bounds [b*hkv][4]
  uint32_t* gbounds; // [b*hkv][4]: the group images' error-bound constants
  float* dbar;       // [b*hkv][d]
  float* gdbar;      // [b*hkv][d]
  float* ub;         // [b*hkv][rows][G]: bounds, row-major
  int32_t* best;     // [b*hkv][rows]: each row's best group
  int32_t* gcnt;     // [b*hkv][chunk][G][kHierChunk]: rows of each tile whose best group is g
  int32_t* goff;     // same: exclusive prefix in (chunk, g, tile) order
  int32_t* gtot;     // [b*hkv]
  int32_t* list;     // [b*hkv][rows]: rows by best group
  size_t bytes;
};

HierWs hier_ws_layout(const Shape& s, int m, void* base) {
  HierWs w{};
  const size_t per = s.d == 64 ? RouteLayout<64>::BLOCK_BYTES : RouteLayout<128>::BLOCK_BYTES;
  const size_t n_bkv = size_t(s.b) * s.hkv, nt = size_t(route_tiles(s));
  const size_t rows = size_t(s.n) * size_t(s.g);
  const size_t G = size_t(hier_groups(s, m));
  w.rw = route_ws_layout(s, base);
  size_t off = w.rw.bytes;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t o_gimg = take(n_bkv * G * per + 1024);
  const size_t o_gb = take(n_bkv * 4 * 4);
  const size_t o_gdb = take(n_bkv * size_t(s.d) * 4);
  const size_t o_ub = take(n_bkv * rows * G * 4);
  const size_t o_best = take(n_bkv * rows * 4);
  const size_t nc = size_t(hier_chunks(int64_t(nt))) * kHierChunk;
  const size_t o_gc = take(n_bkv * G * nc * 4);
  const size_t o_go = take(n_bkv * G * nc * 4);
  const size_t o_gt = take(n_bkv * 4);
  const size_t o_li = take(n_bkv * rows * 4);
  w.bytes = off;
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.img = w.rw.img;
    w.gimg = p + o_gimg;
    w.qmax = w.rw.qmax;
    w.gbounds = reinterpret_cast<uint32_t*>(p + o_gb);
    w.dbar = w.rw.dbar;
    w.gdbar = reinterpret_cast<float*>(p + o_gdb);
    w.ub = reinterpret_cast<float*>(p + o_ub);
    w.best = reinterpret_cast<int32_t*>(p + o_best);
    w.gcnt = reinterpret_cast<int32_t*>(p + o_gc);
    w.goff = reinterpret_cast<int32_t*>(p + o_go);
    w.gtot = reinterpret_cast<int32_t*>(p + o_gt);
    w.list = reinterpret_cast<int32_t*>(p + o_li);
  }
  return w;
}

// ||q'||^2 of the lane's row (tile h, row ln), float16 values, float32 sum.
template <int D>
__device__ __forceinline__ float row_norm2(const f16x8 (&bq)[2][D / 16], int h) {
  float nq[2] = {0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = static_cast<float>(bq[nt][s2][e]);
        nq[nt] = fmaf(x, x, nq[nt]);
      }
  const float a = nq[0] + wave_shfl_xor(nq[0], 32);
  const float b = nq[1] + wave_shfl_xor(nq[1], 32);
  return h ? b : a;
}

// Direct global->LDS copy of one image (all waves of the workgroup), written
// in asm with m0 saved and restored around each copy, as in the single pass:
// the compiler then does not make every later LDS read wait for the copy
// (it cannot tell the buffers apart), so a copy into one buffer overlaps the
// work on the other.  The caller waits (s_waitcnt vmcnt(0)) and barriers
// before reading the copied buffer.
template <int D>
__device__ __forceinline__ void stage_image(const uint8_t* src, uint8_t* dst, int wave, int lane,
                                            int waves) {
  using Lay = RouteLayout<D>;
  const uint32_t base =
      uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(dst)));
  for (int r = wave; r < Lay::DMA_ROWS; r += waves) {
    const uint8_t* g = src + r * 1024 + lane * 16;
    const uint32_t l = __builtin_amdgcn_readfirstlane(base + uint32_t(r * 1024));
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "v"(g), "s"(l)
        : "memory");
  }
}

// Workgroup (tile, KV head), rows in row order: UB_G for the tile's rows and
// every group with a block routable in the tile (-inf where none is routable
// for the row), each row's best group (the lowest of its largest bounds; 0
// when it has none), and the tile's count of rows per best group.
template <int D>
__global__ __launch_bounds__(kRouteThreads) void hier_ub_kernel(
    const bf16_t* __restrict__ Q, const uint8_t* __restrict__ gimg, const float* __restrict__ grl,
    const uint32_t* __restrict__ qmax, const uint32_t* __restrict__ gbounds, float* __restrict__ ub,
    int32_t* __restrict__ best, int32_t* __restrict__ gcnt, int64_t n, int g, int hq, int hkv,
    int B, int64_t nb, int m, int64_t G, int64_t n_tiles, int64_t n_bkv, float beta) {
  using Lay = RouteLayout<D>;
  constexpr int NS = D / 16, BYTES = Lay::BLOCK_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * Lay::LDS_BYTES];
  __shared__ int32_t hist[kHierSortMax];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t wid = blockIdx.x;
  const int64_t bkv = wid % n_bkv;
  const int64_t tile = n_tiles - 1 - wid / n_bkv;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rows_total = n * g;
  const int64_t rho0 = tile * kRouteRows;
  f16x8 bq[2][NS];
  const int eq = query_exponent(qmax[bkv]);
  const float qsc = ldexpf(1.f, -eq);
  {
    const int64_t p0 = rho0 + 64 * wave + ln, p1 = p0 + 32;
    const bool valid[2] = {p0 < rows_total, p1 < rows_total};
    const int64_t rho_of[2] = {p0, p1};
    load_q_tiles<false, D>(bq, Q, rho_of, valid, b, kv, g, hq, n, h, qsc);
  }
  const int r = 64 * wave + 32 * h + ln;
  const int64_t my_rho = rho0 + r;
  const bool my_valid = my_rho < rows_total;
  const int64_t my_t = my_valid ? split_rho(my_rho, g).t : 0;
  const int64_t my_C = my_valid ? min(nb, (my_t + 1) / B) : 0;
  const int64_t t_max = min(n - 1, (rho0 + kRouteRows - 1) / g);
  const int64_t C_wg = min(nb, (t_max + 1) / B);
  const int64_t G_wg = (C_wg + m - 1) / m;
  for (int64_t i = tid; i < G; i += kRouteThreads) hist[i] = 0;
  const float nq2 = row_norm2<D>(bq, h);
  const float qn = sqrtf(nq2);
  // r_G is scored with the hi part only: |hi - (hi + lo)| <= e, the single
  // pass's bound with the group images' own constants (lam, G, nu, max|D|)
  float e_hi;
  {
    const float nq2e = nq2 * (1.f + 0x1p-16f);
    const float lam = __uint_as_float(gbounds[bkv * 4 + 0]);
    const float Gs = __uint_as_float(gbounds[bkv * 4 + 1]);
    const float nu = __uint_as_float(gbounds[bkv * 4 + 2]);
    const float dm = __uint_as_float(gbounds[bkv * 4 + 3]);
    e_hi = 1.25f * (lam * nq2e + 0x1p-17f * (Gs * nq2e + nu * qsc * sqrtf(nq2e)) +
                    0x1p-22f * (dm + Gs) * nq2e);
  }
  float* my_ub = ub + (bkv * rows_total + (my_valid ? my_rho : 0)) * G;
  float best_u = -__builtin_inff();
  int best_g = 0;
  const uint8_t* src = gimg + bkv * G * int64_t(BYTES);
  if (G_wg > 0) stage_image<D>(src, lds, wave, lane, kRouteThreads / 64);
  for (int64_t gi = 0; gi < G_wg; ++gi) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();   // image gi is in LDS; every wave is done with gi - 1's buffer
    if (gi + 1 < G_wg)
      stage_image<D>(src + (gi + 1) * BYTES, lds + ((gi + 1) & 1) * Lay::LDS_BYTES, wave, lane,
                     kRouteThreads / 64);
    // (an empty register constraint keeps the compiler from hoisting float32
    // copies of the loop-invariant q fragments, which would not fit)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) asm volatile("" : "+v"(bq[nt][s2]));
    float lin;   // the mean term <q, mu_G>, in the same (score) units
    const float su = hilo_score<D, false>(lds + (gi & 1) * Lay::LDS_BYTES, bq, lane, &lin) + e_hi;
    const float R = grl[(bkv * G + gi) * 2], lam = grl[(bkv * G + gi) * 2 + 1];
    const float rad = qn * R * qsc, slack = 0.5f * beta * lam * nq2;
    const float mag = fabsf(lin) + fabsf(su - lin) + rad + slack;
    float u = su + rad + slack + kHierPrefillMargin * mag;
    if (u != u) u = __builtin_inff();                   // non-finite inputs: never pruned
    if (!my_valid || gi * m >= my_C) u = -__builtin_inff();
    if (my_valid) my_ub[gi] = u;
    if (u > best_u) {
      best_u = u;
      best_g = int(gi);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();   // hist cleared
  if (my_valid) {
    best[bkv * rows_total + my_rho] = best_g;
    atomicAdd(&hist[best_g], 1);
  }
  __syncthreads();
  const int64_t chunk = tile / kHierChunk, tc = tile % kHierChunk;
  const int64_t n_chunks = hier_chunks(n_tiles);
  for (int64_t i = tid; i < G; i += kRouteThreads)
    gcnt[((bkv * n_chunks + chunk) * G + i) * kHierChunk + tc] = hist[i];
}

// Workgroup (tile, KV head): each row's place in the KV head's list of rows
// by chunk and best group -- the offset of (its chunk, its group, its tile)
// plus the rows of the tile before it with the same group.
__global__ __launch_bounds__(kRouteThreads) void hier_order_kernel(
    const int32_t* __restrict__ best, const int32_t* __restrict__ goff, int32_t* __restrict__ list,
    int64_t rows_total, int64_t G, int64_t n_tiles) {
  __shared__ int32_t tb[kRouteRows];
  const int tid = threadIdx.x;
  const int64_t bkv = blockIdx.x / n_tiles, tile = blockIdx.x % n_tiles;
  const int64_t rho = tile * kRouteRows + tid;
  const bool valid = rho < rows_total;
  const int32_t bg = valid ? best[bkv * rows_total + rho] : -1;
  tb[tid] = bg;
  __syncthreads();
  if (!valid) return;
  int rank = 0;
  for (int j = 0; j < tid; ++j) rank += tb[j] == bg ? 1 : 0;
  const int64_t n_chunks = hier_chunks(n_tiles);
  const int64_t gi = ((bkv * n_chunks + tile / kHierChunk) * G + bg) * kHierChunk + tile % kHierChunk;
  list[bkv * rows_total + goff[gi] + rank] = int32_t(rho);
}

// Workgroup (listed tile, KV head): the visit.  Rows keep their top-k
// sorted by (score descending, block ascending); blocks arrive in any order,
// so the insert compares (score, block) pairs, a total order.
template <int D, int KMAX>
__global__ __launch_bounds__(kRouteThreads) void hier_visit_kernel(
    const bf16_t* __restrict__ Q, const uint8_t* __restrict__ img,
    const uint32_t* __restrict__ qmax, const float* __restrict__ ub,
    const int32_t* __restrict__ list, int32_t* __restrict__ idx, int32_t* __restrict__ evaluated,
    int64_t n, int g, int hq, int hkv, int B, int64_t nb, int m, int64_t G, int k,
    int64_t n_tiles, int64_t n_bkv) {
  using Lay = RouteLayout<D>;
  constexpr int NS = D / 16, BYTES = Lay::BLOCK_BYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * Lay::LDS_BYTES];
  __shared__ uint64_t order[kHierSortMax];
  __shared__ uint32_t gmax[kHierSortMax];
  __shared__ int32_t cmax[kRouteThreads / 64];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t wid = blockIdx.x;
  const int64_t bkv = wid % n_bkv;
  const int64_t tile = wid / n_bkv;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rows_total = n * g;
  const int64_t p0_tile = tile * kRouteRows;
  const int32_t* lst = list + bkv * rows_total;
  f16x8 bq[2][NS];
  {
    const float qsc = ldexpf(1.f, -query_exponent(qmax[bkv]));
    const int64_t p0 = p0_tile + 64 * wave + ln, p1 = p0 + 32;
    const bool valid[2] = {p0 < rows_total, p1 < rows_total};
    const int64_t rho_of[2] = {valid[0] ? int64_t(lst[p0]) : 0, valid[1] ? int64_t(lst[p1]) : 0};
    load_q_tiles<false, D>(bq, Q, rho_of, valid, b, kv, g, hq, n, h, qsc);
  }
  const int64_t my_p = p0_tile + 64 * wave + 32 * h + ln;
  const bool my_valid = my_p < rows_total;
  const int64_t my_rho = my_valid ? int64_t(lst[my_p]) : 0;
  const int64_t my_t = my_valid ? split_rho(my_rho, g).t : 0;
  const int64_t my_C = my_valid ? min(nb, (my_t + 1) / B) : 0;
  const float* my_ub = ub + (bkv * rows_total + my_rho) * G;
  // the tile's routable blocks (largest over its rows) and groups
  {
    int c = int(my_C);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c = max(c, __shfl_xor(c, o, 64));
    if (lane == 0) cmax[wave] = c;
  }
  for (int i = tid; i < kHierSortMax; i += kRouteThreads) gmax[i] = 0u;
  __syncthreads();
  int64_t C_wg = 0;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) C_wg = max(C_wg, int64_t(cmax[w]));
  const int G_wg = int((C_wg + m - 1) / m);
  // the tile's largest bound per group (order-preserving bits, LDS max)
  // (a row's bounds exist for the groups with a block routable for it; the
  // tile's other groups have nothing for the row)
  auto bound = [&](int gi) {
    return (my_valid && int64_t(gi) * m < my_C) ? my_ub[gi] : -__builtin_inff();
  };
  for (int gi = 0; gi < G_wg; ++gi) {
    const float u = bound(gi);
    const uint32_t bits = __float_as_uint(u);
    uint32_t o = bits ^ (uint32_t(int32_t(bits) >> 31) | 0x80000000u);
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) o = max(o, uint32_t(__shfl_xor(int(o), sh, 64)));
    if (lane == 0) atomicMax(&gmax[gi], o);
  }
  __syncthreads();
  // groups in decreasing order of that bound (lower group first among equal
  // bounds): a descending bitonic sort of (bound bits, ~group)
  int P = 1;
  while (P < G_wg) P <<= 1;
  for (int i = tid; i < P; i += kRouteThreads)
    order[i] = i < G_wg ? (uint64_t(gmax[i]) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(i)) : 0;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kRouteThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const uint64_t a = order[i], c = order[j];
          if (desc ? a < c : a > c) {
            order[i] = c;
            order[j] = a;
          }
        }
      }
      __syncthreads();
    }

  float ls[KMAX];
  int li[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    ls[i] = -__builtin_inff();
    li[i] = 0x7FFFFFFF;
  }
  auto kth = [&]() {   // the running k-th score (+inf for k = 0: nothing is needed)
    float t = k == 0 ? __builtin_inff() : -__builtin_inff();
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i == k - 1) t = ls[i];
    return t;
  };
  int scored = 0;
  const uint8_t* src = img + bkv * nb * int64_t(BYTES);
  for (int j = 0; j < G_wg; ++j) {
    const int gi = int(0xFFFFFFFFu - uint32_t(order[j] & 0xFFFFFFFFu));
    const float u = bound(gi);
    const bool need = __syncthreads_or(my_valid && !(u < kth()));
    if (!need) continue;
    const int64_t c0 = int64_t(gi) * m, c1 = min(C_wg, c0 + m);
    stage_image<D>(src + c0 * BYTES, lds, wave, lane, kRouteThreads / 64);
    for (int64_t c = c0; c < c1; ++c) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();   // image c is in LDS; every wave is done with c - 1's buffer
      if (c + 1 < c1)
        stage_image<D>(src + (c + 1) * BYTES, lds + ((c + 1 - c0) & 1) * Lay::LDS_BYTES, wave,
                       lane, kRouteThreads / 64);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)   // (q stays in float16 registers; see hier_ub_kernel)
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) asm volatile("" : "+v"(bq[nt][s2]));
      float sc = hilo_score<D>(lds + ((c - c0) & 1) * Lay::LDS_BYTES, bq, lane);
      if (c >= my_C || !(sc > -__builtin_inff())) continue;   // not routable, -inf or NaN
      int ci = int(c);
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        const bool gt = sc > ls[i] || (sc == ls[i] && ci < li[i]);
        const float ts = ls[i];
        const int ti = li[i];
        ls[i] = gt ? sc : ts;
        li[i] = gt ? ci : ti;
        sc = gt ? ts : sc;
        ci = gt ? ti : ci;
      }
    }
    scored += int(c1 - c0);
    __syncthreads();   // the last image's buffer is free before the next group stages
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (evaluated != nullptr && tid == 0) evaluated[bkv * n_tiles + tile] = scored;
  if (!my_valid || k == 0) return;
  const RowTJ rt = split_rho(my_rho, g);
  int32_t* out = idx + ((b * hq + kv * g + rt.jg) * n + rt.t) * k;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < k) {
      const int ci = li[i] == 0x7FFFFFFF ? -1 : li[i];
      const unsigned key_i = unsigned(ci);
      int rank = 0;
#pragma unroll
      for (int j2 = 0; j2 < KMAX; ++j2)
        if (j2 < k) {
          const unsigned key_j = unsigned(li[j2] == 0x7FFFFFFF ? -1 : li[j2]);
          rank += (key_j < key_i || (key_j == key_i && j2 < i)) ? 1 : 0;
        }
      out[rank] = ci;
    }
  }
}

// Workgroup (listed tile, KV head): the visit with the single pass's
// arithmetic.  Blocks of the needed groups are scored with the hi part alone
// (hilo_score<D, false>) into each row's running top-NL packed keys, exactly
// as the single pass keeps them; a group is skipped when, for every row of
// the tile, its bound is below the row's running k-th key's bucket floor
// minus e (the k listed blocks' exact scores are all above that, so no block
// of the group can displace them).  The rows then leave through the single
// pass's certification (certify_emit): certified rows write their selection,
// the rest become rescore records, full rows or exact-pass rows, resolved
// afterwards by the flat router's kernels -- so every row gets the exact
// pass's selection, as with the flat router.
template <int D, int KMAX>
__global__ __launch_bounds__(kRouteThreads) void hier_visit_fast_kernel(
    const bf16_t* __restrict__ Q, const uint8_t* __restrict__ img,
    const uint32_t* __restrict__ qmax, const uint32_t* __restrict__ bounds,
    const float* __restrict__ ub, const int32_t* __restrict__ list, int32_t* __restrict__ idx,
    int32_t* __restrict__ evaluated, int32_t* __restrict__ tcnt, int32_t* __restrict__ trows,
    int32_t* __restrict__ rcnt, int4* __restrict__ rmeta, int32_t* __restrict__ rblk,
    int32_t* __restrict__ rrank, int32_t* __restrict__ pcnt, int32_t* __restrict__ fcnt,
    int32_t* __restrict__ frow, int32_t* __restrict__ fpos, int64_t n, int g, int hq, int hkv,
    int B, int64_t nb, int m, int64_t G, int k, int key_bits, int64_t n_tiles, int64_t n_bkv) {
  using Lay = RouteLayout<D>;
  constexpr int NS = D / 16, BYTES = Lay::BLOCK_BYTES;
  constexpr int NL = KMAX + 1 + kExtra;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * Lay::LDS_BYTES];
  __shared__ uint64_t order[kHierSortMax];
  __shared__ uint32_t gmax[kHierSortMax];
  __shared__ int32_t cmax[kRouteThreads / 64];
  __shared__ int wave_unc[kRouteThreads / 64];
  __shared__ int wave_rec[kRouteThreads / 64];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t wid = blockIdx.x;
  const int64_t bkv = wid % n_bkv;
  const int64_t tile = wid / n_bkv;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rows_total = n * g;
  const int64_t p0_tile = tile * kRouteRows;
  const int32_t* lst = list + bkv * rows_total;
  const uint32_t mask = (1u << key_bits) - 1u;
  const float qsc = ldexpf(1.f, -query_exponent(qmax[bkv]));
  f16x8 bq[2][NS];
  {
    const int64_t p0 = p0_tile + 64 * wave + ln, p1 = p0 + 32;
    const bool valid[2] = {p0 < rows_total, p1 < rows_total};
    const int64_t rho_of[2] = {valid[0] ? int64_t(lst[p0]) : 0, valid[1] ? int64_t(lst[p1]) : 0};
    load_q_tiles<false, D>(bq, Q, rho_of, valid, b, kv, g, hq, n, h, qsc);
  }
  const int64_t my_p = p0_tile + 64 * wave + 32 * h + ln;
  const bool my_valid = my_p < rows_total;
  const int64_t my_rho = my_valid ? int64_t(lst[my_p]) : 0;
  const int64_t my_t = my_valid ? split_rho(my_rho, g).t : 0;
  const int64_t my_C = my_valid ? min(nb, (my_t + 1) / B) : 0;
  const float* my_ub = ub + (bkv * rows_total + my_rho) * G;
  // the row's ||q||^2 (as the certification takes it) and its score error bound
  const float nq2 = row_norm2<D>(bq, h) * (1.f + 0x1p-16f);
  float e_row;
  {
    const float lam = __uint_as_float(bounds[bkv * 4 + 0]);
    const float Gs = __uint_as_float(bounds[bkv * 4 + 1]);
    const float nu = __uint_as_float(bounds[bkv * 4 + 2]);
    const float dm = __uint_as_float(bounds[bkv * 4 + 3]);
    e_row = 1.25f * (lam * nq2 + 0x1p-17f * (Gs * nq2 + nu * qsc * sqrtf(nq2)) +
                     0x1p-22f * (dm + Gs) * nq2);
  }
  // the tile's routable blocks (largest over its rows) and groups
  {
    int c = int(my_C);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c = max(c, __shfl_xor(c, o, 64));
    if (lane == 0) cmax[wave] = c;
  }
  for (int i = tid; i < kHierSortMax; i += kRouteThreads) gmax[i] = 0u;
  __syncthreads();
  int64_t C_wg = 0;
#pragma unroll
  for (int w = 0; w < kRouteThreads / 64; ++w) C_wg = max(C_wg, int64_t(cmax[w]));
  const int G_wg = int((C_wg + m - 1) / m);
  auto bound = [&](int gi) {
    return (my_valid && int64_t(gi) * m < my_C) ? my_ub[gi] : -__builtin_inff();
  };
  for (int gi = 0; gi < G_wg; ++gi) {
    const float u = bound(gi);
    const uint32_t bits = __float_as_uint(u);
    uint32_t o = bits ^ (uint32_t(int32_t(bits) >> 31) | 0x80000000u);
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) o = max(o, uint32_t(__shfl_xor(int(o), sh, 64)));
    if (lane == 0) atomicMax(&gmax[gi], o);
  }
  __syncthreads();
  // groups in decreasing order of that bound (lower group first among equal
  // bounds): a descending bitonic sort of (bound bits, ~group)
  int P = 1;
  while (P < G_wg) P <<= 1;
  for (int i = tid; i < P; i += kRouteThreads)
    order[i] = i < G_wg ? (uint64_t(gmax[i]) << 32) | uint64_t(0xFFFFFFFFu - uint32_t(i)) : 0;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size / 2; stride > 0; stride >>= 1) {
      for (int i = tid; i < P; i += kRouteThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const bool desc = (i & size) == 0;
          const uint64_t a = order[i], c = order[j];
          if (desc ? a < c : a > c) {
            order[i] = c;
            order[j] = a;
          }
        }
      }
      __syncthreads();
    }

  uint32_t lk[NL];   // running top-NL packed keys, descending (as the single pass)
#pragma unroll
  for (int i = 0; i < NL; ++i) lk[i] = 0u;
  // a lower bound on the exact k-th score of the blocks listed so far (-inf
  // until k are listed; +inf for k = 0: nothing is needed)
  auto kth_floor = [&]() {
    uint32_t kk = 0u;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (i == k - 1) kk = lk[i];
    if (k == 0) return __builtin_inff();
    return kk == 0u ? -__builtin_inff() : key_score(kk & ~mask) - e_row;
  };
  int scored = 0;
  const uint8_t* src = img + bkv * nb * int64_t(BYTES);
  for (int j = 0; j < G_wg; ++j) {
    const int gi = int(0xFFFFFFFFu - uint32_t(order[j] & 0xFFFFFFFFu));
    const float u = bound(gi);
    const bool need = __syncthreads_or(my_valid && !(u < kth_floor()));
    if (!need) continue;
    const int64_t c0 = int64_t(gi) * m, c1 = min(C_wg, c0 + m);
    stage_image<D>(src + c0 * BYTES, lds, wave, lane, kRouteThreads / 64);
    for (int64_t c = c0; c < c1; ++c) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();   // image c is in LDS; every wave is done with c - 1's buffer
      if (c + 1 < c1)
        stage_image<D>(src + (c + 1) * BYTES, lds + ((c + 1 - c0) & 1) * Lay::LDS_BYTES, wave,
                       lane, kRouteThreads / 64);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)   // (q stays in float16 registers; see hier_ub_kernel)
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) asm volatile("" : "+v"(bq[nt][s2]));
      const float a = hilo_score<D, false>(lds + ((c - c0) & 1) * Lay::LDS_BYTES, bq, lane);
      const uint32_t bits = __float_as_uint(a);
      const uint32_t o = bits ^ (uint32_t(int32_t(bits) >> 31) | 0x80000000u);
      uint32_t key = (c < my_C && a == a) ? (o & ~mask) | (mask - uint32_t(c)) : 0u;
#pragma unroll
      for (int i = 0; i < NL; ++i) {   // smaller first: no list copies per block
        const uint32_t v = lk[i];
        const uint32_t lower = min(v, key);
        lk[i] = max(v, key);
        key = lower;
      }
    }
    scored += int(c1 - c0);
    __syncthreads();   // the last image's buffer is free before the next group stages
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (evaluated != nullptr && tid == 0) evaluated[bkv * n_tiles + tile] = scored;
  certify_emit<KMAX>(lk, nq2, qsc, mask, bounds, bkv, tile, n_tiles, my_valid, my_rho, my_t, my_C,
                     wave_rec, wave_unc, tid, wave, lane, idx, tcnt, trows, rcnt, rmeta, rblk, rrank,
                     pcnt, fcnt, frow, fpos, n, g, hq, hkv, nb, k);
}

template <int D, int KMAX>
hipError_t launch_hier_prefill_t(const Shape& s, const void* Q, const float* mu,
                                 const float* sigma, const float* gmu, const float* gS,
                                 const float* grl, int m, int32_t* idx, int32_t* evaluated,
                                 void* ws, hipStream_t st) {
  const int64_t n_bkv = int64_t(s.b) * s.hkv;
  const int64_t n_tiles = route_tiles(s);
  const int64_t rows_total = s.n * s.g;
  const int64_t G = hier_groups(s, m);
  const HierWs w = hier_ws_layout(s, m, ws);
  const unsigned grid = unsigned(n_tiles * n_bkv);
  if (s.nb == 0) {
    // no complete block: every row gets -1 padding; no tile scores anything
    if (s.k > 0)
      hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned(std::min<int64_t>((n_bkv * rows_total * s.k + 255) / 256, 1024))),
                         dim3(256), 0, st, idx, int64_t(s.b) * s.hq * s.n * s.k, -1);
    if (evaluated != nullptr)
      hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned(std::min<int64_t>((grid + 255) / 256, 1024))),
                         dim3(256), 0, st, evaluated, int64_t(grid), 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<int32_t*>(w.qmax),
                     5 * n_bkv, 0);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st,
                     reinterpret_cast<int32_t*>(w.gbounds), 4 * n_bkv, 0);
  // counts of the last chunk's missing tiles stay zero
  const int64_t n_cnt = n_bkv * G * hier_chunks(n_tiles) * kHierChunk;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned(std::min<int64_t>((n_cnt + 255) / 256, 1024))),
                     dim3(256), 0, st, w.gcnt, n_cnt, 0);
  const int64_t per_group = int64_t(s.g) * s.n * D;
  const unsigned gx = value_max_groups(per_group);
  hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bkv)), dim3(256), 0, st,
                     static_cast<const bf16_t*>(Q), w.qmax, per_group);
  hipLaunchKernelGGL((route_prep_kernel<false, D>), dim3(unsigned(s.nb), unsigned(n_bkv)),
                     dim3(256), 0, st, mu, sigma, w.qmax, w.qmax + n_bkv, w.dbar, w.img, s.nb,
                     s.beta, sigma, s.nb);
  hipLaunchKernelGGL((route_prep_kernel<false, D>), dim3(unsigned(G), unsigned(n_bkv)),
                     dim3(256), 0, st, gmu, gS, w.qmax, w.gbounds, w.gdbar, w.gimg, G, s.beta,
                     sigma, s.nb);
  hipLaunchKernelGGL((hier_ub_kernel<D>), dim3(grid), dim3(kRouteThreads), 0, st,
                     static_cast<const bf16_t*>(Q), w.gimg, grl, w.qmax, w.gbounds, w.ub, w.best, w.gcnt,
                     s.n, s.g, s.hq, s.hkv, s.B, s.nb, m, G, n_tiles, n_bkv, s.beta);
  hipLaunchKernelGGL(route_scan_kernel, dim3(unsigned(n_bkv)), dim3(1024), 0, st, w.gcnt, w.goff,
                     w.gtot, G * hier_chunks(n_tiles) * kHierChunk);
  hipLaunchKernelGGL(hier_order_kernel, dim3(grid), dim3(kRouteThreads), 0, st, w.best, w.goff,
                     w.list, rows_total, G, n_tiles);
  int key_bits = 1;
  while ((int64_t(1) << key_bits) < s.nb) ++key_bits;
  if (s.k > 0 && key_bits <= kMaxKeyBits && n_tiles * kRecCap <= (int64_t(1) << 26)) {
    const RouteWs& rw = w.rw;
    route_resolve_clear(s, rw, n_bkv, st);
    hipLaunchKernelGGL((hier_visit_fast_kernel<D, KMAX>), dim3(grid), dim3(kRouteThreads), 0, st,
                       static_cast<const bf16_t*>(Q), rw.img, rw.qmax, rw.bounds, w.ub, w.list,
                       idx, evaluated, rw.tcnt, rw.trows, rw.rcnt, rw.rmeta, rw.rblk, rw.rrank,
                       rw.pcnt, rw.fcnt, rw.frow, rw.fpos, s.n, s.g, s.hq, s.hkv, s.B, s.nb, m, G,
                       s.k, key_bits, n_tiles, n_bkv);
    return route_resolve<D, KMAX>(s, Q, rw, idx, n_tiles, n_bkv, st);
  }
  // (k = 0, or keys or records out of the single pass's range) every needed
  // block scored exactly
  hipLaunchKernelGGL((hier_visit_kernel<D, KMAX>), dim3(grid), dim3(kRouteThreads), 0, st,
                     static_cast<const bf16_t*>(Q), w.img, w.qmax, w.ub, w.list, idx, evaluated,
                     s.n, s.g, s.hq, s.hkv, s.B, s.nb, m, G, s.k, n_tiles, n_bkv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_hier_prefill_d(const Shape& s, const void* Q, const float* mu,
                                 const float* sigma, const float* gmu, const float* gS,
                                 const float* grl, int m, int32_t* idx, int32_t* evaluated,
                                 void* ws, hipStream_t st) {
  if (s.k <= 8)
    return launch_hier_prefill_t<D, 8>(s, Q, mu, sigma, gmu, gS, grl, m, idx, evaluated, ws, st);
  if (s.k <= 16)
    return launch_hier_prefill_t<D, 16>(s, Q, mu, sigma, gmu, gS, grl, m, idx, evaluated, ws, st);
  return launch_hier_prefill_t<D, 32>(s, Q, mu, sigma, gmu, gS, grl, m, idx, evaluated, ws, st);
}

}  // namespace

size_t route_workspace_bytes(const Shape& s) { return route_ws_layout(s, nullptr).bytes; }

hipError_t launch_route_topk(const Shape& s, const void* Q, const float* mu, const float* sigma,
                             int32_t* idx, float* kth, void* ws, hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch_route_d<false, 64>(s, Q, mu, sigma, idx, kth, ws, st)
                     : launch_route_d<false, 128>(s, Q, mu, sigma, idx, kth, ws, st);
  return s.d == 64 ? launch_route_d<true, 64>(s, Q, mu, sigma, idx, kth, ws, st)
                   : launch_route_d<true, 128>(s, Q, mu, sigma, idx, kth, ws, st);
}

size_t route_hier_prefill_workspace_bytes(const Shape& s, int m) {
  return hier_ws_layout(s, m, nullptr).bytes;
}
int hier_prefill_max_groups() { return kHierSortMax; }
int64_t route_tile_count(const Shape& s) { return route_tiles(s); }

hipError_t launch_route_hier_prefill(const Shape& s, const void* Q, const float* mu,
                                     const float* sigma, const float* gmu, const float* gS,
                                     const float* grl, int m, int32_t* idx, int32_t* evaluated,
                                     void* ws, hipStream_t st) {
  return s.d == 64 ? launch_hier_prefill_d<64>(s, Q, mu, sigma, gmu, gS, grl, m, idx, evaluated, ws, st)
                   : launch_hier_prefill_d<128>(s, Q, mu, sigma, gmu, gS, grl, m, idx, evaluated, ws, st);
}

}  // namespace ssa
