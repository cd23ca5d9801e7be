// Sparse attention forward over the routed blocks and the local window (prefill).
//
// Write-up "Subquadratic Sparse Attention (SSA)", introduction steps (ii)-(iii):
// each query attends, with an exact softmax, to the keys of its selected
// blocks plus a local window.  Selections of neighbouring queries are
// unrelated, so a query-major gather would read every selected block once
// per query (~2 MB per query at d = 128, B = 256, k = 16).  The kernels here
// invert the selection instead:
//
//  1. dispatch  -- a counting sort of (query row, slot) pairs by selected
//     (sequence, KV head, block): per-workgroup LDS histograms, one exclusive
//     scan that also cuts every block's row list into tasks of at most
//     kTaskRows rows, and a scatter into the sorted entry list;
//  2. block attention -- one workgroup per task stages its block's K and V
//     once in LDS (64-key chunks, double-buffered), gathers the task's query
//     rows into MFMA registers, and writes one normalised partial per
//     (row, slot): o_i = softmax-weighted values over the block and
//     lse_i (base 2);
//  3. window + merge -- one workgroup per tile of consecutive query rows of a
//     KV head computes the window part as dense local attention (keys of
//     selected blocks masked out, so every key of S(t) counts once), then
//     merges it with the row's k partials into O and LSE.
//
// Every product runs on MFMA (bf16 32x32x16, or f32 32x32x2 for float32
// inputs) with float32 accumulation and a float32 online softmax in the
// base-2 domain.  Operand layouts follow frag_k (ssa_common.hpp): the
// probabilities leave the score accumulators and enter the value product in
// the same registers.
#include <algorithm>
#include <type_traits>

#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kAttnThreads = 256;          // 4 waves, 32 query rows each
constexpr int kTaskRows = 128;             // rows per block-attention task
constexpr int kWinRows = 128;              // rows per window/merge tile
constexpr int kKeyChunk = 64;              // keys per LDS chunk
constexpr int kHistTokens = 2048;          // tokens per dispatch workgroup
constexpr int kScanThreads = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <bool F32, int D>
struct AT {
  using In = typename std::conditional<F32, float, bf16_t>::type;
  using Frag = typename std::conditional<F32, floatx8, bf16x8>::type;
  static constexpr int ES = F32 ? 4 : 2;          // element bytes
  static constexpr int FRAG = 64 * 8 * ES;         // one operand fragment
  static constexpr int NS = D / 16;                // 16-wide chunks of d
  static constexpr int MTD = D / 32;               // 32-wide tiles of d
  static constexpr int KBYTES = 2 * NS * FRAG;     // 64 keys of K
  static constexpr int VBYTES = MTD * 4 * FRAG;    // 64 keys of V
  static constexpr int CHUNK = KBYTES + VBYTES;
  static constexpr int PIECE = 4 * ES;             // 4 elements
};

// ---------------------------------------------------------------- helpers --

template <bool F32, int D>
__device__ __forceinline__ typename AT<F32, D>::Frag load_row_frag(const typename AT<F32, D>::In* row,
                                                                   int s, int h, bool valid) {
  typename AT<F32, D>::Frag v;
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
  } else {
    u32x2 a = {0u, 0u}, b = a;
    if (valid) {
      a = *reinterpret_cast<const u32x2*>(row + 16 * s + 4 * h);
      b = *reinterpret_cast<const u32x2*>(row + 16 * s + 8 + 4 * h);
    }
    u32x4 w = {a[0], a[1], b[0], b[1]};
    v = __builtin_bit_cast(bf16x8, w);
  }
  return v;
}

// Stage keys [key0, key0 + 64) of one head (rows >= n_keys read as zero) into
// LDS as MFMA A-operand fragments:
//   K part: fragment (mt, s), lane (m, h), element e = K[key0 + 32mt + m][frag_k(s,h,e)]
//   V part: fragment (mt, s), lane (m, h), element e = V[key0 + frag_k(s,h,e)][32mt + m]
// Both are moved in 4-element pieces; V is transposed through registers in
// 4-key x 4-column tiles.
template <bool F32, int D>
__device__ __forceinline__ void stage_chunk(uint8_t* lds, const typename AT<F32, D>::In* Kh,
                                            const typename AT<F32, D>::In* Vh, int64_t key0,
                                            int64_t n_keys, int tid) {
  using A = AT<F32, D>;
  using PieceT = typename std::conditional<F32, floatx4, u32x2>::type;
  constexpr int PPR = D / 4;                 // pieces per key row
  constexpr int KP = kKeyChunk * PPR;        // K pieces in the chunk
  for (int w = tid; w < KP; w += kAttnThreads) {
    const int r = w / PPR, p = w % PPR;
    PieceT v = {};
    if (key0 + r < n_keys) v = *reinterpret_cast<const PieceT*>(Kh + (key0 + r) * D + 4 * p);
    const int mt = r / 32, m = r % 32, s = p / 4, h = p & 1, sel = (p >> 1) & 1;
    *reinterpret_cast<PieceT*>(lds + (mt * A::NS + s) * A::FRAG + (h * 32 + m) * 8 * A::ES +
                               sel * A::PIECE) = v;
  }
  constexpr int VT = (kKeyChunk / 4) * (D / 4);   // 4x4 tiles
  uint8_t* vl = lds + A::KBYTES;
  for (int w = tid; w < VT; w += kAttnThreads) {
    const int kq = w / (D / 4), dq = w % (D / 4);
    if constexpr (F32) {
      floatx4 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rows[r] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (key0 + 4 * kq + r < n_keys)
          rows[r] = *reinterpret_cast<const floatx4*>(Vh + (key0 + 4 * kq + r) * D + 4 * dq);
      }
      const int s = kq / 4, kg = kq % 4, sel = kg >> 1, h = kg & 1;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const int d = 4 * dq + dd, mt = d / 32, m = d % 32;
        floatx4 col = {rows[0][dd], rows[1][dd], rows[2][dd], rows[3][dd]};
        *reinterpret_cast<floatx4*>(vl + (mt * 4 + s) * A::FRAG + (h * 32 + m) * 8 * A::ES +
                                    sel * A::PIECE) = col;
      }
    } else {
      u32x2 rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        rows[r] = u32x2{0u, 0u};
        if (key0 + 4 * kq + r < n_keys)
          rows[r] = *reinterpret_cast<const u32x2*>(Vh + (key0 + 4 * kq + r) * D + 4 * dq);
      }
      const int s = kq / 4, kg = kq % 4, sel = kg >> 1, h = kg & 1;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const int d = 4 * dq + dd, mt = d / 32, m = d % 32;
        const int word = dd >> 1, shift = (dd & 1) * 16;
        const uint32_t e0 = (rows[0][word] >> shift) & 0xFFFFu, e1 = (rows[1][word] >> shift) & 0xFFFFu;
        const uint32_t e2 = (rows[2][word] >> shift) & 0xFFFFu, e3 = (rows[3][word] >> shift) & 0xFFFFu;
        u32x2 col = {e0 | (e1 << 16), e2 | (e3 << 16)};
        *reinterpret_cast<u32x2*>(vl + (mt * 4 + s) * A::FRAG + (h * 32 + m) * 8 * A::ES +
                                  sel * A::PIECE) = col;
      }
    }
  }
}

// Running softmax state of one query row, split over the two lane halves.
template <int D>
struct RowState {
  floatx16 o[D / 32];    // unnormalised output, lane half's columns
  float m2;              // running max of scaled logits (base 2), full row
  float l;               // this lane half's share of the running sum
};

template <int D>
__device__ __forceinline__ void row_state_init(RowState<D>& st) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) st.o[i][j] = 0.f;
  st.m2 = -__builtin_inff();
  st.l = 0.f;
}

// One 64-key chunk for the 32 rows of this wave.  mask(mt, a, b) says whether
// key 32mt + 8a + 4h + b of the chunk counts for this lane's row.
template <bool F32, int D, typename Mask>
__device__ __forceinline__ void attend_chunk(const uint8_t* lds,
                                             const typename AT<F32, D>::Frag (&bq)[D / 16],
                                             float scale2, int lane, RowState<D>& st, Mask mask) {
  using A = AT<F32, D>;
  using Frag = typename A::Frag;
  const int h = lane / 32;
  floatx16 sacc[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[mt][j] = 0.f;
#pragma unroll
    for (int s = 0; s < A::NS; ++s) {
      const Frag a = *reinterpret_cast<const Frag*>(lds + (mt * A::NS + s) * A::FRAG + lane * 8 * A::ES);
      sacc[mt] = mma16(a, bq[s], sacc[mt]);
    }
  }
  float mloc = -__builtin_inff();
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float v = sacc[mt][4 * a + b] * scale2;
        if (!mask(mt, a, b)) v = -__builtin_inff();
        sacc[mt][4 * a + b] = v;
        mloc = fmaxf(mloc, v);
      }
  mloc = fmaxf(mloc, wave_shfl_xor(mloc, 32));
  const float mnew = fmaxf(st.m2, mloc);
  const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(st.m2 - mref);
  st.m2 = mnew;
  float lsum = 0.f;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float p = __builtin_amdgcn_exp2f(sacc[mt][j] - mref);
      sacc[mt][j] = p;
      lsum += p;
    }
  st.l = st.l * alpha + lsum;
#pragma unroll
  for (int i = 0; i < A::MTD; ++i) st.o[i] *= alpha;
  // P as the B operand of O^T += V^T P^T: chunk s' covers keys 16s'..16s'+15
  const uint8_t* vl = lds + A::KBYTES;
#pragma unroll
  for (int sp = 0; sp < 4; ++sp) {
    // bfloat16 inputs: P = P_hi + P_lo, both contracted with the exact bf16 V,
    // so the product keeps ~2^-17 relative accuracy instead of 2^-9
    Frag pf, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = sacc[sp >> 1][4 * (2 * (sp & 1) + (e >> 2)) + (e & 3)];
      if constexpr (F32) {
        pf[e] = pv;
      } else {
        const __bf16 hi = static_cast<__bf16>(pv);
        pf[e] = hi;
        pl[e] = static_cast<__bf16>(pv - static_cast<float>(hi));
      }
    }
#pragma unroll
    for (int mt = 0; mt < A::MTD; ++mt) {
      const Frag a = *reinterpret_cast<const Frag*>(vl + (mt * 4 + sp) * A::FRAG + lane * 8 * A::ES);
      st.o[mt] = mma16(a, pf, st.o[mt]);
      if constexpr (!F32) st.o[mt] = mma16(a, pl, st.o[mt]);
    }
  }
  (void)h;
}

// ---------------------------------------------------------------- dispatch --

__global__ void fill_i32_kernel(int32_t* p, int64_t count, int32_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

// SCATTER = false: add this workgroup's histogram of selected blocks into
// counts.  SCATTER = true: reserve ranges at cursor and write entries
// (row id << 5 | slot) into the per-block lists.  A workgroup covers
// kHistTokens tokens of one (sequence, KV head) and all its group's q-heads.
template <bool SCATTER>
__global__ __launch_bounds__(256) void dispatch_kernel(const int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ counts_or_cursor,
                                                       uint32_t* __restrict__ entries, int64_t n,
                                                       int g, int hq, int hkv, int k, int64_t nb) {
  extern __shared__ int32_t hist[];
  const int tid = threadIdx.x;
  const int64_t bkv = blockIdx.y, b = bkv / hkv, kv = bkv % hkv;
  const int64_t t0 = int64_t(blockIdx.x) * kHistTokens;
  const int64_t t1 = min(n, t0 + kHistTokens);
  for (int64_t i = tid; i < nb; i += 256) hist[i] = 0;
  __syncthreads();
  for (int j = 0; j < g; ++j) {
    const int32_t* base = idx + ((b * hq + kv * g + j) * n) * k;
    for (int64_t t = t0 + tid; t < t1; t += 256)
      for (int i = 0; i < k; ++i) {
        const int32_t c = base[t * k + i];
        if (c >= 0 && c < nb) atomicAdd(&hist[c], 1);
      }
  }
  __syncthreads();
  int32_t* seg = counts_or_cursor + bkv * nb;
  for (int64_t i = tid; i < nb; i += 256) {
    const int32_t v = hist[i];
    if (v > 0) {
      const int32_t base = atomicAdd(&seg[i], v);
      if (SCATTER) hist[i] = base;
    }
  }
  if (!SCATTER) return;
  __syncthreads();
  for (int j = 0; j < g; ++j) {
    const int32_t* base = idx + ((b * hq + kv * g + j) * n) * k;
    for (int64_t t = t0 + tid; t < t1; t += 256)
      for (int i = 0; i < k; ++i) {
        const int32_t c = base[t * k + i];
        if (c >= 0 && c < nb) {
          const int32_t pos = atomicAdd(&hist[c], 1);
          entries[pos] = (uint32_t(t * g + j) << 5) | uint32_t(i);
        }
      }
  }
}

// Exclusive scan of the per-block counts (segment offsets, also copied to the
// scatter cursor) and of their task counts; emits the task list in block
// order: task = (segment, first entry, rows).
__global__ __launch_bounds__(kScanThreads) void scan_tasks_kernel(
    const int32_t* __restrict__ counts, int32_t* __restrict__ cursor, int4* __restrict__ tasks,
    int32_t* __restrict__ task_count, int64_t nseg) {
  constexpr int ITEMS = 4;
  __shared__ int32_t sc[kScanThreads], st[kScanThreads];
  __shared__ int32_t carry_c, carry_t;
  const int tid = threadIdx.x;
  if (tid == 0) {
    carry_c = 0;
    carry_t = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < nseg; base += int64_t(kScanThreads) * ITEMS) {
    int32_t c[ITEMS], tk[ITEMS], sum_c = 0, sum_t = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t s = base + int64_t(tid) * ITEMS + i;
      c[i] = s < nseg ? counts[s] : 0;
      tk[i] = (c[i] + kTaskRows - 1) / kTaskRows;
      sum_c += c[i];
      sum_t += tk[i];
    }
    sc[tid] = sum_c;
    st[tid] = sum_t;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
      const int32_t vc = tid >= off ? sc[tid - off] : 0;
      const int32_t vt = tid >= off ? st[tid - off] : 0;
      __syncthreads();
      sc[tid] += vc;
      st[tid] += vt;
      __syncthreads();
    }
    int32_t oc = carry_c + sc[tid] - sum_c, ot = carry_t + st[tid] - sum_t;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t s = base + int64_t(tid) * ITEMS + i;
      if (s < nseg) {
        cursor[s] = oc;
        for (int q = 0; q < tk[i]; ++q)
          tasks[ot + q] = int4{int32_t(s), oc + q * kTaskRows, min(kTaskRows, c[i] - q * kTaskRows), 0};
      }
      oc += c[i];
      ot += tk[i];
    }
    __syncthreads();
    if (tid == kScanThreads - 1) {
      carry_c += sc[tid];
      carry_t += st[tid];
    }
    __syncthreads();
  }
  if (tid == 0) task_count[0] = carry_t;
}

// ---------------------------------------------------------- block attention --

template <bool F32, int D, typename PartT>
__global__ __launch_bounds__(kAttnThreads) void block_attn_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const typename AT<F32, D>::In* __restrict__ K,
    const typename AT<F32, D>::In* __restrict__ V, const int4* __restrict__ tasks,
    const int32_t* __restrict__ task_count, const uint32_t* __restrict__ entries,
    PartT* __restrict__ o_part, float2* __restrict__ lse_part, int64_t n, int g, int hq, int hkv,
    int B, int64_t nb, int k, float scale2) {
  using A = AT<F32, D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int32_t T = *task_count;
  // XCD-aware order: consecutive tasks (same block) land on the same XCD.
  const int64_t per_xcd = (int64_t(T) + 7) / 8;
  const int64_t x = blockIdx.x;
  const int64_t ti = (x % 8) * per_xcd + x / 8;
  if (x / 8 >= per_xcd || ti >= T) return;
  const int4 task = tasks[ti];
  const int64_t seg = task.x, bkv = seg / nb, c = seg % nb;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;

  const int r = 32 * wave + ln;
  const bool valid = r < task.z;
  int64_t orow = 0;
  int slot = 0;
  typename A::Frag bq[A::NS];
  {
    int64_t t = 0, j = 0;
    if (valid) {
      const uint32_t code = entries[task.y + r];
      const int64_t rho = code >> 5;
      slot = int(code & 31u);
      t = rho / g;
      j = rho % g;
    }
    orow = (b * hq + kv * g + j) * n + t;
    const auto* qrow = Q + orow * D;
#pragma unroll
    for (int s = 0; s < A::NS; ++s) bq[s] = load_row_frag<F32, D>(qrow, s, h, valid);
  }
  const bool wave_active = 32 * wave < task.z;

  const auto* Kh = K + (bkv * n + c * B) * D;
  const auto* Vh = V + (bkv * n + c * B) * D;
  RowState<D> st;
  row_state_init(st);
  const int nchunks = B / kKeyChunk;
  stage_chunk<F32, D>(lds, Kh, Vh, 0, B, tid);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    if (ch + 1 < nchunks)
      stage_chunk<F32, D>(lds + ((ch + 1) & 1) * A::CHUNK, Kh, Vh, int64_t(ch + 1) * kKeyChunk, B, tid);
    if (wave_active)
      attend_chunk<F32, D>(lds + (ch & 1) * A::CHUNK, bq, scale2, lane, st,
                           [](int, int, int) { return true; });
    __syncthreads();
  }
  if (!valid) return;
  const float l = st.l + wave_shfl_xor(st.l, 32);
  const float inv = 1.f / l;
  // the partial is a convex combination of value rows; half-precision partials
  // are stored scaled by 2^-e with |o| < 2^e, so every entry keeps ~2^-12
  // relative accuracy of max|o| whatever the value range
  float mx = 0.f;
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(st.o[mt][j]));
  mx = fmaxf(mx, wave_shfl_xor(mx, 32)) * inv;
  int e = 0;
  if (!F32 && mx > 0.f) (void)frexpf(mx, &e);
  const float sc = ldexpf(inv, -e);
  const int64_t pidx = orow * k + slot;
  PartT* dst = o_part + pidx * D + h * (D / 2);
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j) store_from_f32(dst, mt * 16 + j, st.o[mt][j] * sc);
  if (h == 0) lse_part[pidx] = float2{st.m2 + __log2f(l), float(e)};
}

// ----------------------------------------------------------- window + merge --

template <bool F32, int D, typename PartT, typename OutT>
__global__ __launch_bounds__(kAttnThreads) void window_merge_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const typename AT<F32, D>::In* __restrict__ K,
    const typename AT<F32, D>::In* __restrict__ V, const int32_t* __restrict__ idx,
    const PartT* __restrict__ o_part, const float2* __restrict__ lse_part, OutT* __restrict__ O,
    float* __restrict__ lse, int64_t n, int g, int hq, int hkv, int B, int k, int W,
    float scale2, int64_t n_tiles) {
  using A = AT<F32, D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int32_t* sidx = reinterpret_cast<int32_t*>(lds + 2 * A::CHUNK);   // [kWinRows][k]
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t bkv = blockIdx.x / n_tiles;
  const int64_t tile = blockIdx.x % n_tiles;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rho0 = tile * kWinRows, rows_total = n * g;

  const int r = 32 * wave + ln;
  const int64_t rho = rho0 + r;
  const bool valid = rho < rows_total;
  const int64_t t = valid ? rho / g : 0, jg = valid ? rho % g : 0;
  const int64_t orow = (b * hq + kv * g + jg) * n + t;

  for (int w = tid; w < kWinRows * k; w += kAttnThreads) {
    const int rr = w / k, i = w % k;
    const int64_t rh = rho0 + rr;
    int32_t v = -1;
    if (rh < rows_total) {
      const int64_t tt = rh / g, jj = rh % g;
      v = idx[((b * hq + kv * g + jj) * n + tt) * k + i];
    }
    sidx[w] = v;
  }
  typename A::Frag bq[A::NS];
  {
    const auto* qrow = Q + orow * D;
#pragma unroll
    for (int s = 0; s < A::NS; ++s) bq[s] = load_row_frag<F32, D>(qrow, s, h, valid);
  }
  const int64_t t_lo = rho0 / g, t_hi = min(n - 1, (rho0 + kWinRows - 1) / g);
  const int64_t key_lo = max(int64_t(0), t_lo - W + 1);
  const int64_t ch0 = key_lo / kKeyChunk, ch1 = t_hi / kKeyChunk;
  const int64_t wave_t_lo = min(n - 1, (rho0 + 32 * wave) / g);
  const int64_t wave_t_hi = min(n - 1, (rho0 + 32 * wave + 31) / g);
  const bool wave_active = rho0 + 32 * wave < rows_total;

  const auto* Kh = K + bkv * n * D;
  const auto* Vh = V + bkv * n * D;
  RowState<D> st;
  row_state_init(st);
  stage_chunk<F32, D>(lds, Kh, Vh, ch0 * kKeyChunk, n, tid);
  __syncthreads();
  for (int64_t ch = ch0; ch <= ch1; ++ch) {
    const int buf = int((ch - ch0) & 1);
    if (ch + 1 <= ch1)
      stage_chunk<F32, D>(lds + (buf ^ 1) * A::CHUNK, Kh, Vh, (ch + 1) * kKeyChunk, n, tid);
    const int64_t key0 = ch * kKeyChunk;
    // does this wave's token range touch the chunk at all?
    const bool touch = wave_active && key0 <= wave_t_hi && key0 + kKeyChunk - 1 > wave_t_lo - W;
    if (touch) {
      // keys of a selected block already count in that block's partial
      const int32_t blk = int32_t(key0 / B);
      bool excl = false;
      for (int i = 0; i < k; ++i) excl |= sidx[r * k + i] == blk;
      const int64_t tv = valid ? t : -(int64_t(1) << 40);
      attend_chunk<F32, D>(lds + buf * A::CHUNK, bq, scale2, lane, st,
                           [&](int mt, int a, int bb) {
                             const int64_t j = key0 + 32 * mt + 8 * a + 4 * h + bb;
                             return !excl && j <= tv && j > tv - W;
                           });
    }
    __syncthreads();
  }
  if (!valid) return;
  // merge: window part (m2, l, o unnormalised) with the routed partials
  const float lw = st.l + wave_shfl_xor(st.l, 32);
  float M = lw > 0.f ? st.m2 + __log2f(lw) : -__builtin_inff();
  for (int i = 0; i < k; ++i)
    if (sidx[r * k + i] >= 0) M = fmaxf(M, lse_part[orow * k + i].x);
  const float ww = lw > 0.f ? __builtin_amdgcn_exp2f(st.m2 - M) : 0.f;
  float den = ww * lw;
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt) st.o[mt] *= ww;
  for (int i = 0; i < k; ++i) {
    if (sidx[r * k + i] < 0) continue;
    const int64_t pidx = orow * k + i;
    const float2 le = lse_part[pidx];
    const float wi = __builtin_amdgcn_exp2f(le.x - M);
    den += wi;
    const float ws = ldexpf(wi, int(le.y));
    const PartT* src = o_part + pidx * D + h * (D / 2);
#pragma unroll
    for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[mt][j] = fmaf(ws, load_f32(src, mt * 16 + j), st.o[mt][j]);
  }
  const float inv = 1.f / den;
  OutT* out = O + orow * D;
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
        store_from_f32(out, 32 * mt + 8 * a + 4 * h + bb, st.o[mt][4 * a + bb] * inv);
  if (h == 0) lse[orow] = (M + __log2f(den)) * kLn2;
}

// ------------------------------------------------------------------ launch --

struct AttnWs {
  int32_t* counts;
  int32_t* cursor;
  int32_t* task_count;
  int4* tasks;
  uint32_t* entries;
  float2* lse_part;
  void* o_part;
  size_t bytes;
  int64_t max_tasks;
};

AttnWs attn_ws_layout(const Shape& s, void* base) {
  AttnWs w{};
  const int64_t nseg = int64_t(s.b) * s.hkv * s.nb;
  const int64_t pairs = int64_t(s.b) * s.hq * s.n * s.k;
  w.max_tasks = (pairs + kTaskRows - 1) / kTaskRows + nseg;
  const size_t es = s.in_bf16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t o_counts = take(size_t(nseg) * 4), o_cursor = take(size_t(nseg) * 4);
  const size_t o_tc = take(4), o_tasks = take(size_t(w.max_tasks) * 16);
  const size_t o_entries = take(size_t(pairs) * 4), o_lse = take(size_t(pairs) * 8);
  const size_t o_part = take(size_t(pairs) * s.d * es);
  w.bytes = off;
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.counts = reinterpret_cast<int32_t*>(p + o_counts);
    w.cursor = reinterpret_cast<int32_t*>(p + o_cursor);
    w.task_count = reinterpret_cast<int32_t*>(p + o_tc);
    w.tasks = reinterpret_cast<int4*>(p + o_tasks);
    w.entries = reinterpret_cast<uint32_t*>(p + o_entries);
    w.lse_part = reinterpret_cast<float2*>(p + o_lse);
    w.o_part = p + o_part;
  }
  return w;
}

template <bool F32, int D, typename OutT>
hipError_t launch_attn_t(const Shape& s, const void* Qv, const void* Kv, const void* Vv,
                         const int32_t* idx, void* Ov, float* lse, void* ws, hipStream_t st) {
  using A = AT<F32, D>;
  using In = typename A::In;
  using PartT = typename std::conditional<F32, float, f16_t>::type;
  const In* Q = static_cast<const In*>(Qv);
  const In* K = static_cast<const In*>(Kv);
  const In* V = static_cast<const In*>(Vv);
  AttnWs w = attn_ws_layout(s, ws);
  const int64_t n_bkv = int64_t(s.b) * s.hkv;
  const int64_t nseg = n_bkv * s.nb;
  const float scale2 = s.scale * kLog2e;
  hipError_t e;
  if (s.k > 0 && nseg > 0) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned(std::min<int64_t>((nseg + 255) / 256, 4096))),
                       dim3(256), 0, st, w.counts, nseg, 0);
    const dim3 hgrid(unsigned((s.n + kHistTokens - 1) / kHistTokens), unsigned(n_bkv));
    const size_t hshm = size_t(s.nb) * 4;
    for (const void* f : {reinterpret_cast<const void*>(dispatch_kernel<false>),
                          reinterpret_cast<const void*>(dispatch_kernel<true>)})
      if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(hshm))) !=
          hipSuccess)
        return e;
    hipLaunchKernelGGL(dispatch_kernel<false>, hgrid, dim3(256), hshm, st, idx, w.counts,
                       (uint32_t*)nullptr, s.n, s.g, s.hq, s.hkv, s.k, s.nb);
    hipLaunchKernelGGL(scan_tasks_kernel, dim3(1), dim3(kScanThreads), 0, st, w.counts, w.cursor,
                       w.tasks, w.task_count, nseg);
    hipLaunchKernelGGL(dispatch_kernel<true>, hgrid, dim3(256), hshm, st, idx, w.cursor, w.entries,
                       s.n, s.g, s.hq, s.hkv, s.k, s.nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto bk = block_attn_kernel<F32, D, PartT>;
    const size_t bshm = 2 * size_t(A::CHUNK);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(bk),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(bshm))) != hipSuccess)
      return e;
    const int64_t grid = (w.max_tasks + 7) / 8 * 8;
    hipLaunchKernelGGL(bk, dim3(unsigned(grid)), dim3(kAttnThreads), bshm, st, Q, K, V, w.tasks,
                       w.task_count, w.entries, static_cast<PartT*>(w.o_part), w.lse_part, s.n,
                       s.g, s.hq, s.hkv, s.B, s.nb, s.k, scale2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  auto wk = window_merge_kernel<F32, D, PartT, OutT>;
  const size_t wshm = 2 * size_t(A::CHUNK) + size_t(kWinRows) * std::max(s.k, 1) * 4;
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(wk),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(wshm))) != hipSuccess)
    return e;
  const int64_t n_tiles = (s.n * s.g + kWinRows - 1) / kWinRows;
  hipLaunchKernelGGL(wk, dim3(unsigned(n_tiles * n_bkv)), dim3(kAttnThreads), wshm, st, Q, K, V,
                     idx, static_cast<const PartT*>(w.o_part), w.lse_part, static_cast<OutT*>(Ov),
                     lse, s.n, s.g, s.hq, s.hkv, s.B, s.k, s.W, scale2, n_tiles);
  return hipGetLastError();
}

template <bool F32, int D>
hipError_t launch_attn_d(const Shape& s, const void* Q, const void* K, const void* V,
                         const int32_t* idx, void* O, float* lse, void* ws, hipStream_t st) {
  if (s.out_bf16) return launch_attn_t<F32, D, bf16_t>(s, Q, K, V, idx, O, lse, ws, st);
  return launch_attn_t<F32, D, float>(s, Q, K, V, idx, O, lse, ws, st);
}

}  // namespace

size_t attn_workspace_bytes(const Shape& s) { return attn_ws_layout(s, nullptr).bytes; }

hipError_t launch_sparse_attn(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* idx, void* O, float* lse, void* ws, hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch_attn_d<false, 64>(s, Q, K, V, idx, O, lse, ws, st)
                     : launch_attn_d<false, 128>(s, Q, K, V, idx, O, lse, ws, st);
  return s.d == 64 ? launch_attn_d<true, 64>(s, Q, K, V, idx, O, lse, ws, st)
                   : launch_attn_d<true, 128>(s, Q, K, V, idx, O, lse, ws, st);
}

}  // namespace ssa
