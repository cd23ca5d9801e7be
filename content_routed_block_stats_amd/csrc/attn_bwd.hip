// Backward of the sparse attention over fixed selections (prefill).
//
// Write-up "Subquadratic Sparse Attention (SSA)": its module list trains SSA
// models and its "Selected results" adapt a dense model swapped to SSA, so
// gradients flow through the layer; the selection is a discrete choice and is
// held fixed.  For every row t with key set S(t) (introduction steps ii-iii):
//   p_j = softmax_j(scale q.k_j) = exp(scale q.k_j - LSE),  D = dO . O,
//   dP_j = dO . v_j,  dS_j = p_j (dP_j - D),
//   dq = scale sum_j dS_j k_j,  dk_j += scale dS_j q,  dv_j += p_j dO,
// with the forward's LSE, so no softmax is re-normalised.
//
//  1. rowdot     -- D per row (float32), from the forward's O and dO;
//  2. dq_task    -- the forward's block-major tasks again (lanes on rows, as in
//     the forward): per 64-key chunk of the task's block, S^T = K Q^T and
//     dP^T = V dO^T on MFMA, dS^T on the vector units, dQ^T += K^T dS^T on
//     MFMA; one float32 dQ partial per (row, selected block);
//  3. dkv_chunk  -- one workgroup per 64-key chunk of a KV head owns those
//     keys' dK and dV (no atomics across workgroups): it streams every row
//     that attends to them -- the block's selected rows from the dispatch,
//     then the window rows whose window reaches the chunk and whose selection
//     does not hold the block -- and, with lanes on keys, computes S = Q K^T,
//     dP = dO V^T, dS, then dV^T += dO^T P and dK^T += Q^T dS on MFMA;
//  4. dq_window  -- per tile of 128 rows, the window part of dQ (window keys
//     outside the row's selected blocks) plus the row's dQ partials.
//
// Operands: K and V rows (bf16, exact) as they are; K^T, Q^T, dO^T and the
// probabilities / dS enter their products as float16, each tensor scaled by an
// exact power of two that keeps its largest value below 2^15 (bf16 values in
// the float16 normal range convert exactly); float32 inputs use float32 MFMA
// throughout.  Chunk images come from kv_image_kernel: image A = (K rows,
// V^T), image B = (V rows, K^T).
#include <algorithm>
#include <type_traits>

#include "kv_chunks.hpp"
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kDqThreads = 256;      // dQ task pass: 4 waves, half a task; two workgroups per CU
constexpr int kDkvThreads = 256;     // key pass: 4 waves, two workgroups per CU
constexpr int kDkvRows = 64;         // rows staged per iteration of the key pass
constexpr int kWinTile = 128;        // rows per tile of the window pass (4 waves x 32)
constexpr int kDkvWideThreads = 512;  // key pass over chunk pairs: 8 waves, one workgroup per CU
constexpr int kDkvWideWinRows = 16384;  // window rows a chunk pair can have (a byte of LDS each)

// ------------------------------------------------------------------ rowdot --
template <typename InT, typename OutT>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const InT* __restrict__ dO,
                                                         const OutT* __restrict__ O,
                                                         float* __restrict__ Drow, int64_t rows,
                                                         int D) {
  const int lane = threadIdx.x % 64;
  const int64_t r = int64_t(blockIdx.x) * 4 + threadIdx.x / 64;
  if (r >= rows) return;
  float acc = 0.f;
  for (int i = lane; i < D; i += 64) acc += load_f32(dO, r * D + i) * load_f32(O, r * D + i);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc += wave_shfl_xor(acc, o);
  if (lane == 0) Drow[r] = acc;
}

// float16 fragment of 8 values (or float32 for float32 inputs)
template <bool F32>
using VF = typename std::conditional<F32, floatx8, f16x8>::type;

template <bool F32>
__device__ __forceinline__ void set_vf(VF<F32>& f, int e, float v) {
  if constexpr (F32) f[e] = v; else f[e] = static_cast<_Float16>(v);
}

// A whole fragment from eight float32 values (float16: converted in pairs).
template <bool F32>
__device__ __forceinline__ VF<F32> make_vf(const float (&v)[8]) {
  if constexpr (F32) {
    VF<F32> f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = v[e];
    return f;
  } else {
    return to_f16x8(v);
  }
}

// ----------------------------------------------------------------- dq_task --
// Two workgroups (4 waves x 32 rows each) per task of up to 256 rows, two per
// CU; chunk images of the task's block in LDS (image A's K part, then all of
// image B), double-buffered where two workgroups still fit.
template <bool F32, int D>
__global__ __launch_bounds__(kDqThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_task_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const typename AT<F32, D>::In* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Drow, const uint8_t* __restrict__ img_a,
    const uint8_t* __restrict__ img_b, const uint32_t* __restrict__ kmax, int64_t n_chunks,
    const int4* __restrict__ tasks, const int32_t* __restrict__ task_count,
    const uint32_t* __restrict__ entries, uint8_t* __restrict__ dq_part, float* __restrict__ dq_sc,
    int64_t n, int g, int hq,
    int hkv, int B, int64_t nb, float scale2, float scale) {
  using A = AT<F32, D>;
  using Frag = typename A::Frag;
  constexpr int BUF = A::KBYTES + A::CHUNK;
  // double-buffered chunks only where two workgroups still fit a CU's LDS
  constexpr int NBUF = 2 * BUF <= 64 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * BUF];
  // two workgroups per task, 128 rows each, so that two share a CU and one's
  // row gather overlaps the other's products
  const int64_t task = blockIdx.x / 2;
  const int half = blockIdx.x % 2;
  if (task >= task_count[0]) return;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int4 tk = tasks[task];
  const int64_t seg = tk.x, e0 = tk.y;
  const int rows = tk.z;
  if (128 * half >= rows) return;
  const int64_t bkv = seg / nb, c = seg % nb, b = bkv / hkv, kv = bkv % hkv;
  const int r = 128 * half + 32 * wave + ln;
  const bool valid = r < rows;
  int64_t row = 0;
  if (valid) {
    const uint32_t en = entries[e0 + r];
    const RowTJ q = split_rho(en >> 5, g);
    const int64_t t = q.t, jg = q.jg;
    row = (b * hq + kv * g + jg) * n + t;
  }
  Frag bq[A::NS], bdo[A::NS];
#pragma unroll
  for (int s = 0; s < A::NS; ++s) {
    bq[s] = load_row_frag<F32, D>(Q + row * D, s, h, valid);
    bdo[s] = load_row_frag<F32, D>(dO + row * D, s, h, valid);
  }
  const float l2 = valid ? lse[row] * kLog2e : 0.f;
  const float dr = valid ? Drow[row] : 0.f;
  const bool wave_active = 128 * half + 32 * wave < rows;
  const int cpb = B / kKeyChunk;
  const int64_t ch0 = c * cpb;
  const uint8_t* srca = img_a + bkv * n_chunks * A::CHUNK;
  const uint8_t* srcb = img_b + bkv * n_chunks * A::CHUNK;
  floatx16 dq[A::MTD];
#pragma unroll
  for (int i = 0; i < A::MTD; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dq[i][j] = 0.f;

  dma_copy(lds, srca + ch0 * A::CHUNK, A::KBYTES, tid, kDqThreads);
  dma_copy(lds + A::KBYTES, srcb + ch0 * A::CHUNK, A::CHUNK, tid, kDqThreads);
  __syncthreads();
  for (int q = 0; q < cpb; ++q) {
    uint8_t* L = lds + (q % NBUF) * BUF;
    if (NBUF == 2 && q + 1 < cpb) {
      uint8_t* Ln = lds + ((q + 1) % NBUF) * BUF;
      dma_copy(Ln, srca + (ch0 + q + 1) * A::CHUNK, A::KBYTES, tid, kDqThreads);
      dma_copy(Ln + A::KBYTES, srcb + (ch0 + q + 1) * A::CHUNK, A::CHUNK, tid, kDqThreads);
    }
    if (wave_active) {
      auto fa = [&](const uint8_t* base, int mt, int s) {
        return *reinterpret_cast<const Frag*>(base + (mt * A::NS + s) * A::FRAG + lane * 8 * A::ES);
      };
      floatx16 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[mt][j] = pacc[mt][j] = 0.f;
#pragma unroll
      for (int s = 0; s < A::NS; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          sacc[mt] = mma16(fa(L, mt, s), bq[s], sacc[mt]);                  // K rows . q
          pacc[mt] = mma16(fa(L + A::KBYTES, mt, s), bdo[s], pacc[mt]);     // V rows . dO
        }
      // dS^T in the accumulators (keys 32mt + 8a + 4h + b of this lane's row)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][j], scale2, -l2));
          sacc[mt][j] = p * (pacc[mt][j] - dr);
        }
      // dQ^T += K^T dS^T: image B's transposed part as A, dS^T as B (frag_k)
      const uint8_t* kt = L + A::KBYTES + A::KBYTES;
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = sacc[sp >> 1][4 * (2 * (sp & 1) + (e >> 2)) + (e & 3)];
        const VF<F32> pf = make_vf<F32>(pv);
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt)
          dq[mt] = mma16(*reinterpret_cast<const typename A::VFrag*>(kt + (mt * 4 + sp) * A::FRAG +
                                                                      lane * 8 * A::ES),
                         pf, dq[mt]);
      }
    }
    __syncthreads();
    if (NBUF == 1 && q + 1 < cpb) {
      dma_copy(lds, srca + (ch0 + q + 1) * A::CHUNK, A::KBYTES, tid, kDqThreads);
      dma_copy(lds + A::KBYTES, srcb + (ch0 + q + 1) * A::CHUNK, A::CHUNK, tid, kDqThreads);
      __syncthreads();
    }
  }
  if (!valid) return;   // (both lane halves of a row share it)
  const float f = ldexpf(scale, F32 ? 0 : value_exponent(kmax[bkv]));
  if constexpr (F32) {
    float* out = reinterpret_cast<float*>(dq_part) + (e0 + r) * D;
#pragma unroll
    for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<floatx4*>(out + 32 * mt + 8 * a + 4 * h) =
            floatx4{dq[mt][4 * a] * f, dq[mt][4 * a + 1] * f, dq[mt][4 * a + 2] * f,
                    dq[mt][4 * a + 3] * f};
  } else {
    // float16 scaled by a power of two per partial: the row's largest |value|
    // lands in [2^14, 2^15) (relative rounding 2^-11 of that maximum)
    float m = 0.f;
#pragma unroll
    for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) m = fmaxf(m, fabsf(dq[mt][j]));
    m = fmaxf(m, wave_shfl_xor(m, 32)) * f;
    int e = 0;
    if (m > 0.f && m < __builtin_inff()) (void)frexpf(m, &e);   // m < 2^e
    const float sc = ldexpf(f, 15 - e);
    u16* out = reinterpret_cast<u16*>(dq_part) + (e0 + r) * D;
#pragma unroll
    for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        uint32_t w2[2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
          w2[i] = pack_f16x2(dq[mt][4 * a + 2 * i] * sc, dq[mt][4 * a + 2 * i + 1] * sc);
        *reinterpret_cast<uint2*>(out + 32 * mt + 8 * a + 4 * h) = uint2{w2[0], w2[1]};
      }
    if (h == 0) dq_sc[e0 + r] = ldexpf(1.f, e - 15);
  }
}

// --------------------------------------------------------------- dkv_chunk --
// One workgroup (4 waves: key half kh = wave % 2, row group rg = wave / 2) per
// 64-key chunk of one (sequence, KV head); two workgroups share a CU.  Rows
// are staged kDkvRows at a time: Q and dO rows as they are, and per row its
// index, position, log2-domain LSE, D and mode (0 = every key counts, 1 =
// window keys (t - W, t], 2 = none).  The next rows' information is fetched
// while the current rows are computed, so an iteration waits for one gather.
template <bool F32, int D>
__global__ __launch_bounds__(kDkvThreads) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkv_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const typename AT<F32, D>::In* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Drow, const int32_t* __restrict__ idx,
    const uint8_t* __restrict__ img_a, const uint8_t* __restrict__ img_b,
    const uint32_t* __restrict__ qmax, const uint32_t* __restrict__ domax, int64_t n_chunks,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ cursor,
    const uint32_t* __restrict__ entries, float* __restrict__ dK, float* __restrict__ dV, int64_t n,
    int g, int hq, int hkv, int B, int64_t nb, int k, int W, float scale2, float scale,
    int64_t n_work) {
  using A = AT<F32, D>;
  using In = typename A::In;
  using Frag = typename A::Frag;
  constexpr int ES = A::ES;
  constexpr int ROWB = D * ES;
  constexpr int RSTR = ROWB + 16;      // padded row stride: a wave's row reads spread over banks
  constexpr int ROWS = kDkvRows;
  constexpr int TRS = ROWS + 4;        // transposed float16 copy: halves per column
  __shared__ __attribute__((aligned(1024))) uint8_t img[2 * A::KBYTES];   // K rows, V rows
  __shared__ __attribute__((aligned(16))) uint8_t rbuf[2 * ROWS * RSTR];  // Q rows, dO rows
  __shared__ float rl2[ROWS], rd[ROWS];
  __shared__ int64_t rrow[ROWS], rpos[ROWS];
  __shared__ int32_t rmode[ROWS];
  static_assert(2 * ROWS * RSTR >= kKeyChunk * D * 4, "reduction buffer");
  static_assert(D * TRS * 2 <= ROWS * RSTR, "transposed copy");
  uint8_t* rq = rbuf;
  uint8_t* rdo = rbuf + ROWS * RSTR;

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int kh = wave % 2, rg = wave / 2;
  // consecutive work items (the chunks of one block, which stream the same
  // selected rows) go to one XCD (workgroup i runs on XCD i % 8), so the
  // repeated row gathers hit that XCD's L2
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t wi = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (wi >= n_work) return;
  const int64_t ch = wi % n_chunks, bkv = wi / n_chunks;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t key0 = ch * kKeyChunk;
  const int64_t c = key0 / B;
  int64_t sel_start = 0, sel_cnt = 0;
  if (c < nb) {
    const int64_t sg = bkv * nb + c;
    sel_cnt = counts[sg];
    sel_start = cursor[sg] - sel_cnt;
  }
  const int64_t t_hi = min(n - 1, key0 + kKeyChunk - 1 + W - 1);
  const int64_t win_cnt = (t_hi - key0 + 1) * g;
  const int64_t total = sel_cnt + win_cnt;
  // float16 scales of Q^T and dO^T for this KV head's group of q-heads
  int eq = 0, edo = 0;
  if constexpr (!F32) {
    uint32_t mq = 0, md = 0;
    for (int j = 0; j < g; ++j) {
      mq = max(mq, qmax[b * hq + kv * g + j]);
      md = max(md, domax[b * hq + kv * g + j]);
    }
    eq = value_exponent(mq);
    edo = value_exponent(md);
  }
  const float sq = ldexpf(1.f, -eq), sdo = ldexpf(1.f, -edo);

  // row i of this work item: the block's selected rows, then the window rows
  struct Info {
    int64_t row, pos;
    float l2, dd;
    int mode;
  };
  auto info = [&](int64_t i) {
    Info r{-1, -1, 0.f, 0.f, 2};
    if (i < sel_cnt) {
      const uint32_t en = entries[sel_start + i];
      const int64_t rho = en >> 5;
      const RowTJ q = split_rho(rho, g);
      r.pos = q.t;
      r.row = (b * hq + kv * g + q.jg) * n + r.pos;
      r.mode = 0;
    } else if (i < total) {
      const int64_t w = i - sel_cnt;
      r.pos = key0 + w / g;
      r.row = (b * hq + kv * g + w % g) * n + r.pos;
      bool sel = false;
      for (int q = 0; q < k; ++q) sel |= idx[r.row * k + q] == int32_t(c);
      r.mode = sel ? 2 : 1;
    }
    if (r.row >= 0) {
      r.l2 = lse[r.row] * kLog2e;
      r.dd = Drow[r.row];
    }
    return r;
  };
  auto put = [&](const Info& r) {
    rrow[tid] = r.mode == 2 ? -1 : r.row;
    rpos[tid] = r.pos;
    rl2[tid] = r.l2;
    rd[tid] = r.dd;
    rmode[tid] = r.mode;
  };

  dma_copy(img, img_a + (bkv * n_chunks + ch) * A::CHUNK, A::KBYTES, tid, kDkvThreads);
  dma_copy(img + A::KBYTES, img_b + (bkv * n_chunks + ch) * A::CHUNK, A::KBYTES, tid, kDkvThreads);
  if (tid < ROWS) put(info(tid));

  floatx16 dk[A::MTD], dv[A::MTD];
#pragma unroll
  for (int i = 0; i < A::MTD; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dk[i][j] = dv[i][j] = 0.f;
  const int64_t my_key = key0 + 32 * kh + ln;

  for (int64_t i0 = 0; i0 < total; i0 += ROWS) {
    __syncthreads();   // this iteration's row information is in LDS
    constexpr int PIECES = ROWB / 16;
    for (int w = tid; w < ROWS * PIECES; w += kDkvThreads) {
      const int rr = w / PIECES, pc = w % PIECES;
      const int64_t row = rrow[rr];
      u32x4 vq = {0u, 0u, 0u, 0u}, vd = vq;
      if (row >= 0) {
        vq = reinterpret_cast<const u32x4*>(Q + row * D)[pc];
        vd = reinterpret_cast<const u32x4*>(dO + row * D)[pc];
      }
      reinterpret_cast<u32x4*>(rq + rr * RSTR)[pc] = vq;
      reinterpret_cast<u32x4*>(rdo + rr * RSTR)[pc] = vd;
    }
    __syncthreads();   // rows staged
    // the next rows' information, fetched while these rows are computed (the
    // loads go out after the barrier above, whose fence would wait for them)
    Info nx{-1, -1, 0.f, 0.f, 2};
    if (tid < ROWS && i0 + ROWS < total) nx = info(i0 + ROWS + tid);

    const int r0 = 32 * rg;
    const bool active = i0 + r0 < total;
    floatx16 sacc, pacc;
    if (active) {
      // S = Q K^T and dP = dO V^T for this wave's 32 rows x 32 keys (lanes on keys)
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[j] = pacc[j] = 0.f;
#pragma unroll
      for (int s = 0; s < A::NS; ++s) {
        const Frag kf = *reinterpret_cast<const Frag*>(img + (kh * A::NS + s) * A::FRAG + lane * 8 * ES);
        const Frag vf = *reinterpret_cast<const Frag*>(img + A::KBYTES + (kh * A::NS + s) * A::FRAG +
                                                       lane * 8 * ES);
        const Frag qa = *reinterpret_cast<const Frag*>(rq + (r0 + ln) * RSTR + (16 * s + 8 * h) * ES);
        const Frag da = *reinterpret_cast<const Frag*>(rdo + (r0 + ln) * RSTR + (16 * s + 8 * h) * ES);
        sacc = mma16(qa, kf, sacc);
        pacc = mma16(da, vf, pacc);
      }
      // element j: row r0 + 8(j/4) + 4h + j%4, key my_key
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int rr = r0 + 8 * (j / 4) + 4 * h + j % 4;
        const int mode = rmode[rr];
        const int64_t t = rpos[rr];
        // (computed for every element and selected: a conditional exponential
        // becomes a branch per element)
        const bool on = (my_key < n) & ((mode == 0) | ((mode == 1) & (my_key <= t) & (my_key > t - W)));
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[j], scale2, -rl2[rr]));
        const float p = on ? e : 0.f;
        sacc[j] = p;
        pacc[j] = p * (pacc[j] - rd[rr]);
        if (j % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // four rows' reads in flight at a time
      }
    }
    if constexpr (!F32) {
      // Q^T and dO^T as scaled float16, [column][row] (TRS halves per column),
      // written over the row-major copy once every wave has read it.  Thread
      // unit: rows 2 rp, 2 rp + 1 and columns [8 pc, 8 pc + 8); a wave takes 8
      // row pairs x 8 column groups, D / 64 units per thread.
      static_assert(ROWS == 64 && kDkvThreads == 256, "unit map: 32 row pairs over 4 waves");
      constexpr int UNITS = D / 64;
      u32x4 pq[UNITS][2], pd[UNITS][2];
#pragma unroll
      for (int j = 0; j < UNITS; ++j) {
        const int rp = 8 * wave + lane % 8, pc = lane / 8 + 8 * j;
#pragma unroll
        for (int o = 0; o < 2; ++o) {
          pq[j][o] = *reinterpret_cast<const u32x4*>(rq + (2 * rp + o) * RSTR + pc * 16);
          pd[j][o] = *reinterpret_cast<const u32x4*>(rdo + (2 * rp + o) * RSTR + pc * 16);
        }
      }
      __syncthreads();   // every wave has read the row-major copy
#pragma unroll
      for (int j = 0; j < UNITS; ++j) {
        const int rp = 8 * wave + lane % 8, pc = lane / 8 + 8 * j;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int sh = 16 * (i % 2);
          const float q0 = __builtin_bit_cast(float, ((pq[j][0][i / 2] >> sh) & 0xFFFFu) << 16) * sq;
          const float q1 = __builtin_bit_cast(float, ((pq[j][1][i / 2] >> sh) & 0xFFFFu) << 16) * sq;
          const float d0 = __builtin_bit_cast(float, ((pd[j][0][i / 2] >> sh) & 0xFFFFu) << 16) * sdo;
          const float d1 = __builtin_bit_cast(float, ((pd[j][1][i / 2] >> sh) & 0xFFFFu) << 16) * sdo;
          const uint32_t wq = pack_f16x2(q0, q1), wd = pack_f16x2(d0, d1);
          const int at = ((8 * pc + i) * TRS + 2 * rp) * 2;
          *reinterpret_cast<uint32_t*>(rq + at) = wq;
          *reinterpret_cast<uint32_t*>(rdo + at) = wd;
        }
      }
      __syncthreads();   // the transposed copies are complete
    }
    if (active) {
      // dV^T += dO^T P and dK^T += Q^T dS: rows contracted in frag_k order
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        float pv[8], sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 4 * (2 * sp + (e >> 2)) + (e & 3);
          pv[e] = sacc[j];
          sv[e] = pacc[j];
        }
        const VF<F32> pf = make_vf<F32>(pv), sf = make_vf<F32>(sv);
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt) {
          VF<F32> qt, dt;
          const int col = 32 * mt + ln;
          if constexpr (F32) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int rr = r0 + frag_k(sp, h, e);
              set_vf<F32>(qt, e, load_f32(reinterpret_cast<const In*>(rq + rr * RSTR), col) * sq);
              set_vf<F32>(dt, e, load_f32(reinterpret_cast<const In*>(rdo + rr * RSTR), col) * sdo);
            }
          } else {
            // rows r0 + frag_k(sp, h, e): 4 consecutive rows, then 4 more 8 rows on
            const int at = (col * TRS + r0 + 16 * sp + 4 * h) * 2;
            const uint2 q_lo = *reinterpret_cast<const uint2*>(rq + at);
            const uint2 q_hi = *reinterpret_cast<const uint2*>(rq + at + 16);
            const uint2 d_lo = *reinterpret_cast<const uint2*>(rdo + at);
            const uint2 d_hi = *reinterpret_cast<const uint2*>(rdo + at + 16);
            qt = __builtin_bit_cast(f16x8, u32x4{q_lo.x, q_lo.y, q_hi.x, q_hi.y});
            dt = __builtin_bit_cast(f16x8, u32x4{d_lo.x, d_lo.y, d_hi.x, d_hi.y});
          }
          dv[mt] = mma16(dt, pf, dv[mt]);
          dk[mt] = mma16(qt, sf, dk[mt]);
        }
      }
    }
    __syncthreads();   // done with this iteration's rows and information
    if (tid < ROWS) put(nx);
  }
  __syncthreads();

  // the two row groups' partial sums, added in LDS in a fixed order (float32,
  // 64 keys x D): the result does not depend on scheduling
  float* red = reinterpret_cast<float*>(rbuf);
  for (int pass = 0; pass < 2; ++pass) {
    for (int round = 0; round < 2; ++round) {
      if (rg == round) {
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int col = 32 * mt + 8 * (j / 4) + 4 * h + j % 4;
            float* slot = &red[(32 * kh + ln) * D + col];
            const float v = pass == 0 ? dk[mt][j] : dv[mt][j];
            *slot = round == 0 ? v : *slot + v;
          }
      }
      __syncthreads();
    }
    const float f = pass == 0 ? ldexpf(scale, eq) : ldexpf(1.f, edo);
    float* dst = (pass == 0 ? dK : dV) + (bkv * n + key0) * D;
    for (int w = tid; w < kKeyChunk * D; w += kDkvThreads)
      if (key0 + w / D < n) dst[w] = red[w] * f;
    __syncthreads();
  }
}

// ---------------------------------------------------------- dkv_chunk_pair --
// The same pass for bfloat16 inputs at d = 128 when blocks hold a multiple of
// 128 keys: one workgroup of 8 waves (key quarter kq = wave % 4, row group
// rg = wave / 4) owns two consecutive chunks, so every staged row serves 128
// keys and a CU holds one workgroup.  The LDS this frees holds a second row
// buffer: the next batch's rows are copied global -> LDS directly (no
// registers) during the whole of the current batch, whose two inner barriers
// wait for LDS traffic only (the one that opens a batch waits for the copy).
// No ordinary load is waited for while such a copy is in flight except at the
// end of a batch, where the copy has to be complete anyway (the compiler
// counts the copies as stores, so any such wait drains them): row information
// is loaded two batches ahead and stored at the end of a batch, and whether a
// window row's selection holds the block is decided once, in the prologue,
// into a byte per window row.  Padded rows are copied whole: the padding slot
// of a row repeats its last 16 bytes.

// Workgroup barrier over LDS accesses only: global loads still in flight
// (the global -> LDS row copies among them) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(kDkvWideThreads) void bwd_dkv_wide_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ dO, const float* __restrict__ lse,
    const float* __restrict__ Drow, const int32_t* __restrict__ idx,
    const uint8_t* __restrict__ img_a, const uint8_t* __restrict__ img_b,
    const uint32_t* __restrict__ qmax, const uint32_t* __restrict__ domax, int64_t n_chunks,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ cursor,
    const uint32_t* __restrict__ entries, float* __restrict__ dK, float* __restrict__ dV, int64_t n,
    int g, int hq, int hkv, int B, int64_t nb, int k, int W, float scale2, float scale,
    int64_t n_work) {
  using A = AT<false, D>;
  using Frag = typename A::Frag;
  constexpr int ES = 2;
  constexpr int ROWB = D * ES;
  constexpr int RSTR = ROWB + 16;           // padded row stride, as in the chunk pass
  constexpr int SLOTS = RSTR / 16;          // 16-byte slots per staged row (the last is padding)
  constexpr int ROWS = kDkvRows;
  constexpr int TRS = ROWS + 4;
  constexpr int TBYTES = ROWS * RSTR;       // one tensor's staged rows
  constexpr int NCOPY = TBYTES / 1024;      // 1 KB global -> LDS copies per tensor
  constexpr int KEYS = 2 * kKeyChunk;
  constexpr int NW = kDkvWideThreads / 64;
  static_assert(TBYTES % 1024 == 0, "row buffers are whole 1 KB copies");
  static_assert(D * TRS * 2 <= TBYTES, "transposed copy");
  static_assert(4 * A::KBYTES >= KEYS * D * 4, "reduction buffer");
  static_assert(ROWS == 64 && NW == 8 && D == 128, "unit map: 32 row pairs x 16 column groups over 8 waves");
  __shared__ __attribute__((aligned(1024))) uint8_t img[4 * A::KBYTES];    // K rows of both chunks, then V rows
  // row buffers of even and odd batches (Q rows, then dO rows); two separate
  // arrays, so that reads of one are known not to touch the copy into the other
  __shared__ __attribute__((aligned(1024))) uint8_t rbuf0[2 * TBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t rbuf1[2 * TBYTES];
  // per staged row: the keys it attends here, (lo, hi], its LSE and D; its
  // index for the row copy
  __shared__ __attribute__((aligned(16))) int32_t rlo[2][ROWS], rhi[2][ROWS];
  __shared__ __attribute__((aligned(16))) float rlse[2][ROWS], rd[2][ROWS];
  __shared__ int64_t rrow[2][ROWS];
  __shared__ uint8_t wmode[kDkvWideWinRows];   // window row w: 1 = window keys count, 2 = none

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int kq = wave % 4, rg = wave / 4;
  // consecutive work items (the chunk pairs of one block) go to one XCD
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t wi = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (wi >= n_work) return;
  const int64_t n_pairs = (n_chunks + 1) / 2;
  const int64_t ch = 2 * (wi % n_pairs), bkv = wi / n_pairs;
  const bool two = ch + 1 < n_chunks;       // else the second chunk lies past the sequence
  const bool keys_here = two || kq < 2;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t key0 = ch * kKeyChunk;
  const int64_t c = key0 / B;
  int64_t sel_start = 0, sel_cnt = 0;
  if (c < nb) {
    const int64_t sg = bkv * nb + c;
    sel_cnt = counts[sg];
    sel_start = cursor[sg] - sel_cnt;
  }
  const int64_t t_hi = min(n - 1, key0 + KEYS - 1 + W - 1);
  const int64_t win_cnt = (t_hi - key0 + 1) * g;
  const int64_t total = sel_cnt + win_cnt;
  uint32_t mq = 0, md = 0;
  for (int j = 0; j < g; ++j) {
    mq = max(mq, qmax[b * hq + kv * g + j]);
    md = max(md, domax[b * hq + kv * g + j]);
  }
  const int eq = value_exponent(mq), edo = value_exponent(md);
  const float sq = ldexpf(1.f, -eq), sdo = ldexpf(1.f, -edo);

  // Row i of this work item (the block's selected rows, then the window
  // rows), in three steps: pre() loads a selected row's entry; issue() sends
  // the remaining loads and only keeps their values; settle() stores them
  // with the mode (0 = every key counts, 1 = window keys, 2 = none).
  struct Pend {
    int64_t row;   // -1 past the end
    int32_t pos;
    float l, dd;
  };
  // (every lane loads, from row 0 where it has no row: a load under a
  // divergent branch would make the other branch's writes to its registers
  // wait for it)
  auto pre = [&](int64_t i) -> uint32_t {
    return sel_cnt > 0 ? entries[sel_start + min(i, sel_cnt - 1)] : 0u;
  };
  auto issue = [&](int64_t i, uint32_t en) {
    Pend p;
    const bool is_sel = i < sel_cnt;
    const int64_t rho = en >> 5, w = i - sel_cnt;
    const RowTJ q = split_rho(is_sel ? rho : w, g);
    const int64_t pos = is_sel ? q.t : key0 + q.t;
    const int64_t row = (b * hq + kv * g + q.jg) * n + pos;
    p.pos = int32_t(pos);
    p.row = i < total ? row : -1;
    const int64_t sr = i < total ? row : 0;
    p.l = lse[sr];
    p.dd = Drow[sr];
    return p;
  };
  auto settle = [&](int slot, int64_t i, const Pend& p) {
    const int mode = i < sel_cnt ? 0 : (i < total ? int(wmode[i - sel_cnt]) : 2);
    // (the loaded values are stored as they are: arithmetic on them could be
    // moved up to the loads, and its wait with it)
    const int32_t last = int32_t(n - 1);   // keys past the sequence never count
    rrow[slot][tid] = mode == 2 ? -1 : p.row;
    rlo[slot][tid] = mode == 0 ? INT32_MIN : (mode == 1 ? p.pos - W : 0);
    rhi[slot][tid] = mode == 0 ? last : (mode == 1 ? min(p.pos, last) : -1);
    rlse[slot][tid] = p.l;
    rd[slot][tid] = p.dd;
  };
  // Copy a batch's Q and dO rows into a row buffer (its row list is info
  // slot `slot`): copy j fills 1 KB of staged rows, lane l one 16-byte slot.
  // Rows that take no part read row 0; their p and dS are 0.  Every wave
  // issues the same number of copies (the last ones repeat copies of other
  // waves with identical bytes), so waits on later loads can count them.
  constexpr int PER_WAVE = (2 * NCOPY + NW - 1) / NW;
  auto stage_rows = [&](uint8_t* buf, int slot) {
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) {
      int j = wave + NW * u;
      if (j >= 2 * NCOPY) j -= 2 * NCOPY;
      const int s = (j % NCOPY) * 64 + lane;
      const int rr = s / SLOTS, pc = min(s % SLOTS, ROWB / 16 - 1);
      const int64_t row = max(rrow[slot][rr], int64_t(0));
      const bf16_t* src = (j < NCOPY ? Q : dO) + row * D;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(src) + pc * 16,
                                       (__attribute__((address_space(3))) void*)(buf + (j / NCOPY) * TBYTES +
                                                                                 (j % NCOPY) * 1024),
                                       16, 0, 0);
    }
  };

  {
    const uint8_t* ia = img_a + (bkv * n_chunks + ch) * A::CHUNK;
    const uint8_t* ib = img_b + (bkv * n_chunks + ch) * A::CHUNK;
    dma_copy(img, ia, A::KBYTES, tid, kDkvWideThreads);
    dma_copy(img + 2 * A::KBYTES, ib, A::KBYTES, tid, kDkvWideThreads);
    if (two) {
      dma_copy(img + A::KBYTES, ia + A::CHUNK, A::KBYTES, tid, kDkvWideThreads);
      dma_copy(img + 3 * A::KBYTES, ib + A::CHUNK, A::KBYTES, tid, kDkvWideThreads);
    }
  }
  for (int64_t w = tid; w < win_cnt; w += kDkvWideThreads) {
    const int64_t row = (b * hq + kv * g + w % g) * n + key0 + w / g;
    bool sel = false;
    for (int q = 0; q < k; ++q) sel |= idx[row * k + q] == int32_t(c);
    wmode[w] = sel ? 2 : 1;
  }
  __syncthreads();   // window modes
  uint32_t en_next = 0;
  if (tid < ROWS) {
    settle(0, tid, issue(tid, pre(tid)));
    settle(1, ROWS + tid, issue(ROWS + tid, pre(ROWS + tid)));
    en_next = pre(2 * ROWS + tid);
  }
  __syncthreads();   // row lists of batches 0 and 1
  stage_rows(rbuf0, 0);

  floatx16 dk[A::MTD], dv[A::MTD];
#pragma unroll
  for (int i = 0; i < A::MTD; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dk[i][j] = dv[i][j] = 0.f;
  const int32_t mk = int32_t(key0 + 32 * kq + ln);   // this lane's key

  // one batch; CUR = its parity (which row buffer and info slot it uses)
  auto step = [&](auto parity, int64_t i0) {
    constexpr int cur = decltype(parity)::value;
    uint8_t* const rq = cur == 0 ? rbuf0 : rbuf1;
    uint8_t* const rdo = rq + TBYTES;
    __syncthreads();   // this batch's rows have landed; the next batch's row list is in
    // the next batch's rows, into the other buffer (every wave finished with
    // it in the last batch; past the last batch the copy lands where nobody
    // reads), then the row information of the batch after it
    stage_rows(cur == 0 ? rbuf1 : rbuf0, cur ^ 1);
    Pend pend{-1, 0, 0.f, 0.f};
    if (tid < ROWS) {
      pend = issue(i0 + 2 * ROWS + tid, en_next);
      en_next = pre(i0 + 3 * ROWS + tid);
    }

    const int r0 = 32 * rg;
    const bool active = keys_here && i0 + r0 < total;
    floatx16 sacc, pacc;
    if (active) {
      // S = Q K^T and dP = dO V^T for this wave's 32 rows x 32 keys (lanes on keys)
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[j] = pacc[j] = 0.f;
#pragma unroll
      for (int s = 0; s < A::NS; ++s) {
        const Frag kf = *reinterpret_cast<const Frag*>(img + (kq * A::NS + s) * A::FRAG + lane * 8 * ES);
        const Frag vf = *reinterpret_cast<const Frag*>(img + 2 * A::KBYTES + (kq * A::NS + s) * A::FRAG +
                                                       lane * 8 * ES);
        const Frag qa = *reinterpret_cast<const Frag*>(rq + (r0 + ln) * RSTR + (16 * s + 8 * h) * ES);
        const Frag da = *reinterpret_cast<const Frag*>(rdo + (r0 + ln) * RSTR + (16 * s + 8 * h) * ES);
        sacc = mma16(qa, kf, sacc);
        pacc = mma16(da, vf, pacc);
      }
      // element j: row r0 + 8(j/4) + 4h + j%4, key mk.  Everything is read
      // and computed for every element and the mask applied by a select (a
      // conditional exponential becomes a branch per element, each waiting
      // for its own reads)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int rr = r0 + 8 * (j / 4) + 4 * h + j % 4;
        const int32_t lo = rlo[cur][rr], hi = rhi[cur][rr];
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[j], scale2, -rlse[cur][rr] * kLog2e));
        const float p = ((mk > lo) & (mk <= hi)) ? e : 0.f;
        sacc[j] = p;
        pacc[j] = p * (pacc[j] - rd[cur][rr]);
        // four rows' reads in flight at a time: all sixteen at once would
        // not fit in the registers left beside the accumulators
        if (j % 4 == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    // Q^T and dO^T as scaled float16, [column][row] (TRS halves per column),
    // written over the row-major copy once every wave has read it.  Thread
    // unit: rows 2 rp, 2 rp + 1 and columns [8 pc, 8 pc + 8).
    const int rp = 8 * (wave % 4) + lane % 8, pc = lane / 8 + 8 * (wave / 4);
    u32x4 pq[2], pd[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      pq[o] = *reinterpret_cast<const u32x4*>(rq + (2 * rp + o) * RSTR + pc * 16);
      pd[o] = *reinterpret_cast<const u32x4*>(rdo + (2 * rp + o) * RSTR + pc * 16);
    }
    lds_barrier();   // every wave has read the row-major copy
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int sh = 16 * (i % 2);
      const float q0 = __builtin_bit_cast(float, ((pq[0][i / 2] >> sh) & 0xFFFFu) << 16) * sq;
      const float q1 = __builtin_bit_cast(float, ((pq[1][i / 2] >> sh) & 0xFFFFu) << 16) * sq;
      const float d0 = __builtin_bit_cast(float, ((pd[0][i / 2] >> sh) & 0xFFFFu) << 16) * sdo;
      const float d1 = __builtin_bit_cast(float, ((pd[1][i / 2] >> sh) & 0xFFFFu) << 16) * sdo;
      const uint32_t wq = pack_f16x2(q0, q1), wd = pack_f16x2(d0, d1);
      const int at = ((8 * pc + i) * TRS + 2 * rp) * 2;
      *reinterpret_cast<uint32_t*>(rq + at) = wq;
      *reinterpret_cast<uint32_t*>(rdo + at) = wd;
    }
    lds_barrier();   // the transposed copies are complete
    if (active) {
      // dV^T += dO^T P and dK^T += Q^T dS: rows contracted in frag_k order
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        float pv[8], sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 4 * (2 * sp + (e >> 2)) + (e & 3);
          pv[e] = sacc[j];
          sv[e] = pacc[j];
        }
        const f16x8 pf = to_f16x8(pv), sf = to_f16x8(sv);
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt) {
          // rows r0 + frag_k(sp, h, e): 4 consecutive rows, then 4 more 8 rows on
          const int col = 32 * mt + ln;
          const int at = (col * TRS + r0 + 16 * sp + 4 * h) * 2;
          const uint2 q_lo = *reinterpret_cast<const uint2*>(rq + at);
          const uint2 q_hi = *reinterpret_cast<const uint2*>(rq + at + 16);
          const uint2 d_lo = *reinterpret_cast<const uint2*>(rdo + at);
          const uint2 d_hi = *reinterpret_cast<const uint2*>(rdo + at + 16);
          const f16x8 qt = __builtin_bit_cast(f16x8, u32x4{q_lo.x, q_lo.y, q_hi.x, q_hi.y});
          const f16x8 dt = __builtin_bit_cast(f16x8, u32x4{d_lo.x, d_lo.y, d_hi.x, d_hi.y});
          dv[mt] = mma16(dt, pf, dv[mt]);
          dk[mt] = mma16(qt, sf, dk[mt]);
        }
      }
    }
    // batch i0 / ROWS + 2 takes this batch's slot (its waits fall where the
    // next barrier waits for the row copy anyway)
    if (tid < ROWS) settle(cur, i0 + 2 * ROWS + tid, pend);
  };
  for (int64_t i0 = 0; i0 < total; i0 += 2 * ROWS) {
    step(std::integral_constant<int, 0>{}, i0);
    if (i0 + ROWS < total) step(std::integral_constant<int, 1>{}, i0 + ROWS);
  }
  __syncthreads();

  // the two row groups' partial sums, added in LDS in a fixed order (float32,
  // 128 keys x D, over the K/V rows): the result does not depend on scheduling
  float* red = reinterpret_cast<float*>(img);
  for (int pass = 0; pass < 2; ++pass) {
    for (int round = 0; round < 2; ++round) {
      if (rg == round) {
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int col = 32 * mt + 8 * (j / 4) + 4 * h + j % 4;
            float* slot = &red[(32 * kq + ln) * D + col];
            const float v = pass == 0 ? dk[mt][j] : dv[mt][j];
            *slot = round == 0 ? v : *slot + v;
          }
      }
      __syncthreads();
    }
    const float f = pass == 0 ? ldexpf(scale, eq) : ldexpf(1.f, edo);
    float* dst = (pass == 0 ? dK : dV) + (bkv * n + key0) * D;
    for (int w = tid; w < KEYS * D; w += kDkvWideThreads)
      if (key0 + w / D < n) dst[w] = red[w] * f;
    __syncthreads();
  }
}

// --------------------------------------------------------------- dq_window --
// One workgroup (4 waves x 32 rows) per tile of 128 rows (rho = t g + jg) of
// one (sequence, KV head): the window part of dQ over window keys outside the
// row's selected blocks, then the row's dQ partials added.
template <bool F32, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_window_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const typename AT<F32, D>::In* __restrict__ dO,
    const float* __restrict__ lse, const float* __restrict__ Drow, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ pos, const uint8_t* __restrict__ dq_part,
    const float* __restrict__ dq_sc,
    const uint8_t* __restrict__ img_a, const uint8_t* __restrict__ img_b,
    const uint32_t* __restrict__ kmax, int64_t n_chunks, float* __restrict__ dQ, int64_t n, int g,
    int hq, int hkv, int B, int k, int W, float scale2, float scale, int64_t n_tiles) {
  using A = AT<F32, D>;
  using Frag = typename A::Frag;
  constexpr int BUF = A::KBYTES + A::CHUNK;
  // double-buffered chunks only where two workgroups still fit a CU's LDS
  constexpr int NBUF = 2 * BUF <= 64 * 1024 ? 2 : 1;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NBUF * BUF];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int64_t bkv = blockIdx.x / n_tiles, tile = blockIdx.x % n_tiles;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rho0 = tile * kWinTile, rows_total = n * g;
  const int64_t rho = rho0 + 32 * wave + ln;
  const bool valid = rho < rows_total;
  const RowTJ tj = split_rho(valid ? rho : 0, g);
  const int64_t t = tj.t, jg = tj.jg;
  const int64_t row = (b * hq + kv * g + jg) * n + t;
  Frag bq[A::NS], bdo[A::NS];
#pragma unroll
  for (int s = 0; s < A::NS; ++s) {
    bq[s] = load_row_frag<F32, D>(Q + row * D, s, h, valid);
    bdo[s] = load_row_frag<F32, D>(dO + row * D, s, h, valid);
  }
  const float l2 = valid ? lse[row] * kLog2e : 0.f;
  const float dr = valid ? Drow[row] : 0.f;
  const int64_t t_lo = rho0 / g, t_hi = min(n - 1, (rho0 + kWinTile - 1) / g);
  const int64_t ch_lo = max(int64_t(0), t_lo - W + 1) / kKeyChunk, ch_hi = t_hi / kKeyChunk;
  const int64_t wave_t_lo = min(n - 1, (rho0 + 32 * wave) / g);
  const int64_t wave_t_hi = min(n - 1, (rho0 + 32 * wave + 31) / g);
  const bool wave_active = rho0 + 32 * wave < rows_total;
  const uint8_t* srca = img_a + bkv * n_chunks * A::CHUNK;
  const uint8_t* srcb = img_b + bkv * n_chunks * A::CHUNK;
  floatx16 dq[A::MTD];
#pragma unroll
  for (int i = 0; i < A::MTD; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) dq[i][j] = 0.f;

  dma_copy(lds, srca + ch_lo * A::CHUNK, A::KBYTES, tid, 256);
  dma_copy(lds + A::KBYTES, srcb + ch_lo * A::CHUNK, A::CHUNK, tid, 256);
  __syncthreads();
  int32_t excl_blk = -1;   // the block whose selection test excl holds
  bool excl = false;
  for (int64_t ch = ch_lo; ch <= ch_hi; ++ch) {
    const int buf = int((ch - ch_lo) % NBUF);
    uint8_t* L = lds + buf * BUF;
    if (NBUF == 2 && ch + 1 <= ch_hi) {
      uint8_t* Ln = lds + (buf ^ 1) * BUF;
      dma_copy(Ln, srca + (ch + 1) * A::CHUNK, A::KBYTES, tid, 256);
      dma_copy(Ln + A::KBYTES, srcb + (ch + 1) * A::CHUNK, A::CHUNK, tid, 256);
    }
    const int64_t key0 = ch * kKeyChunk;
    if (wave_active && key0 <= wave_t_hi && key0 + kKeyChunk - 1 > wave_t_lo - W) {
      // (the selection test is redone only when a chunk enters another block)
      const int32_t blk = int32_t(key0 / B);
      if (blk != excl_blk) {
        excl = false;
        if (valid)
          for (int i = 0; i < k; ++i) excl |= idx[row * k + i] == blk;
        excl_blk = blk;
      }
      // positions fit in 32 bits; a row that takes no window keys here gets a
      // position no key reaches
      const int32_t tv = valid && !excl ? int32_t(t) : -(1 << 30);
      auto fa = [&](const uint8_t* base, int mt, int s) {
        return *reinterpret_cast<const Frag*>(base + (mt * A::NS + s) * A::FRAG + lane * 8 * A::ES);
      };
      floatx16 sacc[2], pacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[mt][j] = pacc[mt][j] = 0.f;
#pragma unroll
      for (int s = 0; s < A::NS; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          sacc[mt] = mma16(fa(L, mt, s), bq[s], sacc[mt]);
          pacc[mt] = mma16(fa(L + A::KBYTES, mt, s), bdo[s], pacc[mt]);
        }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int32_t kj = int32_t(key0) + 32 * mt + 8 * (j / 4) + 4 * h + j % 4;
          // (computed for every element and selected: a conditional
          // exponential becomes a branch per element)
          const bool on = (kj <= tv) & (kj > tv - W);
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[mt][j], scale2, -l2));
          const float p = on ? e : 0.f;
          sacc[mt][j] = p * (pacc[mt][j] - dr);
          if (j % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bounded register use
        }
      const uint8_t* kt = L + A::KBYTES + A::KBYTES;
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = sacc[sp >> 1][4 * (2 * (sp & 1) + (e >> 2)) + (e & 3)];
        const VF<F32> pf = make_vf<F32>(pv);
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt)
          dq[mt] = mma16(*reinterpret_cast<const typename A::VFrag*>(kt + (mt * 4 + sp) * A::FRAG +
                                                                      lane * 8 * A::ES),
                         pf, dq[mt]);
      }
    }
    __syncthreads();
    if (NBUF == 1 && ch + 1 <= ch_hi) {
      dma_copy(lds, srca + (ch + 1) * A::CHUNK, A::KBYTES, tid, 256);
      dma_copy(lds + A::KBYTES, srcb + (ch + 1) * A::CHUNK, A::CHUNK, tid, 256);
      __syncthreads();
    }
  }
  if (!valid) return;
  const float f = ldexpf(scale, F32 ? 0 : value_exponent(kmax[bkv]));
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j) dq[mt][j] *= f;
  // the row's partials from its selected blocks
  if constexpr (F32) {
    for (int i = 0; i < k; ++i) {
      if (idx[row * k + i] < 0) continue;
      const float* src = reinterpret_cast<const float*>(dq_part) + int64_t(pos[row * k + i]) * D;
#pragma unroll
      for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const floatx4 v = *reinterpret_cast<const floatx4*>(src + 32 * mt + 8 * a + 4 * h);
#pragma unroll
          for (int e = 0; e < 4; ++e) dq[mt][4 * a + e] += v[e];
        }
    }
  } else {
    // float16 partials with their scales; two requested before either is
    // waited for (an absent slot reads partial 0 with weight 0)
    const u16* base = reinterpret_cast<const u16*>(dq_part);
    for (int i0 = 0; i0 < k; i0 += 2) {
      int64_t at[2];
      float w[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = min(i0 + u, k - 1);
        const bool on = i0 + u < k && idx[row * k + i] >= 0;
        at[u] = on ? int64_t(pos[row * k + i]) : 0;
        w[u] = on ? dq_sc[at[u]] : 0.f;
      }
      uint2 v[2][A::MTD][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            v[u][mt][a] = *reinterpret_cast<const uint2*>(base + at[u] * D + 32 * mt + 8 * a + 4 * h);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const uint32_t x[2] = {v[u][mt][a].x, v[u][mt][a].y};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t bits = (e & 1) ? (x[e / 2] >> 16) : (x[e / 2] & 0xFFFFu);
              dq[mt][4 * a + e] = fmaf(static_cast<float>(__builtin_bit_cast(_Float16, u16(bits))), w[u],
                                       dq[mt][4 * a + e]);
            }
          }
    }
  }
  float* out = dQ + row * D;
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a)
      *reinterpret_cast<floatx4*>(out + 32 * mt + 8 * a + 4 * h) =
          floatx4{dq[mt][4 * a], dq[mt][4 * a + 1], dq[mt][4 * a + 2], dq[mt][4 * a + 3]};
}

struct BwdWs {
  DispatchWs disp;
  uint8_t* img_a;
  uint8_t* img_b;
  uint32_t* kmax;
  uint32_t* qmax;
  uint32_t* domax;
  float* Drow;
  uint8_t* dq_part;   // per (row, slot): D float32 (float32 inputs) or D float16 values
  float* dq_sc;       // float16 partials: each one's scale
  int64_t n_chunks;
  size_t bytes;
};

BwdWs bwd_ws_layout(const Shape& s, void* base) {
  BwdWs w{};
  const size_t es = s.in_bf16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const bool use_disp = s.k > 0 && s.nb > 0;
  const DispatchWs dl = use_disp ? dispatch_ws_layout(s, nullptr) : DispatchWs{};
  const size_t o_disp = take(use_disp ? dl.bytes : 0);
  w.n_chunks = (s.n + kKeyChunk - 1) / kKeyChunk;
  const size_t img_bytes = size_t(s.b) * s.hkv * size_t(w.n_chunks) * kKeyChunk * s.d * 2 * es;
  const size_t o_a = take(img_bytes), o_b = take(img_bytes);
  const size_t o_km = take(size_t(s.b) * s.hkv * 4), o_qm = take(size_t(s.b) * s.hq * 4);
  const size_t o_dm = take(size_t(s.b) * s.hq * 4);
  const size_t o_D = take(size_t(s.b) * s.hq * size_t(s.n) * 4);
  const size_t o_part = take(use_disp ? size_t(dl.slots) * s.d * (s.in_bf16 ? 2 : 4) : 0);
  const size_t o_sc = take(use_disp && s.in_bf16 ? size_t(dl.slots) * 4 : 0);
  w.bytes = off;
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    if (use_disp) w.disp = dispatch_ws_layout(s, p + o_disp);
    w.img_a = p + o_a;
    w.img_b = p + o_b;
    w.kmax = reinterpret_cast<uint32_t*>(p + o_km);
    w.qmax = reinterpret_cast<uint32_t*>(p + o_qm);
    w.domax = reinterpret_cast<uint32_t*>(p + o_dm);
    w.Drow = reinterpret_cast<float*>(p + o_D);
    w.dq_part = p + o_part;
    w.dq_sc = reinterpret_cast<float*>(p + o_sc);
  }
  return w;
}

template <bool F32, int D, typename OutT>
hipError_t launch_bwd_t(const Shape& s, const void* Qv, const void* Kv, const void* Vv,
                        const int32_t* idx, const void* Ov, const float* lse, const void* dOv,
                        float* dQ, float* dK, float* dV, void* ws, hipStream_t st) {
  using A = AT<F32, D>;
  using In = typename A::In;
  const In* Q = static_cast<const In*>(Qv);
  const In* K = static_cast<const In*>(Kv);
  const In* V = static_cast<const In*>(Vv);
  const In* dO = static_cast<const In*>(dOv);
  BwdWs w = bwd_ws_layout(s, ws);
  const int64_t n_bkv = int64_t(s.b) * s.hkv, n_bh = int64_t(s.b) * s.hq;
  const int64_t rows = n_bh * s.n;
  const float scale2 = s.scale * kLog2e;
  hipError_t e;
  hipLaunchKernelGGL((bwd_rowdot_kernel<In, OutT>), dim3(unsigned((rows + 3) / 4)), dim3(256), 0, st,
                     dO, static_cast<const OutT*>(Ov), w.Drow, rows, D);
  // float16 scales: largest |K| per KV head, |Q| and |dO| per q-head
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<int32_t*>(w.kmax),
                     n_bkv, 0);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st, reinterpret_cast<int32_t*>(w.qmax),
                     n_bh, 0);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st,
                     reinterpret_cast<int32_t*>(w.domax), n_bh, 0);
  if (!F32) {
    const int64_t per_head = s.n * D;
    const unsigned gx = value_max_groups(per_head);
    hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bkv)), dim3(256), 0, st,
                       reinterpret_cast<const bf16_t*>(Kv), w.kmax, per_head);
    hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bh)), dim3(256), 0, st,
                       reinterpret_cast<const bf16_t*>(Qv), w.qmax, per_head);
    hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bh)), dim3(256), 0, st,
                       reinterpret_cast<const bf16_t*>(dOv), w.domax, per_head);
  }
  // image A = (K rows, V^T; the V part unused), image B = (V rows, K^T scaled)
  hipLaunchKernelGGL((kv_image_kernel<F32, D>), dim3(unsigned(w.n_chunks), unsigned(n_bkv)),
                     dim3(kAttnThreads), 0, st, K, V, w.kmax, w.img_a, s.n, w.n_chunks);
  hipLaunchKernelGGL((kv_image_kernel<F32, D>), dim3(unsigned(w.n_chunks), unsigned(n_bkv)),
                     dim3(kAttnThreads), 0, st, V, K, w.kmax, w.img_b, s.n, w.n_chunks);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool use_disp = s.k > 0 && s.nb > 0;
  if (use_disp) {
    if ((e = launch_dispatch(s, idx, w.disp, st)) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_task_kernel<F32, D>), dim3(unsigned(2 * w.disp.max_tasks)),
                       dim3(kDqThreads), 0, st, Q, dO, lse, w.Drow, w.img_a, w.img_b, w.kmax,
                       w.n_chunks, w.disp.tasks, w.disp.task_count, w.disp.entries, w.dq_part, w.dq_sc, s.n,
                       s.g, s.hq, s.hkv, s.B, s.nb, scale2, s.scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t n_kv_work = n_bkv * w.n_chunks;
  if constexpr (!F32 && D == 128) {
    if (s.B % (2 * kKeyChunk) == 0 &&
        (int64_t(2 * kKeyChunk) + s.W - 1) * s.g <= kDkvWideWinRows) {
      const int64_t n_pair_work = n_bkv * ((w.n_chunks + 1) / 2);
      hipLaunchKernelGGL((bwd_dkv_wide_kernel<D>), dim3(unsigned((n_pair_work + 7) / 8 * 8)),
                         dim3(kDkvWideThreads), 0, st, Q, dO, lse, w.Drow, idx, w.img_a, w.img_b,
                         w.qmax, w.domax, w.n_chunks, use_disp ? w.disp.counts : nullptr,
                         use_disp ? w.disp.cursor : nullptr, use_disp ? w.disp.entries : nullptr,
                         dK, dV, s.n, s.g, s.hq, s.hkv, s.B, use_disp ? s.nb : 0, s.k, s.W, scale2,
                         s.scale, n_pair_work);
    } else {
      hipLaunchKernelGGL((bwd_dkv_kernel<F32, D>), dim3(unsigned((n_kv_work + 7) / 8 * 8)),
                         dim3(kDkvThreads), 0, st, Q, dO, lse, w.Drow, idx, w.img_a, w.img_b,
                         w.qmax, w.domax, w.n_chunks, use_disp ? w.disp.counts : nullptr,
                         use_disp ? w.disp.cursor : nullptr, use_disp ? w.disp.entries : nullptr,
                         dK, dV, s.n, s.g, s.hq, s.hkv, s.B, use_disp ? s.nb : 0, s.k, s.W, scale2,
                         s.scale, n_kv_work);
    }
  } else
  hipLaunchKernelGGL((bwd_dkv_kernel<F32, D>), dim3(unsigned((n_kv_work + 7) / 8 * 8)),
                     dim3(kDkvThreads), 0, st, Q, dO, lse, w.Drow, idx, w.img_a, w.img_b, w.qmax,
                     w.domax, w.n_chunks, use_disp ? w.disp.counts : nullptr,
                     use_disp ? w.disp.cursor : nullptr, use_disp ? w.disp.entries : nullptr, dK,
                     dV, s.n, s.g, s.hq, s.hkv, s.B, use_disp ? s.nb : 0, s.k, s.W, scale2, s.scale,
                     n_kv_work);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n_tiles = (s.n * s.g + kWinTile - 1) / kWinTile;
  hipLaunchKernelGGL((bwd_dq_window_kernel<F32, D>), dim3(unsigned(n_tiles * n_bkv)), dim3(256), 0,
                     st, Q, dO, lse, w.Drow, idx, use_disp ? w.disp.pos : nullptr, w.dq_part, w.dq_sc,
                     w.img_a, w.img_b, w.kmax, w.n_chunks, dQ, s.n, s.g, s.hq, s.hkv, s.B,
                     use_disp ? s.k : 0, s.W, scale2, s.scale, n_tiles);
  return hipGetLastError();
}

template <bool F32, int D>
hipError_t launch_bwd_d(const Shape& s, const void* Q, const void* K, const void* V,
                        const int32_t* idx, const void* O, const float* lse, const void* dO,
                        float* dQ, float* dK, float* dV, void* ws, hipStream_t st) {
  if (s.out_bf16) return launch_bwd_t<F32, D, bf16_t>(s, Q, K, V, idx, O, lse, dO, dQ, dK, dV, ws, st);
  return launch_bwd_t<F32, D, float>(s, Q, K, V, idx, O, lse, dO, dQ, dK, dV, ws, st);
}

}  // namespace

size_t attn_bwd_workspace_bytes(const Shape& s) { return bwd_ws_layout(s, nullptr).bytes; }

hipError_t launch_sparse_attn_bwd(const Shape& s, const void* Q, const void* K, const void* V,
                                  const int32_t* idx, const void* O, const float* lse,
                                  const void* dO, float* dQ, float* dK, float* dV, void* ws,
                                  hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch_bwd_d<false, 64>(s, Q, K, V, idx, O, lse, dO, dQ, dK, dV, ws, st)
                     : launch_bwd_d<false, 128>(s, Q, K, V, idx, O, lse, dO, dQ, dK, dV, ws, st);
  return s.d == 64 ? launch_bwd_d<true, 64>(s, Q, K, V, idx, O, lse, dO, dQ, dK, dV, ws, st)
                   : launch_bwd_d<true, 128>(s, Q, K, V, idx, O, lse, dO, dQ, dK, dV, ws, st);
}

}  // namespace ssa
