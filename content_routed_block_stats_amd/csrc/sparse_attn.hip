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
//     scan that cuts every block's row list into tasks of at most kTaskRows
//     rows, and a scatter into the task-ordered entry list (task j owns
//     entries [j kTaskRows, (j + 1) kTaskRows)) that also records, per
//     (row, slot), where its partial will be;
//  2. block attention -- persistent workgroups keep a block's K and V images
//     resident in LDS across consecutive tasks of that block, gather each
//     task's query rows into MFMA registers, and write one normalised
//     partial per entry (contiguous per task): o_i = softmax-weighted values
//     over the block and lse_i (base 2);
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
#include <mutex>
#include <type_traits>

#include "kv_chunks.hpp"
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kBlockThreads = 512;         // block pass: 8 waves, 32 query rows each
constexpr int kTaskRows = 256;             // rows per block-attention task
constexpr int kResidentBytes = 128 * 1024; // LDS that keeps a block's K/V images resident
constexpr int kRunTasks = 8;               // consecutive tasks a workgroup takes at a time
constexpr int kStageBytes = 4096;          // LDS per wave that lines partials up for storing
constexpr int kWinRows = 128;              // rows per window/merge tile
constexpr int kHistTokens = 2048;          // tokens per dispatch workgroup
constexpr int kScanThreads = 256;           // one workgroup: small, so it finds a CU at once
constexpr int kDispatchThreads = 1024;     // dispatch workgroups: 16 waves each

using f32x2 = float __attribute__((ext_vector_type(2)));

// The partials of a wave's 32 rows (row r: D values, lane half h holds
// columns h D/2 .. in accumulator order, one row after the other in global
// memory).  A lane's registers hold one half row, so storing them directly
// would give each store instruction 64 scattered 16-byte pieces; instead the
// rows pass through kStageBytes of LDS per wave (rounds of kStageBytes / row
// bytes rows, 16-byte chunks XOR-swizzled by row against bank conflicts) and
// leave as fully contiguous 1 KB stores, marked nontemporal: each partial is
// read once, much later, by the merge, and the caches are better kept for the
// query rows and K/V images the pass re-reads.  Lanes read what other lanes of the
// wave wrote, so every round is fenced at wavefront scope on both sides: LDS
// keeps a wave's accesses in order, the fences keep the compiler from reusing
// earlier loads or moving accesses across them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename PartT, int D>
__device__ __forceinline__ void store_partials(uint8_t* stage, PartT* dst, const floatx16 (&o)[D / 32],
                                               float sc, int ln, int h, int lane) {
  constexpr int ROWB = D * int(sizeof(PartT));     // bytes per row
  constexpr int CH = ROWB / 16;                    // 16-byte chunks per row
  constexpr int HALF = CH / 2;                     // chunks per lane half
  constexpr int R = kStageBytes / ROWB;            // rows per round
  // the lane's HALF 16-byte units, converted once (in pairs for float16)
  u32x4 w[HALF];
#pragma unroll
  for (int j = 0; j < HALF; ++j) {
    if constexpr (sizeof(PartT) == 4) {
      const int mt = j / 4, q = j % 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[j][i] = __builtin_bit_cast(uint32_t, o[mt][4 * q + i] * sc);
    } else {
      const int mt = j / 2, q = j % 2;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[j][i] = pack_f16x2(o[mt][8 * q + 2 * i] * sc, o[mt][8 * q + 2 * i + 1] * sc);
    }
  }
#pragma unroll
  for (int rd = 0; rd < 32 / R; ++rd) {
    wave_lds_sync();
    if (ln / R == rd) {
      const int ri = ln % R;
#pragma unroll
      for (int j = 0; j < HALF; ++j) {
        const int c = h * HALF + j;
        *reinterpret_cast<u32x4*>(stage + ri * ROWB + ((c ^ (ri & (CH - 1))) * 16)) = w[j];
      }
    }
    wave_lds_sync();
    uint8_t* out = reinterpret_cast<uint8_t*>(dst) + rd * kStageBytes;
#pragma unroll
    for (int k = 0; k < kStageBytes / 1024; ++k) {
      const int pc = k * 64 + lane, ri = pc / CH, c = pc % CH;
      __builtin_nontemporal_store(
          *reinterpret_cast<const u32x4*>(stage + ri * ROWB + ((c ^ (ri & (CH - 1))) * 16)),
          reinterpret_cast<u32x4*>(out + pc * 16));
    }
  }
}

// o += w * partial (the lane half's values, in the order store_partials writes).
template <typename PartT, int MTD>
__device__ __forceinline__ void accumulate_partial(floatx16 (&o)[MTD], const PartT* src, float w) {
  if constexpr (sizeof(PartT) == 4) {
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 v = reinterpret_cast<const floatx4*>(src)[mt * 4 + q];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[mt][4 * q + i] = fmaf(w, v[i], o[mt][4 * q + i]);
      }
  } else {
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4 v = reinterpret_cast<const u32x4*>(src)[mt * 2 + q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = static_cast<float>(__builtin_bit_cast(_Float16, u16(v[i] & 0xFFFFu)));
          const float b2 = static_cast<float>(__builtin_bit_cast(_Float16, u16(v[i] >> 16)));
          o[mt][8 * q + 2 * i] = fmaf(w, a, o[mt][8 * q + 2 * i]);
          o[mt][8 * q + 2 * i + 1] = fmaf(w, b2, o[mt][8 * q + 2 * i + 1]);
        }
      }
  }
}

// ---------------------------------------------------------------- dispatch --

template <typename PartT, int D>
__global__ void null_partial_kernel(PartT* o_part, float2* lse_part, int64_t slot) {
  for (int i = threadIdx.x; i < D; i += blockDim.x) o_part[slot * D + i] = PartT{};
  if (threadIdx.x == 0) lse_part[slot] = float2{-__builtin_inff(), -__builtin_inff()};
}

// SCATTER = false: add this workgroup's histogram of selected blocks into
// counts.  SCATTER = true: reserve ranges at cursor and write entries
// (row id << 5 | slot) into the per-block lists, and the entry position of
// every selected (row, slot) into pos (same layout as idx).  A workgroup
// covers kHistTokens tokens of one (sequence, KV head) and all its group's
// q-heads.
template <bool SCATTER>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(const int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ counts_or_cursor,
                                                       uint32_t* __restrict__ entries,
                                                       int32_t* __restrict__ pos, int64_t n,
                                                       int g, int hq, int hkv, int k, int64_t nb) {
  extern __shared__ int32_t hist[];
  const int tid = threadIdx.x;
  const int64_t bkv = blockIdx.y, b = bkv / hkv, kv = bkv % hkv;
  const int64_t t0 = int64_t(blockIdx.x) * kHistTokens;
  const int64_t t1 = min(n, t0 + kHistTokens);
  for (int64_t i = tid; i < nb; i += kDispatchThreads) hist[i] = 0;
  __syncthreads();
  // the workgroup's selections of one q-head are one contiguous run of idx
  // (tokens t0..t1, k each): thread tid takes elements tid + i T (T threads),
  // KG at a time, so the loads (and the scatter's pos stores) are coalesced
  // and a group's LDS operations go out together
  constexpr int KG = 8;
  const int run = int((t1 - t0) * k);   // at most kHistTokens x 32
  for (int j = 0; j < g; ++j) {
    const int32_t* src = idx + ((b * hq + kv * g + j) * n + t0) * k;
    for (int w0 = 0; w0 < run; w0 += KG * kDispatchThreads) {
      int32_t c[KG];
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        const int w = w0 + q * kDispatchThreads + tid;
        c[q] = w < run ? src[w] : -1;
      }
#pragma unroll
      for (int q = 0; q < KG; ++q)
        if (c[q] >= 0 && c[q] < nb) atomicAdd(&hist[c[q]], 1);
    }
  }
  __syncthreads();
  int32_t* seg = counts_or_cursor + bkv * nb;
  for (int64_t i = tid; i < nb; i += kDispatchThreads) {
    const int32_t v = hist[i];
    if (v > 0) {
      const int32_t base = atomicAdd(&seg[i], v);
      if (SCATTER) hist[i] = base;
    }
  }
  if (!SCATTER) return;
  __syncthreads();
  for (int j = 0; j < g; ++j) {
    const int64_t base = ((b * hq + kv * g + j) * n + t0) * k;
    for (int w0 = 0; w0 < run; w0 += KG * kDispatchThreads) {
      int32_t c[KG], e[KG];
#pragma unroll
      for (int q = 0; q < KG; ++q) {
        const int w = w0 + q * kDispatchThreads + tid;
        c[q] = w < run ? idx[base + w] : -1;
      }
#pragma unroll
      for (int q = 0; q < KG; ++q) e[q] = (c[q] >= 0 && c[q] < nb) ? atomicAdd(&hist[c[q]], 1) : -1;
#pragma unroll
      for (int q = 0; q < KG; ++q)
        if (e[q] >= 0) {
          const int w = w0 + q * kDispatchThreads + tid;
          const int64_t t = t0 + w / k;
          entries[e[q]] = (uint32_t(t * g + j) << 5) | uint32_t(w % k);
          pos[base + w] = e[q];
        }
    }
  }
}

// Exclusive scan of the per-block task counts: points the scatter cursor of
// every segment at its first task's entries and counts the tasks; the task
// list itself (in block order, task j = (segment, first entry j kTaskRows,
// rows)) is written by emit_tasks_kernel.
__global__ __launch_bounds__(kScanThreads) void scan_tasks_kernel(
    const int32_t* __restrict__ counts, int32_t* __restrict__ cursor,
    int32_t* __restrict__ task_count, int64_t nseg) {
  constexpr int ITEMS = 16;
  __shared__ int32_t st[kScanThreads];
  __shared__ int32_t carry_t;
  const int tid = threadIdx.x;
  if (tid == 0) carry_t = 0;
  __syncthreads();
  for (int64_t base = 0; base < nseg; base += int64_t(kScanThreads) * ITEMS) {
    int32_t c[ITEMS], tk[ITEMS], sum_t = 0;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t s = base + int64_t(tid) * ITEMS + i;
      c[i] = s < nseg ? counts[s] : 0;
      tk[i] = (c[i] + kTaskRows - 1) / kTaskRows;
      sum_t += tk[i];
    }
    st[tid] = sum_t;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
      const int32_t vt = tid >= off ? st[tid - off] : 0;
      __syncthreads();
      st[tid] += vt;
      __syncthreads();
    }
    int32_t ot = carry_t + st[tid] - sum_t;
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
      const int64_t s = base + int64_t(tid) * ITEMS + i;
      if (s < nseg) cursor[s] = ot * kTaskRows;
      ot += tk[i];
    }
    __syncthreads();
    if (tid == kScanThreads - 1) carry_t += st[tid];
    __syncthreads();
  }
  if (tid == 0) task_count[0] = carry_t;
}

// Task j of the list (one thread each, coalesced stores): its segment is the
// last one whose first entry slot is at or below j's (a segment without rows
// starts where the next one does), and its rows are the segment's rows from
// that slot on, at most kTaskRows.  Runs between the scan and the scatter,
// which advances the cursors.
__global__ __launch_bounds__(256) void emit_tasks_kernel(const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ cursor,
                                                         int4* __restrict__ tasks,
                                                         const int32_t* __restrict__ task_count,
                                                         int64_t nseg) {
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j >= int64_t(*task_count)) return;
  const int32_t jr = int32_t(j) * kTaskRows;
  int64_t lo = 0, hi = nseg;   // cursor[lo] <= jr, and every index past hi is above jr
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if (cursor[mid] <= jr) lo = mid; else hi = mid;
  }
  const int32_t q = (jr - cursor[lo]) / kTaskRows;
  tasks[j] = int4{int32_t(lo), jr, min(kTaskRows, counts[lo] - q * kTaskRows), 0};
}

// The scan of the per-segment counts, then the task list.
void launch_scan_tasks(const int32_t* counts, int32_t* cursor, int4* tasks, int32_t* task_count,
                       int64_t nseg, int64_t max_tasks, hipStream_t st) {
  hipLaunchKernelGGL(scan_tasks_kernel, dim3(1), dim3(kScanThreads), 0, st, counts, cursor,
                     task_count, nseg);
  hipLaunchKernelGGL(emit_tasks_kernel, dim3(unsigned((max_tasks + 255) / 256)), dim3(256), 0, st,
                     counts, cursor, tasks, task_count, nseg);
}

// ---------------------------------------------------------- block attention --

// Persistent, one workgroup per CU.  The tasks of one XCD form a contiguous
// range (task order is block order) and each workgroup takes a contiguous
// slice of it, so consecutive tasks of a workgroup mostly share a block.  A
// block's K/V images (up to kResidentBytes, i.e. 256 keys at d = 128 bf16)
// stay resident in LDS and are re-staged only when the block (or, for larger
// blocks, the 256-key segment) changes; within a segment the chunks need no
// barriers.  The next task's row entries are fetched at the start of a task
// and its query rows after the first chunk, so they arrive behind compute.
// SEG > 0 (16-bit inputs): segments of exactly SEG chunks (SEG divides B / 64),
// each run as one unrolled attend_segment; SEG = 0: chunk by chunk.
template <bool F32, int D, typename PartT, int SEG>
__global__ __launch_bounds__(kBlockThreads) void block_attn_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const uint8_t* __restrict__ img,
    int64_t n_chunks, const int4* __restrict__ tasks,
    const int32_t* __restrict__ task_count, const uint32_t* __restrict__ entries,
    const uint32_t* __restrict__ vmax, PartT* __restrict__ o_part, float2* __restrict__ lse_part,
    int64_t n, int g, int hq, int hkv, int B, int64_t nb, float scale2) {
  using A = AT<F32, D>;
  using Frag = typename A::Frag;
  constexpr int SEG_CHUNKS = kResidentBytes / A::CHUNK;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int64_t T = *task_count;
  // this workgroup's p-th task: runs of kRunTasks consecutive tasks, runs
  // dealt round-robin over the workgroups, so that at any moment the whole
  // chip works on a narrow stretch of the task list (one KV head, a few
  // blocks): that head's query rows then stay in the memory-side cache
  // across the k times each of them is gathered
  const int64_t G = gridDim.x;
  auto seq = [&](int64_t p) { return (blockIdx.x + (p / kRunTasks) * G) * kRunTasks + p % kRunTasks; };
  const int64_t tb = seq(0);
  if (tb >= T) return;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  const int r = 32 * wave + ln;             // this lane's row within a task
  const int block_chunks = B / kKeyChunk;
  const int seg_chunks = SEG > 0 ? SEG : min(block_chunks, SEG_CHUNKS);
  const int segs = (block_chunks + seg_chunks - 1) / seg_chunks;

  // (segment ids, (sequence, KV head) pairs and row ids all fit 32 bits:
  // 32-bit divisions are a few instructions, 64-bit ones a long sequence)
  auto image_of = [&](const int4& tk, int seg) {
    const uint32_t bkv = uint32_t(tk.x) / uint32_t(nb), c = uint32_t(tk.x) - bkv * uint32_t(nb);
    return img + (int64_t(bkv) * n_chunks + int64_t(c) * block_chunks + int64_t(seg) * seg_chunks) * A::CHUNK;
  };
  // query row of an entry (row id << 5 | slot) of task tk
  auto row_of = [&](const int4& tk, uint32_t code) {
    const uint32_t bkv = uint32_t(tk.x) / uint32_t(nb);
    const uint32_t b = bkv / uint32_t(hkv), kv = bkv - b * uint32_t(hkv);
    const uint32_t rho = code >> 5, t = rho / uint32_t(g), jg = rho - t * uint32_t(g);
    return (int64_t(b) * hq + int64_t(kv) * g + jg) * n + t;
  };

  // Software pipeline over tasks.  At the top of task i the query rows of
  // task i+1 and the row entries of task i+2 are requested; they arrive
  // while task i computes and are taken (bq, orow_n) only after task i's
  // partials are stored.  Entry and partial slots are padded to kTaskRows per
  // task, so every lane loads and stores unconditionally (lanes past a task's
  // rows read row 0 and write that task's padding): no branch in the loop
  // issues vector memory operations, so the waits at the end of a task count
  // exactly and never wait for the stores just issued (vector loads and
  // stores share one completion counter).
  int4 task = tasks[tb];
  int64_t orow_n;
  Frag bq[1][A::NS];
  {
    const uint32_t code = entries[int64_t(tb) * kTaskRows + r];
    const int64_t orow = row_of(task, r < task.z ? code : 0u);
#pragma unroll
    for (int s = 0; s < A::NS; ++s) bq[0][s] = load_row_frag<F32, D>(Q + orow * D, s, h, true);
  }
  const bool has_1 = seq(1) < T;
  int4 task_n = has_1 ? tasks[seq(1)] : task;
  {
    const uint32_t code = entries[(has_1 ? seq(1) : tb) * kTaskRows + r];
    orow_n = row_of(task_n, has_1 && r < task_n.z ? code : 0u);
  }
  // enter the loop with nothing in flight, as every later iteration does
  __builtin_amdgcn_s_waitcnt(0);
  int64_t resident = -1;                    // segment id held in LDS

  for (int64_t p = 0, ti = tb; ti < T; ti = seq(++p)) {
    // (a) next task's query rows, the entries of the task after it
    Frag bqn[A::NS];
#pragma unroll
    for (int s = 0; s < A::NS; ++s) bqn[s] = load_row_frag<F32, D>(Q + orow_n * D, s, h, true);
    const int64_t t2 = seq(p + 2);
    const bool has_nn = t2 < T;
    const int4 task_nn = has_nn ? tasks[t2] : task;
    const uint32_t code_nn = entries[(has_nn ? t2 : ti) * kTaskRows + r];
    // (b) this task: every chunk of its block against 8 x 32 query rows
    const bool wave_active = 32 * wave < task.z;
    const int ev = F32 ? 0 : value_exponent(vmax[uint32_t(task.x) / uint32_t(nb)]);
    RowState<D> st[1];
    row_state_init(st[0]);
    // a block of several segments is walked in alternating directions by
    // consecutive tasks, so the segment left in LDS by one task is the first
    // the next task of the same block needs
    for (int sg0 = 0; sg0 < segs; ++sg0) {
      const int sg = (p & 1) ? segs - 1 - sg0 : sg0;
      const int64_t sid = int64_t(task.x) * segs + sg;
      const int here = min(seg_chunks, block_chunks - sg * seg_chunks);
      if (sid != resident) {
        __syncthreads();                    // every wave is done with the old segment
        dma_copy(lds, image_of(task, sg), here * A::CHUNK, tid, kBlockThreads);
        __syncthreads();                    // the new segment is in LDS
        resident = sid;
      }
      if (wave_active) {
        if constexpr (SEG > 0 && !F32) {
          attend_segment<D, SEG>(lds, bq[0], scale2, lane, st[0]);
        } else {
          for (int ch = 0; ch < here; ++ch)
            attend_chunk<F32, D, 1>(lds + ch * A::CHUNK, bq, scale2, lane, st,
                                    [](int, int, int, int) { return true; });
        }
      }
    }
    // (c) the partial of every row of the task: the unnormalised sums
    // o = sum_j p_j v_j (values pre-scaled by 2^-ev) times 2^-e, where
    // l = f 2^e with f in [1/2, 1), so |o 2^-e| <= max|v| 2^-ev < 2^15 fits
    // half precision without a per-row maximum; with it go
    // x = m2 + log2 l (the block's log2-sum-exp) and y = m2 + e + ev, and the
    // merge weighs the partial by 2^(x - M) in the denominator and by
    // 2^(y - M) in the numerator
    {
      const float l = st[0].l + wave_shfl_xor(st[0].l, 32);
      int e = 0;
      (void)frexpf(l, &e);
      const int64_t pidx = ti * kTaskRows + r;
      store_partials<PartT, D>(lds + kResidentBytes + wave * kStageBytes,
                               o_part + (pidx - ln) * D, st[0].o, ldexpf(1.f, -e), ln, h, lane);
      __builtin_nontemporal_store(f32x2{st[0].m2 + __log2f(l), st[0].m2 + float(e + ev)},
                                  reinterpret_cast<f32x2*>(lse_part + pidx));
    }
    // (d) rotate the pipeline
    task = task_n;
    task_n = task_nn;
    orow_n = row_of(task_nn, has_nn && r < task_nn.z ? code_nn : 0u);
#pragma unroll
    for (int s = 0; s < A::NS; ++s) bq[0][s] = bqn[s];
  }
}

// ----------------------------------------------------------- window + merge --

// Whether the window/merge pass keeps the partials' positions of its tile in
// its second chunk buffer (free once the window part is done).
__host__ __device__ constexpr bool window_pos_in_chunk(int k, int chunk_bytes) {
  return int64_t(k) * kWinRows * 4 <= chunk_bytes;
}

template <bool F32, int D, typename PartT, typename OutT>
__global__ __launch_bounds__(kAttnThreads) __attribute__((amdgpu_waves_per_eu(2))) void window_merge_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const uint8_t* __restrict__ img,
    int64_t n_chunks, const int32_t* __restrict__ idx, const int32_t* __restrict__ pos,
    const uint32_t* __restrict__ vmax, const PartT* __restrict__ o_part,
    const float2* __restrict__ lse_part, int64_t null_slot, OutT* __restrict__ O,
    float* __restrict__ lse, int64_t n, int g, int hq, int hkv, int B, int k, int W,
    float scale2, int64_t n_tiles, int64_t n_work) {
  using A = AT<F32, D>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  int32_t* sidx = reinterpret_cast<int32_t*>(lds + 2 * A::CHUNK);   // [k][kWinRows]
  float2* wml = reinterpret_cast<float2*>(sidx + kWinRows * k);       // window (m2, l) per row
  // the partials' positions, [k][kWinRows]: loaded once the window part is
  // done, into the second chunk buffer when they fit there (keeping the LDS
  // of a workgroup within half a CU's), else after wml
  int32_t* spos = window_pos_in_chunk(k, A::CHUNK) ? reinterpret_cast<int32_t*>(lds + A::CHUNK)
                                                   : reinterpret_cast<int32_t*>(wml + kWinRows);
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  // workgroups are dealt round-robin over the 8 XCDs; give each XCD a
  // contiguous run of tiles so that neighbouring tiles, whose windows share
  // key chunks, meet in the same L2
  // (the grid is n_work rounded up to a multiple of 8; the extra ones exit)
  const int64_t per_xcd = int64_t(gridDim.x) / 8;
  const int64_t lin = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (lin >= n_work) return;
  const int64_t bkv = lin / n_tiles;
  const int64_t tile = lin % n_tiles;
  const int64_t b = bkv / hkv, kv = bkv % hkv;
  const int64_t rho0 = tile * kWinRows, rows_total = n * g;

  const int r = 32 * wave + ln;
  const int64_t rho = rho0 + r;
  const bool valid = rho < rows_total;
  const RowTJ tj = split_rho(valid ? rho : 0, g);
  const int64_t t = tj.t, jg = tj.jg;
  const int64_t orow = (b * hq + kv * g + jg) * n + t;

  const int64_t t_lo = rho0 / g, t_hi = min(n - 1, (rho0 + kWinRows - 1) / g);
  const int64_t key_lo = max(int64_t(0), t_lo - W + 1);
  const int64_t ch0 = key_lo / kKeyChunk, ch1 = t_hi / kKeyChunk;
  const uint8_t* src = img + bkv * n_chunks * A::CHUNK;
  const int ev = F32 ? 0 : value_exponent(vmax[bkv]);
  dma_copy_async(lds, src + ch0 * A::CHUNK, A::CHUNK, tid, kAttnThreads);

  for (int w = tid; w < kWinRows * k; w += kAttnThreads) {
    const int rr = w / k, i = w % k;   // coalesced idx reads, transposed LDS writes
    const int64_t rh = rho0 + rr;
    int32_t v = -1;
    if (rh < rows_total) {
      const RowTJ q = split_rho(rh, g);
      v = idx[((b * hq + kv * g + q.jg) * n + q.t) * k + i];
    }
    sidx[i * kWinRows + rr] = v;
  }
  typename A::Frag bq[1][A::NS];
  {
    const auto* qrow = Q + orow * D;
#pragma unroll
    for (int s = 0; s < A::NS; ++s) bq[0][s] = load_row_frag<F32, D>(qrow, s, h, valid);
  }
  const int64_t wave_t_lo = min(n - 1, (rho0 + 32 * wave) / g);
  const int64_t wave_t_hi = min(n - 1, (rho0 + 32 * wave + 31) / g);
  const bool wave_active = rho0 + 32 * wave < rows_total;

  RowState<D> st[1];
  row_state_init(st[0]);
  int32_t excl_blk = -1;   // the block whose selection test excl holds
  bool excl = false;
  // the query fragments and index rows are in before the loop, so the
  // compiler's own waits inside it (it cannot see the chunk copies) have
  // nothing left to wait for
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int64_t ch = ch0; ch <= ch1; ++ch) {
    const int buf = int((ch - ch0) & 1);
    const bool more = ch + 1 <= ch1;
    // chunk ch has landed (this wave's copies, then everyone's), and every
    // wave is done with chunk ch-1, whose buffer the next copy refills while
    // chunk ch is computed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (more)
      dma_copy_async(lds + (buf ^ 1) * A::CHUNK, src + (ch + 1) * A::CHUNK, A::CHUNK, tid,
                     kAttnThreads);
    const int64_t key0 = ch * kKeyChunk;
    // does this wave's token range touch the chunk at all?
    const bool touch = wave_active && key0 <= wave_t_hi && key0 + kKeyChunk - 1 > wave_t_lo - W;
    if (touch) {
      // keys of a selected block already count in that block's partial (the
      // test is redone only when the chunk enters another block)
      const int32_t blk = int32_t(key0 / B);
      if (blk != excl_blk) {
        excl = false;
        for (int i = 0; i < k; ++i) excl |= sidx[i * kWinRows + r] == blk;
        excl_blk = blk;
      }
      const bool rowok = valid && !excl;
      // a chunk inside the window of every token of the wave needs no
      // per-key test: the row's own test decides (a lane holds one row's
      // scores, so the test is one per lane)
      const bool inner = key0 + kKeyChunk - 1 <= wave_t_lo && key0 > wave_t_hi - W;
      if (inner) {
        attend_chunk<F32, D, 1>(lds + buf * A::CHUNK, bq, scale2, lane, st,
                                [&](int, int, int, int) { return rowok; });
      } else {
        // 32-bit positions and bitwise tests: no exec-mask blocks per element
        const int32_t tv = rowok ? int32_t(t) : -(1 << 30);
        const int32_t kb = int32_t(key0) + 4 * h;
        attend_chunk<F32, D, 1>(lds + buf * A::CHUNK, bq, scale2, lane, st,
                                [&](int, int mt, int a, int bb) {
                                  const int32_t j = kb + 32 * mt + 8 * a + bb;
                                  return (j <= tv) & (j > tv - W);
                                });
      }
    }
  }
  __syncthreads();   // every wave is done with the chunk buffers
  // ---- hand the window part over to the merge layout (LDS, reusing the
  // first chunk buffer), normalised by its
  // sum and in the partials' precision.  Element e of a row is column
  // pi(e) = 32mt + 8a + 4h + b for e = h D/2 + 16mt + 4a + b -- the order
  // partials are stored in -- so a lane half's values are one contiguous
  // run; 16-byte units are XOR-swizzled by row.
  {
    const RowState<D>& ws = st[0];
    const float lw = ws.l + wave_shfl_xor(ws.l, 32);
    const float inv = lw > 0.f ? 1.f / lw : 0.f;
    if constexpr (sizeof(PartT) == 4) {
      constexpr int U = D / 4;                      // 16-byte units per float32 row
      float* wo = reinterpret_cast<float*>(lds);
#pragma unroll
      for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = (h * (D / 2) + 16 * mt + 4 * q) / 4;
          *reinterpret_cast<floatx4*>(wo + r * D + 4 * (u ^ (r % U))) =
              floatx4{ws.o[mt][4 * q] * inv, ws.o[mt][4 * q + 1] * inv, ws.o[mt][4 * q + 2] * inv,
                      ws.o[mt][4 * q + 3] * inv};
        }
    } else {
      constexpr int U = D / 8;                      // 16-byte units per float16 row
#pragma unroll
      for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int el = h * (D / 2) + 16 * mt + 4 * q, u = el / 8;
          *reinterpret_cast<uint2*>(lds + r * D * 2 + (u ^ (r % U)) * 16 + (el % 8) * 2) =
              uint2{pack_f16x2(ws.o[mt][4 * q] * inv, ws.o[mt][4 * q + 1] * inv),
                    pack_f16x2(ws.o[mt][4 * q + 2] * inv, ws.o[mt][4 * q + 3] * inv)};
        }
    }
    if (h == 0) wml[r] = float2{ws.m2, lw};
  }
  // this wave's rows' partial positions (only the wave's own rows are merged
  // by it, so a wavefront-scope fence suffices)
  for (int w = lane; w < 32 * k; w += 64) {
    const int rr = 32 * wave + w / k, i = w % k;
    const int64_t rh = rho0 + rr;
    int32_t e = 0;
    if (rh < rows_total && sidx[i * kWinRows + rr] >= 0) {
      const RowTJ q = split_rho(rh, g);
      e = pos[((b * hq + kv * g + q.jg) * n + q.t) * k + i];
    }
    spos[i * kWinRows + rr] = e;
  }
  wave_lds_sync();

  // ---- merge, in the partials' own layout: CH lanes per row, each owning
  // one 16-byte unit of every partial (coalesced reads), RPR rows per pass.
  constexpr int CH = D * int(sizeof(PartT)) / 16;   // 16-byte units per partial row
  constexpr int EPU = 16 / int(sizeof(PartT));      // elements per unit
  constexpr int RPR = 64 / CH;
  constexpr int GRP = 16;                           // partials requested at once
  for (int rd = 0; rd < 32 / RPR; ++rd) {
    const int rr = 32 * wave + rd * RPR + lane / CH, sub = lane % CH;
    const int64_t rh = rho0 + rr;
    if (rh >= rows_total) continue;
    const RowTJ q = split_rho(rh, g);
    const int64_t row = (b * hq + kv * g + q.jg) * n + q.t;
    const float2 wl = wml[rr];
    // running (max, sum, weighted values) over the window part and then the
    // partials in groups of GRP; every load is unconditional -- absent slots
    // read the null partial (zeros, lse = -inf) -- so a group's loads all
    // go out before any of them is waited for
    // an empty window part (every window key inside a selected block) has
    // l = 0; a NaN sum (non-finite inputs) is kept, so NaN reaches O and LSE
    const bool wempty = wl.y == 0.f;
    float M = wempty ? -__builtin_inff() : wl.x + __log2f(wl.y);
    float den = wempty ? 0.f : wl.y * __builtin_amdgcn_exp2f(wl.x - M);   // = 1 or 0
    float acc[EPU];
    {
      // the stored window part is normalised: its weight is den itself
      const float wws = ldexpf(den, ev);
      if constexpr (sizeof(PartT) == 4) {
        constexpr int U = D / 4;
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          const int el = sub * EPU + e, u = el / 4;
          acc[e] = reinterpret_cast<const float*>(lds)[rr * D + 4 * (u ^ (rr % U)) + el % 4] * wws;
        }
      } else {
        // a lane's unit of the partial row is unit sub of the stored row
        constexpr int U = D / 8;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + rr * D * 2 + (sub ^ (rr % U)) * 16);
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          const uint32_t w2 = v[e / 2];
          acc[e] = static_cast<float>(__builtin_bit_cast(_Float16, u16((e & 1) ? (w2 >> 16) : (w2 & 0xFFFFu)))) * wws;
        }
      }
    }
    for (int i0 = 0; i0 < k; i0 += GRP) {
      int64_t pidx[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const int i = min(i0 + j, k - 1);
        const int32_t sel = sidx[i * kWinRows + rr], at = spos[i * kWinRows + rr];
        pidx[j] = (i0 + j < k && sel >= 0) ? int64_t(at) : null_slot;
      }
      u32x4 pv[GRP];
      float2 le[GRP];
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        le[j] = lse_part[pidx[j]];
        pv[j] = reinterpret_cast<const u32x4*>(o_part + pidx[j] * D)[sub];
      }
      float Mg = M;
#pragma unroll
      for (int j = 0; j < GRP; ++j) Mg = fmaxf(Mg, le[j].x);
      const float resc = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mg);
      M = Mg;
      den *= resc;
#pragma unroll
      for (int e = 0; e < EPU; ++e) acc[e] *= resc;
#pragma unroll
      for (int j = 0; j < GRP; ++j) {
        const float wi = le[j].x == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(le[j].x - M);
        den += wi;
        const float ws2 = le[j].y == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(le[j].y - M);
#pragma unroll
        for (int e = 0; e < EPU; ++e) {
          float v;
          if constexpr (sizeof(PartT) == 4) {
            // (copy the element out first: bit-casting a vector element
            // lvalue directly reads element 0 with this compiler)
            const uint32_t bits = pv[j][e];
            v = __builtin_bit_cast(float, bits);
          } else {
            const uint32_t w2 = pv[j][e / 2];
            v = static_cast<float>(__builtin_bit_cast(_Float16, u16((e & 1) ? (w2 >> 16) : (w2 & 0xFFFFu))));
          }
          acc[e] = fmaf(ws2, v, acc[e]);
        }
      }
    }
    const float inv = 1.f / den;
    OutT* out = O + row * D;
#pragma unroll
    for (int e = 0; e < EPU; ++e) {
      const int el = sub * EPU + e;                 // element -> column
      const int hh = el / (D / 2), rem = el % (D / 2), mt = rem / 16, j = rem % 16;
      store_from_f32(out, 32 * mt + 8 * (j / 4) + 4 * hh + (j % 4), acc[e] * inv);
    }
    if (sub == 0) lse[row] = (M + __log2f(den)) * kLn2;
  }
}

// ------------------------------------------------------------------ launch --

// Compute units of the current device (queried once; a launch-shape hint only).
int num_cus() {
  static const int cus = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      return v;
    return 256;
  }();
  return cus;
}

// The K/V chunk images do not depend on the selection and the dispatch does
// not depend on the images: the images are built on the device's second
// stream (SideLease) while the caller's stream runs the dispatch, and the
// caller's stream waits for them before the block pass.

struct AttnWs {
  uint32_t* vmax;
  uint8_t* img;
  int64_t n_chunks;
  int32_t* counts;
  int32_t* cursor;
  int32_t* task_count;
  int4* tasks;
  uint32_t* entries;
  int32_t* pos;
  float2* lse_part;
  void* o_part;
  size_t bytes;
  int64_t max_tasks;
  int64_t null_slot;
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
  const size_t o_vmax = take(size_t(s.b) * s.hkv * 4);
  w.n_chunks = (s.n + kKeyChunk - 1) / kKeyChunk;
  const size_t chunk_bytes = size_t(kKeyChunk) * s.d * 2 * es;
  const size_t o_img = take(size_t(s.b) * s.hkv * size_t(w.n_chunks) * chunk_bytes);
  const size_t o_counts = take(size_t(nseg) * 4), o_cursor = take(size_t(nseg) * 4);
  const size_t o_tc = take(4), o_tasks = take(size_t(w.max_tasks) * 16);
  // entries and partials in task order, kTaskRows slots per task
  // one more partial slot past the tasks': the null partial (zeros, lse -inf)
  // that the merge reads for absent selections
  const size_t slots = size_t(w.max_tasks) * kTaskRows;
  w.null_slot = int64_t(slots);
  const size_t o_entries = take(slots * 4), o_pos = take(size_t(pairs) * 4);
  const size_t o_lse = take((slots + 1) * 8), o_part = take((slots + 1) * s.d * es);
  w.bytes = off;
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.vmax = reinterpret_cast<uint32_t*>(p + o_vmax);
    w.img = p + o_img;
    w.counts = reinterpret_cast<int32_t*>(p + o_counts);
    w.cursor = reinterpret_cast<int32_t*>(p + o_cursor);
    w.task_count = reinterpret_cast<int32_t*>(p + o_tc);
    w.tasks = reinterpret_cast<int4*>(p + o_tasks);
    w.entries = reinterpret_cast<uint32_t*>(p + o_entries);
    w.pos = reinterpret_cast<int32_t*>(p + o_pos);
    w.lse_part = reinterpret_cast<float2*>(p + o_lse);
    w.o_part = p + o_part;
  }
  return w;
}

// The block pass for blocks of bc chunks: for 16-bit inputs the instance
// whose segment length is the largest divisor of bc that fits the resident
// LDS; for float32 inputs the chunk-by-chunk one.
template <bool F32, int D, typename PartT, int SEG = kResidentBytes / AT<F32, D>::CHUNK>
auto block_kernel_for(int bc) -> decltype(&block_attn_kernel<F32, D, PartT, 0>) {
  if constexpr (F32) {
    return &block_attn_kernel<F32, D, PartT, 0>;
  } else {
    if constexpr (SEG > 1)
      if (bc % SEG != 0) return block_kernel_for<F32, D, PartT, SEG - 1>(bc);
    return &block_attn_kernel<F32, D, PartT, SEG>;
  }
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
  // the V scale and the chunk images, beside the dispatch below
  SideLease side(st);
  {
    hipStream_t ss = side.stream();
    if (!F32) {
      hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, ss,
                         reinterpret_cast<int32_t*>(w.vmax), n_bkv, 0);
      const int64_t per_head = s.n * D;
      const unsigned gx = value_max_groups(per_head);
      hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bkv)), dim3(256), 0, ss,
                         reinterpret_cast<const bf16_t*>(Vv), w.vmax, per_head);
    }
    hipLaunchKernelGGL((kv_image_kernel<F32, D>), dim3(unsigned(w.n_chunks), unsigned(n_bkv)),
                       dim3(kAttnThreads), 0, ss, K, V, w.vmax, w.img, s.n, w.n_chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (s.k > 0)
    hipLaunchKernelGGL((null_partial_kernel<PartT, D>), dim3(1), dim3(64), 0, st,
                       static_cast<PartT*>(w.o_part), w.lse_part, w.null_slot);
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
    hipLaunchKernelGGL(dispatch_kernel<false>, hgrid, dim3(kDispatchThreads), hshm, st, idx,
                       w.counts, (uint32_t*)nullptr, (int32_t*)nullptr, s.n, s.g, s.hq, s.hkv, s.k, s.nb);
    launch_scan_tasks(w.counts, w.cursor, w.tasks, w.task_count, nseg, w.max_tasks, st);
    hipLaunchKernelGGL(dispatch_kernel<true>, hgrid, dim3(kDispatchThreads), hshm, st, idx,
                       w.cursor, w.entries, w.pos, s.n, s.g, s.hq, s.hkv, s.k, s.nb);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = side.join()) != hipSuccess) return e;
    auto bk = block_kernel_for<F32, D, PartT>(s.B / kKeyChunk);
    const size_t bshm = size_t(kResidentBytes) + (kBlockThreads / 64) * size_t(kStageBytes);
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(bk),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(bshm))) != hipSuccess)
      return e;
    // persistent: one workgroup per CU, a multiple of the 8 XCDs
    const int64_t grid = std::max<int64_t>(8, int64_t(num_cus()) / 8 * 8);
    hipLaunchKernelGGL(bk, dim3(unsigned(grid)), dim3(kBlockThreads), bshm, st, Q, w.img, w.n_chunks,
                       w.tasks, w.task_count, w.entries, w.vmax, static_cast<PartT*>(w.o_part),
                       w.lse_part, s.n, s.g, s.hq, s.hkv, s.B, s.nb, scale2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = side.join()) != hipSuccess) return e;   // (k = 0: the images are still needed)
  auto wk = window_merge_kernel<F32, D, PartT, OutT>;
  const size_t wshm = 2 * size_t(A::CHUNK) + size_t(kWinRows) * std::max(s.k, 1) * 4 +
                      size_t(kWinRows) * 8 +
                      (window_pos_in_chunk(s.k, A::CHUNK) ? 0 : size_t(kWinRows) * s.k * 4);
  if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(wk),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(wshm))) != hipSuccess)
    return e;
  const int64_t n_tiles = (s.n * s.g + kWinRows - 1) / kWinRows;
  // a multiple of 8 workgroups, so that the XCD remapping is a bijection
  hipLaunchKernelGGL(wk, dim3(unsigned((n_tiles * n_bkv + 7) / 8 * 8)), dim3(kAttnThreads), wshm, st, Q, w.img,
                     w.n_chunks, idx, w.pos, w.vmax, static_cast<const PartT*>(w.o_part), w.lse_part,
                     w.null_slot, static_cast<OutT*>(Ov), lse, s.n, s.g, s.hq, s.hkv, s.B, s.k, s.W, scale2, n_tiles,
                     n_tiles * n_bkv);
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

DispatchWs dispatch_ws_layout(const Shape& s, void* base) {
  DispatchWs w{};
  const int64_t nseg = int64_t(s.b) * s.hkv * s.nb;
  const int64_t pairs = int64_t(s.b) * s.hq * s.n * s.k;
  w.max_tasks = (pairs + kTaskRows - 1) / kTaskRows + nseg;
  w.slots = w.max_tasks * kTaskRows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t o_counts = take(size_t(nseg) * 4), o_cursor = take(size_t(nseg) * 4);
  const size_t o_tc = take(4), o_tasks = take(size_t(w.max_tasks) * 16);
  const size_t o_entries = take(size_t(w.slots) * 4), o_pos = take(size_t(pairs) * 4);
  w.bytes = off;
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.counts = reinterpret_cast<int32_t*>(p + o_counts);
    w.cursor = reinterpret_cast<int32_t*>(p + o_cursor);
    w.task_count = reinterpret_cast<int32_t*>(p + o_tc);
    w.tasks = reinterpret_cast<int4*>(p + o_tasks);
    w.entries = reinterpret_cast<uint32_t*>(p + o_entries);
    w.pos = reinterpret_cast<int32_t*>(p + o_pos);
  }
  return w;
}

hipError_t launch_dispatch(const Shape& s, const int32_t* idx, const DispatchWs& w, hipStream_t st) {
  const int64_t n_bkv = int64_t(s.b) * s.hkv;
  const int64_t nseg = n_bkv * s.nb;
  hipError_t e;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned(std::min<int64_t>((nseg + 255) / 256, 4096))),
                     dim3(256), 0, st, w.counts, nseg, 0);
  const dim3 hgrid(unsigned((s.n + kHistTokens - 1) / kHistTokens), unsigned(n_bkv));
  const size_t hshm = size_t(s.nb) * 4;
  for (const void* f : {reinterpret_cast<const void*>(dispatch_kernel<false>),
                        reinterpret_cast<const void*>(dispatch_kernel<true>)})
    if ((e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(hshm))) !=
        hipSuccess)
      return e;
  hipLaunchKernelGGL(dispatch_kernel<false>, hgrid, dim3(kDispatchThreads), hshm, st, idx, w.counts,
                     (uint32_t*)nullptr, (int32_t*)nullptr, s.n, s.g, s.hq, s.hkv, s.k, s.nb);
  launch_scan_tasks(w.counts, w.cursor, w.tasks, w.task_count, nseg, w.max_tasks, st);
  hipLaunchKernelGGL(dispatch_kernel<true>, hgrid, dim3(kDispatchThreads), hshm, st, idx, w.cursor,
                     w.entries, w.pos, s.n, s.g, s.hq, s.hkv, s.k, s.nb);
  return hipGetLastError();
}

int64_t attn_entry_slots(const Shape& s) {
  return attn_ws_layout(s, nullptr).max_tasks * kTaskRows;
}

hipError_t launch_sparse_attn(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* idx, void* O, float* lse, void* ws, hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch_attn_d<false, 64>(s, Q, K, V, idx, O, lse, ws, st)
                     : launch_attn_d<false, 128>(s, Q, K, V, idx, O, lse, ws, st);
  return s.d == 64 ? launch_attn_d<true, 64>(s, Q, K, V, idx, O, lse, ws, st)
                   : launch_attn_d<true, 128>(s, Q, K, V, idx, O, lse, ws, st);
}

}  // namespace ssa
