// One decode step: append, block statistics on completion, routing, top-k,
// attention over the selected blocks and the window, merge.
//
// Write-up "Subquadratic Sparse Attention (SSA)", module table (the decode
// path routes and attends one new query per step) and the mechanism of the
// introduction (steps i-iii) at query position t = L.  With one query per
// (sequence, q-head) there is no query tile to share a Sigma_c with, so the
// router is an HBM stream over the statistics: each workgroup reads the
// upper-triangular 32x32 tiles of Sigma_c (10 of 16 at d = 128) once and
// scores all q-heads of the KV head's group against them in float32 on the
// vector ALUs.  Attention is split by (row, selected block) plus one window
// item per row, each an online-softmax partial read straight from the
// caches, merged per row at the end.  cache_len lives on the device, so steps
// chain on a stream without a host round trip.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecBlocksPerWg = 8;
constexpr int kDecKeyChunk = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename TIn>
__global__ void append_kernel(const TIn* __restrict__ k_new, const TIn* __restrict__ v_new,
                              TIn* __restrict__ Kc, TIn* __restrict__ Vc,
                              const int32_t* __restrict__ cache_len, int hkv, int d, int64_t cap) {
  const int64_t bkv = blockIdx.x, b = bkv / hkv;
  const int64_t L = cache_len[b];
  if (L < 0 || L >= cap) return;   // caller contract violated: write nothing
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    Kc[(bkv * cap + L) * d + i] = k_new[bkv * d + i];
    Vc[(bkv * cap + L) * d + i] = v_new[bkv * d + i];
  }
}

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += wave_shfl_xor(v, o);
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < int(blockDim.x / 64); ++i) s += red[i];
  return s;
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, wave_shfl_xor(v, o));
  const int w = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = -__builtin_inff();
  for (int i = 0; i < int(blockDim.x / 64); ++i) s = fmaxf(s, red[i]);
  return s;
}

// Scores of up to 4 q-heads (one pass) against kDecBlocksPerWg blocks.
// Thread (row i = tid/8 of a 32x32 tile, column quad tid%8) reads 4 floats of
// each upper tile; off-diagonal tiles count twice, as Sigma is symmetric.
template <typename TIn, int D>
__global__ __launch_bounds__(kDecThreads) void decode_route_kernel(
    const TIn* __restrict__ q, const float* __restrict__ mu, const float* __restrict__ sigma,
    const int32_t* __restrict__ cache_len, float* __restrict__ scores, int g, int hq, int hkv,
    int B, int64_t n_slots, float beta) {
  constexpr int MT = D / 32;
  extern __shared__ float qs[];   // [g][D]
  __shared__ float red[kDecThreads / 64];
  const int tid = threadIdx.x;
  const int64_t bkv = blockIdx.y, b = bkv / hkv, kv = bkv % hkv;
  const int64_t L = cache_len[b];
  const int64_t C = L < 0 ? 0 : min(n_slots, (L + 1) / B);
  const int64_t c0 = int64_t(blockIdx.x) * kDecBlocksPerWg;
  if (c0 >= C) return;
  for (int i = tid; i < g * D; i += kDecThreads)
    qs[i] = load_f32(q, (b * hq + kv * g) * D + i);
  __syncthreads();
  const int ri = tid / 8, cq = tid % 8;
  for (int64_t c = c0; c < min(C, c0 + kDecBlocksPerWg); ++c) {
    const float* S = sigma + ((bkv * n_slots) + c) * D * D;
    const float* M = mu + ((bkv * n_slots) + c) * D;
    for (int r0 = 0; r0 < g; r0 += 4) {
      float quad[4] = {0.f, 0.f, 0.f, 0.f}, mean[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ti = 0; ti < MT; ++ti) {
#pragma unroll
        for (int tj = ti; tj < MT; ++tj) {
          const int i = 32 * ti + ri, j = 32 * tj + 4 * cq;
          const floatx4 sv = *reinterpret_cast<const floatx4*>(S + i * D + j);
          const float w = ti == tj ? 1.f : 2.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (r0 + r < g) {
              const float* qr = qs + (r0 + r) * D;
              const float inner = sv[0] * qr[j] + sv[1] * qr[j + 1] + sv[2] * qr[j + 2] + sv[3] * qr[j + 3];
              quad[r] = fmaf(w * qr[i], inner, quad[r]);
            }
          }
        }
      }
      if (tid < D) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r0 + r < g) mean[r] = M[tid] * qs[(r0 + r) * D + tid];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (r0 + r >= g) break;
        const float tot = block_sum(mean[r] + 0.5f * beta * quad[r], red);
        if (tid == 0) scores[(b * hq + kv * g + r0 + r) * n_slots + c] = tot;
      }
    }
  }
}

// Top-k of one row per wave: a per-lane sorted list over c = lane, lane+64, ...
// then k rounds of a wave arg-max (ties to the lower block).
template <int KMAX>
__global__ __launch_bounds__(256) void decode_topk_kernel(const float* __restrict__ scores,
                                                           const int32_t* __restrict__ cache_len,
                                                           int32_t* __restrict__ idx_out, int k,
                                                           int64_t n_slots, int hq, int B,
                                                           int64_t rows) {
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;
  if (row >= rows) return;
  const int64_t b = row / hq;
  const int64_t C = cache_len[b] < 0 ? 0 : min(n_slots, (int64_t(cache_len[b]) + 1) / B);
  float ls[KMAX];
  int li[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    ls[i] = -__builtin_inff();
    li[i] = 0x7FFFFFFF;
  }
  for (int64_t c = lane; c < C; c += 64) {
    const float sn = scores[row * n_slots + c];
    float sc = sn;
    int ci = int(c);
    if (!(sn > ls[KMAX - 1])) continue;
    // sorted insert (score descending, block ascending; blocks arrive in
    // ascending order): the new score against each slot, so entries it
    // displaces move down one and never slip past an equal later entry
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const bool gt = sn > ls[i];
      const float ts = ls[i];
      const int tix = li[i];
      ls[i] = gt ? sc : ts;
      li[i] = gt ? ci : tix;
      sc = gt ? ts : sc;
      ci = gt ? tix : ci;
    }
  }
  // k rounds: the best head among the lanes wins and pops.  A score that is
  // never inserted (NaN, or -inf) leaves the lists holding the sentinel
  // 0x7FFFFFFF; a round that can only find the sentinel ends the selection,
  // so every pick kept is a distinct routable block.
  int sel_mine[KMAX];
  int n_sel = 0;
  const int take = int(min<int64_t>(k, C));
  for (int rnd = 0; rnd < take; ++rnd) {
    float bs = ls[0];
    int bi = li[0];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float os = wave_shfl_xor(bs, o);
      const int oi = __shfl_xor(bi, o, 64);
      if (os > bs || (os == bs && oi < bi)) {
        bs = os;
        bi = oi;
      }
    }
    if (bi == 0x7FFFFFFF) break;   // wave-uniform: every lane saw the same winner
    if (li[0] == bi) {
#pragma unroll
      for (int i = 0; i < KMAX - 1; ++i) {
        ls[i] = ls[i + 1];
        li[i] = li[i + 1];
      }
      ls[KMAX - 1] = -__builtin_inff();
      li[KMAX - 1] = 0x7FFFFFFF;
    }
    if (lane == 0) sel_mine[n_sel] = bi;
    ++n_sel;
  }
  if (lane != 0) return;
  // ascending output (the picks are distinct), -1 padded
  int32_t* out = idx_out + row * k;
  for (int i = n_sel; i < k; ++i) out[i] = -1;
  for (int i = 0; i < n_sel; ++i) {
    int rank = 0;
    for (int j = 0; j < n_sel; ++j) rank += sel_mine[j] < sel_mine[i] ? 1 : 0;
    out[rank] = sel_mine[i];
  }
}

// One (row, item) attention partial: item < k is the row's item-th selected
// block (no partial if -1); item == k is the window [max(0,L-W+1), L] minus
// keys of the row's selected blocks.  Partial = (m2, l, o[D]) unnormalised,
// base-2 logits.  16 lanes share one key: lane quarter (key group) kg =
// lane/16, column chunk cc = lane%16 of D/16 elements.
template <typename TIn, int D>
__global__ __launch_bounds__(kDecThreads) void decode_attn_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ Kc, const TIn* __restrict__ Vc,
    const int32_t* __restrict__ cache_len, const int32_t* __restrict__ idx, float* __restrict__ part,
    int g, int hq, int hkv, int64_t cap, int B, int k, int W, float scale2) {
  constexpr int EPL = D / 16;
  __shared__ float sq[D];
  __shared__ float sp[kDecKeyChunk];
  __shared__ float red[kDecThreads / 64];
  __shared__ float ored[kDecThreads / 64][D];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, kg = lane / 16, cc = lane % 16;
  const int64_t row = blockIdx.y, item = blockIdx.x;
  const int64_t b = row / hq, h = row % hq, kv = h / g, bkv = b * hkv + kv;
  const int64_t L = cache_len[b];
  float* dst = part + (row * (k + 1) + item) * (D + 2);
  int64_t j0, j1;
  bool window = item == k;
  if (L < 0 || L >= cap) {   // caller contract violated: an empty partial, no reads
    if (tid == 0) {
      dst[0] = -__builtin_inff();
      dst[1] = 0.f;
    }
    return;
  }
  if (!window) {
    // a selection must be a complete block before the query; anything else
    // (-1 padding) is an empty partial and nothing is read
    const int32_t c = idx[row * k + item];
    const int64_t C = min(int64_t(cap / B), (L + 1) / B);
    if (c < 0 || c >= C) {
      if (tid == 0) {
        dst[0] = -__builtin_inff();
        dst[1] = 0.f;
      }
      return;
    }
    j0 = int64_t(c) * B;
    j1 = j0 + B;
  } else {
    j0 = max(int64_t(0), L - W + 1);
    j1 = L + 1;
  }
  for (int i = tid; i < D; i += kDecThreads) sq[i] = load_f32(q, row * D + i);
  const TIn* Kh = Kc + bkv * cap * D;
  const TIn* Vh = Vc + bkv * cap * D;
  const int32_t* sel = idx + row * k;
  float m2 = -__builtin_inff(), l = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  __syncthreads();
  for (int64_t base = j0; base < j1; base += kDecKeyChunk) {
    const int nk = int(min<int64_t>(kDecKeyChunk, j1 - base));
    // logits: 16 keys per workgroup step
    for (int kk = wave * 4 + kg; kk < nk; kk += 16) {
      const int64_t j = base + kk;
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(sq[cc * EPL + e], load_f32(Kh, j * D + cc * EPL + e), dot);
#pragma unroll
      for (int o2 = 8; o2 >= 1; o2 >>= 1) dot += wave_shfl_xor(dot, o2);
      bool keep = true;
      if (window) {
        const int32_t blk = int32_t(j / B);
        for (int i = 0; i < k; ++i) keep = keep && sel[i] != blk;
      }
      if (cc == 0) sp[kk] = keep ? dot * scale2 : -__builtin_inff();
    }
    __syncthreads();
    float mloc = -__builtin_inff();
    for (int i = tid; i < nk; i += kDecThreads) mloc = fmaxf(mloc, sp[i]);
    const float mc = block_max(mloc, red);
    const float mnew = fmaxf(m2, mc);
    const float mref = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m2 - mref);
    m2 = mnew;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] *= alpha;
    __syncthreads();
    float lsum = 0.f;
    for (int i = tid; i < nk; i += kDecThreads) {
      const float p = __builtin_amdgcn_exp2f(sp[i] - mref);
      sp[i] = p;
      lsum += p;
    }
    l += block_sum(lsum, red);
    for (int kk = wave * 4 + kg; kk < nk; kk += 16) {
      const float p = sp[kk];
      const int64_t j = base + kk;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(p, load_f32(Vh, j * D + cc * EPL + e), o[e]);
    }
    __syncthreads();
  }
  // reduce o over the 4 key groups of a wave, then over waves
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    o[e] += wave_shfl_xor(o[e], 16);
    o[e] += wave_shfl_xor(o[e], 32);
  }
  if (kg == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) ored[wave][cc * EPL + e] = o[e];
  }
  __syncthreads();
  for (int i = tid; i < D; i += kDecThreads) {
    float s = 0.f;
    for (int w = 0; w < kDecThreads / 64; ++w) s += ored[w][i];
    dst[2 + i] = s;
  }
  if (tid == 0) {
    dst[0] = m2;
    dst[1] = l;
  }
}

template <typename OutT, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part,
                                                          OutT* __restrict__ o,
                                                          float* __restrict__ lse, int k) {
  const int64_t row = blockIdx.x;
  const float* P = part + row * (k + 1) * (D + 2);
  // an empty partial has l = 0 and is skipped; a NaN partial (non-finite
  // inputs) is kept, so NaN reaches o and lse
  float M = -__builtin_inff();
  for (int i = 0; i <= k; ++i) {
    const float* pi = P + i * (D + 2);
    if (pi[1] != 0.f) M = fmaxf(M, pi[0]);
  }
  float den = 0.f;
  for (int i = 0; i <= k; ++i) {
    const float* pi = P + i * (D + 2);
    if (pi[1] != 0.f) den += pi[1] * __builtin_amdgcn_exp2f(pi[0] - M);
  }
  for (int c = threadIdx.x; c < D; c += 64) {
    float acc = 0.f;
    for (int i = 0; i <= k; ++i) {
      const float* pi = P + i * (D + 2);
      if (pi[1] != 0.f) acc = fmaf(__builtin_amdgcn_exp2f(pi[0] - M), pi[2 + c], acc);
    }
    store_from_f32(o, row * D + c, acc / den);
  }
  if (threadIdx.x == 0) lse[row] = (M + __log2f(den)) * kLn2;
}

__global__ void fill_neg1_kernel(int32_t* p, int64_t count) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = -1;
}

__global__ void bump_len_kernel(int32_t* cache_len, int b) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < b) cache_len[i] += 1;
}

struct DecWs {
  float* scores;
  int32_t* idx;
  float* part;
  size_t bytes;
};

DecWs dec_ws_layout(const Shape& s, void* base) {
  DecWs w{};
  const int64_t rows = int64_t(s.b) * s.hq;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t o_sc = take(size_t(rows) * size_t(std::max<int64_t>(s.nb, 1)) * 4);
  const size_t o_idx = take(size_t(rows) * std::max(s.k, 1) * 4);
  const size_t o_part = take(size_t(rows) * (s.k + 1) * (s.d + 2) * 4);
  w.bytes = off;
  if (base) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.scores = reinterpret_cast<float*>(p + o_sc);
    w.idx = reinterpret_cast<int32_t*>(p + o_idx);
    w.part = reinterpret_cast<float*>(p + o_part);
  }
  return w;
}

template <typename TIn, int D, typename OutT>
hipError_t launch_decode_t(const Shape& s, const void* q, const void* k_new, const void* v_new,
                           void* K_cache, void* V_cache, int32_t* cache_len, float* mu,
                           float* sigma, int32_t* idx, void* o, float* lse, void* ws,
                           hipStream_t st) {
  DecWs w = dec_ws_layout(s, ws);
  const int64_t n_bkv = int64_t(s.b) * s.hkv, rows = int64_t(s.b) * s.hq;
  int32_t* sel = idx != nullptr ? idx : w.idx;
  hipError_t e;
  hipLaunchKernelGGL(append_kernel<TIn>, dim3(unsigned(n_bkv)), dim3(128), 0, st,
                     static_cast<const TIn*>(k_new), static_cast<const TIn*>(v_new),
                     static_cast<TIn*>(K_cache), static_cast<TIn*>(V_cache), cache_len, s.hkv, s.d,
                     s.n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (s.nb > 0) {
    if ((e = launch_block_stats(s, K_cache, mu, sigma, cache_len, st)) != hipSuccess) return e;
  }
  if (s.k > 0 && s.nb > 0) {
    const dim3 rgrid(unsigned((s.nb + kDecBlocksPerWg - 1) / kDecBlocksPerWg), unsigned(n_bkv));
    hipLaunchKernelGGL((decode_route_kernel<TIn, D>), rgrid, dim3(kDecThreads),
                       size_t(s.g) * D * 4, st, static_cast<const TIn*>(q), mu, sigma, cache_len,
                       w.scores, s.g, s.hq, s.hkv, s.B, s.nb, s.beta);
    if ((e = launch_decode_topk(w.scores, cache_len, sel, s.k, s.nb, s.hq, s.B, rows, st)) !=
        hipSuccess)
      return e;
  } else if (s.k > 0) {
    hipLaunchKernelGGL(fill_neg1_kernel, dim3(unsigned(std::min<int64_t>((rows * s.k + 255) / 256, 1024))),
                       dim3(256), 0, st, sel, rows * s.k);
  }
  const float scale2 = s.scale * kLog2e;
  hipLaunchKernelGGL((decode_attn_kernel<TIn, D>), dim3(unsigned(s.k + 1), unsigned(rows)),
                     dim3(kDecThreads), 0, st, static_cast<const TIn*>(q),
                     static_cast<const TIn*>(K_cache), static_cast<const TIn*>(V_cache), cache_len,
                     sel, w.part, s.g, s.hq, s.hkv, s.n, s.B, s.k, s.W, scale2);
  hipLaunchKernelGGL((decode_merge_kernel<OutT, D>), dim3(unsigned(rows)), dim3(64), 0, st, w.part,
                     static_cast<OutT*>(o), lse, s.k);
  hipLaunchKernelGGL(bump_len_kernel, dim3(unsigned((s.b + 255) / 256)), dim3(256), 0, st,
                     cache_len, s.b);
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_decode_o(const Shape& s, const void* q, const void* kn, const void* vn, void* Kc,
                           void* Vc, int32_t* cl, float* mu, float* sigma, int32_t* idx, void* o,
                           float* lse, void* ws, hipStream_t st) {
  if (s.out_bf16)
    return launch_decode_t<TIn, D, bf16_t>(s, q, kn, vn, Kc, Vc, cl, mu, sigma, idx, o, lse, ws, st);
  return launch_decode_t<TIn, D, float>(s, q, kn, vn, Kc, Vc, cl, mu, sigma, idx, o, lse, ws, st);
}

}  // namespace

hipError_t launch_decode_topk(const float* scores, const int32_t* pos, int32_t* idx, int k,
                              int64_t n_slots, int hq, int B, int64_t rows, hipStream_t st) {
  const dim3 tgrid(unsigned((rows + 3) / 4));
  if (k <= 8)
    hipLaunchKernelGGL(decode_topk_kernel<8>, tgrid, dim3(256), 0, st, scores, pos, idx, k,
                       n_slots, hq, B, rows);
  else if (k <= 16)
    hipLaunchKernelGGL(decode_topk_kernel<16>, tgrid, dim3(256), 0, st, scores, pos, idx, k,
                       n_slots, hq, B, rows);
  else
    hipLaunchKernelGGL(decode_topk_kernel<32>, tgrid, dim3(256), 0, st, scores, pos, idx, k,
                       n_slots, hq, B, rows);
  return hipGetLastError();
}

size_t decode_workspace_bytes(const Shape& s) { return dec_ws_layout(s, nullptr).bytes; }

// ---- scratch of the allocation-free decode entry point --------------------
//
// The same kernels with their workspace in a file-scope device array.  Each
// GPU holds its own copy for the life of the process; the host reads its
// address once per device (hipGetSymbolAddress, with that device current)
// and only ever passes that address: the array's name in host code is not a
// device address.  Nothing in it must start at zero (every score, selection
// and partial the kernels read is written earlier in the same step), and two
// calls that overlap in time on one GPU share it, so they race.
namespace {
constexpr int kScratchMaxDevices = 64;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kDecodeScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode_step(const Shape& s, const void* q, const void* k_new, const void* v_new,
                              void* K_cache, void* V_cache, int32_t* cache_len, float* mu,
                              float* sigma, int32_t* idx, void* o, float* lse, void* ws,
                              hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64
               ? launch_decode_o<bf16_t, 64>(s, q, k_new, v_new, K_cache, V_cache, cache_len, mu,
                                             sigma, idx, o, lse, ws, st)
               : launch_decode_o<bf16_t, 128>(s, q, k_new, v_new, K_cache, V_cache, cache_len, mu,
                                              sigma, idx, o, lse, ws, st);
  return s.d == 64 ? launch_decode_o<float, 64>(s, q, k_new, v_new, K_cache, V_cache, cache_len, mu,
                                                sigma, idx, o, lse, ws, st)
                   : launch_decode_o<float, 128>(s, q, k_new, v_new, K_cache, V_cache, cache_len,
                                                 mu, sigma, idx, o, lse, ws, st);
}

}  // namespace ssa
