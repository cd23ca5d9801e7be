// K/V chunk images shared by the attention kernels (per-query block
// attention, tile attention) and the exact-score router: every 64-key chunk
// of a head laid out as MFMA operand fragments (K as the A operand of
// S^T = K Q^T; V transposed, as the A operand of O^T = V^T P^T), staged into
// LDS with direct global->LDS loads; and the online-softmax step over one
// staged chunk that all attention kernels share.
//
// K part: fragment (mt, s), lane (m, h), element e = K[key0 + 32mt + m][16s + 8h + e];
// a query row's B-operand fragment s (load_row_frag) holds q[16s + 8h + e]
// in lane half h, so S^T = K Q^T contracts matching d on both sides.
#pragma once
#include <algorithm>
#include <type_traits>

#include "ssa_common.hpp"

namespace ssa {
namespace {

constexpr int kAttnThreads = 256;          // 4 waves
constexpr int kKeyChunk = 64;              // keys per LDS chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// A KV head's query row id rho = t g + jg (below 2^31) split into the
// position t and the group member jg by one 32-bit division (a 64-bit one is
// a long instruction sequence).
struct RowTJ {
  int64_t t, jg;
};
__device__ __forceinline__ RowTJ split_rho(int64_t rho, int g) {
  const uint32_t r = uint32_t(rho), t = r / uint32_t(g);
  return RowTJ{int64_t(t), int64_t(r - t * uint32_t(g))};
}

template <bool F32, int D>
struct AT {
  using In = typename std::conditional<F32, float, bf16_t>::type;
  using Frag = typename std::conditional<F32, floatx8, bf16x8>::type;    // Q, K operands
  using VFrag = typename std::conditional<F32, floatx8, f16x8>::type;    // P, V operands
  static constexpr int ES = F32 ? 4 : 2;          // element bytes
  static constexpr int LOG_NS = D == 128 ? 3 : 2;
  static constexpr int FRAG = 64 * 8 * ES;         // one operand fragment
  static constexpr int NS = D / 16;                // 16-wide chunks of d
  static constexpr int MTD = D / 32;               // 32-wide tiles of d
  static constexpr int KBYTES = 2 * NS * FRAG;     // 64 keys of K
  static constexpr int VBYTES = MTD * 4 * FRAG;    // 64 keys of V
  static constexpr int CHUNK = KBYTES + VBYTES;
  static constexpr int PIECE = 4 * ES;             // 4 elements
};

// ---------------------------------------------------------------- helpers --

// Copy `bytes` (a multiple of 1 KB) from global memory into LDS with direct
// global->LDS loads: each wave moves 1 KB per instruction, waves interleave.
__device__ __forceinline__ void dma_copy(uint8_t* lds, const uint8_t* src, int bytes, int tid,
                                         int nthreads) {
  const int wave = tid / 64, lane = tid % 64, waves = nthreads / 64;
  for (int r = wave; r < bytes / 1024; r += waves)
    __builtin_amdgcn_global_load_lds(src + r * 1024 + lane * 16,
                                     (__attribute__((address_space(3))) void*)(lds + r * 1024), 16,
                                     0, 0);
}

// The same copy written in asm (m0 saved and restored around each
// instruction), so the compiler does not know of it: it then does not make
// every later LDS read wait for the copy (it cannot tell the LDS buffers
// apart), and a copy into one buffer overlaps the work on another.  The
// caller waits for it itself -- s_waitcnt vmcnt(0), then a workgroup
// barrier -- before anything reads the copied bytes.  (Loads complete in
// order, so the compiler's own counted waits for later or earlier loads stay
// correct; they only wait longer.)
__device__ __forceinline__ void dma_copy_async(uint8_t* lds, const uint8_t* src, int bytes, int tid,
                                               int nthreads) {
  const int wave = tid / 64, lane = tid % 64, waves = nthreads / 64;
  const uint32_t base =
      uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t*)(lds)));
  for (int r = wave; r < bytes / 1024; r += waves) {
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

template <bool F32, int D>
__device__ __forceinline__ typename AT<F32, D>::Frag load_row_frag(const typename AT<F32, D>::In* row,
                                                                   int s, int h, bool valid) {
  typename AT<F32, D>::Frag v;
  if constexpr (F32) {
    floatx4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
    if (valid) {
      a = *reinterpret_cast<const floatx4*>(row + 16 * s + 8 * h);
      b = *reinterpret_cast<const floatx4*>(row + 16 * s + 8 * h + 4);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[e + 4] = b[e];
    }
  } else {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (valid) w = *reinterpret_cast<const u32x4*>(row + 16 * s + 8 * h);
    v = __builtin_bit_cast(bf16x8, w);
  }
  return v;
}

// Keys [key0, key0 + 64) of one head (rows >= n_keys read as zero), staged in
// LDS as MFMA A-operand fragments:
//   K part: fragment (mt, s), lane (m, h), element e = K[key0 + 32mt + m][16s + 8h + e]
//   V part: fragment (mt, s), lane (m, h), element e = V[key0 + frag_k(s,h,e)][32mt + m]
// K moves in 4-element pieces, assigned so that the 64 lanes of one LDS store
// fill 512 contiguous bytes (no bank conflicts).  V is transposed through
// registers in 4-key x 4-column tiles and, for bfloat16 inputs, converted to
// float16 after scaling by an exact power of two (vscale) that keeps every
// value of the head inside the float16 range: bf16 values then convert
// exactly, so P V runs as one float16 MFMA with P carrying 11 fraction bits.
// load() issues the global reads into registers and store() writes them to
// LDS, so a chunk's reads are in flight while the previous chunk is computed.
template <bool F32, int D>
struct ChunkRegs {
  using A = AT<F32, D>;
  using In = typename A::In;
  using PieceT = typename std::conditional<F32, floatx4, u32x2>::type;
  static constexpr int KPT = kKeyChunk * (D / 4) / kAttnThreads;         // K pieces per thread
  static constexpr int VPT = (kKeyChunk / 4) * (D / 4) / kAttnThreads;   // V tiles per thread
  PieceT k[KPT];
  PieceT v[VPT][4];

  // piece w of the K chunk: lanes vary (m, sel) fastest, then h, s, mt
  __device__ static __forceinline__ void kpiece(int w, int& mt, int& m, int& s, int& h, int& sel) {
    m = w & 31;
    sel = (w >> 5) & 1;
    h = (w >> 6) & 1;
    s = (w >> 7) & (A::NS - 1);
    mt = w >> (7 + A::LOG_NS);
  }

  __device__ __forceinline__ void load(const In* Kh, const In* Vh, int64_t key0, int64_t n_keys,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int mt, m, s, h, sel;
      kpiece(tid + i * kAttnThreads, mt, m, s, h, sel);
      const int r = 32 * mt + m;
      k[i] = PieceT{};
      if (key0 + r < n_keys)
        k[i] = *reinterpret_cast<const PieceT*>(Kh + (key0 + r) * D + 16 * s + 8 * h + 4 * sel);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int w = tid + i * kAttnThreads, kq = w / (D / 4), dq = w % (D / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[i][r] = PieceT{};
        if (key0 + 4 * kq + r < n_keys)
          v[i][r] = *reinterpret_cast<const PieceT*>(Vh + (key0 + 4 * kq + r) * D + 4 * dq);
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds, int tid, float vscale) const {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int mt, m, s, h, sel;
      kpiece(tid + i * kAttnThreads, mt, m, s, h, sel);
      *reinterpret_cast<PieceT*>(lds + (mt * A::NS + s) * A::FRAG + (h * 32 + m) * 8 * A::ES +
                                 sel * A::PIECE) = k[i];
    }
    uint8_t* vl = lds + A::KBYTES;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int w = tid + i * kAttnThreads, kq = w / (D / 4), dq = w % (D / 4);
      const int s = kq / 4, kg = kq % 4, sel = kg >> 1, h = kg & 1;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        const int d = 4 * dq + dd, mt = d / 32, m = d % 32;
        PieceT col;
        if constexpr (F32) {
          col = floatx4{v[i][0][dd], v[i][1][dd], v[i][2][dd], v[i][3][dd]};
        } else {
          const int word = dd >> 1, shift = (dd & 1) * 16;
          uint32_t e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = bf16_bits_to_f32((v[i][r][word] >> shift) & 0xFFFFu) * vscale;
            e[r] = __builtin_bit_cast(u16, static_cast<_Float16>(x));
          }
          col = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
        }
        *reinterpret_cast<PieceT*>(vl + (mt * 4 + s) * A::FRAG + (h * 32 + m) * 8 * A::ES +
                                   sel * A::PIECE) = col;
      }
    }
  }
};

// Power-of-two scale for the float16 value operand of one head: vexp_bits is
// the largest |v| of the head as bfloat16 bits; returns e >= 0 with
// max|v| * 2^-e < 2^15.
__device__ __forceinline__ int value_exponent(uint32_t vmax_bits) {
  const float vmax = bf16_bits_to_f32(vmax_bits & 0x7FFFu);
  int E = 0;
  if (vmax > 0.f) (void)frexpf(vmax, &E);   // vmax < 2^E
  return E > 15 ? E - 15 : 0;
}

// Chunk images: every 64-key chunk of every head, already in the LDS layout
// above (K fragments, then V transposed and, for bfloat16 inputs, converted to
// float16).  Written once per call; the attention kernels then stage a chunk
// with straight 16-byte global->LDS DMA loads, no registers and no transposes.
template <bool F32, int D>
__global__ __launch_bounds__(kAttnThreads) void kv_image_kernel(
    const typename AT<F32, D>::In* __restrict__ K, const typename AT<F32, D>::In* __restrict__ V,
    const uint32_t* __restrict__ vmax, uint8_t* __restrict__ img, int64_t n, int64_t n_chunks) {
  using A = AT<F32, D>;
  const int64_t ci = blockIdx.x, bkv = blockIdx.y;
  const float vscale = F32 ? 1.f : ldexpf(1.f, -value_exponent(vmax[bkv]));
  ChunkRegs<F32, D> cr;
  cr.load(K + bkv * n * D, V + bkv * n * D, ci * kKeyChunk, n, threadIdx.x);
  cr.store(img + (bkv * n_chunks + ci) * A::CHUNK, threadIdx.x, vscale);
}

// Largest |v| of every (sequence, KV head), as bfloat16 bits (order-preserving
// for non-negative values), for the float16 value scale.  Each thread keeps
// kMaxLoads 16-byte loads in flight per round, and a workgroup folds its
// waves in LDS before a single atomic (thousands of atomics on one address
// serialise at the cache and dominated small inputs).
constexpr int kMaxLoads = 8;

// Workgroups per (sequence, KV head) for value_max_kernel over per_head
// bfloat16 values: one round of kMaxLoads loads per thread, at most 128.
inline unsigned value_max_groups(int64_t per_head) {
  const int64_t n16 = per_head / 8, per_group = 256 * kMaxLoads;
  return unsigned(std::max<int64_t>(1, std::min<int64_t>((n16 + per_group - 1) / per_group, 128)));
}

__global__ __launch_bounds__(256) void value_max_kernel(const bf16_t* __restrict__ V,
                                                        uint32_t* __restrict__ vmax,
                                                        int64_t per_head) {
  __shared__ uint32_t wmax[4];
  const int64_t bkv = blockIdx.y;
  const u32x4* src = reinterpret_cast<const u32x4*>(V + bkv * per_head);
  const int64_t n16 = per_head / 8;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  uint32_t m = 0;
  for (int64_t i0 = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i0 < n16; i0 += kMaxLoads * stride) {
    u32x4 w[kMaxLoads];
#pragma unroll
    for (int u = 0; u < kMaxLoads; ++u) {
      const int64_t i = i0 + u * stride;
      w[u] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kMaxLoads; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max(m, max(w[u][j] & 0x7FFFu, (w[u][j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, uint32_t(__shfl_xor(int(m), o, 64)));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t r = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    atomicMax(&vmax[bkv], r);
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t count, int32_t v) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < count;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

// ------------------------------------------------ attention over a chunk --

constexpr float kLazyLog2 = 8.f;   // probabilities may reach 2^kLazyLog2 before a rescale

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

// One 64-key chunk for the NT 32-row tiles of this wave; every fragment read
// from LDS feeds NT MFMAs.  mask(nt, mt, a, b) says whether key
// 32mt + 8a + 4h + b of the chunk counts for this lane's row of tile nt.
// Probabilities are exp2(s * scale2 - m) with the running row max m in the
// same base-2 units; for bfloat16 inputs they enter P V as float16.
template <bool F32, int D, int NT, typename Mask>
__device__ __forceinline__ void attend_chunk(const uint8_t* lds,
                                             const typename AT<F32, D>::Frag (&bq)[NT][D / 16],
                                             float scale2, int lane, RowState<D> (&st)[NT],
                                             Mask mask) {
  using A = AT<F32, D>;
  using Frag = typename A::Frag;
  using VFrag = typename A::VFrag;
  floatx16 sacc[NT][2];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) sacc[nt][mt][j] = 0.f;
  // S^T = K Q^T: the two 32-key tiles are independent accumulator chains,
  // interleaved; K fragments are read from LDS two steps ahead of use.
  auto kfrag = [&](int mt, int s) {
    return *reinterpret_cast<const Frag*>(lds + (mt * A::NS + s) * A::FRAG + lane * 8 * A::ES);
  };
  Frag ka[3][2];
  ka[0][0] = kfrag(0, 0);
  ka[0][1] = kfrag(1, 0);
  ka[1][0] = kfrag(0, 1);
  ka[1][1] = kfrag(1, 1);
#pragma unroll
  for (int s = 0; s < A::NS; ++s) {
    if (s + 2 < A::NS) {
      ka[(s + 2) % 3][0] = kfrag(0, s + 2);
      ka[(s + 2) % 3][1] = kfrag(1, s + 2);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[nt][mt] = mma16(ka[s % 3][mt], bq[nt][s], sacc[nt][mt]);
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float mloc = -__builtin_inff();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v = sacc[nt][mt][4 * a + b];
          if (!mask(nt, mt, a, b)) v = -__builtin_inff();
          sacc[nt][mt][4 * a + b] = v;
          mloc = fmaxf(mloc, v);
        }
    mloc = fmaxf(mloc, wave_shfl_xor(mloc, 32)) * scale2;
    // Lazy rescaling: the reference m2 moves (and o, l are rescaled) only
    // when some row of the wave sees a logit more than kLazyLog2 above it, so
    // probabilities stay below 2^kLazyLog2 and most chunks skip the rescale.
    if (__builtin_amdgcn_ballot_w64(mloc > st[nt].m2 + kLazyLog2) != 0) {
      const float mold = st[nt].m2;
      const float mnew = fmaxf(mold, mloc);
      const float alpha = __builtin_amdgcn_exp2f(mold - (mnew == -__builtin_inff() ? 0.f : mnew));
      st[nt].m2 = mnew;
      st[nt].l *= alpha;
      // a row whose reference is still -inf has o = 0 (or NaN from a
      // non-finite value), which alpha = 0 leaves as it is: a wave whose
      // rows all start here -- every first chunk -- skips the products
      if (__builtin_amdgcn_ballot_w64(mold != -__builtin_inff()) != 0) {
#pragma unroll
        for (int i = 0; i < A::MTD; ++i) st[nt].o[i] *= alpha;
      }
    }
    const float mref = st[nt].m2 == -__builtin_inff() ? 0.f : st[nt].m2;
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[nt][mt][j], scale2, -mref));
        sacc[nt][mt][j] = p;
        lsum += p;
      }
    st[nt].l += lsum;
  }
  // P as the B operand of O^T += V^T P^T: chunk s' covers keys 16s'..16s'+15.
  // The MTD output tiles are independent chains; V fragments are read one
  // step ahead of use.
  const uint8_t* vl = lds + A::KBYTES;
  auto vfrag = [&](int mt, int sp) {
    return *reinterpret_cast<const VFrag*>(vl + (mt * 4 + sp) * A::FRAG + lane * 8 * A::ES);
  };
  VFrag va[2][A::MTD];
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt) va[0][mt] = vfrag(mt, 0);
#pragma unroll
  for (int sp = 0; sp < 4; ++sp) {
    if (sp + 1 < 4) {
#pragma unroll
      for (int mt = 0; mt < A::MTD; ++mt) va[(sp + 1) & 1][mt] = vfrag(mt, sp + 1);
    }
    VFrag pf[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = sacc[nt][sp >> 1][4 * (2 * (sp & 1) + (e >> 2)) + (e & 3)];
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[nt][e] = pv[e];
      } else {
        pf[nt] = to_f16x8(pv);
      }
    }
#pragma unroll
    for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st[nt].o[mt] = mma16(va[sp & 1][mt], pf[nt], st[nt].o[mt]);
  }
}


// N resident chunks against one 32-row tile, 16-bit inputs and no mask: the
// arithmetic of attend_chunk (the same products in the same order, so the
// same results), with each key tile's score chain for chunk c+1 issued into
// the accumulator that tile's probabilities of chunk c have just left --
// the matrix core works on the next chunk's scores while the vector ALU
// finishes this chunk's softmax, within the registers of one chunk.
template <int D, int N>
__device__ __forceinline__ void attend_segment(const uint8_t* lds, const bf16x8 (&bq)[D / 16],
                                               float scale2, int lane, RowState<D>& st) {
  using A = AT<false, D>;
  constexpr int NS = A::NS, MTD = A::MTD;
  auto kfrag = [&](int c, int mt, int s) {
    return *reinterpret_cast<const bf16x8*>(lds + c * A::CHUNK + (mt * NS + s) * A::FRAG + lane * 16);
  };
  auto vfrag = [&](int c, int mt, int sp) {
    return *reinterpret_cast<const f16x8*>(lds + c * A::CHUNK + A::KBYTES + (mt * 4 + sp) * A::FRAG +
                                           lane * 16);
  };
  auto scores = [&](int c, int mt) {
    floatx16 acc = mma16(kfrag(c, mt, 0), bq[0], floatx16{});
#pragma unroll
    for (int s = 1; s < NS; ++s) acc = mma16(kfrag(c, mt, s), bq[s], acc);
    return acc;
  };
  floatx16 sacc[2] = {scores(0, 0), scores(0, 1)};
#pragma unroll
  for (int c = 0; c < N; ++c) {
    float mloc = -__builtin_inff();
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) mloc = fmaxf(mloc, sacc[mt][j]);
    mloc = fmaxf(mloc, wave_shfl_xor(mloc, 32)) * scale2;
    if (__builtin_amdgcn_ballot_w64(mloc > st.m2 + kLazyLog2) != 0) {
      const float mold = st.m2;
      const float mnew = fmaxf(mold, mloc);
      const float alpha = __builtin_amdgcn_exp2f(mold - (mnew == -__builtin_inff() ? 0.f : mnew));
      st.m2 = mnew;
      st.l *= alpha;
      if (__builtin_amdgcn_ballot_w64(mold != -__builtin_inff()) != 0) {
#pragma unroll
        for (int i = 0; i < MTD; ++i) st.o[i] *= alpha;
      }
    }
    const float mref = st.m2 == -__builtin_inff() ? 0.f : st.m2;
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f16x8 pf[2];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][j], scale2, -mref));
        sacc[mt][j] = p;
        lsum += p;
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = sacc[mt][4 * (2 * q + (e >> 2)) + (e & 3)];
        pf[q] = to_f16x8(pv);
      }
      if (c + 1 < N) sacc[mt] = scores(c + 1, mt);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int m = 0; m < MTD; ++m) st.o[m] = mma16(vfrag(c, m, 2 * mt + q), pf[q], st.o[m]);
    }
    st.l += lsum;
  }
}

}  // namespace
}  // namespace ssa
