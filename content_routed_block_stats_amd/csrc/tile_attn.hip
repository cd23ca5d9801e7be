// Attention for query-tile-shared routing (prefill).
//
// Write-up "Subquadratic Sparse Attention (SSA)", introduction steps (ii)-(iii),
// with the selection made per query tile (tile_route.hip): every row t of
// tile j attends, with an exact softmax, to the keys of the tile's selected
// blocks (all before the tile, so no causal mask inside them) and to its own
// window [max(0, t-W+1), t], each key once.  Since the rows of a tile share
// their blocks, the work is dense: one workgroup per (sequence, q-head, 256
// rows of a tile) streams the selected blocks' 64-key chunk images through
// LDS once for all its rows, then the window chunks (a chunk of a selected
// block is skipped there: its keys already counted), with the same MFMA
// online-softmax step as the per-query attention, and writes O and LSE
// directly -- no partials, no merge.
#include <algorithm>
#include <type_traits>

#include "kv_chunks.hpp"
#include "ssa_common.hpp"
#include "ssa_internal.hpp"

namespace ssa {
namespace {

constexpr int kTileThreads = 512;   // 8 waves x 32 rows
constexpr int kTileRows = 256;      // rows per workgroup (a tile holds B rows)
constexpr int kMaxList = 1024;      // chunk list: the selected blocks' chunks, then the window's

template <bool F32, int D, typename OutT>
__global__ __launch_bounds__(kTileThreads) void tile_attn_kernel(
    const typename AT<F32, D>::In* __restrict__ Q, const uint8_t* __restrict__ img,
    const uint32_t* __restrict__ vmax, const int32_t* __restrict__ tidx, OutT* __restrict__ O,
    float* __restrict__ lse, int64_t n, int g, int hq, int hkv, int B, int k, int W, float scale2,
    int64_t n_tiles, int subs, int64_t n_chunks, int64_t n_work) {
  using A = AT<F32, D>;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * A::CHUNK];
  __shared__ int32_t list[kMaxList];
  __shared__ int32_t nlist[2];   // selected-chunk count, total count

  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, ln = lane % 32, h = lane / 32;
  // Work items run sub-tile fastest, then the group's q-heads, then tiles,
  // then (sequence, KV head); consecutive items go to one XCD (workgroup i
  // runs on XCD i % 8), so the heads of a tile share their window chunks and
  // neighbouring tiles their blocks in that XCD's L2.
  const int64_t per_xcd = gridDim.x / 8;
  const int64_t wi = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (wi >= n_work) return;
  const int sub = int(wi % subs);
  const int64_t jg = (wi / subs) % g, j = (wi / (int64_t(subs) * g)) % n_tiles;
  const int64_t bkv = wi / (int64_t(subs) * g * n_tiles), b = bkv / hkv, kv = bkv % hkv;
  const int64_t bh = b * hq + kv * g + jg;
  const int64_t r0 = j * B + int64_t(sub) * kTileRows;
  const int64_t r_end = min(min(n, (j + 1) * B), r0 + kTileRows) - 1;   // last row (inclusive)
  if (r0 > r_end) return;
  const int cpb = B / kKeyChunk;

  // chunk list: the selected blocks' chunks, then the window chunks that lie
  // in no selected block
  if (tid == 0) {
    const int32_t* sel = tidx + (bh * n_tiles + j) * k;
    int cnt = 0;
    for (int i = 0; i < k; ++i) {
      const int32_t c = sel[i];
      if (c < 0) continue;
      for (int q = 0; q < cpb; ++q) list[cnt++] = c * cpb + q;
    }
    const int nsel = cnt;
    const int64_t ch_lo = max(int64_t(0), r0 - W + 1) / kKeyChunk, ch_hi = r_end / kKeyChunk;
    for (int64_t ch = ch_lo; ch <= ch_hi; ++ch) {
      const int32_t blk = int32_t(ch * kKeyChunk / B);
      bool excl = false;
      for (int i = 0; i < k; ++i) excl |= sel[i] == blk;
      if (!excl) list[cnt++] = int32_t(ch);
    }
    nlist[0] = nsel;
    nlist[1] = cnt;
  }
  const int64_t t = r0 + 32 * wave + ln;
  const bool valid = t <= r_end;
  typename A::Frag bq[1][A::NS];
  {
    const auto* qrow = Q + (bh * n + (valid ? t : r0)) * D;
#pragma unroll
    for (int s = 0; s < A::NS; ++s) bq[0][s] = load_row_frag<F32, D>(qrow, s, h, valid);
  }
  const bool wave_active = r0 + 32 * wave <= r_end;
  const int64_t wave_t_lo = r0 + 32 * wave, wave_t_hi = min(r_end, wave_t_lo + 31);
  const uint8_t* src = img + bkv * n_chunks * A::CHUNK;
  const int64_t tv = valid ? t : -(int64_t(1) << 40);
  RowState<D> st[1];
  row_state_init(st[0]);
  // the query fragments are in before the loop, so the compiler's own waits
  // inside it (it cannot see the chunk copies) have nothing left to wait for
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int nsel = nlist[0], cnt = nlist[1];
  if (cnt > 0) dma_copy_async(lds, src + int64_t(list[0]) * A::CHUNK, A::CHUNK, tid, kTileThreads);
  // chunk i has landed (this wave's copies, then everyone's), and every wave
  // is done with chunk i-1, whose buffer the next copy refills while chunk i
  // is computed
  auto next_chunk = [&](int i) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (i + 1 < cnt)
      dma_copy_async(lds + ((i & 1) ^ 1) * A::CHUNK, src + int64_t(list[i + 1]) * A::CHUNK,
                     A::CHUNK, tid, kTileThreads);
  };
  // A selected block lies before the tile: every key counts for every row, so
  // these chunks take no mask and no branch (a wave past the tile's last row
  // works on zero queries and discards the result).  Kept apart from the
  // window chunks' loop, whose branch would otherwise make the compiler copy
  // the output accumulators on every chunk.
  for (int i = 0; i < nsel; ++i) {
    next_chunk(i);
    attend_chunk<F32, D, 1>(lds + (i & 1) * A::CHUNK, bq, scale2, lane, st,
                            [](int, int, int, int) { return true; });
  }
  // window chunks count keys in (t - W, t]
  for (int i = nsel; i < cnt; ++i) {
    next_chunk(i);
    const int64_t key0 = int64_t(list[i]) * kKeyChunk;
    if (wave_active && key0 <= wave_t_hi && key0 + kKeyChunk - 1 > wave_t_lo - W) {
      // 32-bit positions and bitwise tests: no exec-mask blocks per element
      const int32_t lo = int32_t(max(tv - W, int64_t(INT32_MIN)));
      const int32_t hi = int32_t(max(tv, int64_t(INT32_MIN)));
      const int32_t kb = int32_t(key0) + 4 * h;
      attend_chunk<F32, D, 1>(lds + (i & 1) * A::CHUNK, bq, scale2, lane, st,
                              [&](int, int mt, int a, int bb) {
                                const int32_t kj = kb + 32 * mt + 8 * a + bb;
                                return (kj <= hi) & (kj > lo);
                              });
    }
  }

  // O^T accumulators: lane (ln, h) holds columns 32mt + 8a + 4h + b of row t
  const float l = st[0].l + wave_shfl_xor(st[0].l, 32);
  if (!valid) return;
  const float inv = ldexpf(1.f / l, F32 ? 0 : value_exponent(vmax[bkv]));
  OutT* orow = O + (bh * n + t) * D;
#pragma unroll
  for (int mt = 0; mt < A::MTD; ++mt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int col = 32 * mt + 8 * a + 4 * h;
      if constexpr (std::is_same<OutT, float>::value) {
        *reinterpret_cast<floatx4*>(orow + col) =
            floatx4{st[0].o[mt][4 * a] * inv, st[0].o[mt][4 * a + 1] * inv,
                    st[0].o[mt][4 * a + 2] * inv, st[0].o[mt][4 * a + 3] * inv};
      } else {
        u32x2 w;
        w[0] = uint32_t(f32_to_bf16_bits(st[0].o[mt][4 * a] * inv)) |
               (uint32_t(f32_to_bf16_bits(st[0].o[mt][4 * a + 1] * inv)) << 16);
        w[1] = uint32_t(f32_to_bf16_bits(st[0].o[mt][4 * a + 2] * inv)) |
               (uint32_t(f32_to_bf16_bits(st[0].o[mt][4 * a + 3] * inv)) << 16);
        *reinterpret_cast<u32x2*>(orow + col) = w;
      }
    }
  if (h == 0) lse[bh * n + t] = (st[0].m2 + __log2f(l)) * kLn2;
}

struct TileWs {
  uint32_t* vmax;
  uint8_t* img;
  int64_t n_chunks;
  size_t bytes;
};

TileWs tile_ws_layout(const Shape& s, void* base) {
  TileWs w{};
  const size_t es = s.in_bf16 ? 2 : 4;
  const size_t o_vmax = 0;
  const size_t o_img = align_up(size_t(s.b) * s.hkv * 4);
  w.n_chunks = (s.n + kKeyChunk - 1) / kKeyChunk;
  w.bytes = o_img + align_up(size_t(s.b) * s.hkv * size_t(w.n_chunks) * kKeyChunk * s.d * 2 * es);
  if (base != nullptr) {
    uint8_t* p = static_cast<uint8_t*>(base);
    w.vmax = reinterpret_cast<uint32_t*>(p + o_vmax);
    w.img = p + o_img;
  }
  return w;
}

template <bool F32, int D, typename OutT>
hipError_t launch_tile_attn_t(const Shape& s, const void* Qv, const void* Kv, const void* Vv,
                              const int32_t* tidx, void* Ov, float* lse, void* ws, hipStream_t st) {
  using A = AT<F32, D>;
  using In = typename A::In;
  TileWs w = tile_ws_layout(s, ws);
  const int64_t n_bkv = int64_t(s.b) * s.hkv;
  if (!F32) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(256), 0, st,
                       reinterpret_cast<int32_t*>(w.vmax), n_bkv, 0);
    const int64_t per_head = s.n * D;
    const unsigned gx = value_max_groups(per_head);
    hipLaunchKernelGGL(value_max_kernel, dim3(gx, unsigned(n_bkv)), dim3(256), 0, st,
                       reinterpret_cast<const bf16_t*>(Vv), w.vmax, per_head);
  }
  hipLaunchKernelGGL((kv_image_kernel<F32, D>), dim3(unsigned(w.n_chunks), unsigned(n_bkv)),
                     dim3(kAttnThreads), 0, st, static_cast<const In*>(Kv),
                     static_cast<const In*>(Vv), w.vmax, w.img, s.n, w.n_chunks);
  const int64_t n_tiles = tile_count(s);
  const int subs = (s.B + kTileRows - 1) / kTileRows;
  const int64_t n_work = int64_t(s.b) * s.hq * n_tiles * subs;
  const int64_t grid = (n_work + 7) / 8 * 8;   // a multiple of the 8 XCDs
  hipLaunchKernelGGL((tile_attn_kernel<F32, D, OutT>), dim3(unsigned(grid)), dim3(kTileThreads), 0,
                     st, static_cast<const In*>(Qv), w.img, w.vmax, tidx, static_cast<OutT*>(Ov),
                     lse, s.n, s.g, s.hq, s.hkv, s.B, s.k, s.W, s.scale * kLog2e, n_tiles, subs,
                     w.n_chunks, n_work);
  return hipGetLastError();
}

template <bool F32, int D>
hipError_t launch_tile_attn_d(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* tidx, void* O, float* lse, void* ws, hipStream_t st) {
  if (s.out_bf16) return launch_tile_attn_t<F32, D, bf16_t>(s, Q, K, V, tidx, O, lse, ws, st);
  return launch_tile_attn_t<F32, D, float>(s, Q, K, V, tidx, O, lse, ws, st);
}

}  // namespace

size_t tile_attn_workspace_bytes(const Shape& s) { return tile_ws_layout(s, nullptr).bytes; }

int tile_attn_max_list() { return kMaxList; }

hipError_t launch_tile_attn(const Shape& s, const void* Q, const void* K, const void* V,
                            const int32_t* tidx, void* O, float* lse, void* ws, hipStream_t st) {
  if (s.in_bf16)
    return s.d == 64 ? launch_tile_attn_d<false, 64>(s, Q, K, V, tidx, O, lse, ws, st)
                     : launch_tile_attn_d<false, 128>(s, Q, K, V, tidx, O, lse, ws, st);
  return s.d == 64 ? launch_tile_attn_d<true, 64>(s, Q, K, V, tidx, O, lse, ws, st)
                   : launch_tile_attn_d<true, 128>(s, Q, K, V, tidx, O, lse, ws, st);
}

}  // namespace ssa
