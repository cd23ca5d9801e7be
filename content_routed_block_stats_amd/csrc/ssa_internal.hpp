// Host-side contract between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace ssa {

// Validated shapes and parameters of one call (see include/ssa.h).
struct Shape {
  int b, hq, hkv, g, d;
  int64_t n;      // prefill length, or decode cache capacity
  int B, k, W;
  int64_t nb;     // complete blocks of n (stat slots per (sequence, KV head))
  float beta, scale;
  bool in_bf16, out_bf16;
};

// A second stream of the current device (default priority, created on first
// use) for work that can run beside the caller's stream: everything enqueued
// on stream() after the lease starts follows the caller's stream's work so
// far, and join() (or the destructor) makes the caller's stream wait for it.
// One lease at a time per device (a mutex held while the launches are
// enqueued, not while they run); under stream capture, or if the stream or
// its events cannot be created, stream() is the caller's stream.
class SideLease {
 public:
  explicit SideLease(hipStream_t st) : st_(st) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return;
    Slot& sl = slots()[dev];
    lock_ = std::unique_lock<std::mutex>(sl.mu);
    if (!sl.tried) {
      sl.tried = true;
      sl.ok = hipStreamCreateWithFlags(&sl.s, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&sl.fork, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&sl.join, hipEventDisableTiming) == hipSuccess;
    }
    if (!sl.ok || hipEventRecord(sl.fork, st) != hipSuccess ||
        hipStreamWaitEvent(sl.s, sl.fork, 0) != hipSuccess) {
      lock_.unlock();
      return;
    }
    slot_ = &sl;
  }
  ~SideLease() { (void)join(); }
  SideLease(const SideLease&) = delete;
  SideLease& operator=(const SideLease&) = delete;
  hipStream_t stream() const { return slot_ != nullptr ? slot_->s : st_; }
  // the caller's stream waits for everything enqueued on stream() so far
  hipError_t join() {
    if (slot_ == nullptr) return hipSuccess;
    hipError_t e = hipEventRecord(slot_->join, slot_->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(st_, slot_->join, 0);
    if (e != hipSuccess) e = hipStreamSynchronize(slot_->s);   // ordering at any cost
    slot_ = nullptr;
    lock_.unlock();
    return e;
  }

 private:
  static constexpr int kMaxDev = 64;
  struct Slot {
    std::mutex mu;
    bool tried = false, ok = false;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
  };
  static Slot* slots() {
    static Slot s[kMaxDev];
    return s;
  }
  hipStream_t st_;
  Slot* slot_ = nullptr;
  std::unique_lock<std::mutex> lock_;
};

constexpr size_t kWsAlign = 256;
inline size_t align_up(size_t x, size_t a = kWsAlign) { return (x + a - 1) / a * a; }

// block statistics.  cache_len == nullptr: every block c < s.nb of every
// (sequence, KV head), keys read from K [b, hkv, s.n, d].  Otherwise decode
// mode: only the block completed by the key at position cache_len[b]
// (if any), with K the caches [b, hkv, s.n, d].
hipError_t launch_block_stats(const Shape& s, const void* K, float* mu, float* sigma,
                              const int32_t* cache_len, hipStream_t st);

// routing + top-k (prefill)
size_t route_workspace_bytes(const Shape& s);
hipError_t launch_route_topk(const Shape& s, const void* Q, const float* mu, const float* sigma,
                             int32_t* idx, float* kth, void* ws, hipStream_t st);

// exact tempered block score + top-k (prefill); no workspace.  Grid size in
// workgroups (must stay below 2^31).
int64_t tempered_route_tiles(const Shape& s);
hipError_t launch_route_tempered(const Shape& s, const void* Q, const void* K, int32_t* idx,
                                 float* kth, hipStream_t st);

// query-tile-shared routing (prefill): tiles of B positions per (sequence,
// q-head); idx [b, hq, tile_count, k]
int64_t tile_count(const Shape& s);
size_t route_tiles_workspace_bytes(const Shape& s);
hipError_t launch_route_tiles(const Shape& s, const void* Q, const float* mu, const float* sigma,
                              int32_t* idx, float* kth, void* ws, hipStream_t st);

// attention over tile selections (prefill); the chunk list of one workgroup
// (k B/64 selected chunks + the window's) must fit tile_attn_max_list()
size_t tile_attn_workspace_bytes(const Shape& s);
int tile_attn_max_list();
hipError_t launch_tile_attn(const Shape& s, const void* Q, const void* K, const void* V,
                            const int32_t* tidx, void* O, float* lse, void* ws, hipStream_t st);

// sparse attention (prefill)
size_t attn_workspace_bytes(const Shape& s);
// entry / partial slots of the block pass (tasks padded to whole task rows);
// positions are 32-bit, so this must stay below 2^31
int64_t attn_entry_slots(const Shape& s);
hipError_t launch_sparse_attn(const Shape& s, const void* Q, const void* K, const void* V,
                              const int32_t* idx, void* O, float* lse, void* ws, hipStream_t st);

// The block-major dispatch of the sparse attention (a counting sort of the
// (row, slot) selections by (sequence, KV head, block)), for other passes over
// the same selections.  Segment s = (b * hkv + kv) * nb + c holds counts[s]
// entries, at [cursor[s] - counts[s], cursor[s]) after the dispatch; task j
// = {segment, first entry j * 256, rows, 0} for j < task_count[0]; entry =
// (t * g + j) << 5 | slot; pos[row * k + slot] = the entry's index.
struct DispatchWs {
  int32_t* counts;
  int32_t* cursor;
  int32_t* task_count;
  int4* tasks;
  uint32_t* entries;
  int32_t* pos;
  int64_t max_tasks;
  int64_t slots;
  size_t bytes;
};
DispatchWs dispatch_ws_layout(const Shape& s, void* base);
hipError_t launch_dispatch(const Shape& s, const int32_t* idx, const DispatchWs& w, hipStream_t st);

// backward of the sparse attention over fixed selections (prefill)
size_t attn_bwd_workspace_bytes(const Shape& s);
hipError_t launch_sparse_attn_bwd(const Shape& s, const void* Q, const void* K, const void* V,
                                  const int32_t* idx, const void* O, const float* lse,
                                  const void* dO, float* dQ, float* dK, float* dV, void* ws,
                                  hipStream_t st);

// exact hierarchical routing (branch and bound over groups of m blocks)
int hier_max_rows();
int hier_max_bounds();
int hier_max_group();
size_t route_hier_workspace_bytes(const Shape& s);   // any group size
hipError_t launch_group_stats(const Shape& s, const float* mu, const float* sigma, int m, float* gmu,
                              float* gS, float* grl, hipStream_t st);
hipError_t launch_route_hier(const Shape& s, const void* q, const float* mu, const float* sigma,
                             const float* gmu, const float* gS, const float* grl, int m,
                             const int32_t* pos, int32_t* idx, int32_t* evaluated, void* ws,
                             hipStream_t st);

// exact hierarchical routing of prefill rows (bfloat16 inputs): group bounds
// per 512-row tile of a KV head's rows, then a visit per tile;
// evaluated [b*hkv][route_tile_count] blocks scored per tile (or nullptr)
size_t route_hier_prefill_workspace_bytes(const Shape& s, int m);
int hier_prefill_max_groups();
int64_t route_tile_count(const Shape& s);
hipError_t launch_route_hier_prefill(const Shape& s, const void* Q, const float* mu,
                                     const float* sigma, const float* gmu, const float* gS,
                                     const float* grl, int m, int32_t* idx, int32_t* evaluated,
                                     void* ws, hipStream_t st);

// decode step
size_t decode_workspace_bytes(const Shape& s);
// the allocation-free variant's scratch: a device array of this many bytes,
// whose address on the current device decode_scratch() returns
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** out);
// wave top-k of scores [rows, n_slots] over the blocks c < min(n_slots,
// (pos[row / hq] + 1) / B), ascending, -1 padded (k <= 32)
hipError_t launch_decode_topk(const float* scores, const int32_t* pos, int32_t* idx, int k,
                              int64_t n_slots, int hq, int B, int64_t rows, hipStream_t st);
hipError_t launch_decode_step(const Shape& s, const void* q, const void* k_new, const void* v_new,
                              void* K_cache, void* V_cache, int32_t* cache_len, float* mu,
                              float* sigma, int32_t* idx, void* o, float* lse, void* ws,
                              hipStream_t st);

}  // namespace ssa
