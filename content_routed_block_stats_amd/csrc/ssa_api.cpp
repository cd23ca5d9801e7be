// C ABI of the SSA hot path: host-side validation, workspace sizing and
// dispatch to the gfx950 kernel launchers.  Every check runs before anything
// is enqueued; no C++ exception crosses the interface.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ssa.h"
#include "ssa_internal.hpp"

namespace {

thread_local char g_err[512] = "";

ssa_status fail(ssa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

ssa_status ok() {
  g_err[0] = '\0';
  return SSA_OK;
}

ssa_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxSeq = int64_t(1) << 30;
constexpr int64_t kMaxRowsPerHead = int64_t(1) << 26;   // n * (Hq/Hkv), packed row ids
constexpr int64_t kMaxBlocksAttn = 16384;               // LDS histogram of the dispatch
// query rows b * Hq * n of one call: 2^32 rows of 64 bfloat16 values are already
// 512 GiB, more than one GPU holds; the bound keeps every workspace size and
// index product well inside 64 bits
constexpr int64_t kMaxRowsTotal = int64_t(1) << 32;

ssa_status check_params(const ssa_params* p, ssa::Shape* s) {
  if (p == nullptr) return fail(SSA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->batch < 1) return fail(SSA_ERR_INVALID_ARGUMENT, "batch must be >= 1");
  if (p->n_kv_heads < 1 || p->n_q_heads < 1)
    return fail(SSA_ERR_INVALID_ARGUMENT, "head counts must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(SSA_ERR_INVALID_ARGUMENT, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                p->n_q_heads, p->n_kv_heads);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SSA_ERR_UNSUPPORTED, "head_dim %d not built (64 or 128)", p->head_dim);
  if (p->seq_len < 1 || p->seq_len > kMaxSeq)
    return fail(SSA_ERR_INVALID_ARGUMENT, "seq_len %lld out of [1, 2^30]", (long long)p->seq_len);
  if (p->block_size < 64 || p->block_size > 1024 || p->block_size % 64 != 0)
    return fail(SSA_ERR_INVALID_ARGUMENT, "block_size %d must be a multiple of 64 in [64, 1024]",
                p->block_size);
  if (p->top_k < 0 || p->top_k > 32)
    return fail(SSA_ERR_INVALID_ARGUMENT, "top_k %d out of [0, 32]", p->top_k);
  if (p->window < 1) return fail(SSA_ERR_INVALID_ARGUMENT, "window must be >= 1");
  if (!std::isfinite(p->beta)) return fail(SSA_ERR_INVALID_ARGUMENT, "beta is not finite");
  if (!std::isfinite(p->scale) || !(p->scale > 0.f))
    return fail(SSA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if (p->in_dtype != SSA_F32 && p->in_dtype != SSA_BF16)
    return fail(SSA_ERR_INVALID_ARGUMENT, "in_dtype %d unknown", p->in_dtype);
  if (p->out_dtype != SSA_F32 && p->out_dtype != SSA_BF16)
    return fail(SSA_ERR_INVALID_ARGUMENT, "out_dtype %d unknown", p->out_dtype);
  const int g = p->n_q_heads / p->n_kv_heads;
  if (int64_t(p->batch) * p->n_q_heads > kMaxRowsTotal / p->seq_len)
    return fail(SSA_ERR_UNSUPPORTED, "batch * n_q_heads * seq_len above 2^32 query rows");
  if (p->seq_len * g > kMaxRowsPerHead)
    return fail(SSA_ERR_UNSUPPORTED, "seq_len * (n_q_heads/n_kv_heads) above 2^26");
  s->b = p->batch;
  s->hq = p->n_q_heads;
  s->hkv = p->n_kv_heads;
  s->g = g;
  s->d = p->head_dim;
  s->n = p->seq_len;
  s->B = p->block_size;
  s->k = p->top_k;
  s->W = p->window;
  s->nb = p->seq_len / p->block_size;
  s->beta = p->beta;
  s->scale = p->scale;
  s->in_bf16 = p->in_dtype == SSA_BF16;
  s->out_bf16 = p->out_dtype == SSA_BF16;
  return SSA_OK;
}

#define SSA_NONNULL(ptr)                                                   \
  do {                                                                     \
    if ((ptr) == nullptr) return fail(SSA_ERR_INVALID_ARGUMENT, #ptr " is NULL"); \
  } while (0)

ssa_status check_ws(size_t need, const void* ws, size_t have) {
  if (have < need)
    return fail(SSA_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, needs %zu", have, need);
  if (need > 0 && ws == nullptr) return fail(SSA_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) % ssa::kWsAlign) != 0)
    return fail(SSA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return SSA_OK;
}

}  // namespace

extern "C" {

ssa_status ssa_block_stats(const ssa_params* p, const void* K, float* mu, float* sigma,
                           void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(K);
  SSA_NONNULL(mu);
  SSA_NONNULL(sigma);
  return from_hip(ssa::launch_block_stats(s, K, mu, sigma, nullptr, (hipStream_t)stream),
                  "ssa_block_stats");
}

ssa_status ssa_route_tempered(const ssa_params* p, const void* Q, const void* K, int32_t* idx,
                              float* kth, void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  if (!(p->beta > 0.f)) return fail(SSA_ERR_INVALID_ARGUMENT, "the tempered score needs beta > 0");
  SSA_NONNULL(Q);
  SSA_NONNULL(K);
  if (s.k > 0) SSA_NONNULL(idx);
  if (ssa::tempered_route_tiles(s) >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "too many query rows for one launch");
  if (s.k == 0 && kth == nullptr) return ok();
  return from_hip(ssa::launch_route_tempered(s, Q, K, idx, kth, (hipStream_t)stream),
                  "ssa_route_tempered");
}

ssa_status ssa_route_tiles(const ssa_params* p, const void* Q, const float* mu, const float* sigma,
                           int32_t* idx, float* kth, void* workspace, size_t workspace_bytes,
                           void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(Q);
  if (s.nb > 0) {
    SSA_NONNULL(mu);
    SSA_NONNULL(sigma);
  }
  if (s.k > 0) SSA_NONNULL(idx);
  const int64_t tiles = ssa::tile_count(s);
  if (int64_t(s.b) * s.hq > 65535 || int64_t(s.b) * s.hkv > 65535 ||
      int64_t(s.b) * s.hq * tiles >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "too many (sequence, head) pairs or tiles for one launch");
  st = check_ws(ssa::route_tiles_workspace_bytes(s), workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  if (s.k == 0 && kth == nullptr) return ok();
  return from_hip(ssa::launch_route_tiles(s, Q, mu, sigma, idx, kth, workspace, (hipStream_t)stream),
                  "ssa_route_tiles");
}

ssa_status ssa_tile_attn_fwd(const ssa_params* p, const void* Q, const void* K, const void* V,
                             const int32_t* idx, void* O, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(Q);
  SSA_NONNULL(K);
  SSA_NONNULL(V);
  SSA_NONNULL(O);
  SSA_NONNULL(lse);
  if (s.k > 0) SSA_NONNULL(idx);
  const int64_t list = int64_t(s.k) * (s.B / 64) + (int64_t(s.W) + 254) / 64 + 2;
  if (list > ssa::tile_attn_max_list())
    return fail(SSA_ERR_UNSUPPORTED, "top_k * block_size / 64 + (window + 254) / 64 + 2 = %lld "
                "chunks exceeds %d", (long long)list, ssa::tile_attn_max_list());
  const int64_t subs = (s.B + 255) / 256;
  if (int64_t(s.b) * s.hq * ssa::tile_count(s) * subs >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "too many tiles for one launch");
  st = check_ws(ssa::tile_attn_workspace_bytes(s), workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  return from_hip(ssa::launch_tile_attn(s, Q, K, V, idx, O, lse, workspace, (hipStream_t)stream),
                  "ssa_tile_attn_fwd");
}

ssa_status ssa_sparse_attn_bwd(const ssa_params* p, const void* Q, const void* K, const void* V,
                               const int32_t* idx, const void* O, const float* lse, const void* dO,
                               float* dQ, float* dK, float* dV, void* workspace,
                               size_t workspace_bytes, void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(Q);
  SSA_NONNULL(K);
  SSA_NONNULL(V);
  SSA_NONNULL(O);
  SSA_NONNULL(lse);
  SSA_NONNULL(dO);
  SSA_NONNULL(dQ);
  SSA_NONNULL(dK);
  SSA_NONNULL(dV);
  if (s.k > 0) SSA_NONNULL(idx);
  if (s.k > 0 && s.nb > kMaxBlocksAttn)
    return fail(SSA_ERR_UNSUPPORTED, "%lld blocks per sequence exceed %lld", (long long)s.nb,
                (long long)kMaxBlocksAttn);
  if (s.k > 0 && ssa::attn_entry_slots(s) >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "too many (row, block) selections for 32-bit positions");
  const int64_t chunks = (s.n + 63) / 64;
  if (int64_t(s.b) * s.hkv * chunks >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "too many key chunks for one launch");
  st = check_ws(ssa::attn_bwd_workspace_bytes(s), workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  return from_hip(ssa::launch_sparse_attn_bwd(s, Q, K, V, idx, O, lse, dO, dQ, dK, dV, workspace,
                                              (hipStream_t)stream),
                  "ssa_sparse_attn_bwd");
}

ssa_status ssa_group_stats(const ssa_params* p, const float* mu, const float* sigma,
                           int32_t group_blocks, float* gmu, float* gsigma, float* grl,
                           void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  if (group_blocks < 1 || group_blocks > ssa::hier_max_group())
    return fail(SSA_ERR_INVALID_ARGUMENT, "group_blocks %d out of [1, %d]", group_blocks,
                ssa::hier_max_group());
  if (s.nb == 0) return ok();
  SSA_NONNULL(mu);
  SSA_NONNULL(sigma);
  SSA_NONNULL(gmu);
  SSA_NONNULL(gsigma);
  SSA_NONNULL(grl);
  if (int64_t(s.b) * s.hkv > 65535)
    return fail(SSA_ERR_UNSUPPORTED, "more than 65535 (sequence, KV head) pairs");
  return from_hip(ssa::launch_group_stats(s, mu, sigma, group_blocks, gmu, gsigma, grl,
                                          (hipStream_t)stream),
                  "ssa_group_stats");
}

ssa_status ssa_route_hier(const ssa_params* p, const void* q, const float* mu, const float* sigma,
                          const float* gmu, const float* gsigma, const float* grl,
                          int32_t group_blocks, const int32_t* pos, int32_t* idx,
                          int32_t* evaluated, void* workspace, size_t workspace_bytes,
                          void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  if (!(p->beta >= 0.f))
    return fail(SSA_ERR_INVALID_ARGUMENT, "the group bound needs beta >= 0");
  if (group_blocks < 1 || group_blocks > ssa::hier_max_group())
    return fail(SSA_ERR_INVALID_ARGUMENT, "group_blocks %d out of [1, %d]", group_blocks,
                ssa::hier_max_group());
  if (s.g > ssa::hier_max_rows())
    return fail(SSA_ERR_UNSUPPORTED, "more than %d q-heads per KV head", ssa::hier_max_rows());
  const int64_t G = (s.nb + group_blocks - 1) / group_blocks;
  if (G * s.g > ssa::hier_max_bounds())
    return fail(SSA_ERR_UNSUPPORTED, "groups x q-heads per KV head = %lld exceeds %d",
                (long long)(G * s.g), ssa::hier_max_bounds());
  if (int64_t(s.b) * s.hkv > 65535)
    return fail(SSA_ERR_UNSUPPORTED, "more than 65535 (sequence, KV head) pairs");
  SSA_NONNULL(q);
  SSA_NONNULL(pos);
  if (s.k > 0) SSA_NONNULL(idx);
  if (s.nb > 0) {
    SSA_NONNULL(mu);
    SSA_NONNULL(sigma);
    SSA_NONNULL(gmu);
    SSA_NONNULL(gsigma);
    SSA_NONNULL(grl);
  }
  if (s.k == 0 && evaluated == nullptr) return ok();
  if (s.k > 0) {
    st = check_ws(ssa::route_hier_workspace_bytes(s), workspace, workspace_bytes);
    if (st != SSA_OK) return st;
  }
  return from_hip(ssa::launch_route_hier(s, q, mu, sigma, gmu, gsigma, grl, group_blocks, pos, idx,
                                         evaluated, workspace, (hipStream_t)stream),
                  "ssa_route_hier");
}

namespace {

ssa_status check_hier_prefill(const ssa_params* p, int32_t group_blocks, ssa::Shape* s) {
  ssa_status st = check_params(p, s);
  if (st != SSA_OK) return st;
  if (!(p->beta >= 0.f))
    return fail(SSA_ERR_INVALID_ARGUMENT, "the group bound needs beta >= 0");
  if (group_blocks < 1 || group_blocks > ssa::hier_max_group())
    return fail(SSA_ERR_INVALID_ARGUMENT, "group_blocks %d out of [1, %d]", group_blocks,
                ssa::hier_max_group());
  if (!s->in_bf16)
    return fail(SSA_ERR_UNSUPPORTED, "hierarchical prefill routing is built for bfloat16 inputs");
  const int64_t G = (s->nb + group_blocks - 1) / group_blocks;
  if (G > ssa::hier_prefill_max_groups())
    return fail(SSA_ERR_UNSUPPORTED, "%lld groups per sequence exceed %d", (long long)G,
                ssa::hier_prefill_max_groups());
  if (int64_t(s->b) * s->hkv * ssa::route_tile_count(*s) >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "too many 512-row tiles for one launch");
  if (int64_t(s->b) * s->hkv > 65535)
    return fail(SSA_ERR_UNSUPPORTED, "more than 65535 (sequence, KV head) pairs");
  return SSA_OK;
}

}  // namespace

ssa_status ssa_route_hier_prefill_workspace_size(const ssa_params* p, int32_t group_blocks,
                                                 size_t* bytes) {
  ssa::Shape s;
  ssa_status st = check_hier_prefill(p, group_blocks, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(bytes);
  *bytes = ssa::route_hier_prefill_workspace_bytes(s, group_blocks);
  return ok();
}

ssa_status ssa_route_hier_prefill(const ssa_params* p, const void* Q, const float* mu,
                                  const float* sigma, const float* gmu, const float* gsigma,
                                  const float* grl, int32_t group_blocks, int32_t* idx,
                                  int32_t* evaluated, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  ssa::Shape s;
  ssa_status st = check_hier_prefill(p, group_blocks, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(Q);
  if (s.k > 0) SSA_NONNULL(idx);
  if (s.nb > 0) {
    SSA_NONNULL(mu);
    SSA_NONNULL(sigma);
    SSA_NONNULL(gmu);
    SSA_NONNULL(gsigma);
    SSA_NONNULL(grl);
  }
  if (s.k == 0 && evaluated == nullptr) return ok();
  st = check_ws(ssa::route_hier_prefill_workspace_bytes(s, group_blocks), workspace,
                workspace_bytes);
  if (st != SSA_OK) return st;
  return from_hip(ssa::launch_route_hier_prefill(s, Q, mu, sigma, gmu, gsigma, grl, group_blocks,
                                                 idx, evaluated, workspace, (hipStream_t)stream),
                  "ssa_route_hier_prefill");
}

ssa_status ssa_workspace_size(const ssa_params* p, int32_t op, size_t* bytes) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(bytes);
  switch (op) {
    case SSA_OP_ROUTE: *bytes = ssa::route_workspace_bytes(s); break;
    case SSA_OP_ATTN: *bytes = ssa::attn_workspace_bytes(s); break;
    case SSA_OP_DECODE: *bytes = ssa::decode_workspace_bytes(s); break;
    case SSA_OP_ROUTE_TILES: *bytes = ssa::route_tiles_workspace_bytes(s); break;
    case SSA_OP_TILE_ATTN: *bytes = ssa::tile_attn_workspace_bytes(s); break;
    case SSA_OP_ATTN_BWD: *bytes = ssa::attn_bwd_workspace_bytes(s); break;
    case SSA_OP_ROUTE_HIER: *bytes = ssa::route_hier_workspace_bytes(s); break;
    default: return fail(SSA_ERR_INVALID_ARGUMENT, "unknown op %d", op);
  }
  return ok();
}

ssa_status ssa_route_topk(const ssa_params* p, const void* Q, const float* mu, const float* sigma,
                          int32_t* idx, float* kth, void* workspace, size_t workspace_bytes,
                          void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(Q);
  if (s.nb > 0) {
    SSA_NONNULL(mu);
    SSA_NONNULL(sigma);
  }
  if (s.k > 0) SSA_NONNULL(idx);
  st = check_ws(ssa::route_workspace_bytes(s), workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  if (s.k == 0 && kth == nullptr) return ok();
  return from_hip(ssa::launch_route_topk(s, Q, mu, sigma, idx, kth, workspace, (hipStream_t)stream),
                  "ssa_route_topk");
}

ssa_status ssa_sparse_attn_fwd(const ssa_params* p, const void* Q, const void* K, const void* V,
                               const int32_t* idx, void* O, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(Q);
  SSA_NONNULL(K);
  SSA_NONNULL(V);
  SSA_NONNULL(O);
  SSA_NONNULL(lse);
  if (s.k > 0) SSA_NONNULL(idx);
  if (s.k > 0 && s.nb > kMaxBlocksAttn)
    return fail(SSA_ERR_UNSUPPORTED, "more than %lld blocks per sequence", (long long)kMaxBlocksAttn);
  if (int64_t(s.b) * s.hq * s.n * s.k >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "batch * n_q_heads * seq_len * top_k above 2^31");
  if (s.k > 0 && ssa::attn_entry_slots(s) >= (int64_t(1) << 31))
    return fail(SSA_ERR_UNSUPPORTED, "routed (row, block) pairs plus per-block task padding above 2^31");
  st = check_ws(ssa::attn_workspace_bytes(s), workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  return from_hip(
      ssa::launch_sparse_attn(s, Q, K, V, idx, O, lse, workspace, (hipStream_t)stream),
      "ssa_sparse_attn_fwd");
}

ssa_status ssa_decode_step(const ssa_params* p, const void* q, const void* k_new,
                           const void* v_new, void* K_cache, void* V_cache, int32_t* cache_len,
                           float* mu, float* sigma, int32_t* idx, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(q);
  SSA_NONNULL(k_new);
  SSA_NONNULL(v_new);
  SSA_NONNULL(K_cache);
  SSA_NONNULL(V_cache);
  SSA_NONNULL(cache_len);
  SSA_NONNULL(o);
  SSA_NONNULL(lse);
  if (s.nb > 0) {
    SSA_NONNULL(mu);
    SSA_NONNULL(sigma);
  }
  st = check_ws(ssa::decode_workspace_bytes(s), workspace, workspace_bytes);
  if (st != SSA_OK) return st;
  return from_hip(ssa::launch_decode_step(s, q, k_new, v_new, K_cache, V_cache, cache_len, mu,
                                          sigma, idx, o, lse, workspace, (hipStream_t)stream),
                  "ssa_decode_step");
}

ssa_status ssa_decode_step_noalloc(const ssa_params* p, const void* q, const void* k_new,
                                   const void* v_new, void* K_cache, void* V_cache,
                                   int32_t* cache_len, float* mu, float* sigma, int32_t* idx,
                                   void* o, float* lse, void* stream) {
  ssa::Shape s;
  ssa_status st = check_params(p, &s);
  if (st != SSA_OK) return st;
  SSA_NONNULL(q);
  SSA_NONNULL(k_new);
  SSA_NONNULL(v_new);
  SSA_NONNULL(K_cache);
  SSA_NONNULL(V_cache);
  SSA_NONNULL(cache_len);
  SSA_NONNULL(o);
  SSA_NONNULL(lse);
  if (s.nb > 0) {
    SSA_NONNULL(mu);
    SSA_NONNULL(sigma);
  }
  const size_t need = ssa::decode_workspace_bytes(s);
  if (need > ssa::kDecodeScratchBytes)
    return fail(SSA_ERR_UNSUPPORTED,
                "this decode step needs %zu bytes of scratch; the allocation-free entry point "
                "holds %zu (use ssa_decode_step with a workspace)",
                need, ssa::kDecodeScratchBytes);
  void* ws = nullptr;
  st = from_hip(ssa::decode_scratch(&ws), "ssa_decode_step_noalloc: scratch address");
  if (st != SSA_OK) return st;
  return from_hip(ssa::launch_decode_step(s, q, k_new, v_new, K_cache, V_cache, cache_len, mu,
                                          sigma, idx, o, lse, ws, (hipStream_t)stream),
                  "ssa_decode_step_noalloc");
}

const char* ssa_status_string(ssa_status s) {
  switch (s) {
    case SSA_OK: return "SSA_OK";
    case SSA_ERR_INVALID_ARGUMENT: return "SSA_ERR_INVALID_ARGUMENT";
    case SSA_ERR_UNSUPPORTED: return "SSA_ERR_UNSUPPORTED";
    case SSA_ERR_WORKSPACE_TOO_SMALL: return "SSA_ERR_WORKSPACE_TOO_SMALL";
    case SSA_ERR_HIP: return "SSA_ERR_HIP";
  }
  return "SSA_ERR_UNKNOWN";
}

const char* ssa_last_error(void) { return g_err; }

int32_t ssa_version(void) { return 100; }

}  // extern "C"
