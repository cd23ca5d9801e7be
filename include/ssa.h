/*
 * ssa.h -- C ABI of the MI355X (gfx950) hot path of Subquadratic Sparse
 * Attention (SSA), content-routed block statistics.
 *
 * The method (write-up "Subquadratic Sparse Attention (SSA)",
 * git.hmmc.top/jonsmirl/ssa, introduction paragraph, steps i-iii, and section
 * "The idea in one screen"): for each query, route to a small set of key
 * blocks using only per-block summary statistics, scored by the
 * second-cumulant score r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q; keep the
 * top-k blocks under causal masking; add a local window; compute exact
 * softmax attention over the selected keys.
 *
 * Conventions shared by every call
 *  - Every tensor pointer is a DEVICE pointer owned by the caller, contiguous
 *    row-major in the layout stated at each call, aligned to 16 bytes.  The
 *    library never allocates, frees or retains device memory; scratch space
 *    is the caller's workspace.  It keeps no global mutable data, so calls
 *    on different streams may run concurrently -- except
 *    ssa_decode_step_noalloc, whose scratch is a device array inside the
 *    library (see there).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; results are ready when the stream is.
 *    ssa_sparse_attn_fwd runs part of its work (the K/V chunk images) on a
 *    second stream of the device, created on the first call and kept for the
 *    process, that waits for the caller's stream and that the caller's stream
 *    waits for again before the dependent work: ordering against the
 *    caller's stream is as if everything ran on it.  Under stream capture
 *    everything runs on the caller's stream.
 *  - Validation is synchronous and on the host, before anything is enqueued:
 *    on an error nothing is launched and a status other than SSA_OK is
 *    returned; ssa_last_error() then holds a message (per thread).  A launch
 *    failure reported by the runtime returns SSA_ERR_HIP.  Faults inside a
 *    kernel surface at the caller's next synchronisation.  No C++ exception
 *    crosses this interface.
 *  - Row r of a tensor [b, H, n, x] is (sequence, head, position).  q-head h
 *    reads KV head h / (n_q_heads / n_kv_heads) (contiguous groups).
 *  - Tokens: b = batch, Hq / Hkv = query / KV heads, n = seq_len, d = head_dim,
 *    B = block_size, nb = n / B complete blocks, k = top_k, W = window.
 */
#ifndef SSA_MI355X_SSA_H
#define SSA_MI355X_SSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssa_status {
  SSA_OK = 0,
  SSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, out-of-range size or parameter */
  SSA_ERR_UNSUPPORTED = 2,        /* valid in principle, not built (e.g. d not in {64,128}) */
  SSA_ERR_WORKSPACE_TOO_SMALL = 3,
  SSA_ERR_HIP = 4                 /* the HIP runtime reported an error */
} ssa_status;

typedef enum ssa_dtype { SSA_F32 = 0, SSA_BF16 = 1 } ssa_dtype;

typedef enum ssa_op {
  SSA_OP_ROUTE = 1,   /* workspace of ssa_route_topk */
  SSA_OP_ATTN = 2,    /* workspace of ssa_sparse_attn_fwd */
  SSA_OP_DECODE = 3,  /* workspace of ssa_decode_step */
  SSA_OP_ROUTE_TILES = 4,  /* workspace of ssa_route_tiles */
  SSA_OP_TILE_ATTN = 5,    /* workspace of ssa_tile_attn_fwd */
  SSA_OP_ATTN_BWD = 6,     /* workspace of ssa_sparse_attn_bwd */
  SSA_OP_ROUTE_HIER = 7    /* workspace of ssa_route_hier (any group_blocks) */
} ssa_op;

/* Shapes and method parameters.  Limits checked by every call:
 *   batch >= 1; n_kv_heads >= 1; n_q_heads a positive multiple of n_kv_heads;
 *   head_dim in {64, 128};
 *   seq_len in [1, 2^30] (prefill: n; decode: the cache capacity in tokens);
 *   seq_len * (n_q_heads / n_kv_heads) at most 2^26 and
 *   batch * n_q_heads * seq_len at most 2^32 (SSA_ERR_UNSUPPORTED otherwise);
 *   block_size a multiple of 64 in [64, 1024];
 *   top_k in [0, 32];  window >= 1;
 *   beta finite; scale finite and > 0;
 *   in_dtype in {SSA_F32, SSA_BF16} (Q, K, V and caches);
 *   out_dtype in {SSA_F32, SSA_BF16} (O). */
typedef struct ssa_params {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int64_t seq_len;
  int32_t block_size;
  int32_t top_k;
  int32_t window;
  float beta;    /* routing inverse temperature on raw q (the write-up tunes ~2) */
  float scale;   /* softmax scale on raw logits, normally the float32 of 1/sqrt(d) */
  int32_t in_dtype;
  int32_t out_dtype;
} ssa_params;

/* Per-block statistics (write-up, "The idea in one screen": the block mean
 * mu_c and covariance Sigma_c, whose quadratic form is the variance of the
 * logit across the block).  For every complete block c < nb of every
 * (sequence, KV head):
 *   mu_c    = (1/B) sum_j k_j
 *   Sigma_c = (1/B) sum_j (k_j - mu_c)(k_j - mu_c)^T   (population covariance)
 * accumulated in float32.
 *   K     [b, Hkv, n, d]      in_dtype
 *   mu    [b, Hkv, nb, d]     float32, written
 *   sigma [b, Hkv, nb, d, d]  float32, written (full symmetric matrix)
 * A trailing partial block is ignored. */
ssa_status ssa_block_stats(const ssa_params* p, const void* K, float* mu, float* sigma,
                           void* stream);

/* Bytes of workspace an operation needs for these parameters (0 is valid). */
ssa_status ssa_workspace_size(const ssa_params* p, int32_t op, size_t* bytes);

/* Routing and top-k (write-up, introduction step i, and the routing score of
 * "The idea in one screen").  For every query row (b, h, t) the routable
 * blocks are the complete blocks c with (c+1)B-1 <= t; each gets
 *   r_c = <q, mu_c> + (beta/2) q^T Sigma_c q      (raw q, KV head of h)
 * and the min(k, #routable) highest scores are kept, ties to the lower c.
 *   Q          [b, Hq, n, d]   in_dtype
 *   mu, sigma  as written by ssa_block_stats
 *   idx        [b, Hq, n, k]   int32, written: selected block indices in
 *                              ascending order, padded with -1
 *   kth        [b, Hq, n, 2]   float32, written if not NULL: the k-th and
 *                              (k+1)-th largest scores (-inf where absent)
 *   workspace  >= ssa_workspace_size(p, SSA_OP_ROUTE) bytes of device memory
 * The scores are evaluated on the float16 MFMA with float32 accumulation:
 * Q scaled by one power of two per (sequence, KV head) (exact for bfloat16
 * values), Sigma scaled per block and split into a high and a low float16
 * part (float32 MFMA for float32 inputs), so a selection can differ from an
 * exact one only where two scores are within about 1e-6 relative of each
 * other. */
ssa_status ssa_route_topk(const ssa_params* p, const void* Q, const float* mu,
                          const float* sigma, int32_t* idx, float* kth, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Exact tempered routing and top-k (write-up, "The idea in one screen": the
 * temperature family that links the centroid score, the second-cumulant
 * score and the exact block maximum).  For every query row (b, h, t) and every
 * routable block c ((c+1)B-1 <= t):
 *   T_c = (1/beta) ln( (1/B) sum_{j in block c} exp(beta q.k_j) )   (raw q)
 * whose expansion to second order in beta is the ssa_route_topk score; then
 * the same top-k rule (min(k, #routable) highest, ties to the lower c).
 *   Q    [b, Hq, n, d]   in_dtype
 *   K    [b, Hkv, n, d]  in_dtype (the keys themselves: every key of every
 *                        routable block is read, so the cost is that of
 *                        dense causal Q K^T)
 *   idx  [b, Hq, n, k]   int32, written as by ssa_route_topk
 *   kth  [b, Hq, n, 2]   float32, written if not NULL: k-th and (k+1)-th
 *                        largest T (-inf where absent)
 * beta must be > 0 (SSA_ERR_INVALID_ARGUMENT otherwise).  No workspace.
 * Limits (SSA_ERR_UNSUPPORTED otherwise): b * Hkv * ceil(n Hq/Hkv / 256)
 * below 2^31.
 * Arithmetic: q.k_j on MFMA (bf16 products exact, float32 accumulation;
 * float32 MFMA for float32 inputs), the log-sum-exp in float32 in base 2 with
 * the block's maximum factored out. */
ssa_status ssa_route_tempered(const ssa_params* p, const void* Q, const void* K, int32_t* idx,
                              float* kth, void* stream);

/* Query-tile-shared routing (write-up: the fused kernel routes per query
 * block -- its compute-floor notes name an (n/b)^2 block-score GEMM and an
 * argsort block-mask build).  Tile j of each (sequence, q-head) holds the
 * positions [jB, (j+1)B) (the last tile may be partial: ceil(n/B) tiles).
 * It selects, for all its queries, the min(k, #routable) blocks among those
 * complete before it (c < j) with the highest summed routing score
 *   R_c = sum_{t in tile} r_c(q_t) = s.mu_c + (beta/2) <Sigma_c, M>,
 *   s = sum_t q_t,  M = sum_t q_t q_t^T         (raw q, KV head of the head),
 * ties to the lower c.
 *   Q          [b, Hq, n, d]                in_dtype
 *   mu, sigma  as written by ssa_block_stats
 *   idx        [b, Hq, ceil(n/B), k]       int32, written: ascending, -1 padded
 *   kth        [b, Hq, ceil(n/B), 2]       float32, written if not NULL: the
 *                                          k-th and (k+1)-th largest R (-inf
 *                                          where absent)
 *   workspace  >= ssa_workspace_size(p, SSA_OP_ROUTE_TILES) bytes
 * Arithmetic: M and s on MFMA (bf16 products exact, float32 accumulation),
 * R on float32 MFMA.  Limits (SSA_ERR_UNSUPPORTED otherwise): b * Hq and
 * b * Hkv at most 65535, b * Hq * ceil(n/B) below 2^31. */
ssa_status ssa_route_tiles(const ssa_params* p, const void* Q, const float* mu, const float* sigma,
                           int32_t* idx, float* kth, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Attention over tile selections (write-up, introduction steps ii-iii, with
 * the selection of ssa_route_tiles).  For every query row (b, h, t) of tile
 * j = t / B:
 *   S(t) = union of the keys of the blocks in idx(b, h, j) (entries < 0 are
 *          ignored) and the window [max(0, t-W+1), t], each key once;
 *   O = sum_j softmax(scale * q.k_j) v_j over S(t), LSE = ln sum exp(...).
 *   Q, K, V, O, lse  as for ssa_sparse_attn_fwd
 *   idx        [b, Hq, ceil(n/B), k] int32 as written by ssa_route_tiles:
 *              every entry -1 or a block < j, distinct (other contents are
 *              undefined behaviour)
 *   workspace  >= ssa_workspace_size(p, SSA_OP_TILE_ATTN) bytes
 * Limits (SSA_ERR_UNSUPPORTED otherwise): k * B/64 + (W + 254)/64 + 2 at most
 * 1024 chunks per workgroup; b * Hq * ceil(n/B) * ceil(B/256) below 2^31.
 * Arithmetic: as ssa_sparse_attn_fwd. */
ssa_status ssa_tile_attn_fwd(const ssa_params* p, const void* Q, const void* K, const void* V,
                             const int32_t* idx, void* O, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Sparse attention forward (write-up, introduction steps ii-iii).  For every
 * query row (b, h, t):
 *   S(t) = union of the keys of the blocks in idx(b,h,t) (entries < 0 are
 *          ignored) and the window [max(0, t-W+1), t], each key once;
 *   s_j  = scale * q.k_j for j in S(t);
 *   O    = sum_j softmax(s)_j v_j,   LSE = ln sum_j exp(s_j).
 *   Q    [b, Hq, n, d] in_dtype;  K, V [b, Hkv, n, d] in_dtype
 *   idx  [b, Hq, n, k] int32 as written by ssa_route_topk: every entry is -1
 *        or a complete block routable for t, entries distinct and ascending
 *        (other contents are undefined behaviour)
 *   O    [b, Hq, n, d] out_dtype, written;  lse [b, Hq, n] float32, written
 *   workspace >= ssa_workspace_size(p, SSA_OP_ATTN) bytes
 * Limits (SSA_ERR_UNSUPPORTED otherwise): at most 16384 blocks per sequence
 * when top_k > 0; b * Hq * n * k below 2^31, and so is that count plus 256
 * slots of padding per (sequence, KV head, block).
 * Arithmetic: MFMA products with float32 accumulation and an online softmax
 * in float32. */
ssa_status ssa_sparse_attn_fwd(const ssa_params* p, const void* Q, const void* K,
                               const void* V, const int32_t* idx, void* O, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Backward of the sparse attention over fixed selections (training through
 * the layer: the write-up's module list trains SSA models and its "Selected
 * results" adapt a dense model swapped to SSA; the selection is discrete and
 * is held fixed).  With p_j = exp(scale q.k_j - LSE) over S(t) (the forward's
 * key set and LSE), D = dO . O, dP_j = dO . v_j, dS_j = p_j (dP_j - D):
 *   dQ_t = scale sum_j dS_j k_j;  dK_j = scale sum_t dS_j q_t;  dV_j = sum_t p_j dO_t
 * (dK, dV summed over every row of the KV head's group that attends to j).
 *   Q, K, V, idx  as for ssa_sparse_attn_fwd
 *   O     [b, Hq, n, d]  out_dtype, lse [b, Hq, n] float32: that call's outputs
 *   dO    [b, Hq, n, d]  in_dtype, the upstream gradient
 *   dQ    [b, Hq, n, d], dK, dV [b, Hkv, n, d]  float32, written (not added to)
 *   workspace >= ssa_workspace_size(p, SSA_OP_ATTN_BWD) bytes
 * Limits: those of ssa_sparse_attn_fwd; b * Hkv * ceil(n/64) below 2^31.
 * Arithmetic: q.k and dO.v on MFMA as in the forward (bf16 products exact);
 * K^T, Q^T, dO^T, p and dS enter their products as float16 after scaling by
 * an exact power of two (float32 MFMA for float32 inputs); float32
 * accumulation.  dQ is bitwise repeatable; dK and dV add a block's rows in
 * the dispatch's order, which follows atomic reservations, so repeated calls
 * agree to float32 rounding, not bit for bit. */
ssa_status ssa_sparse_attn_bwd(const ssa_params* p, const void* Q, const void* K, const void* V,
                               const int32_t* idx, const void* O, const float* lse, const void* dO,
                               float* dQ, float* dK, float* dV, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Exact hierarchical routing, decode queries (write-up: the module list pairs
 * the flat router with branch-and-bound exact selection under an admissible
 * bound and a tree router with a recursive radius; "Selected results" report
 * lossless branch-and-bound selection costs).  Groups of m = group_blocks
 * consecutive blocks (G = ceil(nb / m) per (sequence, KV head), nb the
 * complete block slots of seq_len) are summarised by ssa_group_stats:
 *   gmu    [b, Hkv, G, d]     mean of the members' mu_c
 *   gsigma [b, Hkv, G, d, d]  mean of the members' Sigma_c (S_G)
 *   grl    [b, Hkv, G, 2]     R_G = max ||mu_c - mu_G||, lam_G = max (tr (Sigma_c - S_G)^4)^(1/4)
 * (all float32, written; one-time work, recomputed when blocks change).  For
 * beta >= 0 every member's score is at most
 *   UB_G(q) = q.mu_G + ||q|| R_G + (beta/2)(q^T S_G q + lam_G ||q||^2).
 * ssa_route_hier selects, for every (sequence b, q-head h) with query q
 * [b, Hq, d] at position pos[b] (int32, device), the min(k, #routable) blocks
 * c < nb with (c+1)B-1 <= pos[b] of highest r_c = <q, mu_c> + (beta/2) q^T
 * Sigma_c q, ties to the lower c -- the flat top-k, exactly -- visiting groups
 * by decreasing bound (largest over the KV head's q-heads) and skipping a group
 * when its bound is below every row's running k-th score (with a relative
 * margin of 1e-4 over float32 rounding).
 *   idx        [b, Hq, k] int32, written: ascending, -1 padded
 *   evaluated  [b, Hkv] int32, written if not NULL: blocks scored exactly
 *   workspace  >= ssa_workspace_size(p, SSA_OP_ROUTE_HIER) bytes (k > 0)
 * Scores in float32 from Sigma_c's upper triangle (Sigma_c symmetric).
 * gmu/gsigma/grl must summarise the current mu/sigma with the same
 * group_blocks, or the selection may be wrong.  Limits: group_blocks in
 * [1, 64] and beta >= 0 (SSA_ERR_INVALID_ARGUMENT); at most 16 q-heads per KV
 * head, G * (Hq / Hkv) <= 8192 and b * Hkv <= 65535 (SSA_ERR_UNSUPPORTED). */
ssa_status ssa_group_stats(const ssa_params* p, const float* mu, const float* sigma,
                           int32_t group_blocks, float* gmu, float* gsigma, float* grl,
                           void* stream);
ssa_status ssa_route_hier(const ssa_params* p, const void* q, const float* mu, const float* sigma,
                          const float* gmu, const float* gsigma, const float* grl,
                          int32_t group_blocks, const int32_t* pos, int32_t* idx,
                          int32_t* evaluated, void* workspace, size_t workspace_bytes,
                          void* stream);

/* Exact hierarchical routing of prefill query rows (write-up, module table:
 * branch-and-bound exact selection under an admissible bound and a tree
 * router; opening paragraph: near-linear cost with a hierarchical router).
 * Returns the selection ssa_route_topk defines (ties to the lower block),
 * scoring only the groups of group_blocks consecutive blocks whose bound
 *   UB_G(q) = r_G(q) + ||q|| R_G + (beta/2) lam_G ||q||^2
 * (r_G: the routing score of the group's mean centroid and mean covariance;
 * R_G, lam_G: radius and covariance slack, all from ssa_group_stats) reaches
 * some row's running k-th score.  The rows rho = t (Hq/Hkv) + j of one
 * (sequence, KV head) (rho < n Hq/Hkv) are listed chunk by chunk (8192
 * consecutive rows each), within a chunk by the group of their largest bound
 * (ties: lower group; then row order), and taken in tiles of 512 consecutive
 * list entries; a tile visits its groups in decreasing order
 * of their largest bound over its rows and scores a group's blocks against
 * all its rows unless, for every row, the group's bound (with a relative
 * margin of 1e-4 over float32 rounding) is strictly below the row's running
 * k-th score.
 *   Q          [b, Hq, n, d] bfloat16
 *   mu, sigma  as ssa_block_stats writes them for K [b, Hkv, n, d]
 *   gmu, gsigma, grl  ssa_group_stats of mu/sigma with the same group_blocks
 *   idx        [b, Hq, n, k] int32, written as ssa_route_topk writes it
 *   evaluated  [b, Hkv, ceil(n (Hq/Hkv) / 512)] int32, written if not NULL:
 *              blocks each listed tile scored (against all of its rows)
 *   workspace  >= ssa_route_hier_prefill_workspace_size(p, group_blocks, .)
 *              bytes, 256-byte aligned (it grows with the number of groups)
 * Limits: group_blocks in [1, 64] and beta >= 0 (SSA_ERR_INVALID_ARGUMENT);
 * bfloat16 inputs, at most 4096 groups per sequence, b * Hkv <= 65535 and
 * b * Hkv * ceil(n (Hq/Hkv) / 512) < 2^31 (SSA_ERR_UNSUPPORTED). */
ssa_status ssa_route_hier_prefill_workspace_size(const ssa_params* p, int32_t group_blocks,
                                                 size_t* bytes);
ssa_status ssa_route_hier_prefill(const ssa_params* p, const void* Q, const float* mu,
                                  const float* sigma, const float* gmu, const float* gsigma,
                                  const float* grl, int32_t group_blocks, int32_t* idx,
                                  int32_t* evaluated, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* One decode step per sequence (write-up, module table: the decode path routes
 * and attends one new query per step against the cache).  With
 * L = cache_len[b] tokens already cached, for every sequence b:
 *   1. writes k_new, v_new at position L of the caches;
 *   2. if (L+1) % B == 0, writes mu/sigma of the block (L+1)/B - 1 just completed;
 *   3. for every q-head, routes over the complete blocks c < (L+1)/B, keeps
 *      the top k, and attends over the selected blocks and the window
 *      [max(0, L-W+1), L] exactly as ssa_route_topk + ssa_sparse_attn_fwd
 *      would for query position t = L;
 *   4. increments cache_len[b].
 * p->seq_len is the cache capacity C (tokens); the caller guarantees
 * cache_len[b] < C (not checked on the device).
 *   q        [b, Hq, d] in_dtype;  k_new, v_new [b, Hkv, d] in_dtype
 *   K_cache, V_cache [b, Hkv, C, d] in_dtype (read and written)
 *   cache_len [b] int32 on the device (read and incremented)
 *   mu [b, Hkv, C/B, d], sigma [b, Hkv, C/B, d, d] float32 (read, and written
 *      for a completed block); entries of complete blocks must hold the
 *      statistics ssa_block_stats would write
 *   idx [b, Hq, k] int32, written if not NULL (as ssa_route_topk)
 *   o [b, Hq, d] out_dtype, written;  lse [b, Hq] float32, written
 *   workspace >= ssa_workspace_size(p, SSA_OP_DECODE) bytes
 * Routing here reads sigma in float32 on the vector units. */
ssa_status ssa_decode_step(const ssa_params* p, const void* q, const void* k_new,
                           const void* v_new, void* K_cache, void* V_cache, int32_t* cache_len,
                           float* mu, float* sigma, int32_t* idx, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device scratch that ssa_decode_step_noalloc holds per GPU. */
#define SSA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* The decode step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and kernels as ssa_decode_step, without the
 * workspace: its scratch lives in a device array inside the library, one per
 * GPU, held until the process ends (SSA_DECODE_NOALLOC_SCRATCH_BYTES, enough
 * for e.g. 32 sequences x 32 q-heads x 512 blocks with k = 16 at d = 128).
 * Calls whose ssa_workspace_size(p, SSA_OP_DECODE) exceeds it return
 * SSA_ERR_UNSUPPORTED before anything is enqueued.  The call allocates and
 * frees nothing; the first call on a device looks up the array's address
 * there.  The stream must belong to the current device.  Every call on a GPU
 * shares that GPU's array, so calls that overlap in time on one GPU (other
 * streams or threads) race; calls in order on one stream do not.  No state
 * carries over between calls. */
ssa_status ssa_decode_step_noalloc(const ssa_params* p, const void* q, const void* k_new,
                                   const void* v_new, void* K_cache, void* V_cache,
                                   int32_t* cache_len, float* mu, float* sigma, int32_t* idx,
                                   void* o, float* lse, void* stream);

/* Static text for a status code. */
const char* ssa_status_string(ssa_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* ssa_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t ssa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSA_MI355X_SSA_H */
