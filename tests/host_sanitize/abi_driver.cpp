// Host-only driver for the C ABI's validation and workspace arithmetic, built
// with AddressSanitizer and UndefinedBehaviorSanitizer on host code (the
// library's device code is not built into it, and no call here reaches a
// launch).  Exit status 0 when every expectation holds; the sanitizers abort
// on the first report.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "ssa.h"

static int g_fail = 0;

#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      std::fprintf(stderr, "%s:%d: expectation failed: %s (%s)\n", __FILE__, \
                   __LINE__, #cond, ssa_last_error());                        \
      ++g_fail;                                                               \
    }                                                                         \
  } while (0)

static ssa_params base() {
  ssa_params p{};
  p.batch = 1;
  p.n_q_heads = 8;
  p.n_kv_heads = 2;
  p.head_dim = 128;
  p.seq_len = 4096;
  p.block_size = 128;
  p.top_k = 8;
  p.window = 128;
  p.beta = 2.f;
  p.scale = 0.088f;
  p.in_dtype = SSA_BF16;
  p.out_dtype = SSA_BF16;
  return p;
}

// every operation's workspace query, for one parameter set
static void sizes(const ssa_params& p, std::vector<size_t>* out, std::vector<int>* st) {
  for (int op = 1; op <= 7; ++op) {
    size_t b = 0;
    st->push_back(ssa_workspace_size(&p, op, &b));
    out->push_back(b);
  }
}

int main() {
  // parameters out of range, field by field
  {
    ssa_params p;
    size_t b;
    auto bad = [&](ssa_status want) { EXPECT(ssa_workspace_size(&p, 1, &b) == want); };
    p = base(); p.batch = 0; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.batch = INT_MIN; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.n_q_heads = 0; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.n_kv_heads = -3; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.n_q_heads = 7; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.head_dim = 96; bad(SSA_ERR_UNSUPPORTED);
    p = base(); p.seq_len = 0; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.seq_len = INT64_MAX; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.seq_len = INT64_MIN; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.block_size = 96; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.block_size = 2048; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.top_k = 33; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.top_k = -1; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.window = 0; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.beta = 1.f / 0.f; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.scale = 0.f; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.in_dtype = 7; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.out_dtype = -1; bad(SSA_ERR_INVALID_ARGUMENT);
    p = base(); p.n_q_heads = 64; p.n_kv_heads = 1; p.seq_len = (int64_t(1) << 26); bad(SSA_ERR_UNSUPPORTED);
    EXPECT(ssa_workspace_size(nullptr, 1, &b) == SSA_ERR_INVALID_ARGUMENT);
    p = base();
    EXPECT(ssa_workspace_size(&p, 1, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_workspace_size(&p, 0, &b) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_workspace_size(&p, 99, &b) == SSA_ERR_INVALID_ARGUMENT);
  }
  // workspace sizes over a grid of shapes: no overflow (the sanitizers watch
  // the arithmetic), and a call that succeeds reports a size that does not
  // shrink when the batch grows
  {
    const int batches[] = {1, 3, 64, 1 << 16, 1 << 24, INT_MAX};
    const int64_t lens[] = {1, 63, 64, 1000, 4096, 131072, int64_t(1) << 22, int64_t(1) << 26};
    const int blocks[] = {64, 256, 1024};
    const int ks[] = {0, 1, 16, 32};
    const int heads[][2] = {{1, 1}, {8, 8}, {32, 8}, {64, 1}};
    int ok_calls = 0;
    for (int d : {64, 128})
      for (auto& hh : heads)
        for (int B : blocks)
          for (int k : ks)
            for (int64_t n : lens) {
              std::vector<size_t> prev;
              std::vector<int> prev_st;
              for (int bt : batches) {
                ssa_params p = base();
                p.batch = bt;
                p.n_q_heads = hh[0];
                p.n_kv_heads = hh[1];
                p.head_dim = d;
                p.block_size = B;
                p.top_k = k;
                p.seq_len = n;
                p.window = B;
                std::vector<size_t> sz;
                std::vector<int> st;
                sizes(p, &sz, &st);
                for (size_t i = 0; i < sz.size(); ++i) {
                  if (st[i] == SSA_OK) ++ok_calls;
                  if (!prev.empty() && st[i] == SSA_OK && prev_st[i] == SSA_OK && sz[i] < prev[i]) {
                    std::fprintf(stderr, "op %zu: workspace shrinks from %zu to %zu at batch %d "
                                 "(n %lld, B %d, k %d, heads %d/%d, d %d)\n", i + 1, prev[i],
                                 sz[i], bt, (long long)n, B, k, hh[0], hh[1], d);
                    ++g_fail;
                  }
                }
                prev = sz;
                prev_st = st;
              }
            }
    EXPECT(ok_calls > 0);
  }
  // pointers and workspaces checked before anything is enqueued
  {
    ssa_params p = base();
    char dummy_storage[1024];
    void* D = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(dummy_storage) + 255) & ~uintptr_t(255));
    float* F = static_cast<float*>(D);
    int32_t* I = static_cast<int32_t*>(D);
    EXPECT(ssa_block_stats(&p, nullptr, F, F, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_block_stats(&p, D, nullptr, F, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_block_stats(nullptr, D, F, F, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    size_t need = 0;
    EXPECT(ssa_workspace_size(&p, 1, &need) == SSA_OK && need > 0);
    EXPECT(ssa_route_topk(&p, D, F, F, I, nullptr, D, need - 1, nullptr) == SSA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ssa_route_topk(&p, D, F, F, I, nullptr, nullptr, need, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_route_topk(&p, D, F, F, I, nullptr, static_cast<char*>(D) + 4, need, nullptr) ==
           SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_route_topk(&p, nullptr, F, F, I, nullptr, D, need, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_route_topk(&p, D, F, F, nullptr, nullptr, D, need, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_workspace_size(&p, 2, &need) == SSA_OK);
    EXPECT(ssa_sparse_attn_fwd(&p, D, D, D, I, D, F, D, need - 1, nullptr) == SSA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ssa_sparse_attn_fwd(&p, D, D, D, nullptr, D, F, D, need, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_sparse_attn_fwd(&p, D, D, D, I, D, nullptr, D, need, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_workspace_size(&p, 3, &need) == SSA_OK);
    EXPECT(ssa_decode_step(&p, D, D, D, D, D, I, F, F, I, D, F, D, need - 1, nullptr) ==
           SSA_ERR_WORKSPACE_TOO_SMALL);
    EXPECT(ssa_decode_step(&p, D, D, D, D, D, nullptr, F, F, I, D, F, D, need, nullptr) ==
           SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_decode_step_noalloc(&p, D, D, D, D, D, nullptr, F, F, I, D, F, nullptr) ==
           SSA_ERR_INVALID_ARGUMENT);
    ssa_params big = base();
    big.batch = 1 << 20;
    big.seq_len = int64_t(1) << 22;
    EXPECT(ssa_decode_step_noalloc(&big, D, D, D, D, D, I, F, F, I, D, F, nullptr) ==
           SSA_ERR_UNSUPPORTED);
    ssa_params nb = base();
    nb.beta = 0.f;
    EXPECT(ssa_route_tempered(&nb, D, D, I, nullptr, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_group_stats(&p, F, F, 0, F, F, F, nullptr) == SSA_ERR_INVALID_ARGUMENT);
    EXPECT(ssa_group_stats(&p, F, F, 1 << 30, F, F, F, nullptr) == SSA_ERR_INVALID_ARGUMENT);
  }
  // status strings for every code, and for the values of the enum's range
  // that name no code
  for (int c = 0; c < 8; ++c) EXPECT(ssa_status_string(static_cast<ssa_status>(c)) != nullptr);
  EXPECT(ssa_version() >= 100);
  if (g_fail) std::fprintf(stderr, "%d expectation(s) failed\n", g_fail);
  else std::printf("abi driver: all expectations hold\n");
  return g_fail ? 1 : 0;
}
