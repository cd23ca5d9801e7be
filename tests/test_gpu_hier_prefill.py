"""GPU parity of exact hierarchical routing for prefill rows
(ssa_group_stats, ssa_route_hier_prefill).

Branch and bound must return the flat selection whatever it prunes: every
row's selection equals, entry for entry, the GPU's flat router run with its
exact pass on every row (the k-th scores requested), whose scores the visit
computes with the same arithmetic, and sampled rows of every q-head follow
rule R1 of parity.py against the oracle's flat top-k (select_topk over r_c
for every routable block, float64 from the keys).  The blocks each listed
tile scored stay within [0, nb]; the share of (row, block) scores computed is
reported.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import content_routed_block_stats_amd as ssa
import oracle as O
from parity import check_idx_properties, idx_ok
from synth_inputs import CONFIGS, make_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_BASE = CONFIGS["prefill_32k"]
_CLUSTER = dict(center_std=0.05, noise_std=0.05, group_std=1.0)

CASES = {
    # d = 128, GQA 8/2, m = 16, ragged last tile and group
    "g4_m16": (_BASE.replace(batch=1, n_q_heads=8, n_kv_heads=2, seq_len=64 * 150 + 37, block=64,
                             top_k=8, window=64, plants=8), 16),
    # d = 64, two sequences, MHA, m = 5, k = 3
    "d64_b2_m5": (_BASE.replace(batch=2, n_q_heads=2, n_kv_heads=2, head_dim=64,
                                seq_len=128 * 60 + 5, block=128, top_k=3, window=128, plants=3), 5),
    # k = 32, m = 64 (the largest group), g = 16
    "g16_m64_k32": (_BASE.replace(batch=1, n_q_heads=16, n_kv_heads=1, seq_len=64 * 160,
                                  block=64, top_k=32, window=64, plants=4), 64),
    # m = 1: every group is one block (the bound is the score plus its margin)
    "m1": (_BASE.replace(batch=1, n_q_heads=4, n_kv_heads=2, seq_len=128 * 40 + 100, block=128,
                         top_k=8, window=128, plants=2), 1),
    # beta = 0 (centroid score), k = 16
    "beta0_m8": (_BASE.replace(batch=1, n_q_heads=4, n_kv_heads=1, seq_len=64 * 200 + 3, block=64,
                               top_k=16, window=64, beta=0.0, plants=4), 8),
    # clustered keys: most groups pruned
    "clustered_m16": (_BASE.replace(batch=1, n_q_heads=8, n_kv_heads=2, seq_len=64 * 256,
                                    block=64, top_k=8, window=64, plants=2, **_CLUSTER), 16),
    # clustered keys and topical queries (each 1024-token segment leans toward
    # one earlier group), no planted outliers: whole groups pruned per tile
    "topical_m16": (_BASE.replace(batch=1, n_q_heads=8, n_kv_heads=2, seq_len=64 * 512, block=64,
                                  top_k=8, window=64, plants=0, group_blocks=16, query_topic=0.5,
                                  topic_span=1024, **_CLUSTER), 16),
    # k >= nb for the early rows and more: every routable block kept
    "dense_k": (_BASE.replace(batch=1, n_q_heads=2, n_kv_heads=1, seq_len=64 * 20 + 9, block=64,
                              top_k=32, window=64, plants=1), 4),
}


def _run(wl, m, seed=0):
    data = make_prefill(wl, seed=seed, device=DEV)
    Q, K = data["Q"], data["K"]
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    gs = ssa.ssa_group_stats(mu, sigma, block_size=wl.block, group_blocks=m)
    idx, ev = ssa.ssa_route_hier_prefill(Q, mu, sigma, *gs, block_size=wl.block, group_blocks=m,
                                         top_k=wl.top_k, beta=wl.beta, want_evaluated=True)
    flat, _ = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta,
                                 want_kth=True)
    torch.cuda.synchronize()
    return data, idx.cpu().numpy(), ev.cpu().numpy(), flat.cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
def test_hier_prefill_small(name):
    wl, m = CASES[name]
    say(f"case {name}: n={wl.seq_len} heads={wl.n_q_heads}/{wl.n_kv_heads} d={wl.head_dim} "
        f"B={wl.block} k={wl.top_k} m={m} beta={wl.beta}")
    data, idx, ev, flat = _run(wl, m)
    n, B, g = wl.seq_len, wl.block, wl.group
    nb = n // B
    check_idx_properties(idx[0], n, B, wl.top_k)
    diff = np.argwhere((idx != flat).any(-1))
    assert diff.size == 0, f"differs from the flat exact pass at {diff[:5].tolist()}"
    # sampled rows of every (sequence, q-head) against the oracle: 96 uniform
    # positions plus the edges of the first block and the last row
    n_tie = 0
    rng = np.random.default_rng(5)
    for b in range(wl.batch):
        for kv in range(wl.n_kv_heads):
            Kh = O.as_f64(data["K"][b, kv])
            mu, sigma = O.block_stats(Kh, B)
            for j in range(g):
                h = kv * g + j
                Qh = O.as_f64(data["Q"][b, h])
                ts = sorted(set(rng.integers(0, n, size=96).tolist() + [0, B - 2, B - 1, B, n - 1]))
                for t in ts:
                    C = O.routable_blocks(t, B, nb)
                    r = O.route_scores(Qh[t], mu[:C], sigma[:C], wl.beta)
                    sel, rk, rk1 = O.select_topk(r, wl.top_k)
                    ok, exact = idx_ok(idx[b, h, t], dict(idx=sel, scores=r, r_k=rk, r_k1=rk1))
                    assert ok, f"row {(b, h, t)}: gpu {idx[b, h, t].tolist()} oracle {sel.tolist()}"
                    n_tie += not exact
    # blocks scored: per listed tile at most nb; against the rows' routable
    # blocks (each tile's largest over its rows is at most nb, so the share
    # below can only overstate what was scored per row)
    rows = n * g
    tiles = ev.shape[-1]
    assert tiles == -(-rows // 512)
    assert np.all(ev >= 0) and np.all(ev <= nb)
    routable_pairs = sum(min(nb, (t + 1) // B) for t in range(n)) * g * wl.batch * wl.n_kv_heads
    # every listed tile scores its blocks for (up to) 512 rows
    frac = ev.sum() * 512.0 / max(1, routable_pairs)
    say(f"  (row, block) scores computed: {frac:.3f} of the routable pairs")
    say(f"  near-ties {n_tie}")


def test_hier_prefill_no_complete_block():
    """n < B: no block is routable; every row gets k entries of -1."""
    g = torch.Generator(device=DEV).manual_seed(1)
    Q = torch.randn((1, 2, 50, 128), generator=g, device=DEV).to(torch.bfloat16)
    mu = torch.empty((1, 1, 0, 128), dtype=torch.float32, device=DEV)     # no complete block
    sigma = torch.empty((1, 1, 0, 128, 128), dtype=torch.float32, device=DEV)
    gs = ssa.ssa_group_stats(mu, sigma, block_size=64, group_blocks=4)
    idx, ev = ssa.ssa_route_hier_prefill(Q, mu, sigma, *gs, block_size=64, group_blocks=4,
                                         top_k=4, beta=2.0, want_evaluated=True)
    torch.cuda.synchronize()
    assert (idx.cpu().numpy() == -1).all()
    assert (ev.cpu().numpy() == 0).all()
