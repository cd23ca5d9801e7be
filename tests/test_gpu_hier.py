"""GPU parity of exact hierarchical routing for decode queries
(ssa_group_stats, ssa_route_hier) against the oracle.

Group summaries are compared with the oracle's group_summaries evaluated on
the GPU's own float32 block statistics: means within 1e-5 of the tensor's
scale; the radius R_G and the covariance slack lam_G must not fall below the
oracle's value (they carry a small upward margin) and stay within 3e-4 of it.
Every selection follows rule R1 of parity.py against the oracle's flat top-k
(select_topk over r_c for every routable block, float64 from the keys): branch
and bound must return the flat selection, whatever it prunes.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import content_routed_block_stats_amd as ssa
import oracle as O
from parity import idx_ok
from synth_inputs import CONFIGS, make_decode

pytestmark = pytest.mark.gpu
DEV = "cuda"
MEAN_REL = 1e-5
SLACK_REL = 3e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_DEC = CONFIGS["decode_256k"]
# tight blocks scattered around well separated group centres: the geometry in
# which whole groups can be ruled out
_CLUSTER = dict(center_std=0.05, noise_std=0.05, group_std=1.0, plants=2)

CASES = {
    # bfloat16, d = 128, g = 4, m = 16, ragged last group, standard keys
    "bf16_g4_m16": (_DEC.replace(batch=2, n_q_heads=8, n_kv_heads=2, seq_len=64 * 300 + 37,
                                 block=64, top_k=16, window=64, plants=8), 16),
    # float32, d = 64, g = 1, m = 5, k = 3
    "f32_d64_g1_m5": (_DEC.replace(batch=3, n_q_heads=2, n_kv_heads=2, head_dim=64, dtype="f32",
                                   seq_len=128 * 90 + 5, block=128, top_k=3, window=128,
                                   plants=3), 5),
    # bfloat16, g = 16 (the largest group of q-heads), m = 64, k = 32
    "bf16_g16_m64_k32": (_DEC.replace(batch=1, n_q_heads=16, n_kv_heads=1, seq_len=64 * 700,
                                      block=64, top_k=32, window=64, plants=4), 64),
    # m = 1: every group is one block (R = lam = 0, the bound is the score)
    "bf16_m1": (_DEC.replace(batch=1, n_q_heads=4, n_kv_heads=2, seq_len=128 * 40 + 100,
                             block=128, top_k=8, window=128, plants=2), 1),
    # beta = 0 (the centroid score: no covariance term in score or bound), d = 64
    "bf16_d64_beta0_m8": (_DEC.replace(batch=2, n_q_heads=4, n_kv_heads=1, head_dim=64,
                                       seq_len=64 * 200 + 3, block=64, top_k=8, window=64,
                                       beta=0.0, plants=4), 8),
    # clustered keys, d = 128, g = 4, m = 16: most groups pruned
    "bf16_clustered_m16": (_DEC.replace(batch=2, n_q_heads=8, n_kv_heads=2, seq_len=64 * 512,
                                        block=64, top_k=8, window=64, **_CLUSTER), 16),
    # clustered keys, float32, d = 64, m = 8, k = 16
    "f32_clustered_m8": (_DEC.replace(batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64,
                                      dtype="f32", seq_len=128 * 200 + 17, block=128, top_k=16,
                                      window=128, **_CLUSTER), 8),
}


def _inputs(wl, seed):
    """Decode query and the full key history (cache plus the appended key)."""
    data = make_decode(wl, seed=seed)
    L = data["cache_len"]
    K = data["K_cache"].clone()
    K[:, :, L] = data["k_new"]
    return data["q"], K, L


def run(wl, m, pos, seed=0):
    q, K, L = _inputs(wl, seed)
    mu, sigma = ssa.ssa_block_stats(K.to(DEV), wl.block)
    gmu, gsig, grl = ssa.ssa_group_stats(mu, sigma, block_size=wl.block, group_blocks=m)
    pos_d = torch.tensor(pos, dtype=torch.int32, device=DEV)
    idx, ev = ssa.ssa_route_hier(q.to(DEV), mu, sigma, gmu, gsig, grl, pos_d, block_size=wl.block,
                                 group_blocks=m, top_k=wl.top_k, beta=wl.beta,
                                 want_evaluated=True)
    torch.cuda.synchronize()
    return dict(q=q, K=K, mu=mu.cpu(), sigma=sigma.cpu(), gmu=gmu.cpu(), gsig=gsig.cpu(),
                grl=grl.cpu(), idx=idx.cpu().numpy(), ev=ev.cpu().numpy())


def check_groups(res, m):
    b_, hkv = res["mu"].shape[:2]
    for b in range(b_):
        for kv in range(hkv):
            gs = O.group_summaries(res["mu"][b, kv].double().numpy(),
                                   res["sigma"][b, kv].double().numpy(), m)
            for name, got, ref in (("mu_G", res["gmu"][b, kv], gs["mu"]),
                                   ("S_G", res["gsig"][b, kv], gs["S"])):
                err = np.abs(got.double().numpy() - ref).max()
                assert err <= MEAN_REL * max(1.0, np.abs(ref).max()), (name, b, kv, err)
            for col, name in ((0, "R"), (1, "lam")):
                got = res["grl"][b, kv, :, col].double().numpy()
                ref = gs[name]
                assert np.all(got >= ref), (name, b, kv, np.min(got - ref))
                assert np.all(got <= ref * (1 + SLACK_REL) + 1e-6), (name, b, kv)


def check_selection(res, wl, pos):
    g, B, k = wl.group, wl.block, wl.top_k
    n_exact = n_tie = 0
    evaluated = routable = 0
    for b in range(wl.batch):
        for kv in range(wl.n_kv_heads):
            mu, sigma = O.block_stats(O.as_f64(res["K"][b, kv]), B)
            C = O.routable_blocks(pos[b], B, mu.shape[0])
            assert 0 <= res["ev"][b, kv] <= C, (b, kv, res["ev"][b, kv], C)
            evaluated += int(res["ev"][b, kv])
            routable += C
            for h in range(kv * g, (kv + 1) * g):
                r = O.route_scores(O.as_f64(res["q"][b, h]), mu[:C], sigma[:C], wl.beta)
                sel, rk, rk1 = O.select_topk(r, k)
                ok, exact = idx_ok(res["idx"][b, h], dict(idx=sel, scores=r, r_k=rk, r_k1=rk1))
                assert ok, f"selection mismatch at {(b, h)}: {res['idx'][b, h]} vs {sel}"
                n_exact += exact
                n_tie += not exact
    say(f"  rows exact {n_exact}, near-ties {n_tie}; blocks evaluated {evaluated} of {routable}")
    return evaluated, routable


@pytest.mark.parametrize("name", list(CASES))
def test_hier_parity(name):
    wl, m = CASES[name]
    say(f"case {name}: b={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} L={wl.seq_len} "
        f"d={wl.head_dim} {wl.dtype} B={wl.block} k={wl.top_k} m={m}")
    L = wl.seq_len
    pos = [L] + [L - 777 * i for i in range(1, wl.batch)]
    res = run(wl, m, pos, seed=4)
    check_groups(res, m)
    evaluated, routable = check_selection(res, wl, pos)
    if "clustered" in name:
        assert evaluated <= routable // 2, "clustered keys should prune most groups"


def test_hier_positions_before_first_block_and_k0():
    """pos < B - 1 routes nothing (all -1); k = 0 writes nothing and scores nothing."""
    wl, m = CASES["bf16_m1"]
    say("case hier short positions and k = 0")
    res = run(wl, m, [wl.block - 2], seed=5)
    assert (res["idx"] == -1).all() and (res["ev"] == 0).all()
    res = run(wl, m, [wl.block - 1], seed=5)     # exactly one routable block
    assert (res["idx"][:, :, 0] == 0).all() and (res["idx"][:, :, 1:] == -1).all()
    q, K, _ = _inputs(wl, 5)
    mu, sigma = ssa.ssa_block_stats(K.to(DEV), wl.block)
    gs = ssa.ssa_group_stats(mu, sigma, block_size=wl.block, group_blocks=m)
    pos = torch.tensor([wl.seq_len], dtype=torch.int32, device=DEV)
    idx, ev = ssa.ssa_route_hier(q.to(DEV), mu, sigma, *gs, pos, block_size=wl.block,
                                 group_blocks=m, top_k=0, want_evaluated=True)
    assert idx.numel() == 0 and int(ev.sum()) == 0


def test_hier_matches_decode_step_selection():
    """The selection ssa_decode_step makes for the same query (the flat router
    on the same float32 statistics), up to near-ties."""
    wl, m = CASES["bf16_g4_m16"]
    say("case hier vs decode step")
    data = make_decode(wl, seed=6, capacity=wl.seq_len + 1)
    L = data["cache_len"]
    Kc, Vc = data["K_cache"].to(DEV), data["V_cache"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(Kc, wl.block)   # slots of complete blocks only are read
    clen = torch.full((wl.batch,), L, dtype=torch.int32, device=DEV)
    q = data["q"].to(DEV)
    _, _, idx_flat = ssa.ssa_decode_step(q, data["k_new"].to(DEV), data["v_new"].to(DEV), Kc, Vc,
                                         clen, mu, sigma, block_size=wl.block, top_k=wl.top_k,
                                         window=wl.window, beta=wl.beta, return_idx=True)
    gs = ssa.ssa_group_stats(mu, sigma, block_size=wl.block, group_blocks=m)
    pos = torch.full((wl.batch,), L, dtype=torch.int32, device=DEV)
    idx = ssa.ssa_route_hier(q, mu, sigma, *gs, pos, block_size=wl.block, group_blocks=m,
                             top_k=wl.top_k, beta=wl.beta)
    torch.cuda.synchronize()
    a, f = idx.cpu().numpy(), idx_flat.cpu().numpy()
    same = (a == f).all(axis=-1)
    assert same.mean() >= 0.9, f"only {same.mean():.2f} of rows agree with the flat router"
