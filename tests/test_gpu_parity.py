"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case draws a seeded synthetic workload, runs ssa_block_stats ->
ssa_route_topk -> ssa_sparse_attn_fwd (or ssa_decode_step) on the GPU and
compares with the oracle under the rules in parity.py.  Small cases compare
every row; the full-size workloads compare sampled rows one by one and check
properties that hold at any size on every row.
"""
from __future__ import annotations

import math
import json
import os
import sys

import numpy as np
import pytest
import torch

import content_routed_block_stats_amd as ssa
import oracle as O
from parity import LSE_TOL, O_TOL, STATS_REL, attn_errors, check_idx_properties, idx_ok
from synth_inputs import CONFIGS, make_decode, make_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _params(wl):
    return O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)


def run_prefill(Q, K, V, wl, out_dtype=None):
    """Statistics, routing and attention as a caller runs them (no k-th scores
    requested: bfloat16 inputs take the certified single pass), plus a second
    routing call that requests the k-th scores (the exact pass on every row)."""
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta)
    idx_exact, kth = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k,
                                        beta=wl.beta, want_kth=True)
    Oo, lse = ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                      scale=wl.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dict(mu=mu, sigma=sigma, idx=idx, idx_exact=idx_exact, kth=kth, O=Oo, lse=lse)


def compare_prefill(data, res, wl, rows=None, check_stats=True, O32=None, lse32=None):
    """Compare GPU results with the oracle on the given (b, h, t) rows (all if None)."""
    p = _params(wl)
    orc = O.PrefillOracle(data["Q"], data["K"], data["V"], p)
    g = wl.group
    if check_stats:
        mu_g = res["mu"].cpu().double().numpy()
        sg_g = res["sigma"].cpu().double().numpy()
        for b in range(wl.batch):
            for kv in range(wl.n_kv_heads):
                _, _, mu, sigma = orc.head(b, kv)
                if mu.shape[0] == 0:
                    continue
                scale = max(1.0, np.abs(sigma).max())
                assert np.abs(mu_g[b, kv] - mu).max() <= STATS_REL * scale, "mu"
                assert np.abs(sg_g[b, kv] - sigma).max() <= STATS_REL * scale, "sigma"
    idx = res["idx"].cpu().numpy()
    idx_exact = res["idx_exact"].cpu().numpy() if res.get("idx_exact") is not None else None
    bf16_out = res["O"].dtype == torch.bfloat16
    Og = res["O"].float().cpu().numpy()
    lg = res["lse"].cpu().numpy()
    O32 = None if O32 is None else O32.cpu().numpy()
    if rows is None:
        rows = [(b, h, t) for b in range(wl.batch) for h in range(wl.n_q_heads)
                for t in range(wl.seq_len)]
    o_tol = O_TOL[wl.dtype]
    n_exact = n_tie = 0
    worst_o = worst_l = worst_o32 = 0.0
    eps = []
    for (b, h, t) in rows:
        row = orc.row(b, h, t)
        ok, exact = idx_ok(idx[b, h, t], row)
        assert ok, f"selection mismatch at row {(b, h, t)}: gpu {idx[b, h, t].tolist()} " \
                   f"oracle {row['idx'].tolist()}"
        if idx_exact is not None:   # the exact pass on every row (k-th scores requested)
            ok2, _ = idx_ok(idx_exact[b, h, t], row)
            assert ok2, f"exact-pass selection mismatch at row {(b, h, t)}: " \
                        f"gpu {idx_exact[b, h, t].tolist()} oracle {row['idx'].tolist()}"
        n_exact += exact
        n_tie += (not exact)
        kv = h // g
        Kh, Vh, _, _ = orc.head(b, kv)
        qrow = O.as_f64(data["Q"][b, h, t])
        eo, el = attn_errors(Og[b, h, t], lg[b, h, t], qrow, Kh, Vh, idx[b, h, t], t, p,
                             bf16_out=bf16_out)
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
        # dropped softmax mass of the GPU's selection (reported, not checked)
        eps.append(O.dropped_mass(qrow, Kh, O.key_set(t, idx[b, h, t], p.block, p.window), t,
                                  p.scale)[0])
        assert eo <= o_tol, f"O error {eo:.3g} at row {(b, h, t)}"
        assert el <= LSE_TOL, f"LSE error {el:.3g} at row {(b, h, t)}"
        if O32 is not None:       # the same inputs with a float32 output tensor
            e32, _ = attn_errors(O32[b, h, t], lg[b, h, t], qrow, Kh, Vh, idx[b, h, t], t, p)
            worst_o32 = max(worst_o32, e32)
            assert e32 <= o_tol, f"float32-output O error {e32:.3g} at row {(b, h, t)}"
    say(f"  rows {len(rows)}: exact selections {n_exact}, allowed near-ties {n_tie}, "
        f"max|dO| {worst_o:.3g} (f32 out {worst_o32:.3g}), max|dLSE| {worst_l:.3g}")
    e = np.asarray(eps)
    rec = {"case": wl.name, "rows": len(rows), "exact": n_exact, "near_ties": n_tie,
           "dropped_mass": {"rows": int(e.size), "mean": float(e.mean()),
                            "p50": float(np.percentile(e, 50)), "p99": float(np.percentile(e, 99)),
                            "max": float(e.max())}}
    say("  report:", json.dumps(rec))
    path = os.environ.get("SSA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")
    return n_exact, n_tie


SMALL = {
    "tiny_prefill_4k": CONFIGS["tiny_prefill_4k"],
    "bf16_mha_ragged": CONFIGS["prefill_32k"].replace(n_q_heads=2, n_kv_heads=2, seq_len=4096 + 100,
                                                      plants=8),
    "bf16_gqa": CONFIGS["gqa_prefill_128k"].replace(n_q_heads=8, n_kv_heads=2, seq_len=4096,
                                                    plants=8),
    "bf16_d64_batch2": CONFIGS["prefill_32k"].replace(batch=2, n_q_heads=4, n_kv_heads=1,
                                                      head_dim=64, seq_len=2048 + 37, block=64,
                                                      top_k=5, window=40, plants=6),
    "f32_d128_k_over_nb": CONFIGS["tiny_prefill_4k"].replace(head_dim=128, seq_len=1000, block=64,
                                                             top_k=20, window=64, plants=4),
    "f32_window1_k3": CONFIGS["tiny_prefill_4k"].replace(seq_len=1500, window=1, top_k=3, plants=4),
    "bf16_k0_window_only": CONFIGS["prefill_32k"].replace(n_q_heads=2, n_kv_heads=1, seq_len=3000,
                                                          top_k=0, window=200, plants=4),
    "bf16_wide_window": CONFIGS["prefill_32k"].replace(n_q_heads=1, n_kv_heads=1, seq_len=1111,
                                                       block=64, top_k=4, window=300, plants=4),
    # blocks that the block pass walks in more than one LDS-resident segment,
    # with a ragged last segment (d=128 bf16: 256 keys per segment)
    "bf16_block320_two_segments": CONFIGS["gqa_prefill_128k"].replace(
        n_q_heads=4, n_kv_heads=2, seq_len=320 * 12 + 50, block=320, top_k=4, window=100, plants=4),
    "bf16_block1024_four_segments": CONFIGS["gqa_prefill_128k"].replace(
        n_q_heads=2, n_kv_heads=1, seq_len=1024 * 5 + 5, block=1024, top_k=2, window=1024, plants=2),
    # two whole resident segments per block, walked in alternating directions
    # by consecutive tasks (d=128: 256 keys a segment; d=64: 384)
    "bf16_block512_two_segments": CONFIGS["gqa_prefill_128k"].replace(
        n_q_heads=4, n_kv_heads=1, seq_len=512 * 7 + 33, block=512, top_k=3, window=200, plants=4),
    "bf16_d64_block768_two_segments": CONFIGS["prefill_32k"].replace(
        n_q_heads=2, n_kv_heads=1, head_dim=64, seq_len=768 * 5 + 70, block=768, top_k=2,
        window=300, plants=2),
    # d=64 bf16: 512 keys per segment
    "bf16_d64_block576": CONFIGS["prefill_32k"].replace(
        n_q_heads=2, n_kv_heads=2, head_dim=64, seq_len=576 * 6 + 11, block=576, top_k=3, window=64,
        plants=4),
    # block smaller than a segment and not a power of two
    "f32_block192": CONFIGS["tiny_prefill_4k"].replace(seq_len=2000, block=192, top_k=4, window=80,
                                                       plants=4),
}


def _rows_for(wl, limit=6000, seed=0):
    total = wl.batch * wl.n_q_heads * wl.seq_len
    allrows = [(b, h, t) for b in range(wl.batch) for h in range(wl.n_q_heads)
               for t in range(wl.seq_len)]
    if total <= limit:
        return allrows
    rng = np.random.default_rng(seed)
    pick = rng.choice(total, size=limit, replace=False)
    return [allrows[i] for i in sorted(pick)]


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_parity_small(name):
    wl = SMALL[name]
    say(f"case {name}: b={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} n={wl.seq_len} "
        f"d={wl.head_dim} {wl.dtype} B={wl.block} k={wl.top_k} W={wl.window}")
    data = make_prefill(wl, seed=0)
    Q, K, V = data["Q"].to(DEV), data["K"].to(DEV), data["V"].to(DEV)
    res = run_prefill(Q, K, V, wl)
    O32 = None
    if wl.dtype == "bf16":
        O32, _ = ssa.ssa_sparse_attn_fwd(Q, K, V, res["idx"], block_size=wl.block,
                                         window=wl.window, scale=wl.scale,
                                         out_dtype=torch.float32)
        torch.cuda.synchronize()
    compare_prefill(data, res, wl, rows=_rows_for(wl), O32=O32)


def test_dense_reduction_on_gpu():
    """k >= nb and W >= B-1: the HIP path must equal dense causal attention."""
    wl = CONFIGS["tiny_prefill_4k"].replace(seq_len=700, top_k=32, window=64, plants=2)
    say("case dense reduction f32 n=700 B=64 k=32 W=64")
    data = make_prefill(wl, seed=5)
    res = run_prefill(data["Q"].to(DEV), data["K"].to(DEV), data["V"].to(DEV), wl)
    q = data["Q"][0, 0].double()
    k = data["K"][0, 0].double()
    v = data["V"][0, 0].double()
    s = (q @ k.T) * wl.scale
    s = s.masked_fill(torch.ones_like(s, dtype=torch.bool).triu(1), float("-inf"))
    ref_o = torch.softmax(s, -1) @ v
    ref_l = torch.logsumexp(s, -1)
    assert (res["O"][0, 0].double().cpu() - ref_o).abs().max().item() <= O_TOL["f32"]
    assert (res["lse"][0, 0].double().cpu() - ref_l).abs().max().item() <= LSE_TOL


def test_selection_deterministic_and_bf16_output():
    wl = SMALL["bf16_gqa"]
    say("case determinism bf16 gqa")
    data = make_prefill(wl, seed=1)
    Q, K, V = data["Q"].to(DEV), data["K"].to(DEV), data["V"].to(DEV)
    a = run_prefill(Q, K, V, wl)
    b = run_prefill(Q, K, V, wl)
    for key in ("mu", "sigma", "idx", "O", "lse"):
        assert torch.equal(a[key], b[key]), f"{key} differs between identical runs"
    c = run_prefill(Q, K, V, wl, out_dtype=torch.float32)
    assert c["O"].dtype == torch.float32
    # the bf16 output is the float32 output rounded to nearest
    assert torch.equal(a["O"], c["O"].to(torch.bfloat16))


# -------------------------------------------------------------------- decode --

def _decode_case(wl, L, cap, seed=0, steps=1):
    wl = wl.replace(seq_len=L)
    data = make_decode(wl, seed=seed, capacity=cap)
    p = _params(wl)
    Kc, Vc = data["K_cache"].to(DEV), data["V_cache"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(Kc, wl.block)
    cache_len = torch.full((wl.batch,), L, dtype=torch.int32, device=DEV)
    K_host = data["K_cache"].clone()
    V_host = data["V_cache"].clone()
    q, kn, vn = data["q"], data["k_new"], data["v_new"]
    gen = torch.Generator().manual_seed(1234 + seed)
    for step in range(steps):
        Lc = L + step
        say(f"  decode step {step}: L={Lc} completes_block={(Lc + 1) % wl.block == 0}")
        o, lse, idx = ssa.ssa_decode_step(q.to(DEV), kn.to(DEV), vn.to(DEV), Kc, Vc, cache_len, mu,
                                          sigma, block_size=wl.block, top_k=wl.top_k,
                                          window=wl.window, beta=wl.beta, scale=wl.scale,
                                          return_idx=True)
        torch.cuda.synchronize()
        assert cache_len.cpu().tolist() == [Lc + 1] * wl.batch
        idx_h, o_h, l_h = idx.cpu().numpy(), o.float().cpu().numpy(), lse.cpu().numpy()
        for b in range(wl.batch):
            for h in range(wl.n_q_heads):
                kv = h // wl.group
                row = O.decode_step(q[b, h], kn[b, kv], vn[b, kv], K_host[b, kv], V_host[b, kv],
                                    Lc, p)
                ok, _ = idx_ok(idx_h[b, h], row)
                assert ok, f"decode selection mismatch b={b} h={h}: {idx_h[b, h]} vs {row['idx']}"
                Kfull = np.concatenate([O.as_f64(K_host[b, kv, :Lc]), O.as_f64(kn[b, kv])[None]])
                Vfull = np.concatenate([O.as_f64(V_host[b, kv, :Lc]), O.as_f64(vn[b, kv])[None]])
                eo, el = attn_errors(o_h[b, h], l_h[b, h], O.as_f64(q[b, h]), Kfull, Vfull,
                                     idx_h[b, h], Lc, p, bf16_out=o.dtype == torch.bfloat16)
                assert eo <= O_TOL[wl.dtype] and el <= LSE_TOL, (b, h, eo, el)
        # the cache now holds the appended key; continue with fresh step inputs
        K_host[:, :, Lc] = kn
        V_host[:, :, Lc] = vn
        assert torch.equal(Kc[:, :, Lc].cpu(), kn) and torch.equal(Vc[:, :, Lc].cpu(), vn)
        q = torch.randn(q.shape, generator=gen).to(q.dtype)
        kn = torch.randn(kn.shape, generator=gen).to(kn.dtype)
        vn = torch.randn(vn.shape, generator=gen).to(vn.dtype)
    return mu, sigma, K_host


@pytest.mark.parametrize("L,steps", [(1000, 2), (1023, 2), (63, 1), (5, 1)])
def test_decode_parity_small(L, steps):
    wl = CONFIGS["decode_256k"].replace(batch=2, n_q_heads=8, n_kv_heads=2, block=64, top_k=8,
                                        window=64, plants=4)
    say(f"case decode small L={L} steps={steps}")
    mu, sigma, K_host = _decode_case(wl, L, cap=L + 80, steps=steps)
    # the statistics of every block the steps completed match the oracle
    B = wl.block
    done = (L + steps) // B
    for b in range(wl.batch):
        for kv in range(wl.n_kv_heads):
            mu_o, sg_o = O.block_stats(K_host[b, kv, :done * B], B)
            if done == 0:
                continue
            scale = max(1.0, np.abs(sg_o).max())
            assert np.abs(mu[b, kv, :done].cpu().double().numpy() - mu_o).max() <= STATS_REL * scale
            assert np.abs(sigma[b, kv, :done].cpu().double().numpy() - sg_o).max() <= STATS_REL * scale


def test_decode_f32_d64():
    wl = CONFIGS["decode_256k"].replace(batch=3, n_q_heads=2, n_kv_heads=1, head_dim=64,
                                        dtype="f32", block=128, top_k=3, window=100, plants=3)
    say("case decode f32 d64 L=700")
    _decode_case(wl, 700, cap=1024, steps=2)


@pytest.mark.parametrize("qexp", [18, -30])
def test_route_query_scale(qexp):
    """Routing of a KV head whose queries are scaled by 2^qexp (|q| far above
    the float16 range, or far below its normal range): the selections equal
    the oracle's on the scaled inputs (the router rescales Q per (sequence,
    KV head) by an exact power of two)."""
    wl = SMALL["bf16_gqa"].replace(top_k=4)
    say(f"case route with queries of KV head 1 scaled by 2^{qexp}")
    data = make_prefill(wl, seed=9)
    g = wl.group
    data["Q"][:, g:2 * g] = (data["Q"][:, g:2 * g].float() * 2.0 ** qexp).to(torch.bfloat16)
    Q, K = data["Q"].to(DEV), data["K"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx, kth = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta,
                                  want_kth=True)
    idx1 = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta)
    torch.cuda.synchronize()
    idx_h, kth_h, idx1_h = idx.cpu().numpy(), kth.cpu().numpy(), idx1.cpu().numpy()
    n_exact = n_tie = 0
    for kv in range(wl.n_kv_heads):
        muo, sgo = O.block_stats(O.as_f64(data["K"][0, kv]), wl.block)
        for h in range(kv * g, (kv + 1) * g):
            for t in range(0, wl.seq_len, 7):
                C = O.routable_blocks(t, wl.block, muo.shape[0])
                r = O.route_scores(O.as_f64(data["Q"][0, h, t]), muo[:C], sgo[:C], wl.beta)
                sel, rk, rk1 = O.select_topk(r, wl.top_k)
                ok, exact = idx_ok(idx_h[0, h, t], dict(idx=sel, scores=r, r_k=rk, r_k1=rk1))
                assert ok, f"selection mismatch at {(h, t)}: {idx_h[0, h, t]} vs {sel}"
                ok1, _ = idx_ok(idx1_h[0, h, t], dict(idx=sel, scores=r, r_k=rk, r_k1=rk1))
                assert ok1, f"single-pass selection mismatch at {(h, t)}: {idx1_h[0, h, t]} vs {sel}"
                n_exact += exact
                n_tie += not exact
                if C > wl.top_k:   # the k-th score, in the scaled inputs' own units
                    assert abs(kth_h[0, h, t, 0] - rk) <= 1e-5 * np.abs(r).max(), (h, t)
    say(f"  exact {n_exact}, near-ties {n_tie}")
