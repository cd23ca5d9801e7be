"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (the same C ABI calls on inputs resident in HBM).

The oracle cannot evaluate millions of rows, so every row is checked for the
properties a selection has at any size (ascending, distinct, routable,
exactly min(k, #routable) entries), and a stratified sample of rows -- every
q-head at positions drawn from equal strata of [0, n) plus rows in the first
and last blocks, and every row a planted outlier targets -- is compared one
by one with the oracle under the rules in parity.py (worker processes; every
decode row).  Each case also reports the dropped softmax mass of the GPU's
selection on its sampled rows.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os
import sys

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import content_routed_block_stats_amd as ssa
import oracle as O
from parity import (LSE_TOL, O_TOL, STATS_REL, attn_errors, check_idx_properties,
                    check_tile_properties, idx_ok)
from oracle_pool import OraclePool
from synth_inputs import CONFIGS, make_decode, make_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _report(record: dict) -> None:
    """Print a result line; append it as JSON to $SSA_PARITY_REPORT if set."""
    say("  report:", json.dumps(record))
    path = os.environ.get("SSA_PARITY_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


def _eps_stats(eps) -> dict:
    e = np.asarray(eps, np.float64)
    return {"rows": int(e.size), "mean": float(e.mean()), "p50": float(np.percentile(e, 50)),
            "p99": float(np.percentile(e, 99)), "max": float(e.max())}


def _sample_rows(wl, per_head: int, plants: list[dict], seed: int = 0):
    """Stratified rows: per q-head, per_head positions spread over [0, n) (one
    uniform draw in each of per_head equal strata) plus one row in the first
    and one in the last block; and every row a planted outlier targets."""
    rng = np.random.default_rng(seed)
    rows = set()
    n = wl.seq_len
    edges = np.linspace(0, n, per_head + 1).astype(np.int64)
    for h in range(wl.n_q_heads):
        ts = [int(rng.integers(lo, max(lo + 1, hi))) for lo, hi in zip(edges[:-1], edges[1:])]
        ts += [int(rng.integers(0, wl.block)), n - 1 - int(rng.integers(0, wl.block))]
        for t in ts:
            rows.add((0, h, int(t)))
    for p in plants:
        rows.add((p["b"], p["h"], p["t"]))
    return sorted(rows)


def _prefill_fullsize(name: str, per_head: int, stats_blocks: int, fp32_out: bool = False):
    wl = CONFIGS[name]
    say(f"case {name}: generating on the GPU")
    data = make_prefill(wl, seed=0, device=DEV)
    Q, K, V = data["Q"], data["K"], data["V"]
    say("  block stats / route / attention")
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta)
    Oo, lse = ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                      scale=wl.scale)
    outs = {"out": (Oo, lse, Oo.dtype == torch.bfloat16)}
    if fp32_out:
        O32, lse32 = ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                             scale=wl.scale, out_dtype=torch.float32)
        outs["f32"] = (O32, lse32, False)
    torch.cuda.synchronize()
    say("  selection properties on every row")
    idx_h = idx.cpu().numpy()
    check_idx_properties(idx_h[0], wl.seq_len, wl.block, wl.top_k)
    rows = _sample_rows(wl, per_head, data["plants"])
    say(f"  oracle on {len(rows)} sampled rows ({len(data['plants'])} planted) in worker processes")
    hs = torch.tensor([r[1] for r in rows], device=DEV)
    ts = torch.tensor([r[2] for r in rows], device=DEV)
    q_rows = Q[0][hs, ts].double().cpu().numpy()
    got = {lab: (O_[0][hs, ts].float().cpu().numpy(), l_[0][hs, ts].cpu().numpy(), bf)
           for lab, (O_, l_, bf) in outs.items()}
    del idx, outs, Oo, lse
    p = O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)
    g = wl.group
    by_kv: dict[int, list] = {}
    for i, (b, h, t) in enumerate(rows):
        by_kv.setdefault(O.kv_head(h, wl.n_q_heads, wl.n_kv_heads), []).append(i)
    n_exact = n_tie = 0
    worst = {lab: [0.0, 0.0] for lab in got}
    eps = []
    rng = np.random.default_rng(1)
    params = (p.block, p.top_k, p.window, p.beta, p.scale)
    with OraclePool(params) as pool:
        for kv, ids in sorted(by_kv.items()):
            Kh = O.as_f64(K[0, kv])
            Vh = O.as_f64(V[0, kv])
            mu_o, sg_o = O.block_stats(Kh, wl.block)
            # statistics of sampled blocks
            for c in rng.choice(mu_o.shape[0], size=min(stats_blocks, mu_o.shape[0]), replace=False):
                scale_s = max(1.0, np.abs(sg_o[c]).max())
                assert np.abs(mu[0, kv, c].double().cpu().numpy() - mu_o[c]).max() <= STATS_REL * scale_s
                assert np.abs(sigma[0, kv, c].double().cpu().numpy() - sg_o[c]).max() <= STATS_REL * scale_s
            tasks = [dict(key=(rows[i][1], rows[i][2]), t=rows[i][2], q=q_rows[i],
                          idx=idx_h[0, rows[i][1], rows[i][2]],
                          outputs={lab: (v[0][i], float(v[1][i]), v[2]) for lab, v in got.items()})
                     for i in ids]
            for r in pool.run_head(f"kv{kv}", Kh, Vh, mu_o, sg_o, tasks):
                h, t = r["key"]
                assert r["ok"], f"selection mismatch at {(h, t)}: {idx_h[0, h, t]} vs {r['oracle_idx']}"
                n_exact += r["exact"]
                n_tie += not r["exact"]
                for lab in got:
                    eo, el = r["O_err_" + lab], r["lse_err_" + lab]
                    worst[lab] = [max(worst[lab][0], eo), max(worst[lab][1], el)]
                    assert eo <= O_TOL[wl.dtype], f"O error ({lab}) {eo:.3g} at {(h, t)}"
                    assert el <= LSE_TOL, f"LSE error ({lab}) {el:.3g} at {(h, t)}"
                eps.append(r["eps"])
            del Kh, Vh, mu_o, sg_o
            say(f"  kv head {kv}: {len(ids)} rows ok")
    say(f"  {name}: exact {n_exact}, near-ties {n_tie}, worst (|dO|, |dLSE|) {worst}")
    _report({"case": name, "rows": len(rows), "planted_rows": len(data["plants"]),
             "exact": n_exact, "near_ties": n_tie,
             "worst": {lab: {"O": w[0], "lse": w[1]} for lab, w in worst.items()},
             "dropped_mass": _eps_stats(eps)})


@pytest.mark.timeout(900)
def test_prefill_32k_fullsize():
    """16,384 stratified rows (2,048 per q-head) + every planted row; bf16 and
    float32 outputs."""
    _prefill_fullsize("prefill_32k", per_head=2048, stats_blocks=16, fp32_out=True)


@pytest.mark.timeout(900)
def test_gqa_prefill_128k_fullsize():
    """4,096 stratified rows (128 per q-head) + every planted row."""
    _prefill_fullsize("gqa_prefill_128k", per_head=128, stats_blocks=8)


@pytest.mark.timeout(1200)
def test_long_prefill_1m_fullsize():
    """2,048 stratified rows (128 per q-head) + every planted row."""
    _prefill_fullsize("long_prefill_1m", per_head=128, stats_blocks=4)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("keys", ["standard", "topical"])
def test_long_prefill_1m_hier_fullsize(keys):
    """Exact hierarchical prefill routing (groups of 16 blocks) at 1M tokens:
    every row equals the flat router's exact pass (the same arithmetic on
    the blocks it scores), and sampled rows equal the oracle's flat top-k
    under R1; the share of (row, block) scores computed is reported.
    "topical": clustered keys and topical queries (no plants), where whole
    groups are pruned -- the share must then stay well below one."""
    wl = CONFIGS["long_prefill_1m"]
    m = 16
    if keys == "topical":
        wl = wl.replace(center_std=0.05, noise_std=0.05, group_std=1.0, group_blocks=m, plants=0,
                        query_topic=0.5, topic_span=1024)
    say(f"case long_prefill_1m hierarchical routing, {keys} inputs: generating on the GPU")
    data = make_prefill(wl, seed=0, device=DEV)
    Q, K = data["Q"], data["K"]
    del data["V"]
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    gs = ssa.ssa_group_stats(mu, sigma, block_size=wl.block, group_blocks=m)
    idx, ev = ssa.ssa_route_hier_prefill(Q, mu, sigma, *gs, block_size=wl.block, group_blocks=m,
                                         top_k=wl.top_k, beta=wl.beta, want_evaluated=True)
    flat, _ = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta,
                                 want_kth=True)
    torch.cuda.synchronize()
    differ = int((idx != flat).any(-1).sum())
    assert differ == 0, f"{differ} rows differ from the flat exact pass"
    n, B, g = wl.seq_len, wl.block, wl.group
    nb = n // B
    routable = (B * nb * (nb - 1) // 2 + (n - nb * B + 1) * nb) * g * wl.n_kv_heads
    frac = ev.long().sum().item() * 512 / routable
    say(f"  (row, block) scores computed: {frac:.3f} of the routable pairs")
    if keys == "topical":
        assert frac < 0.5, f"topical inputs: {frac:.3f} of the pairs scored, expected pruning"
    idx_h = idx.cpu().numpy()
    del flat, idx
    p = O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)
    rng = np.random.default_rng(7)
    for kv in range(wl.n_kv_heads):
        Kh = O.as_f64(K[0, kv])
        mu_o, sg_o = O.block_stats(Kh, B)
        for _ in range(8):
            h = kv * g + int(rng.integers(g))
            t = int(rng.integers(0, n))
            q = O.as_f64(Q[0, h, t])
            C = O.routable_blocks(t, B, nb)
            r = O.route_scores(q, mu_o[:C], sg_o[:C], wl.beta)
            sel, rk, rk1 = O.select_topk(r, wl.top_k)
            ok, _ = idx_ok(idx_h[0, h, t], dict(idx=sel, scores=r, r_k=rk, r_k1=rk1))
            assert ok, f"row {(h, t)}: gpu {idx_h[0, h, t].tolist()} oracle {sel.tolist()}"
        say(f"  kv head {kv}: 8 sampled rows equal the oracle's flat top-k")


@pytest.mark.timeout(900)
def test_decode_256k_fullsize():
    """Every one of the 1,024 decode rows against the oracle.  A decode step is
    the prefill row at t = L over the L + 1 keys (the oracle's decode_step,
    pinned equal to that composition); the statistics of each (sequence, KV
    head) are computed once for its group's rows, in host threads."""
    wl = CONFIGS["decode_256k"]
    L = wl.seq_len
    say("case decode_256k: generating the 32 x 262144-token caches on the GPU")
    data = make_decode(wl, seed=0, device=DEV, capacity=L + 64)
    Kc, Vc = data["K_cache"], data["V_cache"]
    mu, sigma = ssa.ssa_block_stats(Kc, wl.block)
    cache_len = torch.full((wl.batch,), L, dtype=torch.int32, device=DEV)
    q, kn, vn = data["q"], data["k_new"], data["v_new"]
    say("  decode step")
    o, lse, idx = ssa.ssa_decode_step(q, kn, vn, Kc, Vc, cache_len, mu, sigma, block_size=wl.block,
                                      top_k=wl.top_k, window=wl.window, beta=wl.beta,
                                      scale=wl.scale, return_idx=True)
    torch.cuda.synchronize()
    assert cache_len.cpu().tolist() == [L + 1] * wl.batch
    idx_h = idx.cpu().numpy()
    nbc = (L + 1) // wl.block
    valid = idx_h >= 0
    assert np.all(valid.sum(-1) == min(wl.top_k, nbc))
    assert np.all(np.where(valid, idx_h < nbc, True))
    assert np.all(np.diff(idx_h, axis=-1) > 0)
    p = O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)
    bf16_out = o.dtype == torch.bfloat16
    o_h, lse_h, q_h = o.float().cpu().numpy(), lse.cpu().numpy(), q.double().cpu().numpy()

    def pair(b: int, kv: int) -> list:
        # the cache rows [0, L) now hold the same keys as before the step
        K = np.concatenate([O.as_f64(Kc[b, kv, :L]), O.as_f64(kn[b, kv])[None]])
        V = np.concatenate([O.as_f64(Vc[b, kv, :L]), O.as_f64(vn[b, kv])[None]])
        mu_o, sg_o = O.block_stats(K, wl.block)
        out = []
        for h in range(kv * wl.group, (kv + 1) * wl.group):
            row = O.prefill_row(q_h[b, h], K, V, mu_o, sg_o, p, L)
            ok, exact = idx_ok(idx_h[b, h], row)
            eo, el = attn_errors(o_h[b, h], float(lse_h[b, h]), q_h[b, h], K, V, idx_h[b, h], L, p,
                                 bf16_out=bf16_out)
            e = O.dropped_mass(q_h[b, h], K, O.key_set(L, idx_h[b, h], p.block, p.window), L,
                               p.scale)[0]
            out.append((b, h, ok, exact, eo, el, e, row["idx"].tolist()))
        return out

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    say(f"  oracle on all {wl.batch * wl.n_q_heads} rows, {workers} host threads")
    results = []
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(pair, b, kv) for b in range(wl.batch) for kv in range(wl.n_kv_heads)]
        for i, f in enumerate(futs):
            results.extend(f.result())
            if i % 32 == 31:
                say(f"  {i + 1} of {len(futs)} (sequence, KV head) pairs done")
    n_exact = n_tie = 0
    worst_o = worst_l = 0.0
    for (b, h, ok, exact, eo, el, e, oidx) in results:
        assert ok, f"decode selection mismatch b={b} h={h}: {idx_h[b, h]} vs {oidx}"
        assert eo <= O_TOL[wl.dtype] and el <= LSE_TOL, (b, h, eo, el)
        n_exact += exact
        n_tie += not exact
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    _report({"case": "decode_256k", "rows": len(results), "exact": n_exact, "near_ties": n_tie,
             "worst": {"out": {"O": worst_o, "lse": worst_l}},
             "dropped_mass": _eps_stats([r[6] for r in results])})


@pytest.mark.timeout(600)
def test_gqa_prefill_128k_tiles_fullsize():
    """Query-tile-shared routing and tile attention at the 128K GQA workload:
    properties of every tile's selection, and sampled tiles (their selection
    and sampled rows' O and LSE) against the oracle."""
    wl = CONFIGS["gqa_prefill_128k"]
    say("case gqa_prefill_128k tiles: generating on the GPU")
    data = make_prefill(wl, seed=0, device=DEV)
    Q, K, V = data["Q"], data["K"], data["V"]
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_tiles(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta)
    Oo, lse = ssa.ssa_tile_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                    scale=wl.scale)
    torch.cuda.synchronize()
    idx_h = idx.cpu().numpy()
    say("  selection properties on every tile")
    check_tile_properties(idx_h[0], wl.seq_len, wl.block, wl.top_k)
    p = O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)
    rng = np.random.default_rng(3)
    tiles = idx_h.shape[2]
    picks = [(0, 0), (5, 1), (31, 17), (6, 130), (22, tiles - 1), (13, int(rng.integers(200, tiles)))]
    bf16_out = Oo.dtype == torch.bfloat16
    for (h, j) in picks:
        kv = h // wl.group
        Kh = O.as_f64(K[0, kv])
        Vh = O.as_f64(V[0, kv])
        C = min(j, wl.seq_len // wl.block)          # the tile's routable blocks
        mu_o, sg_o = O.block_stats(Kh[:C * wl.block], wl.block)
        orc = O.tile_select(O.as_f64(Q[0, h, :(j + 1) * wl.block]), mu_o, sg_o, p, j)
        ok, _ = idx_ok(idx_h[0, h, j], orc)
        assert ok, f"tile selection mismatch at head {h}, tile {j}: {idx_h[0, h, j]} vs {orc['idx']}"
        for t in sorted(set([j * wl.block, j * wl.block + wl.block - 1] +
                            list(rng.integers(j * wl.block, (j + 1) * wl.block, size=6)))):
            eo, el = attn_errors(Oo[0, h, t].float().cpu().numpy(), float(lse[0, h, t]),
                                 O.as_f64(Q[0, h, t]), Kh, Vh, idx_h[0, h, j], t, p,
                                 bf16_out=bf16_out)
            assert eo <= O_TOL[wl.dtype] and el <= LSE_TOL, (h, j, t, eo, el)
        say(f"  head {h} tile {j}: selection ok, rows ok")



@pytest.mark.timeout(600)
@pytest.mark.parametrize("keys", ["standard", "clustered", "topical"])
def test_decode_256k_hier_fullsize(keys):
    """Exact hierarchical routing on the 32 x 256K decode caches (groups of 16
    blocks): every row's selection equals the flat decode router's up to
    near-ties, and sampled (sequence, KV head) pairs equal the oracle's flat
    top-k; on clustered keys at most 60% of the blocks are scored, and with a
    topical query (leaning toward one earlier group; no plants) at most 30%."""
    wl = CONFIGS["decode_256k"]
    if keys == "clustered":
        wl = wl.replace(center_std=0.05, noise_std=0.05, group_std=1.0, plants=2)
    if keys == "topical":
        wl = wl.replace(center_std=0.05, noise_std=0.05, group_std=1.0, plants=0, group_blocks=16,
                        query_topic=0.5, topic_span=1024)
    L, m = wl.seq_len, 16
    say(f"case decode_256k hierarchical routing, {keys} keys: generating on the GPU")
    data = make_decode(wl, seed=0, device=DEV, capacity=L + 1)
    Kc, Vc, q = data["K_cache"], data["V_cache"], data["q"]
    mu, sigma = ssa.ssa_block_stats(Kc, wl.block)
    gs = ssa.ssa_group_stats(mu, sigma, block_size=wl.block, group_blocks=m)
    pos = torch.full((wl.batch,), L, dtype=torch.int32, device=DEV)
    idx, ev = ssa.ssa_route_hier(q, mu, sigma, *gs, pos, block_size=wl.block, group_blocks=m,
                                 top_k=wl.top_k, beta=wl.beta, want_evaluated=True)
    cache_len = torch.full((wl.batch,), L, dtype=torch.int32, device=DEV)
    _, _, idx_flat = ssa.ssa_decode_step(q, data["k_new"], data["v_new"], Kc, Vc, cache_len, mu,
                                         sigma, block_size=wl.block, top_k=wl.top_k,
                                         window=wl.window, beta=wl.beta, scale=wl.scale,
                                         return_idx=True)
    torch.cuda.synchronize()
    idx_h, flat_h, ev_h = idx.cpu().numpy(), idx_flat.cpu().numpy(), ev.cpu().numpy()
    nbc = (L + 1) // wl.block
    frac = ev_h.sum() / (ev_h.size * nbc)
    agree = (idx_h == flat_h).all(-1).mean()
    say(f"  blocks scored {frac:.3f}; rows equal to the flat router {agree:.4f}")
    assert np.all((idx_h >= 0).sum(-1) == min(wl.top_k, nbc))
    assert np.all(np.diff(idx_h, axis=-1) > 0) and np.all(idx_h < nbc)
    assert agree >= 0.99
    assert np.all(ev_h <= nbc)
    if keys == "clustered":
        assert frac <= 0.6
    if keys == "topical":
        assert frac <= 0.3
    rng = np.random.default_rng(1)
    for b, kv in [(int(rng.integers(wl.batch)), int(rng.integers(wl.n_kv_heads))) for _ in range(2)]:
        muo, sgo = O.block_stats(O.as_f64(Kc[b, kv, :nbc * wl.block].cpu()), wl.block)
        for h in range(kv * wl.group, (kv + 1) * wl.group):
            r = O.route_scores(O.as_f64(q[b, h].cpu()), muo, sgo, wl.beta)
            sel, rk, rk1 = O.select_topk(r, wl.top_k)
            ok, _ = idx_ok(idx_h[b, h], dict(idx=sel, scores=r, r_k=rk, r_k1=rk1))
            assert ok, f"hierarchical selection mismatch b={b} h={h}"
        say(f"  sequence {b} kv head {kv}: {wl.group} rows ok")


@pytest.mark.timeout(900)
def test_gqa_prefill_128k_backward_fullsize():
    """ssa_sparse_attn_bwd at the 128K GQA workload, called as the benchmark
    calls it (bf16 O from the forward, the same dO seed), on the GPU's own
    selections.  Checked against the oracle's per-row backward
    (attend_backward over S(t)):
      - dQ on sampled rows of every q-head;
      - dK and dV of whole blocks (an early one, a late one and the last),
        each the sum over every row that attends one of its keys: the rows
        that selected the block and the window rows reaching it.
    Tolerance: 2e-3 of the largest reference magnitude in each compared set,
    as for the small backward cases."""
    wl = CONFIGS["gqa_prefill_128k"]
    say("case gqa_prefill_128k backward: generating on the GPU")
    data = make_prefill(wl, seed=0, device=DEV)
    Q, K, V = data["Q"], data["K"], data["V"]
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx = ssa.ssa_route_topk(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k, beta=wl.beta)
    Oo, lse = ssa.ssa_sparse_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                      scale=wl.scale)
    dO = torch.randn(Q.shape, generator=torch.Generator(device=DEV).manual_seed(7), device=DEV,
                     dtype=torch.float32).to(Q.dtype)
    say("  backward")
    dQ, dK, dV = ssa.ssa_sparse_attn_bwd(Q, K, V, idx, Oo, lse, dO, block_size=wl.block,
                                         window=wl.window, scale=wl.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(dQ).all() and torch.isfinite(dK).all() and torch.isfinite(dV).all()
    idx_h = idx[0].cpu().numpy()
    del idx, Oo, lse, mu, sigma
    p = O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)
    n, B, W, g = wl.seq_len, wl.block, wl.window, wl.group
    tol = 2e-3
    kvs: dict[int, tuple] = {}

    def kv_data(kv):
        if kv not in kvs:
            kvs.clear()
            kvs[kv] = (O.as_f64(K[0, kv]), O.as_f64(V[0, kv]))
        return kvs[kv]

    # dQ on sampled rows
    rng = np.random.default_rng(3)
    rows = sorted({(int(h), int(t)) for h in range(wl.n_q_heads)
                   for t in list(rng.integers(0, n, size=1)) + [int(rng.integers(n - 300, n))]})
    got, ref = [], []
    for (h, t) in sorted(rows, key=lambda r: r[0] // g):
        Kh, Vh = kv_data(h // g)
        S = O.key_set(t, idx_h[h, t], B, W)
        dq, _, _ = O.attend_backward(O.as_f64(Q[0, h, t]), Kh, Vh, S, p.scale, O.as_f64(dO[0, h, t]))
        got.append(dQ[0, h, t].double().cpu().numpy())
        ref.append(dq)
    got, ref = np.array(got), np.array(ref)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    say(f"  dQ on {len(rows)} rows: relative error {err:.3g}")
    assert err <= tol, f"dQ relative error {err:.3g}"

    # dK, dV of whole blocks
    for kv, c in ((1, 200), (6, 450), (7, n // B - 1)):
        Kh, Vh = kv_data(kv)
        lo, hi = c * B, min(n, (c + 1) * B)
        heads = range(kv * g, (kv + 1) * g)
        sel = {(h - kv * g, int(t)) for h in heads for t in np.nonzero((idx_h[h] == c).any(axis=1))[0]}
        win = {(h - kv * g, t) for h in heads for t in range(lo, min(n, hi - 1 + W))}
        R = sorted(sel | win)
        say(f"  block {c} of KV head {kv}: {len(sel)} selecting rows, {len(R)} rows in all")
        Qg, dOg = Q[0, kv * g:(kv + 1) * g].cpu(), dO[0, kv * g:(kv + 1) * g].cpu()
        dKr = np.zeros((hi - lo, Kh.shape[1]))
        dVr = np.zeros_like(dKr)
        for (j, t) in R:
            h = kv * g + j
            S = O.key_set(t, idx_h[h, t], B, W)
            _, dk, dv = O.attend_backward(O.as_f64(Qg[j, t]), Kh, Vh, S, p.scale, O.as_f64(dOg[j, t]))
            m = (S >= lo) & (S < hi)
            dKr[S[m] - lo] += dk[m]
            dVr[S[m] - lo] += dv[m]
        for name, g_, r_ in (("dK", dK[0, kv, lo:hi], dKr), ("dV", dV[0, kv, lo:hi], dVr)):
            e = np.abs(g_.double().cpu().numpy() - r_).max() / np.abs(r_).max()
            say(f"    {name} relative error {e:.3g}")
            assert e <= tol, f"{name} of block {c}, KV head {kv}: relative error {e:.3g}"
