"""Pins of the CPU oracle against things other than itself (CPU only).

Each check is a function of the oracle implementation, so the same check can be
run against a copy of the oracle with a planted mistake (see test_mutants_*):
every check must pass on the oracle, and each plausible mistake (a dropped
term, a wrong factor, a wrong index or bound, a transposed operand) must fail
at least one of them.
"""
import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle as O
from oracle import ssa_oracle as OR

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _impl(**overrides):
    """The oracle's functions as a namespace, with some replaced (for mutants)."""
    ns = types.SimpleNamespace(
        block_stats=OR.block_stats, route_scores=OR.route_scores,
        route_scores_from_logits=OR.route_scores_from_logits, select_topk=OR.select_topk,
        routable_blocks=OR.routable_blocks, key_set=OR.key_set, attend=OR.attend,
        dropped_mass=OR.dropped_mass, recovery_weight=OR.recovery_weight,
        tempered_scores=OR.tempered_scores, tile_routable_blocks=OR.tile_routable_blocks,
        tile_scores=OR.tile_scores, attend_backward=OR.attend_backward,
        group_summaries=OR.group_summaries, group_bound=OR.group_bound, route_hier=OR.route_hier,
        kv_head=OR.kv_head)
    for k, v in overrides.items():
        setattr(ns, k, v)

    def tile_select(Qh, mu, sigma, p, j):
        n = Qh.shape[0]
        C = ns.tile_routable_blocks(j, mu.shape[0])
        R = ns.tile_scores(Qh[j * p.block:min(n, (j + 1) * p.block)], mu[:C], sigma[:C], p.beta)
        idx, r_k, r_k1 = ns.select_topk(R, p.top_k)
        return dict(idx=idx, scores=R, r_k=r_k, r_k1=r_k1)

    def tile_prefill_row(q, K, V, tile_idx, p, t):
        S = ns.key_set(t, tile_idx, p.block, p.window)
        Oo, lse = ns.attend(q, K, V, S, p.scale)
        return dict(S=S, O=Oo, lse=lse)
    ns.tile_select = tile_select
    ns.tile_prefill_row = tile_prefill_row

    def head_backward(Qh, K, V, idx_h, p, dOh):
        g, n, d = Qh.shape
        dQ, dK, dV = np.zeros((g, n, d)), np.zeros((n, d)), np.zeros((n, d))
        for j in range(g):
            for t in range(n):
                S = ns.key_set(t, idx_h[j, t], p.block, p.window)
                dq, dk, dv = ns.attend_backward(Qh[j, t], K, V, S, p.scale, dOh[j, t])
                dQ[j, t] = dq
                dK[S] += dk
                dV[S] += dv
        return dQ, dK, dV
    ns.head_backward = head_backward

    def prefill_row(q, K, V, mu, sigma, p, t, with_dense=False):
        C = ns.routable_blocks(t, p.block, mu.shape[0])
        r = ns.route_scores(q, mu[:C], sigma[:C], p.beta)
        idx, r_k, r_k1 = ns.select_topk(r, p.top_k)
        S = ns.key_set(t, idx, p.block, p.window)
        Oo, lse = ns.attend(q, K, V, S, p.scale)
        out = dict(idx=idx, scores=r, S=S, O=Oo, lse=lse)
        if with_dense:
            Of, lf = ns.attend(q, K, V, np.arange(t + 1), p.scale)
            eps, eps_d = ns.dropped_mass(q, K, S, t, p.scale)
            out.update(O_full=Of, lse_full=lf, eps=eps, eps_direct=eps_d)
        return out
    ns.prefill_row = prefill_row

    def planted_recall(Q, K, plants, p, score="cumulant"):
        hq, hkv = Q.shape[1], K.shape[1]
        hits = 0
        for pl in plants:
            Kh = OR.as_f64(K[pl["b"], ns.kv_head(pl["h"], hq, hkv)])
            mu, sigma = ns.block_stats(Kh, p.block)
            C = ns.routable_blocks(pl["t"], p.block, mu.shape[0])
            q = OR.as_f64(Q[pl["b"], pl["h"], pl["t"]])
            if score == "tempered":
                r = ns.tempered_scores(q, Kh, p.block, C, p.beta)
            else:
                r = ns.route_scores(q, mu[:C], sigma[:C], p.beta)
            idx, _, _ = ns.select_topk(r, p.top_k)
            hits += int(pl["block"] in idx.tolist())
        return hits / len(plants)
    ns.planted_recall = planted_recall
    return ns


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


# -- checks (each raises AssertionError on failure) ---------------------------

def check_golden(ns):
    g = _golden()
    rs = g["routing_score"]
    K = np.array(rs["keys"], float)
    mu, sigma = ns.block_stats(K, rs["block_size"])
    np.testing.assert_allclose(mu, rs["mu"], atol=1e-15)
    np.testing.assert_allclose(sigma, rs["sigma"], atol=1e-15)
    q = np.array(rs["q"], float)
    for beta, want in rs["scores"].items():
        r = ns.route_scores(q, mu, sigma, float(beta))
        np.testing.assert_allclose(r, want, atol=1e-12)
        idx, _, _ = ns.select_topk(r, 1)
        assert idx.tolist() == rs["top1"][beta]
    tk = g["topk_ties"]
    for case in tk["cases"]:
        idx, r_k, r_k1 = ns.select_topk(np.array(tk["scores"], float), case["k"])
        assert idx.tolist() == case["idx"]
        for got, want in ((r_k, case["r_k"]), (r_k1, case["r_k1"])):
            assert (math.isnan(got) if want is None else got == want)
    rt = g["routable"]
    for t, want in rt["cases"]:
        assert ns.routable_blocks(t, rt["block_size"], rt["n_blocks"]) == want
    ks = g["key_set"]
    for case in ks["cases"]:
        S = ns.key_set(case["t"], np.array(case["idx"]), ks["block_size"], case["window"])
        assert S.tolist() == case["keys"]
    at = g["attention"]
    for case in at["cases"]:
        Oo, lse = ns.attend(np.array(at["q"]), np.array(at["keys"], float),
                            np.array(at["values"], float), np.array([0, 1]), case["scale"])
        np.testing.assert_allclose(Oo, case["O"], atol=1e-12)
        assert abs(lse - case["lse"]) < 1e-12
    for case in g["recovery_law"]["cases"]:
        assert abs(ns.recovery_weight(case["beta"], case["delta"], case["mu"]) - case["w"]) < 1e-12
    dm = g["dropped_mass"]
    eps, eps_d = ns.dropped_mass(np.array(dm["q"], float), np.array(dm["keys"], float),
                                 np.array(dm["S"]), dm["t"], dm["scale"])
    assert abs(eps - dm["eps"]) < 1e-12 and abs(eps_d - dm["eps"]) < 1e-12


def check_stats_vs_library(ns, seed=0):
    """P1: block stats against np.mean / np.cov(bias=True); quadratic form = logit variance."""
    rng = np.random.default_rng(seed)
    B, d, nb = 16, 8, 5
    K = rng.normal(size=(nb * B + 3, d)) + rng.normal(size=(d,))
    mu, sigma = ns.block_stats(K, B)
    assert mu.shape == (nb, d) and sigma.shape == (nb, d, d)
    for c in range(nb):
        blk = K[c * B:(c + 1) * B]
        np.testing.assert_allclose(mu[c], np.mean(blk, axis=0), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sigma[c], np.cov(blk, rowvar=False, bias=True), rtol=1e-12,
                                   atol=1e-14)
        q = rng.normal(size=d)
        logits = blk @ q
        assert abs(q @ mu[c] - np.mean(logits)) <= 1e-12 * max(1, abs(np.mean(logits)))
        assert abs(q @ sigma[c] @ q - np.var(logits)) <= 1e-12 * np.var(logits)


def check_scores_two_ways(ns, seed=1):
    """P2: the covariance form of the score equals the logit-moment form."""
    rng = np.random.default_rng(seed)
    B, d, C = 32, 16, 6
    K = rng.normal(size=(C * B, d)) * rng.uniform(0.2, 2.0, size=d)
    mu, sigma = ns.block_stats(K, B)
    for beta in (0.0, 0.7, 2.0, 5.0):
        q = rng.normal(size=d)
        a = ns.route_scores(q, mu, sigma, beta)
        b = ns.route_scores_from_logits(q, K, B, C, beta)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def check_centroid_limit(ns, seed=2):
    """P3: beta = 0 ranks blocks by the centroid logit mean_j q.k_j alone."""
    rng = np.random.default_rng(seed)
    B, d, C = 8, 4, 20
    K = rng.normal(size=(C * B, d)) * 3
    mu, sigma = ns.block_stats(K, B)
    q = rng.normal(size=d)
    r = ns.route_scores(q, mu, sigma, 0.0)
    centroid = np.array([np.mean(K[c * B:(c + 1) * B] @ q) for c in range(C)])
    np.testing.assert_allclose(r, centroid, rtol=1e-12, atol=1e-12)
    idx, _, _ = ns.select_topk(r, 5)
    assert sorted(idx.tolist()) == sorted(np.argsort(-centroid, kind="stable")[:5].tolist())


def check_topk_brute(ns, seed=3):
    """P4: top-k equals the first k of Python's stable sort by (-score, index)."""
    rng = np.random.default_rng(seed)
    for trial in range(200):
        E = int(rng.integers(0, 40))
        k = int(rng.integers(0, 12))
        r = rng.integers(-3, 4, size=E).astype(float)   # many exact ties
        idx, r_k, r_k1 = ns.select_topk(r, k)
        ranked = sorted(range(E), key=lambda c: (-r[c], c))
        want = sorted(ranked[:k]) + [-1] * max(0, k - E)
        assert idx.tolist() == want, (r, k)
        want_k = r[ranked[k - 1]] if 0 < k <= E else math.nan
        want_k1 = r[ranked[k]] if k < E else math.nan
        assert (math.isnan(r_k) and math.isnan(want_k)) or r_k == want_k
        assert (math.isnan(r_k1) and math.isnan(want_k1)) or r_k1 == want_k1


def _textbook(q, K, V, mask, scale):
    """Masked-dense softmax attention, one query row."""
    s = np.where(mask, scale * (K @ q), -np.inf)
    m = s.max()
    p = np.exp(s - m)
    return (p @ V) / p.sum(), m + math.log(p.sum())


def _rand_head(rng, n, d, B):
    K = rng.normal(size=(n, d)) + np.repeat(rng.normal(size=(-(-n // B), d)), B, 0)[:n]
    return rng.normal(size=(n, d)), K, rng.normal(size=(n, d))


def check_dense_reduction(ns, seed=4):
    """P5: k >= nb with W >= B-1 is dense causal attention (textbook and torch SDPA)."""
    rng = np.random.default_rng(seed)
    for (n, d, B, W) in ((67, 8, 8, 7), (64, 4, 16, 16), (50, 6, 5, 9)):
        Q, K, V = _rand_head(rng, n, d, B)
        mu, sigma = ns.block_stats(K, B)
        nb = n // B
        scale = 1 / math.sqrt(d)
        p = O.Params(B, nb + 2, W, 2.0, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q)[None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None],
            is_causal=True, scale=scale)[0, 0].numpy()
        for t in range(n):
            row = ns.prefill_row(Q[t], K, V, mu, sigma, p, t, with_dense=True)
            assert row["S"].tolist() == list(range(t + 1))
            tb, tl = _textbook(Q[t], K, V, np.arange(n) <= t, scale)
            np.testing.assert_allclose(row["O"], tb, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(row["O"], ref[t], rtol=1e-12, atol=1e-12)
            assert abs(row["lse"] - tl) < 1e-12
            assert abs(row["eps"]) < 1e-12 and abs(row["eps_direct"]) < 1e-12


def check_window_only(ns, seed=5):
    """P6: k = 0 is sliding-window attention of width W (banded causal mask)."""
    rng = np.random.default_rng(seed)
    n, d, B = 45, 5, 8
    Q, K, V = _rand_head(rng, n, d, B)
    mu, sigma = ns.block_stats(K, B)
    for W in (1, 3, 8, 13):
        p = O.Params(B, 0, W, 2.0, 0.37)
        for t in range(n):
            row = ns.prefill_row(Q[t], K, V, mu, sigma, p, t)
            j = np.arange(n)
            tb, tl = _textbook(Q[t], K, V, (j <= t) & (j > t - W), 0.37)
            np.testing.assert_allclose(row["O"], tb, rtol=1e-12, atol=1e-12)
            assert abs(row["lse"] - tl) < 1e-12


def check_gather_equals_mask(ns, seed=6):
    """P7: attention over the gathered S(t) equals masked-dense attention with M[t,j] = [j in S(t)]."""
    rng = np.random.default_rng(seed)
    n, d, B, W = 96, 8, 8, 5
    Q, K, V = _rand_head(rng, n, d, B)
    mu, sigma = ns.block_stats(K, B)
    p = O.Params(B, 3, W, 2.0, 0.3)
    for t in range(0, n, 7):
        row = ns.prefill_row(Q[t], K, V, mu, sigma, p, t)
        j = np.arange(n)
        blocks = [c for c in row["idx"].tolist() if c >= 0]
        mask = np.isin(j // B, blocks) | ((j <= t) & (j > t - W))
        # every selected block is complete and causal, so the mask needs no j <= t clip
        assert all((c + 1) * B - 1 <= t for c in blocks)
        tb, tl = _textbook(Q[t], K, V, mask, 0.3)
        np.testing.assert_allclose(row["O"], tb, rtol=1e-12, atol=1e-12)
        assert abs(row["lse"] - tl) < 1e-12


def check_recovery_law(ns):
    """P8: target with margin Delta over mu equal distractors gets weight sigma(beta*Delta - log mu)."""
    d = 3
    for mu_count in (1, 7, 63, 511):
        for delta in (-2.0, -0.5, 0.0, 0.3, 1.0, 4.0, 9.0):
            for beta in (0.125, 1 / math.sqrt(128), 1.0, 2.0):
                # bare softmax over [target, distractors]: logits beta*(s + Delta), beta*s
                s0 = 0.7
                logits = np.array([beta * (s0 + delta)] + [beta * s0] * mu_count)
                w = np.exp(logits - logits.max())
                w = w[0] / w.sum()
                law = ns.recovery_weight(beta, delta, mu_count)
                assert abs(w - law) < 1e-12
                # through attention: q.k* = s0+Delta, q.k = s0, V one-hot on the target
                q = np.array([1.0, 0.0, 0.0])
                K = np.zeros((mu_count + 1, d))
                K[0, 0] = s0 + delta
                K[1:, 0] = s0
                K[1:, 1] = np.linspace(-1, 1, mu_count)  # orthogonal to q: logits unchanged
                V = np.zeros((mu_count + 1, d))
                V[0, 2] = 1.0
                Oo, _ = ns.attend(q, K, V, np.arange(mu_count + 1), beta)
                assert abs(Oo[2] - law) < 1e-12


def check_recovery_law_pipeline(ns):
    """P8 through the full row: the planted target and its block-mates as the selected set."""
    B, d = 8, 4
    mu_count = 2 * B - 1            # distractors: the other keys of the two selected blocks
    n = 4 * B
    beta_soft, delta = 0.5, 3.0
    q = np.array([1.0, 0, 0, 0])
    K = np.zeros((n, d))
    K[:, 0] = -50.0                  # keys outside the selected blocks: far below
    K[:2 * B, 0] = 1.0               # blocks 0 and 1: distractors at logit 1 (before scale)
    K[:2 * B, 1] = np.linspace(-3, 3, 2 * B)   # routing spread, orthogonal to q
    K[5, 0] = 1.0 + delta            # the target in block 0
    V = np.zeros((n, d))
    V[5, 3] = 1.0
    mu, sigma = ns.block_stats(K, B)
    t = n - 1
    p = O.Params(B, 2, 1, 2.0, beta_soft)
    # make the window key (t) a distractor-free position: give it a very low logit
    row = ns.prefill_row(q, K, V, mu, sigma, p, t, with_dense=False)
    assert row["idx"].tolist() == [0, 1]
    # S = blocks 0,1 plus window {t} whose logit is -50: weight ~ e^-25 relative
    law = ns.recovery_weight(beta_soft, delta, mu_count)
    assert abs(row["O"][3] - law) < 1e-9


def check_dropped_mass(ns, seed=7):
    """P9: eps two ways agree, lie in [0, 1], and bound ||O_S - O_full||_inf <= 2 eps max|v|."""
    rng = np.random.default_rng(seed)
    n, d, B, W = 128, 8, 16, 4
    Q, K, V = _rand_head(rng, n, d, B)
    mu, sigma = ns.block_stats(K, B)
    p = O.Params(B, 2, W, 2.0, 0.4)
    for t in range(0, n, 5):
        row = ns.prefill_row(Q[t], K, V, mu, sigma, p, t, with_dense=True)
        assert -1e-15 <= row["eps"] <= 1 and abs(row["eps"] - row["eps_direct"]) < 1e-12
        bound = 2 * row["eps"] * np.abs(V[: t + 1]).max()
        assert np.abs(row["O"] - row["O_full"]).max() <= bound + 1e-12


def check_decode_equals_prefill(ns, seed=8):
    """P10: the decode step at t = L equals prefill row L over the same L+1 keys."""
    rng = np.random.default_rng(seed)
    d, B, W = 6, 8, 5
    for L in (0, 7, 8, 31, 40):
        Q, K, V = _rand_head(rng, L + 1, d, B)
        p = O.Params(B, 2, W, 2.0, 0.5)
        dec = O.decode_step(Q[L], K[L], V[L], K[:L], V[:L], L, p)
        mu, sigma = ns.block_stats(K, B)
        pre = ns.prefill_row(Q[L], K, V, mu, sigma, p, L)
        assert dec["idx"].tolist() == pre["idx"].tolist()
        np.testing.assert_allclose(dec["O"], pre["O"], rtol=1e-12, atol=1e-14)
        assert abs(dec["lse"] - pre["lse"]) < 1e-12


def check_invariances(ns, seed=9):
    """P11: permuting keys (with values) inside a block changes nothing; a constant
    added to every logit leaves O unchanged and shifts LSE by that constant."""
    rng = np.random.default_rng(seed)
    n, d, B, W = 80, 6, 16, 6
    Q, K, V = _rand_head(rng, n, d, B)
    mu, sigma = ns.block_stats(K, B)
    perm = np.arange(n)
    for c in range(n // B):
        perm[c * B:(c + 1) * B] = c * B + rng.permutation(B)
    K2, V2 = K[perm], V[perm]
    mu2, sigma2 = ns.block_stats(K2, B)
    np.testing.assert_allclose(mu2, mu, atol=1e-13)
    np.testing.assert_allclose(sigma2, sigma, atol=1e-13)
    p = O.Params(B, 2, W, 2.0, 0.45)
    for t in range(B * 2 + 3, n, 9):     # windows away from permuted rows of the tail
        a = ns.prefill_row(Q[t], K, V, mu, sigma, p, t)
        # keep the window identical: only permute complete blocks strictly before the window
        wstart = t - W + 1
        ok = perm.copy()
        ok[wstart // B * B:] = np.arange(wstart // B * B, n)
        b = ns.prefill_row(Q[t], K[ok], V[ok], *ns.block_stats(K[ok], B), p, t)
        assert a["idx"].tolist() == b["idx"].tolist()
        np.testing.assert_allclose(a["O"], b["O"], rtol=1e-12, atol=1e-13)
    # constant logit shift via an extra coordinate: q' = [q, c/scale], k' = [k, 1]
    cshift = 1.7
    scale = 0.45
    Ka = np.concatenate([K, np.ones((n, 1))], 1)
    t = n - 1
    S = np.arange(0, n, 3)
    O1, l1 = ns.attend(Q[t], K, V, S, scale)
    O2, l2 = ns.attend(np.concatenate([Q[t], [cshift / scale]]), Ka, V, S, scale)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-13)
    assert abs((l2 - l1) - cshift) < 1e-12


def check_tempered_closed_form(ns):
    """Tempered score on hand-worked blocks (golden): two keys whose scaled
    logits 0 and ln 3 average to exp-mean 2 give ln(2)/beta; equal logits give
    the logit for every beta."""
    ts = _golden()["tempered_score"]
    q = np.zeros(4)
    q[0] = 1.0
    for case in ts["cases"]:
        K = np.zeros((2, 4))
        K[1, 0] = case["a"]
        T = ns.tempered_scores(q, K, 2, 1, case["beta"])
        assert abs(T[0] - case["T"]) < 1e-12, (case, T)
    cl = ts["constant_logits"]
    K = np.zeros((8, 4))
    K[:, 0] = cl["s"]
    for beta in cl["betas"]:
        T = ns.tempered_scores(q, K, 4, 2, beta)
        np.testing.assert_allclose(T, [cl["s"], cl["s"]], rtol=0, atol=1e-12)


def check_tempered_limits(ns, seed=7):
    """Tempered score against the logit moments (NumPy mean/var/max): beta -> 0
    gives the block mean, the O(beta^2) remainder of mean + (beta/2) var, the
    bound max - ln(B)/beta <= T <= max, and monotonicity in beta."""
    rng = np.random.default_rng(seed)
    B, d, C = 16, 8, 3
    K = rng.normal(size=(C * B, d))
    q = rng.normal(size=d)
    logits = [K[c * B:(c + 1) * B] @ q for c in range(C)]
    mean = np.array([np.mean(s) for s in logits])
    var = np.array([np.var(s) for s in logits])
    mx = np.array([np.max(s) for s in logits])
    np.testing.assert_allclose(ns.tempered_scores(q, K, B, C, 1e-9), mean, rtol=0, atol=1e-6)
    e2 = np.abs(ns.tempered_scores(q, K, B, C, 1e-2) - (mean + 0.5e-2 * var))
    e3 = np.abs(ns.tempered_scores(q, K, B, C, 1e-3) - (mean + 0.5e-3 * var))
    assert np.all(e2 < 1e-2) and np.all(e3 <= e2 / 30 + 1e-12), (e2, e3)
    for beta in (50.0, 1e3):
        T = ns.tempered_scores(q, K, B, C, beta)
        assert np.all(T <= mx + 1e-12) and np.all(T >= mx - math.log(B) / beta - 1e-12)
    prev = None
    for beta in (0.1, 0.5, 1.0, 2.0, 4.0, 8.0):
        T = ns.tempered_scores(q, K, B, C, beta)
        if prev is not None:
            assert np.all(T >= prev - 1e-12)
        prev = T


def check_tile_scores_moments(ns, seed=11):
    """Tile score two ways: the sum over the tile's rows of the logit moments
    (NumPy mean and population variance of q_t.k_j over each block, no block
    statistics) and the closed form s.mu_c + (beta/2) <Sigma_c, M> with
    s = sum_t q_t and M = sum_t q_t q_t^T."""
    rng = np.random.default_rng(seed)
    for (T, d, B, C, beta) in ((5, 6, 8, 4, 2.0), (1, 3, 4, 3, 0.7), (9, 4, 16, 2, 5.0)):
        Qt = rng.normal(size=(T, d))
        K = rng.normal(size=(C * B, d)) + rng.normal(size=(C, 1, d)).repeat(B, 1).reshape(C * B, d)
        mu, sigma = ns.block_stats(K, B)
        R = ns.tile_scores(Qt, mu, sigma, beta)
        want = np.zeros(C)
        for c in range(C):
            L = Qt @ K[c * B:(c + 1) * B].T          # [T, B] logits
            want[c] = np.sum(np.mean(L, axis=1) + 0.5 * beta * np.var(L, axis=1))
        np.testing.assert_allclose(R, want, rtol=1e-12, atol=1e-11)
        s_, M = Qt.sum(0), Qt.T @ Qt
        closed = np.array([s_ @ mu[c] + 0.5 * beta * np.sum(sigma[c] * M) for c in range(C)])
        np.testing.assert_allclose(R, closed, rtol=1e-12, atol=1e-11)


def check_tile_select_brute(ns, seed=12):
    """The tile's selection is the k-subset of routable blocks with the largest
    total routing score over the tile's rows (brute force over subsets, scores
    from the raw logits), and no block at or after the tile is routable."""
    import itertools
    rng = np.random.default_rng(seed)
    n, d, B = 70, 4, 8
    Q, K, _ = _rand_head(rng, n, d, B)
    mu, sigma = ns.block_stats(K, B)
    nb = n // B
    for k in (1, 2, 3):
        p = O.Params(B, k, B, 2.0, 0.5)
        for j in range(0, (n + B - 1) // B):
            sel = ns.tile_select(Q, mu, sigma, p, j)
            rows = Q[j * B:min(n, (j + 1) * B)]
            C = min(j, nb)
            total = np.zeros(C)
            for c in range(C):
                L = rows @ K[c * B:(c + 1) * B].T
                total[c] = np.sum(np.mean(L, 1) + np.var(L, 1))   # beta / 2 = 1
            got = [c for c in sel["idx"].tolist() if c >= 0]
            assert all(c < j for c in got), (j, got)
            assert len(got) == min(k, C)
            if C:
                best = max(itertools.combinations(range(C), min(k, C)),
                           key=lambda S: sum(total[c] for c in S))
                assert sorted(best) == got, (j, k, got, best)


def check_tile_single_row(ns, seed=13):
    """A tile holding one query (position jB) selects what that row selects by
    itself: the tile's routable blocks are exactly the row's."""
    rng = np.random.default_rng(seed)
    d, B = 5, 8
    for j in (0, 1, 3, 6):
        n = j * B + 1
        Q, K, V = _rand_head(rng, n, d, B)
        mu, sigma = ns.block_stats(K, B)
        p = O.Params(B, 2, 4, 2.0, 0.4)
        tile = ns.tile_select(Q, mu, sigma, p, j)
        row = ns.prefill_row(Q[j * B], K, V, mu, sigma, p, j * B)
        assert tile["idx"].tolist() == row["idx"].tolist(), (j, tile["idx"], row["idx"])
        np.testing.assert_allclose(tile["scores"], row["scores"], rtol=1e-12, atol=1e-12)


def check_tile_dense_reduction(ns, seed=14):
    """k >= nb and W >= B: every row of every tile attends to all keys <= t,
    i.e. dense causal attention (torch SDPA, CPU float64)."""
    rng = np.random.default_rng(seed)
    for (n, d, B, W) in ((67, 8, 8, 8), (50, 6, 5, 9)):
        Q, K, V = _rand_head(rng, n, d, B)
        mu, sigma = ns.block_stats(K, B)
        scale = 1 / math.sqrt(d)
        p = O.Params(B, n // B + 2, W, 2.0, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q)[None, None], torch.tensor(K)[None, None], torch.tensor(V)[None, None],
            is_causal=True, scale=scale)[0, 0].numpy()
        for j in range((n + B - 1) // B):
            sel = ns.tile_select(Q, mu, sigma, p, j)
            for t in range(j * B, min(n, (j + 1) * B)):
                row = ns.tile_prefill_row(Q[t], K, V, sel["idx"], p, t)
                assert row["S"].tolist() == list(range(t + 1)), (t, row["S"])
                np.testing.assert_allclose(row["O"], ref[t], rtol=1e-12, atol=1e-12)


def _bwd_case(rng, g=2, n=40, d=4, B=8, k=2, W=5):
    Q = rng.normal(size=(g, n, d))
    K = rng.normal(size=(n, d)) + np.repeat(rng.normal(size=(n // B + 1, d)), B, 0)[:n]
    V = rng.normal(size=(n, d))
    dO = rng.normal(size=(g, n, d))
    mu, sigma = OR.block_stats(K, B)
    p = O.Params(B, k, W, 2.0, 0.6)
    idx = np.stack([np.stack([OR.prefill_row(Q[j, t], K, V, mu, sigma, p, t)["idx"]
                              for t in range(n)]) for j in range(g)])
    return Q, K, V, dO, idx, p


def _forward_loss(Q, K, V, dO, idx, p):
    """L = sum_t dO_t . O_t with the selections fixed (forward by the textbook
    masked-dense softmax, independent of the oracle's attend)."""
    g, n, _ = Q.shape
    L = 0.0
    for j in range(g):
        for t in range(n):
            S = set(OR.key_set(t, idx[j, t], p.block, p.window).tolist())
            mask = np.array([jj in S for jj in range(n)])
            o, _ = _textbook(Q[j, t], K, V, mask, p.scale)
            L += float(dO[j, t] @ o)
    return L


def check_backward_finite_differences(ns, seed=15):
    """Central differences of L = sum dO.O against the gradients, in every
    coordinate of a few q, k and v entries (selections held fixed)."""
    rng = np.random.default_rng(seed)
    Q, K, V, dO, idx, p = _bwd_case(rng)
    dQ, dK, dV = ns.head_backward(Q, K, V, idx, p, dO)
    h = 1e-6
    for (name, X, G) in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        flat = X.reshape(-1)
        gflat = G.reshape(-1)
        for i in rng.choice(flat.size, size=12, replace=False):
            old = flat[i]
            flat[i] = old + h
            lp = _forward_loss(Q, K, V, dO, idx, p)
            flat[i] = old - h
            lm = _forward_loss(Q, K, V, dO, idx, p)
            flat[i] = old
            num = (lp - lm) / (2 * h)
            assert abs(num - gflat[i]) <= 1e-6 * max(1.0, abs(num)), (name, int(i), num, gflat[i])


def check_backward_autograd(ns, seed=16):
    """Gradients against torch autograd (CPU, float64) of the masked-dense
    formulation with the mask M[t, j] = [j in S(t)], GQA heads sharing K, V."""
    rng = np.random.default_rng(seed)
    Q, K, V, dO, idx, p = _bwd_case(rng, g=3, n=33, d=5, B=4, k=3, W=3)
    g, n, d = Q.shape
    M = np.zeros((g, n, n), dtype=bool)
    for j in range(g):
        for t in range(n):
            M[j, t, OR.key_set(t, idx[j, t], p.block, p.window)] = True
    Qt = torch.tensor(Q, requires_grad=True)
    Kt = torch.tensor(K, requires_grad=True)
    Vt = torch.tensor(V, requires_grad=True)
    sc = (Qt @ Kt.T) * p.scale
    sc = sc.masked_fill(~torch.tensor(M), float("-inf"))
    Ot = torch.softmax(sc, -1) @ Vt
    (Ot * torch.tensor(dO)).sum().backward()
    dQ, dK, dV = ns.head_backward(Q, K, V, idx, p, dO)
    np.testing.assert_allclose(dQ, Qt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, Kt.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, Vt.grad.numpy(), rtol=1e-10, atol=1e-12)


def check_backward_dense(ns, seed=17):
    """k >= nb and W >= B: the gradients are dense causal attention's (torch
    SDPA backward, CPU float64)."""
    rng = np.random.default_rng(seed)
    n, d, B = 30, 4, 6
    Q = rng.normal(size=(1, n, d))
    K = rng.normal(size=(n, d))
    V = rng.normal(size=(n, d))
    dO = rng.normal(size=(1, n, d))
    p = O.Params(B, n // B + 1, B, 2.0, 0.5)
    idx = np.array([[sorted(list(range(min(n // B, (t + 1) // B)))) +
                     [-1] * (p.top_k - min(n // B, (t + 1) // B)) for t in range(n)]])
    Qt = torch.tensor(Q[None], requires_grad=True)
    Kt = torch.tensor(K[None, None], requires_grad=True)
    Vt = torch.tensor(V[None, None], requires_grad=True)
    Ot = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, is_causal=True, scale=0.5)
    (Ot * torch.tensor(dO[None])).sum().backward()
    dQ, dK, dV = ns.head_backward(Q, K, V, idx, p, dO)
    np.testing.assert_allclose(dQ, Qt.grad[0].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dK, Kt.grad[0, 0].numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dV, Vt.grad[0, 0].numpy(), rtol=1e-10, atol=1e-12)


def _clustered(rng, nb, m, B, d, group_std=3.0, block_std=0.1, noise=0.3):
    G = -(-nb // m)
    gc = rng.normal(size=(G, d)) * group_std
    bc = np.repeat(gc, m, 0)[:nb] + rng.normal(size=(nb, d)) * block_std
    return np.repeat(bc, B, 0) + rng.normal(size=(nb * B, d)) * noise


def check_group_bound_admissible(ns, seed=18):
    """UB_G(q) >= every member's score (brute force over random queries, random
    and clustered keys, beta in {0, 0.5, 2, 8}), and lam_G >= the spectral norm
    of every member's Sigma_c - S_G (NumPy eigvalsh)."""
    rng = np.random.default_rng(seed)
    for geo in ("random", "clustered"):
        B, d, nb, m = 6, 5, 22, 4
        K = rng.normal(size=(nb * B, d)) if geo == "random" else _clustered(rng, nb, m, B, d)
        mu, sigma = ns.block_stats(K, B)
        gs = ns.group_summaries(mu, sigma, m)
        for gi in range(gs["mu"].shape[0]):
            for c in range(gi * m, min(nb, (gi + 1) * m)):
                spec = np.abs(np.linalg.eigvalsh(sigma[c] - gs["S"][gi])).max()
                assert gs["lam"][gi] >= spec - 1e-12
                assert np.linalg.norm(mu[c] - gs["mu"][gi]) <= gs["R"][gi] + 1e-12
        for beta in (0.0, 0.5, 2.0, 8.0):
            for _ in range(40):
                q = rng.normal(size=d) * rng.uniform(0.2, 3.0)
                ub = ns.group_bound(q, gs, beta)
                r = OR.route_scores(q, mu, sigma, beta)
                for gi in range(gs["mu"].shape[0]):
                    assert ub[gi] >= r[gi * m:(gi + 1) * m].max() - 1e-9, (geo, beta, gi)


def check_route_hier_exact(ns, seed=19):
    """Branch and bound returns the flat top-k (select_topk over all routable
    scores) for random and clustered keys, every k, partial routable ranges;
    on the clustered keys it evaluates fewer blocks than exist."""
    rng = np.random.default_rng(seed)
    B, d, nb, m = 4, 6, 40, 5
    pruned = 0
    for geo in ("random", "clustered"):
        K = rng.normal(size=(nb * B, d)) if geo == "random" else _clustered(rng, nb, m, B, d)
        mu, sigma = ns.block_stats(K, B)
        gs = ns.group_summaries(mu, sigma, m)
        for trial in range(60):
            q = rng.normal(size=d)
            k = int(rng.integers(0, 9))
            C = int(rng.integers(0, nb + 1))
            out = ns.route_hier(q, mu, sigma, gs, m, k, 2.0, C)
            want, _, _ = OR.select_topk(OR.route_scores(q, mu[:C], sigma[:C], 2.0), k)
            assert out["idx"].tolist() == want.tolist(), (geo, k, C, out, want)
            assert out["evaluated"] <= C
            if geo == "clustered" and k > 0 and out["evaluated"] < C:
                pruned += 1
    assert pruned > 20, pruned


def check_route_hier_hand(ns):
    """Hand-worked pruning: groups of identical blocks (R = lam = 0, so the bound
    is the score).  Scores (q = e_1, beta = 0): group 0 blocks 1, group 1
    blocks 5, group 2 blocks 3, m = 2.  k = 2 visits group 1 (bound 5, two
    blocks evaluated), then prunes group 2 (3 < 5) and group 0 (1 < 5).  Then a
    tie: group 0 blocks 2 (bound 2), group 1 blocks {3, 2} (bound 3 + radius);
    with k = 2 the second pick is block 0 (score 2, lower index than block 3),
    which a prune on equality (2 <= tau = 2) would lose."""
    d, B = 3, 2
    def blocks(vals):
        K = np.zeros((len(vals) * B, d))
        for c, v in enumerate(vals):
            K[c * B:(c + 1) * B, 0] = v
        return K
    q = np.array([1.0, 0.0, 0.0])
    K = blocks([1, 1, 5, 5, 3, 3])
    mu, sigma = ns.block_stats(K, B)
    gs = ns.group_summaries(mu, sigma, 2)
    out = ns.route_hier(q, mu, sigma, gs, 2, 2, 0.0, 6)
    assert out["idx"].tolist() == [2, 3] and out["evaluated"] == 2, out
    K = blocks([2, 2, 3, 2])
    mu, sigma = ns.block_stats(K, B)
    gs = ns.group_summaries(mu, sigma, 2)
    out = ns.route_hier(q, mu, sigma, gs, 2, 2, 0.0, 4)
    assert out["idx"].tolist() == [0, 2], out


def check_planted_recall_hand(ns):
    """Hand-worked planted recall, B = 2, d = 2, n = 4, four query heads on two
    KV heads (heads 0, 1 read KV head 0; heads 2, 3 KV head 1), every query
    row at t = 3 equal to q = (1, 0), k = 1.  KV head 0: block 0 keys (3, 0)
    and (-3, 0) (mu = 0, Sigma = diag(9, 0)), block 1 keys (1, 0) twice
    (mu = (1, 0), Sigma = 0); KV head 1 the same blocks swapped.  Cumulant
    scores: the spread block 4.5 beta, the tight block 1, so beta = 2 picks the
    spread block and beta in {0, 0.2} the tight one.  Tempered scores: the
    spread block log(cosh 3 beta) / beta (2.653 at beta = 2, 0.443 at
    beta = 0.1), the tight block 1.  Plants (head, block) (1, 0), (2, 1),
    (0, 1): recall 2/3 where the spread block wins, 1/3 where the tight one
    does; reading KV head h % 2 instead of h // 2 gives 0 at beta = 2."""
    Q = np.zeros((1, 4, 4, 2))
    Q[0, :, 3] = [1.0, 0.0]
    K = np.zeros((1, 2, 4, 2))
    K[0, 0] = [[3, 0], [-3, 0], [1, 0], [1, 0]]
    K[0, 1] = [[1, 0], [1, 0], [3, 0], [-3, 0]]
    plants = [dict(b=0, h=1, t=3, block=0), dict(b=0, h=2, t=3, block=1),
              dict(b=0, h=0, t=3, block=1)]
    for beta, score, want in ((2.0, "cumulant", 2 / 3), (0.0, "cumulant", 1 / 3),
                              (0.2, "cumulant", 1 / 3), (2.0, "tempered", 2 / 3),
                              (0.1, "tempered", 1 / 3)):
        got = ns.planted_recall(Q, K, plants, O.Params(2, 1, 1, beta, 1.0), score)
        assert abs(got - want) < 1e-15, (beta, score, got, want)


def check_gqa_dense_sdpa(ns, seed=23):
    """k >= nb and W >= B under GQA (8 query heads on 2 KV heads): every row's
    output is dense causal attention as torch's SDPA computes it with
    enable_gqa (CPU, float64), which pins the query-head -> KV-head map."""
    rng = np.random.default_rng(seed)
    hq, hkv, n, d, B = 8, 2, 20, 4, 4
    Q = rng.normal(size=(1, hq, n, d))
    K = rng.normal(size=(1, hkv, n, d))
    V = rng.normal(size=(1, hkv, n, d))
    p = O.Params(B, n // B + 1, B, 2.0, 0.5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Q), torch.tensor(K), torch.tensor(V), is_causal=True, scale=0.5,
        enable_gqa=True).numpy()
    for h in range(hq):
        kv = ns.kv_head(h, hq, hkv)
        mu, sigma = ns.block_stats(K[0, kv], B)
        for t in range(n):
            row = ns.prefill_row(Q[0, h, t], K[0, kv], V[0, kv], mu, sigma, p, t)
            np.testing.assert_allclose(row["O"], ref[0, h, t], rtol=1e-10, atol=1e-12)


CHECKS = [check_golden, check_stats_vs_library, check_scores_two_ways, check_centroid_limit,
          check_topk_brute, check_dense_reduction, check_window_only, check_gather_equals_mask,
          check_recovery_law, check_recovery_law_pipeline, check_dropped_mass,
          check_decode_equals_prefill, check_invariances, check_tempered_closed_form,
          check_tempered_limits, check_tile_scores_moments, check_tile_select_brute,
          check_tile_single_row, check_tile_dense_reduction, check_backward_finite_differences,
          check_backward_autograd, check_backward_dense, check_group_bound_admissible,
          check_route_hier_exact, check_route_hier_hand, check_planted_recall_hand,
          check_gqa_dense_sdpa]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(_impl())


# -- planted mistakes: each must be caught by at least one check ----------------

def _mut_sample_cov(K, B):
    mu, sigma = OR.block_stats(K, B)
    return mu, sigma * B / (B - 1)


def _mut_full_beta(q, mu, sigma, beta):
    return OR.route_scores(q, mu, sigma, 2 * beta)


def _mut_no_var(q, mu, sigma, beta):
    return OR.route_scores(q, mu, sigma, 0.0)


def _mut_minus_var(q, mu, sigma, beta):
    return OR.route_scores(q, mu, sigma, -beta)


def _mut_topk_high_ties(r, k):
    r = np.asarray(r, float)
    E = len(r)
    order = np.lexsort((-np.arange(E), -r))
    idx = np.full(k, -1, np.int32)
    idx[:min(k, E)] = np.sort(order[:min(k, E)])
    return idx, (r[order[k - 1]] if 0 < k <= E else math.nan), (r[order[k]] if k < E else math.nan)


def _mut_routable_partial(t, B, nb):
    return max(0, min(nb, t // B + 1))


def _mut_window_exclusive(t, idx, B, W):
    S = OR.key_set(t, idx, B, W)
    return S[S != t] if len(S) > 1 else S


def _mut_window_wide(t, idx, B, W):
    return OR.key_set(t, idx, B, W + 1)


def _mut_attend_noscale(q, K, V, S, scale):
    return OR.attend(q, K, V, S, 1.0)


def _mut_attend_transposed_v(q, K, V, S, scale):
    Oo, lse = OR.attend(q, K, V, S, scale)
    Vs = np.asarray(V, float)[S]
    s = scale * (np.asarray(K, float)[S] @ np.asarray(q, float))
    p = np.exp(s - s.max())
    p /= p.sum()
    d = Vs.shape[1]
    if Vs.shape[0] >= d:
        Oo = Vs[:d, :].T @ p[:d]   # reads V with its roles swapped on a square slice
    return Oo, lse


def _mut_stats_transposed(K, B):
    K = np.asarray(K, float)
    n, d = K.shape
    nb = n // B
    mu = np.zeros((nb, d))
    sigma = np.zeros((nb, d, d))
    for c in range(nb):
        blk = K[c * B:(c + 1) * B]
        mu[c] = blk.mean(0)
        X = blk - mu[c]
        sigma[c] = (X.T @ X) / B
        sigma[c] = np.triu(sigma[c]) + np.triu(sigma[c], 1).T * 0.5   # loses symmetry
    return mu, sigma


def _mut_recovery_sign(beta, delta, mu):
    return 1 / (1 + math.exp(-(beta * delta + math.log(mu))))


def _mut_dropped_swapped(q, K, S, t, scale):
    a, b = OR.dropped_mass(q, K, S, t, scale)
    return 1 - a, b


def _mut_tempered_log_sum(q, K, B, C, beta):
    return OR.tempered_scores(q, K, B, C, beta) + math.log(B) / beta


def _mut_tempered_undivided(q, K, B, C, beta):
    return OR.tempered_scores(q, K, B, C, beta) * beta


def _mut_tempered_max(q, K, B, C, beta):
    K = np.asarray(K, float)
    return np.array([np.max(K[c * B:(c + 1) * B] @ q) for c in range(C)])


def _mut_tempered_neg_beta(q, K, B, C, beta):
    return -OR.tempered_scores(-np.asarray(q, float), K, B, C, beta)


def _mut_tile_own_block(j, nb):
    return max(0, min(nb, j + 1))


def _mut_tile_first_row(Qt, mu, sigma, beta):
    return OR.tile_scores(np.asarray(Qt)[:1], mu, sigma, beta)


def _mut_tile_max_row(Qt, mu, sigma, beta):
    return np.max([OR.route_scores(q, mu, sigma, beta) for q in OR.as_f64(Qt)], axis=0)


def _mut_tile_no_variance(Qt, mu, sigma, beta):
    return OR.tile_scores(Qt, mu, sigma, 0.0)


def _mut_bwd_no_D(q, K, V, S, scale, dO):
    dq, dK, dV = OR.attend_backward(q, K, V, S, scale, dO)
    Ks = OR.as_f64(K)[S]
    s_ = scale * (Ks @ OR.as_f64(q))
    p_ = np.exp(s_ - s_.max())
    p_ /= p_.sum()
    dS = p_ * (OR.as_f64(V)[S] @ OR.as_f64(dO))       # the -D term dropped
    return scale * (dS @ Ks), scale * np.outer(dS, OR.as_f64(q)), dV


def _mut_bwd_dk_unscaled(q, K, V, S, scale, dO):
    dq, dK, dV = OR.attend_backward(q, K, V, S, scale, dO)
    return dq, dK / scale, dV


def _mut_bwd_dv_unnormalised(q, K, V, S, scale, dO):
    dq, dK, dV = OR.attend_backward(q, K, V, S, scale, dO)
    s_ = scale * (OR.as_f64(K)[S] @ OR.as_f64(q))
    w = np.exp(s_ - s_.max())
    return dq, dK, np.outer(w, OR.as_f64(dO))


def _mut_bwd_dq_uses_v(q, K, V, S, scale, dO):
    dq, dK, dV = OR.attend_backward(q, K, V, S, scale, dO)
    return OR.attend_backward(q, V, V, S, scale, dO)[0], dK, dV


def _mut_bound_no_radius(q, gs, beta):
    g2 = dict(gs)
    g2["R"] = np.zeros_like(gs["R"])
    return OR.group_bound(q, g2, beta)


def _mut_bound_no_lam(q, gs, beta):
    g2 = dict(gs)
    g2["lam"] = np.zeros_like(gs["lam"])
    return OR.group_bound(q, g2, beta)


def _mut_hier_prune_on_equal(q, mu, sigma, gs, m, k, beta, C):
    ub = OR.group_bound(q, gs, beta)
    G = -(-C // m)
    scores = {}
    for gi in sorted(range(G), key=lambda x: (-ub[x], x)):
        if k == 0:
            break
        if len(scores) >= k and ub[gi] <= sorted(scores.values(), reverse=True)[k - 1]:
            continue
        blocks = list(range(gi * m, min(C, (gi + 1) * m)))
        scores.update(zip(blocks, OR.route_scores(q, OR.as_f64(mu)[blocks],
                                                  OR.as_f64(sigma)[blocks], beta).tolist()))
    cs = np.array(sorted(scores), dtype=np.int64)
    sel, _, _ = OR.select_topk(np.array([scores[c] for c in cs]), k)
    idx = np.full(k, -1, dtype=np.int32)
    ch = np.sort(cs[sel[sel >= 0]]) if cs.size else np.zeros(0, dtype=np.int64)
    idx[:ch.size] = ch
    return dict(idx=idx, evaluated=len(scores))


def _mut_hier_bound_unused(q, mu, sigma, gs, m, k, beta, C):
    # a route_hier whose bounds come from the mutated group_bound in ns is
    # exercised by the other mutants; this one ignores the group order
    out = OR.route_hier(q, mu, sigma, gs, m, k, beta, C)
    out["evaluated"] = C
    return out


def _mut_kv_head_modulo(h, hq, hkv):
    return h % hkv


MUTANTS = {
    "sample_covariance": dict(block_stats=_mut_sample_cov),
    "beta_not_halved": dict(route_scores=_mut_full_beta),
    "variance_term_dropped": dict(route_scores=_mut_no_var),
    "variance_sign_flipped": dict(route_scores=_mut_minus_var),
    "ties_to_higher_index": dict(select_topk=_mut_topk_high_ties),
    "partial_block_routable": dict(routable_blocks=_mut_routable_partial),
    "window_excludes_t": dict(key_set=_mut_window_exclusive),
    "window_off_by_one": dict(key_set=_mut_window_wide),
    "softmax_scale_dropped": dict(attend=_mut_attend_noscale),
    "values_transposed": dict(attend=_mut_attend_transposed_v),
    "covariance_asymmetric": dict(block_stats=_mut_stats_transposed),
    "recovery_sign": dict(recovery_weight=_mut_recovery_sign),
    "dropped_mass_complement": dict(dropped_mass=_mut_dropped_swapped),
    "tempered_log_sum_not_mean": dict(tempered_scores=_mut_tempered_log_sum),
    "tempered_not_divided_by_beta": dict(tempered_scores=_mut_tempered_undivided),
    "tempered_block_max": dict(tempered_scores=_mut_tempered_max),
    "tempered_beta_sign": dict(tempered_scores=_mut_tempered_neg_beta),
    "tile_routes_own_block": dict(tile_routable_blocks=_mut_tile_own_block),
    "tile_first_row_only": dict(tile_scores=_mut_tile_first_row),
    "tile_max_over_rows": dict(tile_scores=_mut_tile_max_row),
    "tile_variance_dropped": dict(tile_scores=_mut_tile_no_variance),
    "backward_D_dropped": dict(attend_backward=_mut_bwd_no_D),
    "backward_dk_unscaled": dict(attend_backward=_mut_bwd_dk_unscaled),
    "backward_dv_unnormalised": dict(attend_backward=_mut_bwd_dv_unnormalised),
    "backward_dq_uses_values": dict(attend_backward=_mut_bwd_dq_uses_v),
    "group_bound_no_radius": dict(group_bound=_mut_bound_no_radius),
    "group_bound_no_covariance_slack": dict(group_bound=_mut_bound_no_lam),
    "hier_prune_on_equal": dict(route_hier=_mut_hier_prune_on_equal),
    "hier_never_prunes": dict(route_hier=_mut_hier_bound_unused),
    "gqa_heads_interleaved": dict(kv_head=_mut_kv_head_modulo),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    ns = _impl(**MUTANTS[name])
    failures = 0
    for check in CHECKS:
        try:
            check(ns)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures >= 1, f"no pin catches the planted mistake {name!r}"


def test_planted_recall_report():
    """Planted-outlier recall on the tiny workload, beta = 2 vs beta = 0
    (centroid): the write-up reports that the variance term recovers targets
    the centroid misses; this checks that direction (the function itself is
    pinned by the hand-worked case above)."""
    from synth_inputs import CONFIGS, make_prefill
    wl = CONFIGS["tiny_prefill_4k"]
    data = make_prefill(wl, seed=0)
    orc = O.PrefillOracle(data["Q"], data["K"], data["V"],
                          O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale))
    r2 = O.planted_recall(orc, data["plants"])
    r0 = O.planted_recall(orc, data["plants"], beta=0.0)
    print(f"planted recall beta=2: {r2:.3f}  beta=0: {r0:.3f}")
    assert r2 >= r0


def test_oracle_compositions_match_pinned_copies():
    """The oracle's own row and tile compositions are the step sequences the
    pins exercise (same functions, same order), on random inputs."""
    rng = np.random.default_rng(21)
    n, d, B = 75, 6, 8
    Q, K, V = _rand_head(rng, n, d, B)
    mu, sigma = OR.block_stats(K, B)
    p = O.Params(B, 3, 5, 2.0, 0.45)
    ns = _impl()
    for t in (0, 7, 8, 40, 74):
        a = OR.prefill_row(Q[t], K, V, mu, sigma, p, t)
        b = ns.prefill_row(Q[t], K, V, mu, sigma, p, t)
        assert a["idx"].tolist() == b["idx"].tolist() and a["S"].tolist() == b["S"].tolist()
        assert np.array_equal(a["O"], b["O"]) and a["lse"] == b["lse"]
    for j in range((n + B - 1) // B):
        a = OR.tile_select(Q, mu, sigma, p, j)
        b = ns.tile_select(Q, mu, sigma, p, j)
        assert a["idx"].tolist() == b["idx"].tolist()
        assert np.array_equal(a["scores"], b["scores"])
        for t in range(j * B, min(n, (j + 1) * B), 3):
            ra = OR.tile_prefill_row(Q[t], K, V, a["idx"], p, t)
            rb = ns.tile_prefill_row(Q[t], K, V, b["idx"], p, t)
            assert ra["S"].tolist() == rb["S"].tolist() and np.array_equal(ra["O"], rb["O"])
    rng2 = np.random.default_rng(22)
    Qg = rng2.normal(size=(2, n, d))
    dO = rng2.normal(size=(2, n, d))
    idx = np.stack([np.stack([OR.prefill_row(Qg[j, t], K, V, mu, sigma, p, t)["idx"]
                              for t in range(n)]) for j in range(2)])
    a_ = OR.head_backward(Qg, K, V, idx, p, dO)
    b_ = ns.head_backward(Qg, K, V, idx, p, dO)
    for x, y in zip(a_, b_):
        assert np.array_equal(x, y)
    # whole-input compositions: PrefillOracle rows and planted recall (GQA)
    rng3 = np.random.default_rng(24)
    hq, hkv = 6, 2
    Q4 = rng3.normal(size=(2, hq, n, d))
    K4 = rng3.normal(size=(2, hkv, n, d))
    V4 = rng3.normal(size=(2, hkv, n, d))
    orc = O.PrefillOracle(Q4, K4, V4, p)
    for b, h, t in ((0, 0, 9), (1, 5, 74), (0, 3, 40), (1, 2, 17)):
        kv = ns.kv_head(h, hq, hkv)
        mu4, sg4 = ns.block_stats(K4[b, kv], B)
        a = orc.row(b, h, t)
        r = ns.prefill_row(Q4[b, h, t], K4[b, kv], V4[b, kv], mu4, sg4, p, t)
        assert a["idx"].tolist() == r["idx"].tolist() and np.array_equal(a["O"], r["O"])
    plants = [dict(b=int(rng3.integers(2)), h=int(rng3.integers(hq)), t=int(rng3.integers(n)),
                   block=int(rng3.integers(n // B))) for _ in range(40)]
    for beta, score in ((2.0, "cumulant"), (0.0, "cumulant"), (1.5, "tempered")):
        pb = O.Params(B, 3, 5, beta, 0.45)
        got = O.planted_recall(orc, plants, beta=beta, score=score)
        want = ns.planted_recall(Q4, K4, plants, pb, score)
        assert got == want, (beta, score, got, want)
