"""CPU oracle for Subquadratic Sparse Attention (SSA) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never
calls it and fails loudly when its native library is missing.

What it computes, from the write-up "Subquadratic Sparse Attention (SSA)"
(git.hmmc.top/jonsmirl/ssa), introduction paragraph (mechanism steps i-iii) and
section "The idea in one screen" (recovery law and routing score):

  for each query row (sequence, q-head h, position t):
    1. per complete key block c of the row's KV head: mean mu_c and population
       covariance Sigma_c of its B keys (the "per-block summary statistics");
    2. routing score r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q over the blocks
       whose last key is <= t;
    3. keep the top-k scores (ties to the lower block index);
    4. key set S(t) = union of the selected blocks and the local window
       [max(0, t-W+1), t], each key once;
    5. exact softmax attention over S(t): O and the log-sum-exp LSE;
    6. the dropped softmax mass 1 - (dense causal weight on S(t)).

All arithmetic is float64 on values that are exact copies of the caller's
inputs (float32 or bfloat16 values).  There is no blocking, fusion or
reordering beyond what the definition states; matmul, einsum and lexsort are
used as library primitives.  Readings of points the write-up leaves open:
  * the score uses raw q and raw key statistics, beta on raw logits;
  * Sigma_c is the population (1/B) covariance;
  * only complete blocks are routable, and only if their last key is <= t;
  * the window [max(0, t-W+1), t] includes t; S(t) is a set;
  * k larger than the number of routable blocks selects them all (-1 padding);
  * GQA: q-head h reads KV head h // (Hq/Hkv);
  * LSE is the natural log of sum_{j in S} exp(scale * q.k_j).

Every function here is pinned by a CPU test against something other than
itself (closed forms, textbook formulations, brute force, library routines);
the one study that has no such pin (planted-outlier recall) says so.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Params:
    """Method parameters in the write-up's notation."""

    block: int      # B, keys per block
    top_k: int      # k, blocks kept per query
    window: int     # W, local window length (>= 1)
    beta: float     # routing inverse temperature on raw logits
    scale: float    # softmax scale on raw logits (float32 value of 1/sqrt(d))


def as_f64(x) -> np.ndarray:
    """Exact float64 copy of a float32 / bfloat16 array (torch or numpy)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: only for the dtype check
        if x.dtype != torch.float64:
            x = x.to(torch.float64)
        return x.numpy()
    return np.asarray(x, dtype=np.float64)


# -- step 1: per-block summary statistics ------------------------------------

def block_stats(K: np.ndarray, B: int) -> tuple[np.ndarray, np.ndarray]:
    """Mean and population covariance of every complete block of B keys.

    K: [n, d] keys of one (sequence, KV head).  Returns mu [nb, d] and
    sigma [nb, d, d] with nb = n // B.  Sigma_c = (1/B) sum_j (k_j - mu_c)(k_j - mu_c)^T,
    the covariance whose quadratic form q^T Sigma_c q is the variance of the
    logit q.k_j across the block ("The idea in one screen").
    """
    K = as_f64(K)
    n, d = K.shape
    nb = n // B
    mu = np.zeros((nb, d))
    sigma = np.zeros((nb, d, d))
    for c in range(nb):
        blk = K[c * B:(c + 1) * B]
        m = blk.sum(axis=0) / B
        X = blk - m
        mu[c] = m
        sigma[c] = (X.T @ X) / B
    return mu, sigma


# -- step 2: routing score over routable blocks -------------------------------

def routable_blocks(t: int, B: int, nb: int) -> int:
    """Number of blocks routable for query position t: blocks c with (c+1)B-1 <= t."""
    return max(0, min(nb, (t + 1) // B))


def route_scores(q: np.ndarray, mu: np.ndarray, sigma: np.ndarray, beta: float) -> np.ndarray:
    """r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q for every block given.

    Second-cumulant (tempered) routing score, "The idea in one screen".
    q: [d]; mu: [C, d]; sigma: [C, d, d].  Returns [C].
    """
    q = as_f64(q)
    mean_term = mu @ q
    var_term = np.einsum("i,cij,j->c", q, sigma, q)
    return mean_term + 0.5 * beta * var_term


def route_scores_from_logits(q: np.ndarray, K: np.ndarray, B: int, C: int,
                             beta: float) -> np.ndarray:
    """The same score computed from the logits: mean_j(q.k_j) + (beta/2) var_pop_j(q.k_j).

    This is the reading "block mean plus the variance of the logit across the
    block" of the routing score, evaluated on the B keys of each block directly.
    """
    q = as_f64(q)
    K = as_f64(K)
    out = np.zeros(C)
    for c in range(C):
        s = K[c * B:(c + 1) * B] @ q
        m = s.sum() / B
        out[c] = m + 0.5 * beta * (((s - m) ** 2).sum() / B)
    return out


# -- tempered routing family (exact block score) ------------------------------

def tempered_scores(q: np.ndarray, K: np.ndarray, B: int, C: int, beta: float) -> np.ndarray:
    """T_c(q) = (1/beta) log( (1/B) sum_{j in block c} exp(beta q.k_j) ) for blocks c < C.

    The temperature family of the write-up's module list (centroid <->
    cumulant <-> exact max), read as the exact log-mean-exp of the block's raw
    logits: its second-order expansion in beta is r_c(q) = <q, mu_c> +
    (beta/2) q^T Sigma_c q; beta -> 0 gives the block mean of the logits (the
    centroid score), beta -> infinity the block maximum.  beta > 0.  Evaluated
    with the maximum factored out: with u_j = beta q.k_j and m = max_j u_j,
    T_c = (m + log sum_j exp(u_j - m) - log B) / beta.
    """
    if not beta > 0:
        raise ValueError("the tempered score needs beta > 0")
    q = as_f64(q)
    K = as_f64(K)
    out = np.zeros(C)
    for c in range(C):
        u = beta * (K[c * B:(c + 1) * B] @ q)
        m = u.max()
        out[c] = (m + math.log(np.exp(u - m).sum()) - math.log(B)) / beta
    return out


def tempered_row(q: np.ndarray, K: np.ndarray, B: int, k: int, beta: float, t: int) -> dict:
    """Routing of one query row by the tempered score: the complete causal
    blocks' scores, then the same top-k rule as the cumulant router."""
    nb = as_f64(K).shape[0] // B
    C = routable_blocks(t, B, nb)
    r = tempered_scores(q, K, B, C, beta)
    idx, r_k, r_k1 = select_topk(r, k)
    return dict(idx=idx, scores=r, r_k=r_k, r_k1=r_k1)


# -- query-tile-shared routing (block-level selection) ------------------------
#
# The write-up's fast kernel routes per query block: its cost notes name an
# (n/b)^2 block-score GEMM and an argsort BlockMask build.  Reading: query
# tile j holds positions [jB, (j+1)B) of one (sequence, q-head); the tile
# selects one set of blocks for all its queries, the top k of the tile's
# summed routing score R_c = sum_{t in tile} r_c(q_t) over the blocks complete
# before the tile starts (c < j); each row then attends exactly over the
# tile's blocks plus its own window.

def tile_routable_blocks(j: int, nb: int) -> int:
    """Blocks routable for query tile j: those complete before the tile's first
    query, c < j (c + 1 <= j, so (c+1)B - 1 <= jB - 1 < jB)."""
    return max(0, min(nb, j))


def tile_scores(Qt: np.ndarray, mu: np.ndarray, sigma: np.ndarray, beta: float) -> np.ndarray:
    """R_c = sum over the tile's query rows of r_c(q_t), for every block given."""
    Qt = as_f64(Qt)
    R = np.zeros(np.asarray(mu).shape[0])
    for q in Qt:
        R += route_scores(q, mu, sigma, beta)
    return R


def tile_select(Qh: np.ndarray, mu: np.ndarray, sigma: np.ndarray, p: Params, j: int) -> dict:
    """Selection of query tile j of one (sequence, q-head): Qh [n, d] are the
    head's queries, mu/sigma its KV head's block statistics."""
    Qh = as_f64(Qh)
    n = Qh.shape[0]
    C = tile_routable_blocks(j, mu.shape[0])
    R = tile_scores(Qh[j * p.block:min(n, (j + 1) * p.block)], mu[:C], sigma[:C], p.beta)
    idx, r_k, r_k1 = select_topk(R, p.top_k)
    return dict(idx=idx, scores=R, r_k=r_k, r_k1=r_k1)


def tile_prefill_row(q, K, V, tile_idx: np.ndarray, p: Params, t: int) -> dict:
    """Exact attention of row t over its tile's selected blocks and its window."""
    S = key_set(t, tile_idx, p.block, p.window)
    O, lse = attend(q, K, V, S, p.scale)
    return dict(S=S, O=O, lse=lse)


# -- hierarchical routing: the exact top-k by branch and bound over groups ------
#
# The write-up's module list pairs the flat router with branch-and-bound exact
# selection under an admissible bound and a tree router with a recursive
# radius (Barnes-Hut style), and "Selected results" report lossless
# branch-and-bound selection costs as a fraction of keys.  Reading: groups of
# m consecutive blocks carry a summary from which an upper bound on every
# member's routing score follows; groups are visited in decreasing bound order
# and skipped when their bound is strictly below the running k-th best score,
# so the selection is exactly the flat top-k and only the cost changes.
#   UB_G(q) = q.mu_G + ||q|| R_G + (beta/2) (q^T S_G q + lam_G ||q||^2)   (beta >= 0)
# with mu_G the mean of the members' mu_c, R_G = max ||mu_c - mu_G||, S_G the
# mean of their Sigma_c and lam_G = max (tr (Sigma_c - S_G)^4)^(1/4), which is
# at least the spectral norm ||Sigma_c - S_G||_2: then q.mu_c <= q.mu_G +
# ||q|| R_G (Cauchy-Schwarz) and q^T Sigma_c q <= q^T S_G q + lam_G ||q||^2.

def group_summaries(mu: np.ndarray, sigma: np.ndarray, m: int) -> dict:
    """Summaries of the groups of m consecutive blocks (the last may be partial)."""
    mu, sigma = as_f64(mu), as_f64(sigma)
    nb, d = mu.shape
    G = -(-nb // m)
    out = dict(mu=np.zeros((G, d)), R=np.zeros(G), S=np.zeros((G, d, d)), lam=np.zeros(G))
    for gi in range(G):
        c0, c1 = gi * m, min(nb, (gi + 1) * m)
        mg = mu[c0:c1].mean(0)
        Sg = sigma[c0:c1].mean(0)
        out["mu"][gi] = mg
        out["S"][gi] = Sg
        out["R"][gi] = max(np.linalg.norm(mu[c] - mg) for c in range(c0, c1))
        lam = 0.0
        for c in range(c0, c1):
            A = sigma[c] - Sg
            A2 = A @ A
            lam = max(lam, float(np.sum(A2 * A2)) ** 0.25)      # (tr A^4)^(1/4)
        out["lam"][gi] = lam
    return out


def group_bound(q: np.ndarray, gs: dict, beta: float) -> np.ndarray:
    """UB_G(q) for every group (beta >= 0)."""
    q = as_f64(q)
    nq = float(np.linalg.norm(q))
    quad = np.einsum("i,gij,j->g", q, gs["S"], q)
    return gs["mu"] @ q + nq * gs["R"] + 0.5 * beta * (quad + gs["lam"] * nq * nq)


def route_hier(q: np.ndarray, mu: np.ndarray, sigma: np.ndarray, gs: dict, m: int, k: int,
               beta: float, C: int) -> dict:
    """Exact top-k of r_c(q) over the blocks c < C by branch and bound over the
    groups of m blocks: returns idx (as select_topk) and the number of blocks
    whose score was evaluated."""
    if beta < 0:
        raise ValueError("the group bound needs beta >= 0")
    ub = group_bound(q, gs, beta)
    G = -(-C // m)
    order = sorted(range(G), key=lambda gi: (-ub[gi], gi))
    scores: dict[int, float] = {}
    for gi in order:
        if len(scores) >= k > 0:
            tau = sorted(scores.values(), reverse=True)[k - 1]
            if ub[gi] < tau:
                continue
        elif k == 0:
            break
        blocks = list(range(gi * m, min(C, (gi + 1) * m)))
        r = route_scores(q, as_f64(mu)[blocks], as_f64(sigma)[blocks], beta)
        scores.update(zip(blocks, r.tolist()))
    cs = np.array(sorted(scores), dtype=np.int64)
    r_eval = np.array([scores[c] for c in cs])
    sel, _, _ = select_topk(r_eval, k)
    idx = np.full(k, -1, dtype=np.int32)
    chosen = np.sort(cs[sel[sel >= 0]]) if cs.size else np.zeros(0, dtype=np.int64)
    idx[:chosen.size] = chosen
    return dict(idx=idx, evaluated=len(scores))


# -- step 3: top-k selection ---------------------------------------------------

def select_topk(r: np.ndarray, k: int) -> tuple[np.ndarray, float, float]:
    """Top-k block indices of the scores r (ties to the lower index).

    Returns (idx, r_k, r_k1): idx is int32 [k], the selected block indices in
    ascending order padded with -1 when fewer than k blocks exist; r_k and r_k1
    are the k-th and (k+1)-th largest scores (nan where they do not exist).
    """
    r = np.asarray(r, dtype=np.float64)
    E = r.shape[0]
    order = np.lexsort((np.arange(E), -r))   # primary key -r, then block index
    keep = min(k, E)
    idx = np.full(k, -1, dtype=np.int32)
    idx[:keep] = np.sort(order[:keep])
    r_k = float(r[order[k - 1]]) if 0 < k <= E else math.nan
    r_k1 = float(r[order[k]]) if k < E else math.nan
    return idx, r_k, r_k1


# -- step 4: key-set assembly --------------------------------------------------

def key_set(t: int, idx: np.ndarray, B: int, W: int) -> np.ndarray:
    """S(t) = union of the selected blocks' keys and the window [max(0,t-W+1), t]."""
    keys: set[int] = set()
    for c in np.asarray(idx).tolist():
        if c >= 0:
            keys.update(range(c * B, (c + 1) * B))
    keys.update(range(max(0, t - W + 1), t + 1))
    return np.array(sorted(keys), dtype=np.int64)


# -- step 5: exact softmax attention over the selected keys ------------------

def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, S: np.ndarray,
           scale: float) -> tuple[np.ndarray, float]:
    """Exact softmax attention of q over the keys S: returns (O [d], LSE).

    s_j = scale * q.k_j;  O = sum_j softmax(s)_j v_j;  LSE = ln sum_j exp(s_j).
    """
    q = as_f64(q)
    s = scale * (as_f64(K)[S] @ q)
    m = s.max()
    p = np.exp(s - m)
    l = p.sum()
    O = (p @ as_f64(V)[S]) / l
    return O, float(m + math.log(l))


# -- backward: gradients through the exact attention over S(t) -----------------
#
# Training through the layer (the write-up's module list trains small SSA
# models and its "Selected results" adapt a dense model swapped to SSA): the
# selection is a discrete choice, so gradients flow through the softmax
# attention over the chosen keys, with S(t) held fixed.  For a loss L with
# upstream gradient dO_t = dL/dO_t:
#   p_j = softmax_j(scale q.k_j) over j in S(t),  O = sum_j p_j v_j,
#   dP_j = dO . v_j,   D = sum_j p_j dP_j  (= dO . O),
#   dS_j = p_j (dP_j - D)                 (softmax Jacobian),
#   dq   = scale sum_j dS_j k_j,   dk_j += scale dS_j q,   dv_j += p_j dO.

def attend_backward(q: np.ndarray, K: np.ndarray, V: np.ndarray, S: np.ndarray, scale: float,
                    dO: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(dq [d], dK_S [|S|, d], dV_S [|S|, d]) of one row's attention over keys S."""
    q = as_f64(q)
    Ks = as_f64(K)[S]
    Vs = as_f64(V)[S]
    dO = as_f64(dO)
    s = scale * (Ks @ q)
    p = np.exp(s - s.max())
    p = p / p.sum()
    dP = Vs @ dO
    D = float(p @ dP)
    dS = p * (dP - D)
    dq = scale * (dS @ Ks)
    dK = scale * np.outer(dS, q)
    dV = np.outer(p, dO)
    return dq, dK, dV


def head_backward(Qh, K, V, idx_h, p: Params, dOh, rows=None):
    """Gradients for the q-heads of one KV head with fixed selections.

    Qh, dOh: [g, n, d] (the group's q-heads); K, V: [n, d]; idx_h: [g, n, k]
    per-query selections (as the forward used).  Returns (dQ [g, n, d],
    dK [n, d], dV [n, d]); dK/dV sum over every row of the group.  rows, if
    given, restricts the sum to those (j, t) rows (the other dQ rows stay 0).
    """
    Qh, dOh = as_f64(Qh), as_f64(dOh)
    g, n, d = Qh.shape
    dQ = np.zeros((g, n, d))
    dK = np.zeros((n, d))
    dV = np.zeros((n, d))
    it = rows if rows is not None else [(j, t) for j in range(g) for t in range(n)]
    for (j, t) in it:
        S = key_set(t, np.asarray(idx_h)[j, t], p.block, p.window)
        dq, dk, dv = attend_backward(Qh[j, t], K, V, S, p.scale, dOh[j, t])
        dQ[j, t] = dq
        dK[S] += dk
        dV[S] += dv
    return dQ, dK, dV


# -- step 6: dropped mass ------------------------------------------------------

def dropped_mass(q: np.ndarray, K: np.ndarray, S: np.ndarray, t: int,
                 scale: float) -> tuple[float, float]:
    """Dropped softmax mass of S(t) against dense causal attention over j <= t.

    Returns (eps_from_lse, eps_direct): 1 - exp(LSE_S - LSE_full), and the sum
    of the dense softmax probabilities of the keys j <= t that are not in S.
    """
    q = as_f64(q)
    s = scale * (as_f64(K)[: t + 1] @ q)
    m = s.max()
    p = np.exp(s - m)
    p = p / p.sum()
    inside = np.zeros(t + 1, dtype=bool)
    inside[S] = True
    eps_direct = float(p[~inside].sum())
    l_full = math.log(np.exp(s - m).sum()) + m
    l_sel = math.log(np.exp(s[S] - m).sum()) + m
    return float(-math.expm1(l_sel - l_full)), eps_direct


# -- the full row --------------------------------------------------------------

def prefill_row(q, K, V, mu, sigma, p: Params, t: int, with_dense: bool = False) -> dict:
    """Every step for one query row at position t of one (sequence, q-head).

    K, V: [n, d] of the row's KV head; mu, sigma: that head's block statistics.
    """
    nb = mu.shape[0]
    C = routable_blocks(t, p.block, nb)
    r = route_scores(q, mu[:C], sigma[:C], p.beta)
    idx, r_k, r_k1 = select_topk(r, p.top_k)
    S = key_set(t, idx, p.block, p.window)
    O, lse = attend(q, K, V, S, p.scale)
    out = dict(idx=idx, scores=r, r_k=r_k, r_k1=r_k1, S=S, O=O, lse=lse)
    if with_dense:
        O_full, lse_full = attend(q, K, V, np.arange(t + 1), p.scale)
        eps, eps_direct = dropped_mass(q, K, S, t, p.scale)
        out.update(O_full=O_full, lse_full=lse_full, eps=eps, eps_direct=eps_direct)
    return out


def kv_head(h: int, hq: int, hkv: int) -> int:
    """The KV head query head h reads under grouped-query attention: the hq
    query heads form hkv contiguous groups of hq/hkv, group j sharing KV head
    j (the pages name GQA head counts but not the mapping; this is the usual
    one, the one torch's SDPA uses with enable_gqa)."""
    return h // (hq // hkv)


class PrefillOracle:
    """Per-row oracle over a whole prefill input, caching per-head statistics.

    Q: [b, Hq, n, d]; K, V: [b, Hkv, n, d] (torch or numpy, any float dtype).
    """

    def __init__(self, Q, K, V, p: Params):
        self.Q, self.K, self.V, self.p = Q, K, V, p
        self.hq, self.hkv = Q.shape[1], K.shape[1]
        self._cache: dict[tuple[int, int], tuple] = {}

    def head(self, b: int, kv: int):
        key = (b, kv)
        if key not in self._cache:
            Kh = as_f64(self.K[b, kv])
            Vh = as_f64(self.V[b, kv])
            mu, sigma = block_stats(Kh, self.p.block)
            self._cache[key] = (Kh, Vh, mu, sigma)
        return self._cache[key]

    def drop(self, b: int, kv: int) -> None:
        self._cache.pop((b, kv), None)

    def row(self, b: int, h: int, t: int, with_dense: bool = False) -> dict:
        kv = kv_head(h, self.hq, self.hkv)
        Kh, Vh, mu, sigma = self.head(b, kv)
        return prefill_row(as_f64(self.Q[b, h, t]), Kh, Vh, mu, sigma, self.p, t, with_dense)


# -- decode --------------------------------------------------------------------

def decode_step(q, k_new, v_new, K_cache, V_cache, L: int, p: Params,
                with_dense: bool = False) -> dict:
    """One decode step for one (sequence, q-head): append at L, query at t = L.

    K_cache/V_cache: [>= L, d] of the head's KV head (first L rows valid).
    The step is the prefill definition at t = L over the L+1 keys.
    """
    K = np.concatenate([as_f64(K_cache)[:L], as_f64(k_new)[None]], axis=0)
    V = np.concatenate([as_f64(V_cache)[:L], as_f64(v_new)[None]], axis=0)
    mu, sigma = block_stats(K, p.block)
    return prefill_row(as_f64(q), K, V, mu, sigma, p, L, with_dense)


# -- the recovery law ------------------------------------------------------------

def recovery_weight(beta: float, delta: float, mu: float) -> float:
    """w* = sigma(beta*Delta - log mu): softmax weight of one target with margin
    Delta over mu equal distractors ("The idea in one screen", recovery law)."""
    z = beta * delta - math.log(mu)
    return 1.0 / (1.0 + math.exp(-z))


# -- planted-outlier recall (a study) ------------------------------------------------

def planted_recall(oracle: PrefillOracle, plants: list[dict], beta: float | None = None,
                   score: str = "cumulant") -> float:
    """Fraction of planted outliers whose block the target row selects, routing
    by the second-cumulant score (score="cumulant") or by the exact tempered
    score (score="tempered", beta > 0).

    The write-up states only the qualitative result (second-cumulant routing
    recovers targets that centroid routing misses); the function is pinned by
    a hand-worked case (two blocks whose scores cross as beta grows).
    """
    if not plants:
        return math.nan
    p = oracle.p if beta is None else Params(oracle.p.block, oracle.p.top_k, oracle.p.window,
                                             beta, oracle.p.scale)
    hits = 0
    for pl in plants:
        kv = kv_head(pl["h"], oracle.hq, oracle.hkv)
        Kh, Vh, mu, sigma = oracle.head(pl["b"], kv)
        t = pl["t"]
        C = routable_blocks(t, p.block, mu.shape[0])
        q = as_f64(oracle.Q[pl["b"], pl["h"], t])
        if score == "tempered":
            r = tempered_scores(q, Kh, p.block, C, p.beta)
        else:
            r = route_scores(q, mu[:C], sigma[:C], p.beta)
        idx, _, _ = select_topk(r, p.top_k)
        hits += int(pl["block"] in idx.tolist())
    return hits / len(plants)
