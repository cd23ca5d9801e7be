"""GPU parity of the exact tempered router (ssa_route_tempered) against the
oracle's tempered_row: per row the complete causal blocks' scores
T_c = (1/beta) ln mean_j exp(beta q.k_j) and the top-k rule of the cumulant
router.  Selections follow rule R1 of parity.py (exact, or differing only in
blocks within 1e-5 relative of the k-th score); the reported k-th and
(k+1)-th scores are compared with the oracle's within KTH_REL.
"""
from __future__ import annotations

import math
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

# float32 logits of O(10..100) against a float64 oracle: MFMA accumulation
# over d products and the float32 log-sum-exp (terms <= 2^8, up to 1024 of
# them) stay far inside 1e-5 relative of the score scale
KTH_REL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_TINY = CONFIGS["tiny_prefill_4k"]
_GQA = CONFIGS["gqa_prefill_128k"]
_P32 = CONFIGS["prefill_32k"]

# name -> (workload, beta)
CASES = {
    # float32, d = 64, B = 64, ragged n (not a multiple of B or of 256 rows)
    "f32_d64_beta0.5": (_TINY.replace(seq_len=1500, plants=4), 0.5),
    "f32_d64_beta2": (_TINY.replace(seq_len=1500, plants=4), 2.0),
    # bfloat16 GQA, d = 128, B = 256 (four chunks per block), ragged tail
    "bf16_gqa_B256_beta0.25": (_GQA.replace(n_q_heads=8, n_kv_heads=2, seq_len=2048 + 96,
                                            top_k=4, plants=4), 0.25),
    "bf16_gqa_B256_beta2": (_GQA.replace(n_q_heads=8, n_kv_heads=2, seq_len=2048 + 96,
                                         top_k=4, plants=4), 2.0),
    # large beta: later chunks exceed the first chunk's maximum by far more
    # than 2^8 in the exponent, so the running reference is raised
    "bf16_gqa_B256_beta40": (_GQA.replace(n_q_heads=8, n_kv_heads=2, seq_len=2048 + 96,
                                          top_k=4, plants=4), 40.0),
    # bfloat16, B = 128, k = 16 (rows with fewer routable blocks pad with -1)
    "bf16_B128_k16": (_P32.replace(n_q_heads=2, n_kv_heads=2, seq_len=4096, plants=8), 2.0),
    # bfloat16, d = 64, k = 32, two sequences
    "bf16_d64_k32": (_P32.replace(batch=2, n_q_heads=4, n_kv_heads=1, seq_len=3000, head_dim=64,
                                  block=64, top_k=32, plants=4), 1.0),
    # float32, d = 128, B = 192 (three chunks per block), GQA group 2
    "f32_d128_B192": (_P32.replace(n_q_heads=4, n_kv_heads=2, seq_len=2500, dtype="f32",
                                   block=192, top_k=8, plants=4), 4.0),
}


def _rows(wl, limit, seed=0):
    total = wl.batch * wl.n_q_heads * wl.seq_len
    rng = np.random.default_rng(seed)
    pick = rng.choice(total, size=min(limit, total), replace=False)
    # always include the first and last rows of every (sequence, head)
    rows = {(int(i) // (wl.n_q_heads * wl.seq_len), (int(i) // wl.seq_len) % wl.n_q_heads,
             int(i) % wl.seq_len) for i in pick}
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            rows |= {(b, h, 0), (b, h, wl.block - 1), (b, h, wl.block), (b, h, wl.seq_len - 1)}
    return sorted(rows)


def _kth_close(gpu: float, ref: float, scale: float) -> bool:
    if math.isnan(ref):
        return gpu == -math.inf
    return abs(gpu - ref) <= KTH_REL * max(1.0, scale)


@pytest.mark.parametrize("name", list(CASES))
def test_tempered_route_parity(name):
    wl, beta = CASES[name]
    say(f"case {name}: b={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} n={wl.seq_len} "
        f"d={wl.head_dim} {wl.dtype} B={wl.block} k={wl.top_k} beta={beta}")
    data = make_prefill(wl, seed=3)
    Q, K = data["Q"].to(DEV), data["K"].to(DEV)
    idx, kth = ssa.ssa_route_tempered(Q, K, block_size=wl.block, top_k=wl.top_k, beta=beta,
                                      want_kth=True)
    torch.cuda.synchronize()
    idx_h, kth_h = idx.cpu().numpy(), kth.cpu().numpy()
    for b in range(wl.batch):
        check_idx_properties(idx_h[b], wl.seq_len, wl.block, wl.top_k)
    g = wl.group
    Kd = {}
    n_exact = n_tie = 0
    worst = 0.0
    for (b, h, t) in _rows(wl, limit=1200):
        kv = h // g
        if (b, kv) not in Kd:
            Kd[(b, kv)] = O.as_f64(data["K"][b, kv])
        q = O.as_f64(data["Q"][b, h, t])
        row = O.tempered_row(q, Kd[(b, kv)], wl.block, wl.top_k, beta, t)
        ok, exact = idx_ok(idx_h[b, h, t], row)
        assert ok, f"selection mismatch at {(b, h, t)}: {idx_h[b, h, t]} vs {row['idx']}"
        n_exact += exact
        n_tie += not exact
        scale = float(np.abs(row["scores"]).max()) if row["scores"].size else 1.0
        for j, ref in enumerate((row["r_k"], row["r_k1"])):
            got = float(kth_h[b, h, t, j])
            assert _kth_close(got, ref, scale), f"kth[{j}] at {(b, h, t)}: {got} vs {ref}"
            if not math.isnan(ref):
                worst = max(worst, abs(got - ref) / max(1.0, scale))
    say(f"  {name}: exact {n_exact}, near-ties {n_tie}, max rel kth error {worst:.3g}")


def test_tempered_route_k0_reports_scores_only():
    wl, beta = CASES["bf16_gqa_B256_beta2"]
    wl = wl.replace(top_k=0)
    say("case tempered k=0 with kth")
    data = make_prefill(wl, seed=4)
    Q, K = data["Q"].to(DEV), data["K"].to(DEV)
    idx, kth = ssa.ssa_route_tempered(Q, K, block_size=wl.block, top_k=0, beta=beta,
                                      want_kth=True)
    torch.cuda.synchronize()
    assert idx.numel() == 0
    kh = kth.cpu().numpy()
    # with k = 0 the "k-th" score is absent and the (k+1)-th is the row maximum
    assert np.all(kh[..., 0] == -np.inf)
    Kh = O.as_f64(data["K"][0, 0])
    for t in (0, wl.block - 1, wl.block, 1000, wl.seq_len - 1):
        q = O.as_f64(data["Q"][0, 0, t])
        C = O.routable_blocks(t, wl.block, wl.seq_len // wl.block)
        r = O.tempered_scores(q, Kh, wl.block, C, beta)
        if C == 0:
            assert kh[0, 0, t, 1] == -np.inf
        else:
            assert abs(kh[0, 0, t, 1] - r.max()) <= KTH_REL * max(1.0, np.abs(r).max())


def test_tempered_route_deterministic():
    wl, beta = CASES["bf16_B128_k16"]
    say("case tempered determinism")
    data = make_prefill(wl, seed=5)
    Q, K = data["Q"].to(DEV), data["K"].to(DEV)
    a = ssa.ssa_route_tempered(Q, K, block_size=wl.block, top_k=wl.top_k, beta=beta, want_kth=True)
    b = ssa.ssa_route_tempered(Q, K, block_size=wl.block, top_k=wl.top_k, beta=beta, want_kth=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
