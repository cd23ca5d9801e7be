"""GPU parity of query-tile-shared routing (ssa_route_tiles) and attention over
tile selections (ssa_tile_attn_fwd) against the oracle's tile_select and
tile_prefill_row.

Every tile's selection follows rule R1 of parity.py against the oracle's
summed tile scores (exact, or differing only in blocks within 1e-5 relative of
the k-th score); the reported k-th / (k+1)-th tile scores are compared within
KTH_REL of the score scale; O and LSE of sampled rows are compared with the
oracle evaluated on the GPU's own tile selection (rule R6) under R2/R3.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import content_routed_block_stats_amd as ssa
import oracle as O
from parity import LSE_TOL, O_TOL, attn_errors, check_tile_properties, idx_ok
from synth_inputs import CONFIGS, make_prefill

pytestmark = pytest.mark.gpu
DEV = "cuda"
KTH_REL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


_TINY = CONFIGS["tiny_prefill_4k"]
_GQA = CONFIGS["gqa_prefill_128k"]
_P32 = CONFIGS["prefill_32k"]

CASES = {
    # float32, d = 64, B = 64, ragged n (partial last tile)
    "f32_d64_B64": _TINY.replace(seq_len=1500, plants=4),
    # bfloat16 GQA, d = 128, B = 256 (one workgroup per tile), ragged tail
    "bf16_gqa_B256": _GQA.replace(n_q_heads=8, n_kv_heads=2, seq_len=4096 + 96, top_k=4, plants=8),
    # bfloat16, B = 128 (half-empty workgroups), k = 16
    "bf16_B128_k16": _P32.replace(n_q_heads=2, n_kv_heads=2, seq_len=4096, plants=8),
    # bfloat16, d = 64, k = 32, two sequences
    "bf16_d64_k32": _P32.replace(batch=2, n_q_heads=4, n_kv_heads=1, seq_len=3000, head_dim=64,
                                 block=64, top_k=32, window=64, plants=4),
    # float32, d = 128, B = 192, GQA group 2, W < B
    "f32_d128_B192": _P32.replace(n_q_heads=4, n_kv_heads=2, seq_len=2500, dtype="f32", block=192,
                                  top_k=8, window=100, plants=4),
    # bfloat16, B = 512 (two workgroups per tile), W > B
    "bf16_B512_W700": _GQA.replace(n_q_heads=4, n_kv_heads=2, seq_len=6000, block=512, top_k=3,
                                   window=700, plants=4),
}


def _params(wl):
    return O.Params(wl.block, wl.top_k, wl.window, wl.beta, wl.scale)


def run_tiles(data, wl, out_dtype=None):
    Q, K, V = data["Q"].to(DEV), data["K"].to(DEV), data["V"].to(DEV)
    mu, sigma = ssa.ssa_block_stats(K, wl.block)
    idx, kth = ssa.ssa_route_tiles(Q, mu, sigma, block_size=wl.block, top_k=wl.top_k,
                                   beta=wl.beta, want_kth=True)
    Oo, lse = ssa.ssa_tile_attn_fwd(Q, K, V, idx, block_size=wl.block, window=wl.window,
                                    scale=wl.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return dict(idx=idx, kth=kth, O=Oo, lse=lse)


def compare(data, res, wl, row_limit=600, seed=0):
    p = _params(wl)
    g = wl.group
    idx_h = res["idx"].cpu().numpy()
    kth_h = res["kth"].cpu().numpy()
    tiles = idx_h.shape[2]
    for b in range(wl.batch):
        check_tile_properties(idx_h[b], wl.seq_len, wl.block, wl.top_k)
    n_exact = n_tie = 0
    heads = {}
    for b in range(wl.batch):
        for kv in range(wl.n_kv_heads):
            Kh = O.as_f64(data["K"][b, kv])
            heads[(b, kv)] = (Kh, O.as_f64(data["V"][b, kv])) + O.block_stats(Kh, wl.block)
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            Kh, Vh, mu, sigma = heads[(b, h // g)]
            Qh = O.as_f64(data["Q"][b, h])
            for j in range(tiles):
                orc = O.tile_select(Qh, mu, sigma, p, j)
                ok, exact = idx_ok(idx_h[b, h, j], orc)
                assert ok, f"tile selection mismatch at {(b, h, j)}: {idx_h[b, h, j]} vs {orc['idx']}"
                n_exact += exact
                n_tie += not exact
                scale = float(np.abs(orc["scores"]).max()) if orc["scores"].size else 1.0
                for col, ref in enumerate((orc["r_k"], orc["r_k1"])):
                    got = float(kth_h[b, h, j, col])
                    if math.isnan(ref):
                        assert got == -math.inf, (b, h, j, col, got)
                    else:
                        assert abs(got - ref) <= KTH_REL * max(1.0, scale), (b, h, j, col, got, ref)
    rng = np.random.default_rng(seed)
    total = wl.batch * wl.n_q_heads * wl.seq_len
    pick = rng.choice(total, size=min(row_limit, total), replace=False)
    rows = {(int(i) // (wl.n_q_heads * wl.seq_len), (int(i) // wl.seq_len) % wl.n_q_heads,
             int(i) % wl.seq_len) for i in pick}
    for b in range(wl.batch):
        for h in range(wl.n_q_heads):
            rows |= {(b, h, 0), (b, h, wl.block - 1), (b, h, wl.block), (b, h, wl.seq_len - 1)}
    bf16_out = res["O"].dtype == torch.bfloat16
    worst_o = worst_l = 0.0
    for (b, h, t) in sorted(rows):
        Kh, Vh, _, _ = heads[(b, h // g)]
        q = O.as_f64(data["Q"][b, h, t])
        eo, el = attn_errors(res["O"][b, h, t].float().cpu().numpy(), float(res["lse"][b, h, t]), q,
                             Kh, Vh, idx_h[b, h, t // wl.block], t, p, bf16_out=bf16_out)
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
        assert eo <= O_TOL[wl.dtype], f"O error {eo:.3g} at {(b, h, t)}"
        assert el <= LSE_TOL, f"LSE error {el:.3g} at {(b, h, t)}"
    say(f"  tiles exact {n_exact}, near-ties {n_tie}; rows {len(rows)}: max|dO| {worst_o:.3g}, "
        f"max|dLSE| {worst_l:.3g}")


@pytest.mark.parametrize("name", list(CASES))
def test_tile_parity(name):
    wl = CASES[name]
    say(f"case {name}: b={wl.batch} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} n={wl.seq_len} "
        f"d={wl.head_dim} {wl.dtype} B={wl.block} k={wl.top_k} W={wl.window}")
    data = make_prefill(wl, seed=2)
    res = run_tiles(data, wl)
    compare(data, res, wl)


def test_tile_dense_reduction():
    """k >= nb and W >= B: every row attends to all keys <= t (dense causal)."""
    wl = CONFIGS["tiny_prefill_4k"].replace(seq_len=700, top_k=16, window=64, plants=2)
    say("case tile dense reduction f32 n=700 B=64 k=16 W=64")
    data = make_prefill(wl, seed=5)
    res = run_tiles(data, wl)
    q = data["Q"][0, 0].double()
    k = data["K"][0, 0].double()
    v = data["V"][0, 0].double()
    s = (q @ k.T) * wl.scale
    s = s.masked_fill(torch.ones_like(s, dtype=torch.bool).triu(1), float("-inf"))
    ref_o = torch.softmax(s, -1) @ v
    ref_l = torch.logsumexp(s, -1)
    assert (res["O"][0, 0].double().cpu() - ref_o).abs().max().item() <= O_TOL["f32"]
    assert (res["lse"][0, 0].double().cpu() - ref_l).abs().max().item() <= LSE_TOL


def test_tile_deterministic_and_bf16_output():
    wl = CASES["bf16_gqa_B256"]
    say("case tile determinism bf16 gqa")
    data = make_prefill(wl, seed=1)
    a = run_tiles(data, wl)
    b = run_tiles(data, wl)
    for key in ("idx", "kth", "O", "lse"):
        assert torch.equal(a[key], b[key]), f"{key} differs between identical runs"
    c = run_tiles(data, wl, out_dtype=torch.float32)
    assert torch.equal(a["O"], c["O"].to(torch.bfloat16))


def test_tile_k0_is_window_attention():
    """k = 0: no blocks; every row attends to its window only (banded causal)."""
    wl = CASES["bf16_B128_k16"].replace(top_k=0, window=77)
    say("case tile k=0 window only")
    data = make_prefill(wl, seed=6)
    res = run_tiles(data, wl)
    assert res["idx"].numel() == 0
    q = O.as_f64(data["Q"][0, 1])
    K = O.as_f64(data["K"][0, 1])
    V = O.as_f64(data["V"][0, 1])
    for t in (0, 5, 76, 77, 500, wl.seq_len - 1):
        S = np.arange(max(0, t - wl.window + 1), t + 1)
        Oo, lse = O.attend(q[t], K, V, S, wl.scale)
        got = res["O"][0, 1, t].float().cpu().numpy()
        assert np.abs(got - Oo).max() <= O_TOL["bf16"] + np.abs(Oo).max() * 2.0 ** -8
        assert abs(float(res["lse"][0, 1, t]) - lse) <= LSE_TOL
